/*
 * moe.h -- C ABI of the MI355X post-router MoE layer library (libmoe_mi355x.so).
 *
 * The library executes the post-router part of a Mixture-of-Experts layer on
 * one GPU: token dispatch, the routed SwiGLU experts, the fused shared expert
 * and the probability-weighted combine, forward and backward.  That is the
 * path the megakernel backend replaces (Megatron-LM PR #6572, Summary; the
 * forward takes hidden_states, probs and routing_map and returns an output of
 * the hidden states' shape: Megatron Core API docs, mok.backend,
 * MoKMegakernel.forward).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Ownership.  The caller owns every byte: inputs, outputs, weights,
 *    main_grad, the forward->backward context `saved` and the workspace.  The
 *    library never allocates device memory, never frees, never copies weight
 *    payloads and keeps no pointer across calls: arguments are non-owning
 *    references (Megatron Core API docs, mok.runtime, _MoKWeightArguments).
 *    Pointer tables (`table` fields) are device arrays owned by the caller.
 *  Streams.  All work is enqueued on the caller's `stream`; no host
 *    synchronisation and no device-to-host copy happens inside a call, so a
 *    call can be captured into a HIP graph.  Calls that use distinct `saved`
 *    and workspace buffers may run concurrently.
 *  Errors.  Arguments are validated on the host before anything is enqueued;
 *    a non-OK status means nothing was launched.  MOE_ERR_HIP reports a
 *    failed kernel launch.  Data-dependent errors found on the device (a
 *    routing-map row with more than `topk` true entries) set a status word in
 *    `saved` (see moe_saved_view); outputs of that call are then unspecified.
 *    No entry point throws or aborts.
 *  Layouts.  Every matrix is row-major; strides are in elements.
 *
 * Sizes: T tokens (all leading dims of hidden_states flattened), H hidden,
 * I intermediate (one value for routed and shared experts: PR #6572,
 * Supported configurations, current limitations), E local routed experts,
 * K = topk.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,            /* a required pointer is NULL                               */
  MOE_ERR_SHAPE = 2,           /* a size is out of range or not a multiple the kernels need */
  MOE_ERR_DTYPE = 3,           /* unsupported element type (e.g. non-BF16 shared expert)  */
  MOE_ERR_LAYOUT = 4,          /* inconsistent strides / both or neither of base and table */
  MOE_ERR_UNSUPPORTED = 5,     /* a configuration not implemented (unknown flag bits, flag
                                  combinations, swiglu_limit NaN / negative / infinite)    */
  MOE_ERR_WORKSPACE = 6,       /* saved / workspace buffer missing or too small            */
  MOE_ERR_ROUTE_OVERFLOW = 7,  /* device status word: a row had more than topk routes      */
  MOE_ERR_HIP = 8,             /* a HIP launch failed                                      */
  MOE_ERR_ROUTE_INVALID = 9    /* device status word: a top_experts entry outside [-1, E)
                                  or listed twice in one row (moe_forward_topk)            */
} moe_status;

typedef enum { MOE_BF16 = 1, MOE_FP32 = 2, MOE_MXFP8_E4M3 = 3 } moe_dtype;

/* Set: the shared expert is fused into the same launches (PR #6572, Summary: the
 * backend runs dispatch, routed and shared experts, and combine).  Clear: routed-only
 * mode, the follow-up named in PR #8210 (Summary and the review thread on TP for the
 * shared expert) where the caller runs the shared expert itself; the output and the
 * data gradient then hold the routed terms only, and the shared weights and shared
 * main_grad buffers are neither validated nor touched (they may be all zero/NULL). */
#define MOE_FLAG_HAS_SHARED 1u
/* Set: MoE-layer recompute (PR #6572, Validation: MoE layer recompute; PR #8210, Summary:
 * whole-MoE recomputation).  `saved` then holds only the routing state (a few bytes per
 * token); the forward keeps its activations in its workspace, and moe_backward
 * regenerates them from `hidden` with the same kernels before the backward proper, so
 * every result is bit-identical to the mode without the flag.  The flag must be the same
 * in the forward and the backward of one layer call, and the workspaces grow by the
 * activations (see moe_workspace_bytes). */
#define MOE_FLAG_RECOMPUTE 2u
/* Set: the routing arrives as the router's fixed-width table (top_experts and
 * router_weights, [T][K]), the form the runtime consumes (Megatron Core API docs,
 * mok.runtime, _MoKAutograd.forward), through moe_forward_topk; moe_backward then writes
 * grad_probs as [T][K].  Clear: the dense routing map and probabilities through
 * moe_forward. */
#define MOE_FLAG_TOPK_ROUTING 4u
/* Set (with MOE_FLAG_HAS_SHARED): the shared expert's output gate, MCore's optional
 * shared-expert output gate (PR #6572, Supported configurations) and the runtime's
 * shared_output_gate_weight argument (Megatron Core API docs, mok.runtime,
 * _MoKAutograd.forward).  The pages give no formula; the reading implemented: a BF16
 * weight g [1][H] (moe_weights.shared_out_gate) and one score per token,
 * s_t = sigmoid(x_t . g), multiplying the shared expert's output:
 *     out[t] = s_t shared(x_t) + sum_k w_tk expert_{e_tk}(x_t)
 * The backward adds sum_t s_t (1 - s_t) (grad_out_t . shared(x_t)) x_t to
 * moe_main_grads.shared_out_gate. */
#define MOE_FLAG_SHARED_GATE 8u

/* Problem sizes and options. */
typedef struct {
  int64_t tokens;        /* T >= 0                                                        */
  int64_t hidden;        /* H, multiple of 128                                            */
  int64_t intermediate;  /* I, multiple of 128                                            */
  int32_t experts;       /* E in [1, 255]                                                 */
  int32_t topk;          /* K in [1, min(8, E)]                                           */
  int32_t routed_dtype;  /* MOE_BF16 or MOE_MXFP8_E4M3 (PR #6572, Supported configurations) */
  uint32_t flags;        /* MOE_FLAG_HAS_SHARED (else routed-only) | MOE_FLAG_RECOMPUTE
                            | MOE_FLAG_TOPK_ROUTING | MOE_FLAG_SHARED_GATE                 */
  float swiglu_limit;    /* SwiGLU clamp L >= 0 of every expert (0: none).  The pages pass
                            MCore's activation_func_clamp_value as swiglu_limit (PR #8210,
                            review thread on the config port) without a formula; reading:
                            h = silu(min(a, L)) clamp(b, -L, L), a = gate and b = up
                            pre-activation, no gradient through a clamped input (the bounds
                            themselves pass it).  Whether an input is clamped is decided on
                            its FP32 value in the forward.  NaN, negative or infinite:
                            unsupported                                                      */
} moe_problem;

/* One logical matrix per expert, [rows][cols], row-major.  Exactly one of
 * `base` (single grouped tensor, expert e at base + e*expert_stride elements;
 * PR #6572, MCore-owned parameters, moe_single_grouped_weight) and `table`
 * (per-expert allocations: a DEVICE array of E base pointers; the non-single
 * layout exposed through descriptor tables) is non-NULL.  For the shared
 * expert E == 1 and expert_stride is ignored. */
typedef struct {
  const void* base;
  int64_t expert_stride;     /* elements between experts when `base` is used                */
  const void* const* table;  /* device array of E pointers, or NULL                         */
  int64_t ld;                /* elements between rows                                       */
} moe_mat;

/* A weight operand: logical shape [rows][cols] per expert.  `row_offset`
 * selects the first row inside the storage, so gate (row_offset 0) and up
 * (row_offset I) may alias one combined FC1 tensor [2I][H] (Megatron Core
 * API docs, mok.runtime, _gate_up_weight_arguments: gate/up are zero-copy row
 * views of the combined FC1; logical gate/up offsets inside one payload).
 *
 * BF16: `data` only.
 * MXFP8 (routed only): `data` is the E4M3 payload with blocks of 32 along
 * cols and `scale` its E8M0 bytes [rows][cols/32]; `col_data` is the
 * columnwise payload (same [rows][cols] shape and layout, blocks of 32 along
 * rows) and `col_scale` its E8M0 bytes [rows/32][cols] (PR #8210, review
 * thread on the MXFP8 scale conversion: column scale shape (rows // 32,
 * columns)).  The forward reads the rowwise copy, the backward's data
 * gradient the columnwise copy; `row_offset` must then be a multiple of 32. */
typedef struct {
  int32_t dtype;             /* moe_dtype                                                   */
  int64_t rows, cols;        /* logical per-expert shape                                    */
  int64_t row_offset;        /* first logical row inside the storage                        */
  moe_mat data, scale, col_data, col_scale;
} moe_weight;

/* The six weights in the runtime's argument order (Megatron Core API docs,
 * mok.runtime, _MoKWeightArguments): shared gate [I][H], shared up [I][H],
 * shared down [H][I], routed gate [E][I][H], routed up [E][I][H], routed
 * down [E][H][I].  Shared weights must be BF16 (PR #6572, Supported
 * configurations: shared expert parameters must remain BF16). */
typedef struct {
  moe_weight shared_gate, shared_up, shared_down, routed_gate, routed_up, routed_down;
  moe_weight shared_out_gate;   /* [1][H] BF16, `data.base` only; used with
                                   MOE_FLAG_SHARED_GATE, ignored otherwise */
} moe_weights;

/* A main_grad buffer [rows][cols] per expert, same addressing as moe_mat, in FP32 or
 * BF16 (`dtype`; 0 means FP32).  All six buffers of a call must share one dtype
 * (MOE_ERR_DTYPE otherwise).  Rows are read and written in pieces of 4 elements:
 * `base` (or every table entry) must be 16-byte aligned and `ld` and `expert_stride`
 * multiples of 4 (MOE_ERR_LAYOUT otherwise; table entries live on the device and are
 * not checked).  `base` / `table` point at float or bf16 storage as `dtype` says. */
typedef struct {
  void* base;
  int64_t expert_stride;     /* elements                                                     */
  void* const* table;        /* device array of E pointers, or NULL                         */
  int64_t ld;                /* elements                                                     */
  int64_t row_offset;
  int32_t dtype;             /* 0 or MOE_FP32, or MOE_BF16                                   */
} moe_grad;

/* main_grad buffers in the same six-buffer order (Megatron Core API docs,
 * mok.runtime, _gate_up_main_grad_arguments).  The backward accumulates into all
 * six (PR #6572, Design > Gradient accumulation) with an FP32 GEMM accumulator
 * (PR #8210, review thread on the wgrad accumulation precision): an FP32 main_grad
 * receives main_grad + contribution in FP32; a BF16 main_grad receives the BF16
 * rounding (to nearest even) of main_grad + bf16(contribution), i.e. the call's
 * contribution is rounded to BF16 before a BF16 reduction-store, so the persistent
 * accumulation is BF16. */
typedef struct {
  moe_grad shared_gate, shared_up, shared_down, routed_gate, routed_up, routed_down;
  moe_grad shared_out_gate;     /* [1][H], `base` only, same dtype as the others; used
                                   with MOE_FLAG_SHARED_GATE, ignored otherwise */
} moe_main_grads;
/* In routed-only mode only the three routed buffers are used, and they alone must share
 * one dtype. */

/* Byte offsets of the integer routing state inside `saved` (for tests and
 * callers that want the compacted routing).  All arrays are int32 unless
 * stated.  Offsets are relative, so `saved` may be copied elsewhere. */
typedef struct {
  size_t top_experts;     /* int32 [T][K], -1 for a missing route                            */
  size_t router_weights;  /* float [T][K], probs gathered at top_experts, 0 at -1            */
  size_t counts;          /* int32 [E]                                                       */
  size_t offsets;         /* int32 [E+1], exclusive prefix sum of counts                     */
  size_t slot_of;         /* int32 [T][K], slot of route (t,k) in expert-major order, -1 pad */
  size_t slot_token;      /* int32 [T*K], t*K+k of the route at each slot (first S valid)    */
  size_t status_word;     /* int32: 0, MOE_ERR_ROUTE_OVERFLOW, or (moe_forward_topk)
                             MOE_ERR_ROUTE_INVALID                                          */
} moe_saved_layout;

/* Byte offsets of the MXFP8 activation codes and E8M0 scales inside the workspaces, the
 * inputs the routed FP8 GEMMs are given (for tests that read them back).  Forward workspace
 * (moe_workspace_bytes(p, 0)): x_codes [T][H] and x_scales [T][H/32] (one row per token),
 * h_codes [T*K][I] and h_scales [T*K][I/32] (one row per slot).  Backward workspace:
 * dy_codes [T*K][H] and dy_scales [T*K][H/32] (the BF16 w_tk dy[t] of each slot),
 * dfc1_codes [T*K][2I] and dfc1_scales [T*K][2I/32].  Slot rows at or past the number of
 * valid slots hold nothing.  Blocks of 32 run along the rows; each code is the E4M3
 * rounding (to nearest even) of value * 2^-e, e the smallest exponent in [-127, 127] that
 * brings the block's largest magnitude to at most 448, stored as e + 127.  Returns
 * MOE_ERR_UNSUPPORTED for BF16 routed weights (no staging exists). */
typedef struct {
  size_t x_codes, x_scales, h_codes, h_scales;
  size_t dy_codes, dy_scales, dfc1_codes, dfc1_scales;
} moe_mx_staging_layout;
moe_status moe_mx_staging_view(const moe_problem* p, moe_mx_staging_layout* layout);

/* Bytes of the forward->backward context for this problem (0 on invalid input). */
size_t moe_saved_bytes(const moe_problem* p);

/* Workspace bytes for moe_forward (for_backward = 0) or moe_backward (1). */
size_t moe_workspace_bytes(const moe_problem* p, int for_backward);

/* Fills `layout` with the offsets of the routing state inside `saved`. */
moe_status moe_saved_view(const moe_problem* p, moe_saved_layout* layout);

/* Forward.
 *  hidden       bf16  [T][H]  (device)
 *  probs        float [T][E]  read only where routing_map is non-zero
 *  routing_map  uint8 [T][E]  0/1; at most K non-zero per row.  Converted to a
 *               fixed-width [T][K] table of ascending expert IDs with -1 for a
 *               missing route and the gathered probabilities (PR #6572, Design >
 *               Authoritative routing maps)
 *  out          bf16  [T][H]  overwritten:
 *               out[t] = shared(x_t) + sum_k w_tk * expert_{e_tk}(x_t)
 *               (without the shared(x_t) term in routed-only mode)
 *  saved        moe_saved_bytes(p) bytes, written; pass it to moe_backward
 *  workspace    moe_workspace_bytes(p, 0) bytes of scratch
 */
moe_status moe_forward(const moe_problem* p, const void* hidden, const float* probs,
                       const uint8_t* routing_map, const moe_weights* w, void* out,
                       void* saved, void* workspace, size_t workspace_bytes, void* stream);

/* Forward from the router's fixed-width table (requires MOE_FLAG_TOPK_ROUTING; without
 * it, and moe_forward with it, return MOE_ERR_UNSUPPORTED).
 *  top_experts     int32 [T][K] expert IDs in any order, -1 for a missing route
 *  router_weights  float [T][K] the weight of each listed route (ignored at -1)
 * An ID outside [-1, E) or an ID listed twice in a row is dropped (treated as -1) and
 * sets the status word to MOE_ERR_ROUTE_INVALID.  The layer is the same function as
 * moe_forward on the dense map with routing_map[t][e_tk] = 1 and probs[t][e_tk] =
 * router_weights[t][k].  Other arguments as for moe_forward. */
moe_status moe_forward_topk(const moe_problem* p, const void* hidden, const int32_t* top_experts,
                            const float* router_weights, const moe_weights* w, void* out,
                            void* saved, void* workspace, size_t workspace_bytes, void* stream);

/* Forward that allocates nothing and takes no workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Arguments and results as for moe_forward (the dense routing map; with
 * MOE_FLAG_TOPK_ROUTING it returns MOE_ERR_UNSUPPORTED), computed by the same kernels, so
 * `out` and `saved` are bit-identical to moe_forward's.  The forward's scratch (the MXFP8
 * codes and scales of the routed GEMM inputs, and in recompute mode the forward's
 * activations: moe_workspace_bytes(p, 0) bytes) lives instead in one static device array
 * of MOE_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from its load until the
 * process ends.
 *  Limit: a problem whose forward workspace exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 *  MOE_ERR_WORKSPACE with nothing enqueued.  BF16 routed weights without recompute need no
 *  scratch at any size; MXFP8 routed weights at 4096 tokens, hidden 4096, 96 experts,
 *  top-4, intermediate 1024 need 35 MB.
 *  Sharing: the array used is the current device's, on which `stream` must run.  Every call
 *  on one GPU uses the same array, which keeps the last call's contents; nothing in it has
 *  to start at zero (a kernel reads only bytes written earlier in the same call).  Calls
 *  that overlap on one GPU (several streams or host threads) race on it: the caller
 *  serialises them.
 *  The first call on a device, once its arguments are valid, looks up the array's device
 *  address (hipGetSymbolAddress) and keeps it; no call allocates or frees device memory. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_problem* p, const void* hidden, const float* probs,
                               const uint8_t* routing_map, const moe_weights* w, void* out,
                               void* saved, void* stream);

/* Backward of sum(grad_out * out).
 *  grad_out     bf16  [T][H]
 *  hidden       the same bf16 [T][H] tensor given to moe_forward
 *  saved        the context moe_forward wrote (unchanged since)
 *  grad_hidden  bf16  [T][H]  overwritten (routed terms only in routed-only mode)
 *  grad_probs   float [T][E]  overwritten in full; zero where routing_map was 0
 *               (the router-weight gradient scattered back into the dense
 *               probability tensor: PR #6572, Design > Authoritative routing maps);
 *               with MOE_FLAG_TOPK_ROUTING float [T][K], the gradient of
 *               router_weights, 0 at -1 entries
 *  mg           main_grad buffers (FP32 or BF16, see moe_main_grads), accumulated
 *  workspace    moe_workspace_bytes(p, 1) bytes of scratch
 */
moe_status moe_backward(const moe_problem* p, const void* grad_out, const void* hidden,
                        const moe_weights* w, const void* saved, void* grad_hidden,
                        float* grad_probs, const moe_main_grads* mg, void* workspace,
                        size_t workspace_bytes, void* stream);

/* A static description of a status code. */
const char* moe_status_str(moe_status s);

/* Per-kernel launch timing for measurement.  When enabled, every kernel the
 * library launches is bracketed by HIP events on the caller's stream (the
 * events are created by the library on first use and kept).  Read and reset
 * with moe_kernel_timer_read, which waits for the recorded events.  The
 * timer is process-wide and not thread-safe; it is off by default. */
void moe_kernel_timer_enable(int on);
/* Copies up to `cap` entries: the kernel name, the number of launches timed
 * and their total milliseconds; returns the number of distinct kernels. */
int moe_kernel_timer_read(const char** names, int* launches, double* total_ms, int cap);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
