// Host side of the C ABI declared in include/moe.h: argument validation, the
// layout of the caller-owned `saved` and workspace buffers, and the launch
// sequence on the caller's stream.  Nothing here allocates device memory or
// synchronises with the device.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "common.hpp"
#include "gemm.hpp"
#include "routing.hpp"
#include "rowwise.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Dims {
  int64_t T, H, I, E, K;
  int64_t SM;        // T*K: slot capacity of the routed buffers
  int64_t R;         // SM + T with the shared expert (routed rows, then shared rows), else SM
  int64_t nchunks;
  bool mx;
  bool hs;           // the shared expert is fused in
  bool rc;           // recompute: saved holds the routing state only
  bool tk;           // routing given as the fixed-width [T][K] table
  bool sg;           // the shared expert's output is gated
  float L;           // SwiGLU clamp limit (0: none)
};

Dims dims_of(const moe_problem* p) {
  Dims d;
  d.T = p->tokens; d.H = p->hidden; d.I = p->intermediate; d.E = p->experts; d.K = p->topk;
  d.SM = d.T * d.K;
  d.hs = (p->flags & MOE_FLAG_HAS_SHARED) != 0;
  d.R = d.SM + (d.hs ? d.T : 0);
  d.nchunks = (d.T + kRouteChunk - 1) / kRouteChunk;
  d.mx = p->routed_dtype == MOE_MXFP8_E4M3;
  d.rc = (p->flags & MOE_FLAG_RECOMPUTE) != 0;
  d.tk = (p->flags & MOE_FLAG_TOPK_ROUTING) != 0;
  d.sg = (p->flags & MOE_FLAG_SHARED_GATE) != 0;
  d.L = p->swiglu_limit;
  return d;
}

// The forward's activations the backward reads: the FC1 output ab = [a | b],
// h = silu(a) * b and the unweighted FC2 output y (routed rows, then the shared expert's
// T rows).  Routed FC1 inputs are the hidden-state rows themselves, reached through
// slot_t, so no gathered copy exists.  Placed at the end of `saved`, or in recompute
// mode at the start of the forward and backward workspaces.
struct ActLayout {
  size_t ab, h, y, end;
};

ActLayout act_layout(const Dims& d, size_t o) {
  ActLayout A;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  A.ab = take(2 * d.R * 2 * d.I);
  A.h = take(2 * d.R * d.I);
  A.y = take(2 * d.R * d.H);
  A.end = o;
  return A;
}

// Byte offsets inside `saved`.
struct SavedLayout {
  size_t top, rw, counts, offsets, slot_of, slot_token, status, slot_w, slot_t, gate_s, tile_prefix, chunk_base,
      chunk_counts, chunk_status, total;
  ActLayout act;     // not in recompute mode
};

SavedLayout saved_layout(const Dims& d) {
  SavedLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  L.top = take(4 * d.T * d.K);
  L.rw = take(4 * d.T * d.K);
  L.counts = take(4 * d.E);
  L.offsets = take(4 * (d.E + 1));
  L.slot_of = take(4 * d.T * d.K);
  L.slot_token = take(4 * d.SM);
  L.status = take(4);
  L.slot_w = take(4 * d.SM);
  L.slot_t = take(4 * d.SM);
  L.gate_s = take(d.sg ? 4 * d.T : 0);
  L.tile_prefix = take(4 * (d.E + 2));
  L.chunk_base = take(4 * d.nchunks * d.E);
  L.chunk_counts = take(4 * d.nchunks * d.E);
  L.chunk_status = take(4 * d.nchunks);
  L.act = ActLayout{};
  if (!d.rc) {
    L.act = act_layout(d, o);
    o = L.act.end;
  }
  L.total = o;
  return L;
}

// Backward workspace.  In recompute mode it starts with the activations the backward
// regenerates; y is dead once the dy gather has read it, so the FC1 data gradient dxp
// (the same [R][H] bf16 shape) reuses its bytes, and the forward's MXFP8 staging (xq, xs,
// hq, hs) sits inside the backward's (dyq, dys, dfq, dfs; each at least as large), whose
// first writer runs after the recomputed FC2 has consumed it.
struct BwdLayout {
  size_t dyw, dfc1, dxp, dyq, dys, dfq, dfs, total;
  size_t sdy, gdz, gpart;        // shared output gate: s dy [T][H] bf16, dz [T], partial sums
  ActLayout act;                 // recompute mode only
  size_t fxq, fxs, fhq, fhs;     // recompute mode, MXFP8 only
};

BwdLayout bwd_layout(const Dims& d) {
  BwdLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  L.act = ActLayout{};
  if (d.rc) {
    L.act = act_layout(d, 0);
    o = L.act.end;
  }
  L.dyw = take(2 * d.SM * d.H);
  L.dfc1 = take(2 * d.R * 2 * d.I);
  L.dxp = d.rc ? L.act.y : take(2 * d.R * d.H);
  L.dyq = L.dys = L.dfq = L.dfs = 0;
  if (d.mx) {   // MXFP8 codes + scales of the routed data-gradient GEMM inputs
    L.dyq = take(d.SM * d.H);
    L.dys = take(d.SM * d.H / 32);
    L.dfq = take(d.SM * 2 * d.I);
    L.dfs = take(d.SM * 2 * d.I / 32);
  }
  L.fxq = L.dyq; L.fxs = L.dys; L.fhq = L.dfq; L.fhs = L.dfs;
  L.sdy = L.gdz = L.gpart = 0;
  if (d.sg) {
    L.sdy = take(2 * d.T * d.H);
    L.gdz = take(4 * d.T);
    L.gpart = take(4 * (size_t)kGateChunks * d.H);
  }
  L.total = o;
  return L;
}

// Forward workspace: the activations in recompute mode, then the MXFP8 codes + scales of
// the routed FC1 input (x, one row per token) and FC2 input (h, one row per slot).
struct FwdLayout {
  size_t xq, xs, hq, hs, total;
  ActLayout act;     // recompute mode only
};

FwdLayout fwd_layout(const Dims& d) {
  FwdLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  if (d.rc) {
    L.act = act_layout(d, 0);
    o = L.act.end;
  }
  if (d.mx) {
    L.xq = take(d.T * d.H);
    L.xs = take(d.T * d.H / 32);
    L.hq = take(d.SM * d.I);
    L.hs = take(d.SM * d.I / 32);
  }
  L.total = o > kAlign ? o : kAlign;
  return L;
}

size_t fwd_workspace(const Dims& d) { return fwd_layout(d).total; }

// ---------------------------------------------------------------- validation
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_NULL;
  if (p->tokens < 0 || p->hidden <= 0 || p->intermediate <= 0) return MOE_ERR_SHAPE;
  if (p->hidden % 128 || p->intermediate % 128) return MOE_ERR_SHAPE;
  if (p->experts < 1 || p->experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (p->topk < 1 || p->topk > kMaxTopk || p->topk > p->experts) return MOE_ERR_SHAPE;
  if (p->tokens * (int64_t)p->topk > (int64_t)1 << 30) return MOE_ERR_SHAPE;
  if (p->hidden > (1 << 20) || p->intermediate > (1 << 20)) return MOE_ERR_SHAPE;
  if (p->flags & ~(MOE_FLAG_HAS_SHARED | MOE_FLAG_RECOMPUTE | MOE_FLAG_TOPK_ROUTING | MOE_FLAG_SHARED_GATE))
    return MOE_ERR_UNSUPPORTED;
  if ((p->flags & MOE_FLAG_SHARED_GATE) && !(p->flags & MOE_FLAG_HAS_SHARED)) return MOE_ERR_UNSUPPORTED;
  if (!(p->swiglu_limit >= 0.0f) || p->swiglu_limit > 3.0e38f) return MOE_ERR_UNSUPPORTED;   // NaN, < 0, inf
  if (p->routed_dtype != MOE_BF16 && p->routed_dtype != MOE_MXFP8_E4M3) return MOE_ERR_DTYPE;
  return MOE_OK;
}

moe_status check_mat(const moe_mat& m, int64_t cols, bool routed, int elem_bytes) {
  const bool hb = m.base != nullptr, ht = m.table != nullptr;
  if (!hb && !ht) return MOE_ERR_NULL;
  if (hb && ht) return MOE_ERR_LAYOUT;
  if (!routed && ht) return MOE_ERR_LAYOUT;
  if (m.ld < cols) return MOE_ERR_LAYOUT;
  if ((m.ld * elem_bytes) % 16) return MOE_ERR_LAYOUT;
  if (hb && !aligned16(m.base)) return MOE_ERR_LAYOUT;
  if (hb && routed && (m.expert_stride < 0 || (m.expert_stride * elem_bytes) % 16)) return MOE_ERR_LAYOUT;
  return MOE_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// E8M0 scale matrices are read 4 bytes at a time: row stride and base 4-byte aligned.
moe_status check_scale(const moe_mat& m, int64_t cols) {
  const bool hb = m.base != nullptr, ht = m.table != nullptr;
  if (!hb && !ht) return MOE_ERR_NULL;
  if (hb && ht) return MOE_ERR_LAYOUT;
  if (m.ld < cols || m.ld % 4) return MOE_ERR_LAYOUT;
  if (hb && (!aligned4(m.base) || m.expert_stride < 0 || m.expert_stride % 4)) return MOE_ERR_LAYOUT;
  return MOE_OK;
}

// need_col: the columnwise MXFP8 copy is required (backward).
moe_status check_weight(const moe_weight& w, int64_t rows, int64_t cols, bool routed, int32_t dtype,
                        bool need_col = false) {
  if (w.dtype != dtype) return MOE_ERR_DTYPE;
  if (w.rows != rows || w.cols != cols) return MOE_ERR_SHAPE;
  if (w.row_offset < 0) return MOE_ERR_LAYOUT;
  if (dtype != MOE_MXFP8_E4M3) return check_mat(w.data, cols, routed, 2);
  moe_status s;
  if (w.row_offset % 32 || rows % 32 || cols % 32) return MOE_ERR_LAYOUT;
  if ((s = check_mat(w.data, cols, routed, 1)) != MOE_OK) return s;
  if ((s = check_scale(w.scale, cols / 32)) != MOE_OK) return s;
  if (need_col) {
    if ((s = check_mat(w.col_data, cols, routed, 1)) != MOE_OK) return s;
    if ((s = check_scale(w.col_scale, cols)) != MOE_OK) return s;
  }
  return MOE_OK;
}

moe_status check_weights(const moe_problem* p, const moe_weights* w, bool backward = false) {
  if (!w) return MOE_ERR_NULL;
  const int64_t H = p->hidden, I = p->intermediate;
  moe_status s;
  if (p->flags & MOE_FLAG_HAS_SHARED) {   // shared expert parameters must be BF16
    if ((s = check_weight(w->shared_gate, I, H, false, MOE_BF16)) != MOE_OK) return s;
    if ((s = check_weight(w->shared_up, I, H, false, MOE_BF16)) != MOE_OK) return s;
    if ((s = check_weight(w->shared_down, H, I, false, MOE_BF16)) != MOE_OK) return s;
  }
  if (p->flags & MOE_FLAG_SHARED_GATE) {   // [1][H] BF16, one grouped base
    if ((s = check_weight(w->shared_out_gate, 1, H, false, MOE_BF16)) != MOE_OK) return s;
    if (w->shared_out_gate.row_offset != 0) return MOE_ERR_LAYOUT;
  }
  if ((s = check_weight(w->routed_gate, I, H, true, p->routed_dtype, backward)) != MOE_OK) return s;
  if ((s = check_weight(w->routed_up, I, H, true, p->routed_dtype, backward)) != MOE_OK) return s;
  if ((s = check_weight(w->routed_down, H, I, true, p->routed_dtype, backward)) != MOE_OK) return s;
  return MOE_OK;
}

moe_status check_grad(const moe_grad& g, int64_t cols, bool routed) {
  const bool hb = g.base != nullptr, ht = g.table != nullptr;
  if (!hb && !ht) return MOE_ERR_NULL;
  if (hb && ht) return MOE_ERR_LAYOUT;
  if (!routed && ht) return MOE_ERR_LAYOUT;
  if (g.ld < cols || g.row_offset < 0) return MOE_ERR_LAYOUT;
  if (g.ld % 4 || (hb && (g.expert_stride % 4 || !aligned16(g.base)))) return MOE_ERR_LAYOUT;
  return MOE_OK;
}

bool grad_bf16(const moe_grad& g) { return g.dtype == MOE_BF16; }

moe_status check_grads(const moe_problem* p, const moe_main_grads* g) {
  if (!g) return MOE_ERR_NULL;
  // one dtype for every buffer in use (all six, or the three routed ones in routed-only
  // mode): FP32 (0 or MOE_FP32) or BF16
  const bool hs = (p->flags & MOE_FLAG_HAS_SHARED) != 0;
  const moe_grad* all[6] = {&g->routed_gate, &g->routed_up, &g->routed_down,
                            &g->shared_gate, &g->shared_up, &g->shared_down};
  const int n = hs ? 6 : 3;
  for (int i = 0; i < n; ++i)
    if (all[i]->dtype != 0 && all[i]->dtype != MOE_FP32 && all[i]->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  for (int i = 0; i < n; ++i)
    if (grad_bf16(*all[i]) != grad_bf16(g->routed_gate)) return MOE_ERR_DTYPE;
  const int64_t H = p->hidden, I = p->intermediate;
  moe_status s;
  if (hs) {
    if ((s = check_grad(g->shared_gate, H, false)) != MOE_OK) return s;
    if ((s = check_grad(g->shared_up, H, false)) != MOE_OK) return s;
    if ((s = check_grad(g->shared_down, I, false)) != MOE_OK) return s;
  }
  if (p->flags & MOE_FLAG_SHARED_GATE) {
    const moe_grad& q = g->shared_out_gate;
    if (q.dtype != 0 && q.dtype != MOE_FP32 && q.dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (grad_bf16(q) != grad_bf16(g->routed_gate)) return MOE_ERR_DTYPE;
    if ((s = check_grad(q, H, false)) != MOE_OK) return s;
    if (q.row_offset != 0) return MOE_ERR_LAYOUT;
  }
  if ((s = check_grad(g->routed_gate, H, true)) != MOE_OK) return s;
  if ((s = check_grad(g->routed_up, H, true)) != MOE_OK) return s;
  if ((s = check_grad(g->routed_down, I, true)) != MOE_OK) return s;
  return MOE_OK;
}

MatRef matref(const moe_weight& w, const moe_mat& m, int elem_bytes) {
  MatRef r;
  r.base = static_cast<const uint8_t*>(m.base);
  r.table = reinterpret_cast<const uint8_t* const*>(m.table);
  r.estride_bytes = m.expert_stride * elem_bytes;
  r.ld_bytes = m.ld * elem_bytes;
  r.row_offset = w.row_offset;
  return r;
}

// MXFP8 weight views: the rowwise copy (forward) or the columnwise copy (data gradient);
// a columnwise scale row covers 32 weight rows, so its row offset is row_offset / 32.
MxRef mxref(const moe_weight& w, bool columnwise) {
  MxRef r;
  if (!columnwise) {
    r.data = matref(w, w.data, 1);
    r.scale = matref(w, w.scale, 1);
  } else {
    r.data = matref(w, w.col_data, 1);
    r.scale = matref(w, w.col_scale, 1);
    r.scale.row_offset = w.row_offset / 32;
  }
  return r;
}

GradRef gradref(const moe_grad& g) {
  GradRef r;
  r.base = static_cast<uint8_t*>(g.base);
  r.table = reinterpret_cast<uint8_t* const*>(g.table);
  r.estride = g.expert_stride;
  r.ld = g.ld;
  r.row_offset = g.row_offset;
  return r;
}

// ---------------------------------------------------------------- kernel timer
struct TimedLaunch {
  const char* name;
  hipEvent_t a, b;
};
struct Timer {
  bool on = false;
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> pool;
  std::vector<std::string> names;
  std::vector<int> counts;
  std::vector<double> ms;
  std::mutex mu;
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Timer g_timer;

template <class F>
moe_status launch(const char* name, hipStream_t st, F&& f) {
  hipEvent_t a = nullptr, b = nullptr;
  if (g_timer.on) {
    a = g_timer.get();
    b = g_timer.get();
    if (a) (void)hipEventRecord(a, st);
  }
  f();
  const hipError_t err = hipGetLastError();
  if (g_timer.on && a && b) {
    (void)hipEventRecord(b, st);
    g_timer.pending.push_back({name, a, b});
  }
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

#define MOE_TRY(x)                        \
  do {                                    \
    const moe_status _s = (x);            \
    if (_s != MOE_OK) return _s;          \
  } while (0)

// Token rows per M tile of the token-dimension GEMMs (one value per routed-weight type).
int64_t tok_bm(const Dims& d) { return d.mx ? gemm::bm_of<true>() : gemm::bm_of<false>(); }
int64_t max_mtiles(const Dims& d) {
  const int64_t bm = tok_bm(d);
  return (d.SM + bm - 1) / bm + d.E + (d.hs ? (d.T + bm - 1) / bm : 0);
}
unsigned grid8(int64_t n) { return (unsigned)(((n + 7) / 8) * 8); }
// token-dimension GEMM grid for at most n tiles: each XCD may receive one tile more than
// an even split (the shared and routed tiles are split separately)
unsigned tok_grid(int64_t n) { return grid8(n) + 8; }

// The BF16 token GEMMs take the wide shape set (192 x 128 tiles, two workgroups per CU)
// above this many routed slots per expert on average: a second workgroup's multiplies
// cover each one's waits and epilogue.  At the 4096-token layer (H 4096, I 1024, top-4)
// the step is 0.5-2.6% faster with them from 341 slots per expert up, and 1.4% slower at
// 171 (96 experts), where each weight panel is read by one m-tile and the 192 x 256
// shapes' three-stage weight ring feeds the HBM-bound weight stream better.
#ifndef MOE_WIDE_SLOTS
#define MOE_WIDE_SLOTS 256
#endif
constexpr int64_t kWideSlots = MOE_WIDE_SLOTS;
bool tok_wide(const Dims& d) { return !d.mx && d.SM > kWideSlots * d.E; }

// Weight-gradient launch: the shared expert's tiles first (when present), then E groups
// of routed tiles rounded up to a multiple of 8 blocks (one chunk per XCD).
template <int FC, bool MG16, bool SHORT>
void launch_wgrad_t(const gemm::WgradArgs& a, const Dims& d, hipStream_t st) {
  const int per = gemm::wgrad_tiles_per_group<MG16, SHORT>(a.parts, a.mpart, a.N);
  const dim3 g((d.hs ? per : 0) + grid8((int64_t)d.E * per));
  gemm::launch_wgrad<FC, MG16, SHORT>(g, st, a);
}
// The FP32-main_grad weight gradients take their short-token-loop shape when the routed
// experts average at most this many slots (T K / E).
constexpr int64_t kWgradShortSlots = 256;
template <int FC>
void launch_wgrad(const gemm::WgradArgs& a, const Dims& d, bool mg16, hipStream_t st) {
  if (mg16) launch_wgrad_t<FC, true, false>(a, d, st);
  else if (d.SM <= kWgradShortSlots * d.E) launch_wgrad_t<FC, false, true>(a, d, st);
  else launch_wgrad_t<FC, false, false>(a, d, st);
}

// Pointers of one run of the routed + shared expert forward (F3-F6).
struct FwdPtrs {
  const int32_t *slot_t, *counts, *offsets, *tile_prefix;
  uint16_t *ab, *h, *y;
  uint8_t *xq, *xs, *hq, *hs;   // MXFP8 staging (unused for BF16 routed weights)
};

// FC1 + SwiGLU (routed rows read from x through slot_t: the dispatch gather happens
// in the GEMM's own DMA), FC2; routed and shared expert in the same launches, from the
// routing state already in place.  `again`: the backward's recomputation in
// recompute mode (the same kernels on the same inputs, so the same bits; only the timer
// names differ).
moe_status experts_forward(const Dims& d, const FwdPtrs& P, const uint16_t* x, const moe_weights* w,
                           hipStream_t st, bool again) {
  const int T = (int)d.T, E = (int)d.E, H = (int)d.H, I = (int)d.I;
  // Q: MXFP8 codes of x, one row per token (the routed FC1 input; F3's gather is the
  // FC1 kernel's row addressing)
  if (d.mx) {
    MOE_TRY(launch(again ? "recompute_quantize_x" : "quantize_x", st, [&] {
      hipLaunchKernelGGL(k_quantize_rows, dim3(2048), dim3(kRowThreads), 0, st, x, d.T, H, P.xq, P.xs);
    }));
  }

  gemm::TokArgs ta;
  ta.counts = P.counts;
  ta.offsets = P.offsets;
  ta.tile_prefix = P.tile_prefix;
  ta.T = T; ta.E = E; ta.groups = E + (d.hs ? 1 : 0);
  ta.shared_row0 = d.SM;
  const int64_t mt = max_mtiles(d);

  // F4 + F6: routed and shared FC1 with the SwiGLU epilogue, one launch
  gemm::Fc1Args a1;
  a1.t = ta;
  a1.slot_t = P.slot_t;
  a1.x = x;
  a1.wg = matref(w->routed_gate, w->routed_gate.data, 2);
  a1.wu = matref(w->routed_up, w->routed_up.data, 2);
  a1.sg = matref(w->shared_gate, w->shared_gate.data, 2);
  a1.su = matref(w->shared_up, w->shared_up.data, 2);
  a1.ab = P.ab;
  a1.h = P.h;
  a1.hq = P.hq;   // MXFP8: the epilogue also writes the FC2 input's codes (quantise step Q for h)
  a1.hs = P.hs;
  a1.H = H; a1.I = I;
  a1.limit = d.L;
  a1.mx = gemm::MxOperands{};
  if (d.mx) {
    a1.mx.aq = P.xq;
    a1.mx.as = P.xs;
    a1.mx.b0 = mxref(w->routed_gate, false);
    a1.mx.b1 = mxref(w->routed_up, false);
  }
  MOE_TRY(launch(again ? "recompute_fc1_swiglu" : "fc1_swiglu", st, [&] {
    using S1 = gemm::Shapes<true>::FC1;
    using S0 = gemm::Shapes<false>::FC1;
    using SW = gemm::ShapesWide::FC1;
    if (d.mx) gemm::launch_fc1<true, false>(dim3(tok_grid(mt * (2 * I / S1::TN))), st, a1);
    else if (tok_wide(d)) gemm::launch_fc1<false, true>(dim3(tok_grid(mt * (2 * I / SW::TN))), st, a1);
    else gemm::launch_fc1<false, false>(dim3(tok_grid(mt * (2 * I / S0::TN))), st, a1);
  }));

  // F5 + F6: routed and shared FC2 -> y (unweighted)
  gemm::PlainArgs a2;
  a2.t = ta;
  a2.a_r = P.h;
  a2.a_s = P.h;
  a2.a_s_row0 = d.SM;
  a2.w0 = matref(w->routed_down, w->routed_down.data, 2);
  a2.w1 = a2.w0;
  a2.s0 = matref(w->shared_down, w->shared_down.data, 2);
  a2.s1 = a2.s0;
  a2.ksplit = I;
  a2.c = P.y;
  a2.N = H; a2.K = I;
  a2.mx = gemm::MxOperands{};
  if (d.mx) {
    a2.mx.aq = P.hq;
    a2.mx.as = P.hs;
    a2.mx.b0 = mxref(w->routed_down, false);
    a2.mx.b1 = a2.mx.b0;
  }
  MOE_TRY(launch(again ? "recompute_fc2" : "fc2", st, [&] {
    using S1 = gemm::Shapes<true>::FC2;
    using S0 = gemm::Shapes<false>::FC2;
    using SW = gemm::ShapesWide::FC2;
    if (d.mx) gemm::launch_plain<gemm::KC, true, false>(dim3(tok_grid(mt * ((H + S1::TN - 1) / S1::TN))), st, a2);
    else if (tok_wide(d))
      gemm::launch_plain<gemm::KC, false, true>(dim3(tok_grid(mt * ((H + SW::TN - 1) / SW::TN))), st, a2);
    else gemm::launch_plain<gemm::KC, false, false>(dim3(tok_grid(mt * ((H + S0::TN - 1) / S0::TN))), st, a2);
  }));
  return MOE_OK;
}


}  // namespace

// Scratch of the allocation-free forward (moe_forward_noalloc): one array per GPU, held
// by that GPU from the library's load until the process ends.  In host code this name is
// only a stand-in for the symbol, not a device address: host code reaches the memory
// through the address scratch_address() looks up per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxScratchDevices] = {};

// The device address of the current GPU's `scratch` array, looked up on the first call on
// that GPU (with it current) and kept: every GPU holds its own copy at its own address.
moe_status scratch_address(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

// ================================================================== C ABI
extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or not a supported multiple";
    case MOE_ERR_DTYPE: return "unsupported element type";
    case MOE_ERR_LAYOUT: return "inconsistent layout (strides, alignment, base/table)";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "saved or workspace buffer missing or too small";
    case MOE_ERR_ROUTE_OVERFLOW: return "a routing-map row has more than topk routes";
    case MOE_ERR_HIP: return "a HIP launch failed";
    case MOE_ERR_ROUTE_INVALID: return "a top_experts entry is out of range or repeated in its row";
  }
  return "unknown status";
}

size_t moe_saved_bytes(const moe_problem* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return saved_layout(dims_of(p)).total;
}

size_t moe_workspace_bytes(const moe_problem* p, int for_backward) {
  if (check_problem(p) != MOE_OK) return 0;
  const Dims d = dims_of(p);
  return for_backward ? bwd_layout(d).total : fwd_workspace(d);
}

moe_status moe_saved_view(const moe_problem* p, moe_saved_layout* out) {
  MOE_TRY(check_problem(p));
  if (!out) return MOE_ERR_NULL;
  const SavedLayout L = saved_layout(dims_of(p));
  out->top_experts = L.top;
  out->router_weights = L.rw;
  out->counts = L.counts;
  out->offsets = L.offsets;
  out->slot_of = L.slot_of;
  out->slot_token = L.slot_token;
  out->status_word = L.status;
  return MOE_OK;
}

moe_status moe_mx_staging_view(const moe_problem* p, moe_mx_staging_layout* out) {
  MOE_TRY(check_problem(p));
  if (!out) return MOE_ERR_NULL;
  const Dims d = dims_of(p);
  if (!d.mx) return MOE_ERR_UNSUPPORTED;
  const FwdLayout F = fwd_layout(d);
  const BwdLayout B = bwd_layout(d);
  out->x_codes = F.xq; out->x_scales = F.xs; out->h_codes = F.hq; out->h_scales = F.hs;
  out->dy_codes = B.dyq; out->dy_scales = B.dys; out->dfc1_codes = B.dfq; out->dfc1_scales = B.dfs;
  return MOE_OK;
}

}  // extern "C"

namespace {

// Both forward entry points: the routing is the dense map + probabilities (rmap, probs),
// or the router's fixed-width table (top_in, rw_in).  noalloc: the workspace arguments are
// unused and the forward's scratch is this GPU's static `scratch` array (looked up only
// once every argument has passed validation).
moe_status forward_impl(bool table, const moe_problem* p, const void* hidden, const float* probs,
                        const uint8_t* routing_map, const int32_t* top_in, const float* rw_in,
                        const moe_weights* w, void* out, void* saved, void* workspace,
                        size_t workspace_bytes, void* stream, bool noalloc = false) {
  MOE_TRY(check_problem(p));
  if (((p->flags & MOE_FLAG_TOPK_ROUTING) != 0) != table) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(check_weights(p, w));
  const Dims d = dims_of(p);
  const bool have_routing = d.tk ? (top_in && rw_in) : (probs && routing_map);
  if (d.T > 0 && (!hidden || !have_routing || !out)) return MOE_ERR_NULL;
  if (!saved) return MOE_ERR_WORKSPACE;
  const FwdLayout F = fwd_layout(d);
  if (noalloc) {
    if (F.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  } else if (workspace_bytes < F.total || !workspace) {
    return MOE_ERR_WORKSPACE;
  }
  if ((hidden && !aligned16(hidden)) || (out && !aligned16(out)) || !aligned16(saved) ||
      (!noalloc && !aligned16(workspace)))
    return MOE_ERR_LAYOUT;
  if (noalloc) {
    uint8_t* sp = nullptr;
    MOE_TRY(scratch_address(&sp));
    workspace = sp;
  }
  uint8_t* WS = static_cast<uint8_t*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const SavedLayout L = saved_layout(d);
  uint8_t* S = static_cast<uint8_t*>(saved);
  auto I32 = [&](size_t off) { return reinterpret_cast<int32_t*>(S + off); };
  auto F32 = [&](size_t off) { return reinterpret_cast<float*>(S + off); };
  // activations: in `saved`, or in recompute mode in the workspace
  uint8_t* AB = d.rc ? WS : S;
  const ActLayout A = d.rc ? F.act : L.act;
  auto U16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(AB + off); };

  const int T = (int)d.T, E = (int)d.E, K = (int)d.K, H = (int)d.H;
  const int nch = (int)d.nchunks;

  // F1 compaction (or validation of the router's table), F2 histogram + scan + stable rank
  if (d.tk) {
    MOE_TRY(launch("route_table", st, [&] {
      if (nch > 0)
        hipLaunchKernelGGL(k_route_table, dim3(nch), dim3(kRouteChunk * kMaxTopk), 0, st, top_in, rw_in, T, E, K,
                           I32(L.top), F32(L.rw), I32(L.chunk_counts), I32(L.chunk_status));
    }));
  } else {
    MOE_TRY(launch("route_compact", st, [&] {
      if (nch > 0)
        hipLaunchKernelGGL(k_route_compact, dim3(nch), dim3(256), 0, st, routing_map, probs, T, E, K,
                           I32(L.top), F32(L.rw), I32(L.chunk_counts), I32(L.chunk_status));
    }));
  }
  MOE_TRY(launch("route_scan", st, [&] {
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(kScanThreads), 0, st, I32(L.chunk_counts), nch, E, T, d.hs ? 1 : 0,
                       (int)tok_bm(d), I32(L.chunk_base), I32(L.counts), I32(L.offsets), I32(L.tile_prefix),
                       I32(L.chunk_status), I32(L.status));
  }));
  if (T == 0) return MOE_OK;
  MOE_TRY(launch("route_rank", st, [&] {
    hipLaunchKernelGGL(k_route_rank, dim3(nch), dim3(kRouteChunk * kMaxTopk), 0, st, I32(L.top), F32(L.rw), T, E, K,
                       I32(L.chunk_base), I32(L.offsets), I32(L.slot_of), I32(L.slot_token), I32(L.slot_t),
                       F32(L.slot_w));
  }));
  FwdPtrs P;
  P.slot_t = I32(L.slot_t); P.counts = I32(L.counts); P.offsets = I32(L.offsets);
  P.tile_prefix = I32(L.tile_prefix);
  P.ab = U16(A.ab); P.h = U16(A.h); P.y = U16(A.y);
  P.xq = WS + F.xq; P.xs = WS + F.xs; P.hq = WS + F.hq; P.hs = WS + F.hs;
  MOE_TRY(experts_forward(d, P, static_cast<const uint16_t*>(hidden), w, st, false));

  // F7 combine
  MOE_TRY(launch("combine", st, [&] {
    hipLaunchKernelGGL(k_combine, dim3(T), dim3(kRowThreads), 0, st, P.y, d.hs ? d.SM : -1, H, K,
                       I32(L.slot_of), F32(L.rw), static_cast<uint16_t*>(out), static_cast<const uint16_t*>(hidden),
                       d.sg ? static_cast<const uint16_t*>(w->shared_out_gate.data.base) : (const uint16_t*)nullptr,
                       d.sg ? F32(L.gate_s) : (float*)nullptr);
  }));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_problem* p, const void* hidden, const float* probs,
                       const uint8_t* routing_map, const moe_weights* w, void* out, void* saved,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(false, p, hidden, probs, routing_map, nullptr, nullptr, w, out, saved, workspace,
                      workspace_bytes, stream);
}

moe_status moe_forward_noalloc(const moe_problem* p, const void* hidden, const float* probs,
                               const uint8_t* routing_map, const moe_weights* w, void* out, void* saved,
                               void* stream) {
  return forward_impl(false, p, hidden, probs, routing_map, nullptr, nullptr, w, out, saved, nullptr, 0,
                      stream, true);
}

moe_status moe_forward_topk(const moe_problem* p, const void* hidden, const int32_t* top_experts,
                            const float* router_weights, const moe_weights* w, void* out, void* saved,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(true, p, hidden, nullptr, nullptr, top_experts, router_weights, w, out, saved, workspace,
                      workspace_bytes, stream);
}

moe_status moe_backward(const moe_problem* p, const void* grad_out, const void* hidden,
                        const moe_weights* w, const void* saved, void* grad_hidden, float* grad_probs,
                        const moe_main_grads* mg, void* workspace, size_t workspace_bytes, void* stream) {
  MOE_TRY(check_problem(p));
  MOE_TRY(check_weights(p, w, true));
  MOE_TRY(check_grads(p, mg));
  const Dims d = dims_of(p);
  if (d.T > 0 && (!grad_out || !hidden || !grad_hidden || !grad_probs)) return MOE_ERR_NULL;
  if (!saved) return MOE_ERR_WORKSPACE;
  const BwdLayout B = bwd_layout(d);
  if (!workspace || workspace_bytes < B.total) return MOE_ERR_WORKSPACE;
  if ((grad_out && !aligned16(grad_out)) || (hidden && !aligned16(hidden)) ||
      (grad_hidden && !aligned16(grad_hidden)) || !aligned16(saved) || !aligned16(workspace))
    return MOE_ERR_LAYOUT;
  if (d.T == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const SavedLayout L = saved_layout(d);
  const uint8_t* S = static_cast<const uint8_t*>(saved);
  uint8_t* W = static_cast<uint8_t*>(workspace);
  auto I32 = [&](size_t off) { return reinterpret_cast<const int32_t*>(S + off); };
  auto F32 = [&](size_t off) { return reinterpret_cast<const float*>(S + off); };
  // activations: read from `saved`, or in recompute mode regenerated into the workspace
  const uint8_t* AB = d.rc ? W : S;
  const ActLayout A = d.rc ? B.act : L.act;
  auto U16 = [&](size_t off) { return reinterpret_cast<const uint16_t*>(AB + off); };
  auto WU16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(W + off); };
  const int T = (int)d.T, E = (int)d.E, K = (int)d.K, H = (int)d.H, I = (int)d.I;
  const uint16_t* dy = static_cast<const uint16_t*>(grad_out);
  const uint16_t* x = static_cast<const uint16_t*>(hidden);

  if (d.rc) {   // recompute mode: F3-F6 again from x and the saved routing state
    FwdPtrs P;
    P.slot_t = I32(L.slot_t); P.counts = I32(L.counts); P.offsets = I32(L.offsets);
    P.tile_prefix = I32(L.tile_prefix);
    P.ab = WU16(A.ab); P.h = WU16(A.h); P.y = WU16(A.y);
    P.xq = W + B.fxq; P.xs = W + B.fxs; P.hq = W + B.fhq; P.hs = W + B.fhs;
    MOE_TRY(experts_forward(d, P, x, w, st, true));
  }

  // shared output gate: saved scores, the gated dy rows of the shared expert, dz
  const float* gate_s = d.sg ? F32(L.gate_s) : nullptr;
  float* gdz = d.sg ? reinterpret_cast<float*>(W + B.gdz) : nullptr;
  uint16_t* sdy = d.sg ? WU16(B.sdy) : nullptr;
  const uint16_t* gw = d.sg ? static_cast<const uint16_t*>(w->shared_out_gate.data.base) : nullptr;
  const uint16_t* dy_shared = d.sg ? sdy : dy;   // the shared expert's upstream gradient

  // B1 weighted dy gather (+ Q) + B8 router-probability gradient (dense row, zeros off the map)
  MOE_TRY(launch("gather_dy_dprob", st, [&] {
    if (d.mx)
      hipLaunchKernelGGL(k_gather_dy_dprob<true>, dim3(T), dim3(kRowThreads), 0, st, dy, U16(A.y), H, E, K,
                         I32(L.slot_of), I32(L.top), F32(L.rw), WU16(B.dyw), grad_probs, W + B.dyq, W + B.dys,
                         d.tk ? 0 : 1, d.SM, gate_s, gdz, sdy);
    else
      hipLaunchKernelGGL(k_gather_dy_dprob<false>, dim3(T), dim3(kRowThreads), 0, st, dy, U16(A.y), H, E, K,
                         I32(L.slot_of), I32(L.top), F32(L.rw), WU16(B.dyw), grad_probs, (uint8_t*)nullptr,
                         (uint8_t*)nullptr, d.tk ? 0 : 1, d.SM, gate_s, gdz, sdy);
  }));

  gemm::TokArgs ta;
  ta.counts = I32(L.counts);
  ta.offsets = I32(L.offsets);
  ta.tile_prefix = I32(L.tile_prefix);
  ta.T = T; ta.E = E; ta.groups = E + (d.hs ? 1 : 0);
  ta.shared_row0 = d.SM;
  const int64_t mt = max_mtiles(d);

  // B2 (+B6): FC2 data gradient with the SwiGLU backward epilogue -> dfc1
  gemm::DgradSwigluArgs a3;
  a3.t = ta;
  a3.a_r = WU16(B.dyw);
  a3.a_s = dy_shared;
  a3.wd = matref(w->routed_down, w->routed_down.data, 2);
  a3.sd = matref(w->shared_down, w->shared_down.data, 2);
  a3.ab = U16(A.ab);
  a3.dfc1 = WU16(B.dfc1);
  a3.dfq = W + B.dfq;   // MXFP8: the epilogue also writes the FC1 data-gradient input's codes (Q)
  a3.dfs = W + B.dfs;
  a3.H = H; a3.I = I;
  a3.limit = d.L;
  a3.mx = gemm::MxOperands{};
  if (d.mx) {
    a3.mx.aq = W + B.dyq;
    a3.mx.as = W + B.dys;
    a3.mx.b0 = mxref(w->routed_down, true);
    a3.mx.b1 = a3.mx.b0;
  }
  MOE_TRY(launch("dgrad_fc2_swiglu", st, [&] {
    using S1 = gemm::Shapes<true>::DG2;
    using S0 = gemm::Shapes<false>::DG2;
    using SW = gemm::ShapesWide::DG2;
    if (d.mx) gemm::launch_dgrad_swiglu<true, false>(dim3(tok_grid(mt * ((I + S1::TN - 1) / S1::TN))), st, a3);
    else if (tok_wide(d))
      gemm::launch_dgrad_swiglu<false, true>(dim3(tok_grid(mt * ((I + SW::TN - 1) / SW::TN))), st, a3);
    else gemm::launch_dgrad_swiglu<false, false>(dim3(tok_grid(mt * ((I + S0::TN - 1) / S0::TN))), st, a3);
  }));

  // B3 (+B6): FC1 data gradient -> dxp (routed rows) and the shared rows
  gemm::PlainArgs a4;
  a4.t = ta;
  a4.a_r = WU16(B.dfc1);
  a4.a_s = WU16(B.dfc1);
  a4.a_s_row0 = d.SM;
  a4.w0 = matref(w->routed_gate, w->routed_gate.data, 2);
  a4.w1 = matref(w->routed_up, w->routed_up.data, 2);
  a4.s0 = matref(w->shared_gate, w->shared_gate.data, 2);
  a4.s1 = matref(w->shared_up, w->shared_up.data, 2);
  a4.ksplit = I;
  a4.c = WU16(B.dxp);
  a4.N = H; a4.K = 2 * I;
  a4.mx = gemm::MxOperands{};
  if (d.mx) {
    a4.mx.aq = W + B.dfq;
    a4.mx.as = W + B.dfs;
    a4.mx.b0 = mxref(w->routed_gate, true);
    a4.mx.b1 = mxref(w->routed_up, true);
  }
  MOE_TRY(launch("dgrad_fc1", st, [&] {
    using S1 = gemm::Shapes<true>::DG1;
    using S0 = gemm::Shapes<false>::DG1;
    using SW = gemm::ShapesWide::DG1;
    if (d.mx) gemm::launch_plain<gemm::RC, true, false>(dim3(tok_grid(mt * ((H + S1::TN - 1) / S1::TN))), st, a4);
    else if (tok_wide(d))
      gemm::launch_plain<gemm::RC, false, true>(dim3(tok_grid(mt * ((H + SW::TN - 1) / SW::TN))), st, a4);
    else gemm::launch_plain<gemm::RC, false, false>(dim3(tok_grid(mt * ((H + S0::TN - 1) / S0::TN))), st, a4);
  }));

  // B7 dx combine
  MOE_TRY(launch("dx_combine", st, [&] {
    hipLaunchKernelGGL(k_dx_combine, dim3(T), dim3(kRowThreads), 0, st, WU16(B.dxp), d.hs ? d.SM : -1, H, K,
                       I32(L.slot_of), static_cast<uint16_t*>(grad_hidden), gw, (const float*)gdz);
  }));

  // B4 (+B6): FC2 weight gradient: main_grad_down[e] += dyw^T h
  gemm::WgradArgs a5;
  a5.counts = I32(L.counts);
  a5.offsets = I32(L.offsets);
  a5.T = T; a5.E = E; a5.has_shared = d.hs ? 1 : 0;
  a5.a_r = WU16(B.dyw); a5.a_s = dy_shared; a5.lda = H; a5.a_s_row0 = 0;
  a5.b_r = U16(A.h); a5.b_s = U16(A.h); a5.ldb = I; a5.b_s_row0 = d.SM;
  a5.b_map = nullptr;
  a5.g_lo = gradref(mg->routed_down); a5.g_hi = a5.g_lo;
  a5.s_lo = gradref(mg->shared_down); a5.s_hi = a5.s_lo;
  a5.parts = 1; a5.mpart = H;
  a5.N = I;
  MOE_TRY(launch("wgrad_fc2", st, [&] { launch_wgrad<2>(a5, d, grad_bf16(mg->routed_gate), st); }));

  // B5 (+B6): FC1 weight gradient: main_grad_{gate,up}[e] += dfc1^T x[slot_t]
  gemm::WgradArgs a6;
  a6.counts = I32(L.counts);
  a6.offsets = I32(L.offsets);
  a6.T = T; a6.E = E; a6.has_shared = d.hs ? 1 : 0;
  a6.a_r = WU16(B.dfc1); a6.a_s = WU16(B.dfc1); a6.lda = 2 * (int64_t)I; a6.a_s_row0 = d.SM;
  a6.b_r = x; a6.b_s = x; a6.ldb = H; a6.b_s_row0 = 0;
  a6.b_map = I32(L.slot_t);   // routed rows of x through the slot's token
  a6.g_lo = gradref(mg->routed_gate); a6.g_hi = gradref(mg->routed_up);
  a6.s_lo = gradref(mg->shared_gate); a6.s_hi = gradref(mg->shared_up);
  a6.parts = 2; a6.mpart = I;
  a6.N = H;
  MOE_TRY(launch("wgrad_fc1", st, [&] { launch_wgrad<1>(a6, d, grad_bf16(mg->routed_gate), st); }));

  // shared output gate's weight: main_grad += sum_t dz[t] x[t]
  if (d.sg) {
    float* part = reinterpret_cast<float*>(W + B.gpart);
    MOE_TRY(launch("gate_wgrad", st, [&] {
      hipLaunchKernelGGL(k_gate_wgrad_partial, dim3((H + 511) / 512, kGateChunks), dim3(256), 0, st, x,
                         (const float*)gdz, T, H, part);
      hipLaunchKernelGGL(k_gate_wgrad_final, dim3((H + 255) / 256), dim3(256), 0, st, (const float*)part, H,
                         static_cast<uint8_t*>(mg->shared_out_gate.base), grad_bf16(mg->routed_gate) ? 1 : 0);
    }));
  }
  return MOE_OK;
}

void moe_kernel_timer_enable(int on) { g_timer.on = on != 0; }

int moe_kernel_timer_read(const char** names, int* launches, double* total_ms, int cap) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  for (auto& tl : g_timer.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(tl.b) == hipSuccess && hipEventElapsedTime(&ms, tl.a, tl.b) == hipSuccess) {
      size_t i = 0;
      for (; i < g_timer.names.size(); ++i)
        if (g_timer.names[i] == tl.name) break;
      if (i == g_timer.names.size()) {
        g_timer.names.emplace_back(tl.name);
        g_timer.counts.push_back(0);
        g_timer.ms.push_back(0.0);
      }
      g_timer.counts[i] += 1;
      g_timer.ms[i] += ms;
    }
    g_timer.pool.push_back(tl.a);
    g_timer.pool.push_back(tl.b);
  }
  g_timer.pending.clear();
  const int n = (int)g_timer.names.size();
  for (int i = 0; i < n && i < cap; ++i) {
    if (names) names[i] = g_timer.names[i].c_str();
    if (launches) launches[i] = g_timer.counts[i];
    if (total_ms) total_ms[i] = g_timer.ms[i];
  }
  for (int i = 0; i < n; ++i) {   // the totals restart; the name strings stay valid until the next read
    g_timer.counts[i] = 0;
    g_timer.ms[i] = 0.0;
  }
  return n;
}

}  // extern "C"
