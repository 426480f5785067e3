"""Oracle for the post-router MoE layer: plain, slow, obviously correct, CPU, fp64.

TEST INFRASTRUCTURE ONLY.  Only tests/, the package's smoke() entry and the
benchmark's cpu_baseline leg may import or run this module; the HIP library
never calls it and shares no code with it.

What the layer computes (Megatron-LM PR #6572, Summary and Design: the backend
replaces the post-router path, meaning dispatch, routed and shared expert
computation, and combine; Megatron Core API docs, mok.backend,
MoKMegakernel.forward(hidden_states, probs, routing_map) returns an output of
the hidden states' shape):

    out[t] = FFN_shared(x_t) + sum_{k : e_tk != -1} w_tk * FFN_{e_tk}(x_t)
    FFN_W(x) = W_down (silu(W_gate x) * (W_up x)),   silu(z) = z / (1 + exp(-z))

with the fixed-width routing table (e_tk, w_tk) produced from the dense
routing map as described in PR #6572, Design > Authoritative routing maps.

Precision: inputs are the exact stored bits (BF16, or E4M3 payload times E8M0
block scale) decoded to float64; all arithmetic is float64.  The oracle does
not model any rounding the fast path applies to intermediate activations.

Readings of points the pages leave open:
  * expert IDs in a table row are ascending, valid IDs first, -1 trailing;
    the gathered probability at a -1 slot is 0;
  * a row with more than topk routes is invalid input (raises);
  * inside an expert's segment, routed (token, k) pairs are ordered by
    ascending token;
  * FC1 holds the gate rows [0, I) then the up rows [I, 2I);
  * the shared expert has weight 1 and no output gate;
  * routed-only mode (Weights with shared=None; PR #8210, Summary and the review
    thread on TP for the shared expert, name it as a follow-up that lets the
    caller run the shared expert itself) drops the FFN_shared term from out and
    from every gradient, and yields no shared weight gradient;
  * grad_probs is the full gradient of the dense probs tensor (zero off the
    map); main_grad receives the weight gradient by accumulation (+=), in FP32,
    or for a BF16 main_grad as described in main_grad_after;
  * MXFP8 forward uses the rowwise copy, dgrad the columnwise copy;
  * a router's fixed-width table (the runtime's input form) lists each expert at most
    once per row, in any order, with -1 anywhere; the weight at -1 is ignored.  Its
    layer is the dense-map layer with the table scattered into map and probs, and its
    probability gradient is that of router_weights ([T, K], 0 at -1).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_decode", "bf16_round", "e4m3_round", "mx_block_exponent", "mx_quantize", "main_grad_after", "e4m3_decode", "e8m0_decode", "mxfp8_decode_rowwise",
    "mxfp8_decode_colwise", "compact_routing", "dispatch_index", "silu", "dsilu",
    "swiglu_ffn", "Weights", "moe_forward", "moe_forward_f64", "moe_backward",
    "moe_backward_f64", "RouteOverflow", "RouteInvalid", "check_table", "moe_forward_table",
    "moe_backward_table", "shared_gate_score", "swiglu_clamped",
]


class RouteOverflow(ValueError):
    """A routing-map row has more true entries than the fixed table width."""


class RouteInvalid(ValueError):
    """A top_experts entry outside [-1, E), or an expert listed twice in one row."""


# ----------------------------------------------------------------------------------
# storage decoding
# ----------------------------------------------------------------------------------
def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float64: a bfloat16 is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), returned as
    float64.  A bfloat16 has 8 significant bits and float32's exponent range, so the
    spacing of representable values near |v| in [2^k, 2^(k+1)) is 2^(k-7), and 2^-133
    below 2^-126."""
    v = np.asarray(v, dtype=np.float64)
    m, ex = np.frexp(v)                       # |v| = |m| 2^ex, |m| in [0.5, 1)
    ulp = np.ldexp(1.0, np.maximum(ex - 8, -133))
    return np.round(v / ulp) * ulp            # np.round rounds halves to even


def main_grad_after(before: np.ndarray, dW: np.ndarray, dtype: str) -> np.ndarray:
    """main_grad after one backward call (PR #8210, review thread on the wgrad
    accumulation precision): FP32 main_grad receives before + dW; BF16 main_grad
    receives the BF16 rounding of before + (dW rounded to BF16): the contribution is
    rounded to BF16 before a BF16 reduction-store."""
    if dtype == "fp32":
        return before + dW
    if dtype == "bf16":
        return bf16_round(before + bf16_round(dW))
    raise ValueError(dtype)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN codes -> float64 (the payload format of MXFP8 weights).

    sign s, exponent field f (4 bits, bias 7), mantissa m (3 bits):
      f >= 1 : (-1)^s * 2^(f-7) * (1 + m/8)
      f == 0 : (-1)^s * 2^-6 * (m/8)              (subnormal)
      f == 15 and m == 7 : NaN (the format has no infinities)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    f = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(f == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, f - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((f == 15) & (m == 7), np.nan, val)


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale byte b -> 2^(b - 127); b == 255 is NaN."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


_E4M3_TABLE = e4m3_decode(np.arange(256, dtype=np.uint8))   # the closed form above, tabulated
_E8M0_TABLE = e8m0_decode(np.arange(256, dtype=np.uint8))


def e4m3_round(u) -> np.ndarray:
    """Round to the nearest E4M3 (OCP E4M3FN) value, ties to even, for |u| <= 448: 3
    fraction bits, exponents down to -6, then subnormals spaced 2^-9."""
    u = np.asarray(u, dtype=np.float64)
    _, ex = np.frexp(u)                       # |u| = f 2^ex, f in [0.5, 1)
    ulp = np.ldexp(1.0, np.maximum(ex - 4, -9))
    return np.round(u / ulp) * ulp


def mx_block_exponent(amax) -> np.ndarray:
    """E8M0 exponent of an MX block: the smallest e in [-127, 127] with amax 2^-e <= 448,
    E4M3's largest finite magnitude (-127 for an all-zero block)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = ex.astype(np.int64) - 9               # 2^(ex-1) <= amax < 2^ex, and 448 < 2^9
    for _ in range(3):                        # the smallest e meeting the bound
        e = np.where(np.ldexp(amax, -e) > 448.0, e + 1, e)
        e = np.where(np.ldexp(amax, -(e - 1)) <= 448.0, e - 1, e)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127)


def mx_quantize(v) -> np.ndarray:
    """The MXFP8 value of v along its last axis (blocks of 32 sharing one E8M0 scale, each
    element rounded to E4M3): quantise then decode, as the recipe does to the FP8
    GEMMs' activation inputs (PR #6572, Supported configurations: MXFP8 routed experts)."""
    v = np.asarray(v, dtype=np.float64)
    b = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    e = mx_block_exponent(np.abs(b).max(axis=-1))[..., None]
    return (e4m3_round(np.ldexp(b, -e)) * np.ldexp(1.0, e)).reshape(v.shape)


def mxfp8_decode_rowwise(payload: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """W[r, c] = E4M3(payload[r, c]) * E8M0(scale[r, c // 32])."""
    R, C = payload.shape
    assert scale.shape == (R, C // 32), (scale.shape, (R, C // 32))
    out = _E4M3_TABLE[payload].reshape(R, C // 32, 32)
    out *= _E8M0_TABLE[scale][:, :, None]
    return out.reshape(R, C)


def mxfp8_decode_colwise(payload: np.ndarray, colscale: np.ndarray) -> np.ndarray:
    """W[r, c] = E4M3(payload[r, c]) * E8M0(colscale[r // 32, c]); the column
    scale has shape (rows // 32, columns) (Megatron-LM PR #8210, review thread
    on the per-expert MXFP8 scale conversion)."""
    R, C = payload.shape
    assert colscale.shape == (R // 32, C), (colscale.shape, (R // 32, C))
    out = _E4M3_TABLE[payload].reshape(R // 32, 32, C)
    out *= _E8M0_TABLE[colscale][:, None, :]
    return out.reshape(R, C)


# ----------------------------------------------------------------------------------
# routing: dense map -> fixed-width table -> expert-contiguous dispatch order
# ----------------------------------------------------------------------------------
def compact_routing(routing_map: np.ndarray, probs: np.ndarray, topk: int):
    """Dense routing map -> fixed-width expert-ID table with gathered probabilities.

    Megatron-LM PR #6572, Design > Authoritative routing maps: the dense map is
    converted to a fixed-width representation and the router probabilities at
    those routes are gathered; a missing route is expert ID -1, so a token with
    fewer than topk routes keeps exactly its routing decisions.

    Returns top_experts int32 [T, K] and router_weights [T, K] in probs' dtype
    (a copy of probs at the listed routes, 0 at -1 slots).
    """
    T, E = routing_map.shape
    top = np.full((T, topk), -1, dtype=np.int32)
    rw = np.zeros((T, topk), dtype=np.asarray(probs).dtype)
    for t in range(T):
        listed = [e for e in range(E) if routing_map[t, e]]
        if len(listed) > topk:
            raise RouteOverflow(f"token {t} has {len(listed)} routes > topk={topk}")
        for k, e in enumerate(listed):
            top[t, k] = e
            rw[t, k] = probs[t, e]
    return top, rw


def check_table(top_experts: np.ndarray, num_experts: int) -> None:
    """A router's fixed-width table as the runtime consumes it (Megatron Core API docs,
    mok.runtime, _MoKAutograd.forward takes top_experts and router_weights): every entry
    is an expert ID in [0, E) or -1 for a missing route, and a row names an expert at
    most once (a token has one decision per expert, as in the dense map)."""
    for t, row in enumerate(np.asarray(top_experts)):
        ids = [int(e) for e in row]
        for e in ids:
            if e < -1 or e >= num_experts:
                raise RouteInvalid(f"token {t}: expert id {e} outside [-1, {num_experts})")
        valid = [e for e in ids if e >= 0]
        if len(valid) != len(set(valid)):
            raise RouteInvalid(f"token {t}: an expert is listed twice")


def dispatch_index(top_experts: np.ndarray, num_experts: int):
    """Token dispatch on one device: the permutation of routed (token, k) pairs
    into expert-contiguous segments (PR #6572 Summary: "dispatch").

    counts[e]     number of (t, k) with top_experts[t, k] == e
    offsets[e]    exclusive prefix sum of counts (offsets[E] = S, all valid slots)
    slot_of[t,k]  offsets[e] + (number of earlier tokens t' < t routed to e); -1 at pads
    slot_token[s] t * K + k of the pair placed at slot s
    """
    T, K = top_experts.shape
    counts = np.zeros(num_experts, dtype=np.int32)
    for t in range(T):
        for k in range(K):
            e = int(top_experts[t, k])
            if e >= 0:
                counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    for e in range(num_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    S = int(offsets[num_experts])
    slot_of = np.full((T, K), -1, dtype=np.int32)
    slot_token = np.full(S, -1, dtype=np.int32)
    seen = np.zeros(num_experts, dtype=np.int32)
    for t in range(T):                      # ascending token order inside each expert
        for k in range(K):
            e = int(top_experts[t, k])
            if e >= 0:
                s = offsets[e] + seen[e]
                seen[e] += 1
                slot_of[t, k] = s
                slot_token[s] = t * K + k
    return counts, offsets, slot_of, slot_token


# ----------------------------------------------------------------------------------
# one SwiGLU expert
# ----------------------------------------------------------------------------------
def silu(z):
    return z / (1.0 + np.exp(-z))


def dsilu(z):
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def swiglu_ffn(X, Wg, Wu, Wd, limit=0.0):
    """Rows of X through one SwiGLU expert: a = X Wg^T, b = X Wu^T,
    h = silu(a) * b, y = h Wd^T (with a clamp limit L > 0: see swiglu_clamped).
    Returns (a, b, h, y)."""
    a = X @ Wg.T
    b = X @ Wu.T
    h, _, _ = swiglu_clamped(a, b, limit)
    y = h @ Wd.T
    return a, b, h, y


def swiglu_clamped(a, b, limit=0.0):
    """h = silu(a) b and its partial derivatives dh/da, dh/db.

    With a clamp limit L > 0, the reading of the SwiGLU clamp (PR #8210 passes MCore's
    activation_func_clamp_value to the backend as swiglu_limit; the pages give no
    formula): the gate pre-activation is clamped from above and the linear one to
    [-L, L] before the product, h = silu(min(a, L)) clamp(b, -L, L); a clamped input
    passes no gradient, an input on a bound still passes it (the gradient of a clamp
    inside its closed bounds).  Whether an input is clamped is decided on its exact
    value.  L = 0: no clamp."""
    if limit and limit > 0:
        a_hi = a > limit
        b_out = np.abs(b) > limit
        ac = np.where(a_hi, limit, a)
        bc = np.where(b_out, np.sign(b) * limit, b)
        h = silu(ac) * bc
        dha = bc * dsilu(ac) * ~a_hi
        dhb = silu(ac) * ~b_out
        return h, dha, dhb
    return silu(a) * b, b * dsilu(a), silu(a)


def shared_gate_score(x, g):
    """The shared expert's output gate, one scalar per token: sigmoid(x_t . g).

    Reading of the shared-output gate (named on the pages as MCore's optional
    shared-expert output gate, PR #6572 Supported configurations, and as the runtime's
    shared_output_gate_weight argument, Megatron Core API docs, mok.runtime,
    _MoKAutograd.forward; its formula is not given there): a weight vector g [H] whose
    sigmoid score per token scales the shared expert's output.
    """
    return 1.0 / (1.0 + np.exp(-(np.asarray(x, dtype=np.float64) @ g)))


def _routed_ffn(X, Wg, Wu, Wd, weights):
    """One routed expert's forward on rows X: (a, b, h, y), with the MXFP8 activation
    inputs when weights.mx_activations (FC1 reads MXFP8 x, FC2 MXFP8 of the BF16 h)."""
    if not weights.mx_activations:
        return swiglu_ffn(X, Wg, Wu, Wd, weights.swiglu_limit)
    Xq = mx_quantize(X)
    a = Xq @ Wg.T
    b = Xq @ Wu.T
    h, _, _ = swiglu_clamped(a, b, weights.swiglu_limit)
    y = mx_quantize(bf16_round(h)) @ Wd.T
    return a, b, h, y


def _routed_dgrad_in(v, weights):
    """A data-gradient GEMM's activation input (w dy, or dfc1 = [da | db]): MXFP8 of its
    BF16 rounding when weights.mx_activations, else itself."""
    return mx_quantize(bf16_round(v)) if weights.mx_activations else v


class Weights:
    """Float64 views of the six weights, in the runtime's argument order
    (Megatron Core API docs, mok.runtime, _MoKWeightArguments: shared gate,
    shared up, shared down, routed gate, routed up, routed down).

    shared      : (Wg [I,H], Wu [I,H], Wd [H,I]), or None in routed-only mode
    shared_gate : the shared expert's output gate weight g [H], or None (no gate)
    swiglu_limit: the SwiGLU clamp limit L of every expert (0: none; swiglu_clamped)
    mx_activations: the routed experts' FP8 GEMMs also take their activation inputs in
                  MXFP8 (x for FC1, the BF16 h for FC2, the BF16 w dy and dfc1 for the
                  data gradients), as the MXFP8 recipe does; the weight gradients keep
                  their operands in full precision
    routed(e)   : (Wg, Wu, Wd) as used by the forward
    routed_t(e) : (Wg, Wu, Wd) as used by dgrad (columnwise decode for MXFP8)

    Construct with `from_bits` from the stored payloads; routed experts are
    decoded on demand, one at a time.
    """

    def __init__(self, shared, routed_fn, routed_dgrad_fn=None, shared_gate=None, swiglu_limit=0.0,
                 mx_activations=False):
        self.shared = shared
        self.swiglu_limit = float(swiglu_limit)
        self.mx_activations = bool(mx_activations)
        self.shared_gate = None if shared_gate is None else np.asarray(shared_gate, dtype=np.float64)
        self._routed = routed_fn
        self._routed_t = routed_dgrad_fn or routed_fn

    def routed(self, e):
        return self._routed(e)

    def routed_t(self, e):
        return self._routed_t(e)

    @staticmethod
    def from_bits(inter: int, shared_fc1, shared_fc2, routed_getter, routed_dtype: str, shared_gate=None,
                  swiglu_limit=0.0, mx_activations=False):
        """shared_fc1 u16 [2I, H], shared_fc2 u16 [H, I]; routed_getter(e) -> dict of
        bits (see moe_inputs.routed_expert).  Gate = FC1 rows [0, I), up = rows [I, 2I)
        (Megatron Core API docs, mok.runtime, _gate_up_weight_arguments: gate and up
        are row views of the combined FC1)."""
        I = inter
        shared = None
        gate = None if shared_gate is None else bf16_decode(np.asarray(shared_gate).reshape(-1))
        if shared_fc1 is not None:
            s1 = bf16_decode(shared_fc1)
            s2 = bf16_decode(shared_fc2)
            shared = (s1[:I], s1[I:2 * I], s2)

        if routed_dtype == "bf16":
            def fwd(e):
                d = routed_getter(e)
                w1 = bf16_decode(d["fc1"])
                return w1[:I], w1[I:2 * I], bf16_decode(d["fc2"])
            return Weights(shared, fwd, shared_gate=gate, swiglu_limit=swiglu_limit)

        def fwd(e):
            d = routed_getter(e)
            w1 = mxfp8_decode_rowwise(d["fc1"], d["fc1_s"])
            return w1[:I], w1[I:2 * I], mxfp8_decode_rowwise(d["fc2"], d["fc2_s"])

        def bwd(e):
            d = routed_getter(e)
            w1 = mxfp8_decode_colwise(d["fc1_c"], d["fc1_cs"])
            return w1[:I], w1[I:2 * I], mxfp8_decode_colwise(d["fc2_c"], d["fc2_cs"])
        return Weights(shared, fwd, bwd, shared_gate=gate, swiglu_limit=swiglu_limit,
                       mx_activations=mx_activations)


# ----------------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------------
def _routes_by_expert(top_experts, router_weights, tokens, num_experts):
    """For each expert, the (token, k, weight) triples among `tokens` routed to it."""
    by = [[] for _ in range(num_experts)]
    for t in tokens:
        for k in range(top_experts.shape[1]):
            e = int(top_experts[t, k])
            if e >= 0:
                by[e].append((t, k, float(router_weights[t, k])))
    return by


def moe_forward(x_bits, probs, routing_map, topk, weights: Weights, tokens=None):
    """out rows for `tokens` (all tokens when None), float64 [len(tokens), H],
    from BF16 hidden-state bits."""
    T = routing_map.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    return moe_forward_f64(bf16_decode(x_bits[tokens]), probs, routing_map, topk, weights, tokens)


def moe_forward_f64(x, probs, routing_map, topk, weights: Weights, tokens=None):
    """The forward on float64 hidden states x [len(tokens), H] (rows of `tokens`).

    out[t] = FFN_shared(x_t) + sum over valid routes of w_tk * FFN_{e_tk}(x_t)
    (shared expert weight 1, no output gate: Megatron-LM PR #6572, Supported
    configurations, the shared output gate is not supported).  Without a shared
    expert (routed-only mode) the first term is absent.
    """
    T, E = routing_map.shape
    top, rw = compact_routing(routing_map, probs, topk)
    return _forward_table_f64(x, top, rw, E, weights, tokens)


def moe_forward_table(x_bits, top_experts, router_weights, num_experts, weights: Weights, tokens=None):
    """The forward from the router's fixed-width table (top_experts int [T, K] in any
    order, -1 for a missing route; router_weights [T, K], ignored at -1): out rows for
    `tokens` from BF16 hidden-state bits.  The same function as moe_forward on the dense
    map with routing_map[t, e_tk] = 1 and probs[t, e_tk] = router_weights[t, k]."""
    check_table(top_experts, num_experts)
    T = np.asarray(top_experts).shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    return _forward_table_f64(bf16_decode(x_bits[tokens]), top_experts, router_weights, num_experts,
                              weights, tokens)


def _forward_table_f64(x, top, rw, E, weights: Weights, tokens=None):
    T = np.asarray(top).shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    x = np.asarray(x, dtype=np.float64)
    pos = {int(t): i for i, t in enumerate(tokens)}
    if weights.shared is not None:
        _, _, _, out = swiglu_ffn(x, *weights.shared, weights.swiglu_limit)
        if weights.shared_gate is not None:
            out = shared_gate_score(x, weights.shared_gate)[:, None] * out
    else:
        out = np.zeros_like(x)
    for e, lst in enumerate(_routes_by_expert(top, rw, tokens, E)):
        if not lst:
            continue
        rows = np.array([pos[t] for t, _, _ in lst])
        w = np.array([w for _, _, w in lst])
        _, _, _, y = _routed_ffn(x[rows], *weights.routed(e), weights)
        for j, r in enumerate(rows):     # fixed order; np.add.at would also do
            out[r] += w[j] * y[j]
    return out


def moe_backward(dy_bits, x_bits, probs, routing_map, topk, weights: Weights,
                 tokens=None, experts=None, shared_grads=True):
    """moe_backward_f64 on BF16 bits of dy and x."""
    return moe_backward_f64(bf16_decode(dy_bits), bf16_decode(x_bits), probs, routing_map,
                            topk, weights, tokens, experts, shared_grads)


def moe_backward_f64(dy_all, x_all, probs, routing_map, topk, weights: Weights,
                     tokens=None, experts=None, shared_grads=True):
    """Gradients of sum(dy * out) with respect to x, probs and the six weights.

    Returns dict:
      dx      float64 [len(tokens), H]        rows for `tokens` (all when None)
      dprobs  float64 [len(tokens), E]        zero where routing_map is false
      dW      {e: (dWg, dWu, dWd)} for e in `experts` (all when None), computed from
              every token routed to e;  "shared": (dWg, dWu, dWd) when shared_grads
              and the layer has a shared expert; "shared_out_gate": dg [H] when it
              also has the output gate

    Per route (t, k) to expert e with weight w, g = dy[t]:
      a = Wg x, b = Wu x, h = silu(a) b, y = Wd h
      dprobs[t, e] = g . y
      gh = w Wd^T g ; da = gh * b * silu'(a) ; db = gh * silu(a)
      dx[t] += Wg^T da + Wu^T db
      dWd += w g h^T ; dWg += da x^T ; dWu += db x^T
    and the shared expert likewise with w = 1 and no probability gradient.
    The weight gradients are what the caller's main_grad receives by
    accumulation (Megatron-LM PR #6572, Design > Gradient accumulation; PR #8210,
    review thread on the wgrad accumulation precision).
    """
    T, E = routing_map.shape
    top, rw = compact_routing(routing_map, probs, topk)
    return _backward_table_f64(dy_all, x_all, top, rw, E, weights, tokens, experts, shared_grads)


def moe_backward_table(dy_bits, x_bits, top_experts, router_weights, num_experts, weights: Weights,
                       tokens=None, experts=None, shared_grads=True):
    """moe_backward for the router's fixed-width table: as moe_backward_f64, except that
    "dprobs" is the gradient of router_weights, float64 [len(tokens), K], 0 at -1 entries.
    A token names an expert at most once, so it is the dense gradient read at
    (t, top_experts[t, k])."""
    check_table(top_experts, num_experts)
    top = np.asarray(top_experts)
    g = _backward_table_f64(bf16_decode(dy_bits), bf16_decode(x_bits), top, router_weights, num_experts,
                            weights, tokens, experts, shared_grads)
    T, K = top.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    dense = g["dprobs"]
    tab = np.zeros((len(tokens), K))
    for i, t in enumerate(tokens):
        for k in range(K):
            e = int(top[t, k])
            if e >= 0:
                tab[i, k] = dense[i, e]
    g["dprobs"] = tab
    return g


def _backward_table_f64(dy_all, x_all, top, rw, E, weights: Weights, tokens=None, experts=None,
                        shared_grads=True):
    T = np.asarray(top).shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    experts = range(E) if experts is None else experts

    x_all = np.asarray(x_all, dtype=np.float64)
    dy_all = np.asarray(dy_all, dtype=np.float64)

    # --- token-side gradients for the requested tokens ---
    x = x_all[tokens]
    g = dy_all[tokens]
    pos = {int(t): i for i, t in enumerate(tokens)}
    dx = np.zeros_like(x)
    dprobs = np.zeros((len(tokens), E))

    if weights.shared is not None:
        Wg, Wu, Wd = weights.shared
        a, b, h, ys = swiglu_ffn(x, Wg, Wu, Wd, weights.swiglu_limit)
        _, dha, dhb = swiglu_clamped(a, b, weights.swiglu_limit)
        gs = g
        if weights.shared_gate is not None:
            # out_t = s_t u_t: the shared expert sees s_t dy_t; s_t itself gets dy_t . u_t
            sc = shared_gate_score(x, weights.shared_gate)
            dz = sc * (1.0 - sc) * np.sum(g * ys, axis=1)
            dx += dz[:, None] * weights.shared_gate[None, :]
            gs = sc[:, None] * g
        gh = gs @ Wd
        da = gh * dha
        db = gh * dhb
        dx += da @ Wg + db @ Wu

    for e, lst in enumerate(_routes_by_expert(top, rw, tokens, E)):
        if not lst:
            continue
        rows = np.array([pos[t] for t, _, _ in lst])
        w = np.array([w for _, _, w in lst])
        Wg, Wu, Wd = weights.routed(e)
        a, b, h, y = _routed_ffn(x[rows], Wg, Wu, Wd, weights)
        _, dha, dhb = swiglu_clamped(a, b, weights.swiglu_limit)
        dprobs[rows, e] = np.sum(g[rows] * y, axis=1)
        Tg, Tu, Td = weights.routed_t(e)
        gh = _routed_dgrad_in(w[:, None] * g[rows], weights) @ Td
        da = gh * dha
        db = gh * dhb
        dq = _routed_dgrad_in(np.concatenate([da, db], axis=1), weights)
        dxe = dq[:, :da.shape[1]] @ Tg + dq[:, da.shape[1]:] @ Tu
        for j, r in enumerate(rows):
            dx[r] += dxe[j]

    # --- weight gradients: every token routed to the requested experts ---
    dW = {}
    need = set(int(e) for e in experts)
    if need:
        all_by = _routes_by_expert(top, rw, range(T), E)
        for e in sorted(need):
            lst = all_by[e]
            Wg, Wu, Wd = weights.routed(e)
            if not lst:
                dW[e] = (np.zeros_like(Wg), np.zeros_like(Wu), np.zeros_like(Wd))
                continue
            ts = np.array([t for t, _, _ in lst])
            w = np.array([w for _, _, w in lst])
            X = x_all[ts]
            G = dy_all[ts]
            a, b, h, _ = _routed_ffn(X, Wg, Wu, Wd, weights)
            _, dha, dhb = swiglu_clamped(a, b, weights.swiglu_limit)
            Tg, Tu, Td = weights.routed_t(e)
            gh = _routed_dgrad_in(w[:, None] * G, weights) @ Td
            da = gh * dha
            db = gh * dhb
            dW[e] = (da.T @ X, db.T @ X, (w[:, None] * G).T @ h)
    if shared_grads and weights.shared is not None:
        X = x_all
        G = dy_all
        Wg, Wu, Wd = weights.shared
        a, b, h, ys = swiglu_ffn(X, Wg, Wu, Wd, weights.swiglu_limit)
        _, dha, dhb = swiglu_clamped(a, b, weights.swiglu_limit)
        if weights.shared_gate is not None:
            sc = shared_gate_score(X, weights.shared_gate)
            dz = sc * (1.0 - sc) * np.sum(G * ys, axis=1)
            dW["shared_out_gate"] = dz @ X          # sum over all tokens of dz_t x_t
            G = sc[:, None] * G
        gh = G @ Wd
        da = gh * dha
        db = gh * dhb
        dW["shared"] = (da.T @ X, db.T @ X, G.T @ h)
    return {"dx": dx, "dprobs": dprobs, "dW": dW}
