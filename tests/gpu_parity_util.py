"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the oracle on the same bits."""
import time

import numpy as np
import torch

import moe_inputs as gen
from oracle import moe_oracle as O

BF16_TOL = 2e-2     # max|gpu - ref| / max|ref| for BF16 routed experts
MXFP8_TOL = 6e-2    # ... for MXFP8 routed experts


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(gpu - ref).max() / max(np.abs(ref).max(), 1e-30))


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def tol_of(dp) -> float:
    return MXFP8_TOL if dp.cfg.routed == "mxfp8" else BF16_TOL


def oracle_weights(dp, mx_activations=None) -> "O.Weights":
    """The oracle's weights for a device problem.  MXFP8 routed experts follow the MXFP8
    recipe by default: their FP8 GEMMs take MXFP8 activation inputs as well."""
    cfg = dp.cfg
    shared = getattr(dp, "shared", True)
    if mx_activations is None:
        mx_activations = cfg.routed == "mxfp8"
    return O.Weights.from_bits(cfg.inter, dp.np_s1 if shared else None, dp.np_s2 if shared else None,
                               lambda e: dp.np_routed[e], cfg.routed, shared_gate=getattr(dp, "np_gate", None),
                               swiglu_limit=getattr(dp, "swiglu_limit", 0.0), mx_activations=mx_activations)


def check_routing_state(dp):
    """Compaction table, gathered probabilities, counts, offsets and the permutation:
    bit-exact against the oracle."""
    cfg = dp.cfg
    st = {k: v.cpu().numpy() for k, v in dp.layer.routing_state().items()}
    top, rw = O.compact_routing(dp.np_rmap, dp.np_probs, cfg.topk)
    counts, offsets, slot_of, slot_token = O.dispatch_index(top, cfg.experts)
    S = int(offsets[-1])
    assert int(st["status_word"][0]) == 0
    assert np.array_equal(st["top_experts"], top)
    assert np.array_equal(st["router_weights"].view(np.uint32), rw.astype(np.float32).view(np.uint32))
    assert np.array_equal(st["counts"], counts)
    assert np.array_equal(st["offsets"], offsets)
    assert np.array_equal(st["slot_of"], slot_of)
    assert np.array_equal(st["slot_token"][:S], slot_token)
    return top, offsets


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    if T <= n:
        return np.arange(T)
    return np.sort(rng.choice(T, size=n, replace=False))


def _mg_errs(dp, g, experts, errs):
    cfg = dp.cfg
    I, H = cfg.inter, cfg.hidden
    for e in experts:
        d1 = to_f64(dp.mg_r1_list[e]) - dp.main_grad_start((2 * I, H), e)
        d2 = to_f64(dp.mg_r2_list[e]) - dp.main_grad_start((H, I), e)
        dg, du, dd = g["dW"][e]
        errs[f"gate{e}"] = rel_err(d1[:I], dg) if np.abs(dg).max() > 0 else float(np.abs(d1[:I]).max())
        errs[f"up{e}"] = rel_err(d1[I:], du) if np.abs(du).max() > 0 else float(np.abs(d1[I:]).max())
        errs[f"down{e}"] = rel_err(d2, dd) if np.abs(dd).max() > 0 else float(np.abs(d2).max())


def check_full(dp, W, tol, experts=None, chunk=16, tokens=True, weights=True):
    """Every token's out, dx and dprobs (tokens=True), and the main_grad deltas of `experts`
    (every routed expert when None) and of the shared expert (weights=True), against the
    oracle.  The oracle runs in phases (forward; token gradients; weight gradients a few
    experts at a time; the shared expert), each printing when it ends."""
    cfg = dp.cfg
    args = (dp.np_probs, dp.np_rmap, cfg.topk, W)
    errs = {}
    t0 = time.time()
    if tokens:
        _check_full_tokens(dp, args, errs, t0)
    if weights:
        _check_full_weights(dp, args, errs, t0, experts, chunk)
    worst = max(errs, key=lambda k: errs[k])
    print(f"[parity] full tensors: " + " ".join(f"{k} {errs[k]:.3e}" for k in ("out", "dx", "dprobs") if k in errs)
          + f" worst {worst} {errs[worst]:.3e} (tol {tol})", flush=True)
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"over tolerance {tol}: {bad}"
    return errs


def _check_full_tokens(dp, args, errs, t0):
    ref = O.moe_forward(dp.np_x, *args)
    errs["out"] = rel_err(to_f64(dp.out), ref)
    del ref
    print(f"[full] out {errs['out']:.3e} ({time.time() - t0:.0f} s)", flush=True)
    g = O.moe_backward(dp.np_dy, dp.np_x, *args, experts=[], shared_grads=False)
    errs["dx"] = rel_err(to_f64(dp.dx), g["dx"])
    dpr = dp.dprobs.cpu().numpy().astype(np.float64)
    errs["dprobs"] = rel_err(dpr, g["dprobs"])
    assert np.all(dpr[dp.np_rmap == 0] == 0), "dprobs must be exactly zero off the routing map"
    del g, dpr
    print(f"[full] dx {errs['dx']:.3e} dprobs {errs['dprobs']:.3e} ({time.time() - t0:.0f} s)", flush=True)


def _check_full_weights(dp, args, errs, t0, experts, chunk):
    cfg = dp.cfg
    I, H = cfg.inter, cfg.hidden
    none = np.zeros(0, dtype=np.int64)
    ex = list(range(cfg.experts)) if experts is None else list(experts)
    for i in range(0, len(ex), chunk):
        part = ex[i:i + chunk]
        g = O.moe_backward(dp.np_dy, dp.np_x, *args, tokens=none, experts=part, shared_grads=False)
        _mg_errs(dp, g, part, errs)
        worst = max((k for k in errs if k.startswith(("gate", "up", "down"))), key=lambda k: errs[k])
        print(f"[full] main_grad of experts {part[0]}..{part[-1]} done, worst so far {worst} "
              f"{errs[worst]:.3e} ({time.time() - t0:.0f} s)", flush=True)
    if dp.shared:
        g = O.moe_backward(dp.np_dy, dp.np_x, *args, tokens=none, experts=[], shared_grads=True)
        s1 = to_f64(dp.mg_s1) - dp.main_grad_start((2 * I, H), 0)
        s2 = to_f64(dp.mg_s2) - dp.main_grad_start((H, I), 0)
        dg, du, dd = g["dW"]["shared"]
        errs["shared_gate"] = rel_err(s1[:I], dg)
        errs["shared_up"] = rel_err(s1[I:], du)
        errs["shared_down"] = rel_err(s2, dd)
        print(f"[full] shared main_grad gate {errs['shared_gate']:.3e} up {errs['shared_up']:.3e} down "
              f"{errs['shared_down']:.3e} ({time.time() - t0:.0f} s)", flush=True)


# ----------------------------------------------------------------------------------
# MXFP8 activation codes: every E4M3 code and E8M0 scale byte the GPU produced for the FP8
# GEMM inputs whose values come straight from the inputs (x, and the BF16 w dy), against
# the oracle's block exponent and E4M3 rounding of the same values, bit for bit
# ----------------------------------------------------------------------------------
def _assert_codes(codes, scales, v, what):
    """codes u8 [rows, n], scales u8 [rows, n/32] against values v float64 [rows, n]: the
    scale byte is e + 127 with e the oracle's block exponent, and each code decodes to
    the oracle's E4M3 rounding of v 2^-e, sign of zero included."""
    rows, n = v.shape
    blk = v.reshape(rows, n // 32, 32)
    e = O.mx_block_exponent(np.abs(blk).max(axis=2))
    assert np.array_equal(scales.astype(np.int64), e + 127), f"{what}: E8M0 scale bytes differ"
    want = O.e4m3_round(np.ldexp(blk, -e[:, :, None])).reshape(rows, n)
    got = O.e4m3_decode(codes)
    same = (got == want) & (np.signbit(got) == np.signbit(want))
    assert same.all(), f"{what}: {int((~same).sum())} E4M3 codes differ (first at {np.argwhere(~same)[0]})"


def check_x_codes(dp, chunk=2048):
    """After an MXFP8 forward: the E4M3 codes and scales of x, one row per token."""
    import moe_megakernel_amd as mk
    cfg = dp.cfg
    T, H = cfg.tokens, cfg.hidden
    L = mk.moe_mx_staging_view(dp.p)
    ws = dp.layer.workspace
    xq = ws[L.x_codes:L.x_codes + T * H].view(T, H).cpu().numpy()
    xs = ws[L.x_scales:L.x_scales + T * H // 32].view(T, H // 32).cpu().numpy()
    for t0 in range(0, T, chunk):
        sl = slice(t0, min(T, t0 + chunk))
        _assert_codes(xq[sl], xs[sl], O.bf16_decode(dp.np_x[sl]), f"x rows {t0}..")
    print(f"[codes] x: {T} x {H} codes and scales bit-exact", flush=True)


def check_dy_codes(dp, chunk=2048, max_slots=None):
    """After an MXFP8 backward: the codes and scales of each slot's BF16 w dy (w times dy
    formed in FP32, the precision in which the kernel forms it, then rounded to BF16); all
    slots, or a seeded sample of max_slots of them."""
    import moe_megakernel_amd as mk
    cfg = dp.cfg
    H, K = cfg.hidden, cfg.topk
    top, rw = O.compact_routing(dp.np_rmap, dp.np_probs, K)
    _, offsets, _, slot_token = O.dispatch_index(top, cfg.experts)
    S = int(offsets[-1])
    L = mk.moe_mx_staging_view(dp.p)
    ws = dp.layer.workspace
    dq = ws[L.dy_codes:L.dy_codes + S * H].view(S, H).cpu().numpy()
    ds = ws[L.dy_scales:L.dy_scales + S * H // 32].view(S, H // 32).cpu().numpy()
    dy32 = O.bf16_decode(dp.np_dy).astype(np.float32)
    slots = np.arange(S) if max_slots is None or S <= max_slots else sample_tokens(S, max_slots, seed=S)
    for s0 in range(0, len(slots), chunk):
        sl = slots[s0:s0 + chunk]
        st = slot_token[sl]
        t, k = st // K, st % K
        prod = rw[t, k].astype(np.float32)[:, None] * dy32[t]        # float32 products
        _assert_codes(dq[sl], ds[sl], O.bf16_round(prod.astype(np.float64)), f"w dy slots {sl[0]}..")
    print(f"[codes] w dy: {len(slots)} of {S} slots x {H}: codes and scales bit-exact", flush=True)
