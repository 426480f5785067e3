"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on
the same seeded bits.  Integer routing state and MXFP8 activation codes are compared
bit-exact; floating results by max|gpu - ref| / max|ref| <= 2e-2 (BF16 routed experts)
or <= 6e-2 (MXFP8 routed experts, against the oracle of the MXFP8 recipe, whose FP8
GEMMs take MXFP8 activation inputs too)."""
import numpy as np
import pytest
import torch

import moe_inputs as gen
from oracle import moe_oracle as O
from tests.gpu_parity_util import (BF16_TOL, MXFP8_TOL, check_dy_codes, check_full, check_routing_state,
                                   check_x_codes, oracle_weights, rel_err, to_f64, tol_of)

pytestmark = pytest.mark.gpu


def _dp(cfg, **kw):
    from moe_inputs.device import DeviceProblem
    print(f"[case] {cfg.name} T={cfg.tokens} H={cfg.hidden} E={cfg.experts} K={cfg.topk} I={cfg.inter}",
          flush=True)
    return DeviceProblem(cfg, **kw)


def _check_forward(dp, W, tokens=None, tol=BF16_TOL):
    cfg = dp.cfg
    ref = O.moe_forward(dp.np_x, dp.np_probs, dp.np_rmap, cfg.topk, W, tokens=tokens)
    got = to_f64(dp.out) if tokens is None else to_f64(dp.out[torch.as_tensor(tokens, device=dp.out.device)])
    err = rel_err(got, ref)
    print(f"[parity] out rel err {err:.3e} (tol {tol})", flush=True)
    assert np.isfinite(got).all()
    assert err <= tol, f"out rel err {err:.3e}"
    return err


def _check_backward(dp, W, tokens=None, experts=None, tol=BF16_TOL):
    cfg = dp.cfg
    I = cfg.inter
    g = O.moe_backward(dp.np_dy, dp.np_x, dp.np_probs, dp.np_rmap, cfg.topk, W, tokens=tokens,
                       experts=experts)
    sel = slice(None) if tokens is None else torch.as_tensor(tokens, device=dp.dx.device)
    dx = to_f64(dp.dx[sel])
    dpr = dp.dprobs[sel].cpu().numpy().astype(np.float64)
    errs = {"dx": rel_err(dx, g["dx"]), "dprobs": rel_err(dpr, g["dprobs"])}
    rm = dp.np_rmap if tokens is None else dp.np_rmap[tokens]
    assert np.all(dpr[rm == 0] == 0), "dprobs must be exactly zero off the routing map"
    for e in (range(cfg.experts) if experts is None else experts):
        d1 = to_f64(dp.mg_r1_list[e]) - dp.main_grad_start((2 * I, cfg.hidden), e)
        d2 = to_f64(dp.mg_r2_list[e]) - dp.main_grad_start((cfg.hidden, I), e)
        dg, du, dd = g["dW"][e]
        errs[f"gate{e}"] = rel_err(d1[:I], dg) if np.abs(dg).max() > 0 else float(np.abs(d1[:I]).max())
        errs[f"up{e}"] = rel_err(d1[I:], du) if np.abs(du).max() > 0 else float(np.abs(d1[I:]).max())
        errs[f"down{e}"] = rel_err(d2, dd) if np.abs(dd).max() > 0 else float(np.abs(d2).max())
    s1 = to_f64(dp.mg_s1) - dp.main_grad_start((2 * I, cfg.hidden), 0)
    s2 = to_f64(dp.mg_s2) - dp.main_grad_start((cfg.hidden, I), 0)
    if dp.shared:
        dg, du, dd = g["dW"]["shared"]
        errs["shared_gate"] = rel_err(s1[:I], dg)
        errs["shared_up"] = rel_err(s1[I:], du)
        errs["shared_down"] = rel_err(s2, dd)
    else:   # routed-only: the shared main_grad buffers were not handed over and stay as they were
        assert "shared" not in g["dW"]
        assert np.all(s1 == 0) and np.all(s2 == 0)
    gw = to_f64(dp.mg_gate) - dp.main_grad_start((cfg.hidden,), 0)
    if getattr(dp, "gated", False):
        errs["shared_out_gate"] = rel_err(gw, g["dW"]["shared_out_gate"])
    else:
        assert np.all(gw == 0), "the gate's main_grad must not be touched without the gate"
    worst = max(errs, key=lambda k: errs[k])
    print(f"[parity] dx {errs['dx']:.3e} dprobs {errs['dprobs']:.3e} worst {worst} {errs[worst]:.3e} "
          f"(tol {tol})", flush=True)
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"over tolerance {tol}: {bad}"
    return errs


def test_config0_forward_matches_oracle(gpu_lib):
    dp = _dp(gen.config(0))
    dp.forward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    _check_forward(dp, oracle_weights(dp))


def test_config1_forward_backward_matches_oracle(gpu_lib):
    dp = _dp(gen.config(1))
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    _check_forward(dp, W)
    _check_backward(dp, W)


@pytest.mark.parametrize("shape", [
    (300, 256, 5, 3, 128),     # ragged token count, uneven experts, short rows
    (1, 128, 3, 2, 128),       # a single token
    (777, 384, 13, 4, 256),    # several tiles and ragged tails everywhere
])
def test_ragged_shapes_forward_backward(gpu_lib, shape):
    T, H, E, K, I = shape
    cfg = gen.custom(T, H, E, K, I, short_frac=0.1, short_max=max(1, K - 1), idx=200 + T)
    dp = _dp(cfg)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    _check_forward(dp, W)
    _check_backward(dp, W)


def test_empty_routing_map_gives_shared_expert_only(gpu_lib):
    cfg = gen.custom(200, 256, 6, 2, 128, idx=301)
    probs = np.zeros((200, 6), np.float32)
    rmap = np.zeros((200, 6), np.uint8)
    dp = _dp(cfg, routing=(probs, rmap))
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    st = dp.layer.routing_state()
    assert int(st["counts"].sum()) == 0 and bool((st["top_experts"] == -1).all())
    W = oracle_weights(dp)
    _check_forward(dp, W)
    errs = _check_backward(dp, W)
    assert all(errs[f"down{e}"] == 0 for e in range(6))     # routed main_grad untouched
    assert float(dp.dprobs.abs().max()) == 0.0


def test_all_tokens_on_one_expert(gpu_lib):
    # one expert receives every token (many row tiles), the others none
    T, E = 640, 4
    cfg = gen.custom(T, 256, E, 1, 128, idx=302)
    rmap = np.zeros((T, E), np.uint8)
    rmap[:, 2] = 1
    probs = rmap.astype(np.float32) * np.float32(0.75)
    dp = _dp(cfg, routing=(probs, rmap))
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    _check_forward(dp, W)
    _check_backward(dp, W)


@pytest.mark.parametrize("shape", [
    (1300, 256, 2, 2, 384),    # 1300 slots per expert, ragged row tiles, 3 SwiGLU-backward N tiles
    (2200, 384, 3, 2, 256),    # three experts, shared and routed rows in every launch
    (700, 256, 7, 3, 128),     # 300 slots per expert, just above the threshold, uneven experts
])
def test_many_tokens_per_expert_wide_shapes(gpu_lib, shape):
    """BF16 layers with more than 256 routed slots per expert take the two-workgroups-per-
    CU token-GEMM shapes (192 x 128 tiles): parity with the oracle, and two runs bit for bit."""
    T, H, E, K, I = shape
    assert T * K > 256 * E   # above the library's threshold for the wide shapes
    cfg = gen.custom(T, H, E, K, I, short_frac=0.1, short_max=1, idx=500 + T)
    print(f"[case] wide shapes T={T} H={H} E={E} K={K} I={I}", flush=True)
    dp = _dp(cfg)
    snaps = []
    for _ in range(2):
        dp.reset_main_grads()
        dp.forward()
        dp.backward()
        torch.cuda.synchronize()
        snaps.append(_bitwise_snapshot(dp))
    assert _same_bits(*snaps)
    check_routing_state(dp)
    W = oracle_weights(dp)
    _check_forward(dp, W)
    _check_backward(dp, W)


def test_route_overflow_sets_status_word(gpu_lib):
    T, E, K = 64, 8, 2
    cfg = gen.custom(T, 128, E, K, 128, idx=303)
    probs, rmap = gen.routing(cfg)
    rmap[5, :] = 1                        # 8 routes on a top-2 row: invalid input
    probs[5, :] = 0.125
    dp = _dp(cfg, routing=(probs, rmap), backward=False)
    dp.forward()
    torch.cuda.synchronize()
    assert int(dp.layer.routing_state()["status_word"][0]) == 7   # MOE_ERR_ROUTE_OVERFLOW


def test_forward_backward_bitwise_deterministic(gpu_lib):
    dp = _dp(gen.config(1))
    outs = []
    for _ in range(2):
        dp.reset_main_grads()
        dp.forward()
        dp.backward()
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (dp.out, dp.dx, dp.dprobs, dp.mg_r1, dp.mg_r2, dp.mg_s1, dp.mg_s2)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a, b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("flags", [1, 0, 1 | 2, 1 | 4, 2 | 4])
def test_zero_tokens_is_a_no_op(gpu_lib, flags):
    """An empty batch in every mode (shared, routed-only, recompute, table input): the
    calls succeed, read no input and leave every main_grad as it was."""
    import moe_megakernel_amd as mk
    p = mk.problem(0, 256, 128, 4, 2, flags=flags)
    layer = mk.Layer(p)
    dp = _dp(gen.custom(4, 256, 4, 2, 128, idx=304), backward=True)
    before = [t.clone() for t in dp.mg_r1_list + dp.mg_r2_list + [dp.mg_s1, dp.mg_s2]]
    empty = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    if flags & mk.MOE_FLAG_TOPK_ROUTING:
        layer.forward_topk(empty, torch.empty(0, 2, dtype=torch.int32, device="cuda"),
                           torch.empty(0, 2, device="cuda"), dp.weights, empty)
    else:
        layer.forward(empty, torch.empty(0, 4, device="cuda"), torch.empty(0, 4, dtype=torch.uint8, device="cuda"),
                      dp.weights, empty)
    layer.backward(empty, empty, dp.weights, empty, torch.empty(0, 4, device="cuda"), dp.main_grads)
    torch.cuda.synchronize()
    after = dp.mg_r1_list + dp.mg_r2_list + [dp.mg_s1, dp.mg_s2]
    assert all(torch.equal(a, b) for a, b in zip(before, after))
    assert int(layer.routing_state()["status_word"][0]) == 0


def _bitwise_snapshot(dp):
    return [t.clone() for t in [dp.out, dp.dx, dp.dprobs] + dp.mg_r1_list + dp.mg_r2_list + [dp.mg_s1, dp.mg_s2]]


def _same_bits(a, b):
    return all(torch.equal(x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32),
                           y.view(torch.int16) if y.element_size() == 2 else y.view(torch.int32))
               for x, y in zip(a, b))


def _run_twice_same_bits(dp, after_forward=None):
    """Forward + backward twice from the same main_grad start; every output and main_grad
    bit must match.  after_forward(dp) runs between the second forward and backward."""
    runs = []
    for i in range(2):
        dp.reset_main_grads()
        dp.forward()
        torch.cuda.synchronize()
        if i == 1 and after_forward is not None:
            after_forward(dp)
        dp.backward()
        torch.cuda.synchronize()
        runs.append(_bitwise_snapshot(dp))
    assert _same_bits(*runs), f"two runs of {dp.cfg.name} differ"
    print("[determinism] two runs bit-identical", flush=True)


def test_full_size_bf16_layer_full_tensors(gpu_lib):
    """4096 tokens, hidden 4096, 96 experts, top-4, inter 1024 (force-balanced routing),
    the benchmark's launch configuration: run twice, bit for bit the same; then every
    token's out, dx and dprobs and the main_grad deltas of all 96 routed experts and the
    shared expert against the oracle."""
    cfg = gen.config(2)
    dp = _dp(cfg, threads=16)
    _run_twice_same_bits(dp)
    check_routing_state(dp)
    check_full(dp, oracle_weights(dp), BF16_TOL)


def test_full_size_ep_share_bf16_full_tensors(gpu_lib):
    """The same 4096 tokens on 6 local experts (one GPU's share under 16-way expert
    parallelism, 2730 or 2731 rows per expert), which runs the 192 x 128 token-GEMM tiles at
    two workgroups per CU: run twice, bit for bit the same; then every token's out, dx and
    dprobs and the main_grad deltas of all 6 routed experts and the shared expert against
    the oracle."""
    cfg = gen.config(5)
    dp = _dp(cfg, threads=16)
    _run_twice_same_bits(dp)
    check_routing_state(dp)
    check_full(dp, oracle_weights(dp), BF16_TOL)


# ----------------------------------------------------------------------------------
# MXFP8 routed experts (E4M3 payload + E8M0 scale per 32 along K; shared stays BF16)
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("layout,shape", [
    ("table", (300, 256, 6, 3, 128)),
    ("single", (520, 384, 9, 2, 256)),
    ("single", (260, 128, 5, 2, 256)),   # H = 128: FC1's K loop is a single 128-code stage
])
def test_mxfp8_forward_backward_matches_oracle(gpu_lib, layout, shape):
    T, H, E, K, I = shape
    cfg = gen.custom(T, H, E, K, I, routed="mxfp8", layout=layout, short_frac=0.1, short_max=max(1, K - 1),
                     idx=200 + T)
    dp = _dp(cfg)
    dp.forward()
    torch.cuda.synchronize()
    check_x_codes(dp)
    dp.backward()
    torch.cuda.synchronize()
    check_dy_codes(dp)
    check_routing_state(dp)
    W = oracle_weights(dp)
    _check_forward(dp, W, tol=MXFP8_TOL)
    _check_backward(dp, W, tol=MXFP8_TOL)


def test_full_size_mxfp8_layer_full_tensors(gpu_lib):
    """4096 tokens, hidden 4096, 96 experts, top-4, inter 1024, skewed softmax routing,
    MXFP8 routed weights in per-expert allocations through device pointer tables: run twice,
    bit for bit the same; the x and w dy codes bit for bit; every token's out, dx and dprobs
    and the main_grad deltas of all 96 routed experts and the shared expert against the
    oracle."""
    cfg = gen.config(3)
    dp = _dp(cfg, threads=16)
    _run_twice_same_bits(dp, check_x_codes)
    check_dy_codes(dp)
    check_routing_state(dp)
    check_full(dp, oracle_weights(dp), MXFP8_TOL)


def test_large_mxfp8_layer_every_token(gpu_lib):
    """8192 tokens, hidden 7168, 64 experts, top-6, inter 2048, 2% of tokens with fewer
    than 6 routes, MXFP8 routed weights: run twice, bit for bit the same; x codes in full
    and w dy codes on sampled slots bit for bit; every token's out, dx and dprobs against
    the oracle (the main_grads in the next test)."""
    cfg = gen.config(4)
    dp = _dp(cfg, threads=16)
    _run_twice_same_bits(dp, check_x_codes)
    check_dy_codes(dp, max_slots=8192)
    check_routing_state(dp)
    check_full(dp, oracle_weights(dp), MXFP8_TOL, weights=False)


def test_large_mxfp8_layer_every_main_grad(gpu_lib):
    """The same 8192-token MXFP8 layer: the main_grad deltas of all 64 routed experts and of
    the shared expert against the oracle."""
    cfg = gen.config(4)
    dp = _dp(cfg, threads=16)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_full(dp, oracle_weights(dp), MXFP8_TOL, tokens=False)


def test_full_size_ep_share_mxfp8_full_tensors(gpu_lib):
    """4096 tokens on 6 local experts with MXFP8 routed weights (balanced): run twice, bit
    for bit the same; the x and w dy codes bit for bit; every token's out, dx and dprobs and
    the main_grad deltas of all 6 routed experts and the shared expert against the oracle."""
    cfg = gen.config(6)
    dp = _dp(cfg, threads=16)
    _run_twice_same_bits(dp, check_x_codes)
    check_dy_codes(dp)
    check_routing_state(dp)
    check_full(dp, oracle_weights(dp), MXFP8_TOL)


def test_saved_context_is_relocatable(gpu_lib):
    """`saved` holds offsets and indices only: the backward run from a copy at another
    address, with the original overwritten, gives the same bits."""
    for routed, layout in (("bf16", "single"), ("mxfp8", "table")):
        cfg = gen.custom(300, 256, 6, 3, 128, routed=routed, layout=layout, short_frac=0.1, short_max=2,
                         idx=1200)
        dp = _dp(cfg)
        dp.forward()
        dp.reset_main_grads()
        dp.backward()
        torch.cuda.synchronize()
        ref = [t.clone() for t in [dp.dx, dp.dprobs] + dp.mg_r1_list + dp.mg_r2_list + [dp.mg_s1, dp.mg_s2]]
        original = dp.layer.saved
        moved = torch.empty(original.numel() + 4096, dtype=torch.uint8, device=original.device)[4096:]
        moved.copy_(original)
        original.fill_(0xFF)
        dp.layer.saved = moved
        dp.reset_main_grads()
        dp.backward()
        torch.cuda.synchronize()
        got = [dp.dx, dp.dprobs] + dp.mg_r1_list + dp.mg_r2_list + [dp.mg_s1, dp.mg_s2]
        assert _same_bits(ref, got), f"{routed}: backward from the relocated context differs"
        print(f"[saved] {routed}: backward from a relocated copy bit-identical", flush=True)


# ----------------------------------------------------------------------------------
# limits and degenerate shapes
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("routed,layout", [("bf16", "single"), ("mxfp8", "table")])
def test_max_experts_and_topk(gpu_lib, routed, layout):
    """255 experts (a routing row spans all 64 lanes of a wave) and the widest table, K = 8;
    MXFP8 with 255 per-expert allocations behind device pointer tables."""
    cfg = gen.custom(200, 256, 255, 8, 128, routed=routed, layout=layout, short_frac=0.1, short_max=7, idx=501)
    dp = _dp(cfg)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    _check_forward(dp, W, tol=tol_of(dp))
    _check_backward(dp, W, experts=[0, 1, 127, 254], tol=tol_of(dp))


@pytest.mark.parametrize("routed", ["bf16", "mxfp8"])
def test_single_expert_top1(gpu_lib, routed):
    """E = 1, K = 1: every token takes the one routed expert plus the shared expert."""
    cfg = gen.custom(130, 128, 1, 1, 128, routed=routed, idx=502)
    dp = _dp(cfg)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    _check_forward(dp, W, tol=tol_of(dp))
    _check_backward(dp, W, tol=tol_of(dp))


@pytest.mark.parametrize("routed,layout,shape,mgd", [
    ("bf16", "single", (300, 256, 6, 3, 128), "fp32"),
    ("bf16", "table", (900, 256, 3, 3, 128), "fp32"),    # the wide BF16 shapes
    ("bf16", "single", (300, 384, 6, 3, 256), "bf16"),
    ("mxfp8", "single", (260, 384, 5, 2, 256), "fp32"),
    ("mxfp8", "table", (300, 256, 6, 3, 128), "bf16"),
])
def test_padded_row_strides(gpu_lib, routed, layout, shape, mgd):
    """Every weight (payload and scales, shared and routed) and every main_grad with rows 48
    bytes longer than their columns, the weight pads NaN and the main_grad pads a fill value:
    the results equal the unpadded call's bit for bit, no pad is written, and they match the
    oracle."""
    T, H, E, K, I = shape
    cfg = gen.custom(T, H, E, K, I, routed=routed, layout=layout, short_frac=0.1, short_max=max(1, K - 1),
                     idx=1100 + T)
    runs = []
    for pad in (0, 48):
        dp = _dp(cfg, main_grad_dtype=mgd, pad_bytes=pad)
        dp.forward()
        dp.backward()
        torch.cuda.synchronize()
        runs.append(dp)
    plain, padded = runs
    assert padded.main_grad_pads_untouched(), "a main_grad pad was written"
    _assert_same_bits(plain, padded)
    W = oracle_weights(padded)
    _check_forward(padded, W, tol=tol_of(padded))
    _check_backward(padded, W, tol=tol_of(padded))


@pytest.mark.parametrize("routed,layout,shape,mgd,pad", [
    ("bf16", "single", (300, 256, 6, 3, 128), "fp32", 0),
    ("bf16", "table", (900, 256, 3, 3, 128), "bf16", 48),   # the wide BF16 shapes
    ("mxfp8", "single", (260, 384, 5, 2, 256), "fp32", 0),
    ("mxfp8", "table", (300, 256, 6, 3, 128), "fp32", 48),
])
def test_separate_gate_up_allocations(gpu_lib, routed, layout, shape, mgd, pad):
    """The gate and up halves of every FC1 weight (payload and scales, shared and routed) and
    of every FC1 main_grad in allocations of their own, described with row offset 0: the
    results equal the call on row views of combined tensors bit for bit and match the
    oracle."""
    T, H, E, K, I = shape
    cfg = gen.custom(T, H, E, K, I, routed=routed, layout=layout, short_frac=0.1, short_max=max(1, K - 1),
                     idx=1200 + T)
    runs = []
    for sep in (False, True):
        dp = _dp(cfg, main_grad_dtype=mgd, pad_bytes=pad, separate_gate_up=sep)
        dp.forward()
        dp.backward()
        torch.cuda.synchronize()
        runs.append(dp)
    packed, sep = runs
    assert sep.main_grad_pads_untouched(), "a main_grad pad was written"
    _assert_same_bits(packed, sep)
    W = oracle_weights(sep)
    _check_forward(sep, W, tol=tol_of(sep))
    _check_backward(sep, W, tol=tol_of(sep))


@pytest.mark.parametrize("which", ["small", 2, 3])
def test_hip_graph_replay_matches_eager(gpu_lib, which):
    """Both calls enqueue only kernels on the caller's stream, so a captured graph of
    forward + backward replays bit-identically to the eager calls (main_grad reset
    eagerly between replays, other eager work in between): a small ragged layer, and the
    4096-token layer with BF16 and with MXFP8 routed weights (pointer tables) at full
    size."""
    cfg = (gen.custom(300, 256, 6, 3, 128, short_frac=0.1, short_max=2, idx=503) if which == "small"
           else gen.config(which))
    dp = _dp(cfg, threads=16)
    dp.reset_main_grads()
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    eager = _bitwise_snapshot(dp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        dp.reset_main_grads()
        dp.forward()
        dp.backward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.forward()
        dp.backward()
    torch.cuda.synchronize()
    for rep in range(3):
        dp.reset_main_grads()
        dp.out.fill_(float("nan"))
        dp.dx.fill_(float("nan"))
        dp.dprobs.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same_bits(_bitwise_snapshot(dp), eager), f"replay {rep} differs from the eager call"


# ----------------------------------------------------------------------------------
# routed-only mode: no fused shared expert (flags = 0); out, dx and the main_grads hold
# the routed terms only
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("routed,layout,shape", [
    ("bf16", "single", (777, 384, 13, 4, 256)),
    ("bf16", "table", (1, 128, 3, 2, 128)),
    ("mxfp8", "table", (300, 256, 6, 3, 128)),
    ("mxfp8", "single", (520, 384, 9, 2, 256)),
    ("bf16", "single", (900, 256, 3, 3, 128)),   # 900 slots per expert: the wide BF16 shapes
])
def test_routed_only_forward_backward_matches_oracle(gpu_lib, routed, layout, shape):
    T, H, E, K, I = shape
    cfg = gen.custom(T, H, E, K, I, routed=routed, layout=layout, short_frac=0.1, short_max=max(1, K - 1),
                     idx=500 + T)
    dp = _dp(cfg, shared=False)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    assert W.shared is None
    tol = BF16_TOL if routed == "bf16" else MXFP8_TOL
    _check_forward(dp, W, tol=tol)
    _check_backward(dp, W, tol=tol)


def test_routed_only_empty_map_gives_exact_zeros(gpu_lib):
    cfg = gen.custom(200, 256, 6, 2, 128, idx=501)
    dp = _dp(cfg, shared=False, routing=(np.zeros((200, 6), np.float32), np.zeros((200, 6), np.uint8)))
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    assert float(dp.out.float().abs().max()) == 0.0
    assert float(dp.dx.float().abs().max()) == 0.0
    assert float(dp.dprobs.abs().max()) == 0.0
    W = oracle_weights(dp)
    _check_backward(dp, W)


def test_routed_only_full_size_full_tensors(gpu_lib):
    """4096 tokens, hidden 4096, 96 experts, top-4, inter 1024 without the shared expert:
    every token's out, dx and dprobs and the main_grad deltas of all 96 experts against
    the oracle.  The fused run minus the routed-only run is the shared expert's output, a
    dense SwiGLU MLP on every token."""
    cfg = gen.config(2)
    dp = _dp(cfg, shared=False)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    _check_forward(dp, W)
    _check_backward(dp, W)
    routed_out = to_f64(dp.out)
    del dp, W
    full = _dp(cfg, backward=False)
    full.forward()
    torch.cuda.synchronize()
    Wf = oracle_weights(full)
    x = O.bf16_decode(full.np_x)
    _, _, _, mlp = O.swiglu_ffn(x, *Wf.shared)
    diff = to_f64(full.out) - routed_out
    err = rel_err(diff, mlp)
    print(f"[parity] fused - routed-only vs shared MLP: rel err {err:.3e}", flush=True)
    assert err <= 2 * BF16_TOL


# ----------------------------------------------------------------------------------
# MoE-layer recompute (MOE_FLAG_RECOMPUTE): saved holds the routing state only and the
# backward regenerates the activations with the same kernels, so every result must be
# bit-identical to the mode that saves them
# ----------------------------------------------------------------------------------
def _bits(t):
    return t.detach().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()


def _assert_same_bits(a, b):
    assert torch.equal(_bits(a.out), _bits(b.out)), "out differs"
    assert torch.equal(_bits(a.dx), _bits(b.dx)), "dx differs"
    assert torch.equal(_bits(a.dprobs), _bits(b.dprobs)), "dprobs differs"
    for x, y in zip(a.mg_r1_list + a.mg_r2_list + [a.mg_s1, a.mg_s2],
                    b.mg_r1_list + b.mg_r2_list + [b.mg_s1, b.mg_s2]):
        assert torch.equal(_bits(x), _bits(y)), "main_grad differs"


@pytest.mark.parametrize("routed,layout,shape,shared", [
    ("bf16", "single", (777, 384, 13, 4, 256), True),
    ("mxfp8", "table", (300, 256, 6, 3, 128), True),
    ("mxfp8", "single", (520, 384, 9, 2, 256), False),
    ("bf16", "table", (900, 256, 3, 3, 128), False),   # the wide BF16 shapes
])
def test_recompute_is_bit_identical_and_matches_oracle(gpu_lib, routed, layout, shape, shared):
    T, H, E, K, I = shape
    cfg = gen.custom(T, H, E, K, I, routed=routed, layout=layout, short_frac=0.1, short_max=max(1, K - 1),
                     idx=600 + T)
    ref = _dp(cfg, shared=shared)
    ref.forward()
    ref.backward()
    rc = _dp(cfg, shared=shared, recompute=True)
    assert rc.layer.saved.numel() * 8 < ref.layer.saved.numel()
    rc.forward()
    # the backward must not read anything the forward left in the workspace
    rc.layer.workspace.fill_(0xFF)
    rc.backward()
    torch.cuda.synchronize()
    check_routing_state(rc)
    _assert_same_bits(ref, rc)
    W = oracle_weights(rc)
    tol = BF16_TOL if routed == "bf16" else MXFP8_TOL
    _check_forward(rc, W, tol=tol)
    _check_backward(rc, W, tol=tol)


@pytest.mark.parametrize("idx", [2, 3, 5])
def test_recompute_full_size_bit_identical(gpu_lib, idx):
    """Recompute mode against the saving mode at full size, every output and main_grad bit
    for bit: the 4096-token layer with BF16 and with MXFP8 routed weights (pointer tables),
    and the 6-expert share on the wide BF16 shapes; the saved context shrinks from the
    activations to the routing state."""
    cfg = gen.config(idx)
    ref = _dp(cfg)
    ref.forward()
    ref.backward()
    torch.cuda.synchronize()
    rc = _dp(cfg, recompute=True)
    print(f"[recompute] saved bytes {ref.layer.saved.numel()} -> {rc.layer.saved.numel()}", flush=True)
    rc.forward()
    rc.layer.workspace.fill_(0xFF)
    rc.backward()
    torch.cuda.synchronize()
    _assert_same_bits(ref, rc)


# ----------------------------------------------------------------------------------
# routing given as the router's fixed-width table (moe_forward_topk)
# ----------------------------------------------------------------------------------
def _check_table_state(dp, top_ref):
    """Stored table = the given one with invalid entries dropped; dispatch bit-exact."""
    cfg = dp.cfg
    st = {k: v.cpu().numpy() for k, v in dp.layer.routing_state().items()}
    counts, offsets, slot_of, slot_token = O.dispatch_index(top_ref, cfg.experts)
    S = int(offsets[-1])
    assert np.array_equal(st["top_experts"], top_ref)
    rw = np.where(top_ref >= 0, dp.np_rw, np.float32(0))
    assert np.array_equal(st["router_weights"].view(np.uint32), rw.view(np.uint32))
    assert np.array_equal(st["counts"], counts)
    assert np.array_equal(st["offsets"], offsets)
    assert np.array_equal(st["slot_of"], slot_of)
    assert np.array_equal(st["slot_token"][:S], slot_token)
    return int(st["status_word"][0])


@pytest.mark.parametrize("routed,layout,shape", [
    ("bf16", "single", (777, 384, 13, 4, 256)),
    ("mxfp8", "table", (300, 256, 6, 3, 128)),
])
def test_topk_table_input_matches_oracle_and_map_path(gpu_lib, routed, layout, shape):
    T, H, E, K, I = shape
    cfg = gen.custom(T, H, E, K, I, routed=routed, layout=layout, short_frac=0.1, short_max=max(1, K - 1),
                     idx=700 + T)
    top, rw = gen.routing_table(cfg)
    dp = _dp(cfg, routing_table=(top, rw))
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    assert _check_table_state(dp, top) == 0
    W = oracle_weights(dp)
    tol = BF16_TOL if routed == "bf16" else MXFP8_TOL
    ref = O.moe_forward_table(dp.np_x, top, rw, E, W)
    err = rel_err(to_f64(dp.out), ref)
    print(f"[parity] table out rel err {err:.3e}", flush=True)
    assert err <= tol
    g = O.moe_backward_table(dp.np_dy, dp.np_x, top, rw, E, W)
    dpr = dp.dprobs.cpu().numpy().astype(np.float64)
    assert dpr.shape == (T, K) and np.all(dpr[top < 0] == 0)
    assert rel_err(to_f64(dp.dx), g["dx"]) <= tol and rel_err(dpr, g["dprobs"]) <= tol
    # the dense-map call on the same decisions: same slots, so the weight gradients and
    # the probability gradients agree bit for bit; out and dx sum the routes in another
    # order, so only to rounding
    mp = _dp(cfg)
    mp.forward()
    mp.backward()
    torch.cuda.synchronize()
    for a, b in zip(dp.mg_r1_list + dp.mg_r2_list + [dp.mg_s1, dp.mg_s2],
                    mp.mg_r1_list + mp.mg_r2_list + [mp.mg_s1, mp.mg_s2]):
        assert torch.equal(_bits(a), _bits(b)), "main_grad differs between table and map input"
    dense = mp.dprobs.cpu().numpy()
    m = top >= 0
    dtab = np.zeros((T, K), np.float32)
    dtab[m] = dense[np.nonzero(m)[0], top[m]]
    assert np.array_equal(dtab.view(np.uint32), dp.dprobs.cpu().numpy().view(np.uint32))
    assert rel_err(to_f64(dp.out), to_f64(mp.out)) <= 1e-2


def test_topk_table_invalid_entries_are_dropped_and_reported(gpu_lib):
    T, E, K = 96, 6, 3
    cfg = gen.custom(T, 256, E, K, 128, idx=801)
    top, rw = gen.routing_table(cfg)
    bad = top.copy()
    bad[5, 0], bad[5, 1], bad[5, 2] = 2, 2, -1      # the same expert twice
    bad[40, 1] = E                                  # out of range
    bad[77, 2] = -7                                 # negative other than -1
    dp = _dp(cfg, routing_table=(bad, rw))
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    clean = bad.copy()
    clean[5, 1] = -1
    clean[40, 1] = -1
    clean[77, 2] = -1
    assert _check_table_state(dp, clean) == mk_status("MOE_ERR_ROUTE_INVALID")
    W = oracle_weights(dp)
    ref = O.moe_forward_table(dp.np_x, clean, rw, E, W)
    assert rel_err(to_f64(dp.out), ref) <= BF16_TOL


def mk_status(name):
    import moe_megakernel_amd as mk
    return getattr(mk, name)


def test_topk_table_full_size_full_tensors(gpu_lib):
    """4096 tokens, hidden 4096, 96 experts, top-4, inter 1024 from the router's table:
    every token's out, dx and router-weight gradients and the main_grad deltas of all 96
    routed experts and the shared expert against the oracle."""
    cfg = gen.config(2)
    top, rw = gen.routing_table(cfg)
    dp = _dp(cfg, routing_table=(top, rw))
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    assert _check_table_state(dp, top) == 0
    W = oracle_weights(dp)
    ref = O.moe_forward_table(dp.np_x, top, rw, cfg.experts, W)
    errs = {"out": rel_err(to_f64(dp.out), ref)}
    del ref
    g = O.moe_backward_table(dp.np_dy, dp.np_x, top, rw, cfg.experts, W)
    errs["dx"] = rel_err(to_f64(dp.dx), g["dx"])
    dpr = dp.dprobs.cpu().numpy().astype(np.float64)
    errs["dprobs"] = rel_err(dpr, g["dprobs"])
    assert np.all(dpr[np.asarray(top) < 0] == 0), "pad entries must get a zero gradient"
    I, H = cfg.inter, cfg.hidden
    for e in range(cfg.experts):
        d1 = to_f64(dp.mg_r1_list[e]) - dp.main_grad_start((2 * I, H), e)
        d2 = to_f64(dp.mg_r2_list[e]) - dp.main_grad_start((H, I), e)
        dg, du, dd = g["dW"][e]
        errs[f"gate{e}"], errs[f"up{e}"], errs[f"down{e}"] = rel_err(d1[:I], dg), rel_err(d1[I:], du), rel_err(d2, dd)
    s1 = to_f64(dp.mg_s1) - dp.main_grad_start((2 * I, H), 0)
    s2 = to_f64(dp.mg_s2) - dp.main_grad_start((H, I), 0)
    dg, du, dd = g["dW"]["shared"]
    errs["shared_gate"], errs["shared_up"], errs["shared_down"] = rel_err(s1[:I], dg), rel_err(s1[I:], du), rel_err(s2, dd)
    worst = max(errs, key=lambda k: errs[k])
    print(f"[parity] table input, full tensors: out {errs['out']:.3e} dx {errs['dx']:.3e} "
          f"dprobs {errs['dprobs']:.3e} worst {worst} {errs[worst]:.3e} (tol {BF16_TOL})", flush=True)
    bad = {k: v for k, v in errs.items() if not (v <= BF16_TOL)}
    assert not bad, f"over tolerance {BF16_TOL}: {bad}"


# ----------------------------------------------------------------------------------
# BF16 main_grad: the call's contribution is rounded to BF16, then added with one BF16
# rounding (the persistent accumulation is BF16)
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("routed,layout,shape", [
    ("bf16", "single", (512, 1024, 16, 4, 512)),
    ("mxfp8", "table", (300, 256, 6, 3, 128)),
])
def test_bf16_main_grad_matches_oracle(gpu_lib, routed, layout, shape):
    T, H, E, K, I = shape
    cfg = gen.config(1) if routed == "bf16" else gen.custom(
        T, H, E, K, I, routed=routed, layout=layout, short_frac=0.1, short_max=max(1, K - 1), idx=800 + T)
    dp = _dp(cfg, main_grad_dtype="bf16")
    assert dp.mg_s1.dtype == torch.bfloat16
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    W = oracle_weights(dp)
    tol = BF16_TOL if routed == "bf16" else MXFP8_TOL
    _check_backward(dp, W, tol=tol)
    if routed != "bf16":
        return
    # The same call with FP32 main_grad yields the GPU's own FP32 contribution (the K loop
    # is identical); the BF16 result must be bf16(before + bf16(contribution)) of it.  A
    # contribution within FP32 rounding of a BF16 rounding boundary may land one ulp away.
    dp32 = _dp(cfg, main_grad_dtype="fp32")
    dp32.forward()
    dp32.backward()
    torch.cuda.synchronize()
    match = []
    for e in range(E):
        for t16, t32, shape in ((dp.mg_r1_list[e], dp32.mg_r1_list[e], (2 * I, H)),
                                (dp.mg_r2_list[e], dp32.mg_r2_list[e], (H, I))):
            start = dp.main_grad_start(shape, e)
            model = O.main_grad_after(start, to_f64(t32) - start, "bf16")
            match.append(np.mean(to_f64(t16) == model))
    print(f"[parity] bf16 main_grad = bf16(before + bf16(fp32 contribution)): exact fraction min "
          f"{min(match):.5f}", flush=True)
    assert min(match) >= 0.999


def test_bf16_main_grad_full_size(gpu_lib):
    """The 4096-token BF16 layer with BF16 main_grad: every token's dx and dprobs and the
    main_grad deltas of all 96 routed experts and the shared expert against the oracle, and
    every routed main_grad element against bf16(before + bf16(contribution)) of the same
    call with FP32 main_grad."""
    cfg = gen.config(2)
    dp = _dp(cfg, main_grad_dtype="bf16")
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    W = oracle_weights(dp)
    _check_backward(dp, W)
    dp32 = _dp(cfg, main_grad_dtype="fp32")
    dp32.forward()
    dp32.backward()
    torch.cuda.synchronize()
    I, H = cfg.inter, cfg.hidden
    match = []
    for e in range(cfg.experts):
        for t16, t32, shape in ((dp.mg_r1_list[e], dp32.mg_r1_list[e], (2 * I, H)),
                                (dp.mg_r2_list[e], dp32.mg_r2_list[e], (H, I))):
            start = dp.main_grad_start(shape, e)
            model = O.main_grad_after(start, to_f64(t32) - start, "bf16")
            match.append(np.mean(to_f64(t16) == model))
    print(f"[parity] bf16 main_grad = bf16(before + bf16(fp32 contribution)): exact fraction min "
          f"{min(match):.5f}", flush=True)
    assert min(match) >= 0.999


# ----------------------------------------------------------------------------------
# the shared expert's output gate
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("routed,layout,shape", [
    ("bf16", "single", (777, 384, 13, 4, 256)),
    ("mxfp8", "table", (300, 256, 6, 3, 128)),
])
def test_shared_output_gate_matches_oracle(gpu_lib, routed, layout, shape):
    T, H, E, K, I = shape
    cfg = gen.custom(T, H, E, K, I, routed=routed, layout=layout, short_frac=0.1, short_max=max(1, K - 1),
                     idx=1000 + T)
    dp = _dp(cfg, shared_gate=True)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    assert W.shared_gate is not None
    tol = BF16_TOL if routed == "bf16" else MXFP8_TOL
    _check_forward(dp, W, tol=tol)
    errs = _check_backward(dp, W, tol=tol)
    print(f"[parity] gate weight gradient rel err {errs['shared_out_gate']:.3e}", flush=True)
    # recompute mode: the same bits
    rc = _dp(cfg, shared_gate=True, recompute=True)
    rc.forward()
    rc.layer.workspace.fill_(0xFF)
    rc.backward()
    torch.cuda.synchronize()
    _assert_same_bits(dp, rc)
    assert torch.equal(_bits(dp.mg_gate), _bits(rc.mg_gate))


def test_shared_output_gate_full_size_full_tensors(gpu_lib):
    """4096 tokens, hidden 4096, 96 experts, top-4, inter 1024 with the shared output gate:
    every token's out, dx and dprobs, the main_grad deltas of all 96 routed experts and the
    shared expert, and the gate weight's main_grad delta against the oracle."""
    cfg = gen.config(2)
    dp = _dp(cfg, shared_gate=True)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    W = oracle_weights(dp)
    _check_forward(dp, W)
    _check_backward(dp, W)


# ----------------------------------------------------------------------------------
# SwiGLU clamp (swiglu_limit > 0).  Whether a pre-activation is clamped is decided on its
# exact value in the oracle and on its FP32 value in the kernel; the gradient jumps there,
# so elementwise parity needs a limit that no pre-activation of the inputs lies within the
# FP32 accumulation error of.  The limit is chosen from the oracle's own pre-activations
# (never from GPU results).
# ----------------------------------------------------------------------------------
def _preacts(dp, W):
    """Every FC1 pre-activation (a, b) the layer computes, in FP64 from the oracle's weights
    (with the recipe's MXFP8 x for MXFP8 routed experts), flattened."""
    xs = O.bf16_decode(dp.np_x)
    xq = O.mx_quantize(xs) if W.mx_activations else xs
    top, _ = O.compact_routing(dp.np_rmap, dp.np_probs, dp.cfg.topk)
    a_all, b_all = [], []
    if W.shared is not None:
        a_all.append((xs @ W.shared[0].T).ravel())
        b_all.append((xs @ W.shared[1].T).ravel())
    for e in range(dp.cfg.experts):
        rows = np.nonzero((top == e).any(axis=1))[0]
        if len(rows):
            wg, wu, _ = W.routed(e)
            a_all.append((xq[rows] @ wg.T).ravel())
            b_all.append((xq[rows] @ wu.T).ravel())
    return np.sort(np.concatenate(a_all)), np.sort(np.abs(np.concatenate(b_all)))


def _gap(sorted_v, L):
    i = np.searchsorted(sorted_v, L)
    near = [abs(sorted_v[j] - L) for j in (i - 1, i) if 0 <= j < len(sorted_v)]
    return min(near) if near else np.inf


def _pick_limit(a_sorted, b_sorted, candidates, gap, min_clamped):
    """The first candidate limit with no pre-activation within `gap` of it that clamps at
    least min_clamped gate and linear inputs each."""
    for L in candidates:
        na = len(a_sorted) - np.searchsorted(a_sorted, L, side="right")
        nb = len(b_sorted) - np.searchsorted(b_sorted, L, side="right")
        if na >= min_clamped and nb >= min_clamped and _gap(a_sorted, L) > gap and _gap(b_sorted, L) > gap:
            return float(L), int(na), int(nb)
    raise AssertionError("no candidate limit clear of the pre-activations")


@pytest.mark.parametrize("routed,layout", [("bf16", "single"), ("mxfp8", "table")])
def test_swiglu_clamp_matches_oracle(gpu_lib, routed, layout):
    T, H, E, K, I = 300, 256, 6, 3, 128
    cfg = gen.custom(T, H, E, K, I, routed=routed, layout=layout, short_frac=0.1, short_max=2, idx=1100 + T)
    probe = _dp(cfg, backward=False)
    a_s, b_s = _preacts(probe, oracle_weights(probe))
    del probe
    L, na, nb = _pick_limit(a_s, b_s, np.arange(0.2, 0.6, 2.0 ** -10), 4e-6, len(a_s) // 10)
    print(f"[clamp] {routed} L={L}: {na} gate and {nb} linear inputs clamped", flush=True)
    dp = _dp(cfg, swiglu_limit=L)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    check_routing_state(dp)
    W = oracle_weights(dp)
    assert W.swiglu_limit == L
    _check_forward(dp, W, tol=tol_of(dp))
    _check_backward(dp, W, tol=tol_of(dp))


def test_swiglu_clamp_full_size_bf16(gpu_lib):
    """The 4096-token BF16 layer with a clamp: limit in the tail of the pre-activations,
    clear of every one of them by more than the FP32 accumulation error over 4096 terms;
    every token's out, dx and dprobs and the main_grad deltas of all 96 routed experts and
    the shared expert against the oracle."""
    cfg = gen.config(2)
    dp = _dp(cfg, backward=False)
    a_s, b_s = _preacts(dp, oracle_weights(dp))
    del dp
    L, na, nb = _pick_limit(a_s, b_s, np.arange(3.5, 6.0, 0.01), 2.5e-5, 300)
    del a_s, b_s
    print(f"[clamp] 4096-token layer L={L}: {na} gate and {nb} linear inputs clamped", flush=True)
    dp = _dp(cfg, swiglu_limit=L)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    W = oracle_weights(dp)
    _check_forward(dp, W)
    _check_backward(dp, W)


# ----------------------------------------------------------------------------------
# the options together: routed-only x recompute x table input x BF16 main_grad
# ----------------------------------------------------------------------------------
def test_feature_combinations_are_consistent(gpu_lib):
    """Relations that must hold exactly between the modes, on one set of inputs:
    recompute changes no bit; table input gives the map input's weight and probability
    gradients bit for bit; routed-only leaves the routed gradients unchanged bit for bit;
    BF16 main_grad is bf16(before + bf16(the FP32 run's contribution)).  Plus the oracle
    on the mode with every option on."""
    T, H, E, K, I = 300, 256, 6, 3, 128
    cfg = gen.custom(T, H, E, K, I, short_frac=0.1, short_max=2, idx=900)
    table = gen.routing_table(cfg)
    runs = {}
    for shared in (True, False):
        for rc in (False, True):
            for tab in (False, True):
                for mgd in ("fp32", "bf16"):
                    dp = _dp(cfg, shared=shared, recompute=rc, routing_table=table if tab else None,
                             main_grad_dtype=mgd)
                    dp.forward()
                    dp.backward()
                    runs[(shared, rc, tab, mgd)] = dp
    torch.cuda.synchronize()

    def dprobs_table(dp, tab):
        if tab:
            return dp.dprobs.cpu().numpy()
        dense = dp.dprobs.cpu().numpy()
        top = table[0]
        out = np.zeros(top.shape, np.float32)
        m = top >= 0
        out[m] = dense[np.nonzero(m)[0], top[m]]
        return out

    routed = lambda dp: dp.mg_r1_list + dp.mg_r2_list
    for key, dp in runs.items():
        shared, rc, tab, mgd = key
        base = runs[(shared, False, tab, mgd)]
        if rc:   # recompute: every output bit for bit
            _assert_same_bits(base, dp)
        if tab:  # table vs map: gradients of the weights and of the router weights
            mp = runs[(shared, rc, False, mgd)]
            for a, b in zip(routed(dp) + [dp.mg_s1, dp.mg_s2], routed(mp) + [mp.mg_s1, mp.mg_s2]):
                assert torch.equal(_bits(a), _bits(b))
            assert np.array_equal(dprobs_table(dp, True).view(np.uint32), dprobs_table(mp, False).view(np.uint32))
        if not shared:  # routed gradients do not depend on the shared expert
            fu = runs[(True, rc, tab, mgd)]
            for a, b in zip(routed(dp), routed(fu)):
                assert torch.equal(_bits(a), _bits(b))
            assert np.array_equal(dprobs_table(dp, tab).view(np.uint32), dprobs_table(fu, tab).view(np.uint32))
        if mgd == "bf16":   # per-element semantics against the FP32 run's contribution
            f32 = runs[(shared, rc, tab, "fp32")]
            match = []
            for e in range(E):
                for t16, t32, shape in ((dp.mg_r1_list[e], f32.mg_r1_list[e], (2 * I, H)),
                                        (dp.mg_r2_list[e], f32.mg_r2_list[e], (H, I))):
                    start = dp.main_grad_start(shape, e)
                    model = O.main_grad_after(start, to_f64(t32) - start, "bf16")
                    match.append(np.mean(to_f64(t16) == model))
            assert min(match) >= 0.999, (key, min(match))
    # every option on, against the oracle
    dp = runs[(False, True, True, "fp32")]
    W = O.Weights.from_bits(I, None, None, lambda e: dp.np_routed[e], "bf16")
    ref = O.moe_forward_table(dp.np_x, table[0], table[1], E, W)
    assert rel_err(to_f64(dp.out), ref) <= BF16_TOL
    g = O.moe_backward_table(dp.np_dy, dp.np_x, table[0], table[1], E, W)
    assert rel_err(to_f64(dp.dx), g["dx"]) <= BF16_TOL
    assert rel_err(dp.dprobs.cpu().numpy().astype(np.float64), g["dprobs"]) <= BF16_TOL
    for e in range(E):
        d2 = to_f64(dp.mg_r2_list[e]) - dp.main_grad_start((H, I), e)
        assert rel_err(d2, g["dW"][e][2]) <= BF16_TOL
