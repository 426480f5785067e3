"""Pins for the CPU oracle against things other than itself: brute force on
tiny inputs, a dense formulation with torch autograd, closed forms, special
cases, finite differences and library decoders."""
import itertools

import numpy as np
import pytest
import torch

import moe_inputs as gen
from oracle import moe_oracle as O
from tests.dense_reference import dense_forward, dense_grads


# ----------------------------------------------------------------------------------
# storage decoders against torch's own dtypes and closed forms
# ----------------------------------------------------------------------------------
def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert O.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert O.e4m3_decode(np.array([0x01], np.uint8))[0] == 2.0 ** -9
    assert O.e4m3_decode(np.array([0x08], np.uint8))[0] == 2.0 ** -6


def test_e8m0_decode_matches_torch_and_closed_form():
    codes = np.arange(255, dtype=np.uint8)
    got = O.e8m0_decode(codes)
    assert np.array_equal(got, 2.0 ** (codes.astype(np.float64) - 127))
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert np.isnan(O.e8m0_decode(np.array([255], np.uint8))[0])


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 2 ** 16, 5000).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # skip inf/nan patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_decode(bits), ref)


def test_generator_bf16_rounding_matches_torch():
    a = np.random.default_rng(1).standard_normal(10000).astype(np.float32) * 3
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.to_bf16_bits(a), ref)


@pytest.mark.parametrize("axis", [0, 1])
def test_generator_mxfp8_against_torch_cast_and_oracle_decode(axis):
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 96)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                       # an all-zero block
    w[5, 3] = 448.0 * 2.0 ** -9           # an exact block maximum (power of two times 448)
    payload, scale = gen.mxfp8_quantize(w, axis=axis)
    if axis == 1:
        assert scale.shape == (64, 3)
        dec = O.mxfp8_decode_rowwise(payload, scale)
        sc = np.repeat(2.0 ** (scale.astype(np.float64) - 127), 32, axis=1)
    else:
        assert scale.shape == (2, 96)
        dec = O.mxfp8_decode_colwise(payload, scale)
        sc = np.repeat(2.0 ** (scale.astype(np.float64) - 127), 32, axis=0)
    # payload equals torch's round-to-nearest-even cast of the scaled values
    scaled = torch.from_numpy((w.astype(np.float64) / sc).astype(np.float32))
    ref_codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(payload & 0x7F, ref_codes & 0x7F)
    nz = w != 0
    assert np.array_equal((payload[nz] >> 7), (ref_codes[nz] >> 7))
    # block exponent: the scaled block maximum lies in (224, 448], so after rounding in [224, 448]
    mag = np.abs(O.e4m3_decode(payload))
    blocks = mag.reshape(64, 3, 32).max(2) if axis == 1 else mag.reshape(2, 32, 96).max(1)
    assert np.all((blocks == 0) | ((blocks >= 224) & (blocks <= 448)))
    # quantise -> dequantise relative error at most 2^-4 for normal-range values
    big = np.abs(w) > 2.0 ** -6 * sc
    rel = np.abs(dec[big] - w[big]) / np.abs(w[big])
    assert rel.max() <= 2.0 ** -4 + 1e-12
    assert np.all(dec[~nz] == 0)


def test_generator_is_deterministic_per_expert():
    cfg = gen.config(3)
    a = gen.routed_expert(cfg, 7)
    b = gen.routed_expert(cfg, 7)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    p1, m1 = gen.routing(cfg)
    p2, m2 = gen.routing(cfg)
    assert np.array_equal(p1, p2) and np.array_equal(m1, m2)


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4, 5, 6])
def test_generator_routing_shapes(idx):
    cfg = gen.config(idx)
    probs, rmap = gen.routing(cfg)
    T, E, K = cfg.tokens, cfg.experts, cfg.topk
    assert probs.shape == (T, E) and rmap.shape == (T, E)
    n = rmap.sum(1)
    assert n.max() <= K
    assert np.all(probs[rmap == 0] == 0)
    if cfg.routing == "balanced":
        c = rmap.sum(0)
        assert sorted(set(c.tolist())) == [T * K // E, T * K // E + 1]
        assert c.sum() == T * K and np.all(probs[rmap == 1] == np.float32(1.0 / K))
    else:
        short = int(round(cfg.short_frac * T))
        assert int((n < K).sum()) == short


# ----------------------------------------------------------------------------------
# compaction and dispatch indexing: brute force + invariants
# ----------------------------------------------------------------------------------
def test_compaction_every_row_pattern_e5_k3():
    E, K = 5, 3
    rows = np.array(list(itertools.product([0, 1], repeat=E)), dtype=np.uint8)
    probs = (np.arange(rows.size, dtype=np.float32).reshape(rows.shape) + 1) / 64
    ok = rows.sum(1) <= K
    for r, p, good in zip(rows, probs, ok):
        if not good:
            with pytest.raises(O.RouteOverflow):
                O.compact_routing(r[None], p[None], K)
            continue
        top, rw = O.compact_routing(r[None], p[None], K)
        valid = top[0][top[0] >= 0]
        assert set(valid.tolist()) == set(np.flatnonzero(r).tolist())
        assert list(valid) == sorted(valid)                       # ascending
        n = len(valid)
        assert np.all(top[0][:n] >= 0) and np.all(top[0][n:] == -1)  # -1 trailing
        assert np.array_equal(rw[0][:n], p[valid]) and np.all(rw[0][n:] == 0)


def _check_dispatch_invariants(top, E, rmap):
    counts, offsets, slot_of, slot_token = O.dispatch_index(top, E)
    T, K = top.shape
    assert np.array_equal(counts, rmap.sum(0).astype(np.int32))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    S = int(offsets[-1])
    valid = top >= 0
    assert S == valid.sum()
    assert np.all(slot_of[~valid] == -1)
    s = slot_of[valid]
    assert np.array_equal(np.sort(s), np.arange(S))                 # bijection onto [0, S)
    tk = np.flatnonzero(valid.reshape(-1))
    assert np.array_equal(slot_token[s], tk)                         # slot_token o slot_of = id
    for e in range(E):
        seg = slot_token[offsets[e]:offsets[e + 1]]
        assert np.all(top.reshape(-1)[seg] == e)                     # segment holds expert e
        assert np.all(np.diff(seg // K) > 0)                         # tokens ascend


@pytest.mark.parametrize("idx", [0, 1, 3])
def test_dispatch_invariants_on_configs(idx):
    cfg = gen.config(idx)
    probs, rmap = gen.routing(cfg)
    top, _ = O.compact_routing(rmap, probs, cfg.topk)
    _check_dispatch_invariants(top, cfg.experts, rmap)


def test_dispatch_brute_force_small():
    rng = np.random.default_rng(3)
    E, K, T = 4, 2, 9
    for _ in range(20):
        rmap = np.zeros((T, E), np.uint8)
        for t in range(T):
            m = rng.integers(0, K + 1)
            rmap[t, rng.choice(E, m, replace=False)] = 1
        top, _ = O.compact_routing(rmap, rmap.astype(np.float32), K)
        _check_dispatch_invariants(top, E, rmap)
        # brute force: list all (e, t, k) and sort lexicographically by (e, t)
        pairs = sorted((int(top[t, k]), t, k) for t in range(T) for k in range(K) if top[t, k] >= 0)
        _, _, _, slot_token = O.dispatch_index(top, E)
        assert [t * K + k for _, t, k in pairs] == slot_token.tolist()


# ----------------------------------------------------------------------------------
# forward / backward against the dense formulation (torch float64, autograd)
# ----------------------------------------------------------------------------------
def _small_problem(T, H, E, K, I, seed, short=0.0):
    cfg = gen.custom(T, H, E, K, I, short_frac=short, idx=seed)
    probs, rmap = gen.routing(cfg)
    x = gen.hidden(cfg)
    dy = gen.grad_out(cfg)
    s1, s2 = gen.shared_weights(cfg)
    routed = [gen.routed_expert(cfg, e) for e in range(E)]
    W = O.Weights.from_bits(I, s1, s2, lambda e: routed[e], "bf16")
    dense = dict(
        x=torch.from_numpy(O.bf16_decode(x)), dy=torch.from_numpy(O.bf16_decode(dy)),
        probs=torch.from_numpy(probs.astype(np.float64)), rmap=torch.from_numpy(rmap),
        shared=(torch.from_numpy(O.bf16_decode(s1)), torch.from_numpy(O.bf16_decode(s2))),
        routed=(torch.from_numpy(np.stack([O.bf16_decode(r["fc1"]) for r in routed])),
                torch.from_numpy(np.stack([O.bf16_decode(r["fc2"]) for r in routed]))))
    return cfg, probs, rmap, x, dy, W, dense


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("shape", [(16, 32, 4, 2, 16), (40, 64, 6, 3, 32)])
def test_forward_matches_dense_formulation(shape):
    cfg, probs, rmap, x, dy, W, d = _small_problem(*shape, seed=11, short=0.2)
    out = O.moe_forward(x, probs, rmap, cfg.topk, W)
    ref = dense_forward(d["x"], d["probs"], d["rmap"], d["shared"], d["routed"]).numpy()
    assert _rel(out, ref) < 1e-12


def test_forward_config0_matches_dense_formulation():
    cfg = gen.config(0)
    probs, rmap = gen.routing(cfg)
    x = gen.hidden(cfg)
    s1, s2 = gen.shared_weights(cfg)
    routed = [gen.routed_expert(cfg, e) for e in range(cfg.experts)]
    W = O.Weights.from_bits(cfg.inter, s1, s2, lambda e: routed[e], "bf16")
    out = O.moe_forward(x, probs, rmap, cfg.topk, W)
    ref = dense_forward(torch.from_numpy(O.bf16_decode(x)), torch.from_numpy(probs.astype(np.float64)),
                        torch.from_numpy(rmap),
                        (torch.from_numpy(O.bf16_decode(s1)), torch.from_numpy(O.bf16_decode(s2))),
                        (torch.from_numpy(np.stack([O.bf16_decode(r["fc1"]) for r in routed])),
                         torch.from_numpy(np.stack([O.bf16_decode(r["fc2"]) for r in routed])))).numpy()
    assert _rel(out, ref) < 1e-12


@pytest.mark.parametrize("shape", [(16, 32, 4, 2, 16), (24, 64, 5, 3, 32)])
def test_backward_matches_dense_autograd(shape):
    cfg, probs, rmap, x, dy, W, d = _small_problem(*shape, seed=12, short=0.25)
    g = O.moe_backward(dy, x, probs, rmap, cfg.topk, W)
    ref = dense_grads(d["x"], d["probs"], d["rmap"], d["shared"], d["routed"], d["dy"])
    assert _rel(g["dx"], ref["dx"].numpy()) < 1e-12
    assert _rel(g["dprobs"], ref["dprobs"].numpy()) < 1e-12
    I = cfg.inter
    for e in range(cfg.experts):
        dg, du, dd = g["dW"][e]
        assert _rel(np.concatenate([dg, du]), ref["drouted1"][e].numpy()) < 1e-12
        assert _rel(dd, ref["drouted2"][e].numpy()) < 1e-12
    dg, du, dd = g["dW"]["shared"]
    assert _rel(np.concatenate([dg, du]), ref["dshared1"].numpy()) < 1e-12
    assert _rel(dd, ref["dshared2"].numpy()) < 1e-12
    assert np.all(g["dprobs"][rmap == 0] == 0)
    assert I == d["shared"][1].shape[1]


@pytest.mark.parametrize("shape", [(16, 32, 4, 2, 16), (24, 64, 5, 3, 32)])
def test_routed_only_matches_dense_formulation(shape):
    """Routed-only mode (no shared expert) against the dense form without FFN_shared."""
    cfg, probs, rmap, x, dy, W, d = _small_problem(*shape, seed=19, short=0.25)
    Wr = O.Weights(None, W.routed)
    out = O.moe_forward(x, probs, rmap, cfg.topk, Wr)
    ref_out = dense_forward(d["x"], d["probs"], d["rmap"], None, d["routed"]).numpy()
    assert _rel(out, ref_out) < 1e-12
    g = O.moe_backward(dy, x, probs, rmap, cfg.topk, Wr)
    ref = dense_grads(d["x"], d["probs"], d["rmap"], None, d["routed"], d["dy"])
    assert _rel(g["dx"], ref["dx"].numpy()) < 1e-12
    assert _rel(g["dprobs"], ref["dprobs"].numpy()) < 1e-12
    for e in range(cfg.experts):
        dg, du, dd = g["dW"][e]
        assert _rel(np.concatenate([dg, du]), ref["drouted1"][e].numpy()) < 1e-12
        assert _rel(dd, ref["drouted2"][e].numpy()) < 1e-12
    assert "shared" not in g["dW"]
    # the fused layer is the routed-only layer plus one dense SwiGLU MLP on every token
    full = O.moe_forward(x, probs, rmap, cfg.topk, W)
    mlp = _textbook_swiglu(O.bf16_decode(x), np.concatenate(W.shared[:2]), W.shared[2])
    assert _rel(full - out, mlp) < 1e-12


def test_routed_only_edge_cases():
    cfg, probs, rmap, x, dy, W, d = _small_problem(8, 32, 1, 1, 16, seed=20)
    Wr = O.Weights(None, W.routed)
    xs = O.bf16_decode(x)
    # no route at all: output and every gradient are exactly zero
    z = np.zeros_like(rmap)
    assert np.all(O.moe_forward(x, probs, z, 1, Wr) == 0)
    g = O.moe_backward(dy, x, probs, z, 1, Wr)
    assert np.all(g["dx"] == 0) and np.all(g["dprobs"] == 0)
    assert all(np.all(m == 0) for m in g["dW"][0])
    # one expert, every token routed with weight 1: a single dense SwiGLU MLP
    out = O.moe_forward(x, np.ones_like(probs), np.ones_like(rmap), 1, Wr)
    wg, wu, wd = W.routed(0)
    assert _rel(out, _textbook_swiglu(xs, np.concatenate([wg, wu]), wd)) < 1e-13


def _table_problem(T, H, E, K, I, seed, short=0.3):
    cfg = gen.custom(T, H, E, K, I, short_frac=short, short_max=max(1, K - 1), idx=seed)
    top, rw = gen.routing_table(cfg)
    _, _, _, x, dy, W, d = _small_problem(T, H, E, K, I, seed=seed, short=short)
    # the table scattered into a dense map and probabilities (independent of the oracle)
    P = np.zeros((T, E))
    M = np.zeros((T, E), np.uint8)
    for t in range(T):
        for k in range(K):
            if top[t, k] >= 0:
                P[t, top[t, k]] = rw[t, k]
                M[t, top[t, k]] = 1
    return cfg, top, rw, x, dy, W, d, torch.from_numpy(P), torch.from_numpy(M)


@pytest.mark.parametrize("shape", [(16, 32, 4, 3, 16), (24, 64, 6, 4, 32)])
def test_table_input_matches_dense_autograd(shape):
    """Router table input (any order, -1 anywhere, junk weights at -1) against the dense
    autograd form built from the scattered table; dprobs is the [T, K] gather."""
    cfg, top, rw, x, dy, W, d, P, M = _table_problem(*shape, seed=21)
    assert (top == -1).any() and not np.all(np.diff(np.where(top < 0, 99, top), axis=1) >= 0)
    E, K = cfg.experts, cfg.topk
    out = O.moe_forward_table(x, top, rw, E, W)
    assert _rel(out, dense_forward(d["x"], P, M, d["shared"], d["routed"]).numpy()) < 1e-12
    g = O.moe_backward_table(dy, x, top, rw, E, W)
    ref = dense_grads(d["x"], P, M, d["shared"], d["routed"], d["dy"])
    assert _rel(g["dx"], ref["dx"].numpy()) < 1e-12
    want = np.zeros_like(g["dprobs"])
    for t in range(cfg.tokens):
        for k in range(K):
            if top[t, k] >= 0:
                want[t, k] = ref["dprobs"][t, top[t, k]].item()
    assert g["dprobs"].shape == (cfg.tokens, K)
    assert _rel(g["dprobs"], want) < 1e-12
    assert np.all(g["dprobs"][top < 0] == 0)
    for e in range(E):
        dg, du, dd = g["dW"][e]
        assert _rel(np.concatenate([dg, du]), ref["drouted1"][e].numpy()) < 1e-12
        assert _rel(dd, ref["drouted2"][e].numpy()) < 1e-12


def test_table_row_order_and_pad_weights_do_not_matter():
    cfg, top, rw, x, dy, W, d, P, M = _table_problem(12, 32, 5, 3, 16, seed=22)
    E = cfg.experts
    rng = np.random.default_rng(5)
    perm = np.stack([rng.permutation(cfg.topk) for _ in range(cfg.tokens)])
    top2 = np.take_along_axis(top, perm, axis=1)
    rw2 = np.take_along_axis(rw, perm, axis=1)
    rw2[top2 < 0] = 123.0
    assert np.array_equal(O.moe_forward_table(x, top, rw, E, W), O.moe_forward_table(x, top2, rw2, E, W))
    g1 = O.moe_backward_table(dy, x, top, rw, E, W)
    g2 = O.moe_backward_table(dy, x, top2, rw2, E, W)
    assert np.array_equal(g1["dx"], g2["dx"])
    assert np.array_equal(np.take_along_axis(g1["dprobs"], perm, axis=1), g2["dprobs"])


def test_check_table_rejects_invalid_entries():
    ok = np.array([[0, -1, 2], [-1, -1, -1]], np.int32)
    O.check_table(ok, 3)
    for bad in ([[0, 3, -1], [1, 2, 0]], [[0, -2, 1], [1, 2, 0]], [[1, 1, -1], [0, 2, -1]]):
        with pytest.raises(O.RouteInvalid):
            O.check_table(np.array(bad, np.int32), 3)


@pytest.mark.parametrize("shape", [(16, 32, 4, 2, 16), (24, 64, 5, 3, 32)])
def test_shared_output_gate_matches_dense_autograd(shape):
    """Shared output gate sigmoid(x . g) on the shared expert's output, against the dense
    autograd form (including the gradient of g)."""
    cfg, probs, rmap, x, dy, W, d = _small_problem(*shape, seed=23, short=0.2)
    gbits = gen.shared_gate_weight(cfg)
    gv = O.bf16_decode(gbits)
    Wg = O.Weights(W.shared, W.routed, shared_gate=gv)
    gt = torch.from_numpy(gv)
    out = O.moe_forward(x, probs, rmap, cfg.topk, Wg)
    assert _rel(out, dense_forward(d["x"], d["probs"], d["rmap"], d["shared"], d["routed"], gt).numpy()) < 1e-12
    g = O.moe_backward(dy, x, probs, rmap, cfg.topk, Wg)
    ref = dense_grads(d["x"], d["probs"], d["rmap"], d["shared"], d["routed"], d["dy"], gt)
    assert _rel(g["dx"], ref["dx"].numpy()) < 1e-12
    assert _rel(g["dprobs"], ref["dprobs"].numpy()) < 1e-12
    assert _rel(g["dW"]["shared_out_gate"], ref["dgate"].numpy()) < 1e-12
    dg, du, dd = g["dW"]["shared"]
    assert _rel(np.concatenate([dg, du]), ref["dshared1"].numpy()) < 1e-12
    assert _rel(dd, ref["dshared2"].numpy()) < 1e-12
    for e in range(cfg.experts):
        assert _rel(g["dW"][e][2], ref["drouted2"][e].numpy()) < 1e-12


def test_shared_output_gate_zero_weight_halves_the_shared_expert():
    """g = 0: every score is exactly 1/2, so out = routed + shared / 2, and the gradient of
    g is sum_t (1/4)(dy_t . shared_t) x_t."""
    cfg, probs, rmap, x, dy, W, d = _small_problem(12, 32, 4, 2, 16, seed=24)
    H = cfg.hidden
    Wz = O.Weights(W.shared, W.routed, shared_gate=np.zeros(H))
    xs = O.bf16_decode(x)
    shared = _textbook_swiglu(xs, np.concatenate(W.shared[:2]), W.shared[2])
    routed = O.moe_forward(x, probs, rmap, cfg.topk, O.Weights(None, W.routed))
    assert _rel(O.moe_forward(x, probs, rmap, cfg.topk, Wz), routed + 0.5 * shared) < 1e-13
    g = O.moe_backward(dy, x, probs, rmap, cfg.topk, Wz)
    dys = O.bf16_decode(dy)
    want = (0.25 * np.sum(dys * shared, axis=1)) @ xs
    assert _rel(g["dW"]["shared_out_gate"], want) < 1e-12


@pytest.mark.parametrize("limit", [0.05, 0.15])
def test_swiglu_clamp_matches_dense_autograd(limit):
    """SwiGLU clamp (gate pre-activation clamped above, linear one to [-L, L]) against the
    dense autograd form with torch.clamp; the limits clamp a large share of both."""
    cfg, probs, rmap, x, dy, W, d = _small_problem(24, 64, 5, 3, 32, seed=25, short=0.2)
    Wc = O.Weights(W.shared, W.routed, swiglu_limit=limit)
    xs = O.bf16_decode(x)
    a = xs @ W.shared[0].T
    b = xs @ W.shared[1].T
    assert (a > limit).mean() > 0.05 and (np.abs(b) > limit).mean() > 0.05
    out = O.moe_forward(x, probs, rmap, cfg.topk, Wc)
    ref_out = dense_forward(d["x"], d["probs"], d["rmap"], d["shared"], d["routed"], limit=limit).numpy()
    assert _rel(out, ref_out) < 1e-12
    g = O.moe_backward(dy, x, probs, rmap, cfg.topk, Wc)
    ref = dense_grads(d["x"], d["probs"], d["rmap"], d["shared"], d["routed"], d["dy"], limit=limit)
    assert _rel(g["dx"], ref["dx"].numpy()) < 1e-12
    assert _rel(g["dprobs"], ref["dprobs"].numpy()) < 1e-12
    for e in range(cfg.experts):
        dg, du, dd = g["dW"][e]
        assert _rel(np.concatenate([dg, du]), ref["drouted1"][e].numpy()) < 1e-12
        assert _rel(dd, ref["drouted2"][e].numpy()) < 1e-12
    dg, du, dd = g["dW"]["shared"]
    assert _rel(np.concatenate([dg, du]), ref["dshared1"].numpy()) < 1e-12


def test_swiglu_clamp_limits_reduce_to_closed_forms():
    """A limit above every pre-activation changes nothing; the clamped product itself is
    silu(min(a, L)) clamp(b, -L, L) with derivatives that vanish where clamped."""
    cfg, probs, rmap, x, dy, W, d = _small_problem(12, 32, 4, 2, 16, seed=26)
    big = O.Weights(W.shared, W.routed, swiglu_limit=1e6)
    assert np.array_equal(O.moe_forward(x, probs, rmap, cfg.topk, big), O.moe_forward(x, probs, rmap, cfg.topk, W))
    a = np.array([-3.0, -0.5, 0.2, 0.5, 2.0])
    b = np.array([-2.0, 0.4, -0.4, 1.5, 0.1])
    h, dha, dhb = O.swiglu_clamped(a, b, 0.5)
    sig = lambda v: 1.0 / (1.0 + np.exp(-v))
    ac = np.array([-3.0, -0.5, 0.2, 0.5, 0.5])
    bc = np.array([-0.5, 0.4, -0.4, 0.5, 0.1])
    assert np.allclose(h, ac * sig(ac) * bc, rtol=0, atol=1e-15)
    assert dha[4] == 0 and dha[3] != 0      # a = L still passes the gradient, a > L does not
    assert dhb[0] == 0 and dhb[3] == 0 and dhb[1] != 0
    # the decision is taken on the exact value: the smallest step past L is clamped, L itself
    # is not (torch.clamp's gradient passes inside the closed bounds)
    up, dn = np.nextafter(0.5, 1.0), np.nextafter(-0.5, -1.0)
    h2, dha2, dhb2 = O.swiglu_clamped(np.array([up, 0.5]), np.array([dn, -0.5]), 0.5)
    assert dha2[0] == 0 and dha2[1] != 0 and dhb2[0] == 0 and dhb2[1] != 0
    assert h2[0] == h2[1] == 0.5 * sig(0.5) * -0.5
    # derivatives of the unclamped region are those of silu(a) b
    assert np.allclose(dha[:4], bc[:4] * O.dsilu(a[:4]), rtol=1e-15, atol=0)
    assert np.allclose(dhb[1:3], a[1:3] * sig(a[1:3]), rtol=1e-15, atol=0)


def test_e4m3_round_matches_torch_cast():
    """RNE to E4M3 against torch's float8_e4m3fn cast on values across every binade,
    the subnormals, exact codes and their midpoints."""
    rng = np.random.default_rng(31)
    u = np.concatenate([rng.uniform(-448, 448, 20000),
                        np.ldexp(rng.uniform(0.5, 1.0, 20000), rng.integers(-12, 9, 20000)) * rng.choice([-1, 1], 20000),
                        O.e4m3_decode(np.arange(256, dtype=np.uint8))])
    codes = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.sort(codes[np.isfinite(codes) & (codes >= 0)])
    u = np.concatenate([u, 0.5 * (fin[1:] + fin[:-1]), -0.5 * (fin[1:] + fin[:-1])])
    u = u[np.isfinite(u) & (np.abs(u) <= 448)].astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(u).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.e4m3_round(u), ref)


def test_mx_block_exponent_and_quantize_closed_forms():
    rng = np.random.default_rng(32)
    amax = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 5000), rng.integers(-120, 120, 5000)),
                           [448.0, 448.0 * 2.0 ** 7, 449.0, 1.75, 1.75 * (1 + 2 ** -23), 0.0]])
    e = O.mx_block_exponent(amax)
    pos = amax > 0
    assert np.all(np.ldexp(amax[pos], -e[pos]) <= 448.0)
    assert np.all((np.ldexp(amax[pos], -(e[pos] - 1)) > 448.0) | (e[pos] == -127))
    assert e[-1] == -127 and O.mx_block_exponent(448.0) == 0 and O.mx_block_exponent(449.0) == 1
    v = rng.normal(0, 3, (4, 64))
    q = O.mx_quantize(v)
    for r in range(4):
        for blk in range(2):
            sl = slice(32 * blk, 32 * blk + 32)
            sc = 2.0 ** O.mx_block_exponent(np.abs(v[r, sl]).max())
            assert np.array_equal(q[r, sl], O.e4m3_round(v[r, sl] / sc) * sc)
    assert np.max(np.abs(q - v) / np.abs(v).max()) < 2 ** -3     # 3 fraction bits


def _torch_mx(v):
    """MXFP8 quantise-dequantise along the last axis with torch's own float8_e4m3fn cast
    (an implementation independent of the oracle's)."""
    v = torch.as_tensor(v, dtype=torch.float64)
    b = v.reshape(*v.shape[:-1], v.shape[-1] // 32, 32)
    amax = b.abs().amax(dim=-1, keepdim=True)
    # smallest e with amax 2^-e <= 448, searched over the exponent range
    es = torch.arange(-127, 128, dtype=torch.float64)
    ok = amax * torch.pow(2.0, -es) <= 448.0
    e = torch.where(ok, es, torch.full_like(es, 1e9)).amin(dim=-1, keepdim=True)
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0))
    q = (b * torch.pow(2.0, -e)).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64) * torch.pow(2.0, e)
    return q.reshape(v.shape)


def test_mx_activation_mode_matches_an_independent_recipe():
    """The oracle's MXFP8-activation mode (x, the BF16 h, the BF16 w dy and dfc1 quantised
    before the routed FP8 GEMMs) against the same recipe written with torch ops and torch's
    E4M3 cast, for the forward, dprobs and dx."""
    cfg = gen.custom(12, 64, 3, 2, 32, routed="mxfp8", idx=27)
    probs, rmap = gen.routing(cfg)
    x, dy = gen.hidden(cfg), gen.grad_out(cfg)
    s1, s2 = gen.shared_weights(cfg)
    routed = [gen.routed_expert(cfg, e) for e in range(3)]
    W = O.Weights.from_bits(32, s1, s2, lambda e: routed[e], "mxfp8", mx_activations=True)
    out = O.moe_forward(x, probs, rmap, 2, W)
    g = O.moe_backward(dy, x, probs, rmap, 2, W)
    xs = torch.from_numpy(O.bf16_decode(x))
    dys = torch.from_numpy(O.bf16_decode(dy))
    bf = lambda t: t.to(torch.bfloat16).to(torch.float64)
    I = 32
    ref = torch.zeros_like(xs)
    dx = torch.zeros_like(xs)
    dpr = torch.zeros(12, 3, dtype=torch.float64)
    sh = [torch.from_numpy(m) for m in W.shared]
    a = xs @ sh[0].T
    b = xs @ sh[1].T
    ref += (torch.nn.functional.silu(a) * b) @ sh[2].T
    for t in range(12):
        for e in range(3):
            if not rmap[t, e]:
                continue
            wg, wu, wd = (torch.from_numpy(m) for m in W.routed(e))
            tg, tu, td = (torch.from_numpy(m) for m in W.routed_t(e))
            xq = _torch_mx(xs[t:t + 1])
            a, b = xq @ wg.T, xq @ wu.T
            sg = torch.sigmoid(a)
            h = a * sg * b
            y = _torch_mx(bf(h)) @ wd.T
            w = float(probs[t, e])
            ref[t] += w * y[0]
            dpr[t, e] = (dys[t] * y[0]).sum()
            gh = _torch_mx(bf(w * dys[t:t + 1])) @ td
            da = gh * b * (sg * (1 + a * (1 - sg)))
            db = gh * (a * sg)
            dq = _torch_mx(bf(torch.cat([da, db], dim=1)))
            dx[t] += (dq[:, :I] @ tg + dq[:, I:] @ tu)[0]
    # the shared expert's data gradient (BF16, unquantised)
    a = xs @ sh[0].T
    b = xs @ sh[1].T
    sg = torch.sigmoid(a)
    gh = dys @ sh[2]
    dx += (gh * b * (sg * (1 + a * (1 - sg)))) @ sh[0] + (gh * a * sg) @ sh[1]
    assert _rel(out, ref.numpy()) < 1e-12
    assert _rel(g["dprobs"], dpr.numpy()) < 1e-12
    assert _rel(g["dx"], dx.numpy()) < 1e-12
    # and it is a different function from the plain mode (the quantisation is visible)
    Wp = O.Weights.from_bits(32, s1, s2, lambda e: routed[e], "mxfp8")
    assert _rel(O.moe_forward(x, probs, rmap, 2, Wp), out) > 1e-4


def test_sampled_rows_and_experts_equal_full_run():
    cfg, probs, rmap, x, dy, W, d = _small_problem(30, 32, 5, 2, 16, seed=13, short=0.2)
    full = O.moe_backward(dy, x, probs, rmap, cfg.topk, W)
    fo = O.moe_forward(x, probs, rmap, cfg.topk, W)
    rows = np.array([3, 17, 29])
    part = O.moe_backward(dy, x, probs, rmap, cfg.topk, W, tokens=rows, experts=[2], shared_grads=False)
    # equal up to BLAS summation order
    assert _rel(part["dx"], full["dx"][rows]) < 1e-13
    assert _rel(part["dprobs"], full["dprobs"][rows]) < 1e-13
    assert all(_rel(a, b) < 1e-13 for a, b in zip(part["dW"][2], full["dW"][2]))
    assert np.allclose(O.moe_forward(x, probs, rmap, cfg.topk, W, tokens=rows), fo[rows], rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------------
# special cases with closed forms or textbook results
# ----------------------------------------------------------------------------------
def _textbook_swiglu(x, w1, w2):
    x, w1, w2 = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (x, w1, w2))
    I = w2.shape[1]
    gu = torch.matmul(x, w1.t())
    return torch.matmul(torch.nn.functional.silu(gu[:, :I]) * gu[:, I:], w2.t()).numpy()


def test_all_false_map_gives_shared_expert_only():
    cfg, probs, rmap, x, dy, W, d = _small_problem(12, 32, 4, 2, 16, seed=14)
    z = np.zeros_like(rmap)
    out = O.moe_forward(x, np.zeros_like(probs), z, cfg.topk, W)
    s1 = np.concatenate(W.shared[:2])
    assert _rel(out, _textbook_swiglu(O.bf16_decode(x), s1, W.shared[2])) < 1e-13
    g = O.moe_backward(dy, x, np.zeros_like(probs), z, cfg.topk, W)
    assert np.all(g["dprobs"] == 0)
    assert all(np.all(m == 0) for e in range(cfg.experts) for m in g["dW"][e])


def test_single_route_with_unit_weight_is_expert_plus_shared():
    cfg, probs, rmap, x, dy, W, d = _small_problem(10, 32, 4, 2, 16, seed=15)
    rmap = np.zeros_like(rmap)
    probs = np.zeros_like(probs)
    es = np.arange(10) % 4
    rmap[np.arange(10), es] = 1
    probs[np.arange(10), es] = 1.0
    out = O.moe_forward(x, probs, rmap, cfg.topk, W)
    xs = O.bf16_decode(x)
    shared = _textbook_swiglu(xs, np.concatenate(W.shared[:2]), W.shared[2])
    for t in range(10):
        wg, wu, wd = W.routed(es[t])
        ref = _textbook_swiglu(xs[t:t + 1], np.concatenate([wg, wu]), wd)[0] + shared[t]
        assert _rel(out[t], ref) < 1e-13


def test_one_expert_top1_is_two_dense_mlps():
    cfg, probs, rmap, x, dy, W, d = _small_problem(8, 32, 1, 1, 16, seed=16)
    probs = np.ones_like(probs)
    rmap = np.ones_like(rmap)
    out = O.moe_forward(x, probs, rmap, 1, W)
    xs = O.bf16_decode(x)
    wg, wu, wd = W.routed(0)
    ref = (_textbook_swiglu(xs, np.concatenate([wg, wu]), wd)
           + _textbook_swiglu(xs, np.concatenate(W.shared[:2]), W.shared[2]))
    assert _rel(out, ref) < 1e-13


def test_zero_down_projection_leaves_shared_only_and_linearity_in_w():
    cfg, probs, rmap, x, dy, W, d = _small_problem(12, 32, 4, 2, 16, seed=17)
    zero = O.Weights(W.shared, lambda e: (W.routed(e)[0], W.routed(e)[1], np.zeros_like(W.routed(e)[2])))
    out0 = O.moe_forward(x, probs, rmap, cfg.topk, zero)
    s = _textbook_swiglu(O.bf16_decode(x), np.concatenate(W.shared[:2]), W.shared[2])
    assert _rel(out0, s) < 1e-13
    p1 = probs.astype(np.float64)
    o0 = O.moe_forward(x, 0 * p1, rmap, cfg.topk, W)
    o1 = O.moe_forward(x, p1, rmap, cfg.topk, W)
    o2 = O.moe_forward(x, 2 * p1, rmap, cfg.topk, W)
    assert _rel(o2 - o1, o1 - o0) < 1e-12


def test_pad_routes_contribute_exactly_zero():
    cfg, probs, rmap, x, dy, W, d = _small_problem(12, 32, 4, 3, 16, seed=18, short=0.5)
    assert (rmap.sum(1) < 3).any()
    # probabilities off the map must never be read: poisoning them changes nothing
    poisoned = probs.copy()
    poisoned[rmap == 0] = np.float32(1e30)
    assert np.array_equal(O.moe_forward(x, probs, rmap, 3, W), O.moe_forward(x, poisoned, rmap, 3, W))
    g1 = O.moe_backward(dy, x, probs, rmap, 3, W)
    g2 = O.moe_backward(dy, x, poisoned, rmap, 3, W)
    assert np.array_equal(g1["dx"], g2["dx"])


# ----------------------------------------------------------------------------------
# backward by central finite differences on the forward (float64 inputs)
# ----------------------------------------------------------------------------------
def test_backward_matches_finite_differences():
    T, H, E, K, I = 4, 8, 4, 2, 4
    rng = np.random.default_rng(21)
    x = rng.standard_normal((T, H))
    dy = rng.standard_normal((T, H))
    rmap = np.array([[1, 0, 1, 0], [0, 1, 0, 0], [1, 1, 0, 0], [0, 0, 0, 0]], np.uint8)
    probs = rng.uniform(0.1, 0.9, (T, E)) * rmap
    w1 = [rng.standard_normal((2 * I, H)) * 0.5 for _ in range(E + 1)]
    w2 = [rng.standard_normal((H, I)) * 0.5 for _ in range(E + 1)]

    def weights(w1, w2):
        return O.Weights((w1[E][:I], w1[E][I:], w2[E]), lambda e: (w1[e][:I], w1[e][I:], w2[e]))

    def loss(x, probs, w1, w2):
        return float(np.sum(dy * O.moe_forward_f64(x, probs, rmap, K, weights(w1, w2))))

    g = O.moe_backward_f64(dy, x, probs, rmap, K, weights(w1, w2))
    h = 1e-6

    def fd(get, setv):
        v0 = get()
        setv(v0 + h)
        lp = loss(x, probs, w1, w2)
        setv(v0 - h)
        lm = loss(x, probs, w1, w2)
        setv(v0)
        return (lp - lm) / (2 * h)

    num = np.zeros_like(x)
    for i in range(T):
        for j in range(H):
            num[i, j] = fd(lambda: x[i, j], lambda v: x.__setitem__((i, j), v))
    assert _rel(g["dx"], num) < 1e-6
    nump = np.zeros_like(probs)
    for i in range(T):
        for e in range(E):
            if rmap[i, e]:
                nump[i, e] = fd(lambda: probs[i, e], lambda v: probs.__setitem__((i, e), v))
    assert _rel(g["dprobs"], nump) < 1e-6
    assert np.all(g["dprobs"][rmap == 0] == 0)
    for e in list(range(E)) + ["shared"]:
        idx = E if e == "shared" else e
        n1 = np.zeros_like(w1[idx])
        for a in range(2 * I):
            for b in range(H):
                n1[a, b] = fd(lambda: w1[idx][a, b], lambda v: w1[idx].__setitem__((a, b), v))
        n2 = np.zeros_like(w2[idx])
        for a in range(H):
            for b in range(I):
                n2[a, b] = fd(lambda: w2[idx][a, b], lambda v: w2[idx].__setitem__((a, b), v))
        dg, du, dd = g["dW"][e]
        scale = max(np.abs(n1).max(), 1e-3)
        assert np.abs(np.concatenate([dg, du]) - n1).max() / scale < 1e-6, e
        scale2 = max(np.abs(n2).max(), 1e-3)
        assert np.abs(dd - n2).max() / scale2 < 1e-6, e


def test_mxfp8_weights_use_rowwise_forward_and_colwise_dgrad():
    cfg = gen.custom(8, 64, 2, 1, 32, routed="mxfp8", idx=22)
    probs, rmap = gen.routing(cfg)
    x = gen.hidden(cfg)
    dy = gen.grad_out(cfg)
    s1, s2 = gen.shared_weights(cfg)
    routed = [gen.routed_expert(cfg, e) for e in range(2)]
    W = O.Weights.from_bits(32, s1, s2, lambda e: routed[e], "mxfp8")
    for e in range(2):
        fg, fu, fd_ = W.routed(e)
        tg, tu, td = W.routed_t(e)
        m1, m2 = gen.routed_master(cfg, e)
        # both decodes approximate the same master within E4M3's half-ulp
        for dec, m in ((np.concatenate([fg, fu]), m1), (np.concatenate([tg, tu]), m1), (fd_, m2), (td, m2)):
            assert np.abs(dec - m).max() <= 2.0 ** -4 * np.abs(m).max()
        # E4M3 keeps 3 mantissa bits whatever the power-of-two block scale, so the two
        # decodes differ only where an element falls into one copy's subnormal range
    # the dense formulation with the rowwise decode reproduces the oracle's forward
    out = O.moe_forward(x, probs, rmap, 1, W)
    d_r1 = torch.from_numpy(np.stack([np.concatenate(W.routed(e)[:2]) for e in range(2)]))
    d_r2 = torch.from_numpy(np.stack([W.routed(e)[2] for e in range(2)]))
    ref = dense_forward(torch.from_numpy(O.bf16_decode(x)), torch.from_numpy(probs.astype(np.float64)),
                        torch.from_numpy(rmap),
                        (torch.from_numpy(O.bf16_decode(s1)), torch.from_numpy(O.bf16_decode(s2))),
                        (d_r1, d_r2)).numpy()
    assert _rel(out, ref) < 1e-12
    # dx uses the columnwise decode: equal to autograd of the dense form built on it
    g = O.moe_backward(dy, x, probs, rmap, 1, W)
    t_r1 = torch.from_numpy(np.stack([np.concatenate(W.routed_t(e)[:2]) for e in range(2)]))
    t_r2 = torch.from_numpy(np.stack([W.routed_t(e)[2] for e in range(2)]))
    # a, b, h come from the rowwise weights, products with W^T from the columnwise ones:
    xs = O.bf16_decode(x)
    gs = O.bf16_decode(dy)
    dx_ref = np.array(dense_grads(torch.from_numpy(xs), torch.from_numpy(probs.astype(np.float64)),
                                  torch.from_numpy(rmap),
                                  (torch.from_numpy(O.bf16_decode(s1)), torch.from_numpy(O.bf16_decode(s2))),
                                  (d_r1, d_r2), torch.from_numpy(gs))["dx"])
    # the two decodes differ by at most the quantisation error, so dx agrees loosely
    assert _rel(g["dx"], dx_ref) < 0.1
    assert t_r1.shape == d_r1.shape and t_r2.shape == d_r2.shape


# ----------------------------------------------------------------------------------
# the pins catch planted mistakes (mutations applied to the oracle, on the CPU)
# ----------------------------------------------------------------------------------
def _swapped_gate_up(X, Wg, Wu, Wd, limit=0.0):
    a = X @ Wu.T
    b = X @ Wg.T
    h = O.silu(a) * b
    return a, b, h, h @ Wd.T


def _wrong_dsilu(z):
    return 1.0 / (1.0 + np.exp(-z))          # sigmoid instead of silu'


def _transposed_down(X, Wg, Wu, Wd, limit=0.0):
    a = X @ Wg.T
    b = X @ Wu.T
    h = O.silu(a) * b
    return a, b, h, h @ Wd[: h.shape[1]].T if Wd.shape[0] != Wd.shape[1] else h @ Wd


@pytest.mark.parametrize("mutant", ["swap_gate_up", "wrong_dsilu", "transposed_down"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    cfg, probs, rmap, x, dy, W, d = _small_problem(16, 32, 4, 2, 32, seed=31, short=0.2)
    if mutant == "swap_gate_up":
        monkeypatch.setattr(O, "swiglu_ffn", _swapped_gate_up)
    elif mutant == "wrong_dsilu":
        monkeypatch.setattr(O, "dsilu", _wrong_dsilu)
    else:
        monkeypatch.setattr(O, "swiglu_ffn", _transposed_down)
    ref = dense_grads(d["x"], d["probs"], d["rmap"], d["shared"], d["routed"], d["dy"])
    try:
        out = O.moe_forward(x, probs, rmap, cfg.topk, W)
        g = O.moe_backward(dy, x, probs, rmap, cfg.topk, W)
    except (ValueError, IndexError):
        return                                  # a shape error also exposes the mistake
    errs = [_rel(out, ref["out"].numpy()), _rel(g["dx"], ref["dx"].numpy()),
            _rel(g["dprobs"], ref["dprobs"].numpy())]
    assert max(errs) > 1e-3, errs


def _clamp_grad_leaks(a, b, limit=0.0):
    h, _, dhb = _ORIG_CLAMP(a, b, limit)
    return h, np.clip(b, -limit, limit) * O.dsilu(np.minimum(a, limit)), dhb   # no mask on a


def _clamp_one_sided_b(a, b, limit=0.0):
    ac = np.minimum(a, limit)
    bc = np.minimum(b, limit)                   # the lower bound of the linear input dropped
    return O.silu(ac) * bc, bc * O.dsilu(ac) * (a <= limit), O.silu(ac) * (b <= limit)


def _clamp_ties_clamped(a, b, limit=0.0):
    a_hi, b_out = a >= limit, np.abs(b) >= limit   # an input on a bound treated as clamped
    ac = np.where(a_hi, limit, a)
    bc = np.where(b_out, np.sign(b) * limit, b)
    return O.silu(ac) * bc, bc * O.dsilu(ac) * ~a_hi, O.silu(ac) * ~b_out


_ORIG_CLAMP = O.swiglu_clamped


@pytest.mark.parametrize("mutant", ["grad_leaks", "one_sided_b", "ties_clamped"])
def test_planted_clamp_mistakes_are_caught(monkeypatch, mutant):
    """Each plausible mistake in the clamp fails its pins: the dense autograd form with
    torch.clamp, or (for the decision at the bound itself) the closed forms."""
    if mutant == "ties_clamped":
        monkeypatch.setattr(O, "swiglu_clamped", _clamp_ties_clamped)
        _, dha, dhb = O.swiglu_clamped(np.array([0.5]), np.array([-0.5]), 0.5)
        assert dha[0] == 0 and dhb[0] == 0     # what the closed-form pin rejects
        return
    limit = 0.15
    cfg, probs, rmap, x, dy, W, d = _small_problem(24, 64, 5, 3, 32, seed=25, short=0.2)
    Wc = O.Weights(W.shared, W.routed, swiglu_limit=limit)
    monkeypatch.setattr(O, "swiglu_clamped", _clamp_grad_leaks if mutant == "grad_leaks" else _clamp_one_sided_b)
    out = O.moe_forward(x, probs, rmap, cfg.topk, Wc)
    g = O.moe_backward(dy, x, probs, rmap, cfg.topk, Wc)
    ref = dense_grads(d["x"], d["probs"], d["rmap"], d["shared"], d["routed"], d["dy"], limit=limit)
    errs = [_rel(out, ref["out"].numpy()), _rel(g["dx"], ref["dx"].numpy()),
            _rel(g["dprobs"], ref["dprobs"].numpy())]
    assert max(errs) > 1e-3, errs


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(21)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130, 3 * 2.0 ** -134,
                         0.0, 65504.0, 1.0 + 2.0 ** -8 + 2.0 ** -20]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_main_grad_reduction_store_closed_forms():
    # the contribution is rounded first: 1 + (2^-8 + 2^-20): bf16(c) = 2^-8, 1 + 2^-8 is a tie -> 1.0
    assert O.main_grad_after(np.array([1.0]), np.array([2.0 ** -8 + 2.0 ** -20]), "bf16")[0] == 1.0
    # without that first rounding the exact sum would round up to 1 + 2^-7
    assert O.bf16_round(np.array([1.0 + 2.0 ** -8 + 2.0 ** -20]))[0] == 1.0 + 2.0 ** -7
    assert O.main_grad_after(np.array([1.0]), np.array([3 * 2.0 ** -8]), "bf16")[0] == 1.0 + 2.0 ** -6
    assert O.main_grad_after(np.array([0.5]), np.array([0.25]), "fp32")[0] == 0.75
    with pytest.raises(ValueError):
        O.main_grad_after(np.array([0.0]), np.array([0.0]), "fp16")
