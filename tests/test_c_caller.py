"""The library driven from plain C: tests/c_caller/moe_c_caller.c allocates its own device
buffers and calls moe_forward and moe_backward through include/moe.h alone, with no Python
in the process.  The inputs come from the seeded generator (written to a file here); the
outputs must be bit-identical to the Python binding's on the same inputs, and within the
BF16 bound of the oracle."""
import os
import subprocess

import numpy as np
import pytest

import moe_inputs as gen
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALLER = os.path.join(ROOT, "tests", "c_caller", "moe_c_caller")
BF16_TOL = 2e-2


def test_c_caller_is_built_and_checks_its_arguments():
    # build() compiles it next to its source (host code only, so this CPU test builds it
    # when it is missing); without arguments it prints its usage and exits before any HIP call
    if not os.path.exists(CALLER):
        from moe_megakernel_amd.build import LIB, build_c_caller
        if not os.path.exists(LIB):
            pytest.skip("the library is not built")
        build_c_caller()
    r = subprocess.run([CALLER], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr


def _inputs(cfg):
    probs, rmap = gen.routing(cfg)
    x, dy = gen.hidden(cfg), gen.grad_out(cfg)
    s1, s2 = gen.shared_weights(cfg)
    routed = gen.routed_all(cfg)
    return probs, rmap, x, dy, s1, s2, routed


def _main_grad_starts(cfg):
    """The FP32 starting values the binding's test problems use, in the C caller's six
    buffers: shared expert phase 0, routed expert e phase e."""
    I, H, E = cfg.inter, cfg.hidden, cfg.experts
    pat = lambda rows, cols, ph: gen.main_grad_pattern(rows * cols, ph).reshape(rows, cols)
    s1, s2 = pat(2 * I, H, 0), pat(H, I, 0)
    r1 = [pat(2 * I, H, e) for e in range(E)]
    r2 = [pat(H, I, e) for e in range(E)]
    return [s1[:I], s1[I:], s2, np.stack([a[:I] for a in r1]), np.stack([a[I:] for a in r1]), np.stack(r2)]


def _write_inputs(path, cfg, data):
    probs, rmap, x, dy, s1, s2, routed = data
    T, H, E, K, I = cfg.tokens, cfg.hidden, cfg.experts, cfg.topk, cfg.inter
    parts = [np.array([T, H, E, K, I], np.int64), x.astype(np.uint16), probs.astype(np.float32),
             np.asarray(rmap).astype(np.uint8), s1[:I], s1[I:], s2,
             np.stack([r["fc1"][:I] for r in routed]), np.stack([r["fc1"][I:] for r in routed]),
             np.stack([r["fc2"] for r in routed]), dy.astype(np.uint16)]
    parts += [m.astype(np.float32) for m in _main_grad_starts(cfg)]
    with open(path, "wb") as f:
        for a in parts:
            np.ascontiguousarray(a).tofile(f)


def _read_outputs(path, cfg):
    T, H, E, I = cfg.tokens, cfg.hidden, cfg.experts, cfg.inter
    raw = open(path, "rb").read()
    pos = 0

    def take(dtype, n):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=pos)
        pos += a.nbytes
        return a

    st = take(np.int32, 3)
    out = take(np.uint16, T * H).reshape(T, H)
    dx = take(np.uint16, T * H).reshape(T, H)
    dpr = take(np.float32, T * E).reshape(T, E)
    shapes = [(I, H), (I, H), (H, I), (E, I, H), (E, I, H), (E, H, I)]
    mg = [take(np.float32, int(np.prod(s))).reshape(s) for s in shapes]
    assert pos == len(raw), "output file size"
    return st, out, dx, dpr, mg


@pytest.mark.gpu
def test_c_caller_matches_binding_and_oracle(gpu_lib, tmp_path):
    import torch
    from moe_inputs.device import DeviceProblem
    cfg = gen.custom(300, 256, 6, 3, 128, short_frac=0.1, short_max=2, idx=1400)
    T, H, E, I = cfg.tokens, cfg.hidden, cfg.experts, cfg.inter
    data = _inputs(cfg)
    fin, fout = str(tmp_path / "inputs.bin"), str(tmp_path / "outputs.bin")
    _write_inputs(fin, cfg, data)
    print(f"[case] C caller T={T} H={H} E={E} K={cfg.topk} I={I}", flush=True)
    r = subprocess.run([CALLER, fin, fout], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    st, out, dx, dpr, mg = _read_outputs(fout, cfg)
    assert list(st) == [0, 0, 0], st

    # the Python binding on the same generated problem: the same bits
    dp = DeviceProblem(cfg)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    bits = lambda t: t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(out, bits(dp.out))
    assert np.array_equal(dx, bits(dp.dx))
    assert np.array_equal(dpr.view(np.uint32), dp.dprobs.cpu().numpy().view(np.uint32))
    r1 = [dp.mg_r1_list[e].cpu().numpy() for e in range(E)]
    ref_mg = [dp.mg_s1.cpu().numpy()[:I], dp.mg_s1.cpu().numpy()[I:], dp.mg_s2.cpu().numpy(),
              np.stack([a[:I] for a in r1]), np.stack([a[I:] for a in r1]),
              np.stack([dp.mg_r2_list[e].cpu().numpy() for e in range(E)])]
    for a, b in zip(mg, ref_mg):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))

    # and the oracle on the generator's inputs
    probs, rmap, x, dy, s1, s2, routed = data
    W = O.Weights.from_bits(I, s1, s2, lambda e: routed[e], "bf16")
    ref = O.moe_forward(x, probs, rmap, cfg.topk, W)
    g = O.moe_backward(dy, x, probs, rmap, cfg.topk, W)
    rel = lambda a, b: float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))
    errs = {"out": rel(O.bf16_decode(out), ref), "dx": rel(O.bf16_decode(dx), g["dx"]),
            "dprobs": rel(dpr.astype(np.float64), g["dprobs"])}
    starts = _main_grad_starts(cfg)
    d = [m.astype(np.float64) - s.astype(np.float64) for m, s in zip(mg, starts)]
    sg, su, sd = g["dW"]["shared"]
    errs.update({"shared_gate": rel(d[0], sg), "shared_up": rel(d[1], su), "shared_down": rel(d[2], sd)})
    for e in range(E):
        dg, du, dd = g["dW"][e]
        if np.abs(dd).max() > 0:
            errs[f"gate{e}"] = rel(d[3][e], dg)
            errs[f"up{e}"] = rel(d[4][e], du)
            errs[f"down{e}"] = rel(d[5][e], dd)
    worst = max(errs, key=errs.get)
    print(f"[parity] C caller: out {errs['out']:.3e} dx {errs['dx']:.3e} dprobs {errs['dprobs']:.3e} "
          f"worst {worst} {errs[worst]:.3e}", flush=True)
    assert all(v <= BF16_TOL for v in errs.values()), errs
