"""Host-side accounting of bench.py (no GPU): algorithmic flops and bytes per kernel,
the choice of the binding roofline, and the one-GPU guard."""
import json
import subprocess
import sys

import pytest

import bench
import moe_inputs as gen

ROOT = bench.ROOT


def test_gemm_flops_sum_to_the_layer_total():
    # forward 6 H I R, backward 12 H I R over R = slots + tokens rows
    cfg = gen.config(2)
    S = 16384
    w = bench.gemm_work(cfg, S)
    total = sum(f for f, _ in w.values())
    assert total == 18 * cfg.hidden * cfg.inter * (S + cfg.tokens)
    # routed-only mode drops the shared rows
    w0 = bench.gemm_work(cfg, S, shared=False)
    assert sum(f for f, _ in w0.values()) == 18 * cfg.hidden * cfg.inter * S


@pytest.mark.parametrize("shared", [True, False])
def test_blas_reference_shapes_carry_the_kernels_flops(shared):
    # with S a multiple of E (every expert the same rows), the library GEMMs of each token
    # kernel multiply exactly the flops the kernel is credited with
    cfg = gen.config(5)
    S = 16380                                # 6 experts x 2730 rows
    shapes = bench.blas_shapes(cfg, S, shared)
    w = bench.gemm_work(cfg, S, shared)
    assert set(shapes) == {"fc1_swiglu", "fc2", "dgrad_fc2_swiglu", "dgrad_fc1"}
    for k, gemms in shapes.items():
        assert sum(2 * B * M * K * N for B, M, K, N in gemms) == w[k][0], k
    # the 4096-token layer: 96 uniform products of round(16384 / 96) = 171 rows
    assert bench.blas_shapes(gen.config(2), 16384)["fc1_swiglu"][0] == (96, 171, 4096, 2048)


def test_wgrad_bytes_closed_form():
    # every FC1 main_grad element (E + 1 experts, 2I x H) read and written in FP32, plus the
    # bf16 dfc1 (2I) and input (H) rows of every slot and token read once
    cfg = gen.config(2)
    E, H, I, T, S = cfg.experts, cfg.hidden, cfg.inter, cfg.tokens, 16384
    assert bench.wgrad_fc1_bytes(cfg, S) == (E + 1) * 2 * I * H * 8 + (S + T) * (2 * I + H) * 2
    assert bench.wgrad_fc1_bytes(cfg, S, mg_bytes=2) == (E + 1) * 2 * I * H * 4 + (S + T) * (2 * I + H) * 2
    assert bench.wgrad_fc1_bytes(cfg, S, shared=False) == E * 2 * I * H * 8 + S * (2 * I + H) * 2


def test_row_kernel_bytes_closed_form():
    cfg = gen.config(2)
    H, T, K, E, S = cfg.hidden, cfg.tokens, cfg.topk, cfg.experts, 16384
    w = bench.row_work(cfg, S)
    # combine: every routed row and the shared row read, the output row written
    assert w["combine"] == (S + 2 * T) * 2 * H + T * K * 8
    assert w["dx_combine"] == w["combine"]
    # gather: dy once per token, y and dyw once per slot, the dense dprobs row
    assert w["gather_dy_dprob"] == 2 * H * T + 4 * H * S + 4 * E * T + T * K * 8
    assert "quantize_x" not in w
    mx = bench.row_work(gen.config(3), S)
    assert mx["gather_dy_dprob"] == w["gather_dy_dprob"] + S * (H + H // 32)
    assert mx["quantize_x"] == T * (3 * H + H // 32)
    assert "quantize_h" not in mx and "quantize_dfc1" not in mx      # fused into the GEMM epilogues
    g, g3 = bench.gemm_work(cfg, S), bench.gemm_work(gen.config(3), S)
    I = cfg.inter
    # the MXFP8 epilogues also write the routed rows' codes and scales of h and dfc1
    assert g3["fc1_swiglu"][1] - g["fc1_swiglu"][1] == pytest.approx(
        -(E * 2 * I * H + S * H) * (2 - 33 / 32) + S * I * 33 / 32)
    assert g3["dgrad_fc2_swiglu"][1] - g["dgrad_fc2_swiglu"][1] == pytest.approx(
        -(E * H * I + S * H) * (2 - 33 / 32) + S * 2 * I * 33 / 32)


def test_roofline_picks_the_binding_bound():
    # 4096-token layer: every GEMM is HBM-bound at the vendor peaks; the 6-expert share is
    # MFMA-bound (its weights are read once for about 2731 rows per expert)
    for idx, bound in ((2, "hbm"), (5, "mfma")):
        cfg = gen.config(idx)
        kt = {k: (1, 1.0) for k in bench.gemm_work(cfg, 16384)}
        r = bench.kernel_roofline(cfg, 16384, kt)
        for k in ("fc1_swiglu", "fc2", "dgrad_fc2_swiglu", "dgrad_fc1"):
            assert r[k]["bound"] == bound, (idx, k, r[k])
        assert r["wgrad_fc1"]["bound"] == ("hbm" if idx == 2 else "mfma")
        for v in r.values():
            assert 0 < v["frac"] < 1


def test_mxfp8_peak_mixes_routed_fp8_and_shared_bf16():
    cfg = gen.config(3)
    S, T = 16384, cfg.tokens
    p = bench.mfma_peak(cfg, "fc1_swiglu", S)
    assert bench.MFMA_PEAK["bf16"] < p < bench.MFMA_PEAK["mxfp8"]
    assert p == pytest.approx((S + T) / (S / bench.MFMA_PEAK["mxfp8"] + T / bench.MFMA_PEAK["bf16"]))
    assert bench.mfma_peak(cfg, "wgrad_fc1", S) == bench.MFMA_PEAK["bf16"]


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2
