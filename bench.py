#!/usr/bin/env python3
"""Benchmark of the post-router MoE layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

One step = moe_forward + moe_backward over one batch of seeded synthetic input
(routing compaction, dispatch, routed + shared SwiGLU experts, combine, and the
backward with FP32 main_grad accumulation and the dense probability gradient).
Inputs are resident in HBM before the timed region.  Prints one JSON line.

The step time is the median of K per-step times (HIP events on the layer's stream between
consecutive steps, after W warm-up steps; 50 and 10 by default).  Throughput is
algorithmic TFLOPS: 18 * H * I * (S + T) flops per step, S = valid routed slots, T =
tokens (shared expert; 0 with --routed-only).  Per-kernel times come from a second timed
pass of K steps with the library's kernel timer on; the roofline object describes the
dominant kernel from them.  The cpu_baseline object times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK = {"bf16": 2516.6, "mxfp8": 5033.2}   # dense TFLOP/s, MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2,
                    help="workload index (2: 4096-token BF16 layer; 3: its MXFP8 form; 4: 8192-token "
                         "MXFP8 layer; 5, 6: one GPU's 6-expert share of layer 2 / 3 under 16-way EP)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--main-grad", choices=("fp32", "bf16"), default="fp32",
                    help="main_grad dtype (bf16: contribution rounded to BF16 before a BF16 reduction-store)")
    ap.add_argument("--routed-only", action="store_true",
                    help="no fused shared expert (the layer's routed terms only)")
    ap.add_argument("--recompute", action="store_true",
                    help="MoE-layer recompute: saved holds the routing state only; the backward "
                         "regenerates the activations (same flops counted: the recomputation is overhead)")
    ap.add_argument("--swiglu-limit", type=float, default=0.0, help="SwiGLU clamp limit (0: none)")
    ap.add_argument("--shared-gate", action="store_true",
                    help="the shared expert's output gate sigmoid(x . g) (its few flops are not counted)")
    ap.add_argument("--topk-input", action="store_true",
                    help="routing given as the router's fixed-width [T][K] table (moe_forward_topk)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="BF16 layers: also time the vendor BLAS (torch.mm / torch.bmm, hipBLASLt) on "
                         "the same token-GEMM shapes with uniform expert batches, as a yardstick")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device-to-device copy before the steps (a known-size "
                         "reference for the HBM byte counters)")
    return ap.parse_args()


def wgrad_fc1_bytes(cfg, slots, mg_bytes=4, shared=True):
    """Algorithmic HBM bytes of one launch of the FC1 weight-gradient kernel: every routed
    and shared FC1 main_grad element (2I x H per expert, mg_bytes each) read and written
    once, plus the dfc1 (2I) and input (H) bf16 rows of every routed slot and every token
    read once (without the shared expert: the routed terms only)."""
    E, H, I, T = cfg.experts, cfg.hidden, cfg.inter, cfg.tokens
    ns = 1 if shared else 0
    return (E + ns) * 2 * I * H * 2 * mg_bytes + (slots + ns * T) * (2 * I + H) * 2


def gemm_work(cfg, slots, shared=True, mg_bytes=4):
    """Algorithmic (flops, HBM bytes) per launch of each GEMM kernel of one step.  Rows are
    the routed slots plus, with the shared expert, the tokens.  Weights are read once per
    launch (MXFP8 routed: one E4M3 byte + 1/32 E8M0 byte per element, the copy the GEMM
    contracts along), every gathered activation row once per slot (the routed FP8 GEMMs
    read it quantised), every output row written once, main_grad read and written once."""
    E, H, I, T = cfg.experts, cfg.hidden, cfg.inter, cfg.tokens
    ns = 1 if shared else 0
    Rr, Rs = slots, ns * T
    R = Rr + Rs
    mx = cfg.routed == "mxfp8"
    q = 1 + 1 / 32 if mx else 2                          # routed weight / FP8 GEMM input bytes
    w1 = E * 2 * I * H * q + ns * 2 * I * H * 2
    w2 = E * H * I * q + ns * H * I * 2
    # MXFP8: FC1 also writes the routed rows' h codes + scales, the FC2 data gradient the
    # routed rows' dfc1 codes + scales (the quantisation is fused into their epilogues)
    hq = Rr * I * (1 + 1 / 32) if mx else 0
    dfq = Rr * 2 * I * (1 + 1 / 32) if mx else 0
    return {
        "fc1_swiglu": (4 * H * I * R, w1 + Rr * H * q + Rs * H * 2 + R * 3 * I * 2 + hq),
        "fc2": (2 * H * I * R, w2 + Rr * I * q + Rs * I * 2 + R * H * 2),
        "dgrad_fc2_swiglu": (2 * H * I * R, w2 + Rr * H * q + Rs * H * 2 + R * 2 * I * 2 * 2 + dfq),
        "dgrad_fc1": (4 * H * I * R, w1 + Rr * 2 * I * q + Rs * 2 * I * 2 + R * H * 2),
        "wgrad_fc1": (4 * H * I * R, wgrad_fc1_bytes(cfg, slots, mg_bytes, shared)),
        "wgrad_fc2": (2 * H * I * R, (E + ns) * H * I * 2 * mg_bytes + R * (H + I) * 2),
    }


def row_work(cfg, slots, shared=True, gate=False):
    """Algorithmic HBM bytes per launch of the row kernels (permute-, combine- and
    quantise-type work, all HBM-bound): every row they read or write touched once.
    S = valid routed slots, T = tokens; the routing indices and weights are included."""
    E, H, I, T, K = cfg.experts, cfg.hidden, cfg.inter, cfg.tokens, cfg.topk
    S, Ts = slots, (T if shared else 0)
    idx = T * K * 8                                     # slot_of + router weights
    w = {
        "combine": (S + Ts + T) * 2 * H + idx + (2 * T * H if gate else 0),
        "dx_combine": (S + Ts + T) * 2 * H + idx,
        "gather_dy_dprob": 2 * H * T + 4 * H * S + 4 * E * T + idx + (4 * H * T if gate else 0),
    }
    if cfg.routed == "mxfp8":
        w["gather_dy_dprob"] += S * (H + H // 32)
        w["quantize_x"] = T * (2 * H + H + H // 32)
    return w


def row_roofline(cfg, slots, ktimes, shared=True, gate=False):
    """Per row kernel: achieved algorithmic GB/s from its live average launch time and the
    fraction of the HBM peak."""
    res = {}
    for name, by in row_work(cfg, slots, shared, gate).items():
        n_l, tot = ktimes.get(name, (0, 0.0))
        if n_l == 0:
            continue
        ms = tot / n_l
        ach = by / (ms * 1e-3) / 1e9
        res[name] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "avg_launch_ms": round(ms, 4),
                     "alg_bytes_per_launch": int(by)}
    return res


def mfma_peak(cfg, kernel, slots, shared=True):
    """Dense MFMA peak (TFLOP/s) for a GEMM kernel: BF16, or for the routed FP8 GEMMs of
    an MXFP8 layer the flop-weighted harmonic mix of the FP8 peak (routed rows) and the
    BF16 peak (shared rows, which stay BF16).  Weight gradients run on BF16 operands."""
    if cfg.routed != "mxfp8" or kernel.startswith("wgrad"):
        return MFMA_PEAK["bf16"]
    rr, rs = slots, (cfg.tokens if shared else 0)
    return (rr + rs) / (rr / MFMA_PEAK["mxfp8"] + rs / MFMA_PEAK["bf16"])


def kernel_roofline(cfg, slots, ktimes, shared=True, mg_bytes=4):
    """Per GEMM kernel: the binding roofline (MFMA if its flops take longer at peak than
    its bytes at the HBM peak, else HBM), the achieved rate from its live average launch
    time, and the fraction of that peak."""
    res = {}
    for name, (fl, by) in gemm_work(cfg, slots, shared, mg_bytes).items():
        n_l, tot = ktimes.get(name, (0, 0.0))
        if n_l == 0:
            continue
        ms = tot / n_l
        pk = mfma_peak(cfg, name, slots, shared)
        if fl / (pk * 1e12) >= by / (HBM_PEAK_GBS * 1e9):
            ach = fl / (ms * 1e-3) / 1e12
            res[name] = {"bound": "mfma", "achieved": round(ach, 1), "peak": round(pk, 1), "unit": "TFLOP/s",
                         "frac": round(ach / pk, 4), "avg_launch_ms": round(ms, 4), "alg_flops_per_launch": fl,
                         "launches": n_l}
        else:
            ach = by / (ms * 1e-3) / 1e9
            res[name] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "avg_launch_ms": round(ms, 4),
                         "alg_bytes_per_launch": int(by), "launches": n_l}
    return res


def kernel_source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "moe_megakernel_amd", "csrc")
    for n in sorted(os.listdir(d)):
        with open(os.path.join(d, n), "rb") as f:
            h.update(n.encode() + f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources and this workload; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def hbm_calibration():
    """Achievable HBM rates on this GPU with plain streaming kernels (torch's copy and an
    in-place FP32 add over 1 GiB): context for the roofline's 8 TB/s vendor peak."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    res = {}
    for name, f, nbytes in (("copy_GBps", lambda: b.copy_(a), 8 * n), ("rmw_GBps", lambda: a.add_(1.0), 8 * n)):
        for _ in range(3):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            f()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(nbytes / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9, 1)
    del a, b
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, dp, n_tokens, shared=True):
    """The oracle, as it stands, on the first n_tokens tokens of the same workload
    (forward + backward incl. every routed expert's and the shared expert's weight
    gradients over those tokens)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O

    n = min(n_tokens, cfg.tokens)
    rm = dp.np_rmap[:n]
    pr = dp.np_probs[:n]
    W = O.Weights.from_bits(cfg.inter, dp.np_s1 if shared else None, dp.np_s2 if shared else None,
                            lambda e: dp.np_routed[e], cfg.routed)
    t0 = time.perf_counter()
    O.moe_forward(dp.np_x[:n], pr, rm, cfg.topk, W)
    O.moe_backward(dp.np_dy[:n], dp.np_x[:n], pr, rm, cfg.topk, W)
    dt = time.perf_counter() - t0
    s = int(rm.sum())
    flops = 18.0 * cfg.hidden * cfg.inter * (s + (n if shared else 0))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOPS", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus_visible": len(os.sched_getaffinity(0)),
            "sample": f"first {n} of {cfg.tokens} tokens ({s} routed slots), fp64 numpy oracle, "
                      f"forward+backward incl. all weight gradients; {dt:.1f} s"}


def blas_shapes(cfg, slots, shared=True):
    """The token GEMMs of one step as plain library GEMMs: per kernel a list of
    (batch, M, K, N) products A[M,K] B[K,N], the routed experts as one batch of E products
    of round(slots / E) rows each (uniform batches: the library has no grouped form with a
    row map), the shared expert as one product of T rows.  No gather, no epilogue."""
    E, H, I, T = cfg.experts, cfg.hidden, cfg.inter, cfg.tokens
    m = max(1, round(slots / E))
    kn = {"fc1_swiglu": (H, 2 * I), "fc2": (I, H), "dgrad_fc2_swiglu": (H, I), "dgrad_fc1": (2 * I, H)}
    out = {}
    for k, (K, N) in kn.items():
        out[k] = [(E, m, K, N)] + ([(1, T, K, N)] if shared else [])
    return out


def blas_reference(cfg, slots, shared=True, reps=20):
    """Median time of each token GEMM's library form (torch.bmm for the routed batch,
    torch.mm for the shared rows; BF16, contiguous operands, FP32 accumulation inside the
    library).  A yardstick for the grouped kernels, not part of the layer."""
    import numpy as np
    import torch
    res = {}
    for k, gemms in blas_shapes(cfg, slots, shared).items():
        tot_ms, tot_fl, parts = 0.0, 0.0, []
        for (B, M, K, N) in gemms:
            a = torch.randn(B, M, K, device="cuda", dtype=torch.bfloat16)
            b = torch.randn(B, K, N, device="cuda", dtype=torch.bfloat16)
            if B == 1:
                a2, b2 = a[0], b[0]
                f = lambda: torch.mm(a2, b2)
            else:
                f = lambda: torch.bmm(a, b)
            for _ in range(3):
                f()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                f()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = float(np.median(ts))
            fl = 2.0 * B * M * K * N
            parts.append({"batch": B, "M": M, "K": K, "N": N, "ms": round(ms, 4)})
            tot_ms += ms
            tot_fl += fl
            del a, b
        res[k] = {"ms": round(tot_ms, 4), "TFLOPS": round(tot_fl / (tot_ms * 1e-3) / 1e12, 1), "gemms": parts}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    import moe_inputs as gen
    import moe_megakernel_amd as mk
    from moe_inputs.device import DeviceProblem

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    mk.load()
    cfg = gen.config(args.config)
    t0 = time.time()
    shared = not args.routed_only
    dp = DeviceProblem(cfg, backward=True, main_grad_dtype=args.main_grad, shared=shared,
                       recompute=args.recompute,
                       routing_table=gen.routing_table(cfg) if args.topk_input else None,
                       shared_gate=args.shared_gate, swiglu_limit=args.swiglu_limit)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s: {cfg.name}", file=sys.stderr, flush=True)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        dp.forward()
        dp.backward()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Headline: K steps, synchronised on both sides, an event on the layer's stream between
    # consecutive steps; the step time is the median of the K per-step times.  No per-kernel
    # event is recorded in this region.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        evs[i].record()
        step()
    evs[-1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms = float(np.median(per_step))
    # Per-kernel times: a second timed pass of K steps with the library's kernel timer (HIP
    # events around every launch, on the stream the kernels run on).
    mk.moe_kernel_timer_read()                      # drop earlier records
    mk.moe_kernel_timer_enable(True)
    torch.cuda.synchronize()
    t_k = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed_k = time.perf_counter() - t_k
    mk.moe_kernel_timer_enable(False)
    ktimes = mk.moe_kernel_timer_read()

    slots = dp.slots
    n_shared = cfg.tokens if shared else 0
    flops = 18.0 * cfg.hidden * cfg.inter * (slots + n_shared)
    tflops = flops / (ms * 1e-3) / 1e12
    dtype = cfg.routed
    routed_fl = 18.0 * cfg.hidden * cfg.inter * slots
    shared_fl = 18.0 * cfg.hidden * cfg.inter * n_shared
    mfma_frac = (routed_fl / (MFMA_PEAK[dtype] * 1e12) + shared_fl / (MFMA_PEAK["bf16"] * 1e12)) / (ms * 1e-3)

    # the dominant kernel: the GEMM kernel with the largest share of the step
    krl = kernel_roofline(cfg, slots, ktimes, shared, 2 if args.main_grad == "bf16" else 4)
    dom = max(krl, key=lambda k: krl[k]["avg_launch_ms"] * krl[k]["launches"])
    plain = (args.main_grad == "fp32" and shared and not args.recompute and not args.topk_input
             and not args.shared_gate and args.swiglu_limit == 0)
    roofline = {"kernel": dom, **{k: v for k, v in krl[dom].items() if k != "launches"},
                "traffic": counter_traffic(dom, cfg.name) if plain else None}

    line = {
        "metric": "MoE layer fwd+bwd TFLOPS and % of MFMA peak, 4096 tokens, 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "ms_per_step_stats": {"median": round(ms, 4), "mean": round(elapsed / args.steps * 1e3, 4),
                              "min": round(per_step[0], 4), "max": round(per_step[-1], 4),
                              "kernel_timer_pass_mean": round(elapsed_k / args.steps * 1e3, 4)},
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "mfma_peak_frac": round(mfma_frac, 4),
        "config": {"workload": cfg.name, "tokens": cfg.tokens, "hidden": cfg.hidden,
                   "experts": cfg.experts, "topk": cfg.topk, "intermediate": cfg.inter,
                   "routed_slots": slots, "routed_weights": cfg.routed, "layout": cfg.layout,
                   "routing": cfg.routing, "main_grad": args.main_grad, "shared_expert": shared,
                   "recompute": bool(args.recompute), "routing_input": "table" if args.topk_input else "map",
                   "shared_gate": bool(args.shared_gate), "swiglu_limit": args.swiglu_limit, "saved_bytes": int(dp.layer.saved.numel()),
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "kernels_ms": {k: round(v[1] / max(v[0], 1), 4) for k, v in ktimes.items()},
        "kernels_roofline": {k: {"bound": v["bound"], "frac": v["frac"]} for k, v in krl.items()},
        "row_kernels_hbm": {k: {"achieved_GBps": v["achieved"], "frac": v["frac"]}
                            for k, v in row_roofline(cfg, slots, ktimes, shared, args.shared_gate).items()},
    }
    line["hbm_calibration"] = hbm_calibration()
    if args.blas_reference and cfg.routed == "bf16":
        line["blas_reference"] = blas_reference(cfg, slots, shared)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, dp, args.cpu_sample_tokens, shared)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
