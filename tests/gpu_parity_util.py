"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the oracle on the same bits."""
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


def oracle_weights(dp, mx_activations=False) -> "O.Weights":
    cfg = dp.cfg
    shared = getattr(dp, "shared", True)
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
