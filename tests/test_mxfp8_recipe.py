"""The MXFP8 recipe's own error, on the CPU, with no GPU involved: the oracle with the
recipe's MXFP8 activation inputs (Weights.mx_activations) against the oracle with exact
activations, on the same weights and inputs, for many seeds of the MXFP8 test shapes.

The recipe (PR #6572, Supported configurations: MXFP8 routed experts) feeds each routed
FP8 GEMM MXFP8 operands, so x, the BF16 h, w dy and dfc1 are rounded to E4M3 in blocks of
32 sharing an E8M0 scale (3 fraction bits: up to 1/16 relative per element).  How far that
moves out, dx, dprobs and the weight gradients from the exact-activation result is a
property of the recipe, measured here.  Every seed is reported; none is chosen.

    python -m tests.test_mxfp8_recipe            # the distribution over 20 seeds per shape
    python -m tests.test_mxfp8_recipe --configs 3 4 --samples 20
                                                 # disjoint token samples of the full layers
"""
from __future__ import annotations

import argparse
import functools

import numpy as np
import pytest

import moe_inputs as gen
from oracle import moe_oracle as O

# the MXFP8 shapes of the GPU tests: (T, H, E, K, I, layout)
SHAPES = [(300, 256, 6, 3, 128, "table"), (520, 384, 9, 2, 256, "single")]
OUTPUTS = ("out", "dx", "dprobs", "w1", "w2")


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def _weights(cfg, routed, mx):
    s1, s2 = gen.shared_weights(cfg)
    return O.Weights.from_bits(cfg.inter, s1, s2, lambda e: routed[e], "mxfp8", mx_activations=mx)


def inputs(cfg):
    probs, rmap = gen.routing(cfg)
    return probs, rmap, gen.hidden(cfg), gen.grad_out(cfg), gen.routed_all(cfg)


def cached_weights(cfg, routed):
    """The exact-activation and the recipe oracle weights over one set of decoded experts,
    decoded once per expert and kept (for repeated calls on token samples)."""
    W0 = _weights(cfg, routed, False)
    fwd, bwd = functools.lru_cache(maxsize=None)(W0.routed), functools.lru_cache(maxsize=None)(W0.routed_t)
    return (O.Weights(W0.shared, fwd, bwd), O.Weights(W0.shared, fwd, bwd, mx_activations=True))


def recipe_error(cfg, tokens=None, experts=None, data=None, weights=None):
    """max|recipe - exact| / max|exact| per output (w1, w2: the worst expert)."""
    probs, rmap, x, dy, routed = data if data is not None else inputs(cfg)
    res = {}
    outs = []
    for mx in (False, True):
        W = weights[int(mx)] if weights is not None else _weights(cfg, routed, mx)
        out = O.moe_forward(x, probs, rmap, cfg.topk, W, tokens=tokens)
        g = O.moe_backward(dy, x, probs, rmap, cfg.topk, W, tokens=tokens, experts=experts, shared_grads=False)
        outs.append((out, g))
    (o0, g0), (o1, g1) = outs
    res["out"] = _rel(o1, o0)
    res["dx"] = _rel(g1["dx"], g0["dx"])
    res["dprobs"] = _rel(g1["dprobs"], g0["dprobs"])
    w1, w2 = [], []
    for e, (dg, du, dd) in g0["dW"].items():
        if np.abs(dd).max() == 0:
            continue
        mg, mu, md = g1["dW"][e]
        w1.append(_rel(np.concatenate([mg, mu]), np.concatenate([dg, du])))
        w2.append(_rel(md, dd))
    res["w1"] = max(w1) if w1 else 0.0
    res["w2"] = max(w2) if w2 else 0.0
    return res


def sweep(seeds=20):
    rows = []
    for j, (T, H, E, K, I, layout) in enumerate(SHAPES):
        for i in range(seeds):
            cfg = gen.custom(T, H, E, K, I, routed="mxfp8", layout=layout, short_frac=0.05,
                             short_max=max(1, K - 1), idx=2000 + 100 * j + i)
            rows.append(((T, H, E, K, I), recipe_error(cfg)))
    return rows


def summarize(rows, bound=6e-2):
    lines = []
    for shape in sorted({r[0] for r in rows}):
        errs = [r[1] for r in rows if r[0] == shape]
        cells = []
        for o in OUTPUTS:
            v = np.array([e[o] for e in errs])
            cells.append(f"{o} {v.min():.2e}/{np.median(v):.2e}/{v.max():.2e} (>{bound:g}: {int((v > bound).sum())})")
        lines.append(f"{shape} n={len(errs)}: " + "; ".join(cells))
    return lines


@pytest.mark.slow
def test_mxfp8_recipe_error_distribution():
    """The recipe moves every output, and by a bounded amount.  A wrong block exponent or a
    dropped quantisation point would show as 0 or as errors of order 1."""
    rows = sweep(20)
    for line in summarize(rows):
        print(line)
    for _, e in rows:
        for o in OUTPUTS:
            assert 0 < e[o] < 0.2, (o, e[o])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seeds", type=int, default=20)
    ap.add_argument("--configs", type=int, nargs="*", default=[])
    ap.add_argument("--samples", type=int, default=20)
    ap.add_argument("--sample-tokens", type=int, default=128)
    ap.add_argument("--no-cache", action="store_true", help="decode experts per call (less memory)")
    a = ap.parse_args()
    if not a.configs:
        for line in summarize(sweep(a.seeds)):
            print(line, flush=True)
        return
    for c in a.configs:
        cfg = gen.config(c)
        data = inputs(cfg)
        W = None if a.no_cache else cached_weights(cfg, data[4])
        perm = np.random.default_rng(c).permutation(cfg.tokens)
        errs = []
        for s in range(a.samples):
            toks = np.sort(perm[s * a.sample_tokens:(s + 1) * a.sample_tokens])
            errs.append(recipe_error(cfg, tokens=toks, experts=[], data=data, weights=W))
            print(f"config {c} sample {s}: " + " ".join(f"{k} {v:.3e}" for k, v in errs[-1].items()
                                                        if k in ("out", "dx", "dprobs")), flush=True)
        for o in ("out", "dx", "dprobs"):
            v = np.array([e[o] for e in errs])
            print(f"config {c} {o}: min {v.min():.3e} median {np.median(v):.3e} max {v.max():.3e}", flush=True)


if __name__ == "__main__":
    main()
