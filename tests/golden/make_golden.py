"""Writes the stored expected values under tests/golden/ by calling only the
oracle (and the seeded input generator).  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import moe_inputs as gen            # noqa: E402
from oracle import moe_oracle as O  # noqa: E402

SAMPLE_TOKENS = [0, 7, 21, 40, 63]


def config0():
    cfg = gen.config(0)
    probs, rmap = gen.routing(cfg)
    top, rw = O.compact_routing(rmap, probs, cfg.topk)
    counts, offsets, slot_of, slot_token = O.dispatch_index(top, cfg.experts)
    x = gen.hidden(cfg)
    s1, s2 = gen.shared_weights(cfg)
    routed = [gen.routed_expert(cfg, e) for e in range(cfg.experts)]
    W = O.Weights.from_bits(cfg.inter, s1, s2, lambda e: routed[e], "bf16")
    out = O.moe_forward(x, probs, rmap, cfg.topk, W, tokens=SAMPLE_TOKENS)
    return {
        "what": "config 0 (64 tokens, hidden 256, 8 experts, top-2, inter 128, BF16): routing "
                "table, dispatch indexing and forward rows, as computed by the oracle",
        "top_experts": top.tolist(),
        "router_weights_f32_hex": [[float(v).hex() for v in r] for r in rw],
        "counts": counts.tolist(), "offsets": offsets.tolist(),
        "slot_of": slot_of.tolist(), "slot_token": slot_token.tolist(),
        "sample_tokens": SAMPLE_TOKENS,
        "out_rows_f64_hex": [[float(v).hex() for v in r] for r in out],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "config0_oracle.json"), "w") as f:
        json.dump(config0(), f)
    print("wrote", os.path.join(HERE, "config0_oracle.json"))
