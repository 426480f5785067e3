"""Regression pins: the oracle still reproduces the values it stored under
tests/golden/ (written by tests/golden/make_golden.py, which calls only the
oracle and the input generator)."""
import json
import os

import numpy as np

import moe_inputs as gen
from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "config0_oracle.json")


def test_config0_oracle_matches_stored_values():
    with open(GOLD) as f:
        g = json.load(f)
    cfg = gen.config(0)
    probs, rmap = gen.routing(cfg)
    top, rw = O.compact_routing(rmap, probs, cfg.topk)
    counts, offsets, slot_of, slot_token = O.dispatch_index(top, cfg.experts)
    assert top.tolist() == g["top_experts"]
    assert [[float(v).hex() for v in r] for r in rw] == g["router_weights_f32_hex"]
    assert counts.tolist() == g["counts"] and offsets.tolist() == g["offsets"]
    assert slot_of.tolist() == g["slot_of"] and slot_token.tolist() == g["slot_token"]
    # 3 of 64 tokens (5%) have a single route: their second column is -1
    assert sum(1 for r in g["top_experts"] if r[1] == -1) == 3
    x = gen.hidden(cfg)
    s1, s2 = gen.shared_weights(cfg)
    routed = [gen.routed_expert(cfg, e) for e in range(cfg.experts)]
    W = O.Weights.from_bits(cfg.inter, s1, s2, lambda e: routed[e], "bf16")
    out = O.moe_forward(x, probs, rmap, cfg.topk, W, tokens=g["sample_tokens"])
    ref = np.array([[float.fromhex(v) for v in r] for r in g["out_rows_f64_hex"]])
    assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max()


def test_worked_example_from_the_routing_rule():
    # Routing rule (Megatron-LM PR #6572, Design > Authoritative routing maps): a dense
    # [tokens, experts] map becomes a fixed-width table whose missing routes are -1, and
    # the probabilities at the listed routes are gathered.  Worked by hand for top-3:
    rmap = np.array([[0, 1, 0, 1, 1],
                     [1, 0, 0, 0, 0],
                     [0, 0, 0, 0, 0],
                     [0, 0, 1, 1, 0]], np.uint8)
    probs = rmap * np.float32(0.25)
    probs[0, 4] = np.float32(0.5)
    top, rw = O.compact_routing(rmap, probs, 3)
    assert top.tolist() == [[1, 3, 4], [0, -1, -1], [-1, -1, -1], [2, 3, -1]]
    assert rw.tolist() == [[0.25, 0.25, 0.5], [0.25, 0, 0], [0, 0, 0], [0.25, 0.25, 0]]
    counts, offsets, slot_of, slot_token = O.dispatch_index(top, 5)
    assert counts.tolist() == [1, 1, 1, 2, 1]
    assert offsets.tolist() == [0, 1, 2, 3, 5, 6]
    # expert 3 is used by tokens 0 and 3: slots 3 (token 0) and 4 (token 3), ascending tokens
    assert slot_of.tolist() == [[1, 3, 5], [0, -1, -1], [-1, -1, -1], [2, 4, -1]]
    assert slot_token.tolist() == [3, 0, 9, 1, 10, 2]
