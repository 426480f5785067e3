"""Seeded synthetic inputs for the post-router MoE layer.

This module is shared by the oracle and the HIP path and holds none of the
layer's arithmetic: it draws router outputs, activations and weights, rounds
them to the storage formats the layer consumes (BF16 bits, or an FP8 E4M3
payload with one E8M0 scale per 32 elements), and returns raw bits as numpy
arrays.  Decoding those bits back to numbers is the consumer's business.

Workload shapes follow the pages' Proxy and DSv4-Pro style runs (Megatron-LM
PR #6572, Validation): sequence 4096 with 96 routed experts, and a larger
top-6 layer; their data and weights are not available, so every tensor is
drawn from a fixed distribution with a fixed seed.

Every tensor has its own random stream, derived from the configuration's seed
and a tag (and the expert index for routed weights), so one expert's weights
can be regenerated alone, bit for bit, without drawing the rest.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Config", "CONFIGS", "config", "routing", "routing_table", "hidden", "grad_out",
    "shared_weights", "shared_gate_weight", "routed_expert", "routed_all", "main_grad_pattern",
    "to_bf16_bits", "mxfp8_quantize",
]


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    tokens: int
    hidden: int
    experts: int
    topk: int
    inter: int
    routed: str            # "bf16" or "mxfp8"
    layout: str            # "single" (one grouped tensor) or "table" (per-expert allocations)
    routing: str           # "softmax" or "balanced"
    logit_std: float
    short_frac: float      # fraction of tokens left with fewer than topk routes
    short_max: int         # such a token keeps m ~ U{1..short_max} of its top routes
    backward: bool

    @property
    def seed(self) -> int:
        return 1000 + self.idx


CONFIGS = {
    0: Config(0, "tiny-bf16-fwd", 64, 256, 8, 2, 128, "bf16", "single", "softmax", 1.0, 0.05, 1, False),
    1: Config(1, "small-bf16", 512, 1024, 16, 4, 512, "bf16", "single", "softmax", 1.0, 0.05, 1, True),
    2: Config(2, "proxy-4096-bf16-balanced", 4096, 4096, 96, 4, 1024, "bf16", "single", "balanced", 0.0, 0.0, 0, True),
    3: Config(3, "proxy-4096-mxfp8-skewed-table", 4096, 4096, 96, 4, 1024, "mxfp8", "table", "softmax", 1.5, 0.0, 0, True),
    4: Config(4, "large-8192-mxfp8", 8192, 7168, 64, 6, 2048, "mxfp8", "single", "softmax", 1.0, 0.02, 5, True),
    # one GPU's share of the 96-expert layer under 16-way expert parallelism: 6 local
    # experts, each receiving about 2731 of the 16384 routed rows of 4096 tokens
    5: Config(5, "ep16-share-4096-bf16", 4096, 4096, 6, 4, 1024, "bf16", "single", "balanced", 0.0, 0.0, 0, True),
    6: Config(6, "ep16-share-4096-mxfp8", 4096, 4096, 6, 4, 1024, "mxfp8", "single", "balanced", 0.0, 0.0, 0, True),
}


def config(idx: int) -> Config:
    return CONFIGS[idx]


def custom(tokens, hidden, experts, topk, inter, *, routed="bf16", layout="single",
           routing_kind="softmax", logit_std=1.0, short_frac=0.0, short_max=1,
           backward=True, idx=99) -> Config:
    """A configuration of any size for tests (ragged tails, edge cases)."""
    return Config(idx, "custom", tokens, hidden, experts, topk, inter, routed, layout,
                  routing_kind, logit_std, short_frac, short_max, backward)


# ----------------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------------
_TAGS = {"logits": 1, "x": 2, "shared_fc1": 3, "shared_fc2": 4, "routed_fc1": 5,
         "routed_fc2": 6, "short": 7, "dy": 8, "balanced": 9, "table": 10, "shared_gate": 11}


def _rng(cfg: Config, tag: str, sub: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(cfg.seed, spawn_key=(_TAGS[tag], sub))
    return np.random.Generator(np.random.PCG64(ss))


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


# ----------------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------------
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Values already scaled into [-448, 448] -> OCP E4M3FN codes, round half to even."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v) & (v != 0)).astype(np.uint8) << np.uint8(7)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int32)
    sub = a < 2.0 ** -6
    # subnormals: spacing 2^-9; a value that rounds up to 8 lands on the smallest normal
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int32)
    nrm = ~sub
    if np.any(nrm):
        an = a[nrm]
        _, p = np.frexp(an)                 # an = f * 2^p, f in [0.5, 1)
        ex = p - 1                          # an in [2^ex, 2^(ex+1))
        q = np.rint((an / np.ldexp(1.0, ex) - 1.0) * 8.0).astype(np.int32)
        carry = q == 8
        ex = ex + carry
        q = np.where(carry, 0, q)
        code[nrm] = ((ex + 7) << 3) | q
    if np.any(code > 0x7E):
        raise ValueError("E4M3 encode: value beyond the saturation bound")
    return code.astype(np.uint8) | sign


def _block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest e in [-127, 127] with amax <= 448 * 2^e (amax == 0 -> -127)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.ceil(np.log2(safe / 448.0)).astype(np.int64)
    # repair any off-by-one of the floating log2
    e = np.where(safe > 448.0 * np.ldexp(1.0, e), e + 1, e)
    e = np.where(safe <= 448.0 * np.ldexp(1.0, e - 1), e - 1, e)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127)


def mxfp8_quantize(w: np.ndarray, axis: int) -> tuple[np.ndarray, np.ndarray]:
    """Quantise a 2-D float32 matrix to E4M3 codes with one E8M0 scale per 32
    consecutive elements along `axis` (1: rowwise blocks along columns;
    0: columnwise blocks along rows).

    Returns (payload uint8, same shape as w) and (scale uint8: [R, C/32] for
    axis 1, [R/32, C] for axis 0).  Scale rule: the block exponent is the
    smallest power of two that brings the block's largest magnitude to at most
    448 (E4M3's largest finite value); the payload is the E4M3 rounding of
    value * 2^-e, which therefore never saturates.
    """
    w = np.asarray(w, dtype=np.float32)
    R, C = w.shape
    if axis == 1:
        if C % 32:
            raise ValueError("rowwise MXFP8 needs cols % 32 == 0")
        blk = w.reshape(R, C // 32, 32)
        e = _block_exponent(np.abs(blk).max(axis=2))                      # [R, C/32]
        scaled = blk.astype(np.float64) * np.ldexp(1.0, -e)[:, :, None]
        payload = _e4m3_encode(scaled).reshape(R, C)
    elif axis == 0:
        if R % 32:
            raise ValueError("columnwise MXFP8 needs rows % 32 == 0")
        blk = w.reshape(R // 32, 32, C)
        e = _block_exponent(np.abs(blk).max(axis=1))                      # [R/32, C]
        scaled = blk.astype(np.float64) * np.ldexp(1.0, -e)[:, None, :]
        payload = _e4m3_encode(scaled).reshape(R, C)
    else:
        raise ValueError("axis must be 0 or 1")
    return payload, (e + 127).astype(np.uint8)


# ----------------------------------------------------------------------------------
# router output
# ----------------------------------------------------------------------------------
def routing(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """Router output as the MoE layer receives it: dense probs [T, E] float32
    (zero off the map) and routing_map [T, E] uint8 (0/1)."""
    T, E, K = cfg.tokens, cfg.experts, cfg.topk
    probs = np.zeros((T, E), dtype=np.float32)
    rmap = np.zeros((T, E), dtype=np.uint8)
    if cfg.routing == "balanced":
        # every expert receives floor or ceil of T*K/E slots: slot s = t*K + k goes to
        # expert pi(s mod E); K consecutive residues are distinct while K <= E.
        if K > E:
            raise ValueError("balanced routing needs topk <= experts")
        rng = _rng(cfg, "balanced")
        pi = rng.permutation(E)
        tau = rng.permutation(T)
        s = np.arange(T * K).reshape(T, K)
        ex = pi[s % E]
        rows = np.repeat(tau, K)
        rmap[rows, ex.reshape(-1)] = 1
        probs[rows, ex.reshape(-1)] = np.float32(1.0 / K)
        return probs, rmap
    logits = _normal_f32(_rng(cfg, "logits"), (T, E), cfg.logit_std).astype(np.float64)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    # top-K, larger probability first; ties keep the lower expert index first
    order = np.argsort(-p, axis=1, kind="stable")[:, :K]
    keep = np.full((T, K), True)
    n_short = int(round(cfg.short_frac * T))
    if n_short:
        rs = _rng(cfg, "short")
        who = rs.choice(T, size=n_short, replace=False)
        m = rs.integers(1, cfg.short_max + 1, size=n_short) if cfg.short_max > 1 else np.ones(n_short, int)
        for t, mm in zip(who, m):
            keep[t, mm:] = False
    top_p = np.take_along_axis(p, order, axis=1)
    top_p = top_p / top_p.sum(axis=1, keepdims=True)   # renormalise over the K chosen
    rows = np.repeat(np.arange(T), K).reshape(T, K)
    rmap[rows[keep], order[keep]] = 1
    probs[rows[keep], order[keep]] = top_p[keep].astype(np.float32)  # dropped: prob 0, no renorm
    return probs, rmap


def shared_gate_weight(cfg: Config) -> np.ndarray:
    """The shared expert's output gate weight g ~ N(0, 0.02^2), BF16 bits [H] (x . g then
    spreads over about N(0, 0.0004 H): sigmoid scores across (0, 1))."""
    return to_bf16_bits(_normal_f32(_rng(cfg, "shared_gate"), (cfg.hidden,), 0.02))


def routing_table(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """The same routing decisions as routing(cfg) in the router's fixed-width form:
    top_experts int32 [T, K] and router_weights float32 [T, K].  Each row holds its
    listed experts and K - n entries of -1 at seeded random positions, in a seeded random
    order (a router's own order need not be ascending); the weight at -1 is a seeded
    random value, which the layer must ignore."""
    probs, rmap = routing(cfg)
    T, K = cfg.tokens, cfg.topk
    rng = _rng(cfg, "table")
    top = np.full((T, K), -1, dtype=np.int32)
    rw = rng.random((T, K)).astype(np.float32)
    for t in range(T):
        listed = np.nonzero(rmap[t])[0]
        pos = rng.permutation(K)[:len(listed)]
        top[t, pos] = listed
        rw[t, pos] = probs[t, listed]
    return top, rw


def hidden(cfg: Config) -> np.ndarray:
    """x ~ N(0, 1), BF16 bits [T, H]."""
    return to_bf16_bits(_normal_f32(_rng(cfg, "x"), (cfg.tokens, cfg.hidden), 1.0))


def grad_out(cfg: Config) -> np.ndarray:
    """Upstream gradient dy ~ N(0, 1), BF16 bits [T, H]."""
    return to_bf16_bits(_normal_f32(_rng(cfg, "dy"), (cfg.tokens, cfg.hidden), 1.0))


def shared_weights(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """Shared expert, always BF16: fc1 [2I, H] (gate rows then up rows), fc2 [H, I]."""
    fc1 = _normal_f32(_rng(cfg, "shared_fc1"), (2 * cfg.inter, cfg.hidden), 0.02)
    fc2 = _normal_f32(_rng(cfg, "shared_fc2"), (cfg.hidden, cfg.inter), 0.02)
    return to_bf16_bits(fc1), to_bf16_bits(fc2)


def routed_master(cfg: Config, e: int) -> tuple[np.ndarray, np.ndarray]:
    fc1 = _normal_f32(_rng(cfg, "routed_fc1", e), (2 * cfg.inter, cfg.hidden), 0.02)
    fc2 = _normal_f32(_rng(cfg, "routed_fc2", e), (cfg.hidden, cfg.inter), 0.02)
    return fc1, fc2


def routed_expert(cfg: Config, e: int) -> dict:
    """Routed expert e's weights in the configuration's storage format.

    bf16 : {"fc1": u16 [2I, H], "fc2": u16 [H, I]}
    mxfp8: {"fc1": u8 [2I,H], "fc1_s": u8 [2I, H/32], "fc1_c": u8 [2I,H], "fc1_cs": u8 [2I/32, H],
            "fc2": ..., "fc2_s": [H, I/32], "fc2_c": [H, I], "fc2_cs": [H/32, I]}
    Rowwise and columnwise copies are quantised from the same float32 master.
    """
    fc1, fc2 = routed_master(cfg, e)
    if cfg.routed == "bf16":
        return {"fc1": to_bf16_bits(fc1), "fc2": to_bf16_bits(fc2)}
    out = {}
    for name, w in (("fc1", fc1), ("fc2", fc2)):
        out[name], out[name + "_s"] = mxfp8_quantize(w, axis=1)
        out[name + "_c"], out[name + "_cs"] = mxfp8_quantize(w, axis=0)
    return out


def routed_all(cfg: Config, threads: int = 8) -> list[dict]:
    """All routed experts, generated in parallel (numpy releases the GIL).  The last three
    configurations' results are kept, so that several problems built on one configuration
    generate its weights once; callers must not write into the arrays."""
    if cfg in _ROUTED_CACHE:
        _ROUTED_CACHE[cfg] = _ROUTED_CACHE.pop(cfg)   # most recently used last
        return _ROUTED_CACHE[cfg]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        out = list(ex.map(lambda e: routed_expert(cfg, e), range(cfg.experts)))
    _ROUTED_CACHE[cfg] = out
    while len(_ROUTED_CACHE) > 3:
        _ROUTED_CACHE.pop(next(iter(_ROUTED_CACHE)))
    return out


_ROUTED_CACHE: dict = {}


def main_grad_pattern(n: int, phase: int = 0) -> np.ndarray:
    """A cheap, exactly representable non-zero starting main_grad: ((i mod 7) - 3) * 2^-10."""
    i = np.arange(phase, phase + n, dtype=np.int64)
    return (((i % 7) - 3).astype(np.float32) * np.float32(2.0 ** -10))


def valid_slots(rmap: np.ndarray) -> int:
    return int(np.count_nonzero(rmap))


def layer_flops(cfg: Config, slots: int, backward: bool | None = None) -> float:
    """Algorithmic flops: 6*H*I per routed slot and per token (shared) forward, twice that backward."""
    bwd = cfg.backward if backward is None else backward
    per = 18 if bwd else 6
    return float(per) * cfg.hidden * cfg.inter * (slots + cfg.tokens)

