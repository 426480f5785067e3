"""Places the seeded synthetic inputs of one configuration in GPU memory and
builds the C descriptors the library takes (caller-side plumbing: torch owns
every buffer).  Used by the GPU tests, the benchmark and the smoke entry.

Routed weights use the configuration's layout: "single" stores one grouped
tensor per projection ([E, 2I, H] and [E, H, I]); "table" gives every expert
its own allocations, handed over as device arrays of per-expert pointers.  In
both, gate and up are row views of the combined FC1 (row offsets 0 and I).
"""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as gen
import moe_megakernel_amd as mk


def _bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def _u8(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _padded(a: np.ndarray, pad_bytes: int) -> np.ndarray:
    """a with pad_bytes more bytes at the end of every row, set to all-ones bits (NaN for
    BF16, E4M3 and E8M0), so that a kernel reading a pad poisons its result."""
    if pad_bytes == 0:
        return a
    pe = pad_bytes // a.itemsize
    out = np.full(a.shape[:-1] + (a.shape[-1] + pe,), np.iinfo(a.dtype).max, dtype=a.dtype)
    out[..., :a.shape[-1]] = a
    return out


MAIN_GRAD_PAD_FILL = 7.0   # the pad columns of padded main_grad rows; no call may change them


def fill_main_grad_pattern(t: torch.Tensor, phase: int = 0) -> None:
    """In-place ((i mod 7) - 3) * 2^-10 over the flat index of t's logical elements, the
    same exact pattern as moe_inputs.main_grad_pattern, built on the device in slices."""
    if not t.is_contiguous():
        tmp = torch.empty(t.shape, dtype=t.dtype, device=t.device)
        fill_main_grad_pattern(tmp, phase)
        t.copy_(tmp)
        return
    flat = t.view(-1)
    n = flat.numel()
    step = 1 << 26
    for s in range(0, n, step):
        m = min(step, n - s)
        i = torch.arange(phase + s, phase + s + m, device=t.device, dtype=torch.int64)
        flat[s:s + m] = ((i % 7) - 3).to(torch.float32) * (2.0 ** -10)


class DeviceProblem:
    def __init__(self, cfg: gen.Config, device="cuda", threads: int = 8, backward: bool | None = None,
                 routing=None, main_grad_dtype: str = "fp32", shared: bool = True,
                 recompute: bool = False, routing_table=None, shared_gate: bool = False,
                 swiglu_limit: float = 0.0, pad_bytes: int = 0, separate_gate_up: bool = False):
        """routing: optional (probs [T,E] float32, routing_map [T,E] uint8) replacing the
        configuration's router output (edge cases).  main_grad_dtype: "fp32" or "bf16".
        shared=False: routed-only mode; the shared weight and main_grad descriptors are
        passed all zero (the library must not touch them).  recompute=True: MoE-layer
        recompute mode (saved holds the routing state only; the backward regenerates the
        activations).  routing_table: optional (top_experts [T,K] int32, router_weights
        [T,K] float32), the router's fixed-width table given to moe_forward_topk instead of
        the dense map; grad_probs is then [T,K].  shared_gate: the shared expert's output gate
        (a seeded [H] weight and its main_grad).  swiglu_limit: the SwiGLU clamp (0: none).
        pad_bytes: every weight and main_grad matrix (payload, scales, shared and routed) gets
        rows this many bytes longer than its columns (a multiple of 16), the pads filled with
        NaN bits (weights) or MAIN_GRAD_PAD_FILL (main_grad).  separate_gate_up: the gate and
        up halves of every FC1 weight (payload and scales, shared and routed) and of every FC1
        main_grad in allocations of their own, each described with row offset 0, instead of
        row views of one combined tensor; mg_s1 and mg_r1_list then return fresh [2I, H]
        concatenations of the two halves."""
        assert pad_bytes % 16 == 0
        self.pad_bytes = pad_bytes
        self.cfg = cfg
        self.device = device
        T, H, E, K, I = cfg.tokens, cfg.hidden, cfg.experts, cfg.topk, cfg.inter
        self.backward_enabled = cfg.backward if backward is None else backward
        probs, rmap = gen.routing(cfg) if routing is None else routing
        self.np_probs, self.np_rmap = probs, rmap
        self.table = routing_table is not None
        if self.table:
            self.np_top = np.ascontiguousarray(routing_table[0], dtype=np.int32)
            self.np_rw = np.ascontiguousarray(routing_table[1], dtype=np.float32)
        self.np_x = gen.hidden(cfg)
        self.np_dy = gen.grad_out(cfg) if self.backward_enabled else None
        self.np_s1, self.np_s2 = gen.shared_weights(cfg)
        self.np_routed = gen.routed_all(cfg, threads=threads)
        self.slots = int(rmap.sum()) if not self.table else int(
            sum(len({int(e) for e in row if 0 <= e < E}) for row in self.np_top))

        self.x = _bf16(self.np_x, device)
        self.probs = torch.from_numpy(probs).to(device)
        self.rmap = torch.from_numpy(rmap).to(device)
        if self.table:
            self.top = torch.from_numpy(self.np_top).to(device)
            self.rw = torch.from_numpy(self.np_rw).to(device)
        self.dy = _bf16(self.np_dy, device) if self.np_dy is not None else None
        self.sep = separate_gate_up
        if self.sep:
            self.s1g = _bf16(_padded(self.np_s1[:I], pad_bytes), device)
            self.s1u = _bf16(_padded(self.np_s1[I:], pad_bytes), device)
        else:
            self.s1 = _bf16(_padded(self.np_s1, pad_bytes), device)
        self.s2 = _bf16(_padded(self.np_s2, pad_bytes), device)
        ldp = lambda cols, elem: cols + pad_bytes // elem   # padded row stride in elements
        self._keep = []
        mx = cfg.routed == "mxfp8"
        dt = mk.MOE_MXFP8_E4M3 if mx else mk.MOE_BF16
        self.shared = shared
        self.gated = shared_gate
        flags = ((mk.MOE_FLAG_HAS_SHARED if shared else 0) | (mk.MOE_FLAG_RECOMPUTE if recompute else 0)
                 | (mk.MOE_FLAG_TOPK_ROUTING if self.table else 0) | (mk.MOE_FLAG_SHARED_GATE if shared_gate else 0))
        self.swiglu_limit = float(swiglu_limit)
        self.p = mk.problem(T, H, I, E, K, dt, flags=flags, swiglu_limit=self.swiglu_limit)

        def routed_mat(key, rows, cols, conv, elem_cols, rsel=slice(None)):
            """moe_mat for a routed tensor stored [E][rows][cols] (single) or per expert (table);
            rsel picks the rows of each expert's array that the tensor holds."""
            ld = ldp(elem_cols, self.np_routed[0][key].itemsize)
            if cfg.layout == "single":
                t = conv(_padded(np.stack([r[key][rsel] for r in self.np_routed]), pad_bytes), device)
                self._keep.append(t)
                return mk.mat(base=t, expert_stride=rows * ld, ld=ld), t
            ts = [conv(_padded(r[key][rsel], pad_bytes), device) for r in self.np_routed]
            tab = torch.tensor([int(t.data_ptr()) for t in ts], dtype=torch.int64, device=device)
            self._keep += ts + [tab]
            return mk.mat(table=tab, ld=ld), ts

        halves = (slice(0, I), slice(I, 2 * I))
        if not mx and self.sep:
            rg, ru = (mk.weight(mk.MOE_BF16, I, H, routed_mat("fc1", I, H, _bf16, H, rs)[0]) for rs in halves)
            fc2, _ = routed_mat("fc2", H, I, _bf16, I)
            rd = mk.weight(mk.MOE_BF16, H, I, fc2)
        elif not mx:
            fc1, self.fc1 = routed_mat("fc1", 2 * I, H, _bf16, H)
            fc2, self.fc2 = routed_mat("fc2", H, I, _bf16, I)
            rg = mk.weight(mk.MOE_BF16, I, H, fc1, row_offset=0)
            ru = mk.weight(mk.MOE_BF16, I, H, fc1, row_offset=I)
            rd = mk.weight(mk.MOE_BF16, H, I, fc2)
        elif self.sep:
            def half(h):
                rs, rc = halves[h], slice(h * I // 32, (h + 1) * I // 32)
                return mk.weight(dt, I, H, routed_mat("fc1", I, H, _u8, H, rs)[0], 0,
                                 routed_mat("fc1_s", I, H // 32, _u8, H // 32, rs)[0],
                                 routed_mat("fc1_c", I, H, _u8, H, rs)[0],
                                 routed_mat("fc1_cs", I // 32, H, _u8, H, rc)[0])
            rg, ru = half(0), half(1)
            fc2, _ = routed_mat("fc2", H, I, _u8, I)
            fc2s, _ = routed_mat("fc2_s", H, I // 32, _u8, I // 32)
            fc2c, _ = routed_mat("fc2_c", H, I, _u8, I)
            fc2cs, _ = routed_mat("fc2_cs", H // 32, I, _u8, I)
            rd = mk.weight(dt, H, I, fc2, 0, fc2s, fc2c, fc2cs)
        else:
            fc1, _ = routed_mat("fc1", 2 * I, H, _u8, H)
            fc1s, _ = routed_mat("fc1_s", 2 * I, H // 32, _u8, H // 32)
            fc1c, _ = routed_mat("fc1_c", 2 * I, H, _u8, H)
            fc1cs, _ = routed_mat("fc1_cs", 2 * I // 32, H, _u8, H)
            fc2, _ = routed_mat("fc2", H, I, _u8, I)
            fc2s, _ = routed_mat("fc2_s", H, I // 32, _u8, I // 32)
            fc2c, _ = routed_mat("fc2_c", H, I, _u8, I)
            fc2cs, _ = routed_mat("fc2_cs", H // 32, I, _u8, I)
            rg = mk.weight(dt, I, H, fc1, 0, fc1s, fc1c, fc1cs)
            ru = mk.weight(dt, I, H, fc1, I, fc1s, fc1c, fc1cs)
            rd = mk.weight(dt, H, I, fc2, 0, fc2s, fc2c, fc2cs)
        if shared and self.sep:
            sg = mk.weight(mk.MOE_BF16, I, H, mk.mat(base=self.s1g, ld=ldp(H, 2)))
            su = mk.weight(mk.MOE_BF16, I, H, mk.mat(base=self.s1u, ld=ldp(H, 2)))
            sd = mk.weight(mk.MOE_BF16, H, I, mk.mat(base=self.s2, ld=ldp(I, 2)))
        elif shared:
            sg = mk.weight(mk.MOE_BF16, I, H, mk.mat(base=self.s1, ld=ldp(H, 2)), row_offset=0)
            su = mk.weight(mk.MOE_BF16, I, H, mk.mat(base=self.s1, ld=ldp(H, 2)), row_offset=I)
            sd = mk.weight(mk.MOE_BF16, H, I, mk.mat(base=self.s2, ld=ldp(I, 2)))
        else:
            sg, su, sd = mk.moe_weight(), mk.moe_weight(), mk.moe_weight()
        self.weights = mk.moe_weights(sg, su, sd, rg, ru, rd)
        self.np_gate = gen.shared_gate_weight(cfg) if shared_gate else None
        if shared_gate:
            self.gate = _bf16(self.np_gate, device)
            self.weights.shared_out_gate = mk.weight(mk.MOE_BF16, 1, H, mk.mat(base=self.gate, ld=H))

        self.out = torch.empty(T, H, dtype=torch.bfloat16, device=device)
        self.layer = mk.Layer(self.p, device=device)
        if self.backward_enabled:
            self.dx = torch.empty(T, H, dtype=torch.bfloat16, device=device)
            self.dprobs = torch.empty(T, K if self.table else E, dtype=torch.float32, device=device)
            mgt = {"fp32": torch.float32, "bf16": torch.bfloat16}[main_grad_dtype]
            mgd = mk.MOE_BF16 if main_grad_dtype == "bf16" else mk.MOE_FP32
            eb = 2 if main_grad_dtype == "bf16" else 4
            lh, li = ldp(H, eb), ldp(I, eb)   # main_grad row strides

            def mg(*shape):
                """A main_grad buffer with padded rows: (the padded tensor, its logical view)."""
                t = torch.full(shape[:-1] + (shape[-1] + pad_bytes // eb,), MAIN_GRAD_PAD_FILL, dtype=mgt,
                               device=device)
                return t, t[..., :shape[-1]]
            self._mg_padded = []
            self.mg_gate = torch.empty(H, dtype=mgt, device=device)
            if self.sep:
                self._sep_main_grads(mg, mgd, lh, li)
            else:
                self._packed_main_grads(mg, mgd, lh, li)
            if shared_gate:
                self.main_grads.shared_out_gate = mk.grad(base=self.mg_gate, ld=H, dtype=mgd)

    def _packed_main_grads(self, mg, mgd, lh, li):
        """FC1 main_grads as one [2I, H] matrix per expert, gate and up as row views."""
        cfg, device = self.cfg, self.device
        H, E, I = cfg.hidden, cfg.experts, cfg.inter
        (p1, self._mg_s1), (p2, self.mg_s2) = mg(2 * I, H), mg(H, I)
        self._mg_padded += [p1, p2]
        if cfg.layout == "single":
            (p1, self.mg_r1), (p2, self.mg_r2) = mg(E, 2 * I, H), mg(E, H, I)
            self._mg_padded += [p1, p2]
            g1 = dict(base=p1, expert_stride=2 * I * lh)
            g2 = dict(base=p2, expert_stride=H * li)
            self._mg_r1_list = [self.mg_r1[e] for e in range(E)]
            self.mg_r2_list = [self.mg_r2[e] for e in range(E)]
        else:
            r1 = [mg(2 * I, H) for _ in range(E)]
            r2 = [mg(H, I) for _ in range(E)]
            self._mg_padded += [t for t, _ in r1 + r2]
            self._mg_r1_list = [v for _, v in r1]
            self.mg_r2_list = [v for _, v in r2]
            t1 = torch.tensor([int(t.data_ptr()) for t, _ in r1], dtype=torch.int64, device=device)
            t2 = torch.tensor([int(t.data_ptr()) for t, _ in r2], dtype=torch.int64, device=device)
            self._keep += [t1, t2]
            g1 = dict(table=t1)
            g2 = dict(table=t2)
        self.reset_main_grads()
        sh = ((mk.grad(base=self._mg_s1, ld=lh, row_offset=0, dtype=mgd),
               mk.grad(base=self._mg_s1, ld=lh, row_offset=I, dtype=mgd),
               mk.grad(base=self.mg_s2, ld=li, dtype=mgd)) if self.shared
              else (mk.moe_grad(), mk.moe_grad(), mk.moe_grad()))
        self.main_grads = mk.moe_main_grads(
            *sh,
            mk.grad(ld=lh, row_offset=0, dtype=mgd, **g1), mk.grad(ld=lh, row_offset=I, dtype=mgd, **g1),
            mk.grad(ld=li, dtype=mgd, **g2))

    def _sep_main_grads(self, mg, mgd, lh, li):
        """FC1 main_grads with the gate and up halves in allocations of their own."""
        cfg, device = self.cfg, self.device
        H, E, I = cfg.hidden, cfg.experts, cfg.inter
        (a, sg_), (b, su_), (c, self.mg_s2) = mg(I, H), mg(I, H), mg(H, I)
        self._mg_padded += [a, b, c]
        self._s1_parts = (sg_, su_)
        descs = []
        if cfg.layout == "single":
            (a, rg_), (b, ru_), (c, self.mg_r2) = mg(E, I, H), mg(E, I, H), mg(E, H, I)
            self._mg_padded += [a, b, c]
            self._r1_parts = [(rg_[e], ru_[e]) for e in range(E)]
            self.mg_r2_list = [self.mg_r2[e] for e in range(E)]
            descs = [dict(base=a, expert_stride=I * lh), dict(base=b, expert_stride=I * lh),
                     dict(base=c, expert_stride=H * li)]
        else:
            parts = [[mg(I, H) for _ in range(E)], [mg(I, H) for _ in range(E)], [mg(H, I) for _ in range(E)]]
            self._mg_padded += [t for lst in parts for t, _ in lst]
            self._r1_parts = [(parts[0][e][1], parts[1][e][1]) for e in range(E)]
            self.mg_r2_list = [v for _, v in parts[2]]
            for lst in parts:
                tab = torch.tensor([int(t.data_ptr()) for t, _ in lst], dtype=torch.int64, device=device)
                self._keep.append(tab)
                descs.append(dict(table=tab))
        self.reset_main_grads()
        sh = ((mk.grad(base=sg_, ld=lh, dtype=mgd), mk.grad(base=su_, ld=lh, dtype=mgd),
               mk.grad(base=self.mg_s2, ld=li, dtype=mgd)) if self.shared
              else (mk.moe_grad(), mk.moe_grad(), mk.moe_grad()))
        self.main_grads = mk.moe_main_grads(*sh, mk.grad(ld=lh, dtype=mgd, **descs[0]),
                                            mk.grad(ld=lh, dtype=mgd, **descs[1]),
                                            mk.grad(ld=li, dtype=mgd, **descs[2]))

    @property
    def mg_s1(self) -> torch.Tensor:
        """The shared FC1 main_grad as [2I, H] (a fresh concatenation with separate halves)."""
        return torch.cat(self._s1_parts) if self.sep else self._mg_s1

    @property
    def mg_r1_list(self) -> list:
        """Each routed expert's FC1 main_grad as [2I, H] (fresh concatenations with separate halves)."""
        return [torch.cat(p) for p in self._r1_parts] if self.sep else self._mg_r1_list

    # ------------------------------------------------------------------
    def reset_main_grads(self):
        """Every main_grad buffer starts from the exact pattern (expert e's phase = e), over
        the logical [2I, H] FC1 matrix also when its halves are separate."""
        def fill_fc1(dst, phase):
            if not self.sep:
                fill_main_grad_pattern(dst, phase)
                return
            g, u = dst
            tmp = torch.empty((2 * g.shape[0], g.shape[1]), dtype=g.dtype, device=g.device)
            fill_main_grad_pattern(tmp, phase)
            g.copy_(tmp[:g.shape[0]])
            u.copy_(tmp[g.shape[0]:])
        fill_fc1(self._s1_parts if self.sep else self._mg_s1, 0)
        fill_main_grad_pattern(self.mg_gate, 0)
        fill_main_grad_pattern(self.mg_s2, 0)
        r1 = self._r1_parts if self.sep else self._mg_r1_list
        for e, (a, b) in enumerate(zip(r1, self.mg_r2_list)):
            fill_fc1(a, e)
            fill_main_grad_pattern(b, e)

    def main_grad_pads_untouched(self) -> bool:
        """True when every pad column of the padded main_grad rows still holds its fill."""
        H, I = self.cfg.hidden, self.cfg.inter
        for t in self._mg_padded:
            cols = H if t.shape[-1] - self.pad_bytes // t.element_size() == H else I
            if not bool((t[..., cols:] == MAIN_GRAD_PAD_FILL).all()):
                return False
        return True

    def main_grad_start(self, shape, phase) -> np.ndarray:
        n = int(np.prod(shape))
        return gen.main_grad_pattern(n, phase).reshape(shape)

    def forward(self):
        if self.table:
            self.layer.forward_topk(self.x, self.top, self.rw, self.weights, self.out)
        else:
            self.layer.forward(self.x, self.probs, self.rmap, self.weights, self.out)
        return self.out

    def backward(self):
        self.layer.backward(self.dy, self.x, self.weights, self.dx, self.dprobs, self.main_grads)
