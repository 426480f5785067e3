"""Host-side checks of the test problems' plumbing (moe_inputs.device), built on the CPU:
the descriptors of padded row strides and of separate gate/up allocations point at the
right rows, the pads hold their fill, and every main_grad starts from the exact pattern.
The GPU tests rely on this plumbing; here it is checked without a GPU."""
import numpy as np
import pytest
import torch

import moe_inputs as gen


def _problem(routed, layout, sep, pad, mgd="fp32"):
    from moe_inputs.device import DeviceProblem
    cfg = gen.custom(96, 256, 4, 2, 128, routed=routed, layout=layout, short_frac=0.1, short_max=1, idx=1700)
    return cfg, DeviceProblem(cfg, device="cpu", main_grad_dtype=mgd, pad_bytes=pad, separate_gate_up=sep)


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("routed", ["bf16", "mxfp8"])
@pytest.mark.parametrize("layout", ["single", "table"])
@pytest.mark.parametrize("sep", [False, True])
@pytest.mark.parametrize("pad", [0, 48])
def test_descriptors_and_main_grad_starts(routed, layout, sep, pad):
    cfg, dp = _problem(routed, layout, sep, pad)
    H, I, E = cfg.hidden, cfg.inter, cfg.experts
    w, g = dp.weights, dp.main_grads
    elem = 1 if routed == "mxfp8" else 2
    assert w.routed_gate.data.ld == H + pad // elem and w.routed_down.data.ld == I + pad // elem
    assert w.shared_gate.data.ld == H + pad // 2
    assert (w.routed_gate.row_offset, w.routed_up.row_offset) == ((0, 0) if sep else (0, I))
    assert (w.shared_gate.row_offset, w.shared_up.row_offset) == ((0, 0) if sep else (0, I))
    where = lambda m: (m.base, m.table)
    assert (where(w.routed_gate.data) == where(w.routed_up.data)) == (not sep)
    if routed == "mxfp8":
        assert w.routed_gate.scale.ld == H // 32 + pad and w.routed_gate.col_scale.ld == H + pad
    assert g.routed_gate.ld == H + pad // 4 and g.routed_down.ld == I + pad // 4
    assert (g.routed_up.row_offset, g.shared_up.row_offset) == ((0, 0) if sep else (I, I))
    # main_grads: the exact starting pattern over each logical matrix, pads untouched
    assert np.array_equal(dp.mg_s1.numpy().astype(np.float64), dp.main_grad_start((2 * I, H), 0))
    assert np.array_equal(dp.mg_s2.numpy().astype(np.float64), dp.main_grad_start((H, I), 0))
    for e in range(E):
        assert np.array_equal(dp.mg_r1_list[e].numpy().astype(np.float64), dp.main_grad_start((2 * I, H), e))
        assert np.array_equal(dp.mg_r2_list[e].numpy().astype(np.float64), dp.main_grad_start((H, I), e))
    assert dp.main_grad_pads_untouched()


@pytest.mark.parametrize("sep", [False, True])
def test_bf16_weight_rows_and_pads(sep):
    """The routed and shared FC1 rows the descriptors reach hold the generated bits, in
    order, and every pad is NaN."""
    cfg, dp = _problem("bf16", "table", sep, 48)
    H, I, E = cfg.hidden, cfg.inter, cfg.experts
    pe = 48 // 2
    shared_parts = (dp.s1g, dp.s1u) if sep else (dp.s1,)
    s1 = np.concatenate([_u16(t) for t in shared_parts])
    assert s1.shape == (2 * I, H + pe)
    assert np.array_equal(s1[:, :H], dp.np_s1) and np.all(s1[:, H:] == 0xFFFF)
    kept = [t for t in dp._keep if t.dtype == torch.bfloat16 and t.dim() == 2 and t.shape[1] == H + pe]
    fc1 = [np.asarray(r["fc1"]) for r in dp.np_routed]
    if sep:   # per expert: the gate rows, then (after all gates) the up rows
        gates, ups = kept[:E], kept[E:2 * E]
        for e in range(E):
            assert np.array_equal(_u16(gates[e])[:, :H], fc1[e][:I])
            assert np.array_equal(_u16(ups[e])[:, :H], fc1[e][I:])
            assert np.all(_u16(gates[e])[:, H:] == 0xFFFF) and np.all(_u16(ups[e])[:, H:] == 0xFFFF)
    else:
        for e in range(E):
            assert np.array_equal(_u16(kept[e])[:, :H], fc1[e]) and np.all(_u16(kept[e])[:, H:] == 0xFFFF)
