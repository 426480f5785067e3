"""The C-ABI library on a machine without a GPU: it loads, exports every symbol
include/moe.h declares, and rejects invalid arguments on the host before any
HIP call (no compute call is made here)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import moe_megakernel_amd as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("moe_forward", "moe_backward", "moe_saved_bytes", "moe_workspace_bytes",
              "moe_saved_view", "moe_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = mk.load()
    out = subprocess.run(["nm", "-D", "--defined-only", mk.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(moe_\w+)", out))
    for n in _declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(mk.EXPORTED) == set(_declared_functions())


def test_every_hip_source_is_a_build_unit():
    """The library is linked from one object per csrc/*.hip file (each with its own
    compiler flags): a launcher file left out of the build would leave its kernels'
    launchers undefined in the shared library."""
    from moe_megakernel_amd import build as B
    units = sorted(src for src, _ in B.SOURCES)
    on_disk = sorted(f for f in os.listdir(os.path.join(ROOT, "moe_megakernel_amd", "csrc")) if f.endswith(".hip"))
    assert units == on_disk
    # and the linked library defines every launcher the C ABI unit calls
    out = subprocess.run(["nm", "-D", "--defined-only", "-C", mk.LIB_PATH], capture_output=True, text=True).stdout
    for fn in ("moe::gemm::launch_fc1", "moe::gemm::launch_plain", "moe::gemm::launch_dgrad_swiglu",
               "moe::gemm::launch_wgrad"):
        assert fn in out, fn


def test_status_strings():
    for s in range(9):
        assert mk.moe_status_str(s) and mk.moe_status_str(s) != "unknown status"
    assert mk.moe_status_str(99) == "unknown status"


def _ok_problem(**kw):
    d = dict(tokens=64, hidden=256, inter=128, experts=8, topk=2)
    d.update(kw)
    return mk.problem(d["tokens"], d["hidden"], d["inter"], d["experts"], d["topk"])


def test_sizes_are_positive_and_monotone():
    small = mk.moe_saved_bytes(_ok_problem())
    big = mk.moe_saved_bytes(_ok_problem(tokens=128))
    assert 0 < small < big
    assert mk.moe_workspace_bytes(_ok_problem(), True) > 0
    assert mk.moe_workspace_bytes(_ok_problem(), False) > 0
    lay = mk.moe_saved_view(_ok_problem())
    offs = [lay.top_experts, lay.router_weights, lay.counts, lay.offsets, lay.slot_of,
            lay.slot_token, lay.status_word]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=100), mk.MOE_ERR_SHAPE),
    (dict(inter=64), mk.MOE_ERR_SHAPE),
    (dict(experts=0), mk.MOE_ERR_SHAPE),
    (dict(experts=256), mk.MOE_ERR_SHAPE),
    (dict(topk=9), mk.MOE_ERR_SHAPE),
    (dict(topk=3, experts=2), mk.MOE_ERR_SHAPE),
    (dict(tokens=-1), mk.MOE_ERR_SHAPE),
])
def test_invalid_problem_is_rejected(kw, status):
    p = _ok_problem(**kw)
    assert mk.moe_saved_bytes(p) == 0
    st = mk.moe_forward(p, 0, 0, 0, mk.moe_weights(), 0, 0, 0, 0, 0)
    assert st == status


def test_unsupported_configurations_are_rejected():
    p = _ok_problem()
    p.flags = 16                                  # an unknown flag bit
    assert mk.moe_forward(p, 0, 0, 0, mk.moe_weights(), 0, 0, 0, 0, 0) == mk.MOE_ERR_UNSUPPORTED
    for bad in (-1.0, float("nan"), float("inf")):   # SwiGLU clamp limit must be finite and >= 0
        p = _ok_problem()
        p.swiglu_limit = bad
        assert mk.moe_forward(p, 0, 0, 0, mk.moe_weights(), 0, 0, 0, 0, 0) == mk.MOE_ERR_UNSUPPORTED
    p = _ok_problem()
    p.swiglu_limit = 7.0                          # a clamp is accepted (fails later on the weights)
    assert mk.moe_forward(p, 0, 0, 0, mk.moe_weights(), 0, 0, 0, 0, 0) == mk.MOE_ERR_DTYPE
    p = _ok_problem()
    p.routed_dtype = 2                            # fp32 routed weights
    assert mk.moe_forward(p, 0, 0, 0, mk.moe_weights(), 0, 0, 0, 0, 0) == mk.MOE_ERR_DTYPE


def _fake_weights(p, shared_dtype=mk.MOE_BF16, routed_table=False, ld_pad=0):
    """Descriptors over fake (never dereferenced) 256-byte aligned addresses."""
    H, I = p.hidden, p.intermediate
    base = 1 << 40
    m = lambda ld: mk.moe_mat(base, 0, 0, ld + ld_pad)
    r = lambda ld: mk.moe_mat(0 if routed_table else base, H * I * 2, base if routed_table else 0, ld + ld_pad)
    z = mk.moe_mat(0, 0, 0, 0)
    W = mk.moe_weight
    return mk.moe_weights(W(shared_dtype, I, H, 0, m(H), z, z, z), W(shared_dtype, I, H, I, m(H), z, z, z),
                          W(shared_dtype, H, I, 0, m(I), z, z, z), W(p.routed_dtype, I, H, 0, r(H), z, z, z),
                          W(p.routed_dtype, I, H, I, r(H), z, z, z), W(p.routed_dtype, H, I, 0, r(I), z, z, z))


def test_weight_validation_errors():
    p = _ok_problem()
    args = (1 << 41, 1 << 41, 1 << 41)
    # shared expert must be BF16
    w = _fake_weights(p, shared_dtype=mk.MOE_MXFP8_E4M3)
    assert mk.moe_forward(p, *args, w, 1 << 41, 0, 0, 0, 0) == mk.MOE_ERR_DTYPE
    # both base and table set
    w = _fake_weights(p)
    w.routed_gate.data.table = 1 << 40
    assert mk.moe_forward(p, *args, w, 1 << 41, 0, 0, 0, 0) == mk.MOE_ERR_LAYOUT
    # wrong logical shape
    w = _fake_weights(p)
    w.routed_down.rows = 128
    assert mk.moe_forward(p, *args, w, 1 << 41, 0, 0, 0, 0) == mk.MOE_ERR_SHAPE
    # row stride not a multiple of 16 bytes
    w = _fake_weights(p, ld_pad=3)
    assert mk.moe_forward(p, *args, w, 1 << 41, 0, 0, 0, 0) == mk.MOE_ERR_LAYOUT
    # missing saved buffer / workspace
    w = _fake_weights(p)
    assert mk.moe_forward(p, *args, w, 1 << 41, 0, 1 << 41, 1 << 20, 0) == mk.MOE_ERR_WORKSPACE
    assert mk.moe_forward(p, *args, w, 1 << 41, 1 << 41, 1 << 41, 0, 0) == mk.MOE_ERR_WORKSPACE
    # missing input pointer
    assert mk.moe_forward(p, 0, 1 << 41, 1 << 41, w, 1 << 41, 1 << 41, 1 << 41, 1 << 20, 0) == mk.MOE_ERR_NULL


def test_backward_validation_errors():
    p = _ok_problem()
    w = _fake_weights(p)
    g = mk.moe_main_grads()
    a = 1 << 41
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 1 << 30, 0) == mk.MOE_ERR_NULL
    H, I = p.hidden, p.intermediate
    G = lambda ld, ro=0: mk.moe_grad(a, 0, 0, ld, ro)
    g = mk.moe_main_grads(G(H), G(H, I), G(I), G(H), G(H, I), G(I))
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 16, 0) == mk.MOE_ERR_WORKSPACE
    g.shared_down.ld = I - 1
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 1 << 30, 0) == mk.MOE_ERR_LAYOUT


def test_main_grad_rows_must_be_16_byte_aligned():
    p = _ok_problem()
    w = _fake_weights(p)
    a = 1 << 41
    H, I = p.hidden, p.intermediate
    G = lambda ld, ro=0, base=a, stride=0: mk.moe_grad(base, stride, 0, ld, ro)
    ok = mk.moe_main_grads(G(H), G(H, I), G(I), G(H), G(H, I), G(I))
    assert mk.moe_backward(p, a, a, w, a, a, a, ok, a, 16, 0) == mk.MOE_ERR_WORKSPACE   # layout accepted
    bad_base = mk.moe_main_grads(G(H), G(H, I), G(I), G(H, 0, a + 4), G(H, I), G(I))
    assert mk.moe_backward(p, a, a, w, a, a, a, bad_base, a, 1 << 30, 0) == mk.MOE_ERR_LAYOUT
    bad_ld = mk.moe_main_grads(G(H), G(H, I), G(I + 2), G(H), G(H, I), G(I))
    assert mk.moe_backward(p, a, a, w, a, a, a, bad_ld, a, 1 << 30, 0) == mk.MOE_ERR_LAYOUT
    bad_stride = mk.moe_main_grads(G(H), G(H, I), G(I), G(H), G(H, I), G(I, 0, a, I * H + 2))
    assert mk.moe_backward(p, a, a, w, a, a, a, bad_stride, a, 1 << 30, 0) == mk.MOE_ERR_LAYOUT


def test_main_grad_dtype_validation():
    p = _ok_problem()
    w = _fake_weights(p)
    a = 1 << 41
    H, I = p.hidden, p.intermediate
    G = lambda ld, ro=0, dt=0: mk.moe_grad(a, 0, 0, ld, ro, dt)
    bf = mk.MOE_BF16
    all_bf16 = mk.moe_main_grads(G(H, 0, bf), G(H, I, bf), G(I, 0, bf), G(H, 0, bf), G(H, I, bf), G(I, 0, bf))
    assert mk.moe_backward(p, a, a, w, a, a, a, all_bf16, a, 16, 0) == mk.MOE_ERR_WORKSPACE   # accepted
    mixed = mk.moe_main_grads(G(H, 0, bf), G(H, I, bf), G(I, 0, bf), G(H), G(H, I), G(I))
    assert mk.moe_backward(p, a, a, w, a, a, a, mixed, a, 1 << 30, 0) == mk.MOE_ERR_DTYPE
    bad = mk.moe_main_grads(G(H), G(H, I), G(I), G(H), G(H, I), G(I, 0, mk.MOE_MXFP8_E4M3))
    assert mk.moe_backward(p, a, a, w, a, a, a, bad, a, 1 << 30, 0) == mk.MOE_ERR_DTYPE


def test_routed_only_mode_ignores_shared_descriptors():
    """flags = 0 (routed-only): shared weights and shared main_grads are not validated,
    the saved context drops the T shared rows, and the routed ones are still checked."""
    p = _ok_problem()
    full = mk.moe_saved_bytes(p)
    p.flags = 0
    assert 0 < mk.moe_saved_bytes(p) < full
    assert mk.moe_workspace_bytes(p, 1) < mk.moe_workspace_bytes(_ok_problem(), 1)
    a = 1 << 41
    w = _fake_weights(p)
    w.shared_gate = mk.moe_weight()
    w.shared_up = mk.moe_weight()
    w.shared_down = mk.moe_weight()
    assert mk.moe_forward(p, a, a, a, w, a, a, 0, 0, 0) == mk.MOE_ERR_WORKSPACE   # weights accepted
    H, I = p.hidden, p.intermediate
    G = lambda ld, ro=0, dt=0: mk.moe_grad(a, 0, 0, ld, ro, dt)
    Z = mk.moe_grad()
    bf = mk.MOE_BF16
    g = mk.moe_main_grads(Z, Z, Z, G(H), G(H, I), G(I))
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 16, 0) == mk.MOE_ERR_WORKSPACE      # accepted
    g = mk.moe_main_grads(Z, Z, Z, G(H, 0, bf), G(H, I, bf), G(I, 0, bf))                 # BF16, shared 0
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 16, 0) == mk.MOE_ERR_WORKSPACE
    g = mk.moe_main_grads(Z, Z, Z, G(H, 0, bf), G(H, I), G(I))
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 1 << 30, 0) == mk.MOE_ERR_DTYPE
    w.routed_down.rows = 128
    assert mk.moe_forward(p, a, a, a, w, a, a, a, 1 << 20, 0) == mk.MOE_ERR_SHAPE
    # with the flag set, the same all-zero shared descriptors are rejected
    p.flags = mk.MOE_FLAG_HAS_SHARED
    w = _fake_weights(p)
    w.shared_down = mk.moe_weight()
    assert mk.moe_forward(p, a, a, a, w, a, a, a, 1 << 20, 0) != mk.MOE_OK


def test_recompute_mode_shrinks_saved_to_routing_state():
    """MOE_FLAG_RECOMPUTE: `saved` keeps only the routing state (same offsets as without
    the flag), the activations move to the workspaces."""
    p = _ok_problem(tokens=4096)
    q = _ok_problem(tokens=4096)
    q.flags |= mk.MOE_FLAG_RECOMPUTE
    H, I, T, K = p.hidden, p.intermediate, p.tokens, p.topk
    acts = 2 * (T * K + T) * (3 * I + H)                    # ab, h, y in bf16
    assert mk.moe_saved_bytes(p) - mk.moe_saved_bytes(q) >= acts
    assert mk.moe_saved_bytes(q) < 64 * T * K                 # a few int32 per route
    assert mk.moe_workspace_bytes(q, 0) >= acts
    assert mk.moe_workspace_bytes(q, 1) > mk.moe_workspace_bytes(p, 1)
    lp, lq = mk.moe_saved_view(p), mk.moe_saved_view(q)
    for f, _ in mk.moe_saved_layout._fields_:
        assert getattr(lp, f) == getattr(lq, f)


def test_topk_routing_entry_point_validation():
    """moe_forward_topk needs MOE_FLAG_TOPK_ROUTING and moe_forward refuses it; the table
    pointers are required for a non-empty batch."""
    p = _ok_problem()
    a = 1 << 41
    w = _fake_weights(p)
    assert mk.moe_forward_topk(p, a, a, a, w, a, a, a, 1 << 20, 0) == mk.MOE_ERR_UNSUPPORTED
    p.flags |= mk.MOE_FLAG_TOPK_ROUTING
    assert mk.moe_forward(p, a, a, a, w, a, a, a, 1 << 20, 0) == mk.MOE_ERR_UNSUPPORTED
    assert mk.moe_forward_topk(p, a, 0, a, w, a, a, a, 1 << 20, 0) == mk.MOE_ERR_NULL
    assert mk.moe_forward_topk(p, a, a, 0, w, a, a, a, 1 << 20, 0) == mk.MOE_ERR_NULL
    assert mk.moe_forward_topk(p, a, a, a, w, a, a, 0, 0, 0) == mk.MOE_ERR_WORKSPACE   # accepted so far
    assert mk.moe_saved_bytes(p) == mk.moe_saved_bytes(_ok_problem())
    assert "repeated" in mk.moe_status_str(mk.MOE_ERR_ROUTE_INVALID)


def test_shared_gate_validation():
    """MOE_FLAG_SHARED_GATE needs the shared expert, a [1][H] BF16 gate weight and a
    seventh main_grad of the same dtype as the others."""
    a = 1 << 41
    p = _ok_problem()
    H, I = p.hidden, p.intermediate
    p.flags = mk.MOE_FLAG_SHARED_GATE                       # without the shared expert
    assert mk.moe_forward(p, a, a, a, _fake_weights(_ok_problem()), a, a, a, 1 << 20, 0) == mk.MOE_ERR_UNSUPPORTED
    p.flags = mk.MOE_FLAG_HAS_SHARED | mk.MOE_FLAG_SHARED_GATE
    w = _fake_weights(p)
    assert mk.moe_forward(p, a, a, a, w, a, a, a, 1 << 20, 0) == mk.MOE_ERR_DTYPE      # gate weight missing
    w.shared_out_gate = mk.moe_weight(mk.MOE_BF16, 1, H, 0, mk.moe_mat(a, 0, 0, H))
    assert mk.moe_forward(p, a, a, a, w, a, a, 0, 0, 0) == mk.MOE_ERR_WORKSPACE        # accepted
    w.shared_out_gate.cols = H - 128
    assert mk.moe_forward(p, a, a, a, w, a, a, a, 1 << 20, 0) == mk.MOE_ERR_SHAPE
    w.shared_out_gate.cols = H
    G = lambda ld, ro=0, dt=0: mk.moe_grad(a, 0, 0, ld, ro, dt)
    g = mk.moe_main_grads(G(H), G(H, I), G(I), G(H), G(H, I), G(I))
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 1 << 30, 0) == mk.MOE_ERR_NULL    # gate grad missing
    g.shared_out_gate = G(H, 0, mk.MOE_BF16)
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 1 << 30, 0) == mk.MOE_ERR_DTYPE
    g.shared_out_gate = G(H)
    assert mk.moe_backward(p, a, a, w, a, a, a, g, a, 16, 0) == mk.MOE_ERR_WORKSPACE     # accepted
    q = _ok_problem()
    assert mk.moe_workspace_bytes(p, 1) > mk.moe_workspace_bytes(q, 1)
    assert mk.moe_saved_bytes(p) > mk.moe_saved_bytes(q)


def test_noalloc_forward_validation():
    """moe_forward_noalloc validates like moe_forward and rejects a problem whose forward
    scratch exceeds its static array, all on the host before any HIP call."""
    a = 1 << 41
    p = _ok_problem()
    w = _fake_weights(p)
    assert mk.moe_forward_noalloc(p, 0, a, a, w, a, a, 0) == mk.MOE_ERR_NULL
    assert mk.moe_forward_noalloc(p, a, a, a, w, a, 0, 0) == mk.MOE_ERR_WORKSPACE      # no saved buffer
    q = _ok_problem()
    q.flags |= mk.MOE_FLAG_TOPK_ROUTING
    assert mk.moe_forward_noalloc(q, a, a, a, w, a, a, 0) == mk.MOE_ERR_UNSUPPORTED
    big = _ok_problem(tokens=1 << 16)
    big.flags |= mk.MOE_FLAG_RECOMPUTE                       # activations in the forward scratch
    assert mk.moe_workspace_bytes(big, 0) > mk.MOE_NOALLOC_SCRATCH_BYTES
    assert mk.moe_forward_noalloc(big, a, a, a, _fake_weights(big), a, a, 0) == mk.MOE_ERR_WORKSPACE
    assert mk.moe_forward_noalloc(_ok_problem(hidden=100), a, a, a, w, a, a, 0) == mk.MOE_ERR_SHAPE
    mx = mk.problem(4096, 4096, 1024, 96, 4, mk.MOE_MXFP8_E4M3)   # the 4096-token MXFP8 layer fits
    assert mk.moe_workspace_bytes(mx, 0) <= mk.MOE_NOALLOC_SCRATCH_BYTES
