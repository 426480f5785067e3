"""The allocation-free forward (moe_forward_noalloc), called through the C ABI: its
scratch is the library's static per-GPU array instead of a caller workspace, and its
results must be bit-identical to moe_forward's on the same inputs.  Two calls in a row,
the second on a smaller problem, so the second reads nothing the first left behind."""
import pytest
import torch

import moe_inputs as gen

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()


def _run_both(cfg, **kw):
    """moe_forward then moe_backward, and moe_forward_noalloc then moe_backward, on one
    problem; returns both sets of outputs (main_grad restarted from the same pattern)."""
    import moe_megakernel_amd as mk
    from moe_inputs.device import DeviceProblem
    print(f"[case] noalloc T={cfg.tokens} H={cfg.hidden} E={cfg.experts} K={cfg.topk} I={cfg.inter} "
          f"{cfg.routed} {kw}", flush=True)
    dp = DeviceProblem(cfg, **kw)
    need = mk.moe_workspace_bytes(dp.p, False)
    assert need <= mk.MOE_NOALLOC_SCRATCH_BYTES
    res = []
    for noalloc in (False, True):
        layer = dp.layer if not noalloc else mk.Layer(dp.p)
        out = torch.full_like(dp.out, float("nan"))
        if noalloc:
            layer.forward_noalloc(dp.x, dp.probs, dp.rmap, dp.weights, out)
        else:
            layer.forward(dp.x, dp.probs, dp.rmap, dp.weights, out)
        dp.reset_main_grads()
        dx = torch.full_like(dp.dx, float("nan"))
        dpr = torch.full_like(dp.dprobs, float("nan"))
        layer.backward(dp.dy, dp.x, dp.weights, dx, dpr, dp.main_grads)
        torch.cuda.synchronize()
        st = {k: v.clone() for k, v in layer.routing_state().items()}
        res.append({"out": out.clone(), "dx": dx.clone(), "dprobs": dpr.clone(), "state": st,
                    "mg": [t.clone() for t in dp.mg_r1_list + dp.mg_r2_list + [dp.mg_s1, dp.mg_s2]]})
    return res


def _assert_identical(a, b):
    for n in ("out", "dx", "dprobs"):
        assert torch.equal(_bits(a[n]), _bits(b[n])), n
    S = int(a["state"]["offsets"][-1])            # slot_token holds S valid entries
    for k in a["state"]:
        x, y = a["state"][k].cpu(), b["state"][k].cpu()
        if k == "slot_token":
            x, y = x[:S], y[:S]
        assert torch.equal(x, y), k
    for x, y in zip(a["mg"], b["mg"]):
        assert torch.equal(_bits(x), _bits(y)), "main_grad"


@pytest.mark.parametrize("routed,layout,recompute", [
    ("mxfp8", "table", False),    # scratch: the MXFP8 codes and scales of x and h
    ("bf16", "single", True),     # scratch: the forward's activations (recompute mode)
])
def test_noalloc_forward_is_bit_identical_on_two_calls(gpu_lib, routed, layout, recompute):
    big = gen.custom(520, 384, 9, 3, 256, routed=routed, layout=layout, short_frac=0.05, short_max=2, idx=1300)
    small = gen.custom(77, 256, 5, 2, 128, routed=routed, layout=layout, short_frac=0.1, short_max=1, idx=1301)
    for cfg in (big, small):
        ref, got = _run_both(cfg, recompute=recompute)
        _assert_identical(ref, got)
        assert int(got["state"]["status_word"][0]) == 0
        print(f"[noalloc] {cfg.tokens} tokens: bit-identical to moe_forward", flush=True)
