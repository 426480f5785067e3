"""The dense MoE formulation in plain torch float64 on the CPU: every routed
expert is applied to every token and masked by routing_map * probs.

    out = FFN_shared(x) + sum_e (routing_map[:, e] * probs[:, e]) * FFN_e(x)

(without the first term when `shared` is None: routed-only mode).

It never builds the fixed-width table nor the dispatch permutation, and its
backward comes from torch autograd, so it shares neither the oracle's
formulation nor its hand-derived gradients.  Test infrastructure only.
"""
import torch
import torch.nn.functional as F


def dense_forward(x, probs, rmap, shared, routed, gate=None, limit=0.0):
    """x [T,H]; probs, rmap [T,E]; shared = (W1 [2I,H], W2 [H,I]); routed = (W1 [E,2I,H], W2 [E,H,I]);
    gate: optional [H] weight of the shared output gate, sigmoid(x @ gate) per token;
    limit > 0: the gate pre-activation clamped above and the linear one to [-limit, limit]
    (torch.clamp, whose gradient passes inside the closed bounds)."""
    def ffn(xx, w1, w2):
        I = w2.shape[1]
        gu = xx @ w1.t()
        a, b = gu[:, :I], gu[:, I:]
        if limit > 0:
            a, b = a.clamp(max=limit), b.clamp(min=-limit, max=limit)
        return (F.silu(a) * b) @ w2.t()

    out = ffn(x, *shared) if shared is not None else torch.zeros_like(x)
    if gate is not None:
        out = torch.sigmoid(x @ gate)[:, None] * out
    mask = rmap.to(x.dtype) * probs
    for e in range(routed[0].shape[0]):
        out = out + mask[:, e:e + 1] * ffn(x, routed[0][e], routed[1][e])
    return out


def dense_grads(x, probs, rmap, shared, routed, dy, gate=None, limit=0.0):
    """Autograd gradients of sum(dy * out) w.r.t. x, probs, shared and routed weights (and
    the shared output gate's weight when given)."""
    sh = shared if shared is not None else (torch.zeros(1), torch.zeros(1))
    gt = gate if gate is not None else torch.zeros(1)
    leaves = [t.detach().clone().requires_grad_(True)
              for t in (x, probs, sh[0], sh[1], routed[0], routed[1], gt)]
    out = dense_forward(leaves[0], leaves[1], rmap,
                        (leaves[2], leaves[3]) if shared is not None else None, (leaves[4], leaves[5]),
                        leaves[6] if gate is not None else None, limit)
    (out * dy).sum().backward()
    g = [t.grad for t in leaves]
    return {"out": out.detach(), "dx": g[0], "dprobs": g[1] * rmap.to(g[1].dtype),
            "dshared1": g[2], "dshared2": g[3], "drouted1": g[4], "drouted2": g[5], "dgate": g[6]}
