"""Pins of the oracle's backward of the MoE layer.

The oracle's backward is written out from the derivative of the forward definitions (FP32,
sequential sums). Here it is checked against PyTorch's float64 autograd of the same
forward (a different implementation of the derivative): on FP32 layers for the router
(softmax, top-k, left-to-right renormalisation), the SwiGLU experts and the slot-order
combine with a routed scaling factor, and for routing replay with the stop-gradient form
w - sg[w] + w* ("0 train-infer mismatch ...", "Total Router Recall"), whose router
gradient is taken at the router's own choice. Plus exact properties: one expert gives a
zero logit gradient, logit gradients sum to zero per token, a factor of 2 doubles every
gradient exactly.
"""
import numpy as np
import pytest
import torch

import workloads as W


def _torch_forward(L, sel_fwd, w_used_fn, scale, dout):
    """float64 forward from the definitions; returns (loss, leaves)."""
    dt = torch.float64
    x = torch.tensor(W.to_f32(L.x, L.dtype), dtype=dt, requires_grad=True)
    wr = torch.tensor(W.to_f32(L.w_router, L.dtype), dtype=dt, requires_grad=True)
    w13 = torch.tensor(W.to_f32(L.w13, L.dtype), dtype=dt, requires_grad=True)
    w2 = torch.tensor(W.to_f32(L.w2, L.dtype), dtype=dt, requires_grad=True)
    bias = torch.zeros(L.E, dtype=dt) if L.logit_bias is None else torch.tensor(L.logit_bias, dtype=dt)
    logits = x @ wr.T + bias
    p = torch.softmax(logits, dim=1)
    w_used = w_used_fn(p, logits)
    I = L.I
    out = torch.zeros(L.T, L.d, dtype=dt)
    for j in range(L.k):
        e = torch.as_tensor(sel_fwd[:, j], dtype=torch.long)
        g = torch.einsum("tc,tnc->tn", x, w13[e, :I, :])
        u = torch.einsum("tc,tnc->tn", x, w13[e, I:, :])
        h = g * torch.sigmoid(g) * u
        y = torch.einsum("ti,toi->to", h, w2[e])
        out = out + w_used[:, j:j + 1] * y
    out = scale * out
    loss = (out * torch.tensor(dout, dtype=dt)).sum()
    loss.backward()
    return x, wr, w13, w2


def _renorm_at(p, sel):
    ps = torch.gather(p, 1, torch.as_tensor(sel, dtype=torch.long))
    return ps / ps.sum(dim=1, keepdim=True)


def _close(a, b, what, rel=2e-4):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.abs(b).max(), 1e-30)
    err = np.abs(a - b).max() / scale
    assert err <= rel, f"{what}: {err:.3e}"


def _oracle_backward(orc, L, r, dout, scale, idx, w):
    be = orc.backward_experts(L.x, r["perm"], r["inv"], r["counts"], w, L.w13, L.w2, r["h"],
                              r["y"], dout, L.dtype, scale)
    logits = orc.router_logits(L.x, L.w_router, L.logit_bias, L.dtype)
    br = orc.backward_router(logits, be["dw"], L.x, L.w_router, L.dtype)
    return be, br


@pytest.mark.parametrize("scale", [1.0, 2.5])
def test_router_mode_matches_float64_autograd(orc, scale):
    L = W.make_layer(T=48, d=64, E=8, k=3, I=64, dtype="f32", mode="router", seed=3,
                     bias="zipf")
    L.routed_scale = scale
    r = orc.forward(L)
    dout = np.random.default_rng(0).normal(0, 1, (L.T, L.d)).astype(np.float32)
    be, br = _oracle_backward(orc, L, r, dout, scale, r["idx"], r["w"])
    x, wr, w13, w2 = _torch_forward(L, r["idx"], lambda p, l: _renorm_at(p, r["idx"]), scale,
                                    dout)
    _close(be["dx"] + br["dx"], x.grad, "dx")
    _close(be["dw13"], w13.grad, "dw13")
    _close(be["dw2"], w2.grad, "dw2")
    _close(br["dw_router"], wr.grad, "dw_router")


def test_replay_stop_gradient_matches_float64_autograd(orc):
    """Replay: the experts run on the sampler's ids and weights w*; the layer passes
    w - sg[w] + w*, with w the router's own renormalised weights at its own top-k."""
    L = W.make_layer(T=40, d=64, E=8, k=2, I=64, dtype="f32", mode="replay", seed=5,
                     replay="uniform", weights=True)
    L.w_router = W._normal(5, W.TID_ROUTER, (L.E, L.d), 1.0 / np.sqrt(L.d), "f32")
    r = orc.forward(L)
    dout = np.random.default_rng(1).normal(0, 1, (L.T, L.d)).astype(np.float32)
    be, br = _oracle_backward(orc, L, r, dout, 1.0, L.idx_in, L.w_in)
    logits = orc.router_logits(L.x, L.w_router, None, "f32")
    own, _, _, _ = orc.route_from_logits(logits, L.k)
    w_star = torch.tensor(L.w_in, dtype=torch.float64)

    def used(p, l):
        w = _renorm_at(p, own)
        return w - w.detach() + w_star

    x, wr, w13, w2 = _torch_forward(L, L.idx_in, used, 1.0, dout)
    _close(br["dw_router"], wr.grad, "dw_router")
    _close(be["dx"] + br["dx"], x.grad, "dx")
    _close(be["dw13"], w13.grad, "dw13")
    _close(be["dw2"], w2.grad, "dw2")


def test_exact_properties(orc):
    L = W.make_layer(T=30, d=64, E=6, k=2, I=64, dtype="bf16", mode="router", seed=7)
    r = orc.forward(L)
    dout = W.f32_to_bf16_bits(np.random.default_rng(2).normal(0, 1, (L.T, L.d)).astype(np.float32))
    be, br = _oracle_backward(orc, L, r, dout, 1.0, r["idx"], r["w"])
    # a factor of 2 doubles every gradient exactly
    be2, br2 = _oracle_backward(orc, L, r, dout, 2.0, r["idx"], r["w"])
    for n in ("dw", "dy", "dh", "dgu", "dxp", "dx", "dw13", "dw2"):
        assert (be2[n] == 2 * be[n]).all(), n
    for n in ("dl", "dw_router", "dx"):
        assert (br2[n] == 2 * br[n]).all(), n
    # softmax: each token's logit gradients sum to zero
    tot = br["dl"].astype(np.float64).sum(1)
    assert np.abs(tot).max() <= 1e-6 * np.abs(br["dl"]).max()
    # recomputed pre-activations give back the forward's h (bf16 of silu(g) * u)
    I = L.I
    g, u = be["gu"][:, :I], be["gu"][:, I:]
    h = orc.round_bf16((g / (1 + np.exp(-g.astype(np.float64)))).astype(np.float32) * u)
    assert np.mean(h == r["h"]) > 0.99
    # one expert: the routing weight is 1 whatever the logits, so the logits get no gradient
    L1 = W.make_layer(T=10, d=64, E=1, k=1, I=64, dtype="f32", mode="router", seed=8)
    r1 = orc.forward(L1)
    d1 = np.ones((L1.T, L1.d), np.float32)
    _, b1 = _oracle_backward(orc, L1, r1, d1, 1.0, r1["idx"], r1["w"])
    assert (b1["dl"] == 0).all() and (b1["dw_router"] == 0).all()


def test_rounded_gradient_mode(orc):
    """With dy and dgu rounded once to bf16 where they are formed: dy is exactly the bf16 of
    the FP32 mode's dy, dgu holds bf16 values, and every gradient stays within bf16
    rounding of the float64 autograd gradient."""
    L = W.make_layer(T=48, d=64, E=8, k=3, I=64, dtype="f32", mode="router", seed=13,
                     bias="zipf")
    r = orc.forward(L)
    dout = np.random.default_rng(4).normal(0, 1, (L.T, L.d)).astype(np.float32)
    args = (L.x, r["perm"], r["inv"], r["counts"], r["w"], L.w13, L.w2, r["h"], r["y"], dout,
            "f32", 1.0)
    be32 = orc.backward_experts(*args)
    be16 = orc.backward_experts(*args, round_grads=True)
    assert (orc.round_bf16(be32["dy"]) == W.f32_to_bf16_bits(be16["dy"])).all()
    assert (be16["dy"].view(np.uint32) & 0xffff == 0).all()
    assert (be16["dgu"].view(np.uint32) & 0xffff == 0).all()
    logits = orc.router_logits(L.x, L.w_router, L.logit_bias, "f32")
    br = orc.backward_router(logits, be16["dw"], L.x, L.w_router, "f32")
    x, wr, w13, w2 = _torch_forward(L, r["idx"], lambda p, l: _renorm_at(p, r["idx"]), 1.0,
                                    dout)
    _close(be16["dx"] + br["dx"], x.grad, "dx", rel=2e-2)
    _close(be16["dw13"], w13.grad, "dw13", rel=2e-2)
    _close(be16["dw2"], w2.grad, "dw2", rel=2e-2)
    _close(br["dw_router"], wr.grad, "dw_router", rel=2e-4)     # dw is not rounded
