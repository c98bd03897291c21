"""Backward of the MoE layer on the GPU against the oracle (the derivative of the forward
definitions of "0 train-infer mismatch ...": experts, SwiGLU, combine with the routed
scaling factor, softmax router; under routing replay the router gradient of w - sg[w] + w*
of "Total Router Recall").

Protocol: the GPU forward's saved results (h, y, logits, routing) feed both backwards, so
each gradient is compared stage by stage; every gradient is an FP32 sum over a fixed
order on both sides, compared within |gpu - ref| <= 1e-4 * max(1, |ref|) elementwise (FP32
sums of up to a few thousand terms in different orders: a few 1e-6 relative in practice,
the bound leaves margin for sums with cancellation) and bitwise for the exact steps.
Per-token gradient rows are bitwise independent of the batch size, and every output is
bitwise identical from run to run."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import oracle
import workloads as W
from gpu_util import as_f32, dev, dims_of, host, upload

pytestmark = pytest.mark.gpu
GTOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()
    oracle.lib()


def _close(gpu, ref, what, tol=GTOL):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r) / np.maximum(1.0, np.abs(r))
    worst = float(err.max()) if err.size else 0.0
    print(f"  {what}: max scaled error {worst:.2e} (max |ref| {np.abs(r).max():.3g})")
    assert worst <= tol, f"{what}: {worst:.3e} > {tol}"


def _run(L, inp, dout, scale, slot=None, x_perm=False, router_grads=True, g16=False,
         fused=False, saved_gu=False):
    dims = dims_of(L)
    fb = M.alloc_forward_buffers(dims, "cuda", router=(L.mode == "router"), weighted=True)
    if saved_gu:   # the forward stores the pre-activations; the backward reads them
        fb["gu"] = torch.empty((L.T * L.k, 2 * L.I), dtype=torch.float32, device="cuda")
    fb.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"])
    if L.mode == "router":
        fb["w_router"], fb["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        fb["idx_in"], fb["w_in"] = inp["idx_in"], inp["w_in"]
    if slot is not None:
        inv_m = torch.from_numpy(np.argsort(slot)).cuda().long()
        fb["slot_of_expert"] = dev(slot)
        fb["w13"], fb["w2"] = inp["w13"][inv_m].contiguous(), inp["w2"][inv_m].contiguous()
    if not x_perm:
        del fb["x_perm"]
    ws = M.alloc_workspace(dims)
    M.forward(dims, fb, ws, routed_scale=scale)
    gd = M.MOE_BF16 if g16 else M.MOE_F32
    bb = M.alloc_backward_buffers(dims, "cuda", router=router_grads, grad_dtype=gd,
                                  keep_gu=not fused)
    bb.update(x=inp["x"], x_perm=fb.get("x_perm"), w13=fb["w13"], w2=fb["w2"],
              offsets=fb["offsets"], perm=fb["perm"], inv=fb["inv"], topk_w=fb["topk_w"],
              h=fb["h"], y=fb["y"], d_out=dev(dout))
    if saved_gu:
        bb["gu"] = fb["gu"]
    if router_grads:
        bb["w_router"] = dev(L.w_router)
        bb["logit_bias"] = inp.get("logit_bias")
        bb["logits"] = fb.get("logits")          # replay: recomputed from x and w_router
    M.backward(dims, bb, ws, routed_scale=scale, grad_dtype=gd, gu_saved=saved_gu)
    torch.cuda.synchronize()
    assert int(fb["d_err"].item()) == 0
    return fb, bb


def _oracle(L, fb, dout, scale, slot=None, g16=False):
    offsets = host(fb["offsets"])
    counts = np.diff(offsets)
    w13, w2 = host(fb["w13"]), host(fb["w2"])
    be = oracle.backward_experts(L.x, host(fb["perm"]), host(fb["inv"]), counts,
                                 host(fb["topk_w"]), w13, w2, host(fb["h"]), host(fb["y"]),
                                 dout, L.dtype, scale, round_grads=g16)
    logits = host(fb["logits"]) if "logits" in fb else oracle.router_logits(
        L.x, L.w_router, L.logit_bias, L.dtype)
    br = oracle.backward_router(logits, be["dw"], L.x, L.w_router, L.dtype)
    return be, br


CASES = [
    # (T, d, E, k, I, dtype, mode, scale, placed, x_perm)
    (300, 256, 16, 4, 192, "bf16", "router", 1.0, False, False),
    (300, 128, 32, 8, 128, "bf16", "router", 2.5, True, True),
    (40, 128, 16, 6, 64, "bf16", "router", 2.5, False, False),     # small-batch forward path
    (257, 128, 24, 4, 128, "f32", "router", 1.5, False, False),
    (300, 128, 16, 4, 128, "bf16", "replay", 1.0, False, False),    # router grads recomputed
    (123, 192, 10, 3, 64, "f32", "replay", 1.0, True, True),        # E % 4 != 0
    (1100, 128, 16, 4, 128, "f32", "router", 1.0, False, False),    # d_w_router in 4 segments
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[0]}_d{c[1]}_E{c[2]}_k{c[3]}_I{c[4]}_"
                                                      f"{c[5]}_{c[6]}{'_placed' if c[8] else ''}"
                                                      f"{'_xperm' if c[9] else ''}")
def test_backward_parity(case):
    T, d, E, k, I, dtype, mode, scale, placed, xp = case
    L = W.make_layer(T=T, d=d, E=E, k=k, I=I, dtype=dtype, mode=mode, seed=T + E, bias="zipf",
                     replay="uniform")
    if mode == "replay":
        L.w_router = W._normal(L.seed, W.TID_ROUTER, (E, d), 1.0 / np.sqrt(d), dtype)
    inp = upload(L)
    rng = np.random.default_rng(T)
    dout = rng.normal(0, 1, (T, d)).astype(np.float32)
    if dtype == "bf16":
        dout = W.f32_to_bf16_bits(dout)
    slot = rng.permutation(E).astype(np.int32) if placed else None
    fb, bb = _run(L, inp, dout, scale, slot, xp)
    be, br = _oracle(L, fb, dout, scale, slot)
    # exact steps: dy is one product per element on both sides
    assert host(bb["d_y"]).tobytes() == be["dy"].tobytes()
    for n, r in (("d_topk_w", be["dw"]), ("gu", be["gu"]), ("d_h", be["dh"]),
                 ("d_gu", be["dgu"]), ("d_xp", be["dxp"]), ("d_w2", be["dw2"]),
                 ("d_w13", be["dw13"]), ("d_logits", br["dl"]),
                 ("d_w_router", br["dw_router"]), ("d_x_router", br["dx"])):
        _close(host(bb[n]), r, n)
    _close(host(bb["d_x"]), be["dx"] + br["dx"], "d_x")


def test_backward_deterministic_and_batch_invariant():
    T, d, E, k, I = 300, 128, 16, 4, 128
    L = W.make_layer(T=T, d=d, E=E, k=k, I=I, dtype="bf16", mode="router", seed=31,
                     bias="zipf")
    inp = upload(L)
    dout = W.f32_to_bf16_bits(np.random.default_rng(3).normal(0, 1, (T, d)).astype(np.float32))
    _, b1 = _run(L, inp, dout, 2.5)
    _, b2 = _run(L, inp, dout, 2.5)
    for n in b1:
        if isinstance(b1[n], torch.Tensor) and n.startswith(("d_", "gu")):
            assert host(b1[n]).tobytes() == host(b2[n]).tobytes(), n
    # the first 64 tokens alone: the same per-token gradient rows
    Ls = W.make_layer(T=64, d=d, E=E, k=k, I=I, dtype="bf16", mode="router", seed=31,
                      bias="zipf", weights=False)
    Ls.x, Ls.w13, Ls.w2, Ls.w_router, Ls.logit_bias = (np.ascontiguousarray(L.x[:64]), L.w13,
                                                        L.w2, L.w_router, L.logit_bias)
    inps = dict(inp)
    inps["x"] = dev(Ls.x)
    fs, bs = _run(Ls, inps, np.ascontiguousarray(dout[:64]), 2.5)
    for n in ("d_x", "d_topk_w", "d_logits", "d_x_router"):
        assert host(bs[n]).tobytes() == host(b1[n])[:64].tobytes(), n


G16_CASES = [
    # (T, d, E, k, I, mode, scale, placed, x_perm); the token-tile heights (16 .. 256) select
    # every launch shape of the K-major data-gradient GEMM
    (300, 256, 16, 4, 192, "router", 2.5, False, False),
    (517, 128, 32, 8, 128, "router", 1.0, True, True),
    (40, 192, 8, 6, 64, "replay", 1.0, False, False),
    (12, 128, 16, 4, 128, "router", 1.0, False, False),      # 16-row tiles
    (30, 192, 16, 4, 64, "router", 1.0, False, True),        # 32-row tiles
    (2100, 128, 4, 2, 128, "router", 1.0, False, False),     # 256-row tiles, long segments
]


@pytest.mark.parametrize("case", G16_CASES, ids=lambda c: f"T{c[0]}_d{c[1]}_E{c[2]}_k{c[3]}_"
                                                          f"I{c[4]}_{c[5]}")
def test_backward_bf16_operands_parity(case):
    """bf16 gradient operands: dy and d_gu rounded once where they are formed, the data
    gradients on the forward's bf16 GEMM (weights read K-major), the weight gradients on the
    bf16 weight-gradient kernel; against the oracle with the same rounding points. dy is
    bitwise; d_gu within one bf16 rounding (its FP32 input dh is summed in another order);
    every other gradient within 1e-3 * max(1, |ref|)."""
    T, d, E, k, I, mode, scale, placed, xp = case
    L = W.make_layer(T=T, d=d, E=E, k=k, I=I, dtype="bf16", mode=mode, seed=T + 3, bias="zipf",
                     replay="uniform")
    if mode == "replay":
        L.w_router = W._normal(L.seed, W.TID_ROUTER, (E, d), 1.0 / np.sqrt(d), "bf16")
    inp = upload(L)
    rng = np.random.default_rng(T)
    dout = W.f32_to_bf16_bits(rng.normal(0, 1, (T, d)).astype(np.float32))
    slot = rng.permutation(E).astype(np.int32) if placed else None
    fb, bb = _run(L, inp, dout, scale, slot, xp, g16=True)
    be, br = _oracle(L, fb, dout, scale, slot, g16=True)
    assert host(bb["d_y"]).tobytes() == W.f32_to_bf16_bits(be["dy"]).tobytes()
    _close(as_f32(host(bb["d_gu"]), "bf16"), be["dgu"], "d_gu", tol=2.0 ** -7)
    for n, r in (("d_topk_w", be["dw"]), ("gu", be["gu"]), ("d_h", be["dh"]),
                 ("d_w2", be["dw2"]), ("d_logits", br["dl"]),
                 ("d_w_router", br["dw_router"]), ("d_x_router", br["dx"])):
        _close(host(bb[n]), r, n, tol=1e-3)
    # downstream of the rounded d_gu, whose bf16 rounding can flip by one unit where the two
    # sides' FP32 dh (summed in different orders) straddle a midpoint: the bf16 tolerance
    for n, r in (("d_xp", be["dxp"]), ("d_w13", be["dw13"])):
        _close(host(bb[n]), r, n, tol=2e-2)
    _close(host(bb["d_x"]), be["dx"] + br["dx"], "d_x", tol=2e-2)
    # and tightly, from the GPU's own rounded d_gu (float64 sums of the same operands)
    dgu = as_f32(host(bb["d_gu"]), "bf16").astype(np.float64)
    offs = host(fb["offsets"])
    xr = as_f32(L.x, "bf16").astype(np.float64)[host(fb["perm"]) // k]
    w13 = as_f32(host(fb["w13"]), "bf16").astype(np.float64)
    ref_w13 = np.stack([dgu[offs[e]:offs[e + 1]].T @ xr[offs[e]:offs[e + 1]] for e in range(E)])
    ref_xp = np.concatenate([dgu[offs[e]:offs[e + 1]] @ w13[e] for e in range(E)])
    _close(host(bb["d_w13"]), ref_w13, "d_w13 (GPU d_gu)", tol=1e-4)
    _close(host(bb["d_xp"]), ref_xp, "d_xp (GPU d_gu)", tol=1e-4)


FUSED_CASES = [  # T, d, E, k, I, g16, x_perm: tile heights 16 .. 256, both gradient dtypes
    (12, 128, 16, 4, 128, True, False), (30, 192, 16, 4, 64, True, True),
    (300, 256, 8, 2, 192, False, False), (2100, 128, 4, 2, 128, True, False),
    (1500, 256, 4, 4, 320, False, True), (4096, 128, 2, 2, 64, True, False)]


@pytest.mark.gpu
@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: f"T{c[0]}_d{c[1]}_E{c[2]}_k{c[3]}_"
                                                            f"I{c[4]}_g16{int(c[5])}_xp{int(c[6])}")
def test_backward_fused_swiglu_grad_bitwise(case):
    """Without gu (bf16 layers) the gate/up recomputation runs after dh and forms d_gu in its
    epilogue: every gradient is bitwise the one of the path that materialises gu and runs
    the elementwise SwiGLU derivative."""
    T, d, E, k, I, g16, xp = case
    L = W.make_layer(T=T, d=d, E=E, k=k, I=I, dtype="bf16", mode="router", seed=T + 5,
                     bias="zipf")
    inp = upload(L)
    rng = np.random.default_rng(T + 1)
    dout = W.f32_to_bf16_bits(rng.normal(0, 1, (T, d)).astype(np.float32))
    _, b1 = _run(L, inp, dout, 1.0, None, xp, g16=g16)
    _, b2 = _run(L, inp, dout, 1.0, None, xp, g16=g16, fused=True)
    assert "gu" not in b2
    for n in sorted(b1):
        if n.startswith("d_"):
            assert host(b1[n]).tobytes() == host(b2[n]).tobytes(), n


SAVED_CASES = [
    # (T, d, E, k, I, dtype, g16, x_perm): token-tile heights 16 .. 256, both layer dtypes
    (12, 128, 16, 4, 128, "bf16", True, False), (40, 192, 8, 6, 64, "bf16", False, True),
    (300, 256, 8, 2, 192, "bf16", True, False), (2100, 128, 4, 2, 128, "bf16", False, False),
    (4096, 128, 2, 2, 64, "bf16", True, True), (257, 128, 24, 4, 128, "f32", False, False),
    (48, 128, 8, 2, 64, "f32", False, True)]


@pytest.mark.gpu
@pytest.mark.parametrize("case", SAVED_CASES, ids=lambda c: f"T{c[0]}_d{c[1]}_E{c[2]}_k{c[3]}_"
                                                            f"I{c[4]}_{c[5]}_g16{int(c[6])}_xp{int(c[7])}")
def test_backward_saved_preactivations_bitwise(case):
    """The forward stores g and u (moe_forward_args.gu) and the backward reads them
    (gu_saved): the saved values are bitwise the recomputed ones, every gradient is
    bitwise the recomputing call's, and the forward's own outputs are unchanged."""
    T, d, E, k, I, dtype, g16, xp = case
    L = W.make_layer(T=T, d=d, E=E, k=k, I=I, dtype=dtype, mode="router", seed=T + 9,
                     bias="zipf")
    inp = upload(L)
    rng = np.random.default_rng(T + 3)
    dout = rng.normal(0, 1, (T, d)).astype(np.float32)
    if dtype == "bf16":
        dout = W.f32_to_bf16_bits(dout)
    f1, b1 = _run(L, inp, dout, 1.5, None, xp, g16=g16)                  # recomputes into gu
    f2, b2 = _run(L, inp, dout, 1.5, None, xp, g16=g16, saved_gu=True)   # reads the saved gu
    for n in ("out", "h", "y", "topk_idx", "topk_w", "perm", "inv"):
        assert host(f1[n]).tobytes() == host(f2[n]).tobytes(), n
    assert host(f2["gu"]).tobytes() == host(b1["gu"]).tobytes(), "gu"
    for n in sorted(b1):
        if n.startswith("d_"):
            assert host(b1[n]).tobytes() == host(b2[n]).tobytes(), n
