"""Router variants, expert-parallel output and backward at the training-shaped layer's full
size (T=4096, d=2048, E=64, top-8, inter=1408, bf16), in the launch configuration the
benchmark times. Integer outputs are checked in full against the oracle; floating-point
rows on a sample of tokens the oracle computes one by one (and, for the weight gradients,
on the smallest expert's whole segment)."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import oracle
import workloads as W
from gpu_util import as_f32, assert_close, dev, dims_of, host, sample_tokens, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()
    oracle.lib()


@pytest.fixture(scope="module")
def c2():
    L = W.make_config("c2")
    L.token_mult = W.token_multiplicities(L.T, 2)
    return L, upload(L)


def _forward(L, inp, router=None, scale=0.0, **kw):
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=True, weighted=True)
    del b["x_perm"]
    b.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
             logit_bias=inp["logit_bias"], token_mult=inp["token_mult"])
    b.update(kw.pop("bufs", {}))
    M.forward(dims, b, M.alloc_workspace(dims), router=router, routed_scale=scale, **kw)
    torch.cuda.synchronize()
    assert int(b["d_err"].item()) == 0
    return b


@pytest.mark.parametrize("variant", ["sigmoid_bias", "hash_sqrt_softplus"])
def test_full_router_variant(c2, variant):
    L, inp = c2
    if variant == "sigmoid_bias":
        W.set_router(L, "sigmoid", bias=True, routed_scale=2.5)
    else:
        W.set_router(L, "sqrt_softplus", bias=False, hash_vocab=131072, routed_scale=1.0)
    lse = torch.empty(L.T, dtype=torch.float32, device="cuda")
    router = dict(score=L.score, corr_bias=dev(L.corr_bias), hash_table=dev(L.hash_table),
                  token_ids=dev(L.token_ids), lse=lse)
    b = _forward(L, inp, router, L.routed_scale)
    r = oracle.route_scored(host(b["logits"]), L.k, L.score, L.corr_bias, L.hash_table,
                            L.token_ids, L.token_mult)
    assert r["err"] == 0
    np.testing.assert_array_equal(host(b["topk_idx"]), r["idx"])
    assert_close(host(b["topk_w"]), r["w"], "f32", "topk_w")
    assert_close(host(lse), r["lse"], "f32", "lse")
    counts, offsets, perm, inv, err = oracle.permute(r["idx"], L.E)
    for n, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        np.testing.assert_array_equal(host(b[n]), ref, err_msg=n)
    toks = sample_tokens(L.T, 8, seed=5)
    _, _, out = oracle.forward_tokens(L, toks, r["idx"], r["w"])
    assert_close(as_f32(host(b["out"])[toks], "bf16"), as_f32(out, "bf16"), "bf16", "out")
    W.set_router(L, "softmax", bias=False)          # restore the fixture's layer
    L.routed_scale = 1.0


@pytest.mark.parametrize("R", [8, 16])
def test_full_expert_parallel(c2, R):
    L, inp = c2
    Is = 2048
    rng = np.random.default_rng(R)
    S = Is // R
    w13s = W.f32_to_bf16_bits((rng.standard_normal((R, 2 * S, L.d)) / np.sqrt(L.d)).astype(np.float32))
    w2s = W.f32_to_bf16_bits((rng.standard_normal((R, L.d, S)) / np.sqrt(L.d)).astype(np.float32))
    dims = dims_of(L)
    bufs = dict(partials=torch.empty((R, L.T, L.d), dtype=torch.bfloat16, device="cuda"),
                w13_shared=dev(w13s), w2_shared=dev(w2s),
                h_shared=torch.empty((R, L.T, S), dtype=torch.bfloat16, device="cuda"),
                y_shared=torch.empty((R, L.T, L.d), dtype=torch.float32, device="cuda"))
    b = _forward(L, inp, None, 2.5, bufs=bufs, ranks=R, inter_shared=Is,
                 shared_workspace=M.alloc_shared_workspace(dims, R, Is))
    toks = sample_tokens(L.T, 8, seed=R)
    inv = host(b["inv"]).reshape(L.T, L.k)
    y = host(b["y"])
    rows = inv[toks].reshape(-1)
    ys = host(b["y_shared"])[:, toks]
    parts, out = oracle.combine_ranks(y[rows], np.arange(len(rows), dtype=np.int32),
                                      host(b["topk_w"])[toks], host(b["topk_idx"])[toks], L.E,
                                      R, "bf16", y_shared=ys, scale=2.5)
    assert host(b["out"])[toks].tobytes() == out.tobytes()
    assert host(b["partials"])[:, toks].tobytes() == parts.tobytes()
    r_h, r_y = oracle.shared_ffn(np.ascontiguousarray(L.x[toks]), w13s, w2s, "bf16")
    assert_close(as_f32(host(b["h_shared"])[:, toks], "bf16"), as_f32(r_h, "bf16"), "bf16", "h_shared")
    assert_close(ys, r_y, "bf16", "y_shared")


@pytest.mark.parametrize("g16", [False, True], ids=["f32_operands", "bf16_operands"])
def test_full_backward(c2, g16):
    L, inp = c2
    dims = dims_of(L)
    fb = _forward(L, inp)
    gd = M.MOE_BF16 if g16 else M.MOE_F32
    bb = M.alloc_backward_buffers(dims, "cuda", router=True, grad_dtype=gd)
    dout = W.f32_to_bf16_bits(np.random.default_rng(9).normal(0, 1, (L.T, L.d)).astype(np.float32))
    bb.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
              logit_bias=inp["logit_bias"], logits=fb["logits"], offsets=fb["offsets"],
              perm=fb["perm"], inv=fb["inv"], topk_w=fb["topk_w"], h=fb["h"], y=fb["y"],
              d_out=dev(dout))
    M.backward(dims, bb, M.alloc_workspace(dims), grad_dtype=gd)
    torch.cuda.synchronize()
    k, E = L.k, L.E
    # sampled tokens: the oracle's backward of just these tokens, on the GPU's saved h / y
    toks = sample_tokens(L.T, 6, seed=11)
    idx = host(fb["topk_idx"])[toks]
    w = host(fb["topk_w"])[toks]
    inv_full = host(fb["inv"]).reshape(L.T, k)[toks].reshape(-1)
    counts, offsets, perm, inv, _ = oracle.permute(idx, E)
    src = inv_full[perm]                        # sub-batch row p -> full row
    h = host(fb["h"])[src]
    y = host(fb["y"])[src]
    xs = np.ascontiguousarray(L.x[toks])
    be = oracle.backward_experts(xs, perm, inv, counts, w, L.w13, L.w2, h, y,
                                 np.ascontiguousarray(dout[toks]), "bf16", 1.0, round_grads=g16)
    br = oracle.backward_router(host(fb["logits"])[toks], be["dw"], xs, L.w_router, "bf16")
    def close(got, ref, what, tol):
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        err = float((np.abs(got - ref) / np.maximum(1.0, np.abs(ref))).max())
        assert err <= tol, f"{what}: {err:.3e} > {tol}"

    # the backward's bound: FP32 sums of up to d = 2048 signed terms in different orders
    close(host(bb["d_topk_w"])[toks], be["dw"], "d_topk_w", 1e-4)
    close(host(bb["d_logits"])[toks], br["dl"], "d_logits", 1e-4)
    close(host(bb["d_x"])[toks], be["dx"] + br["dx"], "d_x", 2e-2 if g16 else 1e-4)
    # the smallest non-empty expert's whole segment: its weight gradients in float64 from
    # the GPU's own dy / d_gu (the operands the kernels consumed)
    offs = host(fb["offsets"])
    cnt = np.diff(offs)
    e = int(np.argmin(np.where(cnt > 0, cnt, 1 << 30)))
    p0, p1 = offs[e], offs[e + 1]
    cv = (lambda a: as_f32(a, "bf16")) if g16 else (lambda a: a)
    dy = cv(host(bb["d_y"])[p0:p1]).astype(np.float64)
    dgu = cv(host(bb["d_gu"])[p0:p1]).astype(np.float64)
    hh = as_f32(host(fb["h"])[p0:p1], "bf16").astype(np.float64)
    xr = as_f32(L.x, "bf16").astype(np.float64)[host(fb["perm"])[p0:p1] // k]
    for n, ref in (("d_w2", dy.T @ hh), ("d_w13", dgu.T @ xr)):
        g = host(bb[n])[e].astype(np.float64)
        err = float((np.abs(g - ref) / np.maximum(1.0, np.abs(ref))).max())
        assert err <= 1e-4, f"{n}[{e}] ({p1 - p0} rows): {err:.3e}"
