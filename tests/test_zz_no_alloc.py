"""moe_forward_noalloc (the layer with the library's static per-GPU scratch as workspace)
against moe_forward with a caller workspace: every output bitwise equal, over calls in a
row on one GPU, each later call smaller than the one before (the scratch keeps the larger
call's contents), in router and replay mode, on the multi-kernel and the small-batch
routing paths, and with the shared expert's workspace carved from the same scratch."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import workloads as W
from gpu_util import dims_of, run_forward, upload

pytestmark = pytest.mark.gpu

OUTS = ("topk_idx", "topk_w", "logits", "prob_mass", "counts", "offsets", "perm", "inv",
        "seq_counts", "weighted_counts", "x_perm", "h", "y", "out", "d_err")


def _same(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    return a.shape == b.shape and bool(torch.equal(a, b))


def _noalloc(L, inp, fused_gather=True):
    """The buffers of one moe_forward_noalloc call on layer L (no workspace allocated)."""
    dims = dims_of(L)
    S = 0 if L.cu_seqlens is None else len(L.cu_seqlens) - 1
    b = M.alloc_forward_buffers(dims, "cuda", router=(L.mode == "router"), num_seqs=S,
                                weighted=True)
    for n in ("x", "w13", "w2"):
        b[n] = inp[n]
    if L.mode == "router":
        b["w_router"], b["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        b["idx_in"], b["w_in"] = inp["idx_in"], inp["w_in"]
    b["token_mult"] = inp["token_mult"]
    if S:
        b["cu_seqlens"] = inp["cu_seqlens"]
    if fused_gather:
        del b["x_perm"]
    M.forward_noalloc(dims, b)
    torch.cuda.synchronize()
    return b


def _compare(L, inp, fused_gather=True):
    ref, _ = run_forward(L, inp, fused_gather=fused_gather)
    got = _noalloc(L, inp, fused_gather)
    assert int(got["d_err"].item()) == 0
    n = 0
    for name in OUTS:
        if name in ref and name in got and ref[name] is not None and got[name] is not None:
            assert _same(got[name], ref[name]), (L.name, L.T, name)
            n += 1
    print(f"  noalloc {L.name} T={L.T} mode={L.mode}: {n} outputs bitwise equal", flush=True)


def _layer(T, mode, seed, **kw):
    L = W.make_layer(T=T, d=1024, E=64, k=8, I=512, dtype="bf16", mode=mode, seed=seed,
                     mult=True, **kw)
    L.name = f"noalloc-{mode}"
    return L


def test_noalloc_equals_forward_on_shrinking_calls():
    assert torch.cuda.is_available()
    # router mode: a large call, then a smaller one, then a small batch (routing tail)
    big = _layer(4096, "router", 71, bias="zipf")
    inp = upload(big)
    _compare(big, inp)
    for T in (1000, 37):
        L = _layer(T, "router", 71, bias="zipf")
        _compare(L, upload(L))
    # replay mode with per-sequence statistics, shrinking, materialised gather
    for T in (3000, 500):
        L = _layer(T, "replay", 72, replay="dirichlet")
        _compare(L, upload(L), fused_gather=False)


def test_noalloc_decode_shaped_calls():
    """Decode-sized calls with d = 4096 (T = 64, then 2 and 1: the last two run the down
    GEMM and the combine as one launch) on the same scratch."""
    assert torch.cuda.is_available()
    for T in (64, 2, 1):
        L = W.make_layer(T=T, d=4096, E=16, k=8, I=768, dtype="bf16", mode="router", seed=74,
                         mult=True, bias="zipf")
        L.name = "noalloc-decode"
        _compare(L, upload(L))


def test_noalloc_training_shaped_layer_twice():
    """The training-shaped layer (T=4096, d=2048, E=64, I=1408), then its first 1024
    tokens: the second, smaller call follows the first on the same scratch."""
    L = W.make_config("c2")
    L.token_mult = W.token_multiplicities(L.T, L.seed)
    inp = upload(L)
    _compare(L, inp)
    L.T = 1024
    L.x = np.ascontiguousarray(L.x[:1024])
    L.token_mult = np.ascontiguousarray(L.token_mult[:1024])
    _compare(L, upload(L))


def test_noalloc_shared_expert_and_ranks():
    """With the rank-partial output and a shared expert, whose workspace also comes from
    the scratch (after the layer's)."""
    L = _layer(2048, "router", 73, bias="zipf")
    inp = upload(L)
    dims = dims_of(L)
    R, Is = 8, 1024
    g = torch.Generator(device="cuda").manual_seed(3)
    w13s = (torch.randn((R, 2 * Is // R, L.d), generator=g, device="cuda") * 0.03).to(torch.bfloat16)
    w2s = (torch.randn((R, L.d, Is // R), generator=g, device="cuda") * 0.03).to(torch.bfloat16)

    def bufs():
        b = M.alloc_forward_buffers(dims, "cuda", router=True, weighted=True)
        del b["x_perm"]
        b.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
                 logit_bias=inp["logit_bias"], token_mult=inp["token_mult"],
                 w13_shared=w13s, w2_shared=w2s,
                 h_shared=torch.empty((R, L.T, Is // R), dtype=torch.bfloat16, device="cuda"),
                 y_shared=torch.empty((R, L.T, L.d), dtype=torch.float32, device="cuda"))
        return b

    ref = bufs()
    M.forward(dims, ref, M.alloc_workspace(dims, "cuda"), routed_scale=2.5, ranks=R,
              inter_shared=Is, shared_workspace=M.alloc_shared_workspace(dims, R, Is, "cuda"))
    got = bufs()
    M.forward_noalloc(dims, got, routed_scale=2.5, ranks=R, inter_shared=Is)
    torch.cuda.synchronize()
    for name in ("topk_idx", "topk_w", "perm", "h", "y", "h_shared", "y_shared", "out"):
        assert _same(got[name], ref[name]), name
