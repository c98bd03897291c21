"""Helpers for the GPU parity tests: host<->device copies and tolerance checks."""
import numpy as np
import torch

import moe_layer_routing_amd as M
import workloads as W

# float tolerance from the target: |gpu - ref| <= tol * max(1, |ref|)
TOL = {"f32": 1e-5, "bf16": 2e-2}
U = 2.0 ** -24


def dev(a, device="cuda"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t):
    """Device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f32(a, dtype):
    return W.bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)


def assert_close(gpu, ref, dtype, what):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r) / np.maximum(1.0, np.abs(r))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dtype], f"{what}: max scaled error {worst:.3e} > {TOL[dtype]}"
    return worst


def dims_of(L, tile_m=0):
    return M.make_dims(L.T, L.d, L.E, L.k, L.I, M.MOE_BF16 if L.dtype == "bf16" else M.MOE_F32,
                       tile_m)


def upload(L, device="cuda"):
    return dict(x=dev(L.x, device), w_router=dev(L.w_router, device),
                logit_bias=dev(L.logit_bias, device), idx_in=dev(L.idx_in, device),
                w_in=dev(L.w_in, device), w13=dev(L.w13, device), w2=dev(L.w2, device),
                token_mult=dev(L.token_mult, device), cu_seqlens=dev(L.cu_seqlens, device))


def run_forward(L, inputs=None, tile_m=0, device="cuda", stats=True, fused_gather=False):
    """moe_forward on layer L; returns (buffers dict, dims). fused_gather: pass no x_perm,
    so that the gate/up GEMM gathers token rows itself."""
    dims = dims_of(L, tile_m)
    inp = inputs if inputs is not None else upload(L, device)
    S = 0 if (L.cu_seqlens is None or not stats) else len(L.cu_seqlens) - 1
    b = M.alloc_forward_buffers(dims, device, router=(L.mode == "router"), num_seqs=S,
                                weighted=stats)
    for kname in ("x", "w13", "w2"):
        b[kname] = inp[kname]
    if L.mode == "router":
        b["w_router"] = inp["w_router"]
        b["logit_bias"] = inp["logit_bias"]
    else:
        b["idx_in"] = inp["idx_in"]
        b["w_in"] = inp["w_in"]
    if stats:
        b["token_mult"] = inp["token_mult"]
        if S:
            b["cu_seqlens"] = inp["cu_seqlens"]
    if fused_gather:
        del b["x_perm"]
    ws = M.alloc_workspace(dims, device)
    M.forward(dims, b, ws)
    torch.cuda.synchronize()
    return b, dims


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    n = min(n, T)
    t = set([0, T - 1])
    t.update(rng.choice(T, size=n, replace=False).tolist())
    return np.array(sorted(t))
