"""moe_forward under HIP graph capture: the library enqueues everything on the caller's
stream with no host synchronisation, memset or allocation, so a captured step replays as
the eager one. Each graph is replayed several times with other eager work and host
synchronisations in between, and every replay's outputs must be bitwise the eager
step's."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import workloads as W
from gpu_util import dims_of, host, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()


OUTS = ("out", "topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "h", "y",
        "weighted_counts", "prob_mass", "logits", "d_err")


@pytest.mark.parametrize("T,mode,d", [(1, "router", 256), (48, "router", 256),
                                      (700, "router", 256), (300, "replay", 256),
                                      # d/16 >= 256: the one-launch down GEMM + combine
                                      (1, "router", 4096), (2, "router", 4096),
                                      (2, "replay", 4096)])
def test_graph_replay_matches_eager(T, mode, d):
    E, I = (32, 128) if d == 256 else (16, 768)
    L = W.make_layer(T=T, d=d, E=E, k=8, I=I, dtype="bf16", mode=mode, seed=T,
                     bias="zipf", replay="uniform")
    L.token_mult = W.token_multiplicities(T, 1)
    inp = upload(L)
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=(mode == "router"), weighted=True)
    del b["x_perm"]
    b.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], token_mult=inp["token_mult"])
    if mode == "router":
        b["w_router"], b["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        b["idx_in"], b["w_in"] = inp["idx_in"], inp["w_in"]
    ws = M.alloc_workspace(dims)
    M.forward(dims, b, ws)
    torch.cuda.synchronize()
    ref = {n: host(b[n]).copy() for n in OUTS if n in b}
    # capture on a side stream (torch's graph context makes it the current stream)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.forward(dims, b, ws)                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        M.forward(dims, b, ws)
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for n in OUTS:
            if n in b and n != "d_err":
                b[n].zero_() if b[n].dtype != torch.bfloat16 else b[n].view(torch.int16).zero_()
        junk.mul_(1.0001).sum()                     # other eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, r in ref.items():
            assert host(b[n]).tobytes() == r.tobytes(), (T, mode, rep, n)
    assert int(b["d_err"].item()) == 0
