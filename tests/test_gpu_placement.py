"""Logical -> physical expert placement on the GPU ("RoutePack ...", Sec. 3: the router keeps
logical ids, the dispatcher sends logical expert e to slot slot_of_expert[e], whose weights
are the expert's). Under any placement every output row of the layer is bitwise the one
of the identity placement; counts and statistics move to the slots; the permutation is the
oracle's stable counting sort of the placed ids."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import oracle
import workloads as W
from gpu_util import dev, dims_of, host, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()
    oracle.lib()


def _forward(L, inp, slot=None, fused=False):
    dims = dims_of(L)
    S = 0 if L.cu_seqlens is None else len(L.cu_seqlens) - 1
    b = M.alloc_forward_buffers(dims, "cuda", router=(L.mode == "router"), num_seqs=S,
                                weighted=True)
    w13, w2 = inp["w13"], inp["w2"]
    if slot is not None:
        expert_of_slot = torch.empty_like(slot)
        expert_of_slot[slot.long()] = torch.arange(L.E, dtype=slot.dtype, device=slot.device)
        w13 = w13[expert_of_slot.long()].contiguous()   # slot v holds expert expert_of_slot[v]
        w2 = w2[expert_of_slot.long()].contiguous()
        b["slot_of_expert"] = slot
    b.update(x=inp["x"], w13=w13, w2=w2, token_mult=inp["token_mult"])
    if L.mode == "router":
        b["w_router"], b["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        b["idx_in"], b["w_in"] = inp["idx_in"], inp["w_in"]
    if S:
        b["cu_seqlens"] = inp["cu_seqlens"]
    if fused:
        del b["x_perm"]
    M.forward(dims, b, M.alloc_workspace(dims))
    torch.cuda.synchronize()
    return b


CASES = [
    dict(name="router_T300", T=300, d=256, E=16, k=4, I=192, mode="router", bias="zipf"),
    dict(name="router_T40_small", T=40, d=128, E=32, k=8, I=128, mode="router", bias="zipf"),
    dict(name="replay_seqs", T=500, d=128, E=64, k=8, I=128, mode="replay", replay="dirichlet"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
@pytest.mark.parametrize("fused", [False, True], ids=["xperm", "fused"])
def test_placement_keeps_every_row(case, fused):
    c = dict(case)
    name = c.pop("name")
    L = W.make_layer(dtype="bf16", seed=40 + c["T"], name=name, **c)
    L.token_mult = W.token_multiplicities(L.T, 4)
    inp = upload(L)
    ref = _forward(L, inp, fused=fused)
    assert int(ref["d_err"].item()) == 0
    idx = host(ref["topk_idx"])
    counts_id = host(ref["counts"])
    rng = np.random.default_rng(c["T"])
    lpt, _, _ = oracle.place_lpt(counts_id.astype(np.int64), 4)
    maps = {"lpt": lpt, "random": rng.permutation(L.E).astype(np.int32),
            "reversed": np.arange(L.E, dtype=np.int32)[::-1].copy()}
    inv_id = host(ref["inv"])
    for mname, m in maps.items():
        got = _forward(L, inp, slot=dev(m), fused=fused)
        assert int(got["d_err"].item()) == 0, mname
        # every per-token output is unchanged, bit for bit
        for n in ("out", "topk_idx", "topk_w") + (("logits", "prob_mass") if L.mode == "router"
                                                  else ()):
            assert host(got[n]).tobytes() == host(ref[n]).tobytes(), (mname, n)
        # statistics follow the slots
        counts = host(got["counts"])
        assert (counts[m] == counts_id).all(), mname
        assert (host(got["weighted_counts"])[m] == host(ref["weighted_counts"])).all(), mname
        if "seq_counts" in got:
            assert (host(got["seq_counts"])[:, m] == host(ref["seq_counts"])).all(), mname
        # the permutation is the stable counting sort of the placed ids
        r_counts, r_off, r_perm, r_inv, err = oracle.permute(oracle.place(idx, m), L.E)
        assert err == 0
        for n, r in (("counts", r_counts), ("offsets", r_off), ("perm", r_perm),
                     ("inv", r_inv)):
            np.testing.assert_array_equal(host(got[n]), r, err_msg=f"{mname} {n}")
        # each assignment's expert rows are the same bytes, only at the placed position
        inv = host(got["inv"])
        h_id, h = host(ref["h"]), host(got["h"])
        y_id, y = host(ref["y"]), host(got["y"])
        assert h[inv].tobytes() == h_id[inv_id].tobytes(), mname
        assert y[inv].tobytes() == y_id[inv_id].tobytes(), mname


def test_placement_map_errors():
    L = W.make_layer(T=100, d=128, E=8, k=2, I=64, dtype="bf16", mode="router", seed=77)
    inp = upload(L)
    inp["token_mult"] = None
    for bad in ([0, 1, 2, 3, 4, 5, 6, 6], [0, 1, 2, 3, 4, 5, 6, 9]):
        for T in (100, 20):                   # multi-kernel path and small-batch tail
            L2 = W.make_layer(T=T, d=128, E=8, k=2, I=64, dtype="bf16", mode="router",
                              seed=77, weights=False)
            L2.w13, L2.w2, L2.w_router, L2.logit_bias = L.w13, L.w2, L.w_router, L.logit_bias
            inp2 = dict(inp)
            inp2["x"] = dev(L2.x)
            dims = dims_of(L2)
            b = M.alloc_forward_buffers(dims, "cuda", router=True)
            b.update(x=inp2["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
                     slot_of_expert=dev(np.array(bad, dtype=np.int32)))
            M.forward(dims, b, M.alloc_workspace(dims))
            torch.cuda.synchronize()
            assert int(b["d_err"].item()) & M.DERR_SLOTMAP, (bad, T)
