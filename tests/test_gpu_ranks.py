"""Expert-parallel output on one device, against the oracle ("0 train-infer mismatch ...",
"Sharding the experts" and the shared-expert passage): rank partial outputs (slot-order
FP32 with other ranks' slots as exact zeros, routed scaling factor, shared-expert shard,
one rounding) and their FP64 pairwise tree; the shared expert sharded over the ranks.

The rank combine does the same FP32 and FP64 operations in the same order as the oracle,
so on the same inputs its partials and output must be bitwise the oracle's; the shared
expert's GEMMs are compared within the bf16 tolerance and for batch invariance."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import oracle
import workloads as W
from gpu_util import as_f32, assert_close, dev, dims_of, host, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()
    oracle.lib()


def _shared_weights(R, Is, d, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    S = Is // R
    std = 1.0 / np.sqrt(d)
    w13 = (rng.standard_normal((R, 2 * S, d)) * std).astype(np.float32)
    w2 = (rng.standard_normal((R, d, S)) * std).astype(np.float32)
    if dtype == "bf16":
        return W.f32_to_bf16_bits(w13), W.f32_to_bf16_bits(w2)
    return w13, w2


RANK_CASES = [
    # (T, E, k, R, dtype, placed, shared, scale)
    (300, 64, 8, 8, "bf16", False, True, 2.5),
    (300, 64, 8, 16, "bf16", True, True, 2.5),
    (257, 48, 6, 3, "bf16", True, False, 1.0),
    (100, 40, 4, 5, "f32", False, True, 1.5),
    (64, 16, 8, 1, "bf16", False, False, 2.5),
    (33, 32, 2, 4, "f32", True, False, 1.0),
    (1, 16, 8, 16, "bf16", False, True, 2.5),
]


@pytest.mark.parametrize("case", RANK_CASES,
                         ids=lambda c: f"T{c[0]}_E{c[1]}_k{c[2]}_R{c[3]}_{c[4]}"
                                       f"{'_placed' if c[5] else ''}{'_shared' if c[6] else ''}")
def test_combine_ranks_bitwise(case):
    T, E, k, R, dtype, placed, shared, scale = case
    rng = np.random.default_rng(T + E + R)
    d = 512 + 64 * (T % 3)
    A = T * k
    y = rng.normal(0, 1, (A, d)).astype(np.float32)
    inv = rng.permutation(A).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    idx = np.argsort(rng.random((T, E)), 1)[:, :k].astype(np.int32)
    slot = rng.permutation(E).astype(np.int32) if placed else None
    ys = rng.normal(0, 0.5, (R, T, d)).astype(np.float32) if shared else None
    r_parts, r_out = oracle.combine_ranks(y, inv, w, idx, E, R, dtype, slot, ys, scale)
    dims = M.make_dims(T, d, E, k, 64, M.MOE_BF16 if dtype == "bf16" else M.MOE_F32)
    sd = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty((T, d), dtype=sd, device="cuda")
    parts = torch.empty((R, T, d), dtype=sd, device="cuda")
    M.combine_ranks(dims, R, dev(y), dev(inv), dev(w), dev(idx), out, slot_of_expert=dev(slot),
                    y_shared=dev(ys), routed_scale=scale, partials=parts)
    torch.cuda.synchronize()
    assert host(parts).tobytes() == r_parts.tobytes()
    assert host(out).tobytes() == r_out.tobytes()
    if R == 1 and not shared:
        plain = torch.empty_like(out)
        M.combine(dims, dev(y), dev(inv), dev(w), plain, routed_scale=scale)
        torch.cuda.synchronize()
        assert host(plain).tobytes() == host(out).tobytes()


def test_combine_ranks_tree_cancellation():
    """Partials whose FP64 sum depends on the tree's shape (via the shared shards; zero
    routing weights): the GPU reproduces the tree, not another order."""
    vals = [2.0 ** 100] + [1.0] * 7 + [-2.0 ** 100] + [1.0] * 7
    R, E, k, T, d = 16, 16, 1, 1, 64
    ys = np.zeros((R, T, d), np.float32)
    ys[:, 0, 0] = vals
    dims = M.make_dims(T, d, E, k, 64, M.MOE_BF16)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    M.combine_ranks(dims, R, dev(np.zeros((T * k, d), np.float32)), dev(np.zeros(1, np.int32)),
                    dev(np.zeros((1, 1), np.float32)), dev(np.zeros((1, 1), np.int32)), out,
                    y_shared=dev(ys))
    torch.cuda.synchronize()
    assert float(out[0, 0].float()) == 0.0       # left to right would give 7


def test_combine_ranks_rejects_bad_ranks():
    dims = M.make_dims(4, 64, 12, 2, 64, M.MOE_BF16)
    z = torch.zeros(8, 64, device="cuda")
    i = torch.zeros(8, dtype=torch.int32, device="cuda")
    w = torch.zeros(4, 2, device="cuda")
    o = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    for R in (0, 5, 17, 24):
        with pytest.raises(M.MoeError):
            M.combine_ranks(dims, R, z, i, w, i.view(4, 2), o)


@pytest.mark.parametrize("R,Is", [(8, 1024), (16, 2048), (3, 384), (1, 256)])
def test_shared_ffn_parity_and_invariance(R, Is):
    T, d = 300, 256
    rng = np.random.default_rng(R)
    x = W.f32_to_bf16_bits(rng.normal(0, 1, (T, d)).astype(np.float32))
    w13s, w2s = _shared_weights(R, Is, d, R)
    dims = M.make_dims(T, d, 16, 2, 64, M.MOE_BF16)
    S = Is // R
    h = torch.empty((R, T, S), dtype=torch.bfloat16, device="cuda")
    ys = torch.empty((R, T, d), dtype=torch.float32, device="cuda")
    M.shared_ffn(dims, R, Is, dev(x), dev(w13s), dev(w2s), h, ys)
    torch.cuda.synchronize()
    r_h, r_y = oracle.shared_ffn(x, w13s, w2s, "bf16")
    assert_close(as_f32(host(h), "bf16"), as_f32(r_h, "bf16"), "bf16", "h_shared")
    assert_close(host(ys), r_y, "bf16", "y_shared")
    # the same tokens in a smaller batch: the same bytes
    for Ts in (1, 37, 64):
        dims_s = M.make_dims(Ts, d, 16, 2, 64, M.MOE_BF16)
        h2 = torch.empty((R, Ts, S), dtype=torch.bfloat16, device="cuda")
        y2 = torch.empty((R, Ts, d), dtype=torch.float32, device="cuda")
        M.shared_ffn(dims_s, R, Is, dev(np.ascontiguousarray(x[:Ts])), dev(w13s), dev(w2s), h2, y2)
        torch.cuda.synchronize()
        assert host(h2).tobytes() == host(h)[:, :Ts].tobytes(), Ts
        assert host(y2).tobytes() == host(ys)[:, :Ts].tobytes(), Ts


def test_shared_ffn_rejects_bad_shapes():
    dims = M.make_dims(10, 128, 16, 2, 64, M.MOE_BF16)
    for R, Is in ((3, 1000), (16, 512), (0, 256), (32, 4096)):
        assert M.shared_workspace_size(dims, R, Is) == 0
        with pytest.raises(M.MoeError):
            M.shared_ffn(dims, R, Is, None, None, None, None, None,
                         workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))


def _forward_ep(L, inp, R, Is, w13s, w2s, scale, slot=None, router=None):
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=(L.mode == "router"), weighted=True)
    b.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], token_mult=inp["token_mult"])
    if L.mode == "router":
        b["w_router"], b["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        b["idx_in"], b["w_in"] = inp["idx_in"], inp["w_in"]
    if slot is not None:
        inv_m = np.argsort(slot)
        b["slot_of_expert"] = dev(slot)
        b["w13"] = inp["w13"][dev(inv_m).long()].contiguous()
        b["w2"] = inp["w2"][dev(inv_m).long()].contiguous()
    sd = b["out"].dtype
    S = Is // R
    b.update(partials=torch.empty((R, L.T, L.d), dtype=sd, device="cuda"),
             w13_shared=dev(w13s), w2_shared=dev(w2s),
             h_shared=torch.empty((R, L.T, S), dtype=sd, device="cuda"),
             y_shared=torch.empty((R, L.T, L.d), dtype=torch.float32, device="cuda"))
    M.forward(dims, b, M.alloc_workspace(dims), router=router, routed_scale=scale, ranks=R,
              inter_shared=Is, shared_workspace=M.alloc_shared_workspace(dims, R, Is))
    torch.cuda.synchronize()
    assert int(b["d_err"].item()) == 0
    return b


@pytest.mark.parametrize("T,mode,placed", [(40, "router", False), (500, "router", True),
                                           (300, "replay", False)])
def test_forward_expert_parallel_output(T, mode, placed):
    """The whole layer with 8 emulated ranks and a sharded shared expert: the output is
    bitwise the oracle's rank combine of the GPU's own expert outputs, and within the bf16
    tolerance of the oracle's layer computed from scratch."""
    E, k, R, Is = 64, 8, 8, 1024
    L = W.make_layer(T=T, d=256, E=E, k=k, I=128, dtype="bf16", mode=mode, seed=T,
                     bias="zipf", replay="uniform")
    L.token_mult = W.token_multiplicities(T, 2)
    router = None
    if mode == "router":
        W.set_router(L, "sigmoid", bias=True, routed_scale=2.5)
        router = dict(score="sigmoid", corr_bias=dev(L.corr_bias))
    scale = 2.5 if mode == "router" else 1.0
    w13s, w2s = _shared_weights(R, Is, L.d, 5)
    slot = np.random.default_rng(T).permutation(E).astype(np.int32) if placed else None
    inp = upload(L)
    b = _forward_ep(L, inp, R, Is, w13s, w2s, scale, slot, router)
    # bitwise: the oracle's rank combine on the GPU's expert outputs
    parts, out = oracle.combine_ranks(host(b["y"]), host(b["inv"]), host(b["topk_w"]),
                                      host(b["topk_idx"]), E, R, "bf16", slot,
                                      host(b["y_shared"]), scale)
    assert host(b["partials"]).tobytes() == parts.tobytes()
    assert host(b["out"]).tobytes() == out.tobytes()
    # from scratch: routing on the GPU's logits, experts, shared expert, rank combine
    r = oracle.forward(L, logits=host(b["logits"]) if mode == "router" else None)
    np.testing.assert_array_equal(host(b["topk_idx"]), r["idx"])
    _, r_ys = oracle.shared_ffn(L.x, w13s, w2s, "bf16")
    inv_ref = r["inv"]
    _, r_out = oracle.combine_ranks(r["y"], inv_ref, r["w"], r["idx"], E, R, "bf16", slot,
                                    r_ys, scale)
    assert_close(as_f32(host(b["out"]), "bf16"), as_f32(r_out, "bf16"), "bf16", "out")


def test_forward_expert_parallel_rows_batch_invariant():
    E, k, R, Is = 32, 8, 16, 2048
    L = W.make_layer(T=65, d=256, E=E, k=k, I=128, dtype="bf16", mode="router", seed=9,
                     bias="zipf")
    w13s, w2s = _shared_weights(R, Is, L.d, 9)
    inp = upload(L)
    inp["token_mult"] = None
    big = _forward_ep(L, inp, R, Is, w13s, w2s, 2.5)
    L64 = W.make_layer(T=64, d=256, E=E, k=k, I=128, dtype="bf16", mode="router", seed=9,
                       bias="zipf", weights=False)
    L64.x = np.ascontiguousarray(L.x[:64])
    inp64 = dict(inp)
    inp64["x"] = dev(L64.x)
    small = _forward_ep(L64, inp64, R, Is, w13s, w2s, 2.5)
    for n in ("out", "topk_idx", "topk_w"):
        assert host(small[n]).tobytes() == host(big[n])[:64].tobytes(), n
    assert host(small["partials"]).tobytes() == host(big["partials"])[:, :64].tobytes()
