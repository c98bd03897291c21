"""Router variants, routed scaling factor and objective statistics on the GPU, against the
oracle ("0 train-infer mismatch ...", "Choosing GLM's eight experts" and "Hash and learned
expert routing"; "HARTS ...", eq. (20) and "MoE execution and objectives").

Parity protocol: the GPU's router logits are compared with the oracle's within the FP32
tolerance; the oracle then routes the GPU's logits, and every discrete result (expert ids,
counts, offsets, permutation) must match bit for bit. Weights, probability mass, lse and
outputs are compared within the tolerance; the objectives, computed from the same inputs
on both sides, agree to FP64 rounding."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import oracle
import workloads as W
from gpu_util import TOL, as_f32, assert_close, dev, dims_of, host, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()
    oracle.lib()


def _layer(T, E, k, score, bias, vocab=None, d=128, I=128, seed=0, dtype="bf16", scale=1.0):
    L = W.make_layer(T=T, d=d, E=E, k=k, I=I, dtype=dtype, mode="router", seed=seed,
                     bias="zipf")
    L.token_mult = W.token_multiplicities(T, seed + 1)
    W.set_router(L, score, bias=bias, hash_vocab=vocab, routed_scale=scale)
    return L


def _router_kw(L, lse=None):
    return dict(score=L.score, corr_bias=dev(L.corr_bias), hash_table=dev(L.hash_table),
                token_ids=dev(L.token_ids), lse=lse)


def _route(L, inp, tile_m=0):
    dims = dims_of(L, tile_m)
    T, E, k = L.T, L.E, L.k
    out = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
               topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
               logits=torch.empty((T, E), dtype=torch.float32, device="cuda"),
               prob_mass=torch.empty(E, dtype=torch.float32, device="cuda"),
               lse=torch.empty(T, dtype=torch.float32, device="cuda"),
               d_err=torch.zeros(1, dtype=torch.int32, device="cuda"))
    kw = _router_kw(L, out["lse"])
    M.route_scored(dims, inp["x"], inp["w_router"], inp["logit_bias"], out["topk_idx"],
                   out["topk_w"], logits=out["logits"], prob_mass=out["prob_mass"],
                   token_mult=inp["token_mult"], d_err=out["d_err"], **kw)
    torch.cuda.synchronize()
    return {n: host(v) for n, v in out.items()}


def _check_route(L, g):
    assert int(g["d_err"][0]) == 0
    ref_logits = oracle.router_logits(L.x, L.w_router, L.logit_bias, L.dtype)
    assert_close(g["logits"], ref_logits, "f32", "logits")
    r = oracle.route_scored(g["logits"], L.k, L.score, L.corr_bias, L.hash_table,
                            L.token_ids, L.token_mult)
    assert r["err"] == 0
    np.testing.assert_array_equal(g["topk_idx"], r["idx"])
    assert_close(g["topk_w"], r["w"], "f32", "topk_w")
    assert_close(g["lse"], r["lse"], "f32", "lse")
    np.testing.assert_allclose(g["prob_mass"], r["prob_mass"], rtol=1e-5,
                               atol=1e-5 * max(1.0, float(np.abs(r["prob_mass"]).max())))
    return r


ROUTE_CASES = [
    # (T, E, k, score, bias, vocab)
    (1, 8, 2, "sigmoid", True, None),
    (37, 64, 8, "sigmoid", True, None),
    (300, 256, 8, "sigmoid", True, None),
    (4100, 64, 8, "sigmoid", True, None),
    (300, 160, 8, "sigmoid", False, None),
    (513, 200, 6, "sqrt_softplus", True, None),
    (4100, 256, 6, "sqrt_softplus", True, None),
    (300, 17, 3, "sqrt_softplus", False, None),
    (300, 256, 6, "sqrt_softplus", False, 5000),
    (4100, 64, 6, "sqrt_softplus", False, 129),
    (77, 32, 4, "sigmoid", False, 1000),
    (300, 48, 8, "softmax", False, 700),
    (1, 1, 1, "sigmoid", True, None),
]


@pytest.mark.parametrize("case", ROUTE_CASES,
                         ids=lambda c: f"T{c[0]}_E{c[1]}_k{c[2]}_{c[3]}_{'b' if c[4] else 'nb'}"
                                       f"{'_hash' if c[5] else ''}")
def test_route_scored_parity(case):
    T, E, k, score, bias, vocab = case
    L = _layer(T, E, k, score, bias, vocab, seed=T + E)
    g = _route(L, upload(L))
    _check_route(L, g)


def test_route_scored_batch_invariant():
    """Each token's ids, weights and lse are the same bytes at any batch size."""
    for score, vocab in (("sigmoid", None), ("sqrt_softplus", None), ("sqrt_softplus", 900)):
        L = _layer(1000, 128, 8, score, True, vocab, seed=5)
        inp = upload(L)
        full = _route(L, inp)
        for T in (1, 13, 64, 333):
            Ls = _layer(T, 128, 8, score, True, vocab, seed=5)
            Ls.w_router, Ls.logit_bias, Ls.x = L.w_router, L.logit_bias, np.ascontiguousarray(L.x[:T])
            Ls.corr_bias = L.corr_bias
            if vocab:
                Ls.hash_table, Ls.token_ids = L.hash_table, np.ascontiguousarray(L.token_ids[:T])
            Ls.token_mult = np.ascontiguousarray(L.token_mult[:T])
            part = _route(Ls, upload(Ls))
            for n in ("logits", "topk_idx", "topk_w", "lse"):
                assert part[n].tobytes() == full[n][:T].tobytes(), (score, vocab, T, n)


def test_softmax_options_match_moe_route():
    """route_scored with the softmax router and no options is moe_route, bit for bit."""
    L = W.make_layer(T=1000, d=256, E=64, k=8, I=64, mode="router", seed=3, bias="zipf")
    L.token_mult = W.token_multiplicities(L.T, 3)
    inp = upload(L)
    dims = dims_of(L)
    a = M.alloc_forward_buffers(dims, "cuda")
    M.route(dims, inp["x"], inp["w_router"], inp["logit_bias"], a["topk_idx"], a["topk_w"],
            logits=a["logits"], prob_mass=a["prob_mass"], token_mult=inp["token_mult"])
    L.score = "softmax"
    g = _route(L, inp)
    for n in ("topk_idx", "topk_w", "logits", "prob_mass"):
        assert g[n].tobytes() == host(a[n]).tobytes(), n
    r = oracle.route_scored(g["logits"], L.k, "softmax", token_mult=L.token_mult)
    assert_close(g["lse"], r["lse"], "f32", "lse")


def test_route_scored_rejects_bad_options():
    L = _layer(10, 16, 2, "sigmoid", True)
    inp = upload(L)
    dims = dims_of(L)
    idx = torch.empty((10, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((10, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoeError):      # softmax chooses on logits: no correction bias
        M.route_scored(dims, inp["x"], inp["w_router"], None, idx, w, score="softmax",
                       corr_bias=dev(L.corr_bias))
    with pytest.raises(M.MoeError):      # a table needs token ids
        M.route_scored(dims, inp["x"], inp["w_router"], None, idx, w,
                       hash_table=dev(W.hash_table(10, 16, 2, 0)))


def test_hash_routing_errors():
    E, k, T = 16, 2, 40
    L = _layer(T, E, k, "sigmoid", False, 50, seed=8)
    bad_tok = L.token_ids.copy()
    bad_tok[[3, 17]] = [50, -1]
    tab = L.hash_table.copy()
    for name, tok, table, bit in (("token", bad_tok, L.hash_table, M.DERR_IDX_RANGE),
                                  ("range", L.token_ids, np.where(tab == tab[L.token_ids[5], 1], 99, tab), M.DERR_IDX_RANGE),
                                  ("dup", L.token_ids, np.repeat(tab[:, :1], 2, axis=1), M.DERR_IDX_DUP)):
        L.token_ids, L.hash_table = np.ascontiguousarray(tok, np.int32), np.ascontiguousarray(table, np.int32)
        g = _route(L, upload(L))
        assert int(g["d_err"][0]) & bit, name
        r = oracle.route_scored(g["logits"], k, "sigmoid", None, L.hash_table, L.token_ids)
        assert r["err"] & bit
        np.testing.assert_array_equal(g["topk_idx"], r["idx"])
        np.testing.assert_array_equal(g["topk_w"] == 0, r["w"] == 0)
        # and the layer's other outputs stay inside their buffers
        L.token_ids, L.hash_table = W.token_ids(T, 50, 8), W.hash_table(50, E, k, 8)


# ------------------------------------------------------------------- whole layer

FWD_CASES = [
    # (T, E, k, score, bias, vocab, scale, dtype)
    (40, 64, 8, "sigmoid", True, None, 2.5, "bf16"),       # single-block routing tail
    (64, 160, 8, "sigmoid", True, None, 2.5, "bf16"),
    (500, 160, 8, "sigmoid", True, None, 2.5, "bf16"),     # multi-kernel path
    (20, 64, 6, "sqrt_softplus", False, 300, 1.5, "bf16"),
    (700, 64, 6, "sqrt_softplus", False, 3000, 1.5, "bf16"),
    (300, 32, 6, "sqrt_softplus", True, None, 1.0, "f32"),
    (33, 16, 4, "sigmoid", True, None, 2.5, "f32"),
]


@pytest.mark.parametrize("case", FWD_CASES,
                         ids=lambda c: f"T{c[0]}_E{c[1]}_{c[3]}{'_hash' if c[5] else ''}_{c[7]}")
def test_forward_router_variant(case):
    T, E, k, score, bias, vocab, scale, dtype = case
    L = _layer(T, E, k, score, bias, vocab, d=128, I=192, seed=7 + T, dtype=dtype, scale=scale)
    inp = upload(L)
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=True, weighted=True)
    b.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
             logit_bias=inp["logit_bias"], token_mult=inp["token_mult"])
    lse = torch.empty(T, dtype=torch.float32, device="cuda")
    M.forward(dims, b, M.alloc_workspace(dims), router=_router_kw(L, lse), routed_scale=scale)
    torch.cuda.synchronize()
    assert int(b["d_err"].item()) == 0
    r = oracle.forward(L, logits=host(b["logits"]))
    np.testing.assert_array_equal(host(b["topk_idx"]), r["idx"])
    for n in ("counts", "offsets", "perm", "inv", "weighted_counts"):
        np.testing.assert_array_equal(host(b[n]), r[n], err_msg=n)
    assert_close(host(b["topk_w"]), r["w"], "f32", "topk_w")
    assert_close(host(lse), r["lse"], "f32", "lse")
    assert_close(host(b["prob_mass"]), r["prob_mass"], dtype, "prob_mass")
    assert_close(as_f32(host(b["out"]), dtype), as_f32(r["out"], dtype), dtype, "out")


def test_forward_variant_small_and_large_paths_agree():
    """T = 64 (single-block tail) and T = 65 (multi-kernel path) give the same bytes for
    the first 64 tokens under a scored router, a correction bias and the scaling factor."""
    for score, vocab in (("sigmoid", None), ("sqrt_softplus", 400)):
        L = _layer(65, 64, 8, score, True, vocab, d=256, I=128, seed=21, scale=2.5)
        outs = []
        for T in (65, 64):
            Lt = _layer(T, 64, 8, score, True, vocab, d=256, I=128, seed=21, scale=2.5)
            Lt.w13, Lt.w2, Lt.w_router, Lt.logit_bias = L.w13, L.w2, L.w_router, L.logit_bias
            Lt.x, Lt.corr_bias = np.ascontiguousarray(L.x[:T]), L.corr_bias
            Lt.token_mult = np.ascontiguousarray(L.token_mult[:T])
            if vocab:
                Lt.hash_table, Lt.token_ids = L.hash_table, np.ascontiguousarray(L.token_ids[:T])
            inp = upload(Lt)
            dims = dims_of(Lt)
            b = M.alloc_forward_buffers(dims, "cuda", router=True, weighted=True)
            b.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
                     logit_bias=inp["logit_bias"], token_mult=inp["token_mult"])
            M.forward(dims, b, M.alloc_workspace(dims), router=_router_kw(Lt), routed_scale=2.5)
            torch.cuda.synchronize()
            outs.append({n: host(b[n]) for n in ("topk_idx", "topk_w", "out")})
        for n in ("topk_idx", "topk_w", "out"):
            assert outs[1][n].tobytes() == outs[0][n][:64].tobytes(), (score, n)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_scaled_parity(dtype):
    rng = np.random.default_rng(4)
    T, k, d = 777, 6, 512
    y = rng.normal(0, 1, size=(T * k, d)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    dims = M.make_dims(T, d, 64, k, 64, M.MOE_BF16 if dtype == "bf16" else M.MOE_F32)
    out = torch.empty((T, d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device="cuda")
    for scale in (2.5, 1.0, 0.375):
        M.combine(dims, dev(y), dev(inv), dev(w), out, routed_scale=scale)
        torch.cuda.synchronize()
        ref = oracle.combine(y, inv, w, dtype, scale)
        # same FP32 operations in the same order on both sides
        assert host(out).tobytes() == ref.tobytes(), scale
    base = torch.empty_like(out)
    M.combine(dims, dev(y), dev(inv), dev(w), base)
    M.combine(dims, dev(y), dev(inv), dev(w), out, routed_scale=1.0)
    torch.cuda.synchronize()
    assert host(out).tobytes() == host(base).tobytes()
    with pytest.raises(M.MoeError):
        M.combine(dims, dev(y), dev(inv), dev(w), out, routed_scale=float("inf"))


# -------------------------------------------------------------------- objectives

@pytest.mark.parametrize("placed", [False, True], ids=["identity", "placed"])
def test_objectives_parity(placed):
    L = _layer(3000, 64, 8, "sigmoid", True, None, d=128, I=64, seed=12)
    inp = upload(L)
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=True, weighted=True)
    b.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
             logit_bias=inp["logit_bias"], token_mult=inp["token_mult"])
    slot = None
    if placed:
        m = np.random.default_rng(1).permutation(L.E).astype(np.int32)
        slot = dev(m)
        b["slot_of_expert"] = slot
        inv_m = np.argsort(m)
        b["w13"], b["w2"] = inp["w13"][dev(inv_m).long()], inp["w2"][dev(inv_m).long()]
    lse = torch.empty(L.T, dtype=torch.float32, device="cuda")
    M.forward(dims, b, M.alloc_workspace(dims), router=_router_kw(L, lse), routed_scale=2.5)
    bias = dev(L.corr_bias).clone()
    out = torch.zeros(3, dtype=torch.float64, device="cuda")
    M.objectives(dims, out, lse=lse, token_mult=inp["token_mult"],
                 weighted_counts=b["weighted_counts"], prob_mass=b["prob_mass"],
                 slot_of_expert=slot, bias_rate=1e-3, corr_bias=bias, d_err=b["d_err"])
    torch.cuda.synchronize()
    assert int(b["d_err"].item()) == 0
    wc = host(b["weighted_counts"])
    C = wc[m] if placed else wc
    z, aux, S, nb = oracle.objectives(host(lse), L.token_mult, C, host(b["prob_mass"]), L.k,
                                      1e-3, L.corr_bias)
    g = host(out)
    assert int(g[2]) == S == int(L.token_mult.sum())
    assert g[0] == pytest.approx(z, rel=1e-13)
    assert g[1] == pytest.approx(aux, rel=1e-13)
    assert host(bias).tobytes() == nb.tobytes()
    # and against the oracle's own routing of the same layer (FP32 tolerance)
    r = oracle.forward(L, logits=host(b["logits"]))
    z2, aux2, _, _ = oracle.objectives(r["lse"], L.token_mult, r["weighted_counts"],
                                       r["prob_mass"], L.k)
    assert g[0] == pytest.approx(z2, rel=TOL["f32"])
    assert g[1] == pytest.approx(aux2, rel=TOL["f32"])


def test_objectives_edge_cases():
    dims = M.make_dims(0, 64, 8, 2, 64, M.MOE_BF16)
    out = torch.full((3,), 7.0, dtype=torch.float64, device="cuda")
    M.objectives(dims, out)                    # T = 0: S = 0, both losses 0
    torch.cuda.synchronize()
    assert host(out).tolist() == [0.0, 0.0, 0.0]
    # counts without multiplicities; a bad placement map is reported
    dims = M.make_dims(4, 64, 4, 2, 64, M.MOE_BF16)
    wc = dev(np.array([3, 3, 2, 0], np.int64))
    mass = dev(np.array([1.5, 1.5, 1.0, 0.0], np.float32))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    M.objectives(dims, out, weighted_counts=wc, prob_mass=mass,
                 slot_of_expert=dev(np.array([0, 1, 2, 7], np.int32)), d_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & M.DERR_SLOTMAP
    M.objectives(dims, out, weighted_counts=wc, prob_mass=mass)
    torch.cuda.synchronize()
    # S = 4, aux = 4 / (2 * 16) * (4.5 + 4.5 + 2) = 1.375
    assert host(out).tolist() == [0.0, 1.375, 4.0]
    with pytest.raises(M.MoeError):            # a bias update needs the counts
        M.objectives(dims, out, corr_bias=dev(np.zeros(4, np.float32)))
