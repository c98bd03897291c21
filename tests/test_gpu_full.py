"""Full-size workloads in the launch configuration the benchmark times.

Integer outputs are checked in full against the oracle; expert rows (h, y) and output rows
on a sample of tokens the oracle computes one by one. The decode-shaped workload checks
that every output row is bitwise identical across T = 1..64, across token order, across
token-tile heights, and inside a prefill-shaped batch of 4096 tokens."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import oracle
import workloads as W
from gpu_util import as_f32, assert_close, dev, host, run_forward, sample_tokens, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()
    oracle.lib()


def _print(*a):
    print(*a, flush=True)


def _check_full(L, b, n_sample=12):
    dtype = L.dtype
    assert int(b["d_err"].item()) == 0
    if L.mode == "router":
        g_lg = host(b["logits"])
        ref_lg = oracle.router_logits(L.x, L.w_router, L.logit_bias, dtype)
        assert_close(g_lg, ref_lg, dtype, "logits")
        idx, w, mass, err = oracle.route_from_logits(g_lg, L.k, L.token_mult)
        assert err == 0
        np.testing.assert_array_equal(host(b["topk_idx"]), idx)
        assert_close(host(b["topk_w"]), w, dtype, "topk_w")
        assert_close(host(b["prob_mass"]), mass, dtype, "prob_mass")
    else:
        idx, w = L.idx_in, L.w_in
        assert oracle.replay_check(idx, w, L.E) == 0
        np.testing.assert_array_equal(host(b["topk_idx"]), idx)
        assert host(b["topk_w"]).tobytes() == np.ascontiguousarray(w).tobytes()
    counts, offsets, perm, inv, err = oracle.permute(idx, L.E)
    for n, r in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        np.testing.assert_array_equal(host(b[n]), r, err_msg=n)
    wc, _ = oracle.weighted_counts(idx, L.E, L.token_mult)
    np.testing.assert_array_equal(host(b["weighted_counts"]), wc)
    if "seq_counts" in b:
        sc, _ = oracle.seq_counts(idx, L.E, L.cu_seqlens)
        np.testing.assert_array_equal(host(b["seq_counts"]), sc)
    toks = sample_tokens(L.T, n_sample, seed=L.seed)
    # x_perm rows of the sampled tokens
    xp = host(b["x_perm"])
    for t in toks:
        for j in range(L.k):
            assert xp[inv[t * L.k + j]].tobytes() == L.x[t].tobytes()
    rh, ry, rout = oracle.forward_tokens(L, toks, idx, w)
    rows = inv.reshape(L.T, L.k)[toks]                       # [n, k]
    gh = host(b["h"])[rows.reshape(-1)].reshape(rh.shape)
    gy = host(b["y"])[rows.reshape(-1)].reshape(ry.shape)
    eh = assert_close(as_f32(gh, dtype), as_f32(rh, dtype), dtype, "h")
    ey = assert_close(gy, ry, dtype, "y")
    eo = assert_close(as_f32(host(b["out"])[toks], dtype), as_f32(rout, dtype), dtype, "out")
    _print(f"  {L.name}: sampled {len(toks)} tokens, max scaled err h={eh:.2e} y={ey:.2e} "
           f"out={eo:.2e}; expert rows min/max {counts.min()}/{counts.max()}")


@pytest.mark.parametrize("cfg", ["c2", "c3", "c4"])
def test_full_config(cfg):
    _print("generating", cfg)
    L = W.make_config(cfg)
    L.token_mult = W.token_multiplicities(L.T, L.seed)
    _print("running", cfg, L.T, L.d, L.E, L.k, L.I)
    inp = upload(L)
    b, dims = run_forward(L, inp)
    _check_full(L, b)
    # the launch the benchmark times (gather fused into the gate/up GEMM): same bytes
    f, _ = run_forward(L, inp, fused_gather=True)
    for n in ("topk_idx", "topk_w", "perm", "inv", "h", "y", "out", "counts", "offsets"):
        assert _same(f[n], b[n]), n
    _check_segment_ends(L, f)
    # the automatic tile height is 256 rows on all three layers; 128-row tiles give the
    # same bytes
    t, _ = run_forward(L, inp, tile_m=128, fused_gather=True)
    for n in ("h", "y", "out"):
        assert _same(t[n], f[n]), n


def _same(a, b):
    """Bitwise equality of two device tensors."""
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    if a.dtype == torch.bfloat16:
        return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))
    if a.dtype == torch.float32:
        return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))
    return bool(torch.equal(a, b))


def _check_segment_ends(L, b):
    """The first and last row of every non-empty expert segment (so every expert's ragged
    last token tile, at the tile height the benchmark runs) against the oracle's expert
    FFN of that row."""
    offs, perm, cnt = host(b["offsets"]), host(b["perm"]), host(b["counts"])
    live = np.nonzero(cnt)[0]
    rows = np.unique(np.concatenate([offs[live], offs[live + 1] - 1])).astype(np.int64)
    rowexp = (np.searchsorted(offs, rows, side="right") - 1).astype(np.int32)
    assert (cnt[rowexp] > 0).all()
    xr = np.ascontiguousarray(L.x[perm[rows] // L.k])
    rh, ry = oracle.expert_ffn(xr, rowexp, L.w13, L.w2, L.dtype)
    ri = torch.from_numpy(rows).to(b["h"].device)
    gh, gy = host(b["h"][ri]), host(b["y"][ri])
    eh = assert_close(as_f32(gh, L.dtype), as_f32(rh, L.dtype), L.dtype, "segment-end h")
    ey = assert_close(gy, ry, L.dtype, "segment-end y")
    _print(f"  {L.name}: {len(rows)} segment-end rows of {len(live)} experts, max scaled err "
           f"h={eh:.2e} y={ey:.2e}")


def test_c1_full_exact_oracle():
    L = W.make_config("c1")
    L.token_mult = W.token_multiplicities(L.T, 1)
    b, _ = run_forward(L)
    _check_full(L, b, n_sample=L.T)


def test_c5_batch_invariance():
    """Decode-shaped layer: the same token's routing, expert rows and output row are
    bitwise identical for every T in 1..64, for reversed token order, for each token-tile
    height, and inside a 4096-token batch."""
    _print("generating c5")
    L = W.make_config("c5")
    pool = L.x                                  # 64 rows
    inp = upload(L)
    ref_out = ref_idx = ref_w = None

    def run(x_rows, tile_m=0, fused=False):
        L2 = W.make_config("c5", T=len(x_rows), weights=False)
        L2.x = np.ascontiguousarray(x_rows)
        L2.w13, L2.w2 = L.w13, L.w2
        inp2 = dict(inp)
        inp2["x"] = dev(L2.x)
        b, _ = run_forward(L2, inp2, tile_m=tile_m, stats=False, fused_gather=fused)
        assert int(b["d_err"].item()) == 0
        return host(b["out"]), host(b["topk_idx"]), host(b["topk_w"]), b

    ref_out, ref_idx, ref_w, b64 = run(pool)
    for T in range(1, 65):
        out, idx, w, _ = run(pool[:T])
        assert out.tobytes() == ref_out[:T].tobytes(), T
        assert idx.tobytes() == ref_idx[:T].tobytes(), T
        assert w.tobytes() == ref_w[:T].tobytes(), T
    # one token with the gather fused into the gate/up GEMM (the decode step's launches:
    # the gate/up launch routes the token itself) and for T = 2 (routing tail): same bits
    for rows in (pool[0:1], pool[17:18], pool[63:64], pool[40:42]):
        t0 = int(np.flatnonzero((pool == rows[0]).all(axis=1))[0])
        T = len(rows)
        out, idx, w, b1 = run(rows, fused=True)
        assert out.tobytes() == ref_out[t0:t0 + T].tobytes(), (t0, T)
        assert idx.tobytes() == ref_idx[t0:t0 + T].tobytes(), (t0, T)
        assert w.tobytes() == ref_w[t0:t0 + T].tobytes(), (t0, T)
        assert host(b1["logits"]).tobytes() == host(b64["logits"])[t0:t0 + T].tobytes()
        # every routing output of the self-routing launch (E = 128: eight logits per lane)
        # against the routing tail's for the same rows
        _, _, _, bt = run(rows, fused=False)
        for n in ("counts", "offsets", "perm", "inv", "prob_mass", "h", "y"):
            assert host(b1[n]).tobytes() == host(bt[n]).tobytes(), (t0, T, n)
    out, idx, _, _ = run(pool[::-1])
    assert out.tobytes() == ref_out[::-1].tobytes()
    for tm in (16, 32, 64, 128, 256):
        out, _, _, _ = run(pool, tile_m=tm)
        assert out.tobytes() == ref_out.tobytes(), tm
    # prefill-shaped: the 64 pool rows scattered through 4096 other tokens
    rng = np.random.default_rng(5)
    big = W.make_layer(T=4096, d=L.d, E=L.E, k=L.k, I=L.I, dtype="bf16", mode="router",
                       seed=55, weights=False).x
    pos = np.sort(rng.choice(4096, 64, replace=False))
    big[pos] = pool
    out, idx, _, bb = run(big)
    assert out[pos].tobytes() == ref_out.tobytes()
    assert idx[pos].tobytes() == ref_idx.tobytes()
    # the 4096-token launch groups several expert tiles per logits block; same bits
    assert host(bb["logits"])[pos].tobytes() == host(b64["logits"]).tobytes()
    # and the decode rows agree with the oracle
    toks = np.array([0, 1, 31, 63])
    rh, ry, rout = oracle.forward_tokens(L, toks, ref_idx, ref_w)
    assert_close(as_f32(ref_out[toks], "bf16"), as_f32(rout, "bf16"), "bf16", "c5 out")
    g_lg = host(b64["logits"])
    idx_o, _, _, _ = oracle.route_from_logits(g_lg, L.k)
    np.testing.assert_array_equal(ref_idx, idx_o)
