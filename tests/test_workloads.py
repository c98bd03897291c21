"""Structural claims of the seeded workload generators."""
import numpy as np
import pytest

import workloads as W


def test_determinism_and_chunk_independence():
    a = W.make_layer(T=300, d=64, E=8, k=2, I=64, dtype="bf16", mode="router", seed=3)
    b = W.make_layer(T=300, d=64, E=8, k=2, I=64, dtype="bf16", mode="router", seed=3)
    for n in ("x", "w13", "w2", "w_router"):
        np.testing.assert_array_equal(getattr(a, n), getattr(b, n))
    c = W.make_layer(T=300, d=64, E=8, k=2, I=64, dtype="bf16", mode="router", seed=4)
    assert not np.array_equal(a.x, c.x)


def test_weight_scale():
    L = W.make_layer(T=64, d=1024, E=4, k=2, I=256, dtype="f32", mode="router", seed=1)
    for w in (L.w13, L.w2, L.w_router):
        assert abs(w.std() * np.sqrt(1024) - 1) < 0.02
    assert abs(L.x.std() - 1) < 0.05


def test_c2_zipf_bias():
    b = W.zipf_log_bias(64, 2)
    ranks = np.round(np.exp(-b.astype(np.float64) / 1.1)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, 65))
    assert b.max() == 0.0


def test_c3_packed_lengths():
    cu = W.packed_lengths(16384, 3)
    lens = np.diff(cu)
    assert cu[0] == 0 and cu[-1] == 16384
    assert lens.min() >= 1 and lens.max() <= 8192
    assert 3 <= len(lens) <= 40


def test_c3_replay_rows():
    L = W.make_config("c3", weights=False)
    idx, w = L.idx_in, L.w_in
    assert idx.shape == (16384, 8) and w.shape == (16384, 8)
    assert idx.min() >= 0 and idx.max() < 128
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1])  # distinct
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1) < 1e-5)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert L.cu_seqlens[-1] == 16384


def test_c4_exact_counts():
    """One hot expert in every row (T), 15 experts sharing 4T, 224 sharing 3T, 16 empty."""
    L = W.make_config("c4", weights=False)
    T = L.T
    counts = np.bincount(L.idx_in.reshape(-1), minlength=256)
    meta = L.meta["hot"]
    assert counts[meta["hot"]] == T
    assert counts[meta["group"]].sum() == 4 * T
    assert counts[meta["tail"]].sum() == 3 * T
    assert np.all(counts[meta["zero"]] == 0)
    assert (counts == 0).sum() == 16
    assert np.all(np.sort(L.idx_in, axis=1)[:, 1:] != np.sort(L.idx_in, axis=1)[:, :-1])


def test_c5_pool_prefix():
    a = W.make_config("c5", T=7, weights=False)
    b = W.make_config("c5", weights=False)
    np.testing.assert_array_equal(a.x, b.x[:7])


def test_router_variant_inputs():
    """Correction bias, frozen hash table and token ids: seeded, in range, the table's rows
    k distinct experts, the token ids skewed (frequent ids repeat)."""
    b1, b2 = W.correction_bias(64, 3), W.correction_bias(64, 3)
    assert b1.dtype == np.float32 and (b1 == b2).all() and 0.02 < b1.std() < 0.08
    tab = W.hash_table(5000, 64, 8, 3)
    assert tab.shape == (5000, 8) and tab.dtype == np.int32
    assert (tab >= 0).all() and (tab < 64).all()
    assert all(len(set(r)) == 8 for r in tab.tolist())
    assert (tab == W.hash_table(5000, 64, 8, 3)).all()
    tok = W.token_ids(20000, 5000, 3)
    assert tok.dtype == np.int32 and (tok >= 0).all() and (tok < 5000).all()
    _, cnt = np.unique(tok, return_counts=True)
    assert cnt.max() > 20 * 20000 / 5000                 # Zipf: a few ids dominate
    L = W.make_layer(T=50, d=64, E=16, k=4, I=64, mode="router", seed=2)
    W.set_router(L, "sqrt_softplus", bias=True, hash_vocab=300, routed_scale=2.5)
    assert L.score == "sqrt_softplus" and L.routed_scale == 2.5
    assert L.hash_table.shape == (300, 4) and L.token_ids.shape == (50,)
    with pytest.raises(ValueError):
        W.set_router(L, "tanh")


def test_ep_share_counts():
    """Rank 0's rows under 8 x 8 expert parallelism: 16 experts, about T*k rows in all
    (each of 8 batches sends 1/8 of its T*k assignments on average), reproducible."""
    c = W.ep_share_counts("c3", 8)
    assert c.shape == (16,) and c.dtype == np.int64
    T, k = W.CONFIGS["c3"]["T"], W.CONFIGS["c3"]["k"]
    assert abs(int(c.sum()) - T * k) < 0.1 * T * k
    assert (c == W.ep_share_counts("c3", 8)).all()
