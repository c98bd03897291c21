"""Structural claims of the seeded workload generators."""
import numpy as np

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
