"""Pins of the oracle's rank-partial outputs, FP64 pairwise tree and sharded shared expert.

Sources: "0 train-infer mismatch for Open-weight MoE RL in Open-source code", "Sharding the
experts" (each rank accumulates every routing slot in FP32 in slot order, other ranks'
slots contributing exact zeros, adds its shard of the shared expert and rounds once to
BF16; the partials are placed in logical rank order and reduced by adding adjacent pairs
in FP64, carrying an odd contributor, rounding once at the end; eight contributors take
three levels, sixteen take four) and the shared-expert passage (fixed-K projections and
SwiGLU, each rank adding its shard before the reduction).

The one-step FP64 -> bf16 rounding is checked against exact rational arithmetic; the tree
shape against values whose sum depends on the order of additions; the partials against
the plain combine and exact-zero properties; the sharded shared expert against the
unsharded FFN.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as W

BF16_MAX = Fraction(2 ** 8 - 1, 2 ** 7) * Fraction(2) ** 127


def _bf16_value(b):
    """Exact value of a bf16 bit pattern (finite)."""
    f = np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def _round_exact(x: Fraction, neg_zero=False):
    """bf16 nearest to x (ties to even mantissa) by search over neighbouring patterns."""
    if x == 0:
        return 0x8000 if neg_zero else 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a >= BF16_MAX + Fraction(2) ** (127 - 8):      # at or past the overflow midpoint
        return sign | 0x7f80
    f32 = np.float32(float(a))
    base = int(np.array([f32], np.float32).view(np.uint32)[0]) >> 16
    best = None
    for c in range(max(0, base - 2), min(0x7f7f, base + 2) + 1):
        dist = abs(_bf16_value(c) - a)
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return sign | best[1]


def test_f64_to_bf16_is_correctly_rounded(orc):
    rng = np.random.default_rng(0)
    xs = list(rng.normal(0, 1, 3000) * 10.0 ** rng.integers(-40, 39, 3000))
    # exact midpoints between neighbouring bf16 values, and points just beside them
    for b in rng.integers(1, 0x7f7f, 500):
        lo, hi = _bf16_value(b), _bf16_value(b + 1)
        mid = (lo + hi) / 2
        for v in (mid, mid + (hi - lo) / 2 ** 40, mid - (hi - lo) / 2 ** 40):
            xs.append(float(v))
            xs.append(-float(v))
    xs += [0.0, -0.0, 1e-45, 2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -134, 2.0 ** -135,
           float(BF16_MAX), float(BF16_MAX) * (1 + 2 ** -9), float(BF16_MAX) * (1 + 2 ** -8),
           3.4e38, 1e300, -1e300, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]
    xs = np.array(xs, dtype=np.float64)
    got = orc.round_f64_bf16(xs)
    for x, g in zip(xs, got):
        want = _round_exact(Fraction(float(x)), neg_zero=math.copysign(1, x) < 0)
        assert int(g) == want, (float(x), hex(int(g)), hex(want))
    assert orc.round_f64_bf16(np.array([np.inf, -np.inf]))[:].tolist() == [0x7f80, 0xff80]
    assert orc.round_f64_bf16(np.array([np.nan]))[0] & 0x7fff > 0x7f80


def _parts_via_shared(orc, vals, dtype="bf16", scale=1.0):
    """Rank partials equal to ``vals`` (bf16-exact numbers): zero routing weights, and the
    shared-expert shard of rank r holding vals[r]."""
    R = len(vals)
    T, k, d, E = 1, 1, 1, R
    y = np.zeros((1, 1), np.float32)
    ys = np.array(vals, np.float32).reshape(R, 1, 1)
    parts, out = orc.combine_ranks(y, np.zeros(1, np.int32), np.zeros((1, 1), np.float32),
                                   np.zeros((1, 1), np.int32), E, R, dtype, y_shared=ys,
                                   scale=scale)
    return parts, out


@pytest.mark.parametrize("vals,want,other", [
    # 4 ranks: (2^100 + 1) + (-2^100 + 1) = 0 in FP64; left to right gives 1
    ([2.0 ** 100, 1.0, -2.0 ** 100, 1.0], 0.0, 1.0),
    # 3 ranks: (2^100 - 2^100) + carried 1 = 1; right to left (pairing the last two
    # first) gives 0
    ([2.0 ** 100, -2.0 ** 100, 1.0], 1.0, ("rtl", 0.0)),
    # 8 ranks, three levels: ((2^100+1)+(1+1)) + ((-2^100+1)+(1+1)) = 0; left to right 3
    ([2.0 ** 100, 1.0, 1.0, 1.0, -2.0 ** 100, 1.0, 1.0, 1.0], 0.0, 3.0),
    # 16 ranks, four levels: 2^100 in slot 0 and -2^100 in slot 8 cancel at the top; the
    # ones beside them are absorbed below; left to right keeps the last seven
    ([2.0 ** 100] + [1.0] * 7 + [-2.0 ** 100] + [1.0] * 7, 0.0, 7.0),
    # 5 ranks: level 1 (2^100 + -2^100) = 0, (1 + 2^-100) = 1, carry -1; then 1, carry -1;
    # then 0
    ([2.0 ** 100, -2.0 ** 100, 1.0, 2.0 ** -100, -1.0], 0.0, None),
])
def test_pairwise_tree_shape(orc, vals, want, other):
    parts, out = _parts_via_shared(orc, vals)
    assert W.to_f32(parts, "bf16").reshape(-1).tolist() == vals
    assert float(W.to_f32(out, "bf16").reshape(-1)[0]) == want
    if other is not None:
        order, value = other if isinstance(other, tuple) else ("ltr", other)
        seq = 0.0
        for v in (vals if order == "ltr" else vals[::-1]):
            seq = seq + v                                   # sequential FP64
        assert seq == value != want


def test_scale_applies_to_routed_slots_only(orc):
    """The routed scaling factor multiplies the routed sum, not the shared-expert shard."""
    parts, out = _parts_via_shared(orc, [1.5, -0.25], scale=2.5)
    assert W.to_f32(parts, "bf16").reshape(-1).tolist() == [1.5, -0.25]
    y = np.full((1, 1), 2.0, np.float32)
    parts, out = orc.combine_ranks(y, np.zeros(1, np.int32), np.full((1, 1), 0.5, np.float32),
                                   np.zeros((1, 1), np.int32), 2, 2, "bf16",
                                   y_shared=np.array([1.0, 4.0], np.float32).reshape(2, 1, 1),
                                   scale=2.5)
    # rank 0: 2.5 * (0.5 * 2) + 1 = 3.5; rank 1: 0 + 4 = 4; total 7.5
    assert W.to_f32(parts, "bf16").reshape(-1).tolist() == [3.5, 4.0]
    assert float(W.to_f32(out, "bf16").reshape(-1)[0]) == 7.5


def test_single_rank_is_the_plain_combine(orc):
    rng = np.random.default_rng(1)
    T, k, d, E = 60, 4, 48, 16
    y = rng.normal(0, 1, (T * k, d)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    idx = np.argsort(rng.random((T, E)), 1)[:, :k].astype(np.int32)
    for dtype in ("bf16", "f32"):
        parts, out = orc.combine_ranks(y, inv, w, idx, E, 1, dtype)
        plain = orc.combine(y, inv, w, dtype)
        assert out.tobytes() == plain.tobytes() == parts[0].tobytes()
        # the routed scaling factor: as the scaled plain combine
        _, out2 = orc.combine_ranks(y, inv, w, idx, E, 1, dtype, scale=2.5)
        assert out2.tobytes() == orc.combine(y, inv, w, dtype, 2.5).tobytes()


def test_partials_own_only_their_slots(orc):
    rng = np.random.default_rng(2)
    T, k, d, E, R = 80, 6, 32, 32, 8
    y = rng.normal(0, 1, (T * k, d)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    idx = np.argsort(rng.random((T, E)), 1)[:, :k].astype(np.int32)
    slot = rng.permutation(E).astype(np.int32)
    parts, out = orc.combine_ranks(y, inv, w, idx, E, R, "bf16", slot_of_expert=slot)
    owner = slot[idx] // (E // R)
    pf = W.to_f32(parts, "bf16")
    for t in range(T):
        for r in range(R):
            if r not in owner[t]:
                assert (pf[r, t] == 0).all()               # exact zeros only
    # tokens whose slots all sit on rank 3 (experts 12..15 with the identity map): that
    # rank's partial and the output are the plain combine's rows
    H = E // R
    idx1 = np.tile(np.arange(3 * H, 4 * H, dtype=np.int32), (T, 1))
    w1 = np.ascontiguousarray(w[:, :H])
    inv1 = np.arange(T * H, dtype=np.int32)
    parts, out = orc.combine_ranks(y, inv1, w1, idx1, E, R, "bf16")
    plain = orc.combine(y, inv1, w1, "bf16")
    assert out.tobytes() == plain.tobytes() == parts[3].tobytes()
    # the rank sum tracks the plain combine within bf16 rounding of each partial
    parts, out = orc.combine_ranks(y, inv, w, idx, E, R, "bf16", slot_of_expert=slot)
    plain = W.to_f32(orc.combine(y, inv, w, "f32"), "f32").astype(np.float64)
    got = W.to_f32(out, "bf16").astype(np.float64)
    assert (np.abs(got - plain) <= (k + 1) * 2.0 ** -8 * (np.abs(plain) + 1)).all()


def test_tree_output_is_the_rounded_exact_sum(orc):
    """With moderate magnitudes every FP64 addition in the tree is exact, so the output is
    the correctly rounded exact sum of the bf16 partials."""
    rng = np.random.default_rng(3)
    T, k, d, E, R = 20, 8, 16, 64, 16
    y = rng.normal(0, 1, (T * k, d)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    idx = np.argsort(rng.random((T, E)), 1)[:, :k].astype(np.int32)
    ys = rng.normal(0, 0.5, (R, T, d)).astype(np.float32)
    parts, out = orc.combine_ranks(y, inv, w, idx, E, R, "bf16", y_shared=ys, scale=2.5)
    for t in range(0, T, 3):
        for o in range(0, d, 5):
            exact = sum(_bf16_value(int(parts[r, t, o])) if parts[r, t, o] & 0x8000 == 0
                        else -_bf16_value(int(parts[r, t, o]) & 0x7fff) for r in range(R))
            assert int(out[t, o]) == _round_exact(exact), (t, o)


def test_sharded_shared_expert(orc):
    """Sharding the shared expert's inter dimension over R ranks: each rank's h features
    are the unsharded FFN's features of that shard, bit for bit (every h_i is its own
    fixed-K dot products); the rank outputs sum to the unsharded output within FP32
    rounding."""
    rng = np.random.default_rng(4)
    T, d, Is, R = 24, 64, 256, 4
    x = W.f32_to_bf16_bits(rng.normal(0, 1, (T, d)).astype(np.float32))
    w13 = W.f32_to_bf16_bits((rng.normal(0, 1, (2 * Is, d)) / 8).astype(np.float32))
    w2 = W.f32_to_bf16_bits((rng.normal(0, 1, (d, Is)) / 16).astype(np.float32))
    S = Is // R
    w13s = np.stack([np.concatenate([w13[r * S:(r + 1) * S], w13[Is + r * S:Is + (r + 1) * S]])
                     for r in range(R)])
    w2s = np.stack([np.ascontiguousarray(w2[:, r * S:(r + 1) * S]) for r in range(R)])
    hs, ys = orc.shared_ffn(x, w13s, w2s, "bf16")
    h, y = orc.expert_ffn(x, np.zeros(T, np.int32), w13[None], w2[None], "bf16")
    assert np.concatenate(list(hs), axis=1).tobytes() == h.tobytes()
    tot = ys.astype(np.float64).sum(0)
    assert np.abs(tot - y).max() <= 1e-4 * (np.abs(y).max() + 1)
