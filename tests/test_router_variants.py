"""Pins of the oracle's router variants and objective statistics.

Sources: "0 train-infer mismatch for Open-weight MoE RL in Open-source code", "Choosing
GLM's eight experts" (sigmoid scores, a selection-only FP32 correction bias, pre-bias
scores normalised in FP32, the factor 2.5 applied by the expert kernel) and "Hash and
learned expert routing" (frozen token-id table, sqrt-softplus scores); "HARTS ...",
eq. (20) and "MoE execution and objectives" (multiplicity-weighted z-loss, load-balancing
mass and counts, expert-bias update).

Nothing here re-types the oracle's formulas: scores are checked against other closed
forms of the same functions (tanh, logaddexp), selection against a pairwise-rank
definition and against the softmax router, weights against the golden file, the
objectives against the expanded batch that the multiplicities stand for and against
hand-worked values.
"""
import json
import math
import os

import numpy as np
import pytest

import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24


def ulp_diff(a, b):
    a = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


# ---------------------------------------------------------------------------- golden

def test_golden_route_variants(orc):
    spec = json.load(open(os.path.join(GOLD, "route_variants_small.json")))
    for c in spec["cases"]:
        lg = np.array([c["logits"]], dtype=np.float32)
        kw = {}
        if c.get("corr_bias") is not None:
            kw["corr_bias"] = np.array(c["corr_bias"], dtype=np.float32)
        if "hash_table" in c:
            kw["hash_table"] = np.array(c["hash_table"], dtype=np.int32)
            kw["token_ids"] = np.array([c["token_id"]], dtype=np.int32)
        r = orc.route_scored(lg, c["k"], c["score"], **kw)
        assert r["err"] == 0, c["why"]
        assert r["idx"][0].tolist() == c["idx"], c["why"]
        if c["exact"]:
            assert r["w"][0].tolist() == [float(np.float32(v)) for v in c["w"]], c["why"]
        else:
            np.testing.assert_allclose(r["w"][0], c["w"], rtol=16 * U, err_msg=c["why"])


# ------------------------------------------------------------------- score functions

def test_sigmoid_scores_match_tanh_form(orc):
    """sigmoid(l) = (1 + tanh(l / 2)) / 2: another closed form, in float64, rounded."""
    rng = np.random.default_rng(0)
    lg = np.concatenate([rng.normal(0, 3, 4000), [0.0, 1e-30, -1e-30, 20.0, -20.0, 88.0,
                                                  -88.0, 200.0, -200.0]]).astype(np.float32)
    lg = lg.reshape(-1, 1)
    r = orc.route_scored(lg, 1, "sigmoid")
    l64 = lg.astype(np.float64)
    # the tanh form cancels for very negative l; there e^l / (1 + e^l) is exact enough
    ref = np.where(l64 > -4.0, (1.0 + np.tanh(l64 / 2.0)) / 2.0,
                   np.exp(l64) / (1.0 + np.exp(l64))).astype(np.float32)
    assert ulp_diff(r["scores"], ref).max() <= 1
    from scipy.special import expit
    assert ulp_diff(r["scores"], expit(l64).astype(np.float32)).max() <= 1
    assert r["scores"][-9, 0] == 0.5                     # sigmoid(0) = 1/2 exactly
    # symmetry s(l) + s(-l) = 1
    r2 = orc.route_scored(-lg, 1, "sigmoid")
    tot = r["scores"].astype(np.float64) + r2["scores"].astype(np.float64)
    assert np.abs(tot - 1.0).max() <= 2 * U


def test_sqrt_softplus_scores_match_logaddexp(orc):
    """sqrt(softplus(l)) with softplus(l) = logaddexp(0, l), float64, rounded once."""
    rng = np.random.default_rng(1)
    lg = np.concatenate([rng.normal(0, 4, 4000), [0.0, 50.0, -50.0, 100.0, -100.0, 1e-3]])
    lg = lg.astype(np.float32).reshape(-1, 1)
    r = orc.route_scored(lg, 1, "sqrt_softplus")
    ref = np.sqrt(np.logaddexp(0.0, lg.astype(np.float64))).astype(np.float32)
    assert ulp_diff(r["scores"], ref).max() <= 1
    assert r["scores"][-6, 0] == np.float32(math.sqrt(math.log(2.0)))
    assert r["scores"][-3, 0] == np.float32(10.0)        # softplus(100) = 100 + 4e-44


# ------------------------------------------------------------------------- selection

def _pairwise_select(key, k):
    """Expert e takes slot #{e' ranking before e}, where e' ranks before e when its key is
    larger, or equal with a lower id: a definition that never sorts."""
    E = len(key)
    rank = [sum(1 for f in range(E) if key[f] > key[e] or (key[f] == key[e] and f < e))
            for e in range(E)]
    out = [None] * k
    for e, r in enumerate(rank):
        if r < k:
            out[r] = e
    return out


@pytest.mark.parametrize("score", ["sigmoid", "sqrt_softplus"])
def test_selection_with_bias_brute_force(orc, score):
    rng = np.random.default_rng(2)
    for trial in range(300):
        E = int(rng.integers(1, 13))
        k = int(rng.integers(1, min(E, 8) + 1))
        # coarse values make ties in the keys common
        lg = (rng.integers(-3, 4, size=(1, E)) * 0.5).astype(np.float32)
        b = (rng.integers(-2, 3, size=E) * 0.125).astype(np.float32)
        r = orc.route_scored(lg, k, score, corr_bias=b)
        key = (r["scores"][0] + b).astype(np.float32)      # FP32 key of each expert
        assert r["idx"][0].tolist() == _pairwise_select(key.tolist(), k), (trial, lg, b)
        # weights: the chosen pre-bias scores over their left-to-right sum
        v = r["scores"][0][r["idx"][0]].astype(np.float64)
        np.testing.assert_allclose(r["w"][0], v / v.sum(), rtol=(k + 2) * U)


def test_zero_bias_selects_like_softmax(orc):
    """Sigmoid and sqrt-softplus are increasing, so without a bias they choose the same
    experts in the same order as the softmax router (no ties in these logits)."""
    rng = np.random.default_rng(3)
    lg = rng.normal(0, 1, size=(500, 64)).astype(np.float32)
    idx_soft, _, _, _ = orc.route_from_logits(lg, 8)
    for score in ("sigmoid", "sqrt_softplus"):
        r = orc.route_scored(lg, 8, score)
        np.testing.assert_array_equal(r["idx"], idx_soft)
    r = orc.route_scored(lg, 8, "softmax")
    idx_s, w_s, m_s, _ = orc.route_from_logits(lg, 8)
    np.testing.assert_array_equal(r["idx"], idx_s)
    assert r["w"].tobytes() == w_s.tobytes()


def test_bias_only_chooses(orc):
    """A large bias forces an expert into every row, in slot 0, while its weight stays its
    pre-bias share."""
    rng = np.random.default_rng(4)
    lg = rng.normal(0, 1, size=(200, 16)).astype(np.float32)
    b = np.zeros(16, dtype=np.float32)
    b[5] = 10.0
    r = orc.route_scored(lg, 4, "sigmoid", corr_bias=b)
    assert (r["idx"][:, 0] == 5).all()
    s = r["scores"]
    np.testing.assert_allclose(r["w"][:, 0], s[:, 5] / s[np.arange(200)[:, None], r["idx"]]
                               .astype(np.float64).sum(1), rtol=8 * U)
    assert np.abs(r["w"].astype(np.float64).sum(1) - 1.0).max() <= 8 * U


def test_softmax_with_bias_rejected(orc):
    with pytest.raises(ValueError):
        orc.route_scored(np.zeros((1, 4), np.float32), 2, "softmax",
                         corr_bias=np.zeros(4, np.float32))


# ----------------------------------------------------------------------- hash routing

def test_hash_routing(orc):
    rng = np.random.default_rng(5)
    V, E, k, T = 300, 32, 6, 400
    tab = W.hash_table(V, E, k, 9)
    tok = W.token_ids(T, V, 9)
    lg = rng.normal(0, 1, size=(T, E)).astype(np.float32)
    for score in ("sigmoid", "sqrt_softplus", "softmax"):
        r = orc.route_scored(lg, k, score, hash_table=tab, token_ids=tok)
        assert r["err"] == 0
        np.testing.assert_array_equal(r["idx"], tab[tok])          # the table decides
        v = np.take_along_axis(r["scores"], r["idx"], 1).astype(np.float64)
        np.testing.assert_allclose(r["w"], v / v.sum(1, keepdims=True), rtol=(k + 2) * U)
    # a correction bias does not move a hash row
    r2 = orc.route_scored(lg, k, "sigmoid", corr_bias=np.full(E, 3.0, np.float32),
                          hash_table=tab, token_ids=tok)
    np.testing.assert_array_equal(r2["idx"], tab[tok])


def test_hash_routing_errors(orc):
    E, k = 8, 2
    tab = np.array([[0, 1], [2, 9], [3, 3]], dtype=np.int32)
    lg = np.zeros((4, E), np.float32)
    r = orc.route_scored(lg, k, "sigmoid", hash_table=tab,
                         token_ids=np.array([0, 3, -1, 0], np.int32))
    assert r["err"] == orc.ERR_IDX_RANGE
    assert r["idx"][1].tolist() == [-1, -1] and r["idx"][2].tolist() == [-1, -1]
    assert (r["w"][1:3] == 0).all() and r["idx"][0].tolist() == [0, 1]
    r = orc.route_scored(lg[:1], k, "sigmoid", hash_table=tab, token_ids=np.array([1], np.int32))
    assert r["err"] == orc.ERR_IDX_RANGE and (r["w"] == 0).all()
    r = orc.route_scored(lg[:1], k, "sigmoid", hash_table=tab, token_ids=np.array([2], np.int32))
    assert r["err"] == orc.ERR_IDX_DUP and (r["w"] == 0).all()


# -------------------------------------------------------------- log-sum-exp and mass

def test_lse_closed_forms(orc):
    E = 64
    for c in (0.0, -3.5, 7.25):
        r = orc.route_scored(np.full((1, E), c, np.float32), 2, "sigmoid")
        assert abs(float(r["lse"][0]) - (c + math.log(E))) <= 4 * U * (abs(c) + math.log(E))
    rng = np.random.default_rng(6)
    lg = rng.normal(0, 2, size=(300, 100)).astype(np.float32)
    r = orc.route_scored(lg, 4, "sqrt_softplus")
    ref = np.logaddexp.reduce(lg.astype(np.float64), axis=1)
    assert (np.abs(r["lse"] - ref) <= 64 * U * (np.abs(ref) + 1)).all()


@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sqrt_softplus"])
def test_mass_sums_to_weighted_tokens(orc, score):
    """Each token's routing probabilities sum to 1, so the mass sums to sum_t q_t."""
    rng = np.random.default_rng(7)
    T, E = 700, 48
    lg = rng.normal(0, 1, size=(T, E)).astype(np.float32)
    q = W.token_multiplicities(T, 3)
    r = orc.route_scored(lg, 6, score, token_mult=q)
    assert abs(float(r["prob_mass"].astype(np.float64).sum()) - q.sum()) <= 1e-4 * q.sum()
    r2 = orc.route_scored(lg, 6, score, token_mult=2 * q)     # q doubles -> mass doubles
    assert (r2["prob_mass"] == 2 * r["prob_mass"]).all()


# --------------------------------------------------------------------------- objectives

def test_objectives_balanced_and_hand_worked(orc):
    # balanced: C_e = kS/E, M_e = S/E  ->  aux = 1 exactly
    z, aux, S, _ = orc.objectives(None, np.full(8, 1, np.int32), np.full(4, 4, np.int64),
                                  np.full(4, 2.0, np.float32), k=2)
    assert (aux, S, z) == (1.0, 8, 0.0)
    # everything on experts 0 and 1 (k = 2, E = 4, S = 3): C = (3, 3, 0, 0),
    # M = (2, 1, 0, 0): aux = 4 / (2 * 9) * (6 + 3) = 2
    z, aux, S, _ = orc.objectives(np.array([1.0, -2.0, 0.5], np.float32), None,
                                  np.array([3, 3, 0, 0], np.int64),
                                  np.array([2.0, 1.0, 0.0, 0.0], np.float32), k=2)
    assert aux == 2.0 and S == 3
    assert z == pytest.approx((1.0 + 4.0 + 0.25) / 3.0, rel=1e-15)
    # q weights the z-loss terms: q = (2, 1): (2 * 1 + 4) / 3
    z, _, S, _ = orc.objectives(np.array([1.0, -2.0], np.float32), np.array([2, 1], np.int32),
                                None, None, k=2)
    assert S == 3 and z == pytest.approx(2.0, rel=1e-15)


def test_bias_update_sign_rule(orc):
    C = np.array([10, 2, 6, 6], np.int64)                 # mean 6
    b = np.array([0.5, -0.25, 0.0, 1.0], np.float32)
    _, _, _, nb = orc.objectives(None, None, C, None, k=2, rate=0.125, corr_bias=b)
    assert nb.tolist() == [0.375, -0.125, 0.0, 1.0]
    # a mean that is not an integer: C = (1, 2), mean 1.5
    _, _, _, nb = orc.objectives(None, None, np.array([1, 2], np.int64), None, k=1, rate=1.0,
                                 corr_bias=np.zeros(2, np.float32))
    assert nb.tolist() == [1.0, -1.0]


@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sqrt_softplus"])
def test_multiplicity_equals_expanded_batch(orc, score):
    """HARTS eq. (20): a compact row with multiplicity q stands for q identical semantic
    rows. Routing the expanded batch with q = 1 gives the same ids and weights per row, the
    same weighted counts, and (up to FP32 summation order) the same mass, z-loss and
    load-balancing loss as the compact batch with q."""
    rng = np.random.default_rng(8)
    T, E, k = 120, 32, 4
    lg = rng.normal(0, 1.5, size=(T, E)).astype(np.float32)
    q = W.token_multiplicities(T, 11)
    b = W.correction_bias(E, 11) if score != "softmax" else None
    rc = orc.route_scored(lg, k, score, corr_bias=b, token_mult=q)
    rows = np.repeat(np.arange(T), q)
    re = orc.route_scored(lg[rows], k, score, corr_bias=b)
    np.testing.assert_array_equal(re["idx"], rc["idx"][rows])
    assert re["w"].tobytes() == rc["w"][rows].tobytes()
    wc_c, _ = orc.weighted_counts(rc["idx"], E, q)
    wc_e, _ = orc.weighted_counts(re["idx"], E, None)
    np.testing.assert_array_equal(wc_c, wc_e)
    np.testing.assert_allclose(rc["prob_mass"], re["prob_mass"], rtol=2e-5, atol=1e-5)
    oc = orc.objectives(rc["lse"], q, wc_c, rc["prob_mass"], k)
    oe = orc.objectives(re["lse"], None, wc_e, re["prob_mass"], k)
    assert oc[2] == oe[2] == int(q.sum())
    assert oc[0] == pytest.approx(oe[0], rel=1e-12)      # same terms, FP64 sums
    assert oc[1] == pytest.approx(oe[1], rel=2e-5)


# ----------------------------------------------------------------- routed scale

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_routed_scale_combine(orc, dtype):
    rng = np.random.default_rng(9)
    T, k, d = 50, 4, 96
    y = rng.normal(0, 1, size=(T * k, d)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    base = orc.combine(y, inv, w, dtype)
    assert orc.combine(y, inv, w, dtype, 1.0).tobytes() == base.tobytes()
    # a power of two commutes with rounding (no overflow or underflow here)
    two = W.to_f32(orc.combine(y, inv, w, dtype, 2.0), dtype)
    assert (two == 2.0 * W.to_f32(base, dtype)).all()
    # 2.5: within one rounding of the float64 value of 2.5 * the FP32 slot sum
    got = W.to_f32(orc.combine(y, inv, w, dtype, 2.5), dtype).astype(np.float64)
    acc = np.zeros((T, d), np.float32)
    for j in range(k):
        acc = (acc + (w[:, j:j + 1] * y[inv.reshape(T, k)[:, j]]).astype(np.float32)
               ).astype(np.float32)
    ref = 2.5 * acc.astype(np.float64)
    tol = (2.0 ** -8 if dtype == "bf16" else U) * np.abs(ref) * 1.01 + 1e-30
    assert (np.abs(got - ref) <= tol).all()
