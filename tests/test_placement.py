"""Logical -> physical expert placement ("RoutePack ...", Sec. 3, Algorithm 1: layer-local
LPT; Sec. 5: rank-load coefficient of variation). CPU tests: the oracle against a worked
example and closed forms, and the library's host planner (moe_place_lpt, no GPU work)
against the oracle."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "place_lpt_small.json")


@pytest.fixture(scope="module")
def M():
    import moe_layer_routing_amd as M
    if not os.path.exists(M.LIB_PATH):
        from moe_layer_routing_amd import _build
        _build.build()
    M.lib()
    return M


def test_golden_worked_example():
    g = json.load(open(GOLDEN))
    slots, rank_load, cv = oracle.place_lpt(g["loads"], g["P"])
    assert slots.tolist() == g["slot_of_expert"]
    assert rank_load.tolist() == g["rank_load"]
    assert cv == pytest.approx(g["cv"], rel=1e-15)


@pytest.mark.parametrize("E", [1, 5, 16, 64])
def test_one_slot_per_rank_follows_the_load_order(E):
    """H = 1: the k-th expert in (load desc, id asc) order lands on rank k (every rank
    starts empty when its turn comes, and the lowest empty rank wins)."""
    rng = np.random.default_rng(E)
    loads = rng.integers(0, 4, E)                # many ties
    slots, rank_load, _ = oracle.place_lpt(loads, E)
    order = sorted(range(E), key=lambda e: (-loads[e], e))
    assert [int(slots[e]) for e in order] == list(range(E))
    assert rank_load.tolist() == [int(loads[e]) for e in order]


@pytest.mark.parametrize("E", [1, 7, 32])
def test_single_rank_fills_slots_in_load_order(E):
    rng = np.random.default_rng(100 + E)
    loads = rng.integers(0, 1000, E)
    slots, rank_load, cv = oracle.place_lpt(loads, 1)
    order = sorted(range(E), key=lambda e: (-loads[e], e))
    assert [int(slots[e]) for e in order] == list(range(E))
    assert rank_load.tolist() == [int(loads.sum())]
    assert cv == 0.0


@pytest.mark.parametrize("E,P", [(8, 4), (64, 8), (256, 16), (12, 3)])
def test_equal_loads_go_round_robin(E, P):
    """Equal loads: experts in id order, each to the lowest of the least-loaded ranks, so
    expert e sits in slot (e mod P)*H + e div P and every rank carries the same load."""
    H = E // P
    slots, rank_load, cv = oracle.place_lpt(np.full(E, 7), P)
    assert slots.tolist() == [(e % P) * H + e // P for e in range(E)]
    assert set(rank_load.tolist()) == {7 * H}
    assert cv == 0.0


def test_properties_random():
    rng = np.random.default_rng(7)
    for _ in range(200):
        P = int(rng.choice([1, 2, 4, 8]))
        E = P * int(rng.integers(1, 9))
        loads = rng.integers(0, 50, E) * rng.integers(0, 2, E)
        slots, rank_load, cv = oracle.place_lpt(loads, P)
        H = E // P
        assert sorted(slots.tolist()) == list(range(E))          # a permutation of slots
        for p in range(P):                                        # loads add up per rank
            assert rank_load[p] == sum(int(loads[e]) for e in range(E) if slots[e] // H == p)
        m = rank_load.mean()
        ref = (np.sqrt(((rank_load - m) ** 2).mean()) / m) if m > 0 else 0.0
        assert cv == pytest.approx(ref, rel=1e-12, abs=1e-15)


def test_library_planner_matches_oracle(M):
    rng = np.random.default_rng(11)
    for _ in range(300):
        P = int(rng.choice([1, 2, 4, 8, 16]))
        E = P * int(rng.integers(1, max(2, 256 // P) + 1))
        E = min(E, 256 - 256 % P)
        loads = rng.integers(0, 5000, E) * rng.integers(0, 2, E)
        if rng.random() < 0.3:
            loads = rng.integers(0, 3, E)                         # heavy ties
        s_ref, g_ref, cv_ref = oracle.place_lpt(loads, P)
        s, g, cv = M.place_lpt(loads, P)
        assert s.tolist() == s_ref.tolist()
        assert g.tolist() == g_ref.tolist()
        assert cv == pytest.approx(cv_ref, rel=1e-12, abs=1e-15)


def test_library_planner_rejects_bad_arguments(M):
    with pytest.raises(M.MoeError):
        M.place_lpt(np.ones(6, dtype=np.int64), 4)                # E % P != 0
    with pytest.raises(M.MoeError):
        M.place_lpt(np.array([1, -1, 2, 3]), 2)                   # negative load
    with pytest.raises(M.MoeError):
        M.place_lpt(np.ones(512, dtype=np.int64), 2)              # E > 256


def test_place_maps_ids():
    idx = np.array([[0, 3], [2, 5]], dtype=np.int32)
    m = np.array([6, 0, 3, 2, 5, 4, 1, 7], dtype=np.int32)
    assert oracle.place(idx, m).tolist() == [[6, 2], [3, 4]]
    assert oracle.place(np.array([[9, -1]]), m).tolist() == [[9, -1]]
