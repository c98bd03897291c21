"""Small batches (T <= 64): moe_forward runs the routing tail (top-k or replay check,
probability mass, counts, offsets, stable permutation, weighted counts, tile list) in one
block. Every output must be bitwise what the separate entry points (multi-kernel routing
and permutation) give on the same inputs, and the oracle must agree with both."""
import numpy as np
import pytest
import torch

import moe_layer_routing_amd as M
import oracle
import workloads as W
from gpu_util import as_f32, assert_close, dev, dims_of, host, run_forward, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    M.lib()
    oracle.lib()


def _steps(L, inp, mult=True):
    """The layer through moe_route / moe_route_replay, moe_permute, moe_grouped_ffn and
    moe_combine (multi-kernel routing and permutation at every T)."""
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=(L.mode == "router"), weighted=True)
    ws = M.alloc_workspace(dims)
    q = inp["token_mult"] if mult else None
    if L.mode == "router":
        M.route(dims, inp["x"], inp["w_router"], inp["logit_bias"], b["topk_idx"], b["topk_w"],
                logits=b["logits"], prob_mass=b["prob_mass"], token_mult=q, d_err=b["d_err"],
                workspace=ws)
    else:
        M.route_replay(dims, inp["idx_in"], inp["w_in"], b["topk_idx"], b["topk_w"],
                       d_err=b["d_err"])
    M.permute(dims, b["topk_idx"], inp["x"], b["x_perm"], b["perm"], b["inv"], b["counts"],
              b["offsets"], token_mult=q, weighted_counts=b["weighted_counts"],
              d_err=b["d_err"], workspace=ws)
    M.grouped_ffn(dims, b["x_perm"], b["offsets"], inp["w13"], inp["w2"], b["h"], b["y"],
                  workspace=ws)
    M.combine(dims, b["y"], b["inv"], b["topk_w"], b["out"])
    torch.cuda.synchronize()
    return b


def _fused(L, inp, mult=True):
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=(L.mode == "router"), weighted=True)
    for n in ("x", "w13", "w2"):
        b[n] = inp[n]
    if L.mode == "router":
        b["w_router"], b["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        b["idx_in"], b["w_in"] = inp["idx_in"], inp["w_in"]
    if mult:
        b["token_mult"] = inp["token_mult"]
    M.forward(dims, b, M.alloc_workspace(dims))
    torch.cuda.synchronize()
    return b


OUTS = ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "weighted_counts", "x_perm",
        "h", "y", "out", "d_err")

CASES = [
    dict(T=1, E=16, k=4, mode="router"),
    dict(T=3, E=8, k=8, mode="router"),
    dict(T=16, E=64, k=8, mode="router"),
    dict(T=17, E=64, k=8, mode="router"),     # two 16-token groups in the mass sum
    dict(T=33, E=128, k=6, mode="router"),    # three
    dict(T=48, E=40, k=2, mode="router"),
    dict(T=64, E=256, k=8, mode="router"),    # 512 assignments, 8 ranking waves
    dict(T=64, E=128, k=1, mode="router"),
    dict(T=1, E=1, k=1, mode="router"),
    dict(T=5, E=32, k=8, mode="replay"),
    dict(T=64, E=256, k=8, mode="replay"),
    dict(T=40, E=200, k=3, mode="replay"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c['T']}_E{c['E']}_k{c['k']}_{c['mode']}")
@pytest.mark.parametrize("mult", [True, False], ids=["q", "noq"])
def test_small_tail_matches_steps(case, mult):
    L = W.make_layer(T=case["T"], d=128, E=case["E"], k=case["k"], I=128, dtype="bf16",
                     mode=case["mode"], seed=60 + case["T"] + case["E"], bias="zipf",
                     replay="dirichlet")
    L.token_mult = W.token_multiplicities(L.T, 3)
    inp = upload(L)
    ref = _steps(L, inp, mult)
    got = _fused(L, inp, mult)
    assert int(got["d_err"].item()) == 0
    names = OUTS + (("logits", "prob_mass") if L.mode == "router" else ())
    for n in names:
        assert host(got[n]).tobytes() == host(ref[n]).tobytes(), n
    # and the oracle agrees (on the GPU's logits)
    logits = host(got["logits"]) if L.mode == "router" else None
    r = oracle.forward(L, logits=logits) if mult else None
    if r is not None:
        np.testing.assert_array_equal(host(got["topk_idx"]), r["idx"])
        for n in ("counts", "offsets", "perm", "inv", "weighted_counts"):
            np.testing.assert_array_equal(host(got[n]), r[n], err_msg=n)
        if L.mode == "router":
            assert_close(host(got["prob_mass"]), r["prob_mass"], "bf16", "prob_mass")
        assert_close(as_f32(host(got["out"]), "bf16"), as_f32(r["out"], "bf16"), "bf16", "out")


def test_small_tail_bad_replay_ids():
    """Out-of-range replay ids: the same error bits, counts and inv (-1) as the steps."""
    L = W.make_layer(T=20, d=64, E=16, k=4, I=64, dtype="bf16", mode="replay", seed=77,
                     replay="uniform")
    L.idx_in = L.idx_in.copy()
    L.idx_in[3, 1] = 16
    L.idx_in[11, 0] = -2
    inp = upload(L)
    ref = _steps(L, inp)
    got = _fused(L, inp)
    assert int(got["d_err"].item()) == int(ref["d_err"].item())
    assert int(got["d_err"].item()) & M.DERR_IDX_RANGE
    for n in ("counts", "offsets", "inv", "weighted_counts"):
        assert host(got[n]).tobytes() == host(ref[n]).tobytes(), n
    nvalid = int(host(ref["offsets"])[-1])
    assert nvalid == L.T * L.k - 2
    assert host(got["perm"])[:nvalid].tobytes() == host(ref["perm"])[:nvalid].tobytes()


def test_small_and_large_paths_agree_per_row():
    """T = 64 (single-block tail) and T = 65 (multi-kernel path): the first 64 rows'
    routing and output bytes are the same."""
    L = W.make_layer(T=65, d=256, E=32, k=4, I=128, dtype="bf16", mode="router", seed=90,
                     bias="zipf")
    inp = upload(L)
    big, _ = run_forward(L, inp, stats=False)
    L64 = W.make_layer(T=64, d=256, E=32, k=4, I=128, dtype="bf16", mode="router", seed=90,
                       bias="zipf", weights=False)
    L64.w13, L64.w2, L64.w_router, L64.logit_bias = L.w13, L.w2, L.w_router, L.logit_bias
    L64.x = np.ascontiguousarray(L.x[:64])
    inp64 = dict(inp)
    inp64["x"] = dev(L64.x)
    small, _ = run_forward(L64, inp64, stats=False)
    for n in ("logits", "topk_idx", "topk_w", "out"):
        assert host(small[n]).tobytes() == host(big[n])[:64].tobytes(), n


DC_CASES = [
    dict(T=1, E=16, k=8, I=768, mode="router", scale=None),
    dict(T=2, E=16, k=8, I=768, mode="router", scale=None),
    dict(T=1, E=12, k=3, I=1536, mode="router", scale=2.5),
    dict(T=5, E=16, k=3, I=768, mode="replay", scale=None),
    dict(T=16, E=16, k=1, I=768, mode="replay", scale=0.75),
]


@pytest.mark.parametrize("case", DC_CASES,
                         ids=lambda c: f"T{c['T']}_E{c['E']}_k{c['k']}_I{c['I']}_{c['mode']}")
def test_decode_down_combine_launch_matches_steps(case):
    """At most 16 expert rows, d/16 >= 256 feature blocks and inter a multiple of 768:
    moe_forward runs the down GEMM and the combine as one launch. Its y and output rows
    (and every other output) are bitwise those of moe_grouped_ffn + moe_combine(_scaled)
    after the separate routing and permutation steps; the routed scaling factor too."""
    L = W.make_layer(T=case["T"], d=4096, E=case["E"], k=case["k"], I=case["I"],
                     dtype="bf16", mode=case["mode"], seed=70 + case["T"] + case["k"],
                     bias="zipf", replay="dirichlet")
    inp = upload(L)
    dims = dims_of(L)
    ref = _steps(L, inp, mult=False)
    if case["scale"] is not None:
        M.combine(dims, ref["y"], ref["inv"], ref["topk_w"], ref["out"],
                  routed_scale=case["scale"])
    b = M.alloc_forward_buffers(dims, "cuda", router=(L.mode == "router"), weighted=True)
    for n in ("x", "w13", "w2"):
        b[n] = inp[n]
    if L.mode == "router":
        b["w_router"], b["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        b["idx_in"], b["w_in"] = inp["idx_in"], inp["w_in"]
    M.forward(dims, b, M.alloc_workspace(dims), routed_scale=case["scale"] or 0.0)
    torch.cuda.synchronize()
    assert int(b["d_err"].item()) == 0
    for n in ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "h", "y", "out"):
        assert host(b[n]).tobytes() == host(ref[n]).tobytes(), n


SR_CASES = [
    dict(T=1, E=16, k=8, I=768, mult=True, scale=None, lse=True),
    dict(T=1, E=12, k=3, I=1536, mult=False, scale=2.5, lse=False),
    dict(T=1, E=8, k=8, I=768, mult=True, scale=None, lse=False),     # every expert selected
    dict(T=1, E=33, k=1, I=768, mult=True, scale=0.5, lse=True),
    dict(T=2, E=16, k=8, I=768, mult=True, scale=None, lse=True),     # 16 rows
    dict(T=2, E=12, k=3, I=1536, mult=True, scale=2.5, lse=False),
    dict(T=2, E=8, k=8, I=768, mult=False, scale=None, lse=True),     # 8 tiles of 2 rows
    dict(T=2, E=33, k=1, I=768, mult=True, scale=0.5, lse=False),
    dict(T=2, E=16, k=8, I=768, mult=True, scale=None, lse=False, dup=True),  # same token twice
    # 8 logits per lane with a partly empty last group; short K (2 or 4 ring stages, 4 or 8
    # of the 16 logit chains empty)
    dict(T=1, E=100, k=6, I=128, d=128, mult=True, scale=None, lse=True),
    dict(T=2, E=100, k=8, I=256, d=128, mult=True, scale=2.5, lse=False),
    dict(T=2, E=65, k=2, I=128, d=256, mult=False, scale=None, lse=True),
]
SR_OUTS = ("logits", "topk_idx", "topk_w", "prob_mass", "counts", "offsets", "perm", "inv",
           "weighted_counts", "gu", "h", "y", "out", "d_err")


def _decode_one(L, inp, fused, mult, scale, lse):
    """One-token moe_forward; fused: no x_perm (the gate/up launch gathers, and with the
    plain softmax router routes the token itself), else the routing tail + gather path."""
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=True, weighted=True)
    for n in ("x", "w13", "w2", "w_router", "logit_bias"):
        b[n] = inp[n]
    if mult:
        b["token_mult"] = inp["token_mult"]
    if fused:
        del b["x_perm"]
    # the saved pre-activations: one FP32 row of 2 I values per assignment (T k rows)
    b["gu"] = torch.empty((L.T * L.k, 2 * L.I), dtype=torch.float32, device="cuda")
    assert b["gu"].shape[0] == b["h"].shape[0]
    lse_t = torch.full((L.T,), 7.0, dtype=torch.float32, device="cuda") if lse else None
    M.forward(dims, b, M.alloc_workspace(dims), routed_scale=scale or 0.0,
              router=dict(score="softmax", lse=lse_t) if lse else None)
    torch.cuda.synchronize()
    return b, lse_t


@pytest.mark.parametrize("case", SR_CASES,
                         ids=lambda c: (f"T{c['T']}_E{c['E']}_k{c['k']}_I{c['I']}_q{int(c['mult'])}"
                                        + (f"_d{c['d']}" if "d" in c else "")
                                        + ("_dup" if c.get("dup") else "")))
def test_decode_self_route_matches_tail(case):
    """One or two tokens, plain softmax router, gather fused (the decode step's launch
    shape): the gate/up launch forms the logits from the chain partials and selects the
    experts in every block. Every output is bitwise the routing-tail path's (tail launch,
    gather, gate/up from x_perm), the routing outputs the multi-kernel steps', and the
    oracle agrees on the GPU logits."""
    L = W.make_layer(T=case["T"], d=case.get("d", 4096), E=case["E"], k=case["k"], I=case["I"],
                     dtype="bf16", mode="router", seed=90 + case["E"] + case["k"] + case["T"],
                     bias="zipf")
    if case.get("dup"):
        L.x = np.ascontiguousarray(np.repeat(L.x[:1], L.T, axis=0))
    L.token_mult = np.array([3, 5][:L.T], dtype=np.int32)
    inp = upload(L)
    args = (case["mult"], case["scale"], case["lse"])
    ref, lse_r = _decode_one(L, inp, False, *args)
    got, lse_g = _decode_one(L, inp, True, *args)
    assert int(got["d_err"].item()) == 0
    for n in SR_OUTS:
        assert host(got[n]).tobytes() == host(ref[n]).tobytes(), n
    if case["lse"]:
        assert host(lse_g).tobytes() == host(lse_r).tobytes()
    steps = _steps(L, inp, case["mult"])
    for n in ("logits", "topk_idx", "topk_w", "prob_mass", "counts", "offsets", "perm", "inv",
              "weighted_counts", "h", "y"):
        assert host(got[n]).tobytes() == host(steps[n]).tobytes(), n
    lg = host(got["logits"])
    q = L.token_mult if case["mult"] else None
    idx_o, w_o, mass_o, err_o = oracle.route_from_logits(lg, L.k, q)
    assert err_o == 0
    np.testing.assert_array_equal(host(got["topk_idx"]), idx_o)
    assert_close(host(got["topk_w"]), w_o, "f32", "topk_w")
    assert_close(host(got["prob_mass"]), mass_o, "f32", "prob_mass")
    L.routed_scale = case["scale"] or 1.0
    _, _, rout = oracle.forward_tokens(L, list(range(L.T)), host(got["topk_idx"]),
                                       host(got["topk_w"]))
    assert_close(as_f32(host(got["out"]), "bf16"), as_f32(rout, "bf16"), "bf16", "out")


def test_decode_self_route_nonfinite_logit():
    """An infinite router logit (a +inf bias) on the one-token path: the same error bit
    and the same (NaN-carrying) outputs as the routing tail."""
    L = W.make_layer(T=1, d=4096, E=16, k=4, I=768, dtype="bf16", mode="router", seed=97,
                     bias="zipf")
    L.logit_bias = L.logit_bias.copy()
    L.logit_bias[5] = np.inf
    inp = upload(L)
    ref, _ = _decode_one(L, inp, False, False, None, False)
    got, _ = _decode_one(L, inp, True, False, None, False)
    assert int(got["d_err"].item()) == int(ref["d_err"].item())
    assert int(got["d_err"].item()) & M.DERR_NONFINITE
    for n in ("topk_idx", "counts", "offsets", "perm", "inv", "weighted_counts"):
        assert host(got[n]).tobytes() == host(ref[n]).tobytes(), n
    assert int(host(got["topk_idx"])[0, 0]) == 5
    for n in ("logits", "topk_w", "prob_mass", "out"):
        np.testing.assert_array_equal(host(got[n]).view(np.uint8), host(ref[n]).view(np.uint8),
                                      err_msg=n)


@pytest.mark.parametrize("T", [1, 2])
def test_decode_self_route_optional_outputs_absent(T):
    """The self-routing launch with logits, probability mass and weighted counts not
    requested (NULL; the logits then go to the workspace): the ids, weights, permutation
    and output rows are bitwise those of the call that requests everything."""
    L = W.make_layer(T=T, d=4096, E=64, k=8, I=768, dtype="bf16", mode="router",
                     seed=120 + T, bias="zipf")
    L.token_mult = np.array([2, 7][:T], dtype=np.int32)
    inp = upload(L)
    full, _ = _decode_one(L, inp, True, True, None, False)
    dims = dims_of(L)
    b = M.alloc_forward_buffers(dims, "cuda", router=True, weighted=False)
    for n in ("x", "w13", "w2", "w_router", "logit_bias", "token_mult"):
        b[n] = inp[n]
    for n in ("x_perm", "logits", "prob_mass"):
        del b[n]
    M.forward(dims, b, M.alloc_workspace(dims))
    torch.cuda.synchronize()
    assert int(b["d_err"].item()) == 0
    for n in ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "h", "y", "out"):
        assert host(b[n]).tobytes() == host(full[n]).tobytes(), n
