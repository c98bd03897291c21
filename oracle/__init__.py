"""CPU oracle for one MoE layer (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg
may import this package. The product library never loads it; the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C, FP32, sequential sums, built without
fast-math and with floating-point contraction off). This module only builds and loads it
and marshals numpy arrays. Each wrapper names the page passage its C function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
# A test may point the wrapper at another build of the same source (the sanitizer build).
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")

ERR_IDX_RANGE, ERR_IDX_DUP, ERR_NONFINITE, ERR_SEQLENS = 1, 2, 4, 8

_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-shared", "-fPIC", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build()
            L = ctypes.CDLL(_LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_router_logits.argtypes = [P, P, P, I64, I32, I32, I32, P]
        L.orc_router_logits.restype = None
        L.orc_route_from_logits.argtypes = [P, P, I64, I32, I32, P, P, P, P]
        L.orc_route_from_logits.restype = I32
        L.orc_replay_check.argtypes = [P, P, I64, I32, I32]
        L.orc_replay_check.restype = I32
        L.orc_permute.argtypes = [P, I64, I32, I32, P, P, P, P]
        L.orc_permute.restype = I32
        L.orc_seq_counts.argtypes = [P, I64, I32, I32, P, I32, P]
        L.orc_seq_counts.restype = I32
        L.orc_weighted_counts.argtypes = [P, P, I64, I32, I32, P]
        L.orc_weighted_counts.restype = I32
        L.orc_gather.argtypes = [P, P, I64, I32, I32, I32, P]
        L.orc_gather.restype = None
        L.orc_expert_ffn.argtypes = [P, P, I64, I32, I32, P, P, I32, P, P]
        L.orc_expert_ffn.restype = None
        L.orc_combine.argtypes = [P, P, P, I64, I32, I32, I32, P]
        L.orc_combine.restype = None
        L.orc_combine_scaled.argtypes = [P, P, P, I64, I32, I32, I32, ctypes.c_float, P]
        L.orc_combine_scaled.restype = None
        L.orc_route_scored.argtypes = [P, P, I64, I32, I32, I32, P, P, P, I32, P, P, P, P, P]
        L.orc_route_scored.restype = I32
        L.orc_objectives.argtypes = [P, P, I64, P, P, I32, I32, ctypes.c_float, P, P]
        L.orc_objectives.restype = None
        L.orc_backward_experts.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_float, I64,
                                           I32, I32, I32, I32, I32] + [P] * 9
        L.orc_backward_experts.restype = None
        L.orc_backward_experts_r.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_float,
                                             I64, I32, I32, I32, I32, I32, I32] + [P] * 9
        L.orc_backward_experts_r.restype = None
        L.orc_backward_router.argtypes = [P, P, P, P, I64, I32, I32, I32, I32, P, P, P]
        L.orc_backward_router.restype = I32
        L.orc_round_f64_bf16.argtypes = [P, P, I64]
        L.orc_round_f64_bf16.restype = None
        L.orc_combine_ranks.argtypes = [P, P, P, P, P, I64, I32, I32, I32, I32, P,
                                        ctypes.c_float, I32, P, P]
        L.orc_combine_ranks.restype = I32
        L.orc_round_bf16.argtypes = [P, P, I64]
        L.orc_round_bf16.restype = None
        L.orc_place_lpt.argtypes = [P, I32, I32, P, P]
        L.orc_place_lpt.restype = I32
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = I32
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _dt(dtype: str) -> int:
    return 1 if dtype == "bf16" else 0


def _store_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def num_threads() -> int:
    return lib().orc_num_threads()


def round_bf16(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_round_bf16(_p(a), _p(out), a.size)
    return out


def router_logits(x, w_router, bias, dtype: str) -> np.ndarray:
    """Router logits (fixed-K FP32 projection, plus optional bias). "0 train-infer
    mismatch ...", "The router: matching expert ids and weights"."""
    T, d = x.shape
    E = w_router.shape[0]
    x = np.ascontiguousarray(x)
    w_router = np.ascontiguousarray(w_router)
    bias = _c(bias, np.float32)
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(_p(x), _p(w_router), _p(bias), T, d, E, _dt(dtype), _p(out))
    return out


def route_from_logits(logits, k: int, token_mult=None, want_probs: bool = False):
    """FP32 softmax, top-k (logit desc, id asc), left-to-right renormalisation and
    multiplicity-weighted probability mass. Returns (idx, w, prob_mass, err[, probs])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    q = _c(token_mult, np.int32)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    mass = np.empty(E, dtype=np.float32)
    probs = np.empty((T, E), dtype=np.float32) if want_probs else None
    err = lib().orc_route_from_logits(_p(logits), _p(q), T, E, k, _p(idx), _p(w),
                                      _p(probs), _p(mass))
    if err < 0:
        raise ValueError("bad route dimensions")
    if want_probs:
        return idx, w, mass, err, probs
    return idx, w, mass, err


SCORES = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2}


def route_scored(logits, k: int, score: str = "sigmoid", corr_bias=None, hash_table=None,
                 token_ids=None, token_mult=None):
    """Router variants: softmax, or sigmoid / sqrt-softplus scores (FP64, rounded once to
    FP32) with a selection-only FP32 correction bias ("0 train-infer mismatch ...",
    "Choosing GLM's eight experts"), or hash routing from a frozen token-id table ("Hash and
    learned expert routing"); weights = the selected pre-bias values normalised left to
    right in FP32; q-weighted probability mass and per-token log-sum-exp (HARTS, eq. (20)).
    Returns dict(idx, w, scores, prob_mass, lse, err)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    q = _c(token_mult, np.int32)
    b = _c(corr_bias, np.float32)
    tab = _c(hash_table, np.int32)
    tok = _c(token_ids, np.int32)
    V = 0 if tab is None else tab.shape[0]
    if tab is not None and tab.shape[1] != k:
        raise ValueError("hash table rows must hold k experts")
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    sc = np.empty((T, E), dtype=np.float32)
    mass = np.empty(E, dtype=np.float32)
    lse = np.empty(T, dtype=np.float32)
    err = lib().orc_route_scored(_p(logits), _p(q), T, E, k, SCORES[score], _p(b), _p(tab),
                                 _p(tok), V, _p(idx), _p(w), _p(sc), _p(mass), _p(lse))
    if err < 0:
        raise ValueError("bad router-variant arguments")
    return dict(idx=idx, w=w, scores=sc, prob_mass=mass, lse=lse, err=err)


def objectives(lse, token_mult, weighted_counts, prob_mass, k: int, rate: float = 0.0,
               corr_bias=None):
    """q-weighted router z-loss, load-balancing loss and expert-bias update (HARTS, eq. (20)
    and "MoE execution and objectives"). Counts and mass in logical expert order. Returns
    (z_loss, aux_loss, S, updated bias or None)."""
    lse = _c(lse, np.float32)
    q = _c(token_mult, np.int32)
    C = _c(weighted_counts, np.int64)
    M = _c(prob_mass, np.float32)
    E = len(C) if C is not None else (len(M) if M is not None else 0)
    T = 0 if lse is None else len(lse)
    if lse is None and q is not None:
        T = len(q)
    b = None if corr_bias is None else np.array(corr_bias, dtype=np.float32, copy=True)
    out = np.zeros(3, dtype=np.float64)
    lib().orc_objectives(_p(lse), _p(q), T, _p(C), _p(M), E, k, rate, _p(b), _p(out))
    return float(out[0]), float(out[1]), int(out[2]), b


def replay_check(idx, w, E: int) -> int:
    """Validation of replayed ids/weights ("Total Router Recall")."""
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    T, k = idx.shape
    return lib().orc_replay_check(_p(idx), _p(w), T, E, k)


def permute(idx, E: int):
    """Histogram, exclusive offsets, stable counting sort. Returns
    (counts, offsets, perm, inv, err)."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.full(T * k, -1, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    err = lib().orc_permute(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv, err


def place_lpt(loads, P: int):
    """Layer-local LPT expert placement ("RoutePack ...", Sec. 3, Algorithm 1). Returns
    (slot_of_expert [E] int32, rank_load [P] int64, cv) where cv is the population standard
    deviation of the rank loads over their mean (the rank-load coefficient of variation of
    the same page's Sec. 5; 0 for a zero mean), computed in float64."""
    loads = _c(loads, np.int64)
    E = loads.shape[0]
    slots = np.empty(E, dtype=np.int32)
    rank_load = np.empty(P, dtype=np.int64)
    err = lib().orc_place_lpt(_p(loads), E, P, _p(slots), _p(rank_load))
    if err:
        raise ValueError("place_lpt: need E >= 1, P >= 1 and E % P == 0")
    mean = float(rank_load.sum()) / P
    var = sum((float(g) - mean) ** 2 for g in rank_load) / P
    cv = (var ** 0.5) / mean if mean > 0 else 0.0
    return slots, rank_load, cv


def place(idx, slot_of_expert):
    """The dispatcher's view of a placement ("RoutePack ...", Sec. 3, state-consistent
    materialization): every logical id replaced by the physical slot that stores it. Ids
    outside the map stay out of range (so they are still reported and dropped)."""
    idx = np.asarray(idx)
    m = np.asarray(slot_of_expert)
    out = np.full(idx.shape, -1, dtype=np.int32)
    ok = (idx >= 0) & (idx < len(m))
    out[ok] = m[idx[ok]]
    out[~ok] = idx[~ok]
    return out


def seq_counts(idx, E: int, cu_seqlens):
    idx = _c(idx, np.int32)
    cu = _c(cu_seqlens, np.int32)
    T, k = idx.shape
    S = len(cu) - 1
    out = np.zeros((S, E), dtype=np.int32)
    err = lib().orc_seq_counts(_p(idx), T, k, E, _p(cu), S, _p(out))
    return out, err


def weighted_counts(idx, E: int, token_mult=None):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    q = _c(token_mult, np.int32)
    out = np.empty(E, dtype=np.int64)
    err = lib().orc_weighted_counts(_p(idx), _p(q), T, k, E, _p(out))
    return out, err


def gather(x, perm, k: int, n_rows: Optional[int] = None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    perm = _c(perm, np.int32)
    n = len(perm) if n_rows is None else n_rows
    d = x.shape[1]
    out = np.empty((n, d), dtype=x.dtype)
    lib().orc_gather(_p(x), _p(perm), n, k, d, 1 if x.dtype == np.uint16 else 0, _p(out))
    return out


def expert_ffn(xrows, rowexp, w13, w2, dtype: str):
    """SwiGLU expert FFN per row: FP32 gate/up sums, one rounding of h, FP32 down sum.
    Returns (h, y)."""
    xrows = np.ascontiguousarray(xrows)
    rowexp = _c(rowexp, np.int32)
    n, d = xrows.shape
    I = w13.shape[1] // 2
    h = np.empty((n, I), dtype=_store_dtype(dtype))
    y = np.empty((n, d), dtype=np.float32)
    lib().orc_expert_ffn(_p(xrows), _p(rowexp), n, d, I, _p(np.ascontiguousarray(w13)),
                         _p(np.ascontiguousarray(w2)), _dt(dtype), _p(h), _p(y))
    return h, y


def combine(y, inv, w, dtype: str, scale: float = 1.0):
    """Slot-order FP32 weighted sum, times the routed scaling factor, rounded once to the
    output dtype."""
    y = _c(y, np.float32)
    inv = _c(inv, np.int32)
    w = _c(w, np.float32)
    T, k = w.shape
    d = y.shape[1]
    out = np.empty((T, d), dtype=_store_dtype(dtype))
    if scale == 1.0:
        lib().orc_combine(_p(y), _p(inv), _p(w), T, k, d, _dt(dtype), _p(out))
    else:
        lib().orc_combine_scaled(_p(y), _p(inv), _p(w), T, k, d, _dt(dtype), scale, _p(out))
    return out


def round_f64_bf16(a) -> np.ndarray:
    """float64 -> bfloat16 bits, round to nearest even in one step."""
    a = _c(a, np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_round_f64_bf16(_p(a), _p(out), a.size)
    return out


def shared_ffn(x, w13s, w2s, dtype: str):
    """The shared expert sharded over R ranks along its inter dimension ("0 train-infer
    mismatch ...", shared expert with the dense fixed-K projections and SwiGLU, one shard per
    rank): w13s [R, 2 Is/R, d] (each rank's gate rows then up rows), w2s [R, d, Is/R].
    Every rank's shard is the expert FFN of all T rows. Returns (h [R, T, Is/R],
    y [R, T, d] FP32)."""
    R = w13s.shape[0]
    T = x.shape[0]
    xr = np.ascontiguousarray(np.concatenate([x] * R, axis=0))
    rowexp = np.repeat(np.arange(R, dtype=np.int32), T)
    h, y = expert_ffn(xr, rowexp, w13s, w2s, dtype)
    return h.reshape(R, T, -1), y.reshape(R, T, -1)


def combine_ranks(y, inv, w, idx, E: int, R: int, dtype: str, slot_of_expert=None,
                  y_shared=None, scale: float = 1.0):
    """Rank partial outputs (slot-order FP32 sums with other ranks' slots as exact zeros,
    routed scaling factor, shared-expert shard, one rounding) and their FP64 pairwise tree
    in rank order, rounded once ("0 train-infer mismatch ...", "Sharding the experts").
    Returns (partials [R, T, d], out [T, d]) in the storage type."""
    y = _c(y, np.float32)
    inv = _c(inv, np.int32)
    w = _c(w, np.float32)
    idx = _c(idx, np.int32)
    sm = _c(slot_of_expert, np.int32)
    ys = _c(y_shared, np.float32)
    T, k = w.shape
    d = y.shape[1]
    parts = np.empty((R, T, d), dtype=_store_dtype(dtype))
    out = np.empty((T, d), dtype=_store_dtype(dtype))
    if lib().orc_combine_ranks(_p(y), _p(inv), _p(w), _p(idx), _p(sm), T, k, d, E, R, _p(ys),
                               scale, _dt(dtype), _p(parts), _p(out)) < 0:
        raise ValueError("combine_ranks: need 1 <= k <= E <= 256, d >= 1 and R dividing E")
    return parts, out


def backward_experts(x, perm, inv, counts, w, w13, w2, h, y, dout, dtype: str,
                     scale: float = 1.0, round_grads: bool = False) -> dict:
    """Backward of the expert path (derivative of the forward definitions; FP32, sequential
    sums; with round_grads, dy and dgu rounded once to bf16 where they are formed): dw, dy,
    gu, dh, dgu, dxp, dx (experts' part), dw13, dw2."""
    T, d = x.shape
    k = w.shape[1]
    E = len(counts)
    I = w2.shape[2]
    A = T * k
    rowexp = np.repeat(np.arange(E, dtype=np.int32), counts)
    f = lambda *sh: np.empty(sh, dtype=np.float32)
    r = dict(dw=f(T, k), dy=f(A, d), gu=f(A, 2 * I), dh=f(A, I), dgu=f(A, 2 * I),
             dxp=f(A, d), dx=f(T, d), dw13=f(E, 2 * I, d), dw2=f(E, d, I))
    args = [np.ascontiguousarray(a) for a in (x, perm, inv, rowexp, w, w13, w2, h, y, dout)]
    args[1], args[2], args[3] = (args[1].astype(np.int32), args[2].astype(np.int32),
                                 args[3].astype(np.int32))
    args[4], args[8] = args[4].astype(np.float32), args[8].astype(np.float32)
    lib().orc_backward_experts_r(*[_p(a) for a in args], scale, T, k, d, I, E, _dt(dtype),
                                 int(round_grads),
                                 *[_p(r[n]) for n in ("dw", "dy", "gu", "dh", "dgu", "dxp",
                                                      "dx", "dw13", "dw2")])
    return r


def backward_router(logits, dw, x, w_router, dtype: str) -> dict:
    """Backward of the softmax router from the weights' gradient by slot (its own choice
    recomputed from the logits; also the replay stop-gradient's router gradient): dl,
    dw_router, dx (router's part)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    k = dw.shape[1]
    d = x.shape[1]
    r = dict(dl=np.empty((T, E), np.float32), dw_router=np.empty((E, d), np.float32),
             dx=np.empty((T, d), np.float32))
    if lib().orc_backward_router(_p(logits), _p(_c(dw, np.float32)),
                                 _p(np.ascontiguousarray(x)), _p(np.ascontiguousarray(w_router)),
                                 T, E, k, d, _dt(dtype), _p(r["dl"]), _p(r["dw_router"]),
                                 _p(r["dx"])) < 0:
        raise ValueError("backward_router: need 1 <= k <= E <= 256 and d >= 1")
    return r


def forward(L, logits: Optional[np.ndarray] = None, S_stats: bool = True) -> dict:
    """All stages for a small layer ``L`` (a ``workloads.Layer``). In router mode the
    discrete decisions are taken from ``logits`` when given (the logits exported by the
    implementation under test), else from the oracle's own logits."""
    res = {}
    err = 0
    if L.mode == "router":
        own = router_logits(L.x, L.w_router, L.logit_bias, L.dtype)
        res["logits"] = own
        use = own if logits is None else logits
        score = getattr(L, "score", "softmax")
        if score == "softmax" and getattr(L, "hash_table", None) is None:
            idx, w, mass, e = route_from_logits(use, L.k, L.token_mult)
            res["lse"] = route_scored(use, L.k, "softmax", token_mult=L.token_mult)["lse"]
        else:
            r = route_scored(use, L.k, score, L.corr_bias, L.hash_table, L.token_ids,
                             L.token_mult)
            idx, w, mass, e = r["idx"], r["w"], r["prob_mass"], r["err"]
            res["lse"] = r["lse"]
        res["prob_mass"] = mass
        err |= e
    else:
        idx, w = L.idx_in, L.w_in
        err |= replay_check(idx, w, L.E)
    res["idx"], res["w"] = np.ascontiguousarray(idx), np.ascontiguousarray(w)
    counts, offsets, perm, inv, e = permute(idx, L.E)
    err |= e
    res.update(counts=counts, offsets=offsets, perm=perm, inv=inv)
    if S_stats:
        res["weighted_counts"], e = weighted_counts(idx, L.E, L.token_mult)
        err |= e
        if L.cu_seqlens is not None:
            res["seq_counts"], e = seq_counts(idx, L.E, L.cu_seqlens)
            err |= e
    x_perm = gather(L.x, perm, L.k)
    res["x_perm"] = x_perm
    rowexp = np.repeat(np.arange(L.E, dtype=np.int32), counts)
    h, y = expert_ffn(x_perm, rowexp, L.w13, L.w2, L.dtype)
    res["h"], res["y"] = h, y
    res["out"] = combine(y, inv, w, L.dtype, getattr(L, "routed_scale", 1.0))
    res["err"] = err
    return res


def forward_tokens(L, tokens, idx, w):
    """Expert FFN + combine for a subset of tokens, given their routing rows. Returns
    (h[len(tokens),k,I], y[len(tokens),k,d], out[len(tokens),d])."""
    tokens = np.asarray(tokens, dtype=np.int64)
    k = L.k
    sel_idx = np.ascontiguousarray(idx[tokens], dtype=np.int32)
    sel_w = np.ascontiguousarray(w[tokens], dtype=np.float32)
    xr = np.ascontiguousarray(np.repeat(L.x[tokens], k, axis=0))
    h, y = expert_ffn(xr, sel_idx.reshape(-1), L.w13, L.w2, L.dtype)
    inv = np.arange(len(tokens) * k, dtype=np.int32)
    out = combine(y, inv, sel_w, L.dtype, getattr(L, "routed_scale", 1.0))
    n = len(tokens)
    return h.reshape(n, k, -1), y.reshape(n, k, -1), out
