"""Seeded synthetic inputs for one MoE layer (shared by the oracle tests and the HIP path).

This module holds input generation only: no routing, dispatch, expert or combine
arithmetic. Every tensor comes from its own counter-free PCG64 stream,
``SeedSequence([config_seed, tensor_id, chunk])``, so the same bytes come out on every
machine and thread count.

Workload shapes follow the MoE RL pages:
  * packed, token-capped microbatches of variable-length sequences (RoutePack, "Packing"
    and the GRPO setup of its evaluation; HARTS, "Experimental Setup");
  * long-tailed response lengths and skewed, per-sample-correlated expert demand
    (RoutePack, Introduction and Sec. 2.3 "Sparse expert imbalance");
  * decode-sized batches (FlexFloor, graph-captured decode).
None of the pages' datasets is used; these generators stand in for them.

Dtypes: ``"f32"`` arrays are float32; ``"bf16"`` arrays are uint16 bit patterns of
bfloat16 values, rounded to nearest-even from float32 draws.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor ids of the per-tensor random streams
TID_X, TID_ROUTER, TID_W13, TID_W2, TID_BIAS, TID_LENS, TID_DIRICHLET, TID_REPLAY_IDS, \
    TID_REPLAY_W, TID_MULT, TID_CORR_BIAS, TID_HASH_TABLE, TID_TOKEN_IDS = range(13)

_WORKERS = max(1, min(8, os.cpu_count() or 1))


def _rng(seed: int, tid: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # 32-bit arithmetic suffices: a finite value's bits are at most 0xFF7FFFFF, so adding
    # at most 0x8000 cannot wrap; NaN patterns (which may wrap) are replaced below
    out = ((u + (((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((a.view(np.uint32)[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


def _normal(seed: int, tid: int, shape, std: float, dtype: str, chunks: int = 1) -> np.ndarray:
    """N(0, std^2) draws in float32, stored as ``dtype``; generated in ``chunks`` slices
    along axis 0, each from its own stream (so the bytes do not depend on thread count)."""
    shape = tuple(int(s) for s in shape)
    n0 = shape[0]
    chunks = max(1, min(chunks, n0)) if n0 > 0 else 1
    bounds = [(n0 * i) // chunks for i in range(chunks + 1)]
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def work(i):
        lo, hi = bounds[i], bounds[i + 1]
        if hi <= lo:
            return
        sub = (hi - lo,) + shape[1:]
        v = _rng(seed, tid, i).standard_normal(sub, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(v) if dtype == "bf16" else v

    if chunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_WORKERS) as ex:
            list(ex.map(work, range(chunks)))
    return out


@dataclass
class Layer:
    """One MoE layer's inputs. Weight layouts follow the Linear convention [out, in]:
    ``w_router[E, d]``, ``w13[E, 2I, d]`` (gate rows 0..I-1, then up rows I..2I-1),
    ``w2[E, d, I]``."""
    name: str
    T: int
    d: int
    E: int
    k: int
    I: int
    dtype: str                      # "f32" or "bf16"
    mode: str                       # "router" or "replay"
    seed: int
    x: np.ndarray
    w13: np.ndarray
    w2: np.ndarray
    w_router: Optional[np.ndarray] = None
    logit_bias: Optional[np.ndarray] = None     # float32 [E]
    idx_in: Optional[np.ndarray] = None         # int32 [T, k]  (replay)
    w_in: Optional[np.ndarray] = None           # float32 [T, k] (replay)
    cu_seqlens: Optional[np.ndarray] = None     # int32 [S+1]
    token_mult: Optional[np.ndarray] = None     # int32 [T]
    score: str = "softmax"                      # "softmax", "sigmoid" or "sqrt_softplus"
    corr_bias: Optional[np.ndarray] = None      # float32 [E], selection-only bias
    hash_table: Optional[np.ndarray] = None     # int32 [V, k] frozen token id -> experts
    token_ids: Optional[np.ndarray] = None      # int32 [T] (hash routing)
    routed_scale: float = 1.0                   # routed scaling factor of the combine
    meta: dict = field(default_factory=dict)

    @property
    def A(self) -> int:
        return self.T * self.k


# ---------------------------------------------------------------------------------------
# named configurations
# ---------------------------------------------------------------------------------------
CONFIGS = {
    "c1": dict(desc="tiny fp32 layer", T=256, d=128, E=8, k=2, I=256, dtype="f32",
               mode="router", seed=1),
    "c2": dict(desc="training-shaped bf16 layer, Zipf-skewed router bias", T=4096, d=2048,
               E=64, k=8, I=1408, dtype="bf16", mode="router", seed=2, bias="zipf"),
    "c3": dict(desc="packed RL microbatch, per-sequence Dirichlet replay", T=16384, d=4096,
               E=128, k=8, I=1536, dtype="bf16", mode="replay", seed=3, replay="dirichlet"),
    "c4": dict(desc="heavily imbalanced replay", T=32768, d=2048, E=256, k=8, I=768,
               dtype="bf16", mode="replay", seed=4, replay="hot"),
    "c5": dict(desc="decode-shaped, memory-bound (T = 1..64 from a 64-row pool)", T=64,
               d=4096, E=128, k=8, I=1536, dtype="bf16", mode="router", seed=5),
}


def zipf_log_bias(E: int, seed: int, s: float = 1.1) -> np.ndarray:
    """Per-expert additive router-logit bias ``-s * ln(rank_e)`` where ``rank_e`` is a
    seeded permutation of 1..E (the log of a Zipf(s) pmf, up to a constant)."""
    perm = _rng(seed, TID_BIAS).permutation(E)
    rank = 1.0 + perm.astype(np.float64)
    return (-s * np.log(rank)).astype(np.float32)


def packed_lengths(total: int, seed: int, median: float = 1024.0, sigma: float = 1.0,
                   cap: int = 8192) -> np.ndarray:
    """Lognormal sequence lengths (median ``median``, log-sd ``sigma``, capped at ``cap``)
    appended until they reach ``total`` tokens; the last one is truncated. Returns
    ``cu_seqlens`` (int32, starts at 0, ends at ``total``)."""
    rng = _rng(seed, TID_LENS)
    lens = []
    s = 0
    while s < total:
        z = rng.standard_normal()
        ell = int(min(cap, max(1, round(math.exp(math.log(median) + sigma * z)))))
        ell = min(ell, total - s)
        lens.append(ell)
        s += ell
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=cu[1:])
    return cu.astype(np.int32)


def _sort_slots(ids: np.ndarray, w: np.ndarray):
    """Order each row's slots by weight descending, ties to the lower expert id."""
    order = np.lexsort((ids, -w.astype(np.float64)), axis=1)
    return (np.take_along_axis(ids, order, axis=1).astype(np.int32),
            np.take_along_axis(w, order, axis=1).astype(np.float32))


def replay_dirichlet(cu_seqlens: np.ndarray, E: int, k: int, seed: int):
    """Per-sequence expert popularity ``pi_s ~ Dir(1_E)``; each token draws k distinct
    experts with probability proportional to ``pi_s`` (Gumbel top-k) and gets weights
    ``pi_s[sel] / sum(pi_s[sel])`` in float32, slots sorted by weight."""
    rng = _rng(seed, TID_DIRICHLET)
    T = int(cu_seqlens[-1])
    ids = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k), dtype=np.float64)
    for s in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        pi = rng.dirichlet(np.ones(E))
        g = rng.gumbel(size=(hi - lo, E))
        keys = np.log(np.maximum(pi, 1e-300))[None, :] + g
        sel = np.argsort(-keys, axis=1, kind="stable")[:, :k]
        ps = pi[sel]
        ids[lo:hi] = sel
        w[lo:hi] = ps / ps.sum(axis=1, keepdims=True)
    return _sort_slots(ids, w.astype(np.float32))


def ep_share_counts(cfg: str = "c3", ranks: int = 8, seed0: int = 100) -> np.ndarray:
    """Rows one expert-parallel rank receives: ``ranks`` data-parallel batches shaped like
    ``cfg`` (each its own seed), each routed over all E experts; rank 0 owns experts
    0 .. E/ranks - 1 and receives every batch's rows for them. Returns the per-local-expert
    row counts (int64, length E / ranks)."""
    c = CONFIGS[cfg]
    E, k, T = c["E"], c["k"], c["T"]
    H = E // ranks
    tot = np.zeros(H, dtype=np.int64)
    for r in range(ranks):
        cu = packed_lengths(T, seed0 + r)
        ids, _ = replay_dirichlet(cu, E, k, seed0 + r)
        tot += np.bincount(ids.reshape(-1), minlength=E)[:H]
    return tot


def replay_hot(T: int, E: int, k: int, seed: int):
    """Imbalanced replay for E=256, k=8: one hot expert is in every token's set, four
    slots come from a 15-expert group, three from 224 tail experts (both uniform without
    replacement), and 16 experts receive nothing. Weights ~ Dir(1_k), slots sorted."""
    assert E == 256 and k == 8, "hot replay pattern is defined for E=256, k=8"
    rng = _rng(seed, TID_REPLAY_IDS)
    perm = rng.permutation(E)
    hot, group, zero, tail = perm[0], perm[1:16], perm[16:32], perm[32:]
    g = group[np.argsort(rng.random((T, 15)), axis=1)[:, :4]]
    tl = tail[np.argsort(rng.random((T, 224)), axis=1)[:, :3]]
    ids = np.concatenate([np.full((T, 1), hot), g, tl], axis=1)
    ids = np.take_along_axis(ids, np.argsort(rng.random((T, k)), axis=1), axis=1)
    e = _rng(seed, TID_REPLAY_W).standard_exponential((T, k))
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    ids_s, w_s = _sort_slots(ids, w)
    return ids_s, w_s, dict(hot=int(hot), group=group.astype(np.int32),
                            zero=np.sort(zero).astype(np.int32), tail=tail.astype(np.int32))


def token_multiplicities(T: int, seed: int, qmax: int = 4) -> np.ndarray:
    """Per-token multiplicities q_t in 1..qmax (HARTS, MoE semantics, eq. (20))."""
    return _rng(seed, TID_MULT).integers(1, qmax + 1, size=T).astype(np.int32)


SCORES = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2}


def correction_bias(E: int, seed: int, std: float = 0.05) -> np.ndarray:
    """Selection-only expert correction bias, N(0, std^2) in FP32 (the pages give no
    values; std 0.05 is comparable to the gaps between neighbouring sigmoid scores of
    unit-variance logits, so the bias changes some selections)."""
    return (_rng(seed, TID_CORR_BIAS).standard_normal(E) * std).astype(np.float32)


def hash_table(V: int, E: int, k: int, seed: int) -> np.ndarray:
    """Frozen token-id -> expert table [V, k]: each row k distinct experts, uniformly at
    random, in random order."""
    rng = _rng(seed, TID_HASH_TABLE)
    return np.argsort(rng.random((V, E)), axis=1)[:, :k].astype(np.int32)


def token_ids(T: int, V: int, seed: int, s: float = 1.1) -> np.ndarray:
    """Token ids drawn from a Zipf(s) law over a seeded ranking of the V ids (frequent
    tokens repeat, so the table's experts are unevenly loaded)."""
    rng = _rng(seed, TID_TOKEN_IDS)
    p = 1.0 / np.arange(1, V + 1, dtype=np.float64) ** s
    p /= p.sum()
    rank = rng.choice(V, size=T, p=p)
    return rng.permutation(V).astype(np.int32)[rank]


def set_router(L: "Layer", score: str = "sigmoid", bias: bool = True,
               hash_vocab: Optional[int] = None, routed_scale: float = 1.0) -> "Layer":
    """Switch a router-mode layer to a router variant: score function, correction bias,
    hash routing over a vocabulary of ``hash_vocab`` ids, routed scaling factor."""
    if score not in SCORES:
        raise ValueError(score)
    L.score = score
    L.corr_bias = correction_bias(L.E, L.seed) if bias else None
    if hash_vocab:
        L.hash_table = hash_table(hash_vocab, L.E, L.k, L.seed)
        L.token_ids = token_ids(L.T, hash_vocab, L.seed)
    L.routed_scale = float(routed_scale)
    return L


def make_layer(T: int, d: int, E: int, k: int, I: int, dtype: str = "bf16",
               mode: str = "router", seed: int = 0, bias: Optional[str] = None,
               replay: Optional[str] = None, seqs: bool = False, mult: bool = False,
               name: str = "custom", weights: bool = True) -> Layer:
    """Build one layer's inputs. ``mode='router'`` makes a router weight (and optional
    Zipf bias); ``mode='replay'`` makes replay ids/weights (``replay`` in
    {'dirichlet', 'hot', 'uniform'})."""
    if not (1 <= k <= E):
        raise ValueError(f"need 1 <= k <= E (k={k}, E={E})")
    std = 1.0 / math.sqrt(d)
    x = _normal(seed, TID_X, (T, d), 1.0, dtype, chunks=max(1, min(64, T // 256)))
    if weights:
        w13 = _normal(seed, TID_W13, (E, 2 * I, d), std, dtype, chunks=E)
        w2 = _normal(seed, TID_W2, (E, d, I), std, dtype, chunks=E)
    else:
        w13 = w2 = None
    L = Layer(name=name, T=T, d=d, E=E, k=k, I=I, dtype=dtype, mode=mode, seed=seed,
              x=x, w13=w13, w2=w2)
    cu = None
    if seqs or replay == "dirichlet":
        cu = packed_lengths(T, seed)
        L.cu_seqlens = cu
    if mode == "router":
        L.w_router = _normal(seed, TID_ROUTER, (E, d), std, dtype)
        if bias == "zipf":
            L.logit_bias = zipf_log_bias(E, seed)
    else:
        if replay == "dirichlet":
            L.idx_in, L.w_in = replay_dirichlet(cu, E, k, seed)
        elif replay == "hot":
            L.idx_in, L.w_in, L.meta["hot"] = replay_hot(T, E, k, seed)
        else:
            rng = _rng(seed, TID_REPLAY_IDS)
            ids = np.argsort(rng.random((T, E)), axis=1)[:, :k]
            e = _rng(seed, TID_REPLAY_W).standard_exponential((T, k))
            L.idx_in, L.w_in = _sort_slots(ids, (e / e.sum(axis=1, keepdims=True)).astype(np.float32))
    if mult:
        L.token_mult = token_multiplicities(T, seed)
    return L


def make_config(cfg: str, T: Optional[int] = None, weights: bool = True) -> Layer:
    c = CONFIGS[cfg]
    L = make_layer(T=c["T"], d=c["d"], E=c["E"], k=c["k"], I=c["I"], dtype=c["dtype"],
                   mode=c["mode"], seed=c["seed"], bias=c.get("bias"),
                   replay=c.get("replay"), seqs=(cfg == "c3"), name=cfg, weights=weights)
    if T is not None and cfg == "c5":
        L.x = np.ascontiguousarray(L.x[:T])
        L.T = T
    return L
