"""Python binding of the MI355X MoE-layer hot-path library (``libmoe_hip.so``).

Argument marshalling only: every function passes torch tensors' device pointers and the
current HIP stream to the C ABI declared in ``include/moe.h`` and raises ``MoeError`` on a
non-OK status. All computation runs in the library's HIP kernels; there is no fallback.
If the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_hip.so")

MOE_F32, MOE_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20     # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h
DERR_IDX_RANGE, DERR_IDX_DUP, DERR_NONFINITE, DERR_SEQLENS, DERR_SLOTMAP = 1, 2, 4, 8, 16
STATUS = {0: "MOE_OK", 1: "MOE_E_NULLPTR", 2: "MOE_E_SHAPE", 3: "MOE_E_DTYPE",
          4: "MOE_E_WORKSPACE", 5: "MOE_E_LAUNCH", 6: "MOE_E_SCRATCH"}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("inter", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("tile_m", ctypes.c_int32)]

    def __repr__(self):
        return (f"Dims(T={self.T}, d={self.d}, E={self.E}, k={self.k}, inter={self.inter}, "
                f"dtype={self.dtype}, tile_m={self.tile_m})")


_P = ctypes.c_void_p


class ForwardArgs(ctypes.Structure):
    _fields_ = [("x", _P), ("w_router", _P), ("logit_bias", _P), ("idx_in", _P), ("w_in", _P),
                ("w13", _P), ("w2", _P), ("token_mult", _P), ("cu_seqlens", _P),
                ("num_seqs", ctypes.c_int32), ("out", _P), ("topk_idx", _P), ("topk_w", _P),
                ("logits", _P), ("prob_mass", _P), ("counts", _P), ("offsets", _P),
                ("perm", _P), ("inv", _P), ("seq_counts", _P), ("weighted_counts", _P),
                ("x_perm", _P), ("h", _P), ("y", _P), ("d_err", _P), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t), ("prof_events", _P),
                ("slot_of_expert", _P), ("router", _P), ("routed_scale", ctypes.c_float),
                ("ranks", ctypes.c_int32), ("partials", _P), ("w13_shared", _P),
                ("w2_shared", _P), ("inter_shared", ctypes.c_int32), ("h_shared", _P),
                ("y_shared", _P), ("shared_workspace", _P),
                ("shared_workspace_bytes", ctypes.c_size_t), ("gu", _P)]


class RouterOpts(ctypes.Structure):
    _fields_ = [("score_fn", ctypes.c_int32), ("corr_bias", _P), ("hash_table", _P),
                ("token_ids", _P), ("vocab", ctypes.c_int32), ("lse", _P)]


SCORES = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2}


class BackwardArgs(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("x", "x_perm", "w13", "w2", "w_router", "logit_bias",
                                  "logits", "offsets", "perm", "inv", "topk_w", "h", "y",
                                  "d_out")] + \
               [("routed_scale", ctypes.c_float)] + \
               [(n, _P) for n in ("d_x", "d_w13", "d_w2", "d_topk_w", "d_logits", "d_w_router",
                                  "d_x_router", "d_y", "gu", "d_h", "d_gu", "d_xp",
                                  "workspace")] + \
               [("workspace_bytes", ctypes.c_size_t), ("grad_dtype", ctypes.c_int32),
                ("gu_saved", ctypes.c_int32)]


# exported symbols and their signatures (argument types after the dims pointer)
_SIGS = {
    "moe_workspace_size": ([ctypes.POINTER(Dims)], ctypes.c_size_t),
    "moe_tile_height": ([ctypes.POINTER(Dims)], ctypes.c_int32),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_version": ([], ctypes.c_int),
    "moe_route": ([ctypes.POINTER(Dims)] + [_P] * 9 + [_P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_route_replay": ([ctypes.POINTER(Dims)] + [_P] * 5 + [_P], ctypes.c_int),
    "moe_permute": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                     _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_grouped_ffn": ([ctypes.POINTER(Dims)] + [_P] * 6 + [_P, ctypes.c_size_t, _P],
                        ctypes.c_int),
    "moe_combine": ([ctypes.POINTER(Dims)] + [_P] * 4 + [_P], ctypes.c_int),
    "moe_forward": ([ctypes.POINTER(Dims), ctypes.POINTER(ForwardArgs), _P], ctypes.c_int),
    "moe_forward_noalloc": ([ctypes.POINTER(Dims), ctypes.POINTER(ForwardArgs), _P],
                            ctypes.c_int),
    "moe_permute_placed": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                            ctypes.c_int32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
                           ctypes.c_int),
    "moe_place_lpt": ([_P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P], ctypes.c_int),
    "moe_route_scored": ([ctypes.POINTER(Dims), ctypes.POINTER(RouterOpts)] + [_P] * 9
                         + [_P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_combine_scaled": ([ctypes.POINTER(Dims), _P, _P, _P, ctypes.c_float, _P, _P],
                           ctypes.c_int),
    "moe_objectives": ([ctypes.POINTER(Dims), _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                        _P], ctypes.c_int),
    "moe_backward": ([ctypes.POINTER(Dims), ctypes.POINTER(BackwardArgs), _P], ctypes.c_int),
    "moe_combine_ranks": ([ctypes.POINTER(Dims), ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                           ctypes.c_float, _P, _P, _P], ctypes.c_int),
    "moe_shared_workspace_size": ([ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32],
                                  ctypes.c_size_t),
    "moe_shared_ffn": ([ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P,
                        _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
}

_lib = None


def lib():
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


# ------------------------------------------------------------------------ marshalling

def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise MoeError(status, where)


def storage_dtype(dtype: int) -> torch.dtype:
    return torch.bfloat16 if dtype == MOE_BF16 else torch.float32


def make_dims(T: int, d: int, E: int, k: int, inter: int, dtype: int, tile_m: int = 0) -> Dims:
    return Dims(int(T), int(d), int(E), int(k), int(inter), int(dtype), int(tile_m))


def workspace_size(dims: Dims) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(dims)))


def tile_height(dims: Dims) -> int:
    """Token-tile height of the grouped GEMMs for dims (0 for invalid dims)."""
    return int(lib().moe_tile_height(ctypes.byref(dims)))


def alloc_workspace(dims: Dims, device="cuda") -> torch.Tensor:
    n = workspace_size(dims)
    if n == 0:
        raise MoeError(2, "moe_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


# --------------------------------------------------------------------- entry points

def route(dims, x, w_router, logit_bias, topk_idx, topk_w, logits=None, prob_mass=None,
          token_mult=None, d_err=None, workspace=None, stream=None):
    ws = workspace if workspace is not None else alloc_workspace(dims, x.device)
    _check(lib().moe_route(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                           _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(prob_mass),
                           _ptr(token_mult), _ptr(d_err), _ptr(ws), ws.numel(),
                           _stream(stream)), "moe_route")


def router_opts(score="softmax", corr_bias=None, hash_table=None, token_ids=None,
                lse=None) -> RouterOpts:
    """moe_router_opts from tensors (hash_table [V, k] int32, token_ids [T] int32)."""
    o = RouterOpts()
    o.score_fn = SCORES[score]
    o.corr_bias = _ptr(corr_bias)
    o.hash_table = _ptr(hash_table)
    o.token_ids = _ptr(token_ids)
    o.vocab = 0 if hash_table is None else hash_table.shape[0]
    o.lse = _ptr(lse)
    return o


def route_scored(dims, x, w_router, logit_bias, topk_idx, topk_w, score="sigmoid",
                 corr_bias=None, hash_table=None, token_ids=None, lse=None, logits=None,
                 prob_mass=None, token_mult=None, d_err=None, workspace=None, stream=None):
    ws = workspace if workspace is not None else alloc_workspace(dims, x.device)
    o = router_opts(score, corr_bias, hash_table, token_ids, lse)
    _check(lib().moe_route_scored(ctypes.byref(dims), ctypes.byref(o), _ptr(x), _ptr(w_router),
                                  _ptr(logit_bias), _ptr(topk_idx), _ptr(topk_w), _ptr(logits),
                                  _ptr(prob_mass), _ptr(token_mult), _ptr(d_err), _ptr(ws),
                                  ws.numel(), _stream(stream)), "moe_route_scored")


def objectives(dims, out, lse=None, token_mult=None, weighted_counts=None, prob_mass=None,
               slot_of_expert=None, bias_rate=0.0, corr_bias=None, d_err=None, stream=None):
    """moe_objectives: out is a float64 device tensor of 3 (z_loss, aux_loss, S)."""
    _check(lib().moe_objectives(ctypes.byref(dims), _ptr(lse), _ptr(token_mult),
                                _ptr(weighted_counts), _ptr(prob_mass), _ptr(slot_of_expert),
                                bias_rate, _ptr(corr_bias), _ptr(out), _ptr(d_err),
                                _stream(stream)), "moe_objectives")


def combine_ranks(dims, ranks: int, y, inv, topk_w, topk_idx, out, slot_of_expert=None,
                  y_shared=None, routed_scale: float = 0.0, partials=None, stream=None):
    """moe_combine_ranks: rank partial outputs and their FP64 pairwise tree."""
    _check(lib().moe_combine_ranks(ctypes.byref(dims), ranks, _ptr(y), _ptr(inv), _ptr(topk_w),
                                   _ptr(topk_idx), _ptr(slot_of_expert), _ptr(y_shared),
                                   routed_scale, _ptr(partials), _ptr(out), _stream(stream)),
           "moe_combine_ranks")


def shared_workspace_size(dims, ranks: int, inter_shared: int) -> int:
    return lib().moe_shared_workspace_size(ctypes.byref(dims), ranks, inter_shared)


def alloc_shared_workspace(dims, ranks: int, inter_shared: int, device="cuda") -> torch.Tensor:
    n = shared_workspace_size(dims, ranks, inter_shared)
    if n == 0:
        raise MoeError(2, "moe_shared_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def shared_ffn(dims, ranks: int, inter_shared: int, x, w13_shared, w2_shared, h_shared,
               y_shared, workspace=None, stream=None):
    """moe_shared_ffn: the shared expert sharded over ``ranks`` ranks."""
    ws = workspace if workspace is not None else alloc_shared_workspace(dims, ranks,
                                                                         inter_shared, x.device)
    _check(lib().moe_shared_ffn(ctypes.byref(dims), ranks, inter_shared, _ptr(x),
                                _ptr(w13_shared), _ptr(w2_shared), _ptr(h_shared),
                                _ptr(y_shared), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_shared_ffn")


def route_replay(dims, idx_in, w_in, topk_idx, topk_w, d_err=None, stream=None):
    _check(lib().moe_route_replay(ctypes.byref(dims), _ptr(idx_in), _ptr(w_in), _ptr(topk_idx),
                                  _ptr(topk_w), _ptr(d_err), _stream(stream)),
           "moe_route_replay")


def permute(dims, topk_idx, x, x_perm, perm, inv, counts, offsets, cu_seqlens=None,
            seq_counts=None, token_mult=None, weighted_counts=None, d_err=None,
            workspace=None, stream=None, slot_of_expert=None):
    """moe_permute, or moe_permute_placed when a device slot map is given."""
    ws = workspace if workspace is not None else alloc_workspace(dims, counts.device)
    S = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    if slot_of_expert is None:
        _check(lib().moe_permute(ctypes.byref(dims), _ptr(topk_idx), _ptr(x), _ptr(x_perm),
                                 _ptr(perm), _ptr(inv), _ptr(counts), _ptr(offsets),
                                 _ptr(cu_seqlens), S, _ptr(seq_counts), _ptr(token_mult),
                                 _ptr(weighted_counts), _ptr(d_err), _ptr(ws), ws.numel(),
                                 _stream(stream)), "moe_permute")
    else:
        _check(lib().moe_permute_placed(ctypes.byref(dims), _ptr(topk_idx), _ptr(slot_of_expert),
                                        _ptr(x), _ptr(x_perm), _ptr(perm), _ptr(inv),
                                        _ptr(counts), _ptr(offsets), _ptr(cu_seqlens), S,
                                        _ptr(seq_counts), _ptr(token_mult),
                                        _ptr(weighted_counts), _ptr(d_err), _ptr(ws),
                                        ws.numel(), _stream(stream)), "moe_permute_placed")


def place_lpt(loads, P: int):
    """moe_place_lpt on host arrays: loads [E] int64 -> (slot_of_expert [E] int32,
    rank_load [P] int64, cv float)."""
    import numpy as np
    loads = np.ascontiguousarray(loads, dtype=np.int64)
    E = loads.shape[0]
    slots = np.empty(E, dtype=np.int32)
    rank_load = np.empty(max(P, 1), dtype=np.int64)
    cv = ctypes.c_double()
    _check(lib().moe_place_lpt(loads.ctypes.data, E, P, slots.ctypes.data,
                               rank_load.ctypes.data, ctypes.addressof(cv)), "moe_place_lpt")
    return slots, rank_load[:P], cv.value


def grouped_ffn(dims, x_perm, offsets, w13, w2, h, y, workspace=None, stream=None):
    ws = workspace if workspace is not None else alloc_workspace(dims, offsets.device)
    _check(lib().moe_grouped_ffn(ctypes.byref(dims), _ptr(x_perm), _ptr(offsets), _ptr(w13),
                                 _ptr(w2), _ptr(h), _ptr(y), _ptr(ws), ws.numel(),
                                 _stream(stream)), "moe_grouped_ffn")


def combine(dims, y, inv, topk_w, out, stream=None, routed_scale=None):
    """moe_combine, or moe_combine_scaled when a routed scaling factor is given."""
    if routed_scale is None:
        _check(lib().moe_combine(ctypes.byref(dims), _ptr(y), _ptr(inv), _ptr(topk_w),
                                 _ptr(out), _stream(stream)), "moe_combine")
    else:
        _check(lib().moe_combine_scaled(ctypes.byref(dims), _ptr(y), _ptr(inv), _ptr(topk_w),
                                        routed_scale, _ptr(out), _stream(stream)),
               "moe_combine_scaled")


def forward(dims, bufs: dict, workspace: torch.Tensor, prof_events=None, stream=None,
            router: Optional[dict] = None, routed_scale: float = 0.0, ranks: int = 0,
            inter_shared: int = 0, shared_workspace: Optional[torch.Tensor] = None):
    """Run moe_forward. ``bufs`` maps ForwardArgs field names to tensors (or None);
    ``prof_events`` is None or a sequence of three raw hipEvent_t handles; ``router`` is
    None or the keyword arguments of router_opts; ``routed_scale`` 0 means no factor."""
    keep = _forward_args(bufs, workspace, prof_events, router, routed_scale, ranks,
                         inter_shared, shared_workspace)
    _check(lib().moe_forward(ctypes.byref(dims), ctypes.byref(keep[0]), _stream(stream)),
           "moe_forward")


def forward_noalloc(dims, bufs: dict, prof_events=None, stream=None,
                    router: Optional[dict] = None, routed_scale: float = 0.0, ranks: int = 0,
                    inter_shared: int = 0):
    """Run moe_forward_noalloc: moe_forward with the library's static per-GPU scratch as
    its workspace (the caller allocates no workspace). Same ``bufs`` as ``forward``."""
    keep = _forward_args(bufs, None, prof_events, router, routed_scale, ranks, inter_shared,
                         None)
    _check(lib().moe_forward_noalloc(ctypes.byref(dims), ctypes.byref(keep[0]),
                                     _stream(stream)), "moe_forward_noalloc")


def _forward_args(bufs, workspace, prof_events, router, routed_scale, ranks, inter_shared,
                  shared_workspace):
    """ForwardArgs for ``bufs``, plus the ctypes objects it points into (kept alive by the
    caller for the duration of the call)."""
    a = ForwardArgs()
    for name, _ in ForwardArgs._fields_:
        if name in ("num_seqs", "workspace", "workspace_bytes", "prof_events", "router",
                    "routed_scale", "ranks", "inter_shared", "shared_workspace",
                    "shared_workspace_bytes"):
            continue
        setattr(a, name, _ptr(bufs.get(name)))
    ropts = None
    if router is not None:
        ropts = router_opts(**router)
        a.router = ctypes.cast(ctypes.pointer(ropts), ctypes.c_void_p)
    a.routed_scale = routed_scale
    a.ranks = ranks
    a.inter_shared = inter_shared
    if shared_workspace is not None:
        a.shared_workspace = _ptr(shared_workspace)
        a.shared_workspace_bytes = shared_workspace.numel()
    cu = bufs.get("cu_seqlens")
    a.num_seqs = 0 if cu is None else cu.numel() - 1
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel()
    ev_arr = None
    if prof_events is not None:
        ev_arr = (ctypes.c_void_p * 3)(*prof_events)
        a.prof_events = ctypes.cast(ev_arr, ctypes.c_void_p)
    return a, ropts, ev_arr


def backward(dims, bufs: dict, workspace: torch.Tensor, routed_scale: float = 0.0,
             stream=None, grad_dtype: int = MOE_F32, gu_saved: bool = False):
    """Run moe_backward. ``bufs`` maps BackwardArgs field names to tensors (or None);
    grad_dtype MOE_BF16 selects bf16 gradient operands (then d_y / d_gu are bf16);
    gu_saved: bufs["gu"] holds the forward's pre-activations (forward with bufs["gu"])."""
    a = BackwardArgs()
    for name, _ in BackwardArgs._fields_:
        if name in ("routed_scale", "workspace", "workspace_bytes", "grad_dtype", "gu_saved"):
            continue
        setattr(a, name, _ptr(bufs.get(name)))
    a.routed_scale = routed_scale
    a.grad_dtype = grad_dtype
    a.gu_saved = int(bool(gu_saved))
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel()
    _check(lib().moe_backward(ctypes.byref(dims), ctypes.byref(a), _stream(stream)),
           "moe_backward")


def alloc_backward_buffers(dims: Dims, device="cuda", router: bool = True,
                           grad_dtype: int = MOE_F32, keep_gu: bool = True) -> dict:
    """Allocate every output and intermediate of moe_backward for ``dims`` (with bf16
    gradient operands, d_y / d_gu are bf16). ``keep_gu=False`` (bf16 layers) leaves out the
    recomputed pre-activations gu: the recomputation then forms d_gu itself."""
    T, d, E, k, I = dims.T, dims.d, dims.E, dims.k, dims.inter
    A = T * k
    f = lambda *sh: torch.empty(sh, dtype=torch.float32, device=device)
    g = (lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=device)) \
        if grad_dtype == MOE_BF16 else f
    b = dict(d_x=f(T, d), d_w13=f(E, 2 * I, d), d_w2=f(E, d, I), d_topk_w=f(T, k),
             d_y=g(A, d), d_h=f(A, I), d_gu=g(A, 2 * I), d_xp=f(A, d))
    if keep_gu:
        b["gu"] = f(A, 2 * I)
    if router:
        b.update(d_logits=f(T, E), d_w_router=f(E, d), d_x_router=f(T, d))
    return b


def alloc_forward_buffers(dims: Dims, device="cuda", router: bool = True,
                          num_seqs: int = 0, weighted: bool = False) -> dict:
    """Allocate every output and intermediate of moe_forward for ``dims``."""
    T, d, E, k, I = dims.T, dims.d, dims.E, dims.k, dims.inter
    A = T * k
    sd = storage_dtype(dims.dtype)
    i32 = dict(dtype=torch.int32, device=device)
    b = dict(
        out=torch.empty((T, d), dtype=sd, device=device),
        topk_idx=torch.empty((T, k), **i32),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
        counts=torch.empty(E, **i32),
        offsets=torch.empty(E + 1, **i32),
        perm=torch.empty(A, **i32),
        inv=torch.empty(A, **i32),
        x_perm=torch.empty((A, d), dtype=sd, device=device),
        h=torch.empty((A, I), dtype=sd, device=device),
        y=torch.empty((A, d), dtype=torch.float32, device=device),
        d_err=torch.zeros(1, **i32),
    )
    if router:
        b["logits"] = torch.empty((T, E), dtype=torch.float32, device=device)
        b["prob_mass"] = torch.empty(E, dtype=torch.float32, device=device)
    if num_seqs:
        b["seq_counts"] = torch.empty((num_seqs, E), **i32)
    if weighted:
        b["weighted_counts"] = torch.empty(E, dtype=torch.int64, device=device)
    return b
