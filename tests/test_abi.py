"""The C-ABI library loads on a machine without a GPU, exports every symbol the header
declares, and its host-side checks reject bad arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def M():
    import moe_layer_routing_amd as M
    if not os.path.exists(M.LIB_PATH):
        from moe_layer_routing_amd import _build
        _build.build()
    M.lib()
    return M


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("moe_route", "moe_route_replay", "moe_permute", "moe_grouped_ffn", "moe_combine",
              "moe_forward", "moe_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(M):
    L = M.lib()
    for n in header_functions():
        assert hasattr(L, n), n
    assert sorted(M.exported_symbols()) == header_functions()
    # the exported names are plain C symbols
    assert ctypes.CDLL(M.LIB_PATH).moe_version() == 100


def test_struct_layouts_match_header(M, tmp_path):
    """Field offsets of the ctypes mirrors equal what a C compiler makes of the header."""
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe.h"', 'int main(void){']
    for cname, py in (("moe_dims", M.Dims), ("moe_forward_args", M.ForwardArgs),
                      ("moe_backward_args", M.BackwardArgs), ("moe_router_opts", M.RouterOpts)):
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                 check=True).stdout.splitlines())
    for cname, py in (("moe_dims", M.Dims), ("moe_forward_args", M.ForwardArgs),
                      ("moe_backward_args", M.BackwardArgs), ("moe_router_opts", M.RouterOpts)):
        assert int(got[cname]) == ctypes.sizeof(py)
        for f, _ in py._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(py, f).offset, f


def test_workspace_size(M):
    d = M.make_dims(4096, 2048, 64, 8, 1408, M.MOE_BF16)
    n = M.workspace_size(d)
    assert n > 4096 * 64 * 4          # holds the router logits
    assert n < 64 << 20                # never a full activation
    for bad in (dict(E=0), dict(E=257), dict(k=9), dict(k=0), dict(d=100), dict(inter=96 + 1),
                dict(dtype=7), dict(tile_m=48), dict(T=-1)):
        kw = dict(T=10, d=128, E=8, k=2, inter=128, dtype=M.MOE_F32)
        kw.update(bad)
        assert M.workspace_size(M.make_dims(**kw)) == 0, bad
    assert M.workspace_size(M.make_dims(0, 128, 8, 2, 128, M.MOE_F32)) > 0


def test_tile_height(M):
    """The grouped GEMMs' token-tile height: 256 from 128 mean rows per expert on, else the
    smallest of 16/32/64/128 holding min(T, ceil(1.5 * mean rows)); a nonzero tile_m wins."""
    cases = [  # (T, E, k, tile_m, expected) - mean rows T*k/E, want = min(T, ceil(1.5 mean))
        (16384, 128, 8, 0, 256),   # mean 1024
        (2048, 128, 8, 0, 256),    # mean exactly 128
        (2047, 128, 8, 0, 128),    # mean 127.9 -> want 192, above 128 but not yet 256
        (1024, 128, 8, 0, 128),    # mean 64 -> want 96
        (512, 128, 8, 0, 64),      # mean 32 -> want 48
        (256, 128, 8, 0, 32),      # mean 16 -> want 24
        (64, 128, 8, 0, 16),       # mean 4 -> want 6
        (1, 128, 8, 0, 16),        # one token
        (0, 128, 8, 0, 16),        # empty batch
        (32, 3, 1, 0, 16),         # want exactly 16
        (33, 3, 1, 0, 32),         # want 16.5 -> 17
        (16, 8, 8, 0, 16),         # want 24 capped at T = 16 (no expert has more than T rows)
        (20, 8, 8, 0, 32),         # want 30 capped at T = 20
        (4096, 64, 8, 0, 256),     # mean 512
        (4096, 64, 8, 64, 64),     # forced
        (1, 128, 8, 256, 256),     # forced
    ]
    for T, E, k, tm, want in cases:
        assert M.tile_height(M.make_dims(T, 256, E, k, 256, M.MOE_BF16, tm)) == want, (T, E, k, tm)
    assert M.tile_height(M.make_dims(10, 128, 8, 2, 128, M.MOE_BF16, 48)) == 0
    assert M.tile_height(M.make_dims(10, 128, 8, 2, 128, 7)) == 0


def test_status_strings(M):
    L = M.lib()
    for s in range(7):
        assert L.moe_status_string(s)


def test_host_checks_reject_before_any_launch(M):
    """These calls fail validation, so they return without touching the HIP runtime."""
    L = M.lib()
    good = M.make_dims(16, 128, 8, 2, 128, M.MOE_BF16)
    ws = ctypes.c_void_p(0x1000)
    fake = ctypes.c_void_p(0x2000)
    # NULL dims
    assert L.moe_route(None, *([fake] * 9), ws, 1 << 30, None) == 1
    # bad dtype / shape
    bad = M.make_dims(16, 128, 8, 2, 128, 5)
    assert L.moe_combine(ctypes.byref(bad), fake, fake, fake, fake, None) == 3
    bad = M.make_dims(16, 128, 8, 9, 128, M.MOE_BF16)
    assert L.moe_route_replay(ctypes.byref(bad), fake, fake, fake, fake, None, None) == 2
    # required pointer missing
    assert L.moe_route(ctypes.byref(good), None, fake, None, fake, fake, None, None, None, None,
                       ws, 1 << 30, None) == 1
    assert L.moe_combine(ctypes.byref(good), fake, None, fake, fake, None) == 1
    # workspace too small / missing
    assert L.moe_route(ctypes.byref(good), fake, fake, None, fake, fake, None, None, None, None,
                       ws, 16, None) == 4
    assert L.moe_grouped_ffn(ctypes.byref(good), fake, fake, fake, fake, fake, fake, None,
                             1 << 30, None) == 4
    # cu_seqlens without seq_counts
    assert L.moe_permute(ctypes.byref(good), fake, fake, fake, fake, fake, fake, fake, fake, 2,
                         None, None, None, None, ws, 1 << 30, None) == 1


def test_backward_gu_optional_only_on_bf16_layers(M):
    """moe_backward may be called without gu on a bf16 layer (the recomputation then forms
    d_gu itself): the pointer checks pass and the call stops at the too-small workspace,
    still before any launch. An FP32 layer without gu is rejected as a missing pointer."""
    L = M.lib()
    optional = {"x_perm", "w_router", "logit_bias", "logits", "d_logits", "d_w_router",
                "d_x_router", "gu"}

    def args(gu):
        a = M.BackwardArgs()
        for n, t in a._fields_:
            if t is ctypes.c_void_p and n not in optional:
                setattr(a, n, 0x2000)
        a.gu = 0x2000 if gu else None
        a.workspace, a.workspace_bytes = 0x1000, 16
        a.grad_dtype = M.MOE_F32
        return a

    for dtype, gu, status in ((M.MOE_BF16, False, 4), (M.MOE_BF16, True, 4),
                              (M.MOE_F32, False, 1), (M.MOE_F32, True, 4)):
        dims = M.make_dims(16, 128, 8, 2, 128, dtype)
        a = args(gu)
        assert L.moe_backward(ctypes.byref(dims), ctypes.byref(a), None) == status, (dtype, gu)
    # pre-activations saved by the forward: gu must be there, and the flag is 0 or 1
    dims = M.make_dims(16, 128, 8, 2, 128, M.MOE_BF16)
    for gu, flag, status in ((False, 1, 1), (True, 1, 4), (True, 2, 2)):
        a = args(gu)
        a.gu_saved = flag
        assert L.moe_backward(ctypes.byref(dims), ctypes.byref(a), None) == status, (gu, flag)


def test_noalloc_rejects_layers_beyond_its_scratch(M):
    """moe_forward_noalloc's host checks: a layer whose workspace exceeds the static scratch
    is refused with MOE_E_SCRATCH before any HIP call; NULL args with MOE_E_NULLPTR."""
    L = M.lib()
    big = M.make_dims(100000, 128, 256, 8, 128, M.MOE_BF16)
    assert M.workspace_size(big) > M.NOALLOC_SCRATCH_BYTES
    a = M.ForwardArgs()
    assert L.moe_forward_noalloc(ctypes.byref(big), ctypes.byref(a), None) == 6
    assert L.moe_forward_noalloc(ctypes.byref(big), None, None) == 1
    bad = M.make_dims(16, 128, 8, 9, 128, M.MOE_BF16)
    assert L.moe_forward_noalloc(ctypes.byref(bad), ctypes.byref(a), None) == 2
    # the header's limit is the binding's
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)" in hdr
    assert M.NOALLOC_SCRATCH_BYTES == 64 << 20
