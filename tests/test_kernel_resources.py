"""Compile-time properties of the gfx950 kernels that correctness depends on.

The DMA-fed grouped GEMM waits for its own global->LDS loads with hand-placed vmcnt
counts. Scratch (register spill) traffic would share that counter, so every such kernel
must compile without scratch. Checked on the device assembly hipcc produces here."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_layer_routing_amd", "csrc")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "grouped_ffn.s"
    from moe_layer_routing_amd import _build
    cmd = [_build.HIPCC, *[f for f in _build.FLAGS if f not in ("-shared", "-fPIC")],
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S", "--cuda-device-only",
           os.path.join(CSRC, "grouped_ffn.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _kernels(asm):
    """(name, metadata block) for every kernel in the code object metadata."""
    blocks = asm.split("- .agpr_count:")[1:]
    for b in blocks:
        m = re.search(r"\.name:\s+(\S+)", b)
        yield m.group(1), b


def test_dma_gemm_kernels_have_no_scratch(gemm_asm):
    found = 0
    for name, b in _kernels(gemm_asm):
        if "grouped_gemm_dma" not in name:
            continue
        found += 1
        priv = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", b).group(1))
        spill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", b).group(1))
        assert priv == 0 and spill == 0, f"{name}: scratch {priv} B, {spill} VGPR spills"
    assert found >= 2


def test_gemm_kernels_fit_lds(gemm_asm):
    for name, b in _kernels(gemm_asm):
        lds = int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", b).group(1))
        assert lds <= 160 * 1024, name


def test_one_mfma_shape_per_dtype(gemm_asm):
    """Batch invariance rests on every bf16 GEMM using the same MFMA instruction (and every
    f32 GEMM the same f32 one)."""
    ops = set(re.findall(r"\b(v_mfma_\w+)", gemm_asm))
    assert ops == {"v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x4_f32"}, ops


def test_no_packed_fp32_arithmetic():
    """Packed FP32 add/mul/fma are kept out of every kernel."""
    from moe_layer_routing_amd import _build
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith(".hip"):
            continue
        r = subprocess.run([_build.HIPCC, *[x for x in _build.FLAGS if x not in ("-shared", "-fPIC")],
                            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S",
                            "--cuda-device-only", os.path.join(CSRC, f), "-o", "-"],
                           check=True, capture_output=True, text=True)
        assert not re.search(r"v_pk_(add|mul|fma)_f32", r.stdout), f


def _asm_of(src_name, tmp_path):
    from moe_layer_routing_amd import _build
    out = tmp_path / (src_name + ".s")
    subprocess.run([_build.HIPCC, *[f for f in _build.FLAGS if f not in ("-shared", "-fPIC")],
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S", "--cuda-device-only",
                    os.path.join(CSRC, src_name), "-o", str(out)], check=True,
                   capture_output=True)
    return out.read_text()


def test_decode_kernels_have_no_scratch(gemm_asm, tmp_path):
    """The one-block routing tail (every router variant and register width), the
    self-routing one-token gate/up GEMM and the decode-sized down GEMM + combine run on the
    decode path's critical chain; register spills there are pure latency, so they must
    compile without scratch."""
    checked = []
    for asm, key in ((_asm_of("route_tail.hip", tmp_path), "route_tail_kernel"),
                     (gemm_asm, "gate_up_self_route_kernel"),
                     (gemm_asm, "down_combine_small_kernel")):
        for name, b in _kernels(asm):
            if key not in name:
                continue
            priv = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", b).group(1))
            assert priv == 0, f"{name}: scratch {priv} B"
            checked.append(name)
    assert sum("route_tail_kernel" in n for n in checked) >= 10
    assert any("down_combine_small_kernel" in n for n in checked)
    # 4 and 8 logits per lane, one and two tokens
    assert sum("gate_up_self_route_kernel" in n for n in checked) == 4


def test_dma_ring_reads_wait_only_for_their_stage(gemm_asm):
    """The DMA GEMM kernels keep NS-2 stages of global->LDS copies in flight while the
    fragment reads of the current stage run; the hand-placed vmcnt waits order them. A
    compiler-inserted vmcnt(0) in front of a fragment read would drain the whole ring every
    stage (measured: the decode gate/up launch 39 -> 69 us), so none may appear there."""
    names = re.findall(r"^(_Z\w*(?:dma128_kernel|self_route_kernel)\w*):", gemm_asm, re.M)
    assert len(names) >= 20
    for n in names:
        body = re.search("^" + n + r":[^\n]*\n(.*?)^\s*s_endpgm", gemm_asm, re.S | re.M).group(1)
        lines = body.splitlines()
        for i, line in enumerate(lines):
            if "s_waitcnt vmcnt(0)" in line:
                nxt = " ".join(lines[i + 1:i + 3])
                assert "ds_read" not in nxt, f"{n}: vmcnt(0) before a fragment read"
