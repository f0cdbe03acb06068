"""The hand-issued loads of the weight-streaming GEMM, of the 256 x 256 DMA GEMM and of the
attention chunks' K/V ring, checked on the compiled gfx950 assembly (host only: hipcc
cross-compiles).  See tests/asm_waits.py for the rule."""
import os
import shutil
import subprocess

import pytest

from asm_waits import check_assembly, check_function

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_checker_flags_a_copy_before_the_wait():
    # a load, a copy of its destination before the wait that names it, then the wait
    bad = ["k:", ";;#ASMSTART", "global_load_dwordx4 v[4:7], v[0:1], off", ";;#ASMEND",
           "v_mov_b32_e32 v8, v4",
           ";;#ASMSTART", "s_waitcnt vmcnt(0) ; waits for v[4:7]", ";;#ASMEND", "s_endpgm"]
    good = bad[:4] + bad[5:8] + ["v_mov_b32_e32 v8, v4", "s_endpgm"]
    assert check_function(bad)
    assert not check_function(good)


def test_checker_flags_a_load_landing_on_a_reused_register():
    # a load whose value is never waited for, and a later write to its register
    bad = ["k:", ";;#ASMSTART", "global_load_dwordx4 v[4:7], v[0:1], off", ";;#ASMEND",
           "v_accvgpr_read_b32 v5, a3", "s_waitcnt vmcnt(0)", "s_endpgm"]
    assert check_function(bad)


def _device_assembly(tmp_path, source):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    out = tmp_path / (source + ".s")
    csrc = os.path.join(ROOT, "dflash2_block_drafter_amd", "csrc")
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", csrc, "-x", "hip", "-S",
           "--cuda-device-only", os.path.join(csrc, source), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


needs_hipcc = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                 reason="needs hipcc")


@needs_hipcc
def test_streaming_gemm_waits_cover_every_use(tmp_path):
    result = check_assembly(_device_assembly(tmp_path, "gemm.hip"), r"_ZN3dfl12_GLOBAL__N_118gemm_stream_kernel")
    assert len(result) >= 12, "streaming kernel instances not found"
    bad = {k: v[:3] for k, v in result.items() if v}
    assert not bad, bad


@needs_hipcc
def test_attention_ring_waits_cover_every_use(tmp_path):
    asm = _device_assembly(tmp_path, "attention.hip")
    result = check_assembly(asm, r"_ZN3dfl12_GLOBAL__N_117attn_chunk_kernel")
    assert len(result) == 4, "attention chunk kernel instances (D = 64, 128; rings of 1 and 3) not found"
    bad = {k: v[:3] for k, v in result.items() if v}
    assert not bad, bad


@needs_hipcc
def test_dma_gemm_fragment_reads_are_awaited(tmp_path):
    # the 256 x 256 tile kernel's LDS fragment reads are inline assembly, each tied to a wait
    asm = _device_assembly(tmp_path, "gemm.hip")
    result = check_assembly(asm, r"_ZN3dfl12_GLOBAL__N_115gemm_dma_kernel")
    assert len(result) == 2, "DMA kernel instances (tiled and row-major weights) not found"
    frag = check_assembly(asm, r"_ZN3dfl12_GLOBAL__N_120gemm_dma_frag_kernel")
    assert len(frag) == 2, "fragment-order DMA kernel instances not found"
    bad = {k: v[:3] for k, v in {**result, **frag}.items() if v}
    assert not bad, bad
