"""CPU: the fragment-ordered GEMM's MFMAs are inline assembly that
accumulates in place, so the compiler neither sees them as MFMAs nor inserts
the wait states the hardware needs around them. This compiles gemm_frag.hip
for gfx950 (the library's own flags) to assembly and checks, for each kind of
frag_gemm_kernel, what that relies on:
  * every MFMA is v_mfma_f32_16x16x32 with its destination equal to its
    accumulator (in place);
  * no accumulator is moved or spilled between the first and the last MFMA
    (no v_accvgpr read/write/move, no scratch access);
  * after the last MFMA comes one block of 24 wait states (three s_nop 7),
    and every other instruction reading an accumulation register comes after
    it (the epilogue's reads of the results);
  * the k-loop's 3 wait states after the accumulator zeroing are present.
"""
import os
import re
import shutil
import subprocess

import pytest

from mixture_experts_layer_49_amd import build as B

KINDS = {"0": "up_rows", "1": "up_frag", "2": "down"}


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "gemm_frag.s")
    cmd = [hipcc, *B.COMMON, "-O3", "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "gemm_frag.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def kernel_instructions(s, kind):
    m = re.search(r"(_ZN3moe12_GLOBAL__N_116frag_gemm_kernelILi%sEE\w*):" % kind, s)
    assert m, "frag_gemm_kernel<%s> not found" % KINDS[kind]
    body = s[m.end():s.index(".Lfunc_end", m.end())]
    ins = [l.split(";")[0].strip() for l in body.split("\n")]
    return [l for l in ins if l and not l.startswith(".") and not l.endswith(":")]


@pytest.mark.parametrize("kind", sorted(KINDS))
def test_inline_mfma_invariants(asm, kind):
    ins = kernel_instructions(asm, kind)
    mf = [i for i, l in enumerate(ins) if l.startswith("v_mfma")]
    assert len(mf) == 512, "expected 4 stages x 128 MFMAs in the k-loop, found %d" % len(mf)
    for i in mf:
        assert re.match(r"v_mfma_f32_16x16x32_(bf16|f16) (a\[\d+:\d+\]), v\[\d+:\d+\], v\[\d+:\d+\], \2$", ins[i]), \
            "MFMA not in place: %s" % ins[i]
    loop = ins[mf[0]:mf[-1]]
    moved = [l for l in loop if l.startswith("v_accvgpr") or "scratch_" in l]
    assert not moved, "accumulator moves or spills inside the k-loop: %s" % moved[:4]
    trip = [i for i in range(len(ins) - 2)
            if ins[i] == "s_nop 7" and ins[i + 1] == "s_nop 7" and ins[i + 2] == "s_nop 7"]
    assert len(trip) == 1 and trip[0] > mf[-1], "the wait block before the epilogue is missing or misplaced"
    readers = [i for i, l in enumerate(ins)
               if not l.startswith(("v_mfma", "v_accvgpr_write")) and re.search(r",\s*a(\d+\b|\[\d)", l)]
    assert readers, "no epilogue reads of the accumulators found"
    assert min(readers) > trip[0], "an accumulator is read before the wait block: %s" % ins[min(readers)]
    assert "s_nop 2" in ins, "the k-loop's wait states after the accumulator zeroing are missing"
