"""Code-generation invariants of the grouped GEMM (no GPU needed: hipcc
cross-compiles gfx950 assembly on the host).

The K loop issues its tile loads (LDS DMA) and row-scale loads as inline
assembly and waits for them with explicit vmcnt waits.  These tests check,
on the assembly hipcc produces for every GEMM kernel instance, that
  * from the first tile load on, no wait for vector memory was inserted by
    the compiler (one would serialise the load / multiply pipeline);
  * a register filled by an asynchronous row-scale load is neither read nor
    written by any instruction before the next vmcnt wait (the hardware
    writes it when the load completes);
  * M0, which the DMA sequence sets, is not used by any compiler-generated
    instruction.
  * no kernel spills registers to scratch memory.
"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
SRC = os.path.join(ROOT, "fp8_routed_expert_amd", "csrc", "gemm.hip")
KERNEL = re.compile(r"^(_ZN3moe23grouped_gemm_fp8_kernel\w*):")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    out = tmp_path_factory.mktemp("gemm_asm") / "gemm.s"
    cmd = [HIPCC, "-mllvm", "-amdgpu-mfma-vgpr-form", "--offload-arch=gfx950", "-O3",
           "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "fp8_routed_expert_amd", "csrc"),
           "--cuda-device-only", "-S", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    # kernel name -> list of (line, inside inline asm)
    res, name, in_asm = {}, None, False
    for line in out.read_text().split("\n"):
        m = KERNEL.match(line)
        if m:
            name = m.group(1)
            res[name] = []
            in_asm = False
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            name = None
            continue
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif s and not s.startswith(";") and not s.startswith("."):
            res[name].append((s, in_asm))
    assert len(res) >= 10, "expected every tile configuration and projection"
    return res


def _vregs(operands):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]|\bv(\d+)\b", operands):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def test_no_compiler_inserted_vmcnt_waits(kernels):
    """From the first tile load on (the tile lookup before it reads the
    segment table with ordinary loads and waits for them)."""
    for name, body in kernels.items():
        started, extra = False, []
        for s, in_asm in body:
            if re.match(r"buffer_load_dwordx4 .* lds$", s):
                started = True
            elif started and s.startswith("s_waitcnt") and "vmcnt" in s and not in_asm:
                extra.append(s)
        assert started, name
        assert not extra, (name, extra[:3])


def test_async_scale_registers_untouched_until_waited(kernels):
    n_loads = 0
    for name, body in kernels.items():
        pending = set()
        for s, in_asm in body:
            if s.startswith("s_waitcnt") and "vmcnt" in s:
                pending = set()
                continue
            m = re.match(r"buffer_load_dword (v\d+), (v\d+), s\[\d+:\d+\], 0 offen(?! lds)", s)
            if m:
                n_loads += 1
                assert int(m.group(2)[1:]) not in pending, (name, s)
                pending.add(int(m.group(1)[1:]))
                continue
            parts = s.split(None, 1)
            if pending and len(parts) == 2:
                hit = _vregs(parts[1]) & pending
                assert not hit, (name, s, sorted(hit))
    assert n_loads > 0


def test_m0_used_only_by_the_dma_sequence(kernels):
    for name, body in kernels.items():
        outside = [s for s, in_asm in body if re.search(r"\bm0\b", s) and not in_asm]
        assert not outside, (name, outside[:3])


def test_no_register_spills(kernels):
    """Every kernel instance fits its registers: a spill would put private
    (scratch) memory traffic, and waits for it, into the K loop."""
    for name, body in kernels.items():
        spills = [s for s, _ in body if s.startswith("scratch_")]
        assert not spills, (name, spills[:3])
