"""Code-generation invariants of the grouped GEMM (no GPU needed: hipcc
cross-compiles gfx950 assembly on the host).

The K loop issues its tile loads (LDS DMA) and row-scale loads as inline
assembly and waits for them with explicit vmcnt waits.  These tests check,
on the assembly hipcc produces for every GEMM kernel instance, that
  * from the first tile load on, no wait for vector memory was inserted by
    the compiler (one would serialise the load / multiply pipeline);
  * a register filled by an asynchronous row-scale load is neither read nor
    written by any instruction before the next vmcnt wait on every path of
    the control-flow graph (the hardware writes it when the load completes);
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
        if re.match(r"\.LBB\w+:", s):   # block labels, for the control-flow graph
            res[name].append((s.split(":")[0] + ":", False))
            continue
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


def _basic_blocks(body):
    """(label, instructions, successor labels) per basic block, in order."""
    blocks = [[None, []]]
    for s, in_asm in body:
        if s.endswith(":") and s.startswith(".LBB"):
            blocks.append([s[:-1], []])
            continue
        blocks[-1][1].append((s, in_asm))
        if not in_asm and re.match(r"s_(cbranch_\w+|branch|endpgm)\b", s):
            blocks.append([None, []])
    blocks = [b for b in blocks if b[0] is not None or b[1]]
    for i, b in enumerate(blocks):
        b[0] = b[0] or f"#{i}"
    out = []
    for i, (label, ins) in enumerate(blocks):
        last = ins[-1][0] if ins else ""
        nxt = [blocks[i + 1][0]] if i + 1 < len(blocks) else []
        m = re.match(r"s_(c?)branch\w*\s+(\.LBB\w+)", last)
        if last.startswith("s_endpgm"):
            succ = []
        elif m:
            succ = [m.group(2)] + (nxt if m.group(1) else [])
        else:
            succ = nxt
        out.append((label, ins, succ))
    return out


_SCALE_LOAD = re.compile(r"buffer_load_dword (v\d+), (v\d+), s\[\d+:\d+\], 0 offen(?! lds)")


def _scale_load_hazards(body):
    """Instructions that touch a row-scale load's register before a vmcnt
    wait, on some path: a forward dataflow over the basic blocks, the
    registers pending at a block's entry being the union over its
    predecessors (to a fixed point).  Returns (hazards, number of loads)."""
    blocks = _basic_blocks(body)
    index = {label: i for i, (label, _, _) in enumerate(blocks)}

    def run(i, pending, report):
        pending = set(pending)
        for s, _ in blocks[i][1]:
            if s.startswith("s_waitcnt") and "vmcnt" in s:
                pending = set()
                continue
            m = _SCALE_LOAD.match(s)
            if m:
                if int(m.group(2)[1:]) in pending:
                    report.append(s)
                pending.add(int(m.group(1)[1:]))
                continue
            parts = s.split(None, 1)
            if pending and len(parts) == 2 and _vregs(parts[1]) & pending:
                report.append(s)
        return pending

    entry = [set() for _ in blocks]
    reached, work = {0}, [0]
    while work:
        i = work.pop()
        out = run(i, entry[i], [])
        for lab in blocks[i][2]:
            j = index[lab]
            if j not in reached or not out <= entry[j]:
                reached.add(j)
                entry[j] |= out
                work.append(j)
    # every reachable block once more, with its final entry state
    hazards = []
    for i in sorted(reached):
        run(i, entry[i], hazards)
    n_loads = sum(1 for _, ins, _ in blocks for s, _ in ins if _SCALE_LOAD.match(s))
    return hazards, n_loads


def test_async_scale_registers_untouched_until_waited(kernels):
    n_loads = 0
    for name, body in kernels.items():
        hazards, n = _scale_load_hazards(body)
        n_loads += n
        assert not hazards, (name, hazards[:3])
    assert n_loads > 0


def test_scale_hazard_check_follows_branches():
    """The dataflow sees a hazard reached by a jump, and none across an
    unconditional branch to code that waits first."""
    load = ("buffer_load_dword v5, v1, s[4:7], 0 offen offset:0", True)
    jumped = [load, ("s_branch .LBB0_2", False), (".LBB0_1:", False),
              ("v_mov_b32_e32 v6, v5", False), ("s_endpgm", False),
              (".LBB0_2:", False), ("v_mov_b32_e32 v7, v5", False), ("s_endpgm", False)]
    hz, n = _scale_load_hazards(jumped)
    assert n == 1 and hz == ["v_mov_b32_e32 v7, v5"]
    waited = [load, ("s_cbranch_scc1 .LBB0_2", False), ("s_waitcnt vmcnt(0)", True),
              ("v_mov_b32_e32 v6, v5", False), (".LBB0_2:", False),
              ("s_waitcnt vmcnt(0)", True), ("v_mov_b32_e32 v7, v5", False)]
    assert _scale_load_hazards(waited)[0] == []
    looped = [(".LBB0_1:", False), ("v_mov_b32_e32 v7, v5", False), load,
              ("s_cbranch_scc1 .LBB0_1", False), ("s_endpgm", False)]
    assert _scale_load_hazards(looped)[0] == ["v_mov_b32_e32 v7, v5"]


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
