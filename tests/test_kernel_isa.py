"""Checks on the compiled gfx950 code of the 256 x 256 main loop (CPU only: hipcc -S).

The 16 x 16 main loop issues its MFMAs as assembly statements, so the compiler
neither schedules them nor guards their hazards. These tests compile the kernel
source to AMD assembly and check what that design relies on:

- one basic block per trip of two k-steps, holding all 128 MFMAs, with no
  accumulator copies and no scratch traffic;
- no wait that drains every load (vmcnt(0)) inside the loop;
- hazard distances: a VALU write of a register reaches an MFMA that reads it
  only after many issue slots, and an MFMA result reaches any non-MFMA reader
  only after at least the 19 wait states the longest MFMA needs.
"""

import os
import re
import shutil
import subprocess

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(REPO, "persistent_tiled_gemm_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not installed")

# enough for any MFMA result latency on this part (the 32-pass forms need 19)
MIN_MFMA_RESULT_DISTANCE = 19
# a VALU write feeding an MFMA operand needs a few wait states; demand far more
MIN_VALU_TO_MFMA_DISTANCE = 16


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "gemm_kernel.s"
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(REPO, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, "gemm_kernel.hip")]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def kernel_lines(asm_text, mode, grouped, bt=False):
    name = (f"_ZN3ptg15ptg_gemm_kernelILi256ELi256ELi{mode}ELb{1 if grouped else 0}ELb{1 if bt else 0}"
            "EEEvNS_10KernelArgsE")
    i = asm_text.index(name + ":")
    j = asm_text.index(".Lfunc_end", i)
    return asm_text[i:j]


def instructions(block):
    return [x.strip() for x in block.splitlines()
            if x.strip() and not x.strip().startswith((";", ".")) and not x.strip().endswith(":")]


def regs(operand):
    operand = operand.strip().split()[0] if operand.strip() else ""
    m = re.match(r"([va])\[(\d+):(\d+)\]", operand)
    if m:
        return {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", operand)
    return {(m.group(1), int(m.group(2)))} if m else set()


def operands(line):
    return line.split(None, 1)[1].split(", ") if " " in line else []


def slots(line):
    op = line.split()[0]
    return int(line.split()[1]) + 1 if op == "s_nop" else 1


CASES = [(m, g) for m in (0, 1, 2) for g in (False, True)]
# the B^T (N x K) form of the kernel, single GEMMs, every mode
BT_CASES = [(m, False) for m in (0, 1, 2)]
ALL_CASES = [(m, g, False) for m, g in CASES] + [(m, g, True) for m, g in BT_CASES]


def loop_blocks(text, split_asm_labels=False):
    pattern = r"\n(?:\.LBB\d+_\d+|\d+):" if split_asm_labels else r"\n\.LBB\d+_\d+:"
    blocks = re.split(pattern, text)
    return [instructions(b) for b in blocks if sum(1 for x in instructions(b) if x.startswith("v_mfma_f32_16x16")) > 0]


# each run of the loop has three forms: four-step trips with load offsets computed once per tile
# and compile-time stages, two-step trips with the same offsets, and two-step K-tail trips; the
# dynamic scheduler runs the loop in two parts and claims in between
def expected_loops(mode):
    return 6 if mode == 2 else 3


@pytest.mark.parametrize("mode,grouped,bt", ALL_CASES)
def test_main_loop_is_one_block_without_copies(asm, mode, grouped, bt):
    loops = loop_blocks(kernel_lines(asm, mode, grouped, bt))
    assert len(loops) == expected_loops(mode), "the 16 x 16 MFMAs of a trip sit in more than one basic block"
    for body in loops:
        mfma = sum(1 for x in body if x.startswith("v_mfma_f32_16x16x32_bf16"))
        assert mfma in (128, 256), mfma  # 64 per k-step, two or four k-steps per trip
        steps = mfma // 64
        assert not [x for x in body if x.startswith(("v_accvgpr_read", "v_accvgpr_write", "v_accvgpr_mov"))]
        assert not [x for x in body if x.startswith("scratch_")]
        assert not [x for x in body if x.startswith("s_waitcnt") and "vmcnt(0)" in x]
        # four LDS stages: the end-of-step waits leave two steps of loads in flight
        assert sum(1 for x in body if x.startswith("s_waitcnt") and "vmcnt(16)" in x) == steps
        assert sum(1 for x in body if x.startswith("s_barrier")) == steps
    assert sum(1 for body in loops if sum(1 for x in body if x.startswith("v_mfma")) == 256) == expected_loops(mode) // 3


@pytest.mark.parametrize("mode,grouped,bt", ALL_CASES)
def test_main_loop_has_no_claim_branch_or_exec_write(asm, mode, grouped, bt):
    """A branch or an EXEC write inside a k-step holds the wave until the MFMAs in
    flight drain (measured 70-90 cycles per step), so a trip's only branch is its
    back edge and nothing in it writes EXEC or sends an atomic."""
    loops = loop_blocks(kernel_lines(asm, mode, grouped, bt), split_asm_labels=True)
    assert len(loops) == expected_loops(mode)
    for body in loops:
        # the trip ends at its back edge (the block's text may run on past it)
        ends = [n for n, x in enumerate(body) if x.startswith(("s_cbranch", "s_branch", "s_setpc"))]
        assert ends, "no back edge"
        body = body[: ends[0] + 1]
        assert sum(1 for x in body if x.startswith("v_mfma_f32_16x16x32_bf16")) in (128, 256)
        assert not [x for x in body if "exec" in x.split(",")[0] or x.startswith("s_and_saveexec")]
        assert not [x for x in body if x.startswith(("global_atomic", "buffer_atomic", "flat_atomic"))]


@pytest.mark.parametrize("mode,grouped,bt", ALL_CASES)
def test_mfma_hazard_distances(asm, mode, grouped, bt):
    f = instructions(kernel_lines(asm, mode, grouped, bt))
    mf = [n for n, x in enumerate(f) if x.startswith("v_mfma")]
    # VALU write -> MFMA operand read, over the loop and its back edge
    body = f[mf[0] - 64: mf[-1] + 32] * 2
    last_valu, pos, worst = {}, 0, None
    for x in body:
        pos += slots(x)
        op, ops = x.split()[0], operands(x)
        if op.startswith("v_mfma"):
            for r in ops[1:4]:
                for reg in regs(r):
                    if reg in last_valu:
                        d = pos - last_valu[reg]
                        worst = d if worst is None else min(worst, d)
            for reg in regs(ops[0]):
                last_valu.pop(reg, None)
        elif op.startswith(("ds_read", "buffer_load", "global_load", "global_atomic")) and ops:
            for reg in regs(ops[0]):
                last_valu.pop(reg, None)
        elif op.startswith("v_") and not op.startswith(("v_cmp", "v_readfirstlane", "v_readlane")) and ops:
            for reg in regs(ops[0]):
                last_valu[reg] = pos
    assert worst is None or worst >= MIN_VALU_TO_MFMA_DISTANCE, worst
    # MFMA result -> any other reader, from the loop to the end of the kernel
    last_mfma, pos, worst = {}, 0, None
    for x in f[mf[0]:]:
        pos += slots(x)
        op, ops = x.split()[0], operands(x)
        if op.startswith("v_mfma"):
            for reg in regs(ops[0]):
                last_mfma[reg] = pos
            continue
        if op.startswith("s_") or not ops:
            continue
        store = op.startswith(("global_store", "buffer_store", "flat_store", "ds_write"))
        for r in (ops if store else ops[1:]):
            for reg in regs(r):
                if reg in last_mfma:
                    d = pos - last_mfma[reg]
                    worst = d if worst is None else min(worst, d)
        if not store:
            for reg in regs(ops[0]):
                last_mfma.pop(reg, None)
    assert worst is None or worst >= MIN_MFMA_RESULT_DISTANCE, worst


@pytest.mark.parametrize("mode,grouped,bt", ALL_CASES)
def test_fast_trips_compute_no_load_masks(asm, mode, grouped, bt):
    """Vector instructions interleaved with the MFMAs stall them (recomputing the load masks every
    k-step cost about 220 cycles per step; the LDS read address adds about 80 more), so the
    four-step trips, whose stages are compile-time constants, hold no vector instruction besides
    the MFMAs, and the two-step trips with precomputed load offsets at most 24 (the K-tail trips
    carry about 56)."""
    valu = []
    for body in loop_blocks(kernel_lines(asm, mode, grouped, bt)):
        ends = [n for n, x in enumerate(body) if x.startswith(("s_cbranch", "s_branch"))]
        body = body[: ends[0] + 1]
        mfma = sum(1 for x in body if x.startswith("v_mfma"))
        valu.append((mfma, sum(1 for x in body if x.startswith("v_") and not x.startswith("v_mfma"))))
    runs = expected_loops(mode) // 3
    assert sorted(v for m, v in valu if m == 256) == [0] * runs, valu
    two = sorted(v for m, v in valu if m == 128)
    assert len(two) == 2 * runs and all(v <= 24 for v in two[:runs]) and all(v > 24 for v in two[runs:]), valu


def test_no_kernel_uses_scratch(asm):
    """No kernel of the library spills to scratch memory, in its main loop or anywhere else (a
    spilled epilogue made the 256 x 256 tile several percent slower)."""
    sizes = re.findall(r"\.amdhsa_kernel (\S+).*?\.amdhsa_private_segment_fixed_size (\d+)", asm, re.S)
    assert len(sizes) >= len(ALL_CASES)
    assert not [k for k, s in sizes if int(s) != 0]


@pytest.mark.parametrize("mode,grouped,bt", ALL_CASES)
def test_epilogue_stages_accumulators_through_lds(asm, mode, grouped, bt):
    """The epilogue of a whole tile writes each accumulator quad to LDS straight from its AGPRs
    (two passes of 32 quads per wave, no copies through VGPRs) and stores C in whole rows."""
    body = instructions(kernel_lines(asm, mode, grouped, bt))
    agpr_writes = [x for x in body if x.startswith("ds_write_b128") and ", a[" in x]
    assert len(agpr_writes) == 64
    assert not [x for x in body if x.startswith("v_accvgpr_read")]


@pytest.mark.parametrize("mode,grouped,bt", ALL_CASES)
def test_loads_are_spread_over_the_step(asm, mode, grouped, bt):
    """The direct-to-LDS loads of a k-step sit apart from each other in the MFMA stream (one every
    seven MFMAs): loads bunched together hold the MFMA stream (measured 392k against 302k cycles
    per 8192^3 tile with all eight of a step after its first MFMA)."""
    for body in loop_blocks(kernel_lines(asm, mode, grouped, bt), split_asm_labels=True):
        mfma_seen = 0
        last_load_at = None
        gaps = []
        for x in body:
            if x.startswith("v_mfma"):
                mfma_seen += 1
            elif x.startswith("buffer_load_dwordx4") and x.endswith("lds"):
                if last_load_at is not None:
                    gaps.append(mfma_seen - last_load_at)
                last_load_at = mfma_seen
        assert gaps and min(gaps) >= 6, gaps
