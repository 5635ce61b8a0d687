"""A model of the 8-wave GEMM kernel's copy and read schedule, one per B
layout, and the copy waits it needs -- checked against the waits hipcc
emitted for every instantiation (CPU only: hipcc cross-compiles).

The rules are the stage rules of "Two Waves, One Stage Apart: Warp-Pipelining
Triton GEMMs on AMD Instinct" (sections "Two Waves, One Stage Apart" and
"Dependencies Cross Groups and Iterations", Figure 10).  Group B runs one
stage behind group A, so the barrier that ends A's stage n-1 ends B's stage
n-2.  Then:

* copy -> read: an LDS half read in stage R is copied by every wave, and each
  wave's share must have landed by the wave's own wait at the end of stage
  R-2 (the leading group enters R when the trailing group has finished R-2);
* read -> refill: a wave's reads of stage R are complete at the end of R
  (lgkmcnt(0)), so a copy may overwrite that half from stage R+2 on.

Each wave copies its share of a 16 KiB half with 2 loads, and vmcnt retires
in issue order: the wait at the end of a memory stage may leave at most as
many loads outstanding as the wave issued after the newest load that some
later read, due by then, depends on.  The model lists, per layout, which
halves each memory stage reads (for the next stage) and copies (two K-steps
ahead), derives the largest safe count for each wait, checks every refill's
distance, and compares the counts with the compiled loop's.  The 4-wave
within-wave interleaved kernel (all waves in step, two barriers per K-step)
gets the same treatment at the end of the file.
"""
import os
import re

import pytest

from matrix_core_scheduling_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not found")

PIECES = 2          # loads per wave per half

# Memory stages of K-step t: S1 and S3 (S0 and S2 are the MFMA stages).
# reads: (half, step offset); b0 given K x N is read in two k-slices.
# copies: halves copied for step t + 2, in issue order.
SCHEDULES = {
    "B N x K": {1: {"reads": [("b1", 0)], "copies": ["a0", "a1"]},
                3: {"reads": [("a0", 1), ("a1", 1), ("b0", 1)], "copies": ["b0", "b1"]}},
    "B K x N": {1: {"reads": [("b1", 0), ("b0", 1)], "copies": ["b0", "a0", "a1"]},
                3: {"reads": [("a0", 1), ("a1", 1), ("b0", 1)], "copies": ["b1"]}},
}


def stage_index(t, s):
    return 4 * t + s


def simulate(sched, steps=10):
    """(issue list [(half, step, stage)], reads [(half, step, stage)]) of a
    run of `steps` K-steps, the prologue's copies (steps 0 and 1, in the
    steady-state order) at stage -1."""
    order = sched[1]["copies"] + sched[3]["copies"]
    issues = [(h, u, -1) for u in (0, 1) for h in order for _ in range(PIECES)]
    reads = []
    for t in range(steps):
        for s in (1, 3):
            g = stage_index(t, s)
            reads += [(h, t + d, g) for h, d in sched[s]["reads"]]
            issues += [(h, t + 2, g) for h in sched[s]["copies"] for _ in range(PIECES)]
    # the prologue's reads of step 0's a0, a1, b0 stand for S3 of step -1
    reads += [(h, 0, stage_index(-1, 3)) for h in ("a0", "a1", "b0")]
    return issues, reads


def max_wait(issues, reads, end_stage):
    """Largest vmcnt allowed at the end of stage `end_stage`: for every read in
    stage end_stage + 2, the loads issued after its half's newest load up to
    the end of end_stage may stay outstanding, no more."""
    issued = [i for i, x in enumerate(issues) if x[2] <= end_stage]
    last = issued[-1]
    bound = None
    for h, u, g in reads:
        if g != end_stage + 2:
            continue
        newest = max(i for i, x in enumerate(issues) if x[0] == h and x[1] == u)
        assert newest <= last, f"{h}({u}) read in stage {g} is copied after stage {end_stage}"
        n = last - newest
        bound = n if bound is None else min(bound, n)
    return bound


def refill_distances(issues, reads):
    """For every copy of half h for step u, the stages since the last read of
    the half's previous occupant (h, u - 2) in the same buffer."""
    out = []
    for h, u, g in issues:
        prev = [rg for rh, ru, rg in reads if rh == h and ru == u - 2]
        if prev:
            out.append((h, u, g - max(prev)))
    return out


@pytest.mark.parametrize("layout", sorted(SCHEDULES))
def test_model_refills_wait_two_stages(layout):
    issues, reads = simulate(SCHEDULES[layout])
    short = [x for x in refill_distances(issues, reads) if x[2] < 2]
    assert not short, short


@pytest.mark.parametrize("layout", sorted(SCHEDULES))
def test_model_every_read_finds_its_copy_a_stage_ahead(layout):
    """No half is read before its copy could have been waited for (the wait
    can only sit at the end of an earlier memory stage)."""
    issues, reads = simulate(SCHEDULES[layout])
    for h, u, g in reads:
        if g < 0:
            continue                      # the prologue's own reads: it waits for them itself
        first = min(x[2] for x in issues if x[0] == h and x[1] == u)
        assert first <= g - 2, (h, u, g, first)


def model_waits(layout):
    """(S1 end, S3 end, prologue: before the first reads, at the end of S3 of
    step -1) counts from the steady state of the model."""
    issues, reads = simulate(SCHEDULES[layout])
    t = 4
    s1 = max_wait(issues, reads, stage_index(t, 1))
    s3 = max_wait(issues, reads, stage_index(t, 3))
    # prologue: all 16 loads issued; the first wait covers step 0's a0, a1, b0
    # (read at once), the second the reads of S1 of step 0
    pro = [i for i, x in enumerate(issues) if x[2] == -1]
    newest0 = max(i for i, x in enumerate(issues) if x[1] == 0 and x[0] in ("a0", "a1", "b0"))
    first = pro[-1] - newest0
    second = max_wait(issues, reads, -1)
    return s1, s3, first, second


def test_model_counts():
    """The counts the kernel's comments derive: B N x K ends S1 with 6 (b0 is
    copied in S3) and S3 with 8; B K x N ends S1 with 8 and S3 with 6 (b0
    copied first in S1, k-slice 0 of the next b0 read early); both prologues
    wait with 10 before reading step 0's a0, a1 and b0, then with S3's count
    (the state at the end of S3 of step -1)."""
    assert model_waits("B N x K") == (6, 8, 10, 8)
    assert model_waits("B K x N") == (8, 6, 10, 6)


def loop_lines(asm_text, fn):
    """The instruction lines of the innermost loop of function `fn`."""
    lines = asm_text.splitlines()
    i = next(n for n, l in enumerate(lines) if l.startswith(fn + ":"))
    out, inside = [], False
    for l in lines[i + 1:]:
        if "s_endpgm" in l:
            break
        if re.match(r"^(\.LBB\w+|; %bb\.\d+):", l):
            inside = "Loop Header" in l or "in Loop:" in l
            continue
        t = l.strip()
        if inside and t and not t.startswith((";", ".")):
            out.append(t)
    return out


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("sched")
    return open(build.device_asm("gemm_pipelined.hip", str(d / "p.s"))).read()


def test_compiled_waits_match_the_model(asm):
    """In every instantiation's loop, the memory stage with fewer LDS reads is
    S1 and the other S3; the vmcnt each ends with equals the model's largest
    safe count for its layout (a smaller count would only wait longer, a
    larger one would race)."""
    fns = re.findall(r"^(_Z\w*gemm_pipelined_kernel\w*):", asm, re.M)
    assert len(fns) == 20
    for fn in fns:
        trans_b = int(re.search(r"kernelILi\dELb(\d)E", fn).group(1))
        s1, s3, _, _ = model_waits("B N x K" if trans_b else "B K x N")
        ops = loop_lines(asm, fn)
        # stages cut at the barriers; the loop is a cycle
        stages, cur = [], []
        for o in ops:
            if o.startswith("s_barrier"):
                stages.append(cur)
                cur = []
            else:
                cur.append(o)
        stages[0] = cur + stages[0]
        mem = [st for st in stages if any(o.startswith("buffer_load") for o in st)]
        assert len(mem) == 4, fn
        for st in mem:
            reads = sum(o.startswith("ds_read") for o in st)
            vm = [int(m) for o in st for m in re.findall(r"vmcnt\((\d+)\)", o)]
            assert len(vm) == 1, (fn, vm)
            want = s1 if reads == min(sum(o.startswith("ds_read") for o in x) for x in mem) else s3
            assert vm[0] == want, f"{fn}: memory stage with {reads} reads waits vmcnt({vm[0]}), model {want}"


# ---- the 4-wave within-wave interleaved kernel ------------------------------
# One wave per SIMD, all waves in step: every barrier is passed by all waves
# together, each wave having waited for its own copies (vmcnt) and reads
# (lgkmcnt(0)) first.  Per K-step s two segments, each opened by a barrier:
# after the top barrier clusters c00 and c01 read B1 and A1 of step s and copy
# A0 and B0 of step s + 2; after the middle barrier c10 and c11 read A0 and B0
# of step s + 1 and copy B1 and A1 of step s + 2.  Each wave copies its share
# of a half with 4 loads (4 waves).
PIECES4 = 4
SEGMENTS4 = [  # (reads (half, step offset), copies (halves for step + 2, in issue order))
    ([("b1", 0), ("a1", 0)], ["a0", "b0"]),
    ([("a0", 1), ("b0", 1)], ["b1", "a1"]),
]


def simulate4(steps=10):
    """(issues [(half, step, segment)], reads [(half, step, segment)]); segment
    2s + k follows the k-th barrier of step s; the prologue's copies (steps 0
    and 1 in the steady-state order) are segment -1."""
    order = SEGMENTS4[0][1] + SEGMENTS4[1][1]
    issues = [(h, u, -1) for u in (0, 1) for h in order for _ in range(PIECES4)]
    reads = []
    for s in range(steps):
        for k, (rd, cp) in enumerate(SEGMENTS4):
            g = 2 * s + k
            reads += [(h, s + d, g) for h, d in rd]
            issues += [(h, s + 2, g) for h in cp for _ in range(PIECES4)]
    return issues, reads


def max_wait4(issues, reads, seg):
    """Largest vmcnt allowed at the barrier that opens segment `seg`: the reads
    of that segment need every load of their halves issued before it."""
    last = max(i for i, x in enumerate(issues) if x[2] < seg)
    bound = None
    for h, u, g in reads:
        if g != seg:
            continue
        newest = max(i for i, x in enumerate(issues) if x[0] == h and x[1] == u)
        assert newest <= last, f"{h}({u}) read in segment {g} before its copy"
        bound = last - newest if bound is None else min(bound, last - newest)
    return bound


def test_model4_refills_follow_a_barrier():
    """A copy overwrites a half only in a segment after the one that last read
    its previous occupant (that read completed before the barrier between)."""
    issues, reads = simulate4()
    for h, u, g in issues:
        prev = [rg for rh, ru, rg in reads if rh == h and ru == u - 2]
        if prev:
            assert g > max(prev), (h, u, g, max(prev))


def test_model4_counts():
    issues, reads = simulate4()
    assert {max_wait4(issues, reads, seg) for seg in range(8, 12)} == {16}


def test_compiled_waits_match_the_model_4wave(tmp_path):
    """Every wait in the 4-wave kernel's loops is the model's count."""
    want = {max_wait4(*simulate4(), seg) for seg in range(8, 12)}
    text = open(build.device_asm("gemm_interleaved.hip", str(tmp_path / "i.s"))).read()
    fns = re.findall(r"^(_Z\w*gemm_interleaved_kernel\w*):", text, re.M)
    assert len(fns) == 10
    for fn in fns:
        vm = {int(m) for o in loop_lines(text, fn) for m in re.findall(r"vmcnt\((\d+)\)", o)}
        assert vm == want, f"{fn}: loop waits vmcnt{sorted(vm)}, model {sorted(want)}"


# ---- the attention forward kernel's trips -----------------------------------
# Two stages per trip i: M (both products; reads V(i) and K(i+2) among the
# MFMAs; copies K(i+4) and V(i+2), 2 loads each per wave; ends with a vmcnt
# wait) and V (the softmax; ends with lgkmcnt(0)).  K blocks and V blocks
# live in two rings of four slots.  Group B runs one stage behind group A,
# as in the GEMM: a block read by the leading group in stage R needs the
# trailing group's copies waited at the end of its stage R - 2, and reads
# issued in an M stage complete at the end of the V stage after it, so a
# slot may be refilled from three stages after the reading M stage on.
RING = 4


def simulate_attention(trips=12):
    issues, reads = [], []          # (ring, block, stage)
    for i in range(trips):
        g = 2 * i                    # M stage of trip i
        reads += [("V", i, g), ("K", i + 2, g)]
        issues += [("K", i + 4, g)] * 2 + [("V", i + 2, g)] * 2
    return issues, reads


def test_attention_model_wait_and_ring_distances():
    issues, reads = simulate_attention()
    # copy -> read: the wait at the end of the M stage of trip i covers the
    # reads of the M stage of trip i + 1
    for i in range(3, 9):
        end = 2 * i
        last = max(n for n, x in enumerate(issues) if x[2] <= end)
        need = [max(n for n, x in enumerate(issues) if x[:2] == r[:2]) for r in reads if r[2] == end + 2]
        assert min(last - n for n in need) == 4
    # read -> refill: block j's slot (j mod 4) is refilled by block j + 4
    for ring, j, g in issues:
        prev = [rg for rr, rj, rg in reads if rr == ring and rj == j - RING]
        if prev:
            assert g - max(prev) >= 3, (ring, j, g, max(prev))


def test_attention_trip_loops_wait_as_modelled():
    """Every trip loop of the 8-wave attention kernel waits vmcnt(4) (once, at
    the end of its M stage) and lgkmcnt(0) at the end of its V stage."""
    import tempfile
    from tests.test_kernel_isa import loops
    with tempfile.TemporaryDirectory() as d:
        text = open(build.device_asm("attention_fwd.hip", os.path.join(d, "a.s"))).read()
    seen = 0
    for (fn, hdr), lines in loops(text, full=True).items():
        if "attention_fwd_kernel" not in fn:
            continue
        vm = [int(m) for l in lines for m in re.findall(r"vmcnt\((\d+)\)", l)]
        assert vm == [4], f"{fn} {hdr}: vmcnt {vm}"
        assert any(re.search(r"lgkmcnt\(0\)", l) for l in lines), (fn, hdr)
        seen += 1
    assert seen == 16        # 8 instantiations x (unmasked, masked) trip loops
