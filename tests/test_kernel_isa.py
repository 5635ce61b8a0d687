"""The main loops of the 256x256 kernels, read from the gfx950 assembly hipcc
emits for them (CPU only: hipcc cross-compiles).

Every loop of every instantiation must keep its accumulators and fragments
where they are (no v_accvgpr_read/write/mov copies: the register allocator
has rotated the 4-wave kernel's 256 accumulators through copies after
unrelated source changes, which costs several percent and shows in no
correctness test), use no scratch memory, and issue the MFMA and barrier
counts the schedule defines.  Per loop iteration the 8-wave kernel runs two
K-steps (8 barriers), the 4-wave kernel one (2 barriers), the 128x128-tile
kernel one (1 barrier; FP8: two); a 128-byte K-step is 64 FP16/BF16 MFMAs
16x16x32 or 32 FP8 MFMAs 16x16x128 per wave in the 8-wave kernel, twice
that in the 4-wave kernel and half of it in the 128x128-tile kernel.  The
attention kernel's trips run 64 MFMAs (QK and PV of one 64-key block) and 4
barriers.  No kernel of these files uses scratch memory at all.

The race-stress build of the same files (MCS_STAGGER) must keep every loop
as it is -- the same MFMAs, barriers and no copies or scratch -- and add one
sleep loop on each side of every barrier, while the product build has no
sleep at all.
"""
import os
import re
import shutil
import subprocess

import pytest

from matrix_core_scheduling_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not found")

# kernel -> (MFMAs per loop iteration for FP16/BF16, for FP8, barriers per iteration for each,
#            instantiations)
EXPECT = {"gemm_pipelined_kernel": (128, 64, 8, 8, 20), "gemm_interleaved_kernel": (128, 64, 2, 2, 10),
          "gemm_tile128_kernel": (32, 32, 1, 2, 10), "attention_fwd_kernel": (64, None, 2, None, 8)}
SOURCES = {"gemm_pipelined_kernel": "gemm_pipelined.hip", "gemm_interleaved_kernel": "gemm_interleaved.hip",
           "gemm_tile128_kernel": "gemm_tile128.hip", "attention_fwd_kernel": "attention_fwd.hip"}


def loops(asm: str, innermost: bool = True, full: bool = False):
    """{(kernel symbol, loop header): [instruction mnemonics]} of every loop
    (with innermost, only loops that hold no other loop: the main loops; a
    persistent kernel's loop over its tiles holds them); with full, whole
    instruction lines instead of mnemonics."""
    out, fn, cur, outer = {}, None, None, set()
    lines = asm.splitlines()
    for n, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn, cur = m.group(1), None
            continue
        if re.match(r"^(\.LBB\w+|; %bb\.\d+):", line):
            if "Parent Loop" in line and n + 1 < len(lines):
                line = line + lines[n + 1]       # a nested loop's header: "Loop Header" on the next line
            h = re.search(r"Loop Header", line)
            i = re.search(r"in Loop: Header=(BB\w+)", line)
            cur = (fn, line.split(":")[0].lstrip(".L")) if h else ((fn, i.group(1)) if i else None)
            if h and "Inner Loop Header" not in line:
                outer.add(cur)
            continue
        t = line.strip()
        if cur and fn and t and not t.startswith((";", ".")):
            out.setdefault(cur, []).append(t if full else t.split()[0])
    return {k: v for k, v in out.items() if not (innermost and k in outer)}


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa")
    return {k: open(build.device_asm(src, str(d / (src + ".s")))).read() for k, src in SOURCES.items()}


@pytest.fixture(scope="module")
def stagger_asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa_stagger")
    return {k: open(build.device_asm(src, str(d / (src + ".s")), ["-DMCS_STAGGER=1"])).read()
            for k, src in SOURCES.items()}


SLEEP_LOOP = ["s_cmp_eq_u32", "s_cbranch_scc1", "0:", "s_sleep", "s_sub_u32", "s_cmp_lg_u32", "s_cbranch_scc1",
              "1:"]


def _strip_sleeps(ops):
    """The loop's mnemonics without the race-stress sleep loops (one inline asm
    statement each, local labels 0 and 1 included)."""
    out, i = [], 0
    while i < len(ops):
        if ops[i:i + len(SLEEP_LOOP)] == SLEEP_LOOP:
            i += len(SLEEP_LOOP)
            continue
        out.append(ops[i])
        i += 1
    return out


@pytest.mark.parametrize("kernel", sorted(EXPECT))
def test_main_loops(asm, kernel):
    check_loops(asm[kernel], kernel)


@pytest.mark.parametrize("kernel", sorted(EXPECT))
def test_race_stress_build_keeps_the_loops(asm, stagger_asm, kernel):
    assert "s_sleep" not in asm[kernel]
    n = check_loops(stagger_asm[kernel], kernel, strip=True)
    assert n > 0
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", stagger_asm[kernel])
    assert sizes and all(int(x) == 0 for x in sizes), sizes


def check_loops(text, kernel, strip=False):
    """Check every main loop of `kernel` in `text`; return the number of sleeps seen."""
    found = loops(text)
    sleeps = 0
    per_fn = {}
    for (fn, hdr), ops in found.items():
        if kernel not in fn:
            continue
        per_fn.setdefault(fn, []).append((hdr, ops))
    # one symbol per instantiation: 2 element types x 2 B layouts x 2 outputs (+ FP8 N x K x 2 outputs),
    # times offset/in-phase for the 8-wave kernel; attention: 2 types x causal or not x offset or not
    f16_mfma, f8_mfma, f16_bars, f8_bars, count = EXPECT[kernel]
    assert len(per_fn) == count, sorted(per_fn)
    for fn, ls in per_fn.items():
        fp8 = "ILi2E" in fn
        for hdr, ops in ls:
            where = f"{fn} loop {hdr}"
            if strip:
                bars = ops.count("s_barrier")
                sleeps += ops.count("s_sleep")
                assert ops.count("s_sleep") == 2 * bars, f"{where}: {ops.count('s_sleep')} sleeps, {bars} barriers"
                ops = _strip_sleeps(ops)
            copies = [o for o in ops if o.startswith("v_accvgpr_")]
            assert not copies, f"{where}: {len(copies)} accumulator copies"
            assert not [o for o in ops if o.startswith("scratch_") or o.startswith("buffer_store")], where
            assert sum(o.startswith("v_mfma") for o in ops) == (f8_mfma if fp8 else f16_mfma), where
            assert ops.count("s_barrier") == (f8_bars if fp8 else f16_bars), where
    return sleeps


@pytest.mark.parametrize("kernel", sorted(EXPECT))
def test_no_scratch_anywhere(asm, kernel):
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm[kernel])
    assert sizes and all(int(x) == 0 for x in sizes), sizes
    assert not re.findall(r"\.vgpr_spill_count:\s+[1-9]", asm[kernel])


@pytest.mark.parametrize("kernel", sorted(EXPECT))
def test_m0_only_in_the_copy_asm(asm, kernel):
    """The copies set M0 (the LDS destination of buffer_load ... lds) inside
    their inline assembly.  The compiler treats M0 as reserved and may ignore
    the clobber, so no compiler-generated instruction may read or write M0:
    every mention of m0 must sit between ASMSTART and ASMEND."""
    inside, stray = False, []
    for line in asm[kernel].splitlines():
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
        elif t.startswith(";;#ASMEND"):
            inside = False
        elif not inside and not t.startswith(";") and re.search(r"\bm0\b", t):
            stray.append(t)
    assert not stray, stray[:5]



def test_pipelined_lds_reads_per_layout(asm):
    """LDS reads per two K-steps of the 8-wave kernel: with B given N x K (4 x 2
    waves) 48 ds_read_b128; with B given K x N (2 x 4 waves) 32 ds_read_b128
    for A and 32 transposing ds_read_b64_tr_b16 for B -- 64 reads where the
    4 x 2 layout would issue 16 + 64."""
    seen = set()
    for (fn, hdr), ops in loops(asm["gemm_pipelined_kernel"]).items():
        if "gemm_pipelined_kernel" not in fn:
            continue
        m = re.search(r"kernelILi(\d)ELb(\d)E", fn)
        elem, trans_b = int(m.group(1)), int(m.group(2))
        b128, tr = ops.count("ds_read_b128"), ops.count("ds_read_b64_tr_b16")
        want = (48, 0) if trans_b else (32, 32)
        assert (b128, tr) == want, f"{fn}: {b128} b128 + {tr} tr reads, want {want}"
        seen.add(trans_b)
    assert seen == {0, 1}


def _stages(ops):
    """The loop's instructions cut at every s_barrier: [[mnemonics of one stage], ...].
    The loop is a cycle, and its header can fall inside a stage: the pieces
    before the first barrier and after the last one are one stage."""
    out, cur = [], []
    for o in ops:
        if o == "s_barrier":
            out.append(cur)
            cur = []
        else:
            cur.append(o)
    out[0] = cur + out[0]
    return out


def test_pipelined_stage_tuning(asm):
    """The per-layout stage tuning of the 8-wave loop, as compiled.  With B
    given N x K every memory stage opens (after s_setprio 1) with the last two
    MFMAs of the MFMA stage before it, and nothing else is an MFMA there; each
    memory stage issues four copies (S1 a0 a1, S3 b0 b1).  With B given K x N
    there are no such MFMAs, S1 reads 12 fragments (b1 and k-slice 0 of the
    next b0: 8 + 4 transposing reads) and S3 20 (a0, a1: 16, and k-slice 1 of
    b0: 4), and S1 issues six copies (b0 a0 a1), S3 two (b1)."""
    seen = set()
    for (fn, hdr), ops in loops(asm["gemm_pipelined_kernel"]).items():
        if "gemm_pipelined_kernel" not in fn:
            continue
        m = re.search(r"kernelILi(\d)ELb(\d)E", fn)
        elem, trans_b = int(m.group(1)), int(m.group(2))
        stages = [st for st in _stages(ops)]
        mem = [st for st in stages if "s_setprio" in st and any(o.startswith("buffer_load") for o in st)]
        assert len(mem) == 4, f"{fn}: {len(mem)} memory stages per iteration"
        for st in mem:
            body = st[st.index("s_setprio") + 1:]
            mfma = [o for o in body if o.startswith("v_mfma")]
            if trans_b:
                assert len(mfma) == 2 and all(o.startswith("v_mfma") for o in body[:2]), f"{fn}: {body[:6]}"
            else:
                assert not mfma, f"{fn}: {len(mfma)} MFMAs in a memory stage"
        copies = [sum(o.startswith("buffer_load") for o in st) for st in mem]
        if trans_b:
            assert copies == [4, 4, 4, 4], f"{fn}: copies per memory stage {copies}"
        else:
            reads = [sum(o.startswith("ds_read") for o in st) for st in mem]
            assert reads in ([12, 20, 12, 20], [20, 12, 20, 12]), f"{fn}: reads per memory stage {reads}"
            assert copies in ([6, 2, 6, 2], [2, 6, 2, 6]), f"{fn}: copies per memory stage {copies}"
        seen.add((elem, trans_b))
    assert seen == {(0, 0), (0, 1), (1, 0), (1, 1), (2, 1)}


def test_pipelined_copy_waits(asm):
    """The vmcnt of the waits in the 8-wave kernel (prologue 10, epilogue 0):
    with B given N x K S1 ends with 6 (b0 is copied in S3, before b1) and S3
    with 8; with B given K x N S1 ends with 8 and S3 with 6 (S1's copy order
    puts b0 first, and S1 reads k-slice 0 of the next b0 early)."""
    for fn, lines in _function(asm["gemm_pipelined_kernel"], "gemm_pipelined_kernel").items():
        trans_b = int(re.search(r"kernelILi\dELb(\d)E", fn).group(1))
        vm = set(re.findall(r"s_waitcnt vmcnt\((\d+)\)", "\n".join(lines)))
        want = {"0", "6", "8", "10"}
        assert vm == want, f"{fn}: vmcnt values {sorted(vm)}"


def _function(asm_text, name_part):
    """{symbol: [lines]} of every function whose symbol contains name_part."""
    out, fn = {}, None
    for line in asm_text.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn = m.group(1) if name_part in m.group(1) else None
            if fn:
                out[fn] = []
            continue
        if fn:
            out[fn].append(line)
            if "s_endpgm" in line:
                fn = None
    return out


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok) or re.match(r"([va])(\d+)$", tok)
    if not m:
        return set()
    lo = int(m.group(2))
    hi = int(m.group(3)) if m.lastindex == 3 else lo
    return {(m.group(1), r) for r in range(lo, hi + 1)}


def _mfma_hazards(lines):
    """Wait-state violations around MFMAs, in program order (each instruction
    one wait state, s_nop N counts N + 1): a VALU result read by an MFMA
    fewer than 2 states later, and an MFMA result read by a VALU or store
    fewer than 11 states later (8-pass 16x16x32 MFMA; the compiler pads
    neither around inline-asm MFMAs)."""
    bad, valu_w, mfma_w = [], [], []
    for raw in lines:
        t = raw.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        ops = [x.strip().split()[0] for x in t[len(op):].split(",") if x.strip()]
        cost = int(ops[0], 0) + 1 if op == "s_nop" else 1
        dst = _regs(ops[0]) if ops else set()
        srcs = set().union(*[_regs(x) for x in ops[1:]]) if len(ops) > 1 else set()
        if op.startswith("v_mfma"):
            if any(age < 2 and d & srcs for d, age in valu_w):
                bad.append(("valu->mfma", t))
            srcc = _regs(ops[3]) if len(ops) > 3 else set()
            if any(age < 11 and d & srcs and d != srcc for d, age in mfma_w):
                bad.append(("mfma->mfma", t))
        elif op.startswith(("v_", "ds_write", "global_store", "buffer_store")):
            reads = srcs | (dst if not op.startswith("v_") else set())
            if any(age < 11 and d & reads for d, age in mfma_w):
                bad.append(("mfma->valu", t))
        valu_w = [(d, a + cost) for d, a in valu_w if a + cost < 2]
        mfma_w = [(d, a + cost) for d, a in mfma_w if a + cost < 11]
        if op.startswith("v_mfma"):
            mfma_w.append((dst, 0))
        elif op.startswith("v_") and dst:
            valu_w.append((dst, 0))
    return bad


def test_attention_four_wave_kernel(asm):
    """The 4-wave attention kernel writes its MFMAs as inline assembly (scores
    in VGPRs, Q and O in AGPRs): no MFMA hazard anywhere in it, and per main
    loop trip 128 MFMAs (QK and PV of one 64-key block), one barrier, and O
    left in its AGPRs outside the rescale block: the moves there are the
    few dozen the register allocator uses to park values, not the 128 O
    reads that a rescale merged in VGPRs costs on every trip."""
    fns = _function(asm["attention_fwd_kernel"], "attention_fwd4_kernel")
    assert len(fns) == 4, sorted(fns)
    for fn, lines in fns.items():
        assert not _mfma_hazards(lines), (fn, _mfma_hazards(lines)[:3])
        head = next(i for i, l in enumerate(lines) if "Loop Header" in l)
        label = lines[head].split(":")[0]
        end = next(i for i in range(head + 1, len(lines)) if lines[i].split()[:2] == ["s_branch", label])
        body = lines[head:end + 1]
        blocks, cur = [], []
        for l in body:
            if re.match(r"^(\.LBB\w+|; %bb\.\d+):", l):
                blocks.append(cur)
                cur = []
            cur.append(l)
        blocks.append(cur)
        ops = [[l.strip().split()[0] for l in b if l.strip() and not l.strip().startswith((";", "."))]
               for b in blocks]
        flat = [o for b in ops for o in b]
        assert sum(o.startswith("v_mfma") for o in flat) == 128, fn
        assert flat.count("s_barrier") == 1, fn
        assert not [o for o in flat if o.startswith(("scratch_", "buffer_store"))], fn
        rescale = [b for b in ops if sum(o.startswith("v_accvgpr_write") for o in b) >= 128]
        assert len(rescale) == 1, fn
        rest = sum(o.startswith("v_accvgpr") for b in ops if b is not rescale[0] for o in b)
        assert rest <= 96, f"{fn}: {rest} AGPR moves outside the rescale block"


@pytest.mark.parametrize("kernel", sorted(EXPECT))
def test_no_mfma_hazards(asm, kernel):
    """No function of the file reads an MFMA operand or result too early (the
    compiler pads its own MFMAs; this guards the inline-asm ones)."""
    fns = _function(asm[kernel], "")
    assert fns
    for fn, lines in fns.items():
        assert not _mfma_hazards(lines), (fn, _mfma_hazards(lines)[:3])
