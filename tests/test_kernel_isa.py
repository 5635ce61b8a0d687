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
          "gemm_tile128_kernel": (32, 32, 1, 2, 10), "attention_fwd_kernel": (64, None, 4, None, 8)}
SOURCES = {"gemm_pipelined_kernel": "gemm_pipelined.hip", "gemm_interleaved_kernel": "gemm_interleaved.hip",
           "gemm_tile128_kernel": "gemm_tile128.hip", "attention_fwd_kernel": "attention_fwd.hip"}


def loops(asm: str):
    """{(kernel symbol, loop header): [instruction mnemonics]} of every loop."""
    out, fn, cur = {}, None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn, cur = m.group(1), None
            continue
        if re.match(r"^(\.LBB\w+|; %bb\.\d+):", line):
            h = re.search(r"Loop Header", line)
            i = re.search(r"in Loop: Header=(BB\w+)", line)
            cur = (fn, line.split(":")[0].lstrip(".L")) if h else ((fn, i.group(1)) if i else None)
            continue
        t = line.strip()
        if cur and fn and t and not t.startswith((";", ".")):
            out.setdefault(cur, []).append(t.split()[0])
    return out


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
