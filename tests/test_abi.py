"""The C-ABI library loads, exports what include/mcs_gemm.h declares, and
rejects bad arguments before touching the device (runs without a GPU)."""
import os
import subprocess

import pytest

import matrix_core_scheduling_amd as mcs


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mcs.LIBRARY):
        from matrix_core_scheduling_amd import build
        build.build()
    return mcs.load()


def test_header_declares_the_entry_points():
    names = mcs.header_functions()
    assert set(names) == {"gemm_f16", "gemm_bf16", "gemm_fp8", "gemm_ex", "gemm_ex_splitk",
                          "gemm_ex_splitk_noalloc",
                          "gemm_splitk_workspace_bytes", "gemm_auto_schedule", "gemm_splitk_suggest",
                          "gemm_kernel_info", "attention_fwd", "attention_fwd_ex",
                          "gemm_status_string"}


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", mcs.LIBRARY], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in mcs.header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for st in (mcs.GEMM_OK, mcs.GEMM_EINVAL, mcs.GEMM_EALIGN, mcs.GEMM_EUNSUPPORTED, mcs.GEMM_EHIP,
               mcs.GEMM_ENOSCRATCH):
        assert mcs.gemm_status_string(st).startswith(("GEMM_OK", "GEMM_E"))
    assert "unknown" in mcs.gemm_status_string(12345)


# (M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type) -> expected status; pointers are
# fake non-null integers: validation must reject before any launch.  O stands for
# a valid output type of the entry point (GEMM_OUT_SAME, or GEMM_OUT_BF16 for FP8).
P = 0x1000
O = "valid-out"
BAD = [
    ((-1, 4, 4, P, 4, P, 4, 0, P, 4, O), mcs.GEMM_EINVAL),        # negative M
    ((4, -1, 4, P, 4, P, 4, 0, P, 4, O), mcs.GEMM_EINVAL),        # negative N
    ((4, 4, -3, P, 4, P, 4, 0, P, 4, O), mcs.GEMM_EINVAL),        # negative K
    ((4, 4, 8, P, 7, P, 4, 0, P, 4, O), mcs.GEMM_EINVAL),         # lda < K
    ((4, 4, 8, P, 8, P, 3, 0, P, 4, O), mcs.GEMM_EINVAL),         # ldb < N (B is K x N)
    ((4, 4, 8, P, 8, P, 7, 1, P, 4, O), mcs.GEMM_EINVAL),         # ldb < K (B is N x K)
    ((4, 4, 8, P, 8, P, 8, 0, P, 3, O), mcs.GEMM_EINVAL),         # ldc < N
    ((4, 4, 8, P, 8, P, 8, 2, P, 8, O), mcs.GEMM_EINVAL),         # trans_b not 0/1
    ((4, 4, 8, P, 8, P, 8, 0, P, 8, 7), mcs.GEMM_EINVAL),         # out_type unknown
    ((4, 4, 8, 0, 8, P, 8, 0, P, 8, O), mcs.GEMM_EINVAL),         # null A
    ((4, 4, 8, P, 8, 0, 8, 0, P, 8, O), mcs.GEMM_EINVAL),         # null B
    ((4, 4, 8, P, 8, P, 8, 0, 0, 8, O), mcs.GEMM_EINVAL),         # null C
    ((1 << 31, 4, 8, P, 8, P, 8, 0, P, 8, O), mcs.GEMM_EUNSUPPORTED),
    ((4, 4, 8, P, 1 << 31, P, 8, 0, P, 8, O), mcs.GEMM_EUNSUPPORTED),
    ((0, 4, 8, 0, 8, 0, 8, 0, 0, 8, O), mcs.GEMM_OK),             # empty: no-op, no launch
    ((4, 0, 8, 0, 8, 0, 8, 0, 0, 8, O), mcs.GEMM_OK),
]
VALID_OUT = {"gemm_f16": mcs.GEMM_OUT_SAME, "gemm_bf16": mcs.GEMM_OUT_SAME, "gemm_fp8": mcs.GEMM_OUT_BF16}


@pytest.mark.parametrize("args,want", BAD)
@pytest.mark.parametrize("fn", ["gemm_f16", "gemm_bf16", "gemm_fp8"])
def test_validation_before_launch(lib, fn, args, want):
    args = tuple(VALID_OUT[fn] if a == O else a for a in args)
    assert getattr(mcs, fn)(*args, 0) == want


def test_output_types_per_operand_type(lib):
    """FP16 operands: FP16 or FP32 out; BF16: BF16 (SAME or BF16) or FP32; FP8:
    BF16 or FP32 (no FP8 output).  Checked on an empty product (no launch)."""
    empty = (0, 4, 8, 0, 8, 0, 8, 0, 0, 8)
    assert mcs.gemm_f16(*empty, mcs.GEMM_OUT_BF16, 0) == mcs.GEMM_EINVAL
    assert mcs.gemm_bf16(*empty, mcs.GEMM_OUT_BF16, 0) == mcs.GEMM_OK
    assert mcs.gemm_fp8(*empty, mcs.GEMM_OUT_SAME, 0) == mcs.GEMM_EINVAL
    assert mcs.gemm_fp8(*empty, mcs.GEMM_OUT_F32, 0) == mcs.GEMM_OK


def test_ex_rejects_bad_dtype_and_schedule(lib):
    good = (4, 4, 8, P, 8, P, 8, 0, P, 8, 0)
    assert mcs.gemm_ex(7, *good, 0, 0) == mcs.GEMM_EINVAL
    assert mcs.gemm_ex(0, *good, 9, 0) == mcs.GEMM_EINVAL
    assert mcs.gemm_ex(0, *good, 6, 0) == mcs.GEMM_EINVAL
    assert mcs.gemm_ex(0, *good, -1, 0) == mcs.GEMM_EINVAL


MFMA_SCHEDS = ("AUTO", "PIPELINED", "IN_PHASE", "INTERLEAVED", "TILE128")


@pytest.mark.parametrize("sched", MFMA_SCHEDS)
def test_mfma_schedules_refuse_what_they_cannot_take(lib, sched):
    """Operands the MFMA kernels cannot take are refused before anything is
    launched, with the reason: GEMM_EALIGN for pointers and leading
    dimensions, GEMM_EUNSUPPORTED for shapes.  AUTO (what gemm_f16 runs)
    refuses them too: it never falls back to the plain FMA kernel."""
    s = getattr(mcs, "GEMM_SCHED_" + sched)
    ex = mcs.gemm_ex
    f16, fp8 = mcs.GEMM_DTYPE_F16, mcs.GEMM_DTYPE_FP8_E4M3
    BF = mcs.GEMM_OUT_BF16
    assert ex(f16, 256, 256, 64, P + 2, 64, P, 64, 1, P, 256, 0, s, 0) == mcs.GEMM_EALIGN     # A
    assert ex(f16, 256, 256, 64, P, 64, P + 8, 64, 1, P, 256, 0, s, 0) == mcs.GEMM_EALIGN     # B
    assert ex(f16, 256, 256, 64, P, 64, P, 64, 1, P + 4, 256, 0, s, 0) == mcs.GEMM_EALIGN     # C
    assert ex(f16, 256, 256, 64, P, 68, P, 64, 1, P, 256, 0, s, 0) == mcs.GEMM_EALIGN         # lda
    assert ex(f16, 256, 256, 64, P, 64, P, 260, 0, P, 256, 0, s, 0) == mcs.GEMM_EALIGN        # ldb
    assert ex(f16, 256, 250, 64, P, 64, P, 64, 1, P, 252, 0, s, 0) == mcs.GEMM_EALIGN         # ldc
    assert ex(f16, 256, 256, 60, P, 64, P, 64, 1, P, 256, 0, s, 0) == mcs.GEMM_EUNSUPPORTED   # K % 8
    assert ex(f16, 256, 255, 64, P, 64, P, 256, 0, P, 256, 0, s, 0) == mcs.GEMM_EUNSUPPORTED  # odd N, K x N
    big = (1 << 23)                                                  # a 2^24-byte FP16 row
    assert ex(f16, 4, 4, 64, P, big, P, 64, 1, P, 8, 0, s, 0) == mcs.GEMM_EUNSUPPORTED
    assert ex(fp8, 256, 256, 136, P, 256, P, 256, 1, P, 256, BF, s, 0) == mcs.GEMM_EUNSUPPORTED  # K % 16
    assert ex(fp8, 256, 256, 128, P, 136, P, 256, 1, P, 256, BF, s, 0) == mcs.GEMM_EALIGN        # lda % 16
    assert ex(fp8, 256, 256, 128, P, 128, P, 256, 0, P, 256, BF, s, 0) == mcs.GEMM_EUNSUPPORTED  # B K x N


@pytest.mark.parametrize("fn", ["gemm_f16", "gemm_bf16", "gemm_fp8"])
def test_entry_points_report_alignment(lib, fn):
    """The spec entry points run only the MFMA kernels: a misaligned
    operand is GEMM_EALIGN, never a silent switch to a slower kernel."""
    out = VALID_OUT[fn]
    f = getattr(mcs, fn)
    assert f(256, 256, 128, P + 2, 128, P, 128, 1, P, 256, out, 0) == mcs.GEMM_EALIGN
    assert f(256, 256, 128, P, 136 if fn == "gemm_fp8" else 132, P, 128, 1, P, 256, out, 0) == mcs.GEMM_EALIGN
    assert f(256, 256, 124, P, 128, P, 128, 1, P, 256, out, 0) == mcs.GEMM_EUNSUPPORTED     # K tail


def test_splitk_refuses_what_the_mfma_kernels_cannot_take(lib):
    sk = mcs.gemm_ex_splitk
    args = (512, 512, 8192, P + 2, 8192, P, 8192, 1, P, 512, 0)
    assert sk(0, *args, mcs.GEMM_SCHED_AUTO, 4, P, 1 << 30, 0) == mcs.GEMM_EALIGN
    args = (512, 512, 8188, P, 8192, P, 8192, 1, P, 512, 0)
    assert sk(0, *args, mcs.GEMM_SCHED_AUTO, 4, P, 1 << 30, 0) == mcs.GEMM_EUNSUPPORTED


def test_torch_wrappers_refuse_host_tensors(lib):
    """A host tensor's pointer would be dereferenced by the GPU: refused before
    any library call."""
    torch = pytest.importorskip("torch")
    a = torch.zeros((64, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        mcs.gemm(a, a, trans_b=True)
    q = torch.zeros((1, 1, 16, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        mcs.attention(q, q, q)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(mcs, "_lib", None)
    with pytest.raises(RuntimeError, match="no non-HIP fallback"):
        mcs.load(str(tmp_path / "absent.so"))


def test_splitk_workspace_size(lib):
    f16 = mcs.GEMM_DTYPE_F16
    # K = 1024 is 16 K-steps of 64: 4 slices of 4 steps; rows of the FP32
    # partials are rounded up to 4 floats
    assert mcs.gemm_splitk_workspace_bytes(f16, 1024, 1000, 1024, 4) == 4 * 1024 * 1000 * 4
    assert mcs.gemm_splitk_workspace_bytes(f16, 1024, 1001, 1024, 4) == 4 * 1024 * 1004 * 4
    # 5 steps in 4 requested slices: 2 steps per slice, so 3 slices
    assert mcs.gemm_splitk_workspace_bytes(f16, 64, 64, 320, 4) == 3 * 64 * 64 * 4
    assert mcs.gemm_splitk_workspace_bytes(f16, 64, 64, 64, 8) == 0            # one K-step: no split
    assert mcs.gemm_splitk_workspace_bytes(f16, 64, 64, 1024, 1) == 0
    fp8 = mcs.GEMM_DTYPE_FP8_E4M3                                           # K-steps of 128
    assert mcs.gemm_splitk_workspace_bytes(fp8, 256, 256, 1024, 4) == 4 * 256 * 256 * 4
    with pytest.raises(mcs.GemmError):
        mcs.gemm_splitk_workspace_bytes(f16, 64, 64, 64, 0)
    # 4 x (2^31 - 1) x (2^31 - 8) x 4 bytes does not fit in int64_t
    big = 2 ** 31 - 8
    with pytest.raises(mcs.GemmError) as e:
        mcs.gemm_splitk_workspace_bytes(f16, big + 7, big, 2 ** 20, 4)
    assert e.value.status == mcs.GEMM_EUNSUPPORTED
    assert mcs.gemm_splitk_workspace_bytes(f16, 2 ** 20, 2 ** 20, 2 ** 20, 4) == 2 ** 44


def test_splitk_validation_before_launch(lib):
    args = (1024, 1024, 1024, P, 1024, P, 1024, 1, P, 1024, 0)
    need = mcs.gemm_splitk_workspace_bytes(0, 1024, 1024, 1024, 4)
    sk = mcs.gemm_ex_splitk
    assert sk(0, *args, mcs.GEMM_SCHED_AUTO, 4, 0, need, 0) == mcs.GEMM_EINVAL          # no workspace
    assert sk(0, *args, mcs.GEMM_SCHED_AUTO, 4, P, need - 16, 0) == mcs.GEMM_EINVAL     # too small
    assert sk(0, *args, mcs.GEMM_SCHED_AUTO, 4, P + 4, need, 0) == mcs.GEMM_EINVAL      # misaligned
    assert sk(0, *args, mcs.GEMM_SCHED_GENERIC, 4, P, need, 0) == mcs.GEMM_EINVAL
    assert sk(0, *args, mcs.GEMM_SCHED_AUTO, 0, P, need, 0) == mcs.GEMM_EINVAL          # splits < 1
    assert sk(0, *args, mcs.GEMM_SCHED_AUTO, 257, P, need, 0) == mcs.GEMM_EINVAL
    bad = (1024, 1024, 1024, P + 2, 1024, P, 1024, 1, P, 1024, 0)                      # unaligned A
    assert sk(0, *bad, mcs.GEMM_SCHED_PIPELINED, 4, P, need, 0) == mcs.GEMM_EALIGN
    assert sk(0, 0, 8, 8, 0, 8, 0, 8, 1, 0, 8, 0, mcs.GEMM_SCHED_AUTO, 4, 0, 0, 0) == mcs.GEMM_OK  # empty
    # a workspace size that overflows int64_t is refused, whatever workspace_bytes claims
    big = 2 ** 31 - 8
    huge = (big + 7, big, 2 ** 20, P, 2 ** 20, P, 2 ** 20, 1, P, big, 0)
    assert sk(0, *huge, mcs.GEMM_SCHED_PIPELINED, 4, P, 2 ** 62, 0) == mcs.GEMM_EUNSUPPORTED


def test_auto_schedule(lib):
    P, T = mcs.GEMM_SCHED_PIPELINED, mcs.GEMM_SCHED_TILE128
    assert mcs.gemm_auto_schedule(4096, 4096) == P                   # 256 tiles of 256x256
    assert mcs.gemm_auto_schedule(3072, 3072) == P                   # 144
    assert mcs.gemm_auto_schedule(2048, 4096) == P                   # 128: half the CUs
    assert mcs.gemm_auto_schedule(2048, 3840) == T                   # 120
    assert mcs.gemm_auto_schedule(1024, 1024) == T
    assert mcs.gemm_auto_schedule(512, 4096) == T
    assert mcs.gemm_auto_schedule(1, 1) == T
    assert mcs.gemm_auto_schedule(-1, 8) == mcs.GEMM_EINVAL


def test_splitk_suggest(lib):
    f16, fp8 = mcs.GEMM_DTYPE_F16, mcs.GEMM_DTYPE_FP8_E4M3
    assert mcs.gemm_splitk_suggest(f16, 4096, 4096, 8192) == 1        # 256 tiles fill 256 CUs
    assert mcs.gemm_splitk_suggest(f16, 512, 4096, 8192) == 2         # 128 tiles of 128x128, 128 K-steps
    assert mcs.gemm_splitk_suggest(fp8, 512, 4096, 8192) == 1         # 64 K-steps of 128 FP8 elements
    assert mcs.gemm_splitk_suggest(f16, 1024, 1024, 8192) == 2        # 64 tiles, 128 K-steps
    assert mcs.gemm_splitk_suggest(f16, 1024, 1024, 1024) == 1        # 16 K-steps: too short
    assert mcs.gemm_splitk_suggest(f16, 256, 256, 65536) == 16        # 4 tiles, 1024 K-steps
    assert mcs.gemm_splitk_suggest(f16, 256, 256, 65536, 32) == 8
    assert mcs.gemm_splitk_suggest(f16, 512, 4096, 8192, 128) == 1


def test_attention_argument_errors(lib):
    """Every refusal happens before any device call (none of these launch)."""
    f16, bf16 = mcs.GEMM_DTYPE_F16, mcs.GEMM_DTYPE_BF16
    good = dict(dtype=f16, batch=1, heads=2, seq_q=64, seq_k=64, head_dim=128, Q=P, K=P, V=P, O=P, lse=P,
                scale=0.125, causal=0, stream=0)

    def call(**kw):
        a = dict(good, **kw)
        return mcs.attention_fwd(a["dtype"], a["batch"], a["heads"], a["seq_q"], a["seq_k"], a["head_dim"],
                                 a["Q"], a["K"], a["V"], a["O"], a["lse"], a["scale"], a["causal"], a["stream"])

    assert call(dtype=mcs.GEMM_DTYPE_FP8_E4M3) == mcs.GEMM_EINVAL
    assert call(dtype=7) == mcs.GEMM_EINVAL
    assert call(causal=2) == mcs.GEMM_EINVAL
    assert call(seq_q=-1) == mcs.GEMM_EINVAL
    assert call(batch=-2) == mcs.GEMM_EINVAL
    assert call(scale=0.0) == mcs.GEMM_EINVAL
    assert call(scale=-1.0) == mcs.GEMM_EINVAL
    assert call(scale=float("nan")) == mcs.GEMM_EINVAL
    assert call(scale=float("inf")) == mcs.GEMM_EINVAL
    assert call(head_dim=64) == mcs.GEMM_EUNSUPPORTED
    assert call(Q=0) == mcs.GEMM_EINVAL
    assert call(O=P + 8) == mcs.GEMM_EALIGN                          # misaligned
    assert call(K=P + 2) == mcs.GEMM_EALIGN
    assert call(V=0) == mcs.GEMM_EINVAL
    assert call(lse=P + 2) == mcs.GEMM_EALIGN
    assert call(seq_q=1 << 23) == mcs.GEMM_EUNSUPPORTED
    assert call(batch=1 << 40, heads=1 << 40) == mcs.GEMM_EUNSUPPORTED      # batch * heads would overflow
    assert call(batch=1 << 20, heads=1 << 12) == mcs.GEMM_EUNSUPPORTED      # 2^32 workgroup rows
    # empty problems enqueue nothing
    assert call(batch=0, Q=0, K=0, V=0, O=0) == mcs.GEMM_OK
    assert call(seq_q=0, Q=0, K=0, V=0, O=0) == mcs.GEMM_OK
    assert call(dtype=bf16, heads=0) == mcs.GEMM_OK
    ex = (f16, 1, 2, 64, 64, 128, P, P, P, P, P, 0.125, 0)
    assert mcs.attention_fwd_ex(*ex, mcs.GEMM_SCHED_TILE128, 0) == mcs.GEMM_EINVAL
    assert mcs.attention_fwd_ex(*ex, mcs.GEMM_SCHED_GENERIC, 0) == mcs.GEMM_EINVAL
    assert mcs.attention_fwd_ex(*ex, 9, 0) == mcs.GEMM_EINVAL
    assert mcs.attention_fwd_ex(f16, 0, 2, 64, 64, 128, 0, 0, 0, 0, 0, 0.125, 0, mcs.GEMM_SCHED_IN_PHASE, 0) == mcs.GEMM_OK


def test_noalloc_splitk_validation_before_launch(lib):
    """The allocation-free split K checks everything before touching a
    device: its scratch limit (32 MiB of FP32 partials) included."""
    nk = mcs.gemm_ex_splitk_noalloc
    text = open(mcs.HEADER).read()
    assert "#define GEMM_SPLITK_SCRATCH_BYTES ((int64_t)32 << 20)" in text
    # 4 slices x 1024 x 2048 floats = 32 MiB: the largest that fits; 4 x 1024 x 2052 does not
    assert mcs.gemm_splitk_workspace_bytes(0, 1024, 2048, 8192, 4) == mcs.GEMM_SPLITK_SCRATCH_BYTES
    big = (1024, 2056, 8192, P, 8192, P, 8192, 1, P, 2056, 0)
    assert nk(0, *big, mcs.GEMM_SCHED_AUTO, 4, 0) == mcs.GEMM_ENOSCRATCH
    assert "scratch" in mcs.gemm_status_string(mcs.GEMM_ENOSCRATCH)
    args = (1024, 1024, 1024, P, 1024, P, 1024, 1, P, 1024, 0)
    assert nk(0, *args, mcs.GEMM_SCHED_GENERIC, 4, 0) == mcs.GEMM_EINVAL
    assert nk(0, *args, mcs.GEMM_SCHED_AUTO, 0, 0) == mcs.GEMM_EINVAL
    assert nk(0, *args, mcs.GEMM_SCHED_AUTO, 257, 0) == mcs.GEMM_EINVAL
    bad = (1024, 1024, 1024, P + 2, 1024, P, 1024, 1, P, 1024, 0)
    assert nk(0, *bad, mcs.GEMM_SCHED_AUTO, 4, 0) == mcs.GEMM_EALIGN
    assert nk(0, 0, 8, 8, 0, 8, 0, 8, 1, 0, 8, 0, mcs.GEMM_SCHED_AUTO, 4, 0) == mcs.GEMM_OK   # empty
