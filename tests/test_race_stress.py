"""Race stress: the race-stress build of the library (libmcs_gemm_stagger.so,
the same sources compiled with MCS_STAGGER) must give bitwise the same
results as the product library.

That build idles every wave for a pseudo-random 0..15 sleeps of 64 cycles on
both sides of every workgroup barrier (a fresh seed per launch) and fills the
workgroup's LDS with 0xFF bytes -- NaN in every operand type -- before the
first copy.  The arithmetic and its order are those of the product build, so
a schedule whose waits and barriers are sufficient gives identical bits
under any timing; a missing wait or barrier shows up as changed bits or NaN
once the waves drift apart.  The pages stress that a warp-pipelined kernel
can lose overlap or race silently ("Two Waves, One Stage Apart", section
"Dependencies Cross Groups and Iterations"); this makes such a race loud.

Each product is run once on the product library and three times on the
race-stress library; every run is compared bit for bit, and the product
library's result is checked against the oracle."""
import numpy as np
import pytest

import matrix_core_scheduling_amd as mcs
import oracle
import seeded_inputs as si
from tests.gpu_util import TORCH_DT, _torch, assert_within_tolerance, out_elem, upload

pytestmark = pytest.mark.gpu

DT = {"f16": mcs.GEMM_DTYPE_F16, "bf16": mcs.GEMM_DTYPE_BF16, "fp8": mcs.GEMM_DTYPE_FP8_E4M3}
OUT = {"same": mcs.GEMM_OUT_SAME, "f32": mcs.GEMM_OUT_F32, "bf16": mcs.GEMM_OUT_BF16}
SCHED = {"pipelined": mcs.GEMM_SCHED_PIPELINED, "in_phase": mcs.GEMM_SCHED_IN_PHASE,
         "interleaved": mcs.GEMM_SCHED_INTERLEAVED, "tile128": mcs.GEMM_SCHED_TILE128}
REPEATS = 3


def _operands(elem, M, N, K, trans_b, seed):
    a = si.matrix_bits(elem, "uniform", M, K, seed=seed, stream=0)
    b = (si.matrix_bits(elem, "uniform", N, K, seed=seed, stream=1) if trans_b
         else si.matrix_bits(elem, "uniform", K, N, seed=seed, stream=1))
    return a, b


def _gemm_bits(lib, elem, M, N, K, A, lda, B, ldb, trans_b, out, sched, splits=1):
    """Raw output bits (M x N) of one launch on `lib` (fresh output filled with 0x7F bytes)."""
    torch = _torch()
    oe = out_elem(elem, out)
    C = torch.empty(M * N, dtype=TORCH_DT[oe], device="cuda")
    C.view(torch.uint8).fill_(0x7F)
    stream = torch.cuda.current_stream().cuda_stream
    if splits == 1:
        st = lib.gemm_ex(DT[elem], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, trans_b, C.data_ptr(), N,
                         OUT[out], sched, stream)
    else:
        nbytes = mcs.gemm_splitk_workspace_bytes(DT[elem], M, N, K, splits)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        st = lib.gemm_ex_splitk(DT[elem], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, trans_b, C.data_ptr(),
                                N, OUT[out], sched, splits, ws.data_ptr(), nbytes, stream)
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)
    torch.cuda.synchronize()
    raw = C.view(M, N).cpu()
    return raw.numpy().view(np.uint32) if oe == "f32" else raw.view(torch.int16).numpy().view(np.uint16)


GEMM_CASES = [  # (elem, trans_b, out, M, N, K): several tiles, ragged edges, a partial last K-step;
    # rows of 16-byte multiples, as the tiled schedules require
    ("f16", 1, "same", 520, 392, 2000),
    ("f16", 0, "same", 520, 392, 2000),
    ("bf16", 1, "f32", 264, 776, 1496),
    ("bf16", 0, "same", 300, 520, 1000),
    ("fp8", 1, "bf16", 520, 392, 3008),
]


@pytest.mark.parametrize("sched", list(SCHED))
@pytest.mark.parametrize("elem,trans_b,out,M,N,K", GEMM_CASES)
def test_gemm_bitwise_under_stagger(elem, trans_b, out, M, N, K, sched):
    print(f"[gpu] race stress gemm {elem} trans_b={trans_b} out={out} {M}x{N}x{K} sched={sched}", flush=True)
    a, b = _operands(elem, M, N, K, trans_b, seed=7100 + M + K)
    A, _ = upload(a, elem)
    B, _ = upload(b, elem)
    ref = _gemm_bits(mcs.load(), elem, M, N, K, A, a.shape[1], B, b.shape[1], trans_b, out, SCHED[sched])
    oe = out_elem(elem, out)
    cref, sabs = oracle.gemm(a, b, elem, trans_b, K=K, N=N)
    vals = ref.view(np.float32).astype(np.float64) if oe == "f32" else oracle.decode(ref, oe)
    assert_within_tolerance(vals, cref, sabs, what=f"product library {sched}", out=oe)
    for r in range(REPEATS):
        got = _gemm_bits(mcs.load_stagger(), elem, M, N, K, A, a.shape[1], B, b.shape[1], trans_b, out,
                         SCHED[sched])
        diff = np.argwhere(got != ref)
        assert diff.size == 0, (f"run {r}: {len(diff)} elements differ under stagger; first at "
                                f"{diff[0].tolist()}: {got[tuple(diff[0])]:#x} vs {ref[tuple(diff[0])]:#x}")


@pytest.mark.parametrize("sched", ["pipelined", "tile128"])
@pytest.mark.parametrize("elem,trans_b,out,M,N,K,splits", [
    ("f16", 1, "same", 512, 520, 4000, 3),
    ("bf16", 0, "f32", 264, 256, 3000, 4),
])
def test_splitk_bitwise_under_stagger(elem, trans_b, out, M, N, K, splits, sched):
    print(f"[gpu] race stress splitk {elem} trans_b={trans_b} {M}x{N}x{K} splits={splits} sched={sched}",
          flush=True)
    a, b = _operands(elem, M, N, K, trans_b, seed=7300 + splits)
    A, _ = upload(a, elem)
    B, _ = upload(b, elem)
    ref = _gemm_bits(mcs.load(), elem, M, N, K, A, a.shape[1], B, b.shape[1], trans_b, out, SCHED[sched], splits)
    for r in range(REPEATS):
        got = _gemm_bits(mcs.load_stagger(), elem, M, N, K, A, a.shape[1], B, b.shape[1], trans_b, out,
                         SCHED[sched], splits)
        assert np.array_equal(got, ref), f"run {r}: {(got != ref).sum()} elements differ under stagger"


def _attention_bits(lib, elem, q, k, v, scale, causal, sched):
    torch = _torch()
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    Q, _ = upload(q.reshape(-1, D), elem)
    K, _ = upload(k.reshape(-1, D), elem)
    V, _ = upload(v.reshape(-1, D), elem)
    O = torch.full((B * H * Sq * D,), 3.0, dtype=TORCH_DT[elem], device="cuda")
    L = torch.full((B * H * Sq,), 7.0, dtype=torch.float32, device="cuda")
    st = lib.attention_fwd_ex(DT[elem], B, H, Sq, Sk, D, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                              L.data_ptr(), scale, int(causal), sched, torch.cuda.current_stream().cuda_stream)
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)
    torch.cuda.synchronize()
    return O.cpu().view(torch.int16).numpy().view(np.uint16), L.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("sched", ["pipelined", "in_phase", "interleaved"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("elem", ["f16", "bf16"])
def test_attention_bitwise_under_stagger(elem, causal, sched):
    B, H, Sq, Sk, D = 1, 3, 600, 1000, 128
    print(f"[gpu] race stress attention {elem} causal={causal} sched={sched} {B}x{H}x{Sq}x{Sk}", flush=True)
    q = si.matrix_bits(elem, "normal", B * H * Sq, D, seed=7500, stream=0).reshape(B, H, Sq, D)
    k = si.matrix_bits(elem, "normal", B * H * Sk, D, seed=7500, stream=1).reshape(B, H, Sk, D)
    v = si.matrix_bits(elem, "normal", B * H * Sk, D, seed=7500, stream=2).reshape(B, H, Sk, D)
    s = SCHED[sched]
    o_ref, l_ref = _attention_bits(mcs.load(), elem, q, k, v, 0.088, causal, s)
    assert not np.isnan(oracle.decode(o_ref, elem)).any()
    for r in range(REPEATS):
        o, lse = _attention_bits(mcs.load_stagger(), elem, q, k, v, 0.088, causal, s)
        assert np.array_equal(o, o_ref), f"run {r}: {(o != o_ref).sum()} O elements differ under stagger"
        assert np.array_equal(lse, l_ref), f"run {r}: {(lse != l_ref).sum()} lse values differ under stagger"


@pytest.mark.parametrize("sched", ["pipelined", "in_phase"])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_tile_to_tile_bitwise_under_stagger(causal, sched):
    """More tiles (300) than CUs: every persistent workgroup of the 8-wave
    kernel runs several tiles in a row, with the next tile's blocks and Q
    fetched during the last trips of the one before."""
    B, H, Sq, Sk, D = 1, 100, 768, 512, 128
    print(f"[gpu] race stress attention tiles f16 causal={causal} sched={sched} {B}x{H}x{Sq}x{Sk}", flush=True)
    q = si.matrix_bits("f16", "normal", B * H * Sq, D, seed=7501, stream=0).reshape(B, H, Sq, D)
    k = si.matrix_bits("f16", "normal", B * H * Sk, D, seed=7501, stream=1).reshape(B, H, Sk, D)
    v = si.matrix_bits("f16", "normal", B * H * Sk, D, seed=7501, stream=2).reshape(B, H, Sk, D)
    s = SCHED[sched]
    o_ref, l_ref = _attention_bits(mcs.load(), "f16", q, k, v, 0.088, causal, s)
    assert not np.isnan(oracle.decode(o_ref, "f16")).any()
    for r in range(REPEATS):
        o, lse = _attention_bits(mcs.load_stagger(), "f16", q, k, v, 0.088, causal, s)
        assert np.array_equal(o, o_ref), f"run {r}: {(o != o_ref).sum()} O elements differ under stagger"
        assert np.array_equal(lse, l_ref), f"run {r}: {(lse != l_ref).sum()} lse values differ under stagger"


def test_stagger_build_is_the_one_that_runs():
    """The race-stress library really runs its own, slower kernels: its pauses
    add ~1,000 cycles per barrier against ~500 cycles of work per stage."""
    torch = _torch()
    M = N = 2048
    K = 4096
    print(f"[gpu] race stress timing {M}x{N}x{K}", flush=True)
    A = torch.zeros(M * K, dtype=torch.float16, device="cuda")
    B = torch.zeros(N * K, dtype=torch.float16, device="cuda")
    C = torch.empty(M * N, dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(lib):
        for _ in range(3):
            assert lib.gemm_ex(DT["f16"], M, N, K, A.data_ptr(), K, B.data_ptr(), K, 1, C.data_ptr(), N,
                               OUT["same"], SCHED["pipelined"], stream) == mcs.GEMM_OK
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            lib.gemm_ex(DT["f16"], M, N, K, A.data_ptr(), K, B.data_ptr(), K, 1, C.data_ptr(), N,
                        OUT["same"], SCHED["pipelined"], stream)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 10

    t_product, t_stagger = timed(mcs.load()), timed(mcs.load_stagger())
    print(f"[gpu] product {t_product * 1e3:.1f} us, race-stress build {t_stagger * 1e3:.1f} us", flush=True)
    assert t_stagger > 1.5 * t_product
