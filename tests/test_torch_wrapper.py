"""The torch marshalling layer (``matrix_core_scheduling_amd.gemm``) on the GPU:
operands and outputs that are row-padded views of wider buffers go through
with their row strides as leading dimensions, the output type follows the
``out`` tensor, and the result is bit for bit that of the plain C-ABI call
on the same values (and within the oracle's tolerance)."""
import numpy as np
import pytest

import matrix_core_scheduling_amd as mcs
import oracle
import seeded_inputs as si
from tests.gpu_util import TORCH_DT, _torch, assert_within_tolerance, out_elem, run

pytestmark = pytest.mark.gpu


def _padded_view(bits, elem, pad):
    """Device tensor of `bits` (rows x cols) inside a buffer `pad` elements wider
    per row; the pad columns hold 0x7F bytes."""
    torch = _torch()
    rows, cols = bits.shape
    raw_dt, np_dt = (torch.uint8, np.uint8) if elem == "fp8" else (torch.int16, np.int16)
    big = torch.full((rows, cols + pad), 0x7F if elem == "fp8" else 0x7F7F, dtype=raw_dt)
    big[:, :cols] = torch.from_numpy(np.ascontiguousarray(bits).view(np_dt))
    return big.cuda().view(TORCH_DT[elem])[:, :cols]


@pytest.mark.parametrize("elem,trans_b,out", [
    ("f16", 1, "same"), ("f16", 0, "f32"), ("bf16", 1, "bf16"), ("bf16", 0, "f32"),
    ("fp8", 1, "bf16"), ("fp8", 1, "f32"),
])
def test_gemm_wrapper_matches_the_c_abi(elem, trans_b, out):
    torch = _torch()
    M, N, K = 300, 264, 528
    print(f"[gpu] torch wrapper {elem} trans_b={trans_b} out={out} {M}x{N}x{K}", flush=True)
    a = si.matrix_bits(elem, "uniform", M, K, seed=9100, stream=0)
    b = (si.matrix_bits(elem, "uniform", N, K, seed=9100, stream=1) if trans_b
         else si.matrix_bits(elem, "uniform", K, N, seed=9100, stream=1))
    A = _padded_view(a, elem, 16)
    B = _padded_view(b, elem, 32)
    oe = out_elem(elem, out)
    C_big = torch.full((M, N + 8), 5.0, dtype=TORCH_DT[oe], device="cuda")
    C = C_big[:, :N]
    got = mcs.gemm(A, B, trans_b=bool(trans_b), out=C)
    assert got.data_ptr() == C.data_ptr()
    torch.cuda.synchronize()
    assert torch.all(C_big[:, N:] == 5.0), "the wrapper wrote past the output's columns"
    raw = C.cpu().contiguous()
    bits = raw.numpy().view(np.uint32) if oe == "f32" else raw.view(torch.int16).numpy().view(np.uint16)
    _, want = run(elem, M, N, K, a, b, trans_b, out=out)
    assert np.array_equal(bits, want), f"{(bits != want).sum()} elements differ from the C-ABI call"
    cref, sabs = oracle.gemm(a, b, elem, trans_b, K=K, N=N)
    vals = bits.view(np.float32).astype(np.float64) if oe == "f32" else oracle.decode(bits, oe)
    assert_within_tolerance(vals, cref, sabs, f"torch wrapper {elem}", out=oe)


def test_gemm_wrapper_allocates_the_operand_type():
    """Without ``out`` the result is a fresh M x N tensor of the operand type
    (BF16 for FP8 operands), on the current stream."""
    torch = _torch()
    M, N, K = 64, 96, 128
    print(f"[gpu] torch wrapper allocation {M}x{N}x{K}", flush=True)
    for elem, want in (("f16", torch.float16), ("bf16", torch.bfloat16), ("fp8", torch.bfloat16)):
        a = si.matrix_bits(elem, "uniform", M, K, seed=9200, stream=0)
        b = si.matrix_bits(elem, "uniform", N, K, seed=9200, stream=1)
        C = mcs.gemm(_padded_view(a, elem, 0), _padded_view(b, elem, 0), trans_b=True)
        torch.cuda.synchronize()
        assert C.shape == (M, N) and C.dtype == want and C.is_cuda
        cref, sabs = oracle.gemm(a, b, elem, 1, K=K, N=N)
        oe = "bf16" if elem == "fp8" else elem
        assert_within_tolerance(oracle.decode(C.cpu().view(torch.int16).numpy().view(np.uint16), oe),
                                cref, sabs, f"allocated output {elem}", out=oe)


def test_gemm_wrapper_reports_operands_the_mfma_kernels_cannot_take():
    """A view whose rows are not whole 16-byte multiples raises GEMM_EALIGN
    (nothing is launched); the plain kernel takes it when asked for."""
    torch = _torch()
    M, N, K = 64, 96, 120
    print(f"[gpu] torch wrapper refusal {M}x{N}x{K}", flush=True)
    a = si.matrix_bits("f16", "uniform", M, K, seed=9300, stream=0)
    b = si.matrix_bits("f16", "uniform", N, K, seed=9300, stream=1)
    A = _padded_view(a, "f16", 4)                # lda = 124: 248-byte rows
    B = _padded_view(b, "f16", 8)
    with pytest.raises(mcs.GemmError) as e:
        mcs.gemm(A, B, trans_b=True)
    assert e.value.status == mcs.GEMM_EALIGN
    C = mcs.gemm(A, B, trans_b=True, schedule=mcs.GEMM_SCHED_GENERIC)
    torch.cuda.synchronize()
    cref, sabs = oracle.gemm(a, b, "f16", 1, K=K, N=N)
    assert_within_tolerance(oracle.decode(C.cpu().view(torch.int16).numpy().view(np.uint16), "f16"),
                            cref, sabs, "plain kernel on request", out="f16")
