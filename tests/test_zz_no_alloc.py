"""The allocation-free split K (gemm_ex_splitk_noalloc) against the split K
with a caller workspace (gemm_ex_splitk): the same kernels, so bitwise the
same C, and both within the oracle's tolerance -- on two calls in a row on
one GPU, the second smaller than the first (the static scratch keeps the
first call's partials; nothing of them may leak into the second)."""
import numpy as np
import pytest

import matrix_core_scheduling_amd as mcs
import oracle
import seeded_inputs as si
from tests.gpu_util import TORCH_DT, _torch, assert_within_tolerance, out_elem, upload

pytestmark = pytest.mark.gpu

DT = {"f16": mcs.GEMM_DTYPE_F16, "bf16": mcs.GEMM_DTYPE_BF16, "fp8": mcs.GEMM_DTYPE_FP8_E4M3}
OUT = {"same": mcs.GEMM_OUT_SAME, "f32": mcs.GEMM_OUT_F32, "bf16": mcs.GEMM_OUT_BF16}


def _call(noalloc, elem, M, N, K, A, lda, B, ldb, trans_b, out, schedule, splits, ldc):
    torch = _torch()
    oe = out_elem(elem, out)
    C = torch.full((M, ldc), -3.0, dtype=TORCH_DT[oe], device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = mcs.gemm_ex_splitk_noalloc(DT[elem], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, trans_b,
                                        C.data_ptr(), ldc, OUT[out], schedule, splits, stream)
    else:
        nbytes = mcs.gemm_splitk_workspace_bytes(DT[elem], M, N, K, splits)
        ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
        st = mcs.gemm_ex_splitk(DT[elem], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, trans_b,
                                C.data_ptr(), ldc, OUT[out], schedule, splits, ws.data_ptr(), nbytes, stream)
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)
    torch.cuda.synchronize()
    raw = C.cpu()
    if oe == "f32":
        return raw.numpy().view(np.uint32), raw.double().numpy()
    bits = raw.view(torch.int16).numpy().view(np.uint16)
    return bits, oracle.decode(bits, oe)


PAIRS = [  # two calls in a row: (elem, trans_b, out, M, N, K, splits, schedule); the second is smaller
    [("f16", 1, "same", 512, 4096, 8192, 4, mcs.GEMM_SCHED_AUTO),       # 32 MiB of partials: the limit
     ("f16", 1, "same", 300, 520, 2000, 3, mcs.GEMM_SCHED_AUTO)],
    [("bf16", 0, "f32", 1024, 1024, 4096, 4, mcs.GEMM_SCHED_PIPELINED),
     ("bf16", 0, "f32", 264, 256, 3000, 4, mcs.GEMM_SCHED_TILE128)],
    [("fp8", 1, "bf16", 768, 1024, 4096, 5, mcs.GEMM_SCHED_INTERLEAVED),
     ("fp8", 1, "bf16", 258, 130, 1008, 3, mcs.GEMM_SCHED_AUTO)],
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}-{p[0][3]}x{p[0][4]}x{p[0][5]}")
def test_noalloc_splitk_matches_workspace_splitk(pair):
    for n, (elem, trans_b, out, M, N, K, splits, schedule) in enumerate(pair):
        print(f"[gpu] noalloc call {n}: {elem} tb={trans_b} out={out} {M}x{N}x{K} splits={splits} "
              f"sched={schedule}", flush=True)
        a = si.matrix_bits(elem, "normal", M, K, seed=9500 + n + M, stream=0)
        b = (si.matrix_bits(elem, "normal", N, K, seed=9500 + n + M, stream=1) if trans_b
             else si.matrix_bits(elem, "normal", K, N, seed=9500 + n + M, stream=1))
        need = mcs.gemm_splitk_workspace_bytes(DT[elem], M, N, K, splits)
        assert 0 < need <= mcs.GEMM_SPLITK_SCRATCH_BYTES
        A, _ = upload(a, elem)
        B, _ = upload(b, elem)
        ldc = (N + 7) // 8 * 8 + 8                   # padded output rows must stay untouched
        ref_bits, _ = _call(False, elem, M, N, K, A, a.shape[1], B, b.shape[1], trans_b, out, schedule,
                            splits, ldc)
        bits, vals = _call(True, elem, M, N, K, A, a.shape[1], B, b.shape[1], trans_b, out, schedule,
                           splits, ldc)
        diff = np.argwhere(bits != ref_bits)
        assert diff.size == 0, f"call {n}: {len(diff)} elements differ from gemm_ex_splitk, first {diff[0]}"
        assert np.all(vals[:, N:] == -3.0)
        cref, sabs = oracle.gemm(a, b, elem, trans_b)
        assert_within_tolerance(vals[:, :N], cref, sabs, f"noalloc call {n}", out=out_elem(elem, out))
