"""Python binding of libmcs_gemm.so: the gfx950 warp-pipelined FP16/BF16/FP8 GEMM
and the attention forward pass built in the same stage abstraction.

The functions ``gemm_f16``, ``gemm_bf16``, ``gemm_fp8``, ``gemm_ex``,
``gemm_ex_splitk``, ``gemm_splitk_workspace_bytes``, ``gemm_auto_schedule``,
``gemm_splitk_suggest``, ``gemm_ex_splitk_noalloc``,
``gemm_kernel_info``, ``gemm_status_string``, ``attention_fwd`` and
``attention_fwd_ex`` mirror the
C ABI in ``include/mcs_gemm.h`` and ``include/mcs_attention.h`` one to one
(sizes, raw device pointers as integers, a raw ``hipStream_t``).  ``gemm``
marshals torch tensors onto them: torch provides device memory and the
current stream, every step of the product runs in the library's HIP kernels;
``attention`` does the same for the attention forward pass.

There is no fallback: if the library is not built, every call raises.
Build it with ``python -m matrix_core_scheduling_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libmcs_gemm.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "mcs_gemm.h")
ATTN_HEADER = os.path.join(os.path.dirname(_PKG), "include", "mcs_attention.h")

GEMM_OK, GEMM_EINVAL, GEMM_EALIGN, GEMM_EUNSUPPORTED, GEMM_EHIP, GEMM_ENOSCRATCH = 0, -1, -2, -3, -4, -5
GEMM_SPLITK_SCRATCH_BYTES = 32 << 20   # the static scratch of gemm_ex_splitk_noalloc
GEMM_OUT_SAME, GEMM_OUT_F32, GEMM_OUT_BF16 = 0, 1, 2
GEMM_DTYPE_F16, GEMM_DTYPE_BF16, GEMM_DTYPE_FP8_E4M3 = 0, 1, 2
GEMM_SCHED_AUTO, GEMM_SCHED_PIPELINED, GEMM_SCHED_IN_PHASE, GEMM_SCHED_GENERIC, GEMM_SCHED_INTERLEAVED = 0, 1, 2, 3, 4
GEMM_SCHED_TILE128 = 5


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {gemm_status_string(status)} ({status})" if what else
                         f"{gemm_status_string(status)} ({status})")


class GemmKernelAttrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("num_regs", "local_bytes", "shared_bytes", "max_threads",
                                            "block_threads", "tile_m", "tile_n", "tile_k")]


_lib = None
_stagger_lib = None

# The race-stress build of the same sources (compiled with MCS_STAGGER: random
# sleeps at every workgroup barrier, NaN-filled LDS at kernel start).  Only the
# tests load it, through load_stagger(); it exports the same C ABI.
STAGGER_LIBRARY = os.path.join(_PKG, "libmcs_gemm_stagger.so")


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m matrix_core_scheduling_amd.build` "
                           "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    sig = [i64, i64, i64, vp, i64, vp, i64, ci, vp, i64, ci]
    for name in ("gemm_f16", "gemm_bf16", "gemm_fp8"):
        f = getattr(lib, name)
        f.argtypes = sig + [vp]
        f.restype = ci
    lib.gemm_ex.argtypes = [ci] + sig + [ci, vp]
    lib.gemm_ex.restype = ci
    lib.gemm_ex_splitk.argtypes = [ci] + sig + [ci, ci, vp, i64, vp]
    lib.gemm_ex_splitk.restype = ci
    lib.gemm_ex_splitk_noalloc.argtypes = [ci] + sig + [ci, ci, vp]
    lib.gemm_ex_splitk_noalloc.restype = ci
    lib.gemm_splitk_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, ctypes.POINTER(i64)]
    lib.gemm_splitk_workspace_bytes.restype = ci
    lib.gemm_auto_schedule.argtypes = [i64, i64]
    lib.gemm_auto_schedule.restype = ci
    lib.gemm_splitk_suggest.argtypes = [ci, i64, i64, i64, ci]
    lib.gemm_splitk_suggest.restype = ci
    lib.gemm_kernel_info.argtypes = [ci, ci, ci, ci, ctypes.POINTER(GemmKernelAttrs)]
    lib.gemm_kernel_info.restype = ci
    lib.attention_fwd.argtypes = [ci, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, ctypes.c_float, ci, vp]
    lib.attention_fwd.restype = ci
    lib.attention_fwd_ex.argtypes = [ci, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, ctypes.c_float, ci, ci, vp]
    lib.attention_fwd_ex.restype = ci
    lib.gemm_status_string.argtypes = [ci]
    lib.gemm_status_string.restype = ctypes.c_char_p
    return lib


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(path)
    return _lib


def load_stagger() -> ctypes.CDLL:
    """Load the race-stress build (once): the same C ABI, for tests only."""
    global _stagger_lib
    if _stagger_lib is None:
        _stagger_lib = _open(STAGGER_LIBRARY)
    return _stagger_lib


def header_functions(paths=(HEADER, ATTN_HEADER)) -> list[str]:
    """Names of the functions the headers under include/ declare."""
    if isinstance(paths, str):
        paths = (paths,)
    names = []
    for path in paths:
        text = open(path).read()
        names += re.findall(r"^(?:int|const char \*)\s*(\w+)\s*\(", text, flags=re.M)
    return names


# ---- the C ABI, one to one --------------------------------------------------

def gemm_f16(M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, stream) -> int:
    return load().gemm_f16(M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, stream)


def gemm_bf16(M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, stream) -> int:
    return load().gemm_bf16(M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, stream)


def gemm_fp8(M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, stream) -> int:
    return load().gemm_fp8(M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, stream)


def gemm_ex(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule, stream) -> int:
    return load().gemm_ex(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule, stream)


def gemm_ex_splitk(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule, splits,
                   workspace, workspace_bytes, stream) -> int:
    return load().gemm_ex_splitk(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule,
                                 splits, workspace, workspace_bytes, stream)


def gemm_ex_splitk_noalloc(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule, splits,
                           stream) -> int:
    return load().gemm_ex_splitk_noalloc(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule,
                                         splits, stream)


def gemm_splitk_workspace_bytes(dtype: int, M: int, N: int, K: int, splits: int) -> int:
    """Bytes of workspace gemm_ex_splitk needs (0 when it would not split)."""
    n = ctypes.c_int64(0)
    st = load().gemm_splitk_workspace_bytes(dtype, M, N, K, splits, ctypes.byref(n))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_splitk_workspace_bytes")
    return n.value


def gemm_auto_schedule(M: int, N: int) -> int:
    return load().gemm_auto_schedule(M, N)


def gemm_splitk_suggest(dtype: int, M: int, N: int, K: int, cus: int = 0) -> int:
    return load().gemm_splitk_suggest(dtype, M, N, K, cus)


def gemm_kernel_info(dtype: int, trans_b: int, out_type: int, schedule: int) -> dict:
    a = GemmKernelAttrs()
    st = load().gemm_kernel_info(dtype, trans_b, out_type, schedule, ctypes.byref(a))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_kernel_info")
    return {n: getattr(a, n) for n, _ in GemmKernelAttrs._fields_}


def gemm_status_string(status: int) -> str:
    return load().gemm_status_string(status).decode()


def attention_fwd(dtype, batch, heads, seq_q, seq_k, head_dim, Q, K, V, O, lse, scale, causal, stream) -> int:
    return load().attention_fwd(dtype, batch, heads, seq_q, seq_k, head_dim, Q, K, V, O, lse, scale,
                                causal, stream)


# ---- torch marshalling ---------------------------------------------------

def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def _same_gpu(*tensors):
    """The kernels dereference every pointer on the GPU: host tensors, or
    tensors on different devices, are refused before any library call."""
    dev = tensors[0].device
    for t in tensors:
        if not t.is_cuda or t.device != dev:
            raise ValueError(f"all tensors must be on one GPU device (got {t.device} and {dev})")


def gemm(A, B, trans_b: bool = False, out=None, out_dtype=None,
         schedule: int = GEMM_SCHED_AUTO, stream=None):
    """C = A @ B (trans_b=False, B is K x N) or A @ B.T (trans_b=True, B is N x K).

    A, B: 2-D float16, bfloat16 or float8_e4m3fn CUDA tensors with unit
    column stride (rows may be padded: the row stride is passed as the
    leading dimension).  ``out`` (M x N, unit column stride) is written in
    place if given; otherwise a tensor of ``out_dtype`` is allocated by torch
    (default: the operand dtype, bfloat16 for FP8 operands; float32 allowed).
    Operands the MFMA kernels cannot take (misaligned views, K not a whole
    number of 16-byte chunks, ...) raise GemmError with GEMM_EALIGN or
    GEMM_EUNSUPPORTED; ``schedule=GEMM_SCHED_GENERIC`` asks for the plain FMA
    kernel, which takes anything.
    Runs on the current stream (or ``stream``) and does not synchronise."""
    import torch

    dtypes = {torch.float16: GEMM_DTYPE_F16, torch.bfloat16: GEMM_DTYPE_BF16,
              torch.float8_e4m3fn: GEMM_DTYPE_FP8_E4M3}
    if A.dtype != B.dtype or A.dtype not in dtypes:
        raise TypeError("A and B must both be float16, bfloat16 or float8_e4m3fn")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    _same_gpu(A, B)
    if A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A and B need unit column stride")
    M, K = A.shape
    if trans_b:
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    fp8 = A.dtype == torch.float8_e4m3fn
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or (torch.bfloat16 if fp8 else A.dtype), device=A.device)
    if out.shape != (M, N) or (out.stride(1) != 1 and N > 1):
        raise ValueError("out must be M x N with unit column stride")
    _same_gpu(A, out)
    if out.dtype == torch.float32:
        out_type = GEMM_OUT_F32
    elif out.dtype == torch.bfloat16 and A.dtype != torch.float16:
        out_type = GEMM_OUT_BF16
    elif out.dtype == A.dtype and not fp8:
        out_type = GEMM_OUT_SAME
    else:
        raise TypeError("out must be float32, or the operand dtype (bfloat16 for FP8 operands)")
    dtype = dtypes[A.dtype]
    lda = A.stride(0) if M > 1 else max(K, 1)
    ldb = B.stride(0) if B.shape[0] > 1 else max(B.shape[1], 1)
    ldc = out.stride(0) if M > 1 else max(N, 1)
    st = gemm_ex(dtype, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, int(bool(trans_b)),
                 out.data_ptr(), ldc, out_type, schedule, _stream_handle(stream))
    if st != GEMM_OK:
        raise GemmError(st, "gemm")
    return out


def attention_fwd_ex(dtype, batch, heads, seq_q, seq_k, head_dim, Q, K, V, O, lse, scale, causal, schedule,
                     stream) -> int:
    return load().attention_fwd_ex(dtype, batch, heads, seq_q, seq_k, head_dim, Q, K, V, O, lse, scale,
                                   causal, schedule, stream)


def attention(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
              with_lse: bool = True, stream=None):
    """Attention forward through ``attention_fwd``: q (B, H, Sq, D), k and v
    (B, H, Sk, D) contiguous float16 or bfloat16 CUDA tensors, D = 128.
    Returns (out, lse) -- out like q, lse float32 (B, H, Sq) or None -- both
    allocated by torch unless given.  Runs on the current stream (or
    ``stream``) and does not synchronise."""
    import math

    import torch

    dtypes = {torch.float16: GEMM_DTYPE_F16, torch.bfloat16: GEMM_DTYPE_BF16}
    if q.dtype not in dtypes or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must all be float16 or all bfloat16")
    if q.dim() != 4 or k.shape != v.shape or k.dim() != 4 or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q (B,H,Sq,D), k and v (B,H,Sk,D) expected")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k and v must be contiguous")
    _same_gpu(q, k, v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    _same_gpu(q, out)
    if with_lse and lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        if lse.dtype != torch.float32 or lse.numel() != B * H * Sq or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 tensor of B*H*Sq elements")
        _same_gpu(q, lse)
    st = attention_fwd(dtypes[q.dtype], B, H, Sq, Sk, D, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                       out.data_ptr(), lse.data_ptr() if lse is not None else None, scale, int(bool(causal)),
                       _stream_handle(stream))
    if st != GEMM_OK:
        raise GemmError(st, "attention")
    return out, lse
