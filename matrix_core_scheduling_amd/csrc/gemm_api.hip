// C-ABI entry points of libmcs_gemm.so (declared in include/mcs_gemm.h).
//
// Every check runs before any HIP call, so argument errors are reported
// without touching the device; the kernel is then enqueued on the caller's
// stream and the call returns without synchronising.  The boundary follows
// the launcher shape of "Porting High-Performance HIP Kernels to FlyDSL"
// (section "A More Complex Kernel": pointers plus the caller's stream, the
// kernel compiled ahead of time) with the sizes passed at run time.
#include "mcs_gemm.h"

#include "internal.h"

namespace {

using mcs::GemmParams;

constexpr int64_t kIntMax = 0x7FFFFFFF;
constexpr int64_t kMaxRowBytes = int64_t(1) << 24;    // keeps 128 rows of a copy window < 2^31 bytes

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int elem_of(int dtype) {
    return dtype == GEMM_DTYPE_FP8_E4M3 ? mcs::kElemFP8
         : dtype == GEMM_DTYPE_BF16 ? mcs::kElemBF16 : mcs::kElemF16;
}

// Can the 256x256 kernels take these operands?
bool pipelined_ok(int elem, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                  int64_t ldb, int trans_b, const void *C, int64_t ldc) {
    const int64_t eb = mcs::elem_bytes(elem);
    if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return false;
    if ((lda * eb) % 16 || (ldb * eb) % 16 || (K * eb) % 16 || ldc % 8) return false;
    if (lda * eb >= kMaxRowBytes || ldb * eb >= kMaxRowBytes) return false;
    if (!trans_b) {
        if (elem == mcs::kElemFP8) return false;
        // A K x N operand is copied in whole dwords up to the last valid column.
        if (N % 2) return false;
    }
    return true;
}

bool out_ok(int dtype, int out_type) {
    switch (out_type) {
        case GEMM_OUT_SAME: return dtype != GEMM_DTYPE_FP8_E4M3;
        case GEMM_OUT_F32: return true;
        case GEMM_OUT_BF16: return dtype != GEMM_DTYPE_F16;
        default: return false;
    }
}

int validate(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
             int64_t ldb, int trans_b, const void *C, int64_t ldc, int out_type, int schedule) {
    if (dtype < GEMM_DTYPE_F16 || dtype > GEMM_DTYPE_FP8_E4M3) return GEMM_EINVAL;
    if (trans_b != 0 && trans_b != 1) return GEMM_EINVAL;
    if (!out_ok(dtype, out_type)) return GEMM_EINVAL;
    if (schedule < GEMM_SCHED_AUTO || schedule > GEMM_SCHED_INTERLEAVED) return GEMM_EINVAL;
    if (M < 0 || N < 0 || K < 0) return GEMM_EINVAL;
    if (M > kIntMax || N > kIntMax || K > kIntMax) return GEMM_EUNSUPPORTED;
    if (M == 0 || N == 0) return GEMM_OK;
    if (lda < (K > 1 ? K : 1) || ldc < N) return GEMM_EINVAL;
    if (ldb < (trans_b ? (K > 1 ? K : 1) : N)) return GEMM_EINVAL;
    if (lda > kIntMax || ldb > kIntMax || ldc > kIntMax) return GEMM_EUNSUPPORTED;
    if (!C) return GEMM_EINVAL;
    if (K > 0 && (!A || !B)) return GEMM_EINVAL;
    return GEMM_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? GEMM_OK : GEMM_EHIP; }

int launch(const void *fn, dim3 grid, dim3 block, GemmParams &prm, hipStream_t stream) {
    void *args[] = {&prm};
    return to_status(hipLaunchKernel(fn, grid, block, args, 0, stream));
}

}  // namespace

extern "C" int gemm_ex(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                       const void *B, int64_t ldb, int trans_b, void *C, int64_t ldc, int out_type,
                       int schedule, hipStream_t stream) {
    const int v = validate(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule);
    if (v != GEMM_OK || M == 0 || N == 0) return v;

    const int elem = elem_of(dtype);
    const bool out_f32 = out_type == GEMM_OUT_F32;
    GemmParams prm{};
    prm.A = static_cast<const uint16_t *>(A);
    prm.B = static_cast<const uint16_t *>(B);
    prm.C = C;
    prm.lda = lda;
    prm.ldb = ldb;
    prm.ldc = ldc;
    prm.M = static_cast<int>(M);
    prm.N = static_cast<int>(N);
    prm.K = static_cast<int>(K);

    if (K == 0) {
        const int64_t total = M * N;
        int64_t blocks = (total + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        return launch(mcs::zero_fill_kernel(out_f32), dim3(static_cast<unsigned>(blocks)), dim3(256),
                      prm, stream);
    }

    const bool fast = pipelined_ok(elem, N, K, A, lda, B, ldb, trans_b, C, ldc);
    if (schedule == GEMM_SCHED_AUTO) schedule = fast ? GEMM_SCHED_PIPELINED : GEMM_SCHED_GENERIC;
    if (schedule != GEMM_SCHED_GENERIC && !fast) return GEMM_EINVAL;

    if (schedule == GEMM_SCHED_GENERIC) {
        const int64_t gx = (N + mcs::kGenTile - 1) / mcs::kGenTile;
        const int64_t gy = (M + mcs::kGenTile - 1) / mcs::kGenTile;
        if (gx > kIntMax || gy > 65535) return GEMM_EUNSUPPORTED;
        return launch(mcs::generic_kernel(elem, trans_b != 0, out_f32),
                      dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                      dim3(mcs::kGenThreads), prm, stream);
    }

    const int64_t tm = (M + mcs::kTileM - 1) / mcs::kTileM;
    const int64_t tn = (N + mcs::kTileN - 1) / mcs::kTileN;
    if (tm * tn > kIntMax) return GEMM_EUNSUPPORTED;
    const int64_t nk = (K + mcs::step_k(elem) - 1) / mcs::step_k(elem);
    prm.tiles_m = static_cast<int>(tm);
    prm.tiles_n = static_cast<int>(tn);
    prm.steps = static_cast<int>(nk < 2 ? 2 : (nk + 1) / 2 * 2);
    prm.group_m = 4;
    if (schedule == GEMM_SCHED_INTERLEAVED) {
        prm.steps = static_cast<int>(nk);   // one K-step per loop iteration
        return launch(mcs::interleaved_kernel(elem, trans_b != 0, out_f32),
                      dim3(static_cast<unsigned>(tm * tn)), dim3(mcs::kInterThreads), prm, stream);
    }
    return launch(mcs::pipelined_kernel(elem, trans_b != 0, out_f32, schedule == GEMM_SCHED_PIPELINED),
                  dim3(static_cast<unsigned>(tm * tn)), dim3(mcs::kPipeThreads), prm, stream);
}

extern "C" int gemm_f16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                        int64_t ldb, int trans_b, void *C, int64_t ldc, int out_type,
                        hipStream_t stream) {
    return gemm_ex(GEMM_DTYPE_F16, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type,
                   GEMM_SCHED_AUTO, stream);
}

extern "C" int gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                         int64_t ldb, int trans_b, void *C, int64_t ldc, int out_type,
                         hipStream_t stream) {
    return gemm_ex(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type,
                   GEMM_SCHED_AUTO, stream);
}

extern "C" int gemm_fp8(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                        int64_t ldb, int trans_b, void *C, int64_t ldc, int out_type,
                        hipStream_t stream) {
    return gemm_ex(GEMM_DTYPE_FP8_E4M3, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type,
                   GEMM_SCHED_AUTO, stream);
}

extern "C" int gemm_kernel_info(int dtype, int trans_b, int out_type, int schedule,
                                gemm_kernel_attrs *out) {
    if (!out) return GEMM_EINVAL;
    if (dtype < GEMM_DTYPE_F16 || dtype > GEMM_DTYPE_FP8_E4M3) return GEMM_EINVAL;
    if ((trans_b != 0 && trans_b != 1) || !out_ok(dtype, out_type)) return GEMM_EINVAL;
    const int elem = elem_of(dtype);
    const bool out_f32 = out_type == GEMM_OUT_F32;
    const void *fn = nullptr;
    int threads = 0, tm = 0, tn = 0, tk = 0;
    if (schedule == GEMM_SCHED_AUTO || schedule == GEMM_SCHED_PIPELINED || schedule == GEMM_SCHED_IN_PHASE) {
        fn = mcs::pipelined_kernel(elem, trans_b != 0, out_f32, schedule != GEMM_SCHED_IN_PHASE);
        threads = mcs::kPipeThreads;
        tm = mcs::kTileM; tn = mcs::kTileN; tk = mcs::step_k(elem);
    } else if (schedule == GEMM_SCHED_INTERLEAVED) {
        fn = mcs::interleaved_kernel(elem, trans_b != 0, out_f32);
        threads = mcs::kInterThreads;
        tm = mcs::kTileM; tn = mcs::kTileN; tk = mcs::step_k(elem);
    } else if (schedule == GEMM_SCHED_GENERIC) {
        fn = mcs::generic_kernel(elem, trans_b != 0, out_f32);
        threads = mcs::kGenThreads;
        tm = tn = mcs::kGenTile; tk = 16;
    } else {
        return GEMM_EINVAL;
    }
    if (!fn) return GEMM_EUNSUPPORTED;       // e.g. a 256x256 kernel for FP8 B given K x N
    hipFuncAttributes a{};
    if (hipFuncGetAttributes(&a, fn) != hipSuccess) return GEMM_EHIP;
    out->num_regs = a.numRegs;
    out->local_bytes = static_cast<int>(a.localSizeBytes);
    out->shared_bytes = static_cast<int>(a.sharedSizeBytes);
    out->max_threads = a.maxThreadsPerBlock;
    out->block_threads = threads;
    out->tile_m = tm;
    out->tile_n = tn;
    out->tile_k = tk;
    return GEMM_OK;
}

extern "C" const char *gemm_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "GEMM_OK: success";
        case GEMM_EINVAL: return "GEMM_EINVAL: invalid argument";
        case GEMM_EUNSUPPORTED: return "GEMM_EUNSUPPORTED: size outside what the kernels can index";
        case GEMM_EHIP: return "GEMM_EHIP: HIP launch failure (see hipGetLastError)";
        default: return "unknown gemm_status";
    }
}
