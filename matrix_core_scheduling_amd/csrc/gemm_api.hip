// C-ABI entry points of libmcs_gemm.so (declared in include/mcs_gemm.h).
//
// Every check runs before any HIP call, so argument errors are reported
// without touching the device; the kernel is then enqueued on the caller's
// stream and the call returns without synchronising.  The boundary follows
// the launcher shape of "Porting High-Performance HIP Kernels to FlyDSL"
// (section "A More Complex Kernel": pointers plus the caller's stream, the
// kernel compiled ahead of time) with the sizes passed at run time.
#include "mcs_gemm.h"

#include <atomic>
#include <mutex>

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

// Can the tiled MFMA kernels take these operands?  GEMM_EALIGN: a pointer or
// a leading dimension that 16-byte loads and stores cannot use (A, B and C
// 16-byte aligned; lda and ldb whole 16-byte multiples; ldc a multiple of 8
// elements).  GEMM_EUNSUPPORTED: a shape they do not cover -- a K extent that
// is not a whole number of 16-byte chunks (copies move whole chunks), an odd
// N with B given K x N (a K x N row is copied in whole dwords up to its last
// valid column), FP8 with B given K x N, or rows of 2^24 bytes or more (128
// rows of one copy window must stay below 2^31 bytes of buffer offset).
int tiled_status(int elem, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                 int64_t ldb, int trans_b, const void *C, int64_t ldc) {
    const int64_t eb = mcs::elem_bytes(elem);
    if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return GEMM_EALIGN;
    if ((lda * eb) % 16 || (ldb * eb) % 16 || ldc % 8) return GEMM_EALIGN;
    if ((K * eb) % 16) return GEMM_EUNSUPPORTED;
    if (lda * eb >= kMaxRowBytes || ldb * eb >= kMaxRowBytes) return GEMM_EUNSUPPORTED;
    if (!trans_b && (elem == mcs::kElemFP8 || N % 2)) return GEMM_EUNSUPPORTED;
    return GEMM_OK;
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
    if (schedule < GEMM_SCHED_AUTO || schedule > GEMM_SCHED_TILE128) return GEMM_EINVAL;
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
    prm.stagger_seed = mcs::next_stagger_seed();
    void *args[] = {&prm};
    return to_status(hipLaunchKernel(fn, grid, block, args, 0, stream));
}

// One of the tiled MFMA kernels over `slices` K-slices of kslice elements
// each (slices == 1: the whole product into C).  prm holds A, B, C, sizes and
// leading dimensions; tiles, steps and the slice fields are filled here.
int launch_tiles(int elem, int trans_b, bool out_f32, int schedule, GemmParams &prm, int64_t kslice,
                 int slices, hipStream_t stream) {
    const int64_t edge = schedule == GEMM_SCHED_TILE128 ? mcs::kTile128 : mcs::kTileM;
    const int64_t tm = (prm.M + edge - 1) / edge;
    const int64_t tn = (prm.N + edge - 1) / edge;
    if (tm * tn > kIntMax) return GEMM_EUNSUPPORTED;
    const int64_t nk = (kslice + mcs::step_k(elem) - 1) / mcs::step_k(elem);
    prm.tiles_m = static_cast<int>(tm);
    prm.tiles_n = static_cast<int>(tn);
    prm.group_m = 4;
    prm.kslice = static_cast<int>(kslice);
    const dim3 grid(static_cast<unsigned>(tm * tn), static_cast<unsigned>(slices));
    if (schedule == GEMM_SCHED_INTERLEAVED) {
        prm.steps = static_cast<int>(nk);   // one K-step per loop iteration
        return launch(mcs::interleaved_kernel(elem, trans_b != 0, out_f32), grid,
                      dim3(mcs::kInterThreads), prm, stream);
    }
    prm.steps = static_cast<int>(nk < 2 ? 2 : (nk + 1) / 2 * 2);
    if (schedule == GEMM_SCHED_TILE128) {
        if (elem != mcs::kElemFP8) prm.steps = static_cast<int>(nk);   // one K-step per iteration
        return launch(mcs::tile128_kernel(elem, trans_b != 0, out_f32), grid,
                      dim3(mcs::kTile128Threads), prm, stream);
    }
    return launch(mcs::pipelined_kernel(elem, trans_b != 0, out_f32, schedule == GEMM_SCHED_PIPELINED),
                  grid, dim3(mcs::kPipeThreads), prm, stream);
}

constexpr int kMaxSplits = 256;

// K-slice length (a whole number of K-steps) and slice count for a request
// of `splits` slices.
void split_plan(int elem, int64_t K, int splits, int64_t &kslice, int &slices) {
    const int64_t sk = mcs::step_k(elem);
    const int64_t steps = (K + sk - 1) / sk;
    const int64_t per = (steps + splits - 1) / splits;
    kslice = per * sk;
    slices = static_cast<int>((K + kslice - 1) / kslice);
}

int64_t ws_row(int64_t N) { return (N + 3) / 4 * 4; }

// Bytes of `slices` FP32 partial products of M rows of ws_row(N) floats, or
// -1 where that count does not fit in int64_t (M and N up to 2^31 - 1).
int64_t ws_bytes(int64_t slices, int64_t M, int64_t N) {
    const int64_t row = ws_row(N) * 4;
    if (M > INT64_MAX / row / slices) return -1;
    return slices * M * row;
}

// The tiled kernel AUTO runs for aligned operands: the 256x256 warp-pipelined
// kernel, or the 128x128-tile kernel when the product has fewer 256x256 tiles
// than half of MI355X's 256 compute units (measured: 1024^3 22.1 -> 10.6 us,
// 2048x2048x8192 124.7 -> 70.1 us; 3072x3072x4096, 144 tiles, stays faster on
// the 256x256 kernel, 75.0 against 99.8 us).
constexpr int64_t kChipCUs = 256;
int auto_tiled_schedule(int64_t M, int64_t N) {
    const int64_t tiles = ((M + mcs::kTileM - 1) / mcs::kTileM) * ((N + mcs::kTileN - 1) / mcs::kTileN);
    return tiles < kChipCUs / 2 ? GEMM_SCHED_TILE128 : GEMM_SCHED_PIPELINED;
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

    if (schedule == GEMM_SCHED_GENERIC) {
        const int64_t gx = (N + mcs::kGenTile - 1) / mcs::kGenTile;
        const int64_t gy = (M + mcs::kGenTile - 1) / mcs::kGenTile;
        if (gx > kIntMax || gy > 65535) return GEMM_EUNSUPPORTED;
        return launch(mcs::generic_kernel(elem, trans_b != 0, out_f32),
                      dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                      dim3(mcs::kGenThreads), prm, stream);
    }

    const int st = tiled_status(elem, N, K, A, lda, B, ldb, trans_b, C, ldc);
    if (st != GEMM_OK) return st;
    if (schedule == GEMM_SCHED_AUTO) schedule = auto_tiled_schedule(M, N);
    return launch_tiles(elem, trans_b, out_f32, schedule, prm, K, 1, stream);
}

extern "C" int gemm_splitk_workspace_bytes(int dtype, int64_t M, int64_t N, int64_t K, int splits,
                                           int64_t *bytes) {
    if (!bytes || splits < 1 || splits > kMaxSplits || M < 0 || N < 0 || K < 0) return GEMM_EINVAL;
    if (dtype < GEMM_DTYPE_F16 || dtype > GEMM_DTYPE_FP8_E4M3) return GEMM_EINVAL;
    if (M > kIntMax || N > kIntMax || K > kIntMax) return GEMM_EUNSUPPORTED;
    int64_t kslice = 0;
    int slices = 1;
    if (K > 0) split_plan(elem_of(dtype), K, splits, kslice, slices);
    const int64_t need = slices > 1 && M > 0 && N > 0 ? ws_bytes(slices, M, N) : 0;
    if (need < 0) return GEMM_EUNSUPPORTED;
    *bytes = need;
    return GEMM_OK;
}

extern "C" int gemm_auto_schedule(int64_t M, int64_t N) {
    if (M < 0 || N < 0) return GEMM_EINVAL;
    return auto_tiled_schedule(M, N);
}

extern "C" int gemm_splitk_suggest(int dtype, int64_t M, int64_t N, int64_t K, int cus) {
    if (dtype < GEMM_DTYPE_F16 || dtype > GEMM_DTYPE_FP8_E4M3 || M <= 0 || N <= 0 || K <= 0) return 1;
    if (cus <= 0) cus = kChipCUs;
    const int64_t edge = auto_tiled_schedule(M, N) == GEMM_SCHED_TILE128 ? mcs::kTile128 : mcs::kTileM;
    const int64_t tiles = ((M + edge - 1) / edge) * ((N + edge - 1) / edge);
    const int64_t steps = (K + mcs::step_k(elem_of(dtype)) - 1) / mcs::step_k(elem_of(dtype));
    int64_t s = steps / 64;                          // at least 64 K-steps per slice
    if (cus / tiles < s) s = cus / tiles;            // no more workgroups than CUs
    return static_cast<int>(s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s));
}

namespace {

// The split-K product: validation, then the slices' FP32 partials into the
// workspace the caller gives (ws_kind kCallerWorkspace) or into the static
// scratch array below (kStaticScratch, which the caller cannot see).
enum WsKind { kCallerWorkspace, kStaticScratch };
int scratch_address(hipStream_t stream, void **out);

int splitk(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
           int64_t ldb, int trans_b, void *C, int64_t ldc, int out_type, int schedule, int splits,
           WsKind ws_kind, void *workspace, int64_t workspace_bytes, hipStream_t stream) {
    const int v = validate(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule);
    if (v != GEMM_OK) return v;
    if (splits < 1 || splits > kMaxSplits || schedule == GEMM_SCHED_GENERIC) return GEMM_EINVAL;
    if (M == 0 || N == 0) return GEMM_OK;
    const int elem = elem_of(dtype);
    int64_t kslice = 0;
    int slices = 1;
    if (K > 0) split_plan(elem, K, splits, kslice, slices);
    if (slices == 1)
        return gemm_ex(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule, stream);
    const int tst = tiled_status(elem, N, K, A, lda, B, ldb, trans_b, C, ldc);
    if (tst != GEMM_OK) return tst;
    const int64_t need = ws_bytes(slices, M, N);
    if (need < 0) return GEMM_EUNSUPPORTED;
    if (ws_kind == kStaticScratch) {
        if (need > GEMM_SPLITK_SCRATCH_BYTES) return GEMM_ENOSCRATCH;
        const int st = scratch_address(stream, &workspace);
        if (st != GEMM_OK) return st;
    } else if (!workspace || !aligned16(workspace) || workspace_bytes < need) {
        return GEMM_EINVAL;
    }
    if (schedule == GEMM_SCHED_AUTO) schedule = auto_tiled_schedule(M, N);

    GemmParams prm{};
    prm.A = A;
    prm.B = B;
    prm.C = C;
    prm.lda = lda;
    prm.ldb = ldb;
    prm.ldc = ldc;
    prm.M = static_cast<int>(M);
    prm.N = static_cast<int>(N);
    prm.K = static_cast<int>(K);
    prm.ws = static_cast<float *>(workspace);
    prm.ldws = ws_row(N);
    // pass 1: the FP32 partial product of every K-slice
    int st = launch_tiles(elem, trans_b, true, schedule, prm, kslice, slices, stream);
    if (st != GEMM_OK) return st;
    // pass 2: sum the slices in order, round to the output type, write C
    const int out_kind = out_type == GEMM_OUT_F32 ? 2 : (elem == mcs::kElemF16 ? 0 : 1);
    const int64_t items = M * ((N + 3) / 4);
    int64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    void *args[] = {&prm, &slices};
    return to_status(hipLaunchKernel(mcs::splitk_reduce_kernel(out_kind),
                                     dim3(static_cast<unsigned>(blocks)), dim3(256), args, 0, stream));
}

// ---- the allocation-free split K ------------------------------------------
//
// The FP32 partials of gemm_ex_splitk_noalloc live in this file-scope device
// array.  Every GPU the library runs on holds its own copy from the moment
// the code object is loaded until the process ends.  Host code never uses
// the array's name as an address: on the host it is only a stand-in that the
// runtime maps to each device's copy.  scratch_address asks the runtime for
// that device address once per device, with the device current, and keeps
// it; kernels only ever receive the kept address.  The slice kernels write
// every partial element the reduction reads for its output (it also reads,
// and discards, up to three pad columns per row), so nothing has to be
// cleared between calls.
static __device__ __align__(256) float scratch[GEMM_SPLITK_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

int scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return GEMM_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return GEMM_EUNSUPPORTED;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = -1;
            if (hipGetDevice(&cur) != hipSuccess) return GEMM_EHIP;
            if (cur != dev && hipSetDevice(dev) != hipSuccess) return GEMM_EHIP;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (cur != dev && hipSetDevice(cur) != hipSuccess) return GEMM_EHIP;
            if (e != hipSuccess || !p) return GEMM_EHIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return GEMM_OK;
}

}  // namespace

extern "C" int gemm_ex_splitk(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                              const void *B, int64_t ldb, int trans_b, void *C, int64_t ldc,
                              int out_type, int schedule, int splits, void *workspace,
                              int64_t workspace_bytes, hipStream_t stream) {
    return splitk(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule, splits,
                  kCallerWorkspace, workspace, workspace_bytes, stream);
}

extern "C" int gemm_ex_splitk_noalloc(int dtype, int64_t M, int64_t N, int64_t K, const void *A,
                                      int64_t lda, const void *B, int64_t ldb, int trans_b, void *C,
                                      int64_t ldc, int out_type, int schedule, int splits,
                                      hipStream_t stream) {
    return splitk(dtype, M, N, K, A, lda, B, ldb, trans_b, C, ldc, out_type, schedule, splits,
                  kStaticScratch, nullptr, 0, stream);
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
    } else if (schedule == GEMM_SCHED_TILE128) {
        fn = mcs::tile128_kernel(elem, trans_b != 0, out_f32);
        threads = mcs::kTile128Threads;
        tm = tn = mcs::kTile128; tk = mcs::step_k(elem);
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
        case GEMM_EALIGN: return "GEMM_EALIGN: pointer or leading dimension not 16-byte aligned";
        case GEMM_EUNSUPPORTED: return "GEMM_EUNSUPPORTED: shape or size the kernel does not cover";
        case GEMM_EHIP: return "GEMM_EHIP: HIP launch failure (see hipGetLastError)";
        case GEMM_ENOSCRATCH:
            return "GEMM_ENOSCRATCH: split-K partials larger than the library's static scratch "
                   "(GEMM_SPLITK_SCRATCH_BYTES)";
        default: return "unknown gemm_status";
    }
}
