/*
 * mcs_gemm.h -- C ABI of libmcs_gemm.so, a gfx950 (MI355X) dense GEMM
 *
 *     C = A . B        FP16, BF16 or FP8 (E4M3) operands, FP32 accumulation,
 *                      FP16/BF16 (same as the operands; BF16 for FP8
 *                      operands) or FP32 output.
 *
 * The operation is the tiled dense product of "Two Waves, One Stage Apart:
 * Warp-Pipelining Triton GEMMs on AMD Instinct" (opening section: the loop
 * overlaps the matrix work on the current K-step with fetching the operands
 * of later ones; throughput is 2MNK / elapsed time, Table 1).  The kernel holds
 * two wave groups one stage apart (sections "Two Waves, One Stage Apart",
 * "Creating and Closing the Offset", "MI350 Series (gfx950, CDNA 4): Three
 * Overlapping Flows"); its buffer-resource loads with out-of-range reads
 * returning zero follow "Porting High-Performance HIP Kernels to FlyDSL",
 * section "Buffer Resource Descriptors".  The FP8 product is the second GEMM
 * of that page (section "MFMA in FlyDSL": E4M3 operands through the scaled
 * 16x16x128 MFMA with unit scales, B given transposed).
 *
 * Definition (every element, exactly up to FP32 rounding):
 *     C[i*ldc + j] = sum_{k<K} A[i*lda + k] * b(k, j)
 *     b(k, j) = B[k*ldb + j]   if trans_b == 0   (B stored K x N, row-major)
 *             = B[j*ldb + k]   if trans_b == 1   (B stored N x K, row-major)
 * All matrices are row-major; leading dimensions are in ELEMENTS.  C is
 * overwritten (no alpha/beta).  K == 0 writes zeros.  M == 0 or N == 0 is a
 * no-op.  The FP32 -> FP16/BF16 output conversion rounds to nearest even.
 *
 * Ownership and threading: the caller owns every buffer and the stream.  The
 * library keeps no per-call state and allocates nothing, so calls from
 * several host threads are safe.  Every call is ASYNCHRONOUS: it validates,
 * enqueues one kernel on `stream` (0 = the null stream) and returns; the
 * caller synchronises.  C must not overlap A or B.
 *
 * Errors are reported before anything is enqueued (nothing runs on error):
 *   GEMM_EINVAL       null pointer where data is needed, negative size,
 *                     leading dimension below its minimum, bad flag value;
 *   GEMM_EALIGN       A, B or C not 16-byte aligned, lda or ldb times the
 *                     element size not a multiple of 16 bytes, or ldc not a
 *                     multiple of 8 elements (the MFMA kernels move 16 bytes
 *                     per lane);
 *   GEMM_EUNSUPPORTED a shape the MFMA kernels do not cover: K times the
 *                     element size not a multiple of 16 bytes, an odd N with
 *                     B given K x N, FP8 with B given K x N, rows of A or B
 *                     of 2^24 bytes or more; or a size they cannot index
 *                     (any dimension or leading dimension >= 2^31, or more
 *                     than 2^31-1 tiles);
 *   GEMM_EHIP         the launch itself failed (hipGetLastError() holds it).
 * gemm_f16, gemm_bf16 and gemm_fp8 only ever run the MFMA kernels.  A plain
 * FMA kernel that takes any alignment and shape is available, on request
 * only, as gemm_ex(..., GEMM_SCHED_GENERIC, ...).
 */
#ifndef MCS_GEMM_H
#define MCS_GEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gemm_status {
    GEMM_OK = 0,
    GEMM_EINVAL = -1,
    GEMM_EALIGN = -2,
    GEMM_EUNSUPPORTED = -3,
    GEMM_EHIP = -4,
    GEMM_ENOSCRATCH = -5   /* gemm_ex_splitk_noalloc: partials exceed its scratch */
};

enum gemm_out_type {
    GEMM_OUT_SAME = 0,   /* FP16 for gemm_f16, BF16 for gemm_bf16; not for FP8 */
    GEMM_OUT_F32 = 1,
    GEMM_OUT_BF16 = 2    /* BF16: FP8 and BF16 operands */
};

enum gemm_dtype {
    GEMM_DTYPE_F16 = 0,
    GEMM_DTYPE_BF16 = 1,
    GEMM_DTYPE_FP8_E4M3 = 2   /* OCP FP8 E4M3 (no infinities), one byte */
};

/* Kernel schedule selector for gemm_ex. */
enum gemm_schedule {
    GEMM_SCHED_AUTO = 0,       /* what gemm_f16 / gemm_bf16 / gemm_fp8 use:
                                  PIPELINED, or TILE128 for products with
                                  fewer than 128 output tiles of 256x256
                                  (gemm_auto_schedule) */
    GEMM_SCHED_PIPELINED = 1,  /* 8 waves, two groups held one stage apart */
    GEMM_SCHED_IN_PHASE = 2,   /* same kernel and stages, groups kept in phase
                                  (no entry/exit offset): the ablation baseline */
    GEMM_SCHED_GENERIC = 3,    /* plain LDS-tiled FMA kernel, no MFMA: any
                                  alignment and shape, on request only */
    GEMM_SCHED_INTERLEAVED = 4, /* 4 waves, one per SIMD, each interleaving its
                                  own MFMA, LDS reads and copies ("Porting
                                  High-Performance HIP Kernels to FlyDSL",
                                  section "A More Complex Kernel"); same tile,
                                  loader, LDS layout and epilogue as PIPELINED:
                                  the ablation of warp-pipelining itself */
    GEMM_SCHED_TILE128 = 5     /* 128x128 output tiles, 4 waves, a ring of four
                                  K-step buffers in LDS: for products with few
                                  256x256 tiles; same operand conditions as
                                  PIPELINED */
};

/*
 * gemm_f16 / gemm_bf16 -- C = A . B with FP16 / BF16 operands.
 *   M, N, K    sizes (>= 0)
 *   A          device pointer, M x K operand, row stride lda >= max(K, 1)
 *   B          device pointer, K x N (trans_b = 0, ldb >= max(N, 1)) or
 *              N x K (trans_b = 1, ldb >= max(K, 1))
 *   C          device pointer, M x N result, row stride ldc >= max(N, 1);
 *              element type set by out_type (gemm_out_type)
 *   stream     HIP stream the kernel is enqueued on
 * Returns a gemm_status (GEMM_EALIGN / GEMM_EUNSUPPORTED for operands the
 * MFMA kernels cannot take, see above).
 */
int gemm_f16(int64_t M, int64_t N, int64_t K,
             const void *A, int64_t lda,
             const void *B, int64_t ldb, int trans_b,
             void *C, int64_t ldc, int out_type,
             hipStream_t stream);

int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const void *A, int64_t lda,
              const void *B, int64_t ldb, int trans_b,
              void *C, int64_t ldc, int out_type,
              hipStream_t stream);

/*
 * gemm_fp8 -- C = A . B with FP8 E4M3 operands (one byte per element, leading
 * dimensions in elements), FP32 accumulation; out_type GEMM_OUT_BF16 or
 * GEMM_OUT_F32 (GEMM_OUT_SAME is GEMM_EINVAL).  Other arguments as gemm_f16.
 * The MFMA kernels take B given N x K (trans_b = 1) only; B given K x N is
 * GEMM_EUNSUPPORTED here (gemm_ex with GEMM_SCHED_GENERIC takes it).  NaN
 * operands (0x7F, 0xFF) propagate.
 */
int gemm_fp8(int64_t M, int64_t N, int64_t K,
             const void *A, int64_t lda,
             const void *B, int64_t ldb, int trans_b,
             void *C, int64_t ldc, int out_type,
             hipStream_t stream);

/*
 * gemm_ex -- the same product with the operand type (gemm_dtype) and the
 * kernel schedule (gemm_schedule) chosen by the caller.  AUTO, PIPELINED,
 * IN_PHASE, INTERLEAVED and TILE128 run MFMA kernels and return GEMM_EALIGN
 * or GEMM_EUNSUPPORTED (nothing launched) for operands they cannot take, as
 * gemm_f16 does; GENERIC runs the plain FMA kernel on any operands.
 */
int gemm_ex(int dtype, int64_t M, int64_t N, int64_t K,
            const void *A, int64_t lda,
            const void *B, int64_t ldb, int trans_b,
            void *C, int64_t ldc, int out_type, int schedule,
            hipStream_t stream);

/* The tiled schedule AUTO runs for an M x N product: GEMM_SCHED_PIPELINED,
 * or GEMM_SCHED_TILE128 when there are fewer than 128 output tiles of
 * 256x256 (half of MI355X's compute units).  GEMM_EINVAL for negative sizes.
 * No device call. */
int gemm_auto_schedule(int64_t M, int64_t N);

/*
 * Split K for products with few output tiles (shapes whose 256x256 tiles
 * cannot fill the GPU; the pages' kernels take one workgroup per output tile,
 * this entry point is not from them).  gemm_ex_splitk computes the same C as
 * gemm_ex in two kernels on `stream`: the K range is cut into at most
 * `splits` slices of whole K-steps, each slice's FP32 partial product is
 * written to `workspace` by the tiled kernel of `schedule` (AUTO: the one
 * gemm_auto_schedule names), and a second kernel sums the slices in order
 * and writes C
 * rounded to out_type.  The caller owns the workspace (device memory, 16-byte
 * aligned, at least the size gemm_splitk_workspace_bytes reports); the
 * library allocates nothing.  Calls that share a workspace must not overlap.
 *   splits     1 .. 256; 1, or a K too short for two slices, runs gemm_ex
 *              (no workspace needed)
 * Returns GEMM_EINVAL for a missing, misaligned or too small workspace or
 * for schedule GENERIC; GEMM_EALIGN / GEMM_EUNSUPPORTED for operands the
 * MFMA kernels cannot take (as gemm_ex), and GEMM_EUNSUPPORTED when the
 * workspace size does not fit in int64_t.
 */
int gemm_ex_splitk(int dtype, int64_t M, int64_t N, int64_t K,
                   const void *A, int64_t lda,
                   const void *B, int64_t ldb, int trans_b,
                   void *C, int64_t ldc, int out_type, int schedule,
                   int splits, void *workspace, int64_t workspace_bytes,
                   hipStream_t stream);

/*
 * gemm_ex_splitk_noalloc -- gemm_ex_splitk for callers that cannot allocate
 * (code under HIP graph capture, serving loops that forbid hipMalloc,
 * harnesses without an allocator): the same product, kernels and results,
 * bit for bit, with the FP32 partials kept in a device array of the library
 * instead of a caller workspace.  The call allocates nothing and calls no
 * allocating routine.
 *   The array holds GEMM_SPLITK_SCRATCH_BYTES (32 MiB); every GPU the
 *   library runs on keeps its own copy until the process ends.  Products
 *   whose partials need more (gemm_splitk_workspace_bytes for the same
 *   sizes and splits) return GEMM_ENOSCRATCH before anything is enqueued.
 *   Products that would not split (splits 1, or K too short) run gemm_ex.
 *   All calls on one GPU share its array: calls that overlap in time on one
 *   GPU (several streams or host threads) race on the partials and give
 *   wrong results; serialise them.  The device is the one `stream` belongs
 *   to.  On its first call on a device the library looks up that device's
 *   copy (hipGetSymbolAddress, which may load the code object there).
 * Other arguments and errors as gemm_ex_splitk, minus the workspace.
 */
#define GEMM_SPLITK_SCRATCH_BYTES ((int64_t)32 << 20)

int gemm_ex_splitk_noalloc(int dtype, int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t lda,
                           const void *B, int64_t ldb, int trans_b,
                           void *C, int64_t ldc, int out_type, int schedule,
                           int splits, hipStream_t stream);

/* Workspace bytes gemm_ex_splitk needs for these sizes and splits (0 when it
 * would not split).  Returns a gemm_status: GEMM_EINVAL for a null `bytes`,
 * negative sizes or splits outside 1 .. 256, GEMM_EUNSUPPORTED for a size
 * that does not fit in int64_t. */
int gemm_splitk_workspace_bytes(int dtype, int64_t M, int64_t N, int64_t K, int splits,
                                int64_t *bytes);

/* A split count for gemm_ex_splitk with AUTO: 1 unless the output tiles of
 * the kernel AUTO picks fill fewer than `cus` compute units (0 = 256,
 * MI355X) and every slice keeps at least 64 K-steps of 128 bytes; then as
 * many slices as the idle CUs allow.  (Each slice pays the pipeline's fill
 * and drain and the workspace traffic: on MI355X the 512x4096x8192 FP16
 * product on 128x128 tiles runs 54.1 us unsplit and 44.7 us with 2 slices,
 * while 1024^3, with 16 K-steps, only loses.) */
int gemm_splitk_suggest(int dtype, int64_t M, int64_t N, int64_t K, int cus);

/* Static description of one compiled kernel variant (from the code object). */
typedef struct gemm_kernel_attrs {
    int num_regs;          /* VGPRs per lane as reported by the runtime */
    int local_bytes;       /* private (scratch) bytes per lane: 0 means no spills */
    int shared_bytes;      /* static LDS per workgroup */
    int max_threads;       /* maximum workgroup size */
    int block_threads;     /* workgroup size the library launches */
    int tile_m, tile_n, tile_k;
} gemm_kernel_attrs;

/*
 * gemm_kernel_info -- attributes of the kernel gemm_ex would launch for
 * (dtype, trans_b, out_type, schedule).  Needs a HIP device.  Returns a
 * gemm_status (GEMM_EUNSUPPORTED for a combination no 256x256 kernel is
 * compiled for: FP8 with B given K x N); *out is filled on GEMM_OK.
 */
int gemm_kernel_info(int dtype, int trans_b, int out_type, int schedule,
                     gemm_kernel_attrs *out);

/* Static text for a gemm_status value. */
const char *gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MCS_GEMM_H */
