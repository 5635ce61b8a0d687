/*
 * mcs_attention.h -- C ABI of the attention forward pass in libmcs_gemm.so
 * (gfx950, MI355X).
 *
 * The operation is the inner loop "Two Waves, One Stage Apart:
 * Warp-Pipelining Triton GEMMs on AMD Instinct" extends the stage
 * abstraction to (section "Beyond GEMM: FlashAttention", Figure 11): per
 * block of keys, a QK matrix product, an online softmax, and a PV matrix
 * product, with one wave group's matrix work overlapping the other group's
 * softmax and operand movement.  What it computes is plain scaled
 * dot-product attention; for batch b, head h, query row i:
 *
 *     s_ij   = scale * sum_d Q[b,h,i,d] K[b,h,j,d]        (keys j allowed for i)
 *     lse_i  = ln(sum_j exp(s_ij))
 *     O[b,h,i,:] = sum_j exp(s_ij - lse_i) V[b,h,j,:]
 *
 * Allowed keys: all, or with causal != 0 the keys j <= i + (seq_k - seq_q)
 * (masks aligned at the bottom right: the last query row sees every key).  A
 * row with no allowed key gets O = 0 and lse = -inf.
 *
 * Layout: Q and O are [batch][heads][seq_q][head_dim], K and V
 * [batch][heads][seq_k][head_dim], contiguous row-major (head_dim elements
 * per row, no padding); lse is [batch][heads][seq_q] FP32.  Operands and O
 * share one type, FP16 or BF16 (gemm_dtype); scores, softmax and sums are
 * FP32; the probabilities are rounded to the operand type before the PV
 * product; O rounds to nearest even.
 *
 * Ownership and threading as for the GEMM entry points: the caller owns
 * every buffer and the stream, nothing is allocated, the call validates,
 * enqueues one kernel on `stream` and returns without synchronising.  O and
 * lse must not overlap the inputs.
 */
#ifndef MCS_ATTENTION_H
#define MCS_ATTENTION_H

#include "mcs_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attention_fwd -- O (and lse) for the whole batch.
 *   dtype      GEMM_DTYPE_F16 or GEMM_DTYPE_BF16
 *   batch, heads, seq_q, seq_k   sizes (>= 0)
 *   head_dim   128 (other sizes: GEMM_EUNSUPPORTED)
 *   Q, K, V    device pointers, 16-byte aligned
 *   O          device pointer, 16-byte aligned
 *   lse        device pointer to batch*heads*seq_q floats, or NULL
 *   scale      the score scale, finite and > 0 (usually 1/sqrt(head_dim))
 *   causal     0 or 1
 * Returns GEMM_OK; GEMM_EINVAL for a bad type, flag, scale, negative size,
 * a null pointer where data is needed; GEMM_EALIGN for Q, K, V or O not
 * 16-byte aligned or lse not 4-byte aligned; GEMM_EUNSUPPORTED for
 * another head_dim or sizes whose element counts reach 2^31 per head (or
 * more than 2^31-1 query tiles of 256 rows); GEMM_EHIP if the device query
 * (compute units, read once per device) or the launch fails.  Empty
 * problems (batch, heads or seq_q zero) enqueue nothing; seq_k == 0 writes
 * O = 0 and lse = -inf.
 */
int attention_fwd(int dtype, int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                  int64_t head_dim, const void *Q, const void *K, const void *V, void *O,
                  float *lse, float scale, int causal, hipStream_t stream);

/*
 * attention_fwd_ex -- the same with the schedule chosen: AUTO (what
 * attention_fwd runs), GEMM_SCHED_PIPELINED (8 waves, two wave groups one
 * stage apart: one group's matrix products overlap the other's softmax),
 * GEMM_SCHED_IN_PHASE (the same stages with the groups in step: the ablation
 * of the offset) or GEMM_SCHED_INTERLEAVED (4 waves, one per SIMD, 64 query
 * rows each, every wave interleaving its own matrix products with its own
 * softmax: half the LDS reads per query row).  Other schedules: GEMM_EINVAL.
 * Results are bitwise identical across all of them.
 */
int attention_fwd_ex(int dtype, int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                     int64_t head_dim, const void *Q, const void *K, const void *V, void *O,
                     float *lse, float scale, int causal, int schedule, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MCS_ATTENTION_H */
