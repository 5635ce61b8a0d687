// Warp-pipelined FP16/BF16 GEMM for gfx950 (MI355X, CDNA 4).
//
// Method: "Two Waves, One Stage Apart: Warp-Pipelining Triton GEMMs on AMD
// Instinct".  An 8-wave workgroup is split into two groups of four waves
// (waves 0-3 = group A, 4-7 = group B, one wave of each group per SIMD).  Both
// groups run the same staged loop; group B takes one extra barrier before the
// loop and group A one extra barrier after it, so at every stage boundary the
// groups meet while group A is one stage ahead (sections "Two Waves, One Stage
// Apart" and "Creating and Closing the Offset", Figures 2-3).  Stages
// alternate MFMA work with memory work, so on each SIMD one wave issues MFMA
// while the other reads LDS, issues copies and computes addresses.
//
// gfx950 layout (section "MI350 Series (gfx950, CDNA 4): Three Overlapping
// Flows", Figure 7): a 256x256 output tile is four 128x128 quadrants.  The
// pages give each quadrant its own MFMA stage and memory stage (eight stages
// per 64-deep K-step); here two quadrants share a stage, four stages per
// K-step, because each rendezvous costs the MFMA pipe ~75 cycles (measured
// with the memory work removed) and 16 MFMAs (256 cycles) were too little
// work to amortise it (section "Stage Size and Register Pressure" weighs
// the same trade: bigger stages hide more of the other group's memory work
// per rendezvous, at the price of registers).  The loop is unrolled twice so
// each LDS buffer is addressed statically.  Copies of future tiles go
// straight from global memory into
// LDS (buffer_load ... lds), the operand halves are double buffered, and
// three flows overlap: copies of a future K-step, LDS reads for the next
// stage, and MFMA on the current one.
//
// Stage boundary (section "What Lands in the Instruction Stream"):
//     [s_waitcnt only where a dependency needs it] sched_barrier s_barrier sched_barrier
// Memory stages run at s_setprio 1, MFMA stages at 0 (section "Writing a
// Warp-Pipelined Loop").  Waits (section "Dependencies Cross Groups and
// Iterations", Figure 10):
//   * copy -> read: data read in stage R is copied by waves of both groups,
//     so every wave waits for its own copies (vmcnt) before the barrier that
//     ENDS stage R-2; the trailing group therefore completes them before the
//     rendezvous that releases the leading group into R.
//   * read -> refill: every memory stage ends with lgkmcnt(0), and a half is
//     refilled no earlier than two stages after the stage that read it, one
//     stage later than an in-phase schedule would allow because group B lags.
//
// Base schedule of K-step t (each B layout adjusts it, below; cur = buffer
// of t, nxt = buffer of t+1); aX/bX are
// the A rows / B columns of half X; reads fill registers for the next stage:
//     S0 MFMA Q00 + Q10 (a0 a1 . b0)
//     S1 mem: read b1[cur];          copy a0, a1, b0 [cur] <- t+2
//     S2 MFMA Q01 + Q11 (a0 a1 . b1)
//     S3 mem: read a0, a1, b0 [nxt];  copy b1[cur] <- t+2
// Every refill comes two stages after the last read of its half (a0/a1/b0
// of step t are read in S3 of step t-1, b1 in S1).  Each half read in stage
// R was copied with eight copies of this wave issued after it by the end of
// stage R-2 (S1 copies six, S3 two), so both memory stages end with
// vmcnt(8) lgkmcnt(0); every copy has a full K-step to land.  At most 64
// fragment VGPRs are live with B given N x K (a0 a1 b0 b1 is 16+16+32+32,
// never all four), 88 with B given K x N (32+32+16+16, plus the 8 of the
// next b0 that S1 reads early).
// Per-layout adjustments (StageTuning below):
//   * B given N x K: each MFMA stage's last two MFMAs are issued at the head
//     of the next memory stage, after the rendezvous (they read only
//     registers, so no LDS dependency moves); and b0 is copied in S3 before
//     b1 instead of in S1, so S1 ends with vmcnt(6): after the b0 copy of
//     step t+1 (S3 of t-1) come b1's two and S1's four by the end of S1 of
//     t.  That copy has about two and a half stages to land.  b0 of step t
//     was last read in S3 of t-1, four stages before its refill.
//   * B given K x N: S1 also reads k-slice 0 of b0[nxt] (S0 is done with b0)
//     and S3 only k-slice 1; S1 copies b0 first, so after the b0 copy of
//     step t+1 (issued in S1 of t-1) only a0, a1 and S3's b1 follow by the end
//     of S3 of t-1: S3 ends with vmcnt(6).  That copy has three stages to
//     land; every other keeps a full K-step.
// The LDS reads open each memory stage so that their latency overlaps the
// address and descriptor work of the copies.  Copies of K-steps past the end
// use an empty buffer window, so they write zeros (buffer loads outside the
// window return zero), which keeps every stage identical; an odd K-step
// count is padded with one zero step.
//
// Data layout.  LDS: two buffers of 64 KiB, each [A0 | A1 | B0 | B1] halves of
// 16 KiB.  A half (and a B half when B is N x K) is 128 rows x 64 k, 128-byte
// rows of eight 16-byte chunks stored at chunk ^ (row & 7).  With this XOR
// the fragment reads (16 consecutive rows, one k-chunk per 16 lanes) show no
// LDS bank conflicts on gfx950, where (r ^ (r >> 3)) & 7 showed two-way
// conflicts (SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE measured per layout).  A B half when B is K x N is 64 k-rows x 128 n (256-byte
// rows) with chunk ^ 2*((k & 3) + 4*((k >> 3) & 1)), read with the gfx950
// transposing ds_read_b64_tr_b16 into the K-major MFMA operand.
// Wave (wm, wn) = (wave & 3, wave >> 2) owns rows 32wm..32wm+31 of every A half
// and columns 64wn..64wn+63 of every B half: a 32x64 block of each quadrant
// (B given K x N: (wave & 1, wave >> 1), a 64x32 block; see WaveLayout).
// MFMA: v_mfma_f32_16x16x32_{f16,bf16} with the B fragment as the first
// operand, so each lane ends with four consecutive columns of one row; for a
// 16-bit output, lanes l and l^16 trade halves of two neighbouring tiles so
// every lane stores eight consecutive columns (16 bytes).
#include "device.h"

namespace mcs {
namespace {

constexpr int kCopyWait = 8;               // vmcnt at the end of each memory stage

// Per-layout stage tuning (A/B measured in one process on rotating inputs,
// results bitwise identical):
//   kTail: with B given N x K each MFMA stage leaves its last two MFMAs to the
//     start of the following memory stage, issued there at the memory stage's
//     raised priority; the matrix pipe then has work queued the moment the
//     rendezvous releases both groups (+0.6..1.4 % on 4096^2 x 8192, BF16
//     8192^3 and FP8 8192^3).  With B given K x N it gained nothing.
//   kEarlyB: with B given K x N the S3 reads (a0, a1 and b0: 24 read
//     instructions, the transposing ones included) outweigh S1's (8), so S1
//     also reads k-slice 0 of the next step's b0; its copy then goes first in
//     S1's copy order and S3 ends with vmcnt(6) (+1.5..2.2 % on
//     16384x2048x8192, 4096^2 x 8192 and 8192^3).  With B given N x K it lost.
//   kLateB0: with B given N x K the copies of b0 move from S1 to S3 (S1
//     copies a0 a1, S3 b0 b1: four each), so S1 ends with vmcnt(6) and the
//     b0 copy has about two and a half stages to land (+0.2..1 % on
//     4096^2 x 8192, 4096^2 x 16384, BF16 and FP8 8192^3).
template <bool kTransB> struct StageTuning {
    static constexpr int kTail = kTransB ? 2 : 0;
    static constexpr bool kEarlyB = !kTransB;
    static constexpr bool kLateB0 = kTransB;
    static constexpr int kWaitS1 = kLateB0 ? 6 : kCopyWait;
    static constexpr int kWaitS3 = kEarlyB ? 6 : kCopyWait;
};

// Wave layout.  B given N x K: 4 (M) x 2 (N) waves, wave (wm, wn) owning rows
// 32wm.. of every A half and columns 64wn.. of every B half.  B given K x N:
// 2 x 4, rows 64wm.. and columns 32wn..: a B fragment of 16 columns then
// takes two transposing 8-byte reads against one 16-byte read for A, and this
// layout issues 16 + 16 LDS reads per wave per K-step where 4 x 2 issues
// 8 + 32 (measured on 16384x2048x8192: the 4 x 2 layout spent 30 % more
// wave-cycles waiting to issue LDS instructions per FLOP than B given N x K).
template <bool kTransB>
struct WaveLayout {
    static constexpr int kWM = kTransB ? 4 : 2;     // waves along M
    static constexpr int kRows = 128 / kWM;         // rows of each A half per wave
    static constexpr int kCols = 128 * kWM / 8;     // columns of each B half per wave
    static constexpr int kMT = kRows / 16, kNT = kCols / 16;
    static constexpr int kShift = kWM == 4 ? 2 : 1;  // wave >> kShift = wn
};

// Per-wave state of the 8-wave kernel: the shared copy loader plus this
// wave's fragment read offsets.
template <int kElem, bool kTransB, bool kOutF32, bool kOffset>
struct Pipeline : Loader<kElem, kTransB, 8> {
    using Loader<kElem, kTransB, 8>::lds0;
    using L = WaveLayout<kTransB>;
    FragOffsets fa, fb;

    __device__ __forceinline__ Pipeline(const GemmParams &prm, int tm, int tn)
        : Loader<kElem, kTransB, 8>(prm, tm, tn) {
        const int lane = threadIdx.x & 63;
        const int wm = this->wave & (L::kWM - 1), wn = this->wave >> L::kShift;
        fa.rows(L::kRows * wm, lane);
        if constexpr (kTransB)
            fb.rows(L::kCols * wn, lane);
        else
            fb.cols_tr(L::kCols * wn, lane);
    }

    __device__ __forceinline__ void read_a(i32x4 (&a)[L::kMT][2], uint32_t buf, int h) const {
        const uint32_t base = lds0 + buf + kOffA + h * kHalf;
        for (int mt = 0; mt < L::kMT; ++mt)
            for (int ks = 0; ks < 2; ++ks)
                a[mt][ks] = lds_read128(base + fa.row[ks] + mt * 2048);
    }

    // The fragment pieces b[nt][ks] with kNt0 <= nt < kNt1 and kKs0 <= ks < kKs1.
    template <int kNt0 = 0, int kNt1 = L::kNT, int kKs0 = 0, int kKs1 = 2>
    __device__ __forceinline__ void read_b(i32x4 (&b)[L::kNT][2], uint32_t buf, int h) const {
        const uint32_t base = lds0 + buf + kOffB + h * kHalf;
        if constexpr (kTransB) {
            for (int nt = kNt0; nt < kNt1; ++nt)
                for (int ks = kKs0; ks < kKs1; ++ks)
                    b[nt][ks] = lds_read128(base + fb.row[ks] + nt * 2048);
        } else {
            for (int nt = kNt0; nt < kNt1; ++nt)
                for (int ks = kKs0; ks < kKs1; ++ks) {
                    const i32x2 lo = lds_read64_tr(base + fb.tr[nt] + (32 * ks + 0) * 256);
                    const i32x2 hi = lds_read64_tr(base + fb.tr[nt] + (32 * ks + 4) * 256);
                    b[nt][ks] = i32x4{lo.x, lo.y, hi.x, hi.y};
                }
        }
    }
};

// One quadrant's MFMAs over the K-step: two 16x16x32 k-slices for 16-bit
// operands, or one 16x16x128 FP8 MFMA over both chunks.  The tiles go in a
// snake (columns forward on even rows of tiles, backward on odd ones), so
// within a k-slice consecutive MFMAs differ in one operand only.  Only the
// MFMAs numbered kBegin..kEnd-1 of that sequence are issued, so a stage can
// leave its last few for after the rendezvous.
template <int kElem, int kMT, int kNT, int kBegin = 0, int kEnd = 1 << 30>
__device__ __forceinline__ void quadrant(f32x4 (&acc)[kMT][kNT], const i32x4 (&a)[kMT][2],
                                         const i32x4 (&b)[kNT][2]) {
    if constexpr (kElem == kElemFP8) {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                const int i = mt * kNT + j;
                if (i < kBegin || i >= kEnd) continue;
                const int nt = mt & 1 ? kNT - 1 - j : j;
                acc[mt][nt] = mfma_fp8(b[nt][0], b[nt][1], a[mt][0], a[mt][1], acc[mt][nt]);
            }
    } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int j = 0; j < kNT; ++j) {
                    const int i = (ks * kMT + mt) * kNT + j;
                    if (i < kBegin || i >= kEnd) continue;
                    const int nt = mt & 1 ? kNT - 1 - j : j;
                    acc[mt][nt] = mfma<kElem>(b[nt][ks], a[mt][ks], acc[mt][nt]);
                }
    }
}

__device__ __forceinline__ void mem_stage_begin() { __builtin_amdgcn_s_setprio(1); }

// End of a memory stage: this wave's copies for the reads two stages later
// have landed, and so have its own LDS reads (their registers feed the next
// stage and their half may be refilled two stages on).
template <int kWait = kCopyWait>
__device__ __forceinline__ void mem_stage_end(Stagger &sg) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kWait>();
    wait_lgkmcnt<0>();
    __builtin_amdgcn_s_setprio(0);
    rendezvous(sg);
}

template <int kElem, bool kTransB, bool kOutF32, bool kOffset>
__global__ void __launch_bounds__(kPipeThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_pipelined_kernel(GemmParams pin) {
    const GemmParams p = slice_view<elem_bytes(kElem), kTransB>(pin);
    __shared__ __attribute__((aligned(1024))) char smem[2 * kBuf];

    int tm, tn;
    tile_coords(p, blockIdx.x, tm, tn);
    Pipeline<kElem, kTransB, kOutF32, kOffset> pl(p, tm, tn);
    pl.lds0 = lds_address(smem);
    stagger_poison_lds<2 * kBuf, kPipeThreads>(pl.lds0);
    const int wave = pl.wave;

    using L = WaveLayout<kTransB>;
    constexpr int kQ = (kElem == kElemFP8 ? 1 : 2) * L::kMT * L::kNT;   // MFMAs per quadrant
    using T = StageTuning<kTransB>;
    constexpr int kTail = T::kTail < kQ ? T::kTail : kQ;   // MFMAs issued after the rendezvous
    f32x4 acc[2][2][L::kMT][L::kNT];
    for (int qa = 0; qa < 2; ++qa)
        for (int qb = 0; qb < 2; ++qb)
            for (int mt = 0; mt < L::kMT; ++mt)
                for (int nt = 0; nt < L::kNT; ++nt)
                    acc[qa][qb][mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x4 a0[L::kMT][2], a1[L::kMT][2], b0[L::kNT][2], b1[L::kNT][2];

    // ---- prologue: the copy stream of steps 0 and 1 in steady-state order
    // (a0 a1 b0 -- b0 a0 a1 when b0 is read early -- then b1, per step), then
    // the fragments S0 of step 0 needs.
    if constexpr (T::kEarlyB) pl.copy_b(0, 0, 0);
    pl.copy_a(0, 0, 0);
    pl.copy_a(0, 0, 1);
    if constexpr (!T::kEarlyB) pl.copy_b(0, 0, 0);
    pl.copy_b(0, 0, 1);
    if constexpr (T::kEarlyB) pl.copy_b(1, kBuf, 0);
    pl.copy_a(1, kBuf, 0);
    pl.copy_a(1, kBuf, 1);
    if constexpr (!T::kEarlyB) pl.copy_b(1, kBuf, 0);
    pl.copy_b(1, kBuf, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<10>();                   // a0(0) a1(0) b0(0) landed (this wave's part)
    rendezvous(pl.sg);                  // ... and every wave's part
    pl.read_a(a0, 0, 0);
    pl.read_a(a1, 0, 1);
    pl.read_b(b0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt<0>();
    wait_vmcnt<T::kWaitS3>();           // b1(0) landed (with b0 read early, b0(1) too): the state at the end of S3 of step -1
    rendezvous(pl.sg);

    if constexpr (kOffset) {
        if (wave >= 4) group_barrier(pl.sg);           // group B waits: entry offset
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- steady state, two K-steps per iteration (buffer 0 then buffer 1)
    for (int t = 0; t < p.steps; t += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t cur = u ? kBuf : 0u, nxt = u ? 0u : kBuf;
            const int s = t + u;
            // S0: quadrants Q00 and Q10
            quadrant<kElem>(acc[0][0], a0, b0);
            quadrant<kElem, L::kMT, L::kNT, 0, kQ - kTail>(acc[1][0], a1, b0);
            rendezvous(pl.sg);
            // S1
            mem_stage_begin();
            quadrant<kElem, L::kMT, L::kNT, kQ - kTail, kQ>(acc[1][0], a1, b0);
            __builtin_amdgcn_sched_barrier(0);
            pl.read_b(b1, cur, 1);
            if constexpr (T::kEarlyB) {
                pl.template read_b<0, L::kNT, 0, 1>(b0, nxt, 0);
                pl.copy_b(s + 2, cur, 0);
            }
            pl.copy_a(s + 2, cur, 0);
            pl.copy_a(s + 2, cur, 1);
            if constexpr (!T::kEarlyB && !T::kLateB0) pl.copy_b(s + 2, cur, 0);
            mem_stage_end<T::kWaitS1>(pl.sg);
            // S2: quadrants Q01 and Q11
            quadrant<kElem>(acc[0][1], a0, b1);
            quadrant<kElem, L::kMT, L::kNT, 0, kQ - kTail>(acc[1][1], a1, b1);
            rendezvous(pl.sg);
            // S3
            mem_stage_begin();
            quadrant<kElem, L::kMT, L::kNT, kQ - kTail, kQ>(acc[1][1], a1, b1);
            __builtin_amdgcn_sched_barrier(0);
            pl.read_a(a0, nxt, 0);
            pl.read_a(a1, nxt, 1);
            if constexpr (T::kEarlyB)
                pl.template read_b<0, L::kNT, 1, 2>(b0, nxt, 0);
            else
                pl.read_b(b0, nxt, 0);
            if constexpr (T::kLateB0) pl.copy_b(s + 2, cur, 0);
            pl.copy_b(s + 2, cur, 1);
            mem_stage_end<T::kWaitS3>(pl.sg);
        }
    }

    if constexpr (kOffset) {
        __builtin_amdgcn_sched_barrier(0);
        if (wave < 4) group_barrier(pl.sg);            // group A waits: exit offset
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();   // the zero-window copies of steps past the end, before LDS is released

    // ---- epilogue.  The lane id is recomputed here so no lane-derived value
    // stays live across the loop.
    const int lane = __lane_id();
    const int wm = wave & (L::kWM - 1), wn = wave >> L::kShift;
    for (int qa = 0; qa < 2; ++qa)
        for (int mt = 0; mt < L::kMT; ++mt) {
            const int row = pl.win.m0 + 128 * qa + L::kRows * wm + 16 * mt + (lane & 15);
            if (row >= p.M) continue;
            for (int qb = 0; qb < 2; ++qb)
                store_strip<kElem != kElemF16, kOutF32>(p, acc[qa][qb][mt], row,
                                                        pl.win.n0 + 128 * qb + L::kCols * wn, lane);
        }
}

}  // namespace

const void *pipelined_kernel(int elem, bool trans_b, bool out_f32, bool offset) {
#define MCS_PICK(E, T, O, S)                                                         \
    if (elem == E && trans_b == T && out_f32 == O && offset == S)                   \
        return reinterpret_cast<const void *>(&gemm_pipelined_kernel<E, T, O, S>);
#define MCS_PICK_S(E, T, O) MCS_PICK(E, T, O, true) MCS_PICK(E, T, O, false)
#define MCS_PICK_O(E, T) MCS_PICK_S(E, T, false) MCS_PICK_S(E, T, true)
    MCS_PICK_O(kElemF16, false)
    MCS_PICK_O(kElemF16, true)
    MCS_PICK_O(kElemBF16, false)
    MCS_PICK_O(kElemBF16, true)
    MCS_PICK_O(kElemFP8, true)
#undef MCS_PICK_O
#undef MCS_PICK_S
#undef MCS_PICK
    return nullptr;
}

}  // namespace mcs
