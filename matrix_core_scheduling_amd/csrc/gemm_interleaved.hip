// Within-wave interleaved FP16/BF16 GEMM for gfx950: the 4-wave counterpart
// of the warp-pipelined kernel, built from the same parts (256x256x64 tile,
// the same global -> LDS loader, LDS layout and swizzle, MFMA instruction,
// tile order and fused epilogue) so that the two differ only in how the
// schedule overlaps matrix and memory work.
//
// "Two Waves, One Stage Apart: Warp-Pipelining Triton GEMMs on AMD Instinct"
// compares its 8-wave kernel with a hand-tuned 4-wave kernel on MI355X
// (section "MI350 Series (gfx950, CDNA 4): Three Overlapping Flows") and notes
// that the two differ in layout, compiler settings and tooling, so the
// comparison does not isolate warp-pipelining.  The structure of the 4-wave
// kernel follows "Porting High-Performance HIP Kernels to FlyDSL" (section
// "A More Complex Kernel", "Putting it All Together"): each wave owns a
// 128x128 block of the output as a 2x2 arrangement of 64x64 sub-tiles and
// computes them in the order c00, c01, c10, c11; while the MFMAs of one
// sub-tile run, the same wave reads the operand fragment the next sub-tile
// needs and issues the copy of one operand half of a future K-step (an
// "interleaved cluster"); a wait plus a workgroup barrier precedes c00 and
// c10.  That page's kernel is FP8 with a 128-deep K-step; here the K-step is
// 64 deep (two 16x16x32 MFMA k-slices), as in the 8-wave kernel.
//
// One wave per SIMD: wave w = (wm, wn) = (w & 1, w >> 1) owns rows 64wm..+63
// of both A halves and columns 64wn..+63 of both B halves, i.e. one 64x64 block
// of every 128x128 quadrant; its 256 FP32 accumulators live in the
// accumulation registers.  Fragments: a0/a1 = the wave's 64 rows of A half 0/1,
// b0/b1 = its 64 columns of B half 0/1 (4 tiles x 2 k-slices, 32 VGPRs each).
//
// Schedule of K-step s (cur = buffer of s, nxt = buffer of s+1):
//     [wait, barrier]
//     c00 += a0.b0   read b1 <- B1[cur]   copy A0[cur] <- s+2
//     c01 += a0.b1   read a1 <- A1[cur]   copy B0[cur] <- s+2
//     [wait, barrier]
//     c10 += a1.b0   read a0 <- A0[nxt]   copy B1[cur] <- s+2
//     c11 += a1.b1   read b0 <- B0[nxt]   copy A1[cur] <- s+2
// Waits (derived the same way as for the 8-wave kernel):
//   * read -> refill: each half is refilled only after a barrier that follows
//     the cluster that last read it (A0/B0 of cur were read in c10/c11 of
//     step s-1, B1/A1 in c00/c01 of step s), and every barrier is preceded
//     by lgkmcnt(0).
//   * copy -> read: each wave issues four copies per cluster.  The halves read
//     after the first barrier (B1, A1 of cur) were copied in c10/c11 of step
//     s-2 and the halves read after the second (A0, B0 of nxt) in c00/c01 of
//     step s-1; in both cases at least sixteen copies of this wave follow, so
//     both barriers are preceded by vmcnt(16): every copy has about one
//     K-step to land.
// Inside a cluster the 32 MFMAs run in eight groups of four (one k-slice and
// one 16-row tile of A against four 16-column tiles of B); group g also
// issues piece g of the next fragment and, for odd g, one copy, with a
// scheduling wall after each group so the compiler keeps the interleaving.
// With one wave per SIMD nothing else issues while this wave spends issue
// slots on address, descriptor or wait instructions: measured on MI355X, a
// lone wave keeps the matrix pipe full with about three other instructions
// per 16x16x32 MFMA (fewer if they are vector ALU), so the memory work is
// kept lean: each K-step computes its LDS read bases once (every read is a
// base plus an immediate offset), the copies take their LDS destination as
// an immediate on M0, and the per-lane k mask of the copies is compiled out
// of every K-step except the partial last one.  Per K-step each wave reads
// 32 KiB of LDS (the 8-wave kernel: 24 KiB for each of 8 waves) and waits at
// two barriers.
#include "device.h"

namespace mcs {
namespace {

constexpr int kWaves = kInterThreads / 64;
constexpr int kCopyWait = 16;              // vmcnt before each barrier

template <int kElem, bool kTransB>
struct Interleave : Loader<kElem, kTransB, kWaves>, Block64Reader<kTransB, kOffB> {
    using Loader<kElem, kTransB, kWaves>::lds0;
    using Reader = Block64Reader<kTransB, kOffB>;
    using typename Reader::Bases;
    using Reader::read_a;
    using Reader::read_b;

    __device__ __forceinline__ Interleave(const GemmParams &prm, int tm, int tn)
        : Loader<kElem, kTransB, kWaves>(prm, tm, tn) {
        this->init(this->wave & 1, this->wave >> 1, threadIdx.x & 63);
    }

    // LDS read bases of one K-step (buffers cur and nxt).
    __device__ __forceinline__ Bases bases(uint32_t cur, uint32_t nxt) const {
        return this->bases_at(lds0, cur, nxt);
    }

    // One cluster: acc += a . b over the K-step while fragment `nf` (operand
    // kind kReadB ? B : A, half rh, buffer u of bs) is read and half ch of
    // operand kCopyB ? B : A is copied for K-step cs into buffer cbuf.  Group
    // g issues one fragment piece and, for odd g, one copy.  For 16-bit
    // operands a group is one k-slice of one A tile against four B tiles and
    // the pieces go k-slice-major (the next cluster's first groups use k-slice
    // 0 of every tile).  For FP8 a group is two 16x16x128 MFMAs, each taking
    // both 16-byte chunks of its tiles, so the pieces go tile-major; with
    // kNtMajor the groups walk B tiles (the cluster whose B fragment was read
    // by the previous cluster), otherwise A tiles.
    template <bool kReadB, bool kCopyB, bool kMask, bool kNtMajor>
    __device__ __forceinline__ void cluster(f32x4 (&acc)[4][4], const i32x4 (&a)[4][2],
                                            const i32x4 (&b)[4][2], i32x4 (&nf)[4][2],
                                            const Bases &bs, int u, int rh, int cs, uint32_t cbuf,
                                            int ch) const {
        static_for<0, 8>([&](auto g) {
            constexpr int j = kElem == kElemFP8 ? (g & 1) * 4 + (g >> 1) : int(g);
            nf[j & 3][j >> 2] = kReadB ? read_b(bs, u, rh, j) : read_a(bs, u, rh, j);
            if constexpr (g & 1) {
                if constexpr (kCopyB)
                    this->template copy_b<kMask, g / 2, g / 2 + 1>(cs, cbuf, ch);
                else
                    this->template copy_a<kMask, g / 2, g / 2 + 1>(cs, cbuf, ch);
            }
            if constexpr (kElem == kElemFP8) {
                constexpr int t = g >> 1, o0 = 2 * (g & 1);
                for (int o = o0; o < o0 + 2; ++o) {
                    const int mt = kNtMajor ? o : t, nt = kNtMajor ? t : o;
                    acc[mt][nt] = mfma_fp8(b[nt][0], b[nt][1], a[mt][0], a[mt][1], acc[mt][nt]);
                }
            } else {
                constexpr int ks = g >> 2, mt = g & 3;
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = mfma<kElem>(b[nt][ks], a[mt][ks], acc[mt][nt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    }
};

// This wave's copies for the reads after the barrier have landed, and its own
// LDS reads are complete (their halves are refilled after the barrier).
__device__ __forceinline__ void wait_and_rendezvous(Stagger &sg) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kCopyWait>();
    wait_lgkmcnt<0>();
    rendezvous(sg);
}

template <int kElem, bool kTransB, bool kOutF32>
__global__ void __launch_bounds__(kInterThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_interleaved_kernel(GemmParams pin) {
    const GemmParams p = slice_view<elem_bytes(kElem), kTransB, true>(pin);
    __shared__ __attribute__((aligned(1024))) char smem[2 * kBuf];

    int tm, tn;
    tile_coords(p, blockIdx.x, tm, tn);
    Interleave<kElem, kTransB> il(p, tm, tn);
    il.lds0 = lds_address(smem);
    stagger_poison_lds<2 * kBuf, kInterThreads>(il.lds0);
    const int wave = il.wave;

    f32x4 acc[2][2][4][4];
    for (int qa = 0; qa < 2; ++qa)
        for (int qb = 0; qb < 2; ++qb)
            for (int mt = 0; mt < 4; ++mt)
                for (int nt = 0; nt < 4; ++nt)
                    acc[qa][qb][mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x4 a0[4][2], a1[4][2], b0[4][2], b1[4][2];

    // ---- prologue: the copy stream of steps 0 and 1 in steady-state order
    // (A0 B0 B1 A1 per step), then the fragments c00 of step 0 needs.
    for (int s = 0; s < 2; ++s) {
        const uint32_t buf = s ? kBuf : 0u;
        il.copy_a(s, buf, 0);
        il.copy_b(s, buf, 0);
        il.copy_b(s, buf, 1);
        il.copy_a(s, buf, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<24>();                   // A0(0) and B0(0) landed (this wave's part)
    rendezvous(il.sg);                  // ... and every wave's part
    {
        const auto bs = il.bases(0, kBuf);
        for (int j = 0; j < 8; ++j) {
            a0[j & 3][j >> 2] = il.read_a(bs, 0, 0, j);
            b0[j & 3][j >> 2] = il.read_b(bs, 0, 0, j);
        }
    }

    // ---- steady state, one K-step per iteration.  (Unrolling two K-steps so
    // the buffers are addressed statically, as the 8-wave kernel does, makes
    // the register allocator rotate the 256 accumulators through copies.)
    // The copies of K-step s+2 need the per-lane k mask only when that step
    // is the partial last one (p.steps is exactly ceil(K / step) here).
    // Written as steps - 1 rather than from K: deriving it from K by a
    // division made the allocator rotate the accumulators for B given N x K.
    const int tail = (p.K % step_k(kElem)) ? p.steps - 1 : -1;   // the partial K-step, if any
    auto kstep = [&](int s, auto mask) {
        constexpr bool kMask = decltype(mask)::value;
        const uint32_t cur = (s & 1) ? kBuf : 0u, nxt = kBuf - cur;
        const auto bs = il.bases(cur, nxt);
        wait_and_rendezvous(il.sg);
        il.template cluster<true, false, kMask, true>(acc[0][0], a0, b0, b1, bs, 0, 1, s + 2, cur, 0);
        il.template cluster<false, true, kMask, true>(acc[0][1], a0, b1, a1, bs, 0, 1, s + 2, cur, 0);
        wait_and_rendezvous(il.sg);
        il.template cluster<false, true, kMask, false>(acc[1][0], a1, b0, a0, bs, 1, 0, s + 2, cur, 1);
        il.template cluster<true, false, kMask, false>(acc[1][1], a1, b1, b0, bs, 1, 0, s + 2, cur, 1);
    };
    int s = 0;
    if constexpr (kTransB) {
        const int plain = tail >= 2 ? tail - 2 : (tail < 0 ? p.steps : 0);
#pragma unroll 1
        for (; s < plain; ++s) kstep(s, std::false_type{});
    }
#pragma unroll 1
    for (; s < p.steps; ++s) kstep(s, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();   // the zero-window copies of steps past the end, before LDS is released

    // ---- epilogue (fully unrolled: the accumulators are only ever indexed
    // by constants, so they stay in registers)
    const int lane = __lane_id();
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int qa = 0; qa < 2; ++qa)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int row = il.win.m0 + 128 * qa + 64 * wm + 16 * mt + (lane & 15);
            if (row >= p.M) continue;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
                store_strip<kElem != kElemF16, kOutF32>(p, acc[qa][qb][mt], row, il.win.n0 + 128 * qb + 64 * wn, lane);
        }
}

}  // namespace

const void *interleaved_kernel(int elem, bool trans_b, bool out_f32) {
#define MCS_PICK(E, T, O)                                                            \
    if (elem == E && trans_b == T && out_f32 == O)                                  \
        return reinterpret_cast<const void *>(&gemm_interleaved_kernel<E, T, O>);
#define MCS_PICK_O(E, T) MCS_PICK(E, T, false) MCS_PICK(E, T, true)
    MCS_PICK_O(kElemF16, false)
    MCS_PICK_O(kElemF16, true)
    MCS_PICK_O(kElemBF16, false)
    MCS_PICK_O(kElemBF16, true)
    MCS_PICK_O(kElemFP8, true)
#undef MCS_PICK_O
#undef MCS_PICK
    return nullptr;
}

}  // namespace mcs
