// 128x128-tile GEMM for gfx950: the products the 256x256 kernels leave most
// of the chip idle on (1024 x 1024 has 16 tiles of 256x256 for 256 compute
// units, 64 of 128x128).  Same parts as the 4-wave kernel -- the global ->
// LDS loader, LDS layout and swizzle, fragment reads, MFMA instructions,
// tile order and fused epilogue -- on one 128x128 quadrant per workgroup.
//
// Four waves, one per SIMD; wave w = (wm, wn) = (w & 1, w >> 1) owns the
// 64x64 block at rows 64wm, columns 64wn: 4x4 tiles of 16x16, 64 FP32
// accumulators per lane.  A K-step moves 128 bytes of k of every operand row
// (64 FP16/BF16 or 128 FP8 elements): 16 KiB of A and 16 KiB of B.
//
// LDS is a ring of four K-step buffers [A | B] (32 KiB each).  K-step s runs
// as one cluster of MFMAs in eight groups, each also issuing fragment reads
// and one 1-KiB copy of K-step s+3 (groups 0-3: this wave's four A pieces,
// 4-7: its four B pieces), with a scheduling wall after each group so the
// compiler keeps the interleaving.  16-bit operands keep one fragment set and
// refill each piece after its last use (K-step s reads fragments of K-steps s
// and s+1); FP8 alternates two sets (K-step s reads K-step s+1 whole), so its
// loop body is two K-steps and its step count is padded to even.  Waits,
// derived as for the 256x256 kernels:
//   * copy -> read: K-step s+1 is read during K-step s; its copies were
//     issued during K-step s-2 and only the eight copies of K-step s+2 follow
//     them, so every wave waits vmcnt(8) and then meets the others at a
//     barrier at the top of K-step s.  Each copy has two K-steps to land.
//   * read -> refill: K-step s refills the buffer of K-step s-1, read during
//     K-steps s-2 and s-1.  Those reads were consumed by K-step s-1's MFMAs
//     before each wave reached the barrier at the top of K-step s, which
//     every refill follows.
// Copies of K-steps at or past the end use an empty window and write zeros,
// which add nothing.
#include "device.h"

namespace mcs {
namespace {

constexpr int kT = kTile128;
constexpr int kWaves128 = kTile128Threads / 64;
constexpr int kRing = 4;                          // K-step buffers in LDS
constexpr uint32_t kSlot = 2 * kHalf;             // one K-step: A | B
constexpr int kAhead = 3;                         // K-steps between a copy and its use

template <int kElem, bool kTransB>
struct Tile128 : Loader<kElem, kTransB, kWaves128, kT, kHalf>, Block64Reader<kTransB, kHalf> {
    using Base = Loader<kElem, kTransB, kWaves128, kT, kHalf>;
    using Reader = Block64Reader<kTransB, kHalf>;
    using typename Reader::Bases;
    using Base::lds0;

    __device__ __forceinline__ Tile128(const GemmParams &prm, int tm, int tn) : Base(prm, tm, tn) {
        this->init(this->wave & 1, this->wave >> 1, threadIdx.x & 63);
    }

    static __device__ __forceinline__ uint32_t slot(int s) { return static_cast<uint32_t>(s & (kRing - 1)) * kSlot; }

    // Fragments of K-step s into (a, b).
    __device__ __forceinline__ void read_all(int s, i32x4 (&a)[4][2], i32x4 (&b)[4][2]) const {
        const Bases bs = this->bases_at(lds0, slot(s), slot(s));
        for (int j = 0; j < 8; ++j) {
            a[j & 3][j >> 2] = this->read_a(bs, 0, 0, j);
            b[j & 3][j >> 2] = this->read_b(bs, 0, 0, j);
        }
    }

    // FP8 K-step s: acc += a . b while (an, bn) <- K-step s+1 (tile-major:
    // both chunks of a tile together) and the copies of K-step s+3 go out.
    // kMask: the copies need the per-lane k mask.
    template <bool kMask>
    __device__ __forceinline__ void kstep(f32x4 (&acc)[4][4], const i32x4 (&a)[4][2],
                                          const i32x4 (&b)[4][2], i32x4 (&an)[4][2],
                                          i32x4 (&bn)[4][2], int s) const {
        wait_vmcnt<2 * Base::P>();
        rendezvous(this->sg);
        const Bases bs = this->bases_at(lds0, slot(s + 1), slot(s + 1));
        const uint32_t cbuf = slot(s + kAhead);
        static_for<0, 8>([&](auto g) {
            constexpr int j = kElem == kElemFP8 ? (g & 1) * 4 + (g >> 1) : int(g);
            an[j & 3][j >> 2] = this->read_a(bs, 0, 0, j);
            bn[j & 3][j >> 2] = this->read_b(bs, 0, 0, j);
            if constexpr (g < 4)
                this->template copy_a<kMask, g, g + 1>(s + kAhead, cbuf, 0);
            else
                this->template copy_b<kMask, g - 4, g - 3>(s + kAhead, cbuf, 0);
            constexpr int mt = g >> 1, n0 = 2 * (g & 1);
            for (int nt = n0; nt < n0 + 2; ++nt)
                acc[mt][nt] = mfma_fp8(b[nt][0], b[nt][1], a[mt][0], a[mt][1], acc[mt][nt]);
            __builtin_amdgcn_sched_barrier(0);
        });
    }

    // 16-bit operands, one fragment set updated in place.  K-step s: group g
    // = (k-chunk ks, A tile mt) runs a[mt][ks] against b[0..3][ks], then reads
    // a[mt][ks] of K-step s+1 into the registers it just used.  B chunk 1 of
    // K-step s (needed from group 4 on) is read in groups 0-1, B chunk 0 of
    // K-step s+1 in groups 4-7 (free after group 3).
    template <bool kMask>
    __device__ __forceinline__ void kstep16(f32x4 (&acc)[4][4], i32x4 (&a)[4][2], i32x4 (&b)[4][2],
                                            int s) const {
        wait_vmcnt<2 * Base::P>();
        rendezvous(this->sg);
        const Bases bs = this->bases_at(lds0, slot(s), slot(s + 1));
        const uint32_t cbuf = slot(s + kAhead);
        static_for<0, 8>([&](auto g) {
            constexpr int ks = g >> 2, mt = g & 3;
            if constexpr (g < 2) {
                b[2 * g][1] = this->read_b(bs, 0, 0, 4 + 2 * g);
                b[2 * g + 1][1] = this->read_b(bs, 0, 0, 5 + 2 * g);
            }
            if constexpr (g < 4)
                this->template copy_a<kMask, g, g + 1>(s + kAhead, cbuf, 0);
            else
                this->template copy_b<kMask, g - 4, g - 3>(s + kAhead, cbuf, 0);
            for (int nt = 0; nt < 4; ++nt)
                acc[mt][nt] = mfma<kElem>(b[nt][ks], a[mt][ks], acc[mt][nt]);
            a[mt][ks] = this->read_a(bs, 1, 0, g);
            if constexpr (g >= 4)
                b[g - 4][0] = this->read_b(bs, 1, 0, g - 4);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
};

template <int kElem, bool kTransB, bool kOutF32>
__global__ void __launch_bounds__(kWaves128 * 64)
__attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_tile128_kernel(GemmParams pin) {
    const GemmParams p = slice_view<elem_bytes(kElem), kTransB>(pin);
    __shared__ __attribute__((aligned(1024))) char smem[kRing * kSlot];

    int tm, tn;
    tile_coords(p, blockIdx.x, tm, tn);
    Tile128<kElem, kTransB> t(p, tm, tn);
    t.lds0 = lds_address(smem);
    stagger_poison_lds<kRing * kSlot, kWaves128 * 64>(t.lds0);

    f32x4 acc[4][4];
    for (int mt = 0; mt < 4; ++mt)
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x4 a0[4][2], b0[4][2], a1[4][2], b1[4][2];

    // prologue: copies of K-steps 0 .. kAhead-1, then the fragments of step 0
    for (int s = 0; s < kAhead; ++s) {
        t.copy_a(s, Tile128<kElem, kTransB>::slot(s), 0);
        t.copy_b(s, Tile128<kElem, kTransB>::slot(s), 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 * (kAhead - 1) * Tile128<kElem, kTransB>::P>();   // step 0 landed (this wave)
    rendezvous(t.sg);                                              // ... and every wave's part
    t.read_all(0, a0, b0);

    // A given M x K (and B given N x K) needs the per-lane k mask on the
    // copies of a partial last K-step; B given K x N never does.
    if constexpr (kElem == kElemFP8) {
#pragma unroll 1
        for (int s = 0; s < p.steps; s += 2) {
            t.template kstep<true>(acc, a0, b0, a1, b1, s);
            t.template kstep<true>(acc, a1, b1, a0, b0, s + 1);
        }
    } else {
#pragma unroll 1
        for (int s = 0; s < p.steps; ++s) t.template kstep16<true>(acc, a0, b0, s);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();   // the zero-window copies past the end, before LDS is released

    const int lane = __lane_id();
    const int wave = t.wave;
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int row = t.win.m0 + 64 * wm + 16 * mt + (lane & 15);
        if (row >= p.M) continue;
        store_strip<kElem != kElemF16, kOutF32>(p, acc[mt], row, t.win.n0 + 64 * wn, lane);
    }
}

}  // namespace

const void *tile128_kernel(int elem, bool trans_b, bool out_f32) {
#define MCS_PICK(E, T, O)                                 \
    if (elem == E && trans_b == T && out_f32 == O)        \
        return reinterpret_cast<const void *>(&gemm_tile128_kernel<E, T, O>);
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
