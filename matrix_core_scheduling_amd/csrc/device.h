// Device-side pieces shared by the 256x256x64 MFMA kernels (the 8-wave
// warp-pipelined kernel and the 4-wave within-wave-interleaved kernel): the
// LDS layout, the global -> LDS copy loader, the instruction helpers, the
// tile order and the fused output store.  The two kernels differ only in how
// their waves divide the tile and schedule the work.
#pragma once

#include "internal.h"

#include <type_traits>

namespace mcs {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS: two buffers (one per K-step in flight), each [A0 | A1 | B0 | B1]
// halves of 16 KiB.  An A half (and a B half when B is N x K) is 128 rows x
// 128 bytes of k (64 FP16/BF16 or 128 FP8 elements), eight 16-byte chunks per
// row stored at chunk ^ (row & 7).  A B half when B is K x N (16-bit operands
// only) is 64 k-rows x 128 n, 256-byte rows with chunk ^ 2*((k & 3) + 4*((k >>
// 3) & 1)), read with ds_read_b64_tr_b16.
constexpr uint32_t kHalf = 16384;          // bytes of one operand half in LDS
constexpr uint32_t kBuf = 4 * kHalf;       // one K-step: A0 A1 B0 B1
constexpr uint32_t kOffA = 0, kOffB = 2 * kHalf;
constexpr uint32_t kOutOfWindow = 0x80000000u;  // >= every buffer window used here

// ---- instruction helpers -----------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // GFX9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

// ---- race-stress build ---------------------------------------------------
//
// Compiled with MCS_STAGGER (a separate test library, never the product
// one), every wave idles for a pseudo-random 0..15 sleeps of 64 cycles on
// both sides of every workgroup barrier, and the workgroup's LDS starts out
// filled with 0xFF bytes (a NaN in FP16, BF16, FP8 E4M3 and FP32).  A wait
// or barrier missing from a schedule then shows up as a result that differs
// from the unperturbed run, or as NaN, instead of hiding behind the waves'
// usual timing; the arithmetic and its order are unchanged, so a correct
// schedule gives bitwise the same result.  The sleeps add no memory
// instruction and no s_waitcnt.  In the product build a Stagger is empty and
// every pause compiles to nothing.
struct Stagger {
#ifdef MCS_STAGGER
    uint32_t x;   // wave-uniform generator state (an SGPR)

    __device__ __forceinline__ explicit Stagger(uint32_t seed) {
        const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        uint32_t h = seed ^ (blockIdx.x * 0x9E3779B9u) ^ (blockIdx.y * 0x85EBCA6Bu) ^ (wave * 0xC2B2AE35u);
        h ^= h >> 16;   // murmur3 finaliser
        h *= 0x85EBCA6Bu;
        h ^= h >> 13;
        h *= 0xC2B2AE35u;
        h ^= h >> 16;
        x = __builtin_amdgcn_readfirstlane(h);
    }

    // The sleep loop sits inside one asm statement, so the compiler sees no
    // new control flow and allocates registers as in the product build.
    __device__ __forceinline__ void pause() {
        x = x * 1664525u + 1013904223u;   // LCG step; the top four bits pick the count
        uint32_t n = __builtin_amdgcn_readfirstlane(x >> 28);
        asm volatile(
            "s_cmp_eq_u32 %0, 0\n\t"
            "s_cbranch_scc1 1f\n"
            "0:\n\t"
            "s_sleep 1\n\t"
            "s_sub_u32 %0, %0, 1\n\t"
            "s_cmp_lg_u32 %0, 0\n\t"
            "s_cbranch_scc1 0b\n"
            "1:"
            : "+s"(n)
            :
            : "scc");
    }
#else
    __device__ __forceinline__ explicit Stagger(uint32_t) {}
    __device__ __forceinline__ void pause() {}
#endif
};

// Race-stress build: fill kBytes of LDS from lds0 with 0xFF, then meet, so
// no copy lands before the fill is complete.  Nothing in the product build.
template <uint32_t kBytes, int kThreads>
__device__ __forceinline__ void stagger_poison_lds(uint32_t lds0) {
#ifdef MCS_STAGGER
    static_assert(kBytes % (16 * kThreads) == 0, "whole 16-byte stores per thread");
#pragma unroll
    for (uint32_t i = 0; i < kBytes / (16u * kThreads); ++i) {
        const uint32_t off = (i * kThreads + threadIdx.x) * 16u;
        *reinterpret_cast<lds_i32x4 *>(static_cast<uintptr_t>(lds0 + off)) = i32x4{-1, -1, -1, -1};
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#else
    (void)lds0;
#endif
}

// Stage boundary: scheduling wall, workgroup rendezvous, scheduling wall
// (with the race-stress pauses on both sides of the barrier).
__device__ __forceinline__ void rendezvous(Stagger &sg) {
    sg.pause();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    sg.pause();
}

// A barrier only some waves take (the entry and exit offsets of two wave
// groups), with the race-stress pause before it.
__device__ __forceinline__ void group_barrier(Stagger &sg) {
    sg.pause();
    __builtin_amdgcn_s_barrier();
}

// 128-bit buffer resource: base, stride 0, num_records bytes, GFX9 config word.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_records) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = static_cast<int>(static_cast<uint32_t>(p));
    r.y = static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xFFFFu);
    r.z = static_cast<int>(num_records);
    r.w = 0x00020000;
    return r;
}

// One 16-byte-per-lane copy global -> LDS.  The lane's 16 bytes land at
// lds_base + kOff + 16*lane; voff selects the global bytes (>= num_records
// reads 0).  Issued from inline assembly so the compiler neither reorders it
// nor adds waits of its own: the schedule's explicit vmcnt waits cover it.
// M0 (the LDS destination) needs one wait state before the load reads it.
// The compiler treats M0 as reserved and may not honour the clobber; these
// kernels leave M0 to this asm alone (no compiler-generated instruction
// touches it, checked in the ISA).
template <uint32_t kOff>
__device__ __forceinline__ void copy16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    // Both values are wave-uniform by construction; readfirstlane states it so
    // the "s" operands always land in SGPRs (it folds away for SGPR values).
    rsrc.x = __builtin_amdgcn_readfirstlane(rsrc.x);
    rsrc.y = __builtin_amdgcn_readfirstlane(rsrc.y);
    rsrc.z = __builtin_amdgcn_readfirstlane(rsrc.z);
    rsrc.w = __builtin_amdgcn_readfirstlane(rsrc.w);
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile(
        "s_add_u32 m0, %0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_base), "v"(voff), "s"(rsrc), "n"(kOff)
        : "memory", "m0", "scc");
}

// Calls f(std::integral_constant<int, I>) for I = I0 .. I1-1.
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I0 < I1) {
        f(std::integral_constant<int, I0>{});
        static_for<I0 + 1, I1>(f);
    }
}

__device__ __forceinline__ i32x4 lds_read128(uint32_t addr) {
    return *reinterpret_cast<const lds_i32x4 *>(static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ i32x2 lds_read64_tr(uint32_t addr) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_i16x4 *>(static_cast<uintptr_t>(addr)));
    return __builtin_bit_cast(i32x2, v);
}

// One 16x16x32 FP16/BF16 MFMA: x holds the 16-column operand (k-slice of
// 8 elements per lane), y the 16-row operand.
template <int kElem>
__device__ __forceinline__ f32x4 mfma(i32x4 x, i32x4 y, f32x4 c) {
    static_assert(kElem != kElemFP8, "FP8 takes mfma_fp8");
    if constexpr (kElem == kElemBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                       __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                      __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
}

// One 16x16x128 FP8 E4M3 MFMA (the scaled f8f6f4 form with the identity
// scale 2^0 = E8M0 0x7F in every byte, operand formats 0 = E4M3, as in
// "Porting High-Performance HIP Kernels to FlyDSL", section "MFMA in
// FlyDSL").  A lane's 32 bytes of each operand are the same two 16-byte LDS
// chunks a FP16 lane reads for its two k-slices; both operands use the same
// lane -> k assignment, so the sum runs over the whole 128-deep K-step.
__device__ __forceinline__ f32x4 mfma_fp8(i32x4 x0, i32x4 x1, i32x4 y0, i32x4 y1, f32x4 c) {
    const i32x8 x = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const i32x8 y = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
}

// 32-bit LDS byte address of a __shared__ array.
template <typename T>
__device__ __forceinline__ uint32_t lds_address(T *smem) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) char *)smem));
}

// ---- global -> LDS loader ----------------------------------------------
//
// The kWaves waves of a workgroup share every copy: each operand half (16
// KiB) is sixteen 1-KiB pieces, and wave w moves pieces P*w .. P*w+P-1
// (P = 16 / kWaves), one buffer_load_dwordx4 ... lds per piece.  A piece of an
// A half (or of a B half given N x K) is 8 rows x 128 bytes: lane (x, pch)
// fills physical chunk pch of row x, which holds logical k-chunk pch ^ x, so
// the copy itself writes the XOR-swizzled layout.  A piece of a B half given
// K x N is 4 k-rows x 256 bytes, swizzled the same way for the transposing
// read.
// Copy windows of one 256x256 output tile (uniform values).  For A and for B
// given N x K, per half: byte address of the half's first row at k = 0, the
// window's extent at k = 0 (start of the last valid row + the K elements'
// bytes KB), and KB, or 0 when the half holds no valid row; at K-step s the
// window starts 128*s bytes on and holds data while 128*s < KB.  For B given
// K x N, per half: first column, bytes of one k-row's valid columns, and
// whether the half holds any valid column.  A tile with no valid row or
// column (the "no tile" value) copies zeros.
struct TileWindows {
    int m0, n0;
    uint64_t aAddr[2], bAddr[2];
    uint32_t aEnd[2], bEnd[2], aKB[2], bKB[2];
    const char *bBase[2];
    uint32_t bSpan[2];
    bool bLive[2];
};

// kTile: output tile edge (256: two halves per operand; 128: one, half 0);
// kBOff: byte offset of the B halves within an LDS buffer.
template <int kElem, bool kTransB, int kWaves, int kTile = kTileM, uint32_t kBOff = kOffB>
struct Loader {
    static constexpr int P = 16 / kWaves;   // pieces per wave per half
    static constexpr int kEB = elem_bytes(kElem), kStepK = step_k(kElem);
    static_assert(P * kWaves == 16, "waves must divide the 16 pieces of a half");
    static_assert(kTransB || kElem != kElemFP8, "FP8 B is taken given N x K");
    static_assert(kTile == 256 || kTile == 128, "tile edge");

    uint32_t lds0;                   // LDS byte address of buffer 0
    uint32_t cpA[P], cpB[P];         // copy voffsets
    int cpAchunk[P];                 // 16-byte k-chunk (of 8) each A / N x K B copy lane moves
    int wave;
    const GemmParams &p;
    TileWindows win;                 // the tile being computed
    mutable Stagger sg;              // race-stress pauses (empty in the product build)

    __device__ __forceinline__ Loader(const GemmParams &prm, int tm, int tn) : p(prm), sg(prm.stagger_seed) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        lds0 = 0;
        win = windows(tm, tn);
        const int x = lane >> 3, pch = lane & 7;
        for (int i = 0; i < P; ++i) {
            const int row = 8 * (P * wave + i) + x;           // row of the half
            const int c = pch ^ x;                             // logical 16-byte k-chunk (row & 7 = x)
            cpAchunk[i] = c;
            cpA[i] = static_cast<uint32_t>(row * p.lda * kEB + c * 16);
            if constexpr (kTransB)
                cpB[i] = static_cast<uint32_t>(row * p.ldb * kEB + c * 16);
        }
        if constexpr (!kTransB) {
            const int y = lane >> 4, pc = lane & 15;
            for (int i = 0; i < P; ++i) {
                const int krow = 4 * (P * wave + i) + y;
                const int ch = pc ^ (2 * ((krow & 3) + 4 * ((krow >> 3) & 1)));   // logical n-chunk
                cpB[i] = static_cast<uint32_t>(krow * p.ldb * kEB + ch * 16);
            }
        }
    }

    // Windows of output tile (tm, tn); tm >= tiles_m gives the no-tile value.
    __device__ __forceinline__ TileWindows windows(int tm, int tn) const {
        TileWindows w;
        w.m0 = tm * kTile;
        w.n0 = tn * kTile;
        const bool live = w.m0 < p.M;
        const uint32_t kb = static_cast<uint32_t>(kEB) * static_cast<uint32_t>(p.K);
        const char *A = static_cast<const char *>(p.A), *B = static_cast<const char *>(p.B);
        for (int h = 0; h < 2; ++h) {
            const int rows = min(max(p.M - (w.m0 + 128 * h), 0), 128);
            w.aAddr[h] = reinterpret_cast<uint64_t>(A + (int64_t)(w.m0 + 128 * h) * p.lda * kEB);
            w.aEnd[h] = rows > 0 ? static_cast<uint32_t>((rows - 1) * p.lda * kEB) + kb : 0u;
            w.aKB[h] = rows > 0 ? kb : 0u;
            const int cols = live ? min(max(p.N - (w.n0 + 128 * h), 0), 128) : 0;
            if constexpr (kTransB) {
                w.bAddr[h] = reinterpret_cast<uint64_t>(B + (int64_t)(w.n0 + 128 * h) * p.ldb * kEB);
                w.bEnd[h] = cols > 0 ? static_cast<uint32_t>((cols - 1) * p.ldb * kEB) + kb : 0u;
                w.bKB[h] = cols > 0 ? kb : 0u;
            } else {
                w.bLive[h] = cols > 0;
                w.bBase[h] = B + (w.n0 + 128 * h) * kEB;
                w.bSpan[h] = static_cast<uint32_t>(cols * kEB);
            }
        }
        return w;
    }

    // Buffer resource of a row-major (k contiguous) half at K-step s.
    static __device__ __forceinline__ i32x4 step_rsrc(uint64_t addr, uint32_t end, uint32_t kb, int s) {
        const uint32_t koff = static_cast<uint32_t>(s) * kStepBytes;
        const uint64_t a = addr + koff;
        i32x4 r;
        r.x = static_cast<int>(static_cast<uint32_t>(a));
        r.y = static_cast<int>(static_cast<uint32_t>(a >> 32));   // < 2^16: stride 0
        r.z = static_cast<int>(koff < kb ? end - koff : 0u);
        r.w = 0x00020000;
        return r;
    }

    // Copy half h of operand A (rows m0+128h.. of tile w) for K-step s into
    // buffer `buf`.  The window ends at the last valid byte of the half's last
    // valid row, so rows >= M and every k >= K (steps past the end: an empty
    // window) read 0.  Pieces I0 .. I1-1 of this wave's share (all of them by
    // default).  kMask = false skips the per-lane k-chunk mask: allowed when
    // the step is either whole (all its k valid) or wholly past the end.
    template <bool kMask = true, int I0 = 0, int I1 = P>
    __device__ __forceinline__ void copy_a(const TileWindows &w, int s, uint32_t buf, int h) const {
        const int kvb = (p.K - s * kStepK) * kEB;             // bytes of k left (may be <= 0)
        const i32x4 rs = step_rsrc(w.aAddr[h], w.aEnd[h], w.aKB[h], s);
        const uint32_t dst = lds0 + buf + kOffA + h * kHalf + P * wave * 1024;
        static_for<I0, I1>([&](auto i) {
            const uint32_t v = (!kMask || cpAchunk[i] * 16 < kvb) ? cpA[i] : kOutOfWindow;
            copy16<i * 1024>(rs, dst, v);
        });
    }

    // Copy half h of operand B (columns n0+128h.. of tile w) for K-step s into buffer `buf`.
    template <bool kMask = true, int I0 = 0, int I1 = P>
    __device__ __forceinline__ void copy_b(const TileWindows &w, int s, uint32_t buf, int h) const {
        const int kv = p.K - s * kStepK;                      // k left (may be <= 0)
        const uint32_t dst = lds0 + buf + kBOff + h * kHalf + P * wave * 1024;
        if constexpr (kTransB) {
            const i32x4 rs = step_rsrc(w.bAddr[h], w.bEnd[h], w.bKB[h], s);
            static_for<I0, I1>([&](auto i) {
                const uint32_t v = (!kMask || cpAchunk[i] * 16 < kv * kEB) ? cpB[i] : kOutOfWindow;
                copy16<i * 1024>(rs, dst, v);
            });
        } else {
            // k-rows k0 .. k0+rows-1; the window ends at the last valid column
            // of the last valid k-row, so k-rows >= K read 0 without a mask
            const int rows = min(kv, kStepK);
            const uint32_t nrec = (w.bLive[h] && kv > 0)
                ? static_cast<uint32_t>(rows - 1) * static_cast<uint32_t>(p.ldb * kEB) + w.bSpan[h] : 0u;
            const i32x4 rs = make_rsrc(w.bBase[h] + (int64_t)s * kStepK * p.ldb * kEB, nrec);
            static_for<I0, I1>([&](auto i) { copy16<i * 1024>(rs, dst, cpB[i]); });
        }
    }

    // The same for the tile being computed.
    template <bool kMask = true, int I0 = 0, int I1 = P>
    __device__ __forceinline__ void copy_a(int s, uint32_t buf, int h) const {
        copy_a<kMask, I0, I1>(win, s, buf, h);
    }
    template <bool kMask = true, int I0 = 0, int I1 = P>
    __device__ __forceinline__ void copy_b(int s, uint32_t buf, int h) const {
        copy_b<kMask, I0, I1>(win, s, buf, h);
    }
};

// LDS offsets of one lane's MFMA operand fragments within a half.  A fragment
// (16 rows x 32 k) is one 16-byte chunk per lane: row row0 + (lane & 15),
// k-chunk 4*ks + (lane >> 4).  For B given K x N the fragment of 16 columns
// is two transposing 8-byte reads per lane (k-rows 32ks + 8g + r and
// 32ks + 4 + 8g + r, r = (lane & 15) >> 2), at the per-nt offsets below
// plus the constant (32*ks + {0, 4}) * 256.
struct FragOffsets {
    uint32_t row[2];   // chunk-read offset for rows row0.., ks = 0, 1 (add 2048 per 16 rows)
    uint32_t tr[4];    // transposing-read offset for columns col0 + 16nt, k-row 8g + r

    __device__ __forceinline__ void rows(int row0, int lane) {
        const int l16 = lane & 15, lg = lane >> 4;
        const int swz = lane & 7;                  // = row & 7 for the 16 rows of a read
        for (int ks = 0; ks < 2; ++ks)
            row[ks] = (row0 + l16) * 128 + (((4 * ks) | lg) ^ swz) * 16;
    }

    // col0 a multiple of 32
    __device__ __forceinline__ void cols_tr(int col0, int lane) {
        // lane (lg, l16) of a transposed read for (nt, ks, h) loads 8 bytes of
        // k-row 32ks + 4h + 8lg + (l16 >> 2), columns col0 + 16nt + 4(l16 & 3):
        // the (ks, h) part of the row is a constant offset, the swizzle only
        // sees the lane part of the row.
        const int l16 = lane & 15, lg = lane >> 4;
        const int fb = 2 * ((l16 >> 2) + 4 * (lg & 1));
        for (int nt = 0; nt < 4; ++nt) {
            const int ch = col0 / 8 + 2 * nt + ((l16 & 3) >> 1);
            tr[nt] = (8 * lg + (l16 >> 2)) * 256 + ((ch ^ fb) * 16) + 8 * (l16 & 1);
        }
    }
};

// Fragment reads of one wave's 64x64 block of a 128x128 quadrant: A rows
// 64wm.. of an A half, B columns 64wn.. of a B half (the B halves at byte
// offset kBOff of an LDS buffer).  A fragment is four 16-row (16-column)
// tiles x two 16-byte k-chunks per lane, read as eight pieces.  The read
// bases of a K-step are computed once and kept opaque to the compiler, so
// every piece is a base plus an immediate offset.
template <bool kTransB, uint32_t kBOff>
struct Block64Reader {
    FragOffsets fa, fb;

    __device__ __forceinline__ void init(int wm, int wn, int lane) {
        fa.rows(64 * wm, lane);
        if constexpr (kTransB)
            fb.rows(64 * wn, lane);
        else
            fb.cols_tr(64 * wn, lane);
    }

    struct Bases {
        uint32_t a[2][2];    // [buffer cur/nxt][ks]: A fragment rows, A half 0
        uint32_t b[2][2];    // [buffer][ks]: B fragment rows (B given N x K), B half 0
        uint32_t buf[2];     // LDS byte address of buffer cur / nxt (uniform)
    };

    __device__ __forceinline__ Bases bases_at(uint32_t lds0, uint32_t cur, uint32_t nxt) const {
        Bases r;
        for (int u = 0; u < 2; ++u) {
            r.buf[u] = lds0 + (u ? nxt : cur);
            for (int ks = 0; ks < 2; ++ks) {
                r.a[u][ks] = r.buf[u] + kOffA + fa.row[ks];
                asm volatile("" : "+v"(r.a[u][ks]));
                if constexpr (kTransB) {
                    r.b[u][ks] = r.buf[u] + kBOff + fb.row[ks];
                    asm volatile("" : "+v"(r.b[u][ks]));
                }
            }
        }
        return r;
    }

    // Piece j (k-chunk j >> 2, 16-row tile j & 3) of a fragment of A half h.
    __device__ __forceinline__ i32x4 read_a(const Bases &bs, int u, int h, int j) const {
        return lds_read128(bs.a[u][j >> 2] + h * kHalf + (j & 3) * 2048);
    }

    // Piece j (k-chunk j >> 2, 16-column tile j & 3) of a fragment of B half h.
    __device__ __forceinline__ i32x4 read_b(const Bases &bs, int u, int h, int j) const {
        const int ks = j >> 2, nt = j & 3;
        if constexpr (kTransB) {
            return lds_read128(bs.b[u][ks] + h * kHalf + nt * 2048);
        } else {
            // one address add per piece; the k-row offsets are immediates
            uint32_t base = bs.buf[u] + kBOff + h * kHalf + fb.tr[nt];
            asm volatile("" : "+v"(base));
            const i32x2 lo = lds_read64_tr(base + (32 * ks + 0) * 256);
            const i32x2 hi = lds_read64_tr(base + (32 * ks + 4) * 256);
            return i32x4{lo.x, lo.y, hi.x, hi.y};
        }
    }
};

// Output tile of virtual workgroup wg (the workgroup id, or for a workgroup
// that computes several tiles wg = id + r * grid for its r-th tile, the grid
// a multiple of 8 so every tile stays on its workgroup's XCD).
__device__ __forceinline__ void tile_coords(const GemmParams &p, int wg, int &tm, int &tn) {
    // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2);
    // renumber so each XCD gets a contiguous range of tiles, then walk that
    // range in groups of group_m tile rows so neighbours share A and B tiles.
    const int total = p.tiles_m * p.tiles_n;
    const int xcd = wg & 7, j = wg >> 3;
    const int q = total >> 3, r = total & 7;
    const int tile = xcd * q + min(xcd, r) + j;
    const int width = p.group_m * p.tiles_n;
    const int g = tile / width;
    const int first_m = g * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int in = tile - g * width;
    tm = first_m + in % gm;
    tn = in / gm;
}

// ---- fused epilogue ------------------------------------------------------
//
// Store one lane's part of kN (2 or 4) neighbouring 16x16 accumulator tiles
// (columns col0 .. col0+16kN-1 of row `row`).  With the B fragment as the first MFMA
// operand, lane l of tile nt holds columns 16nt + 4(l >> 4) .. +3 of row
// l & 15.  FP32 output stores those four values (16 bytes).  For a 16-bit
// output (FP16, or BF16 with kBF16; round to nearest even), lanes l and l^16
// trade halves of tiles nt and nt+1 so every lane stores eight consecutive
// columns (16 bytes).  The trade is two v_permlane16_swap (gfx950), which swap
// the odd 16-lane rows of their first operand with the even rows of their
// second: with tile nt's packed values as the first operand and tile nt+1's
// as the second, an even lane group ends up holding its own four columns of
// tile nt followed by its partner's, and an odd group its partner's four
// columns of tile nt+1 followed by its own, with no LDS round trip.  Columns
// at or past N are not written.
template <bool kBF16, bool kOutF32, int kN>
__device__ __forceinline__ void store_strip(const GemmParams &p, const f32x4 (&v4)[kN], int row,
                                            int col0, int lane) {
    static_assert(kN == 2 || kN == 4, "pairs of 16-column tiles");
    const int g = lane >> 4;
    if constexpr (kOutF32) {
        for (int nt = 0; nt < kN; ++nt) {
            const int col = col0 + 16 * nt + 4 * g;
            f32x4 v = v4[nt];
            asm volatile("" : "+v"(v));   // stage through VGPRs: keeps the accumulators' allocation free
            float *c = reinterpret_cast<float *>(p.C) + (int64_t)row * p.ldc + col;
            if (col + 4 <= p.N) {
                *reinterpret_cast<f32x4 *>(c) = v;
            } else {
                for (int r = 0; r < 4; ++r)
                    if (col + r < p.N) c[r] = v[r];
            }
        }
    } else {
        for (int nt = 0; nt < kN; nt += 2) {
            i32x2 h0, h1;
            if constexpr (kBF16) {
                h0 = __builtin_bit_cast(i32x2, __builtin_convertvector(v4[nt], bf16x4));
                h1 = __builtin_bit_cast(i32x2, __builtin_convertvector(v4[nt + 1], bf16x4));
            } else {
                h0 = __builtin_bit_cast(i32x2, __builtin_convertvector(v4[nt], f16x4));
                h1 = __builtin_bit_cast(i32x2, __builtin_convertvector(v4[nt + 1], f16x4));
            }
            const bool odd = g & 1;
            const auto sx = __builtin_amdgcn_permlane16_swap(h0.x, h1.x, false, false);
            const auto sy = __builtin_amdgcn_permlane16_swap(h0.y, h1.y, false, false);
            const i32x4 out = {static_cast<int>(sx[0]), static_cast<int>(sy[0]), static_cast<int>(sx[1]),
                               static_cast<int>(sy[1])};
            const int col = col0 + 16 * nt + (odd ? 16 + 4 * (g - 1) : 4 * g);
            uint16_t *c = reinterpret_cast<uint16_t *>(p.C) + (int64_t)row * p.ldc + col;
            if (col + 8 <= p.N) {
                *reinterpret_cast<i32x4 *>(c) = out;
            } else {
                const i16x8 e = __builtin_bit_cast(i16x8, out);
                for (int r = 0; r < 8; ++r)
                    if (col + r < p.N) c[r] = static_cast<uint16_t>(e[r]);
            }
        }
    }
}

}  // namespace
}  // namespace mcs
