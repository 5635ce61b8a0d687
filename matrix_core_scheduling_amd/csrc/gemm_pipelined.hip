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
// work to cover it ("Stage Size and Register Pressure": stages must hold
// enough matrix work to cover preparation without excessive barrier
// overhead).  The loop is unrolled twice so each LDS buffer is addressed
// statically.  Copies of future tiles go straight from global memory into
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
// Schedule of K-step t (cur = buffer of t, nxt = buffer of t+1); aX/bX are
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
// fragment VGPRs are live (a0 a1 b0 b1 is 16+16+32+32, never all four).
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
// and columns 64wn..64wn+63 of every B half: a 32x64 block of each quadrant.
// MFMA: v_mfma_f32_16x16x32_{f16,bf16} with the B fragment as the first
// operand, so each lane ends with four consecutive columns of one row; for a
// 16-bit output, lanes l and l^16 trade halves of two neighbouring tiles so
// every lane stores eight consecutive columns (16 bytes).
#include "internal.h"

namespace mcs {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr uint32_t kHalf = 16384;          // bytes of one operand half in LDS
constexpr uint32_t kBuf = 4 * kHalf;       // one K-step: A0 A1 B0 B1
constexpr uint32_t kOffA = 0, kOffB = 2 * kHalf;
constexpr uint32_t kOutOfWindow = 0x80000000u;  // >= every buffer window used here
constexpr int kCopyWait = 8;               // vmcnt at the end of each memory stage

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

// Stage boundary: scheduling wall, workgroup rendezvous, scheduling wall.
__device__ __forceinline__ void rendezvous() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
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
// lds_base + 16*lane; voff selects the global bytes (>= num_records reads 0).
// Issued from inline assembly so the compiler neither reorders it nor adds
// waits of its own: the schedule's explicit vmcnt waits cover it.
__device__ __forceinline__ void copy16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    // Both values are wave-uniform by construction; readfirstlane states it so
    // the "s" operands always land in SGPRs (it folds away for SGPR values).
    rsrc.x = __builtin_amdgcn_readfirstlane(rsrc.x);
    rsrc.y = __builtin_amdgcn_readfirstlane(rsrc.y);
    rsrc.z = __builtin_amdgcn_readfirstlane(rsrc.z);
    rsrc.w = __builtin_amdgcn_readfirstlane(rsrc.w);
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_base), "v"(voff), "s"(rsrc)
        : "memory", "m0");
}

__device__ __forceinline__ i32x4 lds_read128(uint32_t addr) {
    return *reinterpret_cast<const lds_i32x4 *>(static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ i32x2 lds_read64_tr(uint32_t addr) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_i16x4 *>(static_cast<uintptr_t>(addr)));
    return __builtin_bit_cast(i32x2, v);
}

template <bool kBF16>
__device__ __forceinline__ f32x4 mfma(i32x4 x, i32x4 y, f32x4 c) {
    if constexpr (kBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                       __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                      __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
}

// ---- the kernel -----------------------------------------------------------

template <bool kBF16, bool kTransB, bool kOutF32, bool kOffset>
struct Pipeline {
    // per-lane constants
    uint32_t lds0;                   // LDS byte address of buffer 0
    uint32_t rdA[2], rdB[2];         // fragment read offsets within a half (ks = 0, 1)
    uint32_t rdBt[4];                // K x N B: per-nt transposed-read offsets (ks, h add constants)
    uint32_t cpA[2], cpB[2];         // copy voffsets (two copies per half per wave)
    int cpAchunk[2];                 // k-chunk (of 8) each A / N x K B copy lane moves
    int cpBrow[2];                   // k-row each K x N B copy lane moves
    int wave;
    const GemmParams &p;
    int m0, n0;
    // per-half copy windows (uniform; computed once): first row (A, or B given
    // N x K) or first column (B given K x N) of the half, the window's bytes
    // before the k-extent, and whether the half holds any valid row/column
    const uint16_t *aRow[2], *bBase[2];
    uint32_t aSpan[2], bSpan[2];
    bool aLive[2], bLive[2];

    __device__ __forceinline__ Pipeline(const GemmParams &prm, int tm, int tn) : p(prm) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave & 3, wn = wave >> 2;
        m0 = tm * kTileM;
        n0 = tn * kTileN;
        lds0 = 0;
        for (int h = 0; h < 2; ++h) {
            const int rows = min(max(p.M - (m0 + 128 * h), 0), 128);
            aLive[h] = rows > 0;
            aRow[h] = p.A + (int64_t)(m0 + 128 * h) * p.lda;
            aSpan[h] = rows > 0 ? static_cast<uint32_t>((rows - 1) * p.lda * 2) : 0u;
            const int cols = min(max(p.N - (n0 + 128 * h), 0), 128);
            bLive[h] = cols > 0;
            if constexpr (kTransB) {
                bBase[h] = p.B + (int64_t)(n0 + 128 * h) * p.ldb;
                bSpan[h] = cols > 0 ? static_cast<uint32_t>((cols - 1) * p.ldb * 2) : 0u;
            } else {
                bBase[h] = p.B + n0 + 128 * h;
                bSpan[h] = static_cast<uint32_t>(cols * 2);
            }
        }

        const int l16 = lane & 15, lg = lane >> 4;
        const int swz = lane & 7;                  // = row & 7 for the 16 rows of a read
        for (int ks = 0; ks < 2; ++ks) {
            rdA[ks] = (32 * wm + l16) * 128 + (((4 * ks) | lg) ^ swz) * 16;
            rdB[ks] = (64 * wn + l16) * 128 + (((4 * ks) | lg) ^ swz) * 16;
        }
        if constexpr (!kTransB) {
            // lane (lg, l16) of a transposed read for (nt, ks, h) loads 8 bytes of
            // k-row 32ks + 4h + 8lg + (l16 >> 2), columns 64wn + 16nt + 4(l16 & 3):
            // the (ks, h) part of the row is a constant offset, the swizzle
            // only sees the lane part of the row.
            const int fb = 2 * ((l16 >> 2) + 4 * (lg & 1));
            for (int nt = 0; nt < 4; ++nt) {
                const int ch = 8 * wn + 2 * nt + ((l16 & 3) >> 1);
                rdBt[nt] = (8 * lg + (l16 >> 2)) * 256 + ((ch ^ fb) * 16) + 8 * (l16 & 1);
            }
        }
        // copies: wave w moves 1-KiB pieces 2w and 2w+1 of every half; lane
        // (x, pch) fills physical chunk pch of row 8*piece + x
        const int x = lane >> 3, pch = lane & 7;
        for (int i = 0; i < 2; ++i) {
            const int row = 16 * wave + 8 * i + x;            // row of the half
            const int c = pch ^ x;                             // logical 16-byte k-chunk (row & 7 = x)
            cpAchunk[i] = c;
            cpA[i] = static_cast<uint32_t>(row * p.lda * 2 + c * 16);
            if constexpr (kTransB)
                cpB[i] = static_cast<uint32_t>(row * p.ldb * 2 + c * 16);
        }
        if constexpr (!kTransB) {
            const int y = lane >> 4, pc = lane & 15;
            const int ch = pc ^ (2 * (y + 4 * (wave & 1)));    // logical 16-byte n-chunk
            for (int i = 0; i < 2; ++i) {
                const int krow = 8 * wave + 4 * i + y;
                cpBrow[i] = krow;
                cpB[i] = static_cast<uint32_t>(krow * p.ldb * 2 + ch * 16);
            }
        }
    }

    // Copy half h of operand A (rows m0+128h..) for K-step s into buffer `buf`.
    // The window ends at the last valid byte of the half's last valid row, so
    // rows >= M and every k >= K (steps past the end: an empty window) read 0.
    __device__ __forceinline__ void copy_a(int s, uint32_t buf, int h) const {
        const int kv = p.K - s * kTileK;                      // k left (may be <= 0)
        const uint32_t nrec = (aLive[h] && kv > 0) ? aSpan[h] + 2u * static_cast<uint32_t>(kv) : 0u;
        const i32x4 rs = make_rsrc(aRow[h] + s * kTileK, nrec);
        const uint32_t dst = lds0 + buf + kOffA + h * kHalf + 2 * wave * 1024;
        for (int i = 0; i < 2; ++i) {
            const uint32_t v = (cpAchunk[i] * 8 < kv) ? cpA[i] : kOutOfWindow;
            copy16(rs, dst + i * 1024, v);
        }
    }

    // Copy half h of operand B (columns n0+128h..) for K-step s into buffer `buf`.
    __device__ __forceinline__ void copy_b(int s, uint32_t buf, int h) const {
        const int kv = p.K - s * kTileK;
        const uint32_t dst = lds0 + buf + kOffB + h * kHalf + 2 * wave * 1024;
        if constexpr (kTransB) {
            const uint32_t nrec = (bLive[h] && kv > 0) ? bSpan[h] + 2u * static_cast<uint32_t>(kv) : 0u;
            const i32x4 rs = make_rsrc(bBase[h] + s * kTileK, nrec);
            for (int i = 0; i < 2; ++i) {
                const uint32_t v = (cpAchunk[i] * 8 < kv) ? cpB[i] : kOutOfWindow;
                copy16(rs, dst + i * 1024, v);
            }
        } else {
            // k-rows k0 .. k0+rows-1; the window ends at the last valid column
            // of the last valid k-row
            const int rows = min(kv, kTileK);
            const uint32_t nrec = (bLive[h] && kv > 0)
                ? static_cast<uint32_t>(rows - 1) * static_cast<uint32_t>(p.ldb * 2) + bSpan[h] : 0u;
            const i32x4 rs = make_rsrc(bBase[h] + (int64_t)s * kTileK * p.ldb, nrec);
            for (int i = 0; i < 2; ++i) {
                const uint32_t v = (cpBrow[i] < kv) ? cpB[i] : kOutOfWindow;
                copy16(rs, dst + i * 1024, v);
            }
        }
    }

    __device__ __forceinline__ void read_a(i32x4 (&a)[2][2], uint32_t buf, int h) const {
        const uint32_t base = lds0 + buf + kOffA + h * kHalf;
        for (int mt = 0; mt < 2; ++mt)
            for (int ks = 0; ks < 2; ++ks)
                a[mt][ks] = lds_read128(base + rdA[ks] + mt * 2048);
    }

    __device__ __forceinline__ void read_b(i32x4 (&b)[4][2], uint32_t buf, int h) const {
        const uint32_t base = lds0 + buf + kOffB + h * kHalf;
        if constexpr (kTransB) {
            for (int nt = 0; nt < 4; ++nt)
                for (int ks = 0; ks < 2; ++ks)
                    b[nt][ks] = lds_read128(base + rdB[ks] + nt * 2048);
        } else {
            for (int nt = 0; nt < 4; ++nt)
                for (int ks = 0; ks < 2; ++ks) {
                    const i32x2 lo = lds_read64_tr(base + rdBt[nt] + (32 * ks + 0) * 256);
                    const i32x2 hi = lds_read64_tr(base + rdBt[nt] + (32 * ks + 4) * 256);
                    b[nt][ks] = i32x4{lo.x, lo.y, hi.x, hi.y};
                }
        }
    }
};

template <bool kBF16>
__device__ __forceinline__ void quadrant(f32x4 (&acc)[2][4], const i32x4 (&a)[2][2],
                                         const i32x4 (&b)[4][2]) {
    for (int ks = 0; ks < 2; ++ks)
        for (int mt = 0; mt < 2; ++mt)
            for (int nt = 0; nt < 4; ++nt)
                acc[mt][nt] = mfma<kBF16>(b[nt][ks], a[mt][ks], acc[mt][nt]);
}

__device__ __forceinline__ void mem_stage_begin() { __builtin_amdgcn_s_setprio(1); }

// End of a memory stage: this wave's copies for the reads two stages later
// have landed, and so have its own LDS reads (their registers feed the next
// stage and their half may be refilled two stages on).
__device__ __forceinline__ void mem_stage_end() {
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kCopyWait>();
    wait_lgkmcnt<0>();
    __builtin_amdgcn_s_setprio(0);
    rendezvous();
}

__device__ __forceinline__ void tile_coords(const GemmParams &p, int &tm, int &tn) {
    // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2);
    // renumber so each XCD gets a contiguous range of tiles, then walk that
    // range in groups of group_m tile rows so neighbours share A and B tiles.
    const int wg = blockIdx.x;
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

template <bool kBF16, bool kTransB, bool kOutF32, bool kOffset>
__global__ void __launch_bounds__(kPipeThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_pipelined_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * kBuf];

    int tm, tn;
    tile_coords(p, tm, tn);
    Pipeline<kBF16, kTransB, kOutF32, kOffset> pl(p, tm, tn);
    // generic -> LDS address space: the 32-bit LDS byte address of smem
    pl.lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) char *)smem));
    const int wave = pl.wave;

    f32x4 acc[2][2][2][4];
    for (int qa = 0; qa < 2; ++qa)
        for (int qb = 0; qb < 2; ++qb)
            for (int mt = 0; mt < 2; ++mt)
                for (int nt = 0; nt < 4; ++nt)
                    acc[qa][qb][mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x4 a0[2][2], a1[2][2], b0[4][2], b1[4][2];

    // ---- prologue: the copy stream of steps 0 and 1 in steady-state order
    // (a0 a1 b0, then b1, per step), then the fragments S0 of step 0 needs.
    pl.copy_a(0, 0, 0);
    pl.copy_a(0, 0, 1);
    pl.copy_b(0, 0, 0);
    pl.copy_b(0, 0, 1);
    pl.copy_a(1, kBuf, 0);
    pl.copy_a(1, kBuf, 1);
    pl.copy_b(1, kBuf, 0);
    pl.copy_b(1, kBuf, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<10>();                   // a0(0) a1(0) b0(0) landed (this wave's part)
    rendezvous();                       // ... and every wave's part
    pl.read_a(a0, 0, 0);
    pl.read_a(a1, 0, 1);
    pl.read_b(b0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt<0>();
    wait_vmcnt<kCopyWait>();            // b1(0) landed: the state at the end of S3 of step -1
    rendezvous();

    if constexpr (kOffset) {
        if (wave >= 4) __builtin_amdgcn_s_barrier();   // group B waits: entry offset
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- steady state, two K-steps per iteration (buffer 0 then buffer 1)
    for (int t = 0; t < p.steps; t += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t cur = u ? kBuf : 0u, nxt = u ? 0u : kBuf;
            const int s = t + u;
            // S0: quadrants Q00 and Q10
            quadrant<kBF16>(acc[0][0], a0, b0);
            quadrant<kBF16>(acc[1][0], a1, b0);
            rendezvous();
            // S1
            mem_stage_begin();
            pl.read_b(b1, cur, 1);
            pl.copy_a(s + 2, cur, 0);
            pl.copy_a(s + 2, cur, 1);
            pl.copy_b(s + 2, cur, 0);
            mem_stage_end();
            // S2: quadrants Q01 and Q11
            quadrant<kBF16>(acc[0][1], a0, b1);
            quadrant<kBF16>(acc[1][1], a1, b1);
            rendezvous();
            // S3
            mem_stage_begin();
            pl.read_a(a0, nxt, 0);
            pl.read_a(a1, nxt, 1);
            pl.read_b(b0, nxt, 0);
            pl.copy_b(s + 2, cur, 1);
            mem_stage_end();
        }
    }

    if constexpr (kOffset) {
        __builtin_amdgcn_sched_barrier(0);
        if (wave < 4) __builtin_amdgcn_s_barrier();    // group A waits: exit offset
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();   // the zero-window copies of steps past the end, before LDS is released

    // ---- epilogue: lane holds C[row][col .. col+3] of each 16x16 tile.  The
    // lane id is recomputed here so no lane-derived value stays live across
    // the loop.
    const int lane = __lane_id();
    const int wm = wave & 3, wn = wave >> 2;
    const int g = lane >> 4;
    for (int qa = 0; qa < 2; ++qa)
        for (int mt = 0; mt < 2; ++mt) {
            const int row = pl.m0 + 128 * qa + 32 * wm + 16 * mt + (lane & 15);
            if (row >= p.M) continue;
            for (int qb = 0; qb < 2; ++qb) {
                const int col0 = pl.n0 + 128 * qb + 64 * wn;
                if constexpr (kOutF32) {
                    for (int nt = 0; nt < 4; ++nt) {
                        const int col = col0 + 16 * nt + 4 * g;
                        const f32x4 v = acc[qa][qb][mt][nt];
                        float *c = reinterpret_cast<float *>(p.C) + (int64_t)row * p.ldc + col;
                        if (col + 4 <= p.N) {
                            *reinterpret_cast<f32x4 *>(c) = v;
                        } else {
                            for (int r = 0; r < 4; ++r)
                                if (col + r < p.N) c[r] = v[r];
                        }
                    }
                } else {
                    // Tiles nt and nt+1: lanes g and g^1 trade four values so
                    // each lane holds eight consecutive columns (16 bytes).
                    for (int nt = 0; nt < 4; nt += 2) {
                        i32x2 h0, h1;
                        if constexpr (kBF16) {
                            h0 = __builtin_bit_cast(i32x2, __builtin_convertvector(acc[qa][qb][mt][nt], bf16x4));
                            h1 = __builtin_bit_cast(i32x2, __builtin_convertvector(acc[qa][qb][mt][nt + 1], bf16x4));
                        } else {
                            h0 = __builtin_bit_cast(i32x2, __builtin_convertvector(acc[qa][qb][mt][nt], f16x4));
                            h1 = __builtin_bit_cast(i32x2, __builtin_convertvector(acc[qa][qb][mt][nt + 1], f16x4));
                        }
                        const bool odd = g & 1;
                        const i32x2 send = odd ? h0 : h1;
                        i32x2 recv;
                        recv.x = __shfl_xor(send.x, 16);
                        recv.y = __shfl_xor(send.y, 16);
                        const i32x4 out = odd ? i32x4{recv.x, recv.y, h1.x, h1.y}
                                              : i32x4{h0.x, h0.y, recv.x, recv.y};
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
        }
}

}  // namespace

const void *pipelined_kernel(bool bf16, bool trans_b, bool out_f32, bool offset) {
#define MCS_PICK(B, T, O, S)                                                         \
    if (bf16 == B && trans_b == T && out_f32 == O && offset == S)                   \
        return reinterpret_cast<const void *>(&gemm_pipelined_kernel<B, T, O, S>);
#define MCS_PICK_S(B, T, O) MCS_PICK(B, T, O, true) MCS_PICK(B, T, O, false)
#define MCS_PICK_O(B, T) MCS_PICK_S(B, T, false) MCS_PICK_S(B, T, true)
    MCS_PICK_O(false, false)
    MCS_PICK_O(false, true)
    MCS_PICK_O(true, false)
    MCS_PICK_O(true, true)
#undef MCS_PICK_O
#undef MCS_PICK_S
#undef MCS_PICK
    return nullptr;
}

}  // namespace mcs
