// Attention forward pass for gfx950 in the stage abstraction of the GEMM
// kernel: "Two Waves, One Stage Apart: Warp-Pipelining Triton GEMMs on AMD
// Instinct", section "Beyond GEMM: FlashAttention" (Figure 11) lays out the
// loop: for each block of keys, the score product, an online softmax in two
// halves, the product with V, and the copies that bring in later K and V
// blocks; the scores of block i+1 are computed before block i's product
// with V, and while one wave group multiplies the other runs its softmax.  That page gives the schedule
// for MI450 only, with no measurements; this is its MI355X form.
//
// Workgroup: 8 waves; a tile is 256 query rows of one (batch, head), wave w
// owning rows 32w..32w+31 (two 16-row MFMA tiles).  Group A = waves 0-3,
// group B = waves 4-7; each SIMD holds one wave of each.  Head size 128, keys
// in blocks of 64.  Per block each wave runs 32 MFMAs 16x16x32 for
// S = Q K^T (its 32 rows x 64 keys) and 32 for O += P V (32 rows x 128),
// FP32 accumulation.
//
// Persistent: one workgroup per CU (the 128 KiB of LDS admit no second)
// takes its tiles in a fixed order (attn_tile).  Between two tiles nothing
// waits for a new workgroup: the copies that would run past a tile's last
// block (zero windows) fetch the next tile's K blocks 0-3 and V blocks 0-1
// instead, and its last trip loads the next tile's Q, so the next prologue
// finds its operands in place and waits only for them, not for this tile's
// stores (a fixed number per wave: buffer stores whose window ends at the
// last row).
//
// Two stages per trip (i = 0 .. blocks-2), each ended by a workgroup
// barrier; group B runs one stage behind group A (an extra barrier on entry
// for B and on exit for A, as in the GEMM), so the MFMA stage of one group
// overlaps the softmax stage of the other:
//   M  MFMA   S(i+1) = Q K(i+1)^T, then O += P(i) V(i) (64 MFMAs).  The
//             fragment reads go out one after each MFMA, into registers the
//             stage has just freed: the first half of the V(i) fragments
//             during the second half of the score MFMAs (into the used K
//             fragments' registers), the second half of V(i) during the
//             first half of the P V MFMAs, and K(i+2) during the second
//             half.  This wave's copies of K(i+4) and V(i+2) follow every
//             fourth of the first 16 MFMAs; wait for the previous trip's.
//   V  VALU   row max of S(i+1): m(i+1), alpha(i+1) = 2^(m(i) - m(i+1));
//             O *= alpha(i+1); P(i+1) = 2^(c S(i+1) - m(i+1)) rounded to the
//             operand type; l = alpha(i+1) l + row sums
// with c = scale * log2(e).  The page's figure splits the softmax into two
// stages between the two products; here both products share one stage and
// the whole softmax the other, which halves the barriers per block and
// pairs each group's 64 MFMAs with the other group's whole softmax.  The
// sequence of operations on every accumulator is the same either way.  Per
// tile a prologue computes S(0), P(0); a drain does P V of the last block;
// then O / l is stored with lse = (m + log2 l) ln 2.
//
// LDS: two rings of four 16-KiB slots (64 keys x 256 bytes), one for K
// blocks and one for V blocks, filled by buffer_load ... lds (all 8 waves,
// two 1-KiB pieces of each block per wave); keys past the end read as zeros
// and are masked.  The rings run on across tiles: block j of a tile sits in
// slot (g0 + j) mod 4, g0 the number of blocks of the workgroup's earlier
// tiles, so the next tile's first blocks land where this tile's would have
// gone, under the same waits (the last trips' copies are the next tile's).
// K rows store 16-byte chunk c at c ^ (row & 15) (the
// ds_read_b128 of 16 rows at one chunk is conflict-free); V rows at
// c ^ 2(row & 7) (each half-wave of a transposing ds_read_b64_tr_b16 touches
// 8 rows x 32 bytes, distinct banks).  K(j) is read two trips before V(j)
// (in the M stage of trip j-2 against trip j), so each has its own ring.
// With global stage g (group A's stage g, group B's stage g-1; A's trip i
// is stages 2i and 2i+1):
//   * read -> refill: a wave's reads of the M stage complete before the
//     barrier that ends its V stage (lgkmcnt(0)).  K(j) is read last by
//     group B in stage 2j-3, done before barrier 2j-2; its slot takes
//     K(j+4), copied in trip j (stage 2j for A, 2j+1 for B).  V(j) is read
//     last in stage 2j+1, done before barrier 2j+2; V(j+4) is copied in
//     trip j+2 (stage 2j+4 or later).
//   * copy -> read: a wave waits for its copies of trip k (vmcnt(4): only
//     trip k+1's four may still fly) at the end of its M stage of trip k+1,
//     that is before barrier 2k+3 in group B and 2k+2 in group A.  Their
//     first reader is group A in stage 2k+4 (K(k+4) in trip k+2, V(k+2) in
//     trip k+2), after that barrier.
//
// The probabilities are packed straight from the S accumulators: a lane
// holds 4 consecutive keys of one row per 16-key tile, so the PV MFMA takes
// keys {4g..4g+3, 16+4g..16+4g+3} of a 32-key chunk in lane group g, and the
// V fragment is read with the same key order (transposing reads of k-rows
// 4g+e and 16+4g+e).
#include "device.h"

#include "mcs_attention.h"

#include <algorithm>
#include <atomic>
#include <cmath>

namespace mcs {
namespace {

constexpr int kHeadDim = 128;
constexpr int kRowBytes = kHeadDim * 2;                    // one K / V / Q row
constexpr int kQRows = 256;                                // query rows per workgroup
constexpr int kKeys = 64;                                  // keys per block
constexpr int kAttnWaves = 8;
constexpr uint32_t kKVTile = kKeys * kRowBytes;            // 16 KiB
constexpr uint32_t kKVSlot = 2 * kKVTile;                  // K | V
constexpr int kKVSlots = 4;
constexpr int kRing = 4;                                   // 8-wave form: K ring, V ring
static_assert(2 * kRing * kKVTile == kKVSlots * kKVSlot, "both forms use 128 KiB of LDS");
constexpr float kLazy = 8.f;                               // shift slack of the online softmax
constexpr int kStoresO = 8;                                // O stores per wave and tile (8-wave form)
constexpr int kStoresL = 2;                                // lse stores per wave and tile

struct AttnParams {
    const char *Q, *K, *V;
    char *O;
    float *lse;
    int Sq, Sk;
    int nq;        // query blocks per (batch, head)
    int groups;    // batch * heads
    float c;       // scale * log2(e)
    int off;       // Sk - Sq (causal masks aligned at the bottom right)
    uint32_t stagger_seed;   // race-stress pauses (read only by the race-stress build)
};

// Workgroup -> (batch*head, query block): each XCD takes a contiguous range,
// so the query blocks of one head share that XCD's L2 copy of K and V.  With
// causal masks query block qb sees qb + 1 blocks of keys, so the order matters
// for the tail: the range is taken in pairs of heads, and within a pair the
// blocks go heaviest first, alternating the two heads (15 of head 2c, 15 of
// head 2c+1, 14, 14, ...).  That is longest-first dispatch within 2 nq
// workgroups, which keeps the two heads' K and V in L2 together; dispatching
// one head after the other, heaviest first, leaves the last CUs of an XCD
// about 10 % more work than the mean (list scheduling over 16 heads of 16
// blocks on 32 CUs: 75 units against 68).  A last unpaired head keeps its
// heaviest-first order, and so does every head when an XCD's range holds
// fewer than two heads (pairs would then put the heavy halves of two heads on
// one XCD and the light halves on the next).  Each (batch*head, query block)
// is produced once.
template <bool kCausal>
__device__ __forceinline__ void attn_item(const AttnParams &p, int v, int &bh, int &qb) {
    const int q = (p.nq * p.groups) >> 3;
    if constexpr (kCausal) {
        const int pair = v / (2 * p.nq), t = v - pair * 2 * p.nq;
        if (q >= 2 * p.nq && 2 * pair + 1 < p.groups) {
            bh = 2 * pair + (t & 1);
            qb = p.nq - 1 - (t >> 1);
        } else {
            bh = v / p.nq;
            qb = p.nq - 1 - (v - bh * p.nq);
        }
    } else {
        bh = v / p.nq;
        qb = v - bh * p.nq;
    }
}

template <bool kCausal>
__device__ __forceinline__ void attn_coords(const AttnParams &p, int wg, int &bh, int &qb) {
    const int total = p.nq * p.groups;
    const int xcd = wg & 7, j = wg >> 3;
    const int q = total >> 3, r = total & 7;
    attn_item<kCausal>(p, xcd * q + min(xcd, r) + j, bh, qb);
}

// Tile k of a workgroup of the persistent 8-wave kernel, whose grid holds
// 8 * per workgroups, one per CU: workgroup w stays on XCD w mod 8 and takes
// position L = w / 8 of every round of per tiles in that XCD's range, the
// rounds alternating in direction (L, then per - 1 - L, ...).  With the
// heaviest-first causal order that gives every workgroup the same work
// (a heavy and a light tile per pair of rounds).  Returns false past the end
// of the range; bh, qb and the tile's number of key blocks otherwise.
template <bool kCausal>
__device__ __forceinline__ bool attn_tile(const AttnParams &p, int k, int &bh, int &qb, int &nblk) {
    const int per = static_cast<int>(gridDim.x >> 3), xcd = blockIdx.x & 7, L = blockIdx.x >> 3;
    const int total = p.nq * p.groups, q = total >> 3, r = total & 7;
    const int j = k * per + ((k & 1) ? per - 1 - L : L);
    if (j >= q + (xcd < r ? 1 : 0)) return false;
    attn_item<kCausal>(p, xcd * q + min(xcd, r) + j, bh, qb);
    // key blocks: every key, or (causal) those the tile's last row sees
    int kend = p.Sk;
    if constexpr (kCausal) kend = max(0, min(p.Sk, min(p.Sq, qb * kQRows + kQRows) + p.off));
    nblk = (kend + kKeys - 1) / kKeys;
    return true;
}

// Combine the values of lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes
// that hold one row of an MFMA accumulator tile) with VALU lane swaps: each
// swap exchanges 16-lane (32-lane) halves between two copies of x, and the
// pairwise result is the same in every lane of a pair.
template <typename F>
__device__ __forceinline__ float row_reduce(float x, F op) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// This lane's index in its wave, computed afresh from the execution mask
// (through an opaque all-ones value): code after it in a loop cannot use a
// copy kept in a register since the loop began.
__device__ __forceinline__ int fresh_lane() {
    uint32_t ones = ~0u;
    asm volatile("" : "+s"(ones));
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(ones, __builtin_amdgcn_mbcnt_lo(ones, 0u)));
}

template <int kElem>
__device__ __forceinline__ i32x2 pack4(f32x4 v) {
    if constexpr (kElem == kElemBF16)
        return __builtin_bit_cast(i32x2, __builtin_convertvector(v, bf16x4));
    else
        return __builtin_bit_cast(i32x2, __builtin_convertvector(v, f16x4));
}

// Two neighbouring 16x16 accumulator tiles of one row, rounded to the operand
// type and traded between lanes l and l ^ 16 (two v_permlane16_swap) so that
// every lane holds 8 consecutive columns: columns 16 + 4 (g - 1) .. of the
// pair for an odd lane group g, 4 g .. for an even one (the same trade as the
// GEMM epilogue's).
template <int kElem>
__device__ __forceinline__ i32x4 pack_pair(f32x4 a, f32x4 b) {
    const i32x2 h0 = pack4<kElem>(a), h1 = pack4<kElem>(b);
    const auto sx = __builtin_amdgcn_permlane16_swap(h0.x, h1.x, false, false);
    const auto sy = __builtin_amdgcn_permlane16_swap(h0.y, h1.y, false, false);
    return i32x4{static_cast<int>(sx[0]), static_cast<int>(sy[0]), static_cast<int>(sx[1]),
                 static_cast<int>(sy[1])};
}


// kOffset = false keeps the two groups in phase (no entry / exit barrier):
// the same stages and arithmetic, the ablation of the offset.
template <int kElem, bool kCausal, bool kOffset>
__global__ void __launch_bounds__(kAttnWaves * 64) attention_fwd_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[kKVSlots * kKVSlot];
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const bool groupB = wave >= kAttnWaves / 2;
    const uint32_t lds0 = lds_address(smem);
    stagger_poison_lds<kKVSlots * kKVSlot, kAttnWaves * 64>(lds0);
    Stagger sg(p.stagger_seed);

    // Q fragments (MFMA row operand) of query tile (bh, qb): rows
    // 256 qb + 32 wave + 16 mt + r16, d 32 dc + 8 g ..; rows past the end
    // read the last row (and are zeroed where used)
    // (the lane index is taken afresh, so that no address part of it stays
    // in registers across the tiles)
    auto load_q = [&](int bh_, int qb_, i32x4 (&qr)[2][4]) {
        const int t = fresh_lane();
        const int64_t base = static_cast<int64_t>(bh_) * p.Sq * kRowBytes;
        for (int mt = 0; mt < 2; ++mt) {
            const int row = qb_ * kQRows + 32 * wave + 16 * mt + (t & 15);
            const char *src = p.Q + base + static_cast<int64_t>(min(row, p.Sq - 1)) * kRowBytes + 16 * ((t >> 4) & 3);
            for (int dc = 0; dc < 4; ++dc) qr[mt][dc] = *reinterpret_cast<const i32x4 *>(src + 64 * dc);
        }
    };
    int bh, qb, nblk;
    if (!attn_tile<kCausal>(p, 0, bh, qb, nblk)) return;
    // Q of the tile: loaded ahead (for the next tile, during this tile's last
    // trip), rows past the end zeroed in the prologue
    i32x4 qf[2][4];
    load_q(bh, qb, qf);
    // A previous tile's stores, with empty windows (nothing is written):
    // every path into a tile then has the same stores issued after its Q
    // loads, so the wait the compiler places before Q is used lets the
    // previous tile's stores fly on every tile
    {
        const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(p.O, 0, 0, 0x00020000);
        for (int n = 0; n < kStoresO; ++n)          // (distinct offsets: none of them is merged away)
            __builtin_amdgcn_raw_buffer_store_b128(i32x4{0, 0, 0, 0}, none, 16 * n, 0, 0);
        if (p.lse)
            for (int n = 0; n < kStoresL; ++n) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 4 * n, 0, 0);
    }
    // g0: ring position of the tile's block 0 (block j of the tile sits in
    // slot (g0 + j) mod 4 of each ring); pre: the previous tile already
    // copied this tile's K blocks 0-3 and V blocks 0-1 and loaded its Q;
    // settle: the previous tile's copies past its end (zero windows) may
    // still be landing in this tile's slots
    int g0 = 0;
    bool pre = false, settle = false;
#pragma unroll 1
    for (int k = 0;; ++k) {
        int bhn = bh, qbn = qb, nbn = 0;
        const bool more = attn_tile<kCausal>(p, k + 1, bhn, qbn, nbn);
        if (!more) {        // the last tile reloads its own Q below (in bounds, unused)
            bhn = bh;
            qbn = qb;
            nbn = 0;
        }
        // copies past this tile's last block fetch the next tile's first blocks
        // (K 0-3 and V 0-1, the last two from the tile's last trip).  Only
        // when all of them are the next tile's own: with fewer than 4 blocks
        // its K 3 would be a block of the tile after it, which this tile does
        // not fetch.
        const bool pf = more && nblk >= 2 && nbn >= 4;
        // The lane index and the sequence lengths are opaque per tile: what
        // derives from them is computed in the tile, not kept in registers
        // across all of the workgroup's tiles
        const int lane = fresh_lane();
        int Sk = p.Sk, Sq = p.Sq, off = p.off;
        asm volatile("" : "+s"(Sk), "+s"(Sq), "+s"(off));
        const int g = lane >> 4, r16 = lane & 15;
        const int q0 = qb * kQRows;
        const int wrow = q0 + 32 * wave;                           // this wave's first query row
        const int64_t qbase = static_cast<int64_t>(bh) * Sq * kRowBytes;
        const int64_t kbase = static_cast<int64_t>(bh) * Sk * kRowBytes;

        const int64_t kbase_n = static_cast<int64_t>(bhn) * Sk * kRowBytes;

        f32x4 o[2][2][4];                                          // [mt][d half][16-column tile]
        for (int mt = 0; mt < 2; ++mt)
            for (int h = 0; h < 2; ++h)
                for (int t = 0; t < 4; ++t) o[mt][h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f}, alpha[2] = {1.f, 1.f};

        if (nblk > 0) {
            // two rings of kRing 16-KiB slots: K blocks, then V blocks
            auto slot_of = [&](int j) { return static_cast<uint32_t>((g0 + j) & (kRing - 1)); };
            auto k_slot = [&](int j) { return lds0 + slot_of(j) * kKVTile; };
            auto v_slot = [&](int j) { return lds0 + (kRing + slot_of(j)) * kKVTile; };
            // copy lanes: wave w moves pieces 2w, 2w+1 (4 rows x 256 bytes each)
            // of the K and of the V block; lane (x, pch) fills physical chunk pch
            // of row x of a piece
            uint32_t cpK[2], cpV[2];
            {
                const int x = lane >> 4, pch = lane & 15;
                for (int i = 0; i < 2; ++i) {
                    const int row = 4 * (2 * wave + i) + x;
                    cpK[i] = static_cast<uint32_t>(row * kRowBytes + (pch ^ (row & 15)) * 16);
                    cpV[i] = static_cast<uint32_t>(row * kRowBytes + (pch ^ (2 * (row & 7))) * 16);
                }
            }
            // Window of block j: whole for the blocks of 64 existing keys, the
            // tail's rows for a partial last block, empty past the last block the
            // workgroup needs.  Compares and selects of uniform values only, so
            // the descriptor stays on the scalar unit.
            const int nfull = Sk / kKeys;
            const uint32_t tail_rec = static_cast<uint32_t>(Sk - nfull * kKeys) * kRowBytes;
            // Source offset and window of block j of this tile; with pf, blocks
            // past the last are the next tile's blocks j - nblk (at most its
            // fourth, which it has).  Selects of uniform values only: branches
            // here would sit in every trip.
            const int64_t xbase = pf ? kbase_n - static_cast<int64_t>(nblk) * kKVTile : kbase;
            auto source = [&](int j, int64_t &at, uint32_t &nrec, auto tail) {
                if constexpr (!decltype(tail)::value) {     // block j is the tile's own
                    at = kbase + static_cast<int64_t>(j) * kKVTile;
                    nrec = j < nfull ? kKVTile : tail_rec;
                    return;
                }
                const bool own = j < nblk;
                at = (own ? kbase : xbase) + static_cast<int64_t>(j) * kKVTile;
                const int t = own ? j : j - nblk;
                const uint32_t w = t < nfull ? kKVTile : tail_rec;
                nrec = (own || (pf && t < nbn)) ? w : 0u;
            };
            // The descriptors and LDS destinations of the copies of K block jk and
            // V block jv, and this wave's four pieces of them (K pieces 0, 1, then
            // V pieces 0, 1).
            struct CopySet { i32x4 rk, rv; uint32_t dk, dv; };
            auto copy_set = [&](int jk, int jv, auto tail) {
                int64_t ak, av;
                uint32_t nk, nv;
                source(jk, ak, nk, tail);
                source(jv, av, nv, tail);
                return CopySet{make_rsrc(p.K + ak, nk), make_rsrc(p.V + av, nv),
                               k_slot(jk) + 2 * wave * 1024, v_slot(jv) + 2 * wave * 1024};
            };
            auto copy_piece = [&](const CopySet &cs, int q) {
                if (q == 0) copy16<0>(cs.rk, cs.dk, cpK[0]);
                else if (q == 1) copy16<1024>(cs.rk, cs.dk, cpK[1]);
                else if (q == 2) copy16<0>(cs.rv, cs.dv, cpV[0]);
                else copy16<1024>(cs.rv, cs.dv, cpV[1]);
            };
            auto copy_k = [&](int j) {
                const CopySet cs = copy_set(j, j, std::true_type{});
                copy_piece(cs, 0);
                copy_piece(cs, 1);
            };
            auto copy_v = [&](int j) {
                const CopySet cs = copy_set(j, j, std::true_type{});
                copy_piece(cs, 2);
                copy_piece(cs, 3);
            };

            // fragment read offsets within a slot
            uint32_t kofs[4], vofs[4 * 2];
            for (int dc = 0; dc < 4; ++dc)
                kofs[dc] = static_cast<uint32_t>(r16 * kRowBytes + (((4 * dc + g) ^ r16) * 16));
            {
                const int rr = 4 * (g & 1) + (r16 >> 2);               // (k-row) & 7 of this lane's reads
                const int base = (4 * g + (r16 >> 2)) * kRowBytes + 16 * ((r16 & 3) >> 1) + 8 * (r16 & 1);
                for (int dt = 0; dt < 8; ++dt) vofs[dt] = static_cast<uint32_t>(base + 32 * (dt ^ rr));
            }

            i32x4 kf[4][4];     // K block fragments [16-key tile][32-d chunk]
            i32x4 vf[8][2];     // V block fragments [16-d tile][32-key chunk]
            i32x4 pf[2][2];     // P [mt][32-key chunk], operand type
            f32x4 s[2][4];      // S [mt][16-key tile]

            // One address add per lane base (kept opaque to the compiler); the
            // rest of every read's address is its immediate offset.
            // K fragments of d-chunks dc0 .. dc1-1, V fragments of key chunks c0 .. c1-1
            auto read_k = [&](int j, int dc0, int dc1) {
                const uint32_t b = k_slot(j);
                for (int dc = dc0; dc < dc1; ++dc) {
                    uint32_t a = b + kofs[dc];
                    asm volatile("" : "+v"(a));
                    for (int kt = 0; kt < 4; ++kt) kf[kt][dc] = lds_read128(a + kt * 16 * kRowBytes);
                }
            };
            // V bases of block j, once for both halves of its reads (computing
            // them per half had the compiler share the adds and copy them into
            // each half's opaque register)
            auto v_bases = [&](int j, uint32_t (&vb)[8]) {
                const uint32_t b = v_slot(j);
                for (int dt = 0; dt < 8; ++dt) {
                    vb[dt] = b + vofs[dt];
                    asm volatile("" : "+v"(vb[dt]));
                }
            };
            uint32_t vb[8];                                     // V bases of the block being read
            // one transposing read: half u & 1 of the V fragment [u >> 1][c]
            auto read_v_piece = [&](int c, int u) {
                const int dt = u >> 1;
                const i32x2 x = lds_read64_tr(vb[dt] + (32 * c + 16 * (u & 1)) * kRowBytes);
                if (u & 1) {
                    vf[dt][c].z = x.x;
                    vf[dt][c].w = x.y;
                } else {
                    vf[dt][c].x = x.x;
                    vf[dt][c].y = x.y;
                }
            };
            auto read_v = [&](const uint32_t (&vb)[8], int c0, int c1) {
                for (int dt = 0; dt < 8; ++dt)
                    for (int c = c0; c < c1; ++c) {
                        const i32x2 lo = lds_read64_tr(vb[dt] + (32 * c) * kRowBytes);
                        const i32x2 hi = lds_read64_tr(vb[dt] + (32 * c + 16) * kRowBytes);
                        vf[dt][c] = i32x4{lo.x, lo.y, hi.x, hi.y};
                    }
            };
            // The score products.  With `inter`, every fourth MFMA of the first
            // half is followed by one of this wave's copies of later blocks
            // (`copies(q)`, q = 0 .. 3) and each MFMA of the second half by one
            // transposing read of the first half of the V fragments, into the
            // registers of the K fragments already used (a block of 16 reads
            // would hold this wave's MFMAs back while it issues them).
            auto qk = [&](auto inter, auto copies) {
                constexpr bool kInter = decltype(inter)::value;
                for (int dc = 0; dc < 4; ++dc) {
                    if (dc == 2) __builtin_amdgcn_sched_barrier(0);
                    for (int mt = 0; mt < 2; ++mt)
                        for (int kt = 0; kt < 4; ++kt) {
                            s[mt][kt] = mfma<kElem>(kf[kt][dc], qf[mt][dc],
                                                    dc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[mt][kt]);
                            if constexpr (kInter) {
                                const int n = 8 * dc + 4 * mt + kt;
                                if (n < 16 && (n & 3) == 3) {            // copy piece n / 4 after MFMAs 3, 7, 11, 15
                                    copies(n >> 2);
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                            }
                            if constexpr (kInter) {
                                if (dc >= 2) {
                                    const int u = 8 * (dc - 2) + 4 * mt + kt;     // 0 .. 15
                                    read_v_piece(0, u);
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                            }
                        }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            // The P V stage.  With `inter` (the block index of the K fragments to
            // read), each MFMA of the first half is followed by one transposing
            // read of the second half of the V fragments (the registers of the K
            // fragments the score stage used up) and each MFMA of the second half
            // by one read of the next K fragments (16 b128 reads: d-chunks 0 and 1
            // into the registers of the V fragments of the first half, 2 and 3
            // into those of the second half as its MFMAs use them).
            auto pv = [&](auto inter, int jk) {
                constexpr bool kInter = decltype(inter)::value;
                uint32_t kb[4];
                if constexpr (kInter) {
                    const uint32_t b = k_slot(jk);
                    for (int dc = 0; dc < 4; ++dc) {
                        kb[dc] = b + kofs[dc];
                        asm volatile("" : "+v"(kb[dc]));
                    }
                }
                for (int c = 0; c < 2; ++c) {
                    if (c == 1) __builtin_amdgcn_sched_barrier(0);
                    for (int mt = 0; mt < 2; ++mt)
                        for (int dt = 0; dt < 8; ++dt) {
                            o[mt][dt >> 2][dt & 3] = mfma<kElem>(vf[dt][c], pf[mt][c], o[mt][dt >> 2][dt & 3]);
                            if constexpr (kInter) {
                                const int n = 8 * mt + dt;                          // 0 .. 15
                                if (c == 0) read_v_piece(1, n);
                                else kf[n & 3][n >> 2] = lds_read128(kb[n >> 2] + (n & 3) * 16 * kRowBytes);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            // keys past the end, and (causal) keys above the diagonal, score -inf
            auto mask = [&](int j) {
                const int k0 = j * kKeys;
                bool need = k0 + kKeys > Sk;
                if constexpr (kCausal) need = need || (k0 + kKeys - 1 > wrow + off);
                if (need) {
                    const int ln = fresh_lane();                      // (no lane value kept since the tile began)
                    for (int mt = 0; mt < 2; ++mt) {
                        const int lim = kCausal ? min(Sk, wrow + 16 * mt + (ln & 15) + off + 1) : Sk;
                        const int t = lim - k0 - 4 * (ln >> 4);       // first masked 16kt + e of this lane
                        for (int kt = 0; kt < 4; ++kt)
                            for (int e = 0; e < 4; ++e)
                                if (16 * kt + e >= t) s[mt][kt][e] = -INFINITY;
                    }
                }
            };
            // The two softmax halves are pure arithmetic, which the compiler would
            // otherwise move across the stage walls; each half starts from values
            // passed through an empty asm, so its work stays in its stage.
            auto pin_s = [&]() {
                for (int mt = 0; mt < 2; ++mt)
                    for (int kt = 0; kt < 4; ++kt) asm volatile("" : "+v"(s[mt][kt]));
            };
            // first half: row maxima of S and the running shift m.  m moves only
            // when a row's maximum exceeds it by more than kLazy (log2 units): the
            // exponentials then stay below 2^kLazy, and O and l are rescaled by
            // alpha = 2^(m_old - m_new) only in those rows (lazy rescaling).  Each
            // lane first compares the maximum of its own 16 scores of the row (times
            // c) with m + kLazy; only when some lane of the wave exceeds it does the
            // wave combine the four lanes of each row (c > 0 and rounding is
            // monotonic, so the largest lane product is the row maximum times c:
            // the decision is the same as from the row maximum itself).
            auto softmax_max = [&]() {
                pin_s();
                float lm[2];
                bool up = false;
                for (int mt = 0; mt < 2; ++mt) {
                    // a tree of three-input maxima (depth 3, not a chain of 15)
                    const f32x4 *x = s[mt];
                    const float t0 = fmaxf(fmaxf(x[0][0], x[0][1]), x[0][2]);
                    const float t1 = fmaxf(fmaxf(x[0][3], x[1][0]), x[1][1]);
                    const float t2 = fmaxf(fmaxf(x[1][2], x[1][3]), x[2][0]);
                    const float t3 = fmaxf(fmaxf(x[2][1], x[2][2]), x[2][3]);
                    const float t4 = fmaxf(fmaxf(x[3][0], x[3][1]), x[3][2]);
                    lm[mt] = fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(fmaxf(t3, t4), x[3][3])) * p.c;
                    up = up || lm[mt] > m[mt] + kLazy;
                }
                alpha[0] = alpha[1] = 1.f;
                if (__builtin_amdgcn_ballot_w64(up) != 0) {
                    for (int mt = 0; mt < 2; ++mt) {
                        const float mx = row_reduce(lm[mt], [](float a, float b) { return fmaxf(a, b); });
                        if (mx > m[mt] + kLazy) {
                            alpha[mt] = __builtin_amdgcn_exp2f(m[mt] - mx);
                            m[mt] = mx;
                        }
                    }
                }
                asm volatile("" : "+v"(m[0]), "+v"(m[1]), "+v"(alpha[0]), "+v"(alpha[1]));
            };
            // second half: P = 2^(c S - m) in the operand type, running row sums
            auto softmax_exp = [&]() {
                pin_s();
                for (int mt = 0; mt < 2; ++mt) {
                    const float ref = m[mt] == -INFINITY ? 0.f : m[mt];
                    float part[4];                          // per 16-key tile, then a tree
                    for (int c = 0; c < 2; ++c) {
                        i32x2 h[2];
                        for (int u = 0; u < 2; ++u) {
                            f32x4 pr;
                            for (int e = 0; e < 4; ++e)
                                pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][2 * c + u][e], p.c, -ref));
                            part[2 * c + u] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                            h[u] = pack4<kElem>(pr);
                        }
                        pf[mt][c] = i32x4{h[0].x, h[0].y, h[1].x, h[1].y};
                    }
                    l[mt] = l[mt] * alpha[mt] + ((part[0] + part[1]) + (part[2] + part[3]));
                }
            };
            // O *= alpha, skipped when no row of the wave changed its max
            auto rescale = [&]() {
                if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.f || alpha[1] != 1.f) == 0) return;
                for (int mt = 0; mt < 2; ++mt)
                    for (int h = 0; h < 2; ++h)
                        for (int t = 0; t < 4; ++t) o[mt][h][t] *= alpha[mt];
            };

            // ---- prologue (both groups in step): K blocks 0-3 and V blocks 0-1 in
            // flight (or, after a tile that fetched them and this tile's Q, only
            // the previous tile's stores), S(0), P(0)
            auto wait_pre = [&] {
                if (p.lse)
                    wait_vmcnt<kStoresO + kStoresL>();
                else
                    wait_vmcnt<kStoresO>();
            };
            if (settle) wait_vmcnt<0>();
            if (!pre) {
                copy_k(0);
                copy_k(1);
                copy_v(0);
                copy_k(2);
                copy_v(1);
                copy_k(3);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (pre)
                wait_pre();                     // everything but the previous tile's stores
            else
                wait_vmcnt<10>();               // K(0) (this wave's pieces) and Q
            for (int mt = 0; mt < 2; ++mt) {
                const bool in = wrow + 16 * mt + r16 < Sq;
                for (int dc = 0; dc < 4; ++dc) qf[mt][dc] = in ? qf[mt][dc] : i32x4{0, 0, 0, 0};
            }
            rendezvous(sg);                     // ... and everyone's
            read_k(0, 0, 4);
            wait_lgkmcnt<0>();
            qk(std::false_type{}, [](int) {});
            mask(0);
            softmax_max();
            rescale();
            softmax_exp();
            __builtin_amdgcn_sched_barrier(0);
            if (pre)
                wait_pre();
            else
                wait_vmcnt<4>();                // K(1), V(0), K(2)
            rendezvous(sg);
            read_k(1, 0, 4);
            wait_lgkmcnt<0>();
            if (kOffset && groupB) rendezvous(sg);  // group B falls one stage behind

            // one trip; kMasked: block i+1 may hold keys some row must not see
            // tail: copies may reach past the tile's last block; last: the tile's
            // last trip, whose softmax stage also loads the next tile's Q into
            // the registers of this tile's (free once its last scores are made)
            auto trip = [&](int i, auto masked, auto tail, auto last) {
                // MFMA stage: S(i+1) and O += P(i) V(i), the V(i) and K(i+2)
                // fragments read among them; the copies of K(i+4) and V(i+2) go
                // out in the first quarter; wait for the previous trip's copies
                v_bases(i, vb);
                // (the descriptors are made after the first MFMAs, not ahead of them)
                CopySet cs;
                qk(std::true_type{}, [&](int q) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (q == 0) cs = copy_set(i + 4, i + 2, tail);
                    copy_piece(cs, q);
                });
                pv(std::true_type{}, i + 2);
                wait_vmcnt<4>();                // K(i+3), V(i+1) (only this trip's four copies may fly)
                rendezvous(sg);
                // softmax stage: row max of S(i+1): m(i+1), alpha(i+1); O and l
                // rescaled; P(i+1)
                if constexpr (decltype(last)::value) {
                    if (pf) {                   // the next tile's V(1) and K(3)
                        copy_v(nblk + 1);
                        copy_k(nblk + 3);
                    }
                    load_q(bhn, qbn, qf);
                }
                if constexpr (decltype(masked)::value) mask(i + 1);
                softmax_max();
                rescale();
                softmax_exp();
                wait_lgkmcnt<0>();              // this wave's reads of the MFMA stage
                rendezvous(sg);
            };
            // leading blocks no row of the workgroup needs masked: every key
            // exists and (causal) every key is visible to the first row
            int nplain = Sk / kKeys;
            if constexpr (kCausal) nplain = min(nplain, max(0, (q0 + off + 1) / kKeys));
            // Trips: unmasked ones whose copies stay in the tile, then the rest
            // (masked where a row needs it), then the last
            using F = std::false_type;
            using T = std::true_type;
            int i = 0;
#pragma unroll 1
            for (; i + 4 < nblk && i + 1 < nplain; ++i) trip(i, F{}, F{}, F{});
#pragma unroll 1
            for (; i + 2 < nblk; ++i) trip(i, T{}, T{}, F{});
            if (i + 1 < nblk) trip(i, T{}, T{}, T{});
            // ---- drain: P V of the last block (and the next tile's Q after a
            // tile of one block, which has no trip)
            v_bases(nblk - 1, vb);
            read_v(vb, 0, 2);
            wait_lgkmcnt<0>();
            pv(std::false_type{}, 0);
            if (nblk < 2) load_q(bhn, qbn, qf);
            if (kOffset && !groupB) rendezvous(sg); // group A closes the offset
            __builtin_amdgcn_sched_barrier(0);
        } else {
            load_q(bhn, qbn, qf);
        }

        // ---- O / l and lse, by buffer stores whose window ends at the head's last
        // row: every wave issues the same stores (kStoresO, and kStoresL with an
        // lse buffer), rows past the end are dropped by the window
        {
            const int ln = fresh_lane(), gl = ln >> 4;
            const __amdgpu_buffer_rsrc_t ro =
                __builtin_amdgcn_make_buffer_rsrc(p.O + qbase, 0, Sq * kRowBytes, 0x00020000);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const float lt = row_reduce(l[mt], [](float a, float b) { return a + b; });
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                for (int h = 0; h < 2; ++h)
                    for (int t = 0; t < 4; ++t) o[mt][h][t] *= inv;
                const int row = wrow + 16 * mt + (ln & 15);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    for (int nt = 0; nt < 4; nt += 2) {
                        const i32x4 v = pack_pair<kElem>(o[mt][h][nt], o[mt][h][nt + 1]);
                        const int col = 64 * h + 16 * nt + ((gl & 1) ? 16 + 4 * (gl - 1) : 4 * gl);
                        __builtin_amdgcn_raw_buffer_store_b128(v, ro, row * kRowBytes + 2 * col, 0, 0);
                    }
                if (p.lse) {
                    const __amdgpu_buffer_rsrc_t rl =
                        __builtin_amdgcn_make_buffer_rsrc(p.lse + static_cast<int64_t>(bh) * Sq, 0, Sq * 4, 0x00020000);
                    const float v = lt > 0.f ? (m[mt] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f : -INFINITY;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rl, gl == 0 ? 4 * row : 0x7FFFFFF0, 0, 0);
                }
            }
        }
        if (!more) break;
        settle = nblk > 0 && !pf;
        g0 = (g0 + nblk) & (kRing - 1);  // only the ring position matters
        pre = pf;
        bh = bhn;
        qb = qbn;
        nblk = nbn;
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();                        // copies past the last tile's end
}

// ---- the 4-wave form: one wave per SIMD, each interleaving its own matrix
// work with its own softmax ------------------------------------------------
//
// Every wave of the 8-wave form reads the whole 64-key K and V block for its
// 32 query rows: 256 KiB of LDS reads per CU per block, against 2,048 MFMA
// cycles per SIMD.  Here a workgroup of 4 waves (one per SIMD, 512 registers
// each: the O accumulators go to AGPRs) takes the same 256 query rows, 64 per
// wave, so each byte read from LDS feeds twice the MFMAs (128 KiB per block).
// With one wave per SIMD nothing runs beside a wave's softmax, so each wave
// software-pipelines its own loop over key blocks j (the scheme "Two Waves,
// One Stage Apart" compares against, within-wave interleaving):
//   phase A   S(j+1) = Q K(j+1)^T (64 MFMAs, the K fragments streamed from
//             LDS), each group of 4 MFMAs carrying a quarter row-tile of the
//             exponentials of block j: P(j) = 2^(S'(j)) in the operand type,
//             row sums l = alpha(j) l + sums
//   phase B   O *= alpha(j) (only when a row's shift moved); O += P(j) V(j)
//             (64 MFMAs, V fragments streamed), the first half carrying the
//             row maxima of S(j+1) -> m(j+1), alpha(j+1), the second half the
//             scaling S'(j+1) = c S(j+1) - m(j+1)
// and one barrier per block (after the wave's LDS reads and its part of the
// copies of block j+2 completed).  The copies of block j+3 go out during
// phase A into the slot of block j-1, whose last reads (V(j-1), phase B of
// block j-1) every wave finished before that barrier.  Same LDS layout,
// fragment formats, MFMA order per output element and softmax arithmetic as
// the 8-wave form, so the two give the same bits.
constexpr int kW4Waves = 4;

// O += x . y with the accumulator in AGPRs, where the 4-wave form keeps O
// (128 registers per lane) so that its VGPRs hold the scores, P and the
// operands.  The instruction is written out; the compiler does not see it
// as an MFMA and pads no wait states around it, so the form keeps every
// hazard out of reach by construction: x (V fragments, from LDS) and y (P,
// from VALU work at least one phase earlier) are written long before, O is
// read by a VALU only after mfma_drain and written back (rescale) at least
// two wait states before the next product, and an accumulator's two
// products of a block are 32 MFMAs apart.
template <int kElem>
__device__ __forceinline__ void mfma_agpr(f32x4 &acc, i32x4 x, i32x4 y) {
    if constexpr (kElem == kElemBF16)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
    else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
}

// S = x . y (+ S) with the scores in VGPRs (the softmax reads them) and the
// row operand y (the Q fragments) in AGPRs, so that the 4-wave form's Q
// (64 registers per lane) and O both live in AGPRs and its VGPRs hold the
// scores, P and the streamed operands.  Written out like mfma_agpr, with
// the same care for what the compiler cannot see: the K fragments come from
// LDS (the compiler waits for them), Q is moved into its AGPRs right after
// its load and followed by s_nop before any product reads it, an
// accumulator's products are 4 MFMAs apart (the hardware interlocks that),
// and the softmax reads S only after at least 11 more instructions or an
// explicit mfma_drain.  kFirst starts from zero (its result early-clobber:
// it is a new value).
template <int kElem, bool kFirst>
__device__ __forceinline__ void mfma_qk(f32x4 &acc, i32x4 x, i32x4 y) {
    if constexpr (kFirst) {
        if constexpr (kElem == kElemBF16)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(x), "a"(y));
        else
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(x), "a"(y));
    } else {
        if constexpr (kElem == kElemBF16)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(x), "a"(y));
        else
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(x), "a"(y));
    }
}

// Wait states between an MFMA of mfma_agpr / mfma_qk writing its result and
// a VALU (or v_accvgpr_read) reading it: more than the 18 a 16x16x32 MFMA
// (8 passes) may need.  The scheduling
// walls keep the compiler, which sees no dependence on the nops, from
// moving the reads above them.
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int kElem, bool kCausal>
__global__ void __launch_bounds__(kW4Waves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
attention_fwd4_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[kKVSlots * kKVSlot];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r16 = lane & 15;

    int bh, qb;
    attn_coords<kCausal>(p, blockIdx.x, bh, qb);
    const int q0 = qb * kQRows;
    const int wrow = q0 + 64 * wave;                           // this wave's first query row
    const int64_t qbase = static_cast<int64_t>(bh) * p.Sq * kRowBytes;
    const int64_t kbase = static_cast<int64_t>(bh) * p.Sk * kRowBytes;

    int kend = p.Sk;
    if constexpr (kCausal) kend = max(0, min(p.Sk, min(p.Sq, q0 + kQRows) + p.off));
    const int nblk = (kend + kKeys - 1) / kKeys;

    // Q fragments (MFMA row operand): rows wrow + 16rt + r16, d 32dc + 8g ..
    i32x4 qf[4][4];
    for (int rt = 0; rt < 4; ++rt) {
        const int row = wrow + 16 * rt + r16;
        const char *src = p.Q + qbase + static_cast<int64_t>(min(row, p.Sq - 1)) * kRowBytes + 16 * g;
        for (int dc = 0; dc < 4; ++dc) {
            const i32x4 v = *reinterpret_cast<const i32x4 *>(src + 64 * dc);
            qf[rt][dc] = row < p.Sq ? v : i32x4{0, 0, 0, 0};
        }
    }
    // Q moves to its AGPRs here, well before the first score MFMA: the
    // compiler does not pad a VALU write followed by an asm MFMA reading it
    for (int rt = 0; rt < 4; ++rt)
        for (int dc = 0; dc < 4; ++dc) asm volatile("" : "+a"(qf[rt][dc]));
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 2");
    __builtin_amdgcn_sched_barrier(0);

    f32x4 o[4][8];                                             // [rt][16-column tile of d]
    for (int rt = 0; rt < 4; ++rt)
        for (int dt = 0; dt < 8; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m[4], l[4], alpha[4];
    for (int rt = 0; rt < 4; ++rt) { m[rt] = -INFINITY; l[rt] = 0.f; alpha[rt] = 1.f; }

    if (nblk > 0) {
        const uint32_t lds0 = lds_address(smem);
        stagger_poison_lds<kKVSlots * kKVSlot, kW4Waves * 64>(lds0);
        Stagger sg(p.stagger_seed);
        // copy lanes: wave w moves pieces 4w .. 4w+3 (4 rows x 256 bytes each)
        // of the K and of the V block
        uint32_t cpK[4], cpV[4];
        {
            const int x = lane >> 4, pch = lane & 15;
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * (4 * wave + i) + x;
                cpK[i] = static_cast<uint32_t>(row * kRowBytes + (pch ^ (row & 15)) * 16);
                cpV[i] = static_cast<uint32_t>(row * kRowBytes + (pch ^ (2 * (row & 7))) * 16);
            }
        }
        const int nfull = p.Sk / kKeys;
        const uint32_t tail_rec = static_cast<uint32_t>(p.Sk - nfull * kKeys) * kRowBytes;
        struct CopySet { i32x4 rk, rv; uint32_t dst; };
        auto copy_set = [&](int j) {
            const uint32_t nrec = j < nfull ? (j < nblk ? kKVTile : 0u) : (j < nblk ? tail_rec : 0u);
            const int64_t at = kbase + static_cast<int64_t>(j) * kKVTile;
            return CopySet{make_rsrc(p.K + at, nrec), make_rsrc(p.V + at, nrec),
                           lds0 + static_cast<uint32_t>(j & (kKVSlots - 1)) * kKVSlot + 4 * wave * 1024};
        };
        // piece q (0..7) of this wave's share: K pieces 0..3, then V pieces 0..3
        auto copy_piece = [&](const CopySet &cs, auto q) {
            constexpr int kq = decltype(q)::value;
            if constexpr (kq < 4) copy16<kq * 1024>(cs.rk, cs.dst, cpK[kq]);
            else copy16<kKVTile + (kq - 4) * 1024>(cs.rv, cs.dst, cpV[kq - 4]);
        };
        auto copy_block = [&](int j) {
            const CopySet cs = copy_set(j);
            static_for<0, 8>([&](auto q) { copy_piece(cs, q); });
        };

        uint32_t kofs[4], vofs[8];
        for (int dc = 0; dc < 4; ++dc)
            kofs[dc] = static_cast<uint32_t>(r16 * kRowBytes + (((4 * dc + g) ^ r16) * 16));
        {
            const int rr = 4 * (g & 1) + (r16 >> 2);
            const int base = (4 * g + (r16 >> 2)) * kRowBytes + 16 * ((r16 & 3) >> 1) + 8 * (r16 & 1);
            for (int dt = 0; dt < 8; ++dt) vofs[dt] = static_cast<uint32_t>(base + 32 * (dt ^ rr));
        }
        // read bases of one block (one address add per lane base, kept opaque
        // to the compiler; the rest of every read's address is an immediate)
        auto k_bases = [&](uint32_t slot, uint32_t (&kb)[4]) {
            for (int dc = 0; dc < 4; ++dc) {
                kb[dc] = slot + kofs[dc];
                asm volatile("" : "+v"(kb[dc]));
            }
        };
        auto v_bases = [&](uint32_t slot, uint32_t (&vb)[8]) {
            for (int dt = 0; dt < 8; ++dt) {
                vb[dt] = slot + kKVTile + vofs[dt];
                asm volatile("" : "+v"(vb[dt]));
            }
        };
        auto k_frag = [&](const uint32_t (&kb)[4], int kt, int dc) { return lds_read128(kb[dc] + kt * 16 * kRowBytes); };
        auto v_frag = [&](const uint32_t (&vb)[8], int dt, int c) {
            const i32x2 lo = lds_read64_tr(vb[dt] + (32 * c) * kRowBytes);
            const i32x2 hi = lds_read64_tr(vb[dt] + (32 * c + 16) * kRowBytes);
            return i32x4{lo.x, lo.y, hi.x, hi.y};
        };
        auto slot_of = [&](int j) { return lds0 + static_cast<uint32_t>(j & (kKVSlots - 1)) * kKVSlot; };

        i32x4 pf[4][2];                                        // P [rt][32-key chunk], operand type
        f32x4 s[4][4];                                         // S of one block [rt][16-key tile]
        // row sums of P per row-tile, in the order ((p0 + p1) + (p2 + p3)) of the
        // four 16-key tiles' parts: p0, then p0 + p1, then p2, then the total
        float psum[4], ppart[4];

        // P and the row sum part of tile (rt, kt) from the scaled scores
        auto exp_tile = [&](int rt, int kt) {
            f32x4 pr;
            for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(s[rt][kt][e]);
            const float part = (pr[0] + pr[1]) + (pr[2] + pr[3]);
            if (kt == 0) psum[rt] = part;
            else if (kt == 1) psum[rt] += part;
            else if (kt == 2) ppart[rt] = part;
            else psum[rt] += ppart[rt] + part;
            const i32x2 h = pack4<kElem>(pr);
            if (kt & 1) {
                pf[rt][kt >> 1].z = h.x;
                pf[rt][kt >> 1].w = h.y;
            } else {
                pf[rt][kt >> 1].x = h.x;
                pf[rt][kt >> 1].y = h.y;
            }
        };
        auto row_sums = [&]() {
            for (int rt = 0; rt < 4; ++rt) l[rt] = l[rt] * alpha[rt] + psum[rt];
        };
        // S(j) = Q K(j)^T into s, K-tile column major.  The first MFMA of
        // column kt overwrites it, so with kExp the previous block's scaled
        // scores are turned into P one column ahead: group (kt, dc) exponentiates
        // tile (dc, kt + 1) (column 0 was done at the end of the previous P V)
        auto phase_a = [&](int j, auto exp_on, auto copy_on, const CopySet &cs) {
            constexpr bool kExp = decltype(exp_on)::value, kCopy = decltype(copy_on)::value;
            uint32_t kb[4];
            k_bases(slot_of(j), kb);
            i32x4 kf[4];
            for (int dc = 0; dc < 4; ++dc) kf[dc] = k_frag(kb, 0, dc);
            static_for<0, 4>([&](auto kt_) {
                constexpr int kt = decltype(kt_)::value;
                static_for<0, 4>([&](auto dc_) {
                    constexpr int dc = decltype(dc_)::value;
                    for (int rt = 0; rt < 4; ++rt) {
                        if constexpr (dc == 0) mfma_qk<kElem, true>(s[rt][kt], kf[dc], qf[rt][dc]);
                        else mfma_qk<kElem, false>(s[rt][kt], kf[dc], qf[rt][dc]);
                    }
                    if constexpr (kt < 3) kf[dc] = k_frag(kb, kt + 1, dc);
                    if constexpr (kCopy && kt * 4 + dc < 8) copy_piece(cs, std::integral_constant<int, kt * 4 + dc>{});
                    if constexpr (kExp && kt < 3) exp_tile(dc, kt + 1);
                    __builtin_amdgcn_sched_barrier(0);
                });
            });
            if constexpr (kExp) row_sums();
        };
        // keys past the end, and (causal) keys above the diagonal, score -inf
        auto mask = [&](int j) {
            const int k0 = j * kKeys;
            bool need = k0 + kKeys > p.Sk;
            if constexpr (kCausal) need = need || (k0 + kKeys - 1 > wrow + p.off);
            if (need) {
                mfma_drain();               // the last score MFMAs of the block
                for (int rt = 0; rt < 4; ++rt) {
                    const int lim = kCausal ? min(p.Sk, wrow + 16 * rt + r16 + p.off + 1) : p.Sk;
                    const int t = lim - k0 - 4 * g;
                    for (int kt = 0; kt < 4; ++kt)
                        for (int e = 0; e < 4; ++e)
                            if (16 * kt + e >= t) s[rt][kt][e] = -INFINITY;
                }
            }
        };
        // lane-local row maxima of row-tile rt (times c) and the lazy test
        auto local_max = [&](int rt) {
            const f32x4 *x = s[rt];
            const float t0 = fmaxf(fmaxf(x[0][0], x[0][1]), x[0][2]);
            const float t1 = fmaxf(fmaxf(x[0][3], x[1][0]), x[1][1]);
            const float t2 = fmaxf(fmaxf(x[1][2], x[1][3]), x[2][0]);
            const float t3 = fmaxf(fmaxf(x[2][1], x[2][2]), x[2][3]);
            const float t4 = fmaxf(fmaxf(x[3][0], x[3][1]), x[3][2]);
            return fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(fmaxf(t3, t4), x[3][3])) * p.c;
        };
        // new shifts from the lane-local maxima (see the 8-wave form)
        auto new_shift = [&](const float (&lm)[4]) {
            bool up = false;
            for (int rt = 0; rt < 4; ++rt) up = up || lm[rt] > m[rt] + kLazy;
            for (int rt = 0; rt < 4; ++rt) alpha[rt] = 1.f;
            if (__builtin_amdgcn_ballot_w64(up) != 0) {
                for (int rt = 0; rt < 4; ++rt) {
                    const float mx = row_reduce(lm[rt], [](float a, float b) { return fmaxf(a, b); });
                    if (mx > m[rt] + kLazy) {
                        alpha[rt] = __builtin_amdgcn_exp2f(m[rt] - mx);
                        m[rt] = mx;
                    }
                }
            }
            for (int rt = 0; rt < 4; ++rt) asm volatile("" : "+v"(m[rt]), "+v"(alpha[rt]));
        };
        auto scale_tile = [&](int rt, int kt) {
            const float ref = m[rt] == -INFINITY ? 0.f : m[rt];
            for (int e = 0; e < 4; ++e) s[rt][kt][e] = __builtin_fmaf(s[rt][kt][e], p.c, -ref);
        };
        // O *= alpha, skipped when no row of the wave changed its shift
        auto rescale = [&]() {
            bool any = false;
            for (int rt = 0; rt < 4; ++rt) any = any || alpha[rt] != 1.f;
            // O is pinned to its AGPRs on both sides of the branch and goes
            // through VGPRs only inside it (a VALU cannot multiply an AGPR):
            // left to itself, the compiler moves all of O out of its AGPRs on
            // every block, whether the branch is taken or not
            for (int rt = 0; rt < 4; ++rt)
                for (int dt = 0; dt < 8; ++dt) asm volatile("" : "+a"(o[rt][dt]));
            if (__builtin_amdgcn_ballot_w64(any) == 0) return;
            mfma_drain();
            for (int rt = 0; rt < 4; ++rt)
                for (int dt = 0; dt < 8; ++dt) {
                    o[rt][dt] *= alpha[rt];
                    asm volatile("" : "+a"(o[rt][dt]));
                }
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_nop 1");        // the last AGPR writes, before an MFMA reads O
            __builtin_amdgcn_sched_barrier(0);
        };
        // O += P(j) V(j).  With kMax the groups also carry the softmax of the
        // next block's scores: lane-local maxima (groups 1, 3, 5, 7), the new
        // shifts (after group 7), the scaling of all 16 tiles (groups 8-15,
        // column 0 first) and column 0's P (groups 12-15, after the first
        // half of P(j) -- chunk 0 -- has been consumed)
        auto phase_b = [&](int j, auto max_on) {
            constexpr bool kMax = decltype(max_on)::value;
            uint32_t vb[8];
            v_bases(slot_of(j), vb);
            i32x4 vf[2];
            vf[0] = v_frag(vb, 0, 0);
            float lm[4];
            static_for<0, 16>([&](auto u_) {
                constexpr int u = decltype(u_)::value, c = u >> 3, dt = u & 7;
                if constexpr (u + 1 < 16) vf[(u + 1) & 1] = v_frag(vb, (u + 1) & 7, (u + 1) >> 3);
                const i32x4 cur = vf[u & 1];
                for (int rt = 0; rt < 4; ++rt) mfma_agpr<kElem>(o[rt][dt], cur, pf[rt][c]);
                if constexpr (kMax) {
                    if constexpr (u < 8 && (u & 1)) lm[u >> 1] = local_max(u >> 1);
                    if constexpr (u == 7) {
                        __builtin_amdgcn_sched_barrier(0);
                        new_shift(lm);
                    }
                    if constexpr (u == 8 || u == 9) {
                        scale_tile(2 * (u - 8), 0);
                        scale_tile(2 * (u - 8) + 1, 0);
                    }
                    if constexpr (u >= 10) {
                        // tiles (rt, kt) with kt >= 1, two per group: index 2(u-10), 2(u-10)+1 of 12
                        constexpr int i0 = 2 * (u - 10), i1 = i0 + 1;
                        scale_tile(i0 / 3, 1 + i0 % 3);
                        scale_tile(i1 / 3, 1 + i1 % 3);
                    }
                    if constexpr (u >= 12) exp_tile(u - 12, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };

        // ---- prologue: blocks 0-2 in flight; S(0) scaled, its column 0 of P
        for (int j = 0; j < 3; ++j) copy_block(j);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<16>();                   // block 0 (this wave's pieces)
        rendezvous(sg);                     // ... and everyone's
        phase_a(0, std::false_type{}, std::false_type{}, copy_set(0));
        mfma_drain();
        mask(0);
        {
            float lm[4];
            for (int rt = 0; rt < 4; ++rt) lm[rt] = local_max(rt);
            new_shift(lm);
            for (int rt = 0; rt < 4; ++rt)
                for (int kt = 0; kt < 4; ++kt) scale_tile(rt, kt);
            for (int rt = 0; rt < 4; ++rt) exp_tile(rt, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<8>();                    // block 1
        wait_lgkmcnt<0>();
        rendezvous(sg);

        // one block: S(j+1) with the rest of P(j), then P(j) V(j) with the
        // softmax of S(j+1)
#pragma unroll 1
        for (int j = 0; j + 1 < nblk; ++j) {
            const CopySet cs = copy_set(j + 3);
            phase_a(j + 1, std::true_type{}, std::true_type{}, cs);
            mask(j + 1);
            rescale();                      // by alpha(j), before phase_b sets alpha(j+1)
            phase_b(j, std::true_type{});
            __builtin_amdgcn_sched_barrier(0);
            wait_lgkmcnt<0>();
            wait_vmcnt<8>();                // block j+2 (only block j+3's eight copies may fly)
            rendezvous(sg);
        }
        // ---- drain: the rest of the last block's P, its P V
        for (int rt = 0; rt < 4; ++rt)
            for (int kt = 1; kt < 4; ++kt) exp_tile(rt, kt);
        row_sums();
        rescale();
        phase_b(nblk - 1, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<0>();                    // zero-window copies past the end
        mfma_drain();                       // the last P V MFMAs, before O is read
    }

    // ---- O / l and lse
    GemmParams out{};
    out.C = p.O + qbase;
    out.ldc = kHeadDim;
    out.N = kHeadDim;
    out.M = p.Sq;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const float lt = row_reduce(l[rt], [](float a, float b) { return a + b; });
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        for (int dt = 0; dt < 8; ++dt) o[rt][dt] *= inv;
        const int row = wrow + 16 * rt + r16;
        if (row >= p.Sq) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4 v4[4] = {o[rt][4 * h], o[rt][4 * h + 1], o[rt][4 * h + 2], o[rt][4 * h + 3]};
            store_strip<kElem == kElemBF16, false>(out, v4, row, 64 * h, lane);
        }
        if (p.lse && g == 0)
            p.lse[static_cast<int64_t>(bh) * p.Sq + row] =
                lt > 0.f ? (m[rt] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f : -INFINITY;
    }
}

int attn_status(hipError_t e) { return e == hipSuccess ? GEMM_OK : GEMM_EHIP; }

// Compute units of the current device, read once per device (every thread
// that races here stores the same value).
int cu_count(int &n) {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_EHIP;
    if (dev >= 0 && dev < 64 && (n = cached[dev].load(std::memory_order_relaxed)) > 0) return GEMM_OK;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return GEMM_EHIP;
    if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return GEMM_OK;
}

}  // namespace
}  // namespace mcs

namespace {

int attention_launch(int dtype, int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                     const void *Q, const void *K, const void *V, void *O, float *lse, float scale, int causal,
                     int schedule, hipStream_t stream) {
    using namespace mcs;
    auto aligned16 = [](const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; };
    if (dtype != GEMM_DTYPE_F16 && dtype != GEMM_DTYPE_BF16) return GEMM_EINVAL;
    if (causal != 0 && causal != 1) return GEMM_EINVAL;
    if (schedule != GEMM_SCHED_AUTO && schedule != GEMM_SCHED_PIPELINED && schedule != GEMM_SCHED_IN_PHASE &&
        schedule != GEMM_SCHED_INTERLEAVED)
        return GEMM_EINVAL;
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0 || head_dim < 0) return GEMM_EINVAL;
    if (!(scale > 0.f) || !std::isfinite(scale)) return GEMM_EINVAL;
    if (head_dim != kHeadDim) return GEMM_EUNSUPPORTED;
    if (batch == 0 || heads == 0 || seq_q == 0) return GEMM_OK;
    if (!Q || !O || (seq_k > 0 && (!K || !V))) return GEMM_EINVAL;
    if (!aligned16(Q) || !aligned16(O)) return GEMM_EALIGN;
    if (seq_k > 0 && (!aligned16(K) || !aligned16(V))) return GEMM_EALIGN;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return GEMM_EALIGN;
    // row indices and per-head element offsets stay below 2^31
    if (seq_q >= (int64_t(1) << 23) || seq_k >= (int64_t(1) << 23)) return GEMM_EUNSUPPORTED;
    if (batch > 0x7FFFFFFF || heads > 0x7FFFFFFF) return GEMM_EUNSUPPORTED;   // batch * heads fits int64_t
    const int64_t groups = batch * heads;
    const int64_t nq = (seq_q + kQRows - 1) / kQRows;
    if (groups > 0x7FFFFFFF || nq * groups > 0x7FFFFFFF) return GEMM_EUNSUPPORTED;

    AttnParams prm{};
    prm.Q = static_cast<const char *>(Q);
    prm.K = static_cast<const char *>(K);
    prm.V = static_cast<const char *>(V);
    prm.O = static_cast<char *>(O);
    prm.lse = lse;
    prm.Sq = static_cast<int>(seq_q);
    prm.Sk = static_cast<int>(seq_k);
    prm.nq = static_cast<int>(nq);
    prm.groups = static_cast<int>(groups);
    prm.c = scale * 1.4426950408889634f;
    prm.off = static_cast<int>(seq_k - seq_q);
    prm.stagger_seed = next_stagger_seed();
    const bool offset = schedule != GEMM_SCHED_IN_PHASE;
    const void *fn = nullptr;
    if (schedule == GEMM_SCHED_INTERLEAVED) {
#define MCS_ATTN4(E, C) \
    if ((dtype == GEMM_DTYPE_BF16) == (E == kElemBF16) && (causal != 0) == C) \
        fn = reinterpret_cast<const void *>(&attention_fwd4_kernel<E, C>);
        MCS_ATTN4(kElemF16, false) MCS_ATTN4(kElemF16, true) MCS_ATTN4(kElemBF16, false) MCS_ATTN4(kElemBF16, true)
#undef MCS_ATTN4
        void *args4[] = {&prm};
        return attn_status(hipLaunchKernel(fn, dim3(static_cast<unsigned>(nq * groups)), dim3(kW4Waves * 64),
                                           args4, 0, stream));
    }
#define MCS_ATTN(E, C, F) \
    if ((dtype == GEMM_DTYPE_BF16) == (E == kElemBF16) && (causal != 0) == C && offset == F) \
        fn = reinterpret_cast<const void *>(&attention_fwd_kernel<E, C, F>);
    MCS_ATTN(kElemF16, false, true) MCS_ATTN(kElemF16, true, true)
    MCS_ATTN(kElemBF16, false, true) MCS_ATTN(kElemBF16, true, true)
    MCS_ATTN(kElemF16, false, false) MCS_ATTN(kElemF16, true, false)
    MCS_ATTN(kElemBF16, false, false) MCS_ATTN(kElemBF16, true, false)
#undef MCS_ATTN
    // persistent: one workgroup per CU (8 per round of each XCD's range, see
    // attn_tile), fewer when there are fewer tiles
    int cus = 0;
    if (const int st = cu_count(cus); st != GEMM_OK) return st;
    const int64_t per = std::min<int64_t>((nq * groups + 7) / 8, std::max(1, cus / 8));
    void *args[] = {&prm};
    return attn_status(hipLaunchKernel(fn, dim3(static_cast<unsigned>(8 * per)), dim3(kAttnWaves * 64),
                                       args, 0, stream));
}

}  // namespace

extern "C" int attention_fwd(int dtype, int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                             int64_t head_dim, const void *Q, const void *K, const void *V, void *O,
                             float *lse, float scale, int causal, hipStream_t stream) {
    return attention_launch(dtype, batch, heads, seq_q, seq_k, head_dim, Q, K, V, O, lse, scale, causal,
                            GEMM_SCHED_AUTO, stream);
}

extern "C" int attention_fwd_ex(int dtype, int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                                int64_t head_dim, const void *Q, const void *K, const void *V, void *O,
                                float *lse, float scale, int causal, int schedule, hipStream_t stream) {
    return attention_launch(dtype, batch, heads, seq_q, seq_k, head_dim, Q, K, V, O, lse, scale, causal,
                            schedule, stream);
}
