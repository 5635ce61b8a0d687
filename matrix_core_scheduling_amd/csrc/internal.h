// Shared between the host entry points and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

// Operand element kinds (a template parameter of every kernel).
enum Elem : int { kElemF16 = 0, kElemBF16 = 1, kElemFP8 = 2 };

// Everything a kernel needs, passed by value as the single kernel argument.
struct GemmParams {
    const void *A;      // M x K operand bits, row stride lda (elements)
    const void *B;      // K x N (trans_b = 0) or N x K (trans_b = 1), row stride ldb
    void *C;            // M x N result, row stride ldc
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;  // output tiles of the launched kernel
    int steps;             // K-steps the main loop runs (the pipelined kernel: even, >= 2)
    int group_m;           // tile rows per group in the L2-friendly tile order
    // Split K (launched with gridDim.y = number of slices > 1): slice y covers
    // k in [y * kslice, min(K, (y + 1) * kslice)) and writes its FP32 partial
    // product to ws + y * M * ldws (row stride ldws floats) instead of C.
    int kslice;
    float *ws;
    int64_t ldws;
    // Seed of the race-stress pauses (read only by the race-stress build).
    uint32_t stagger_seed;
};

// The view of the product one workgroup computes: the whole of it, or with
// several K-slices (gridDim.y > 1) slice blockIdx.y of it, whose FP32 result
// goes to the workspace.  `steps` is already a full slice's step count; with
// kExactSteps it becomes this slice's own count of 128-byte K-steps (the last
// slice may be shorter), so the last of them is the partial one if K is not a
// whole number of K-steps.
template <int kElemBytes, bool kTransB, bool kExactSteps = false>
__device__ __forceinline__ GemmParams slice_view(const GemmParams &p) {
    if (gridDim.y == 1) return p;
    GemmParams q = p;
    const int y = blockIdx.y;
    const int64_t k0 = static_cast<int64_t>(y) * p.kslice;
    q.K = static_cast<int>(min(static_cast<int64_t>(p.K) - k0, static_cast<int64_t>(p.kslice)));
    if constexpr (kExactSteps) q.steps = (q.K * kElemBytes + 127) / 128;
    q.A = static_cast<const char *>(p.A) + k0 * kElemBytes;
    q.B = static_cast<const char *>(p.B) + k0 * kElemBytes * (kTransB ? 1 : p.ldb);
    q.C = p.ws + static_cast<int64_t>(y) * p.M * p.ldws;
    q.ldc = p.ldws;
    return q;
}

// Pipelined 256x256 kernel: 8 waves, two wave groups.  A K-step moves 128
// bytes of every operand row: 64 FP16/BF16 or 128 FP8 elements.
constexpr int kTileM = 256, kTileN = 256, kStepBytes = 128, kPipeThreads = 512;
constexpr int elem_bytes(int elem) { return elem == kElemFP8 ? 1 : 2; }
constexpr int step_k(int elem) { return kStepBytes / elem_bytes(elem); }
// Within-wave interleaved kernel: the same 256x256x64 tile with 4 waves.
constexpr int kInterThreads = 256;
// 128x128-tile kernel: 4 waves.
constexpr int kTile128 = 128, kTile128Threads = 256;
// Generic kernel: 64x64 tiles of 256 threads.
constexpr int kGenTile = 64, kGenThreads = 256;

// The host-side accessors below stay inside the library (hidden), so two
// builds of it loaded into one process (the product and the race-stress
// build) each launch their own kernels.
#pragma GCC visibility push(hidden)

// Return the device function for (elem, trans_b, out_f32[, offset]) so the host
// can launch it or query its attributes; nullptr for a combination that is not
// compiled (the 256x256 kernels take FP8 operands only with B given N x K).
// A 16-bit output is FP16 for FP16 operands and BF16 otherwise.
const void *pipelined_kernel(int elem, bool trans_b, bool out_f32, bool offset);
const void *interleaved_kernel(int elem, bool trans_b, bool out_f32);
const void *tile128_kernel(int elem, bool trans_b, bool out_f32);
const void *generic_kernel(int elem, bool trans_b, bool out_f32);
const void *zero_fill_kernel(bool out_f32);
// Split-K reduction into C: out_kind 0 FP16, 1 BF16, 2 FP32.
const void *splitk_reduce_kernel(int out_kind);

#pragma GCC visibility pop

// Seed for the next launch's race-stress pauses: a fresh value per launch in
// the race-stress build (MCS_STAGGER), 0 in the product build.
inline uint32_t next_stagger_seed() {
#ifdef MCS_STAGGER
    static uint32_t counter = 0;
    return __atomic_add_fetch(&counter, 1u, __ATOMIC_RELAXED) * 0x9E3779B9u;
#else
    return 0;
#endif
}

}  // namespace mcs
