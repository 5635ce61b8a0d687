// Shared between the host entry points and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

// Everything a kernel needs, passed by value as the single kernel argument.
struct GemmParams {
    const uint16_t *A;  // M x K operand bits, row stride lda (elements)
    const uint16_t *B;  // K x N (trans_b = 0) or N x K (trans_b = 1), row stride ldb
    void *C;            // M x N result, row stride ldc
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;  // output tiles of the launched kernel
    int steps;             // K-steps the main loop runs (the pipelined kernel: even, >= 2)
    int group_m;           // tile rows per group in the L2-friendly tile order
};

// Pipelined 256x256x64 kernel: 8 waves, two wave groups.
constexpr int kTileM = 256, kTileN = 256, kTileK = 64, kPipeThreads = 512;
// Within-wave interleaved kernel: the same 256x256x64 tile with 4 waves.
constexpr int kInterThreads = 256;
// Generic kernel: 64x64 tiles of 256 threads.
constexpr int kGenTile = 64, kGenThreads = 256;

// Return the device function for (bf16, trans_b, out_f32[, offset]) so the host
// can launch it or query its attributes; nullptr for an unknown combination.
const void *pipelined_kernel(bool bf16, bool trans_b, bool out_f32, bool offset);
const void *interleaved_kernel(bool bf16, bool trans_b, bool out_f32);
const void *generic_kernel(bool bf16, bool trans_b, bool out_f32);
const void *zero_fill_kernel(bool out_f32);

}  // namespace mcs
