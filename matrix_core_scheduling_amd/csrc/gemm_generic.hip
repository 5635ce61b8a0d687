// Generic GEMM kernel for operands the 256x256 kernels cannot take (pointers
// or leading dimensions not 16-byte aligned, rows of K not a whole number of
// 16-byte chunks, very wide rows, FP8 B given K x N): C = A . B with FP32
// fused multiply-adds in increasing k, 64-bit indexing, element loads.  Same
// definition as the 256x256 kernels, slower.
#include "internal.h"

namespace mcs {
namespace {

// Element idx of an operand, widened exactly to FP32 (FP8 E4M3 through the
// hardware conversion).
template <int kElem>
__device__ __forceinline__ float widen(const void *base, int64_t idx) {
    if constexpr (kElem == kElemFP8) {
        return __builtin_amdgcn_cvt_f32_fp8(static_cast<const uint8_t *>(base)[idx], 0);
    } else {
        const uint16_t bits = static_cast<const uint16_t *>(base)[idx];
        if constexpr (kElem == kElemBF16)
            return __uint_as_float(static_cast<uint32_t>(bits) << 16);
        else
            return static_cast<float>(__builtin_bit_cast(_Float16, bits));
    }
}

constexpr int kGenK = 16;

// 64x64 output tile per 256-thread workgroup; thread (ty, tx) owns rows
// ty + 16*i and columns tx + 16*j, i, j < 4.
template <int kElem, bool kTransB, bool kOutF32>
__global__ void __launch_bounds__(kGenThreads) gemm_generic_kernel(GemmParams p) {
    __shared__ float As[kGenK][kGenTile + 1];
    __shared__ float Bs[kGenK][kGenTile + 1];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kGenTile;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kGenTile;
    float acc[4][4];
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int64_t k0 = 0; k0 < p.K; k0 += kGenK) {
        for (int e = threadIdx.x; e < kGenK * kGenTile; e += kGenThreads) {
            const int kk = e % kGenK, mm = e / kGenK;
            const int64_t gm = m0 + mm, gk = k0 + kk;
            As[kk][mm] = (gm < p.M && gk < p.K) ? widen<kElem>(p.A, gm * p.lda + gk) : 0.f;
        }
        for (int e = threadIdx.x; e < kGenK * kGenTile; e += kGenThreads) {
            int kk, nn;
            if constexpr (kTransB) { kk = e % kGenK; nn = e / kGenK; }
            else { nn = e % kGenTile; kk = e / kGenTile; }
            const int64_t gn = n0 + nn, gk = k0 + kk;
            float v = 0.f;
            if (gn < p.N && gk < p.K)
                v = widen<kElem>(p.B, kTransB ? gn * p.ldb + gk : gk * p.ldb + gn);
            Bs[kk][nn] = v;
        }
        __syncthreads();
        for (int kk = 0; kk < kGenK; ++kk)
            for (int i = 0; i < 4; ++i)
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_fmaf(As[kk][ty + 16 * i], Bs[kk][tx + 16 * j], acc[i][j]);
        __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
        const int64_t gm = m0 + ty + 16 * i;
        if (gm >= p.M) continue;
        for (int j = 0; j < 4; ++j) {
            const int64_t gn = n0 + tx + 16 * j;
            if (gn >= p.N) continue;
            if constexpr (kOutF32) {
                reinterpret_cast<float *>(p.C)[gm * p.ldc + gn] = acc[i][j];
            } else if constexpr (kElem != kElemF16) {
                reinterpret_cast<__bf16 *>(p.C)[gm * p.ldc + gn] = static_cast<__bf16>(acc[i][j]);
            } else {
                reinterpret_cast<_Float16 *>(p.C)[gm * p.ldc + gn] = static_cast<_Float16>(acc[i][j]);
            }
        }
    }
}

// C = 0 for K == 0 (an empty sum).  One thread per element, grid-stride.
template <bool kOutF32>
__global__ void __launch_bounds__(256) zero_fill(GemmParams p) {
    const int64_t total = static_cast<int64_t>(p.M) * p.N;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t i = e / p.N, j = e % p.N;
        if constexpr (kOutF32)
            reinterpret_cast<float *>(p.C)[i * p.ldc + j] = 0.f;
        else
            reinterpret_cast<uint16_t *>(p.C)[i * p.ldc + j] = 0;
    }
}

// Split-K reduction: C = round(sum over the S slices of the FP32 partials),
// summed in slice order.  One thread per 4 consecutive columns of a row
// (rows of the workspace start 16-byte aligned); columns at or past N are not
// written.  kOut: 0 FP16, 1 BF16, 2 FP32.
template <int kOut>
__global__ void __launch_bounds__(256) splitk_reduce(GemmParams p, int slices) {
    const int64_t per_row = (p.N + 3) / 4;
    const int64_t total = static_cast<int64_t>(p.M) * per_row;
    const int64_t slice_stride = static_cast<int64_t>(p.M) * p.ldws;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t i = e / per_row, j = (e % per_row) * 4;
        const float *src = p.ws + i * p.ldws + j;
        float4 acc = *reinterpret_cast<const float4 *>(src);
        for (int y = 1; y < slices; ++y) {
            const float4 v = *reinterpret_cast<const float4 *>(src + y * slice_stride);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        const float r[4] = {acc.x, acc.y, acc.z, acc.w};
        for (int c = 0; c < 4 && j + c < p.N; ++c) {
            const int64_t o = i * p.ldc + j + c;
            if constexpr (kOut == 2)
                reinterpret_cast<float *>(p.C)[o] = r[c];
            else if constexpr (kOut == 1)
                reinterpret_cast<__bf16 *>(p.C)[o] = static_cast<__bf16>(r[c]);
            else
                reinterpret_cast<_Float16 *>(p.C)[o] = static_cast<_Float16>(r[c]);
        }
    }
}

}  // namespace

const void *splitk_reduce_kernel(int out_kind) {
    switch (out_kind) {
        case 0: return reinterpret_cast<const void *>(&splitk_reduce<0>);
        case 1: return reinterpret_cast<const void *>(&splitk_reduce<1>);
        case 2: return reinterpret_cast<const void *>(&splitk_reduce<2>);
        default: return nullptr;
    }
}

const void *generic_kernel(int elem, bool trans_b, bool out_f32) {
#define MCS_PICK(E, T, O)                                 \
    if (elem == E && trans_b == T && out_f32 == O)        \
        return reinterpret_cast<const void *>(&gemm_generic_kernel<E, T, O>);
#define MCS_PICK_E(E) MCS_PICK(E, false, false) MCS_PICK(E, false, true) \
                      MCS_PICK(E, true, false) MCS_PICK(E, true, true)
    MCS_PICK_E(kElemF16)
    MCS_PICK_E(kElemBF16)
    MCS_PICK_E(kElemFP8)
#undef MCS_PICK_E
#undef MCS_PICK
    return nullptr;
}

const void *zero_fill_kernel(bool out_f32) {
    return out_f32 ? reinterpret_cast<const void *>(&zero_fill<true>)
                   : reinterpret_cast<const void *>(&zero_fill<false>);
}

}  // namespace mcs
