// Output epilogue shared by the bf16 GEMM kernels: bias, SwiGLU and one rounding.
#pragma once

#include "tp_internal.h"

namespace tp {

struct OutDesc {
    void* Y;
    int64_t ldy;
    int M, N;
    const bf16* b0;  // bias of the (gate) product, or nullptr
    const bf16* b1;  // bias of the up product (SwiGLU), or nullptr
    int vec_store;   // 1 when 4 consecutive outputs may be written as one vector
    int vec16;       // 1 when 16-byte aligned runs of a row may be written as one vector
};

template <typename OutT>
__device__ __forceinline__ void store_out4(OutT* row, int n_base, int N, const float y[4], bool vec);

template <>
__device__ __forceinline__ void store_out4<bf16>(bf16* row, int n_base, int N, const float y[4], bool vec) {
    if (vec && n_base + 3 < N) {
        bf16x4 v = {(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
        *reinterpret_cast<bf16x4*>(row + n_base) = v;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n_base + e < N) row[n_base + e] = (bf16)y[e];
    }
}

template <>
__device__ __forceinline__ void store_out4<float>(float* row, int n_base, int N, const float y[4], bool vec) {
    if (vec && n_base + 3 < N) {
        floatx4 v = {y[0], y[1], y[2], y[3]};
        *reinterpret_cast<floatx4*>(row + n_base) = v;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n_base + e < N) row[n_base + e] = y[e];
    }
}

// gelu(z) = z * Phi(z) = z * (1 + erf(z / sqrt(2))) / 2, the exact form the pages'
// FFN applies ("Understanding Tensor Parallelism for Multi-GPU LLM Serving",
// section "Implementing Tensor Parallelism with Hugging Face Accelerate").
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }

// Output activation of a product, a compile-time choice of every kernel.
enum : int { kActNone = 0, kActSwiglu = 1, kActGelu = 2 };

// Four consecutive outputs n_base..n_base+3 from fp32 sums g (and u):
//   none:   y = g + b0[n]
//   GELU:   y = gelu(g + b0[n])
//   SwiGLU: y = silu(g + b0[n]) * (u + b1[n]),  silu(z) = z / (1 + exp(-z))
template <int ACT, bool BIAS>
__device__ __forceinline__ void epilogue_vals4(const OutDesc& o, int n_base, const float g[4], const float u[4],
                                               float y[4]) {
    constexpr bool SWIGLU = ACT == kActSwiglu;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int n = n_base + e;
        float a = g[e];
        float c = SWIGLU ? u[e] : 0.f;
        if (BIAS && n < o.N) {
            a += (float)o.b0[n];
            if (SWIGLU) c += (float)o.b1[n];
        }
        y[e] = SWIGLU ? a / (1.f + expf(-a)) * c : (ACT == kActGelu ? gelu_erf(a) : a);
    }
}

// The same four outputs of token row m, rounded once to OutT and stored.
template <int ACT, bool BIAS, typename OutT>
__device__ __forceinline__ void epilogue4(const OutDesc& o, int n_base, int m, const float g[4], const float u[4]) {
    if (m >= o.M) return;
    float y[4];
    epilogue_vals4<ACT, BIAS>(o, n_base, g, u, y);
    OutT* row = reinterpret_cast<OutT*>(o.Y) + (int64_t)m * o.ldy;
    store_out4<OutT>(row, n_base, o.N, y, o.vec_store != 0);
}

template <typename OutT>
inline int vec_store_ok(const void* Y, int64_t ldy) {
    return ((uintptr_t)Y % (4 * sizeof(OutT)) == 0 && ldy % 4 == 0) ? 1 : 0;
}

template <typename OutT>
inline int vec16_ok(const void* Y, int64_t ldy) {
    return ((uintptr_t)Y % 16 == 0 && (ldy * (int64_t)sizeof(OutT)) % 16 == 0) ? 1 : 0;
}

}  // namespace tp
