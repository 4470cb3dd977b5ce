// On-device combines and shard copies: all bound by HBM bandwidth, no arithmetic
// beyond the sum.
//
//   combine_sum: Y = sum_r P_r + b with fp32 accumulation in rank order and one
//     rounding ("Understanding Tensor Parallelism for Multi-GPU LLM Serving":
//     RowParallelLinear sums the partials with all_reduce(SUM), then adds the
//     bias once). Each thread owns 8 consecutive elements: one 16-byte load per
//     bf16 partial, so every partial is streamed once, coalesced.
//   concat: the column shards' outputs side by side in rank order ("Tensor
//     parallel serving": torch.cat on the last axis), per segment for a fused
//     Q | K | V output. 16-byte units when every width allows, else elements.
//   copy2d: a strided block copy (taking a weight shard).
#include <algorithm>

#include <type_traits>

#include "tp_internal.h"

namespace tp {
namespace {

constexpr int MAXP = 64;
constexpr int MAXSEG = 8;

struct PtrPack {
    const void* p[MAXP];
};

template <typename T>
__device__ __forceinline__ void load8(const T* src, float v[8]);

template <>
__device__ __forceinline__ void load8<bf16>(const bf16* src, float v[8]) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(src);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}

template <>
__device__ __forceinline__ void load8<float>(const float* src, float v[8]) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(src);
    const floatx4 b = *reinterpret_cast<const floatx4*>(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[e + 4] = b[e];
    }
}

template <typename T>
__device__ __forceinline__ void store8(T* dst, const float v[8]);

template <>
__device__ __forceinline__ void store8<bf16>(bf16* dst, const float v[8]) {
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8*>(dst) = x;
}

template <>
__device__ __forceinline__ void store8<float>(float* dst, const float v[8]) {
    *reinterpret_cast<floatx4*>(dst) = floatx4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<floatx4*>(dst + 4) = floatx4{v[4], v[5], v[6], v[7]};
}

// PC: the number of partials when known at compile time (their loads are then all issued
// before the first add, instead of one HBM round trip per partial), else 0.
template <typename PT, typename OT, bool BIAS, int PC>
__global__ __launch_bounds__(256) void combine_sum_kernel(PtrPack pk, int P, const OT* b, OT* Y, int64_t total,
                                                          int64_t N, int vec) {
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i0 >= total) return;
    if (vec && i0 + 8 <= total) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if constexpr (PC > 0) {
            float v[PC][8];
#pragma unroll
            for (int r = 0; r < PC; ++r) load8<PT>(static_cast<const PT*>(pk.p[r]) + i0, v[r]);
#pragma unroll
            for (int r = 0; r < PC; ++r)  // rank order
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += v[r][e];
        } else {
            for (int r = 0; r < P; ++r) {
                float v[8];
                load8<PT>(static_cast<const PT*>(pk.p[r]) + i0, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += v[e];
            }
        }
        if (BIAS) {
            int64_t n = i0 % N;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc[e] += (float)b[n];
                n = (n + 1 == N) ? 0 : n + 1;
            }
        }
        store8<OT>(Y + i0, acc);
    } else {
        for (int64_t i = i0; i < i0 + 8 && i < total; ++i) {
            float a = 0.f;
            for (int r = 0; r < P; ++r) a += (float)static_cast<const PT*>(pk.p[r])[i];
            if (BIAS) a += (float)b[i % N];
            Y[i] = (OT)a;
        }
    }
}

struct ConcatArgs {
    const void* src[MAXP];
    int64_t seg[MAXSEG];     // segment widths, in units
    int64_t segoff[MAXSEG];  // segment offsets inside one shard row, in units
    int nseg;
    int p;
    int64_t S;  // units per shard row
};

// One thread per output unit (16 bytes, or one element). Output row layout:
// for each segment j, p blocks of seg[j] units, shard r at block r.
template <typename U>
__global__ __launch_bounds__(256) void concat_kernel(ConcatArgs a, U* Y, int64_t M) {
    const int64_t row_units = a.S * a.p;
    const int64_t total = M * row_units;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t m = i / row_units;
        int64_t c = i - m * row_units;
        int j = 0;
        while (j + 1 < a.nseg && c >= a.p * a.seg[j]) {
            c -= a.p * a.seg[j];
            ++j;
        }
        const int64_t r = c / a.seg[j];
        const int64_t cc = c - r * a.seg[j];
        Y[i] = static_cast<const U*>(a.src[r])[m * a.S + a.segoff[j] + cc];
    }
}

template <typename U>
__global__ __launch_bounds__(256) void copy2d_kernel(const U* src, int64_t lds, U* dst, int64_t ldd, int64_t rows,
                                                     int64_t cols) {
    const int64_t total = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / cols;
        const int64_t c = i - r * cols;
        dst[r * ldd + c] = src[r * lds + c];
    }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(unsigned* p, size_t n, unsigned v) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}

struct alignas(16) Unit16 {
    uint32_t w[4];
};

unsigned grid_for(int64_t items) {
    const int64_t blocks = ceil_div(items, 256);
    return (unsigned)std::min<int64_t>(std::max<int64_t>(blocks, 1), 65536);
}

template <typename PT, typename OT>
tp_status_t sum_typed(const PtrPack& pk, int p, const void* b, void* Y, int64_t M, int64_t N, int vec,
                      hipStream_t stream) {
    const int64_t total = M * N;
    const unsigned grid = (unsigned)ceil_div(ceil_div(total, 8), 256);
    auto go = [&](auto pc) {
        constexpr int PC = decltype(pc)::value;
        if (b)
            hipLaunchKernelGGL((combine_sum_kernel<PT, OT, true, PC>), dim3(grid), dim3(256), 0, stream, pk, p,
                               static_cast<const OT*>(b), static_cast<OT*>(Y), total, N, vec);
        else
            hipLaunchKernelGGL((combine_sum_kernel<PT, OT, false, PC>), dim3(grid), dim3(256), 0, stream, pk, p,
                               static_cast<const OT*>(nullptr), static_cast<OT*>(Y), total, N, vec);
    };
    switch (p) {
        case 2: go(std::integral_constant<int, 2>{}); break;
        case 4: go(std::integral_constant<int, 4>{}); break;
        case 8: go(std::integral_constant<int, 8>{}); break;
        default: go(std::integral_constant<int, 0>{}); break;
    }
    return hip_status();
}

}  // namespace

tp_status_t launch_combine_sum(const void* const* partials, int p, tp_dtype_t pdt, const void* b, void* Y,
                               int64_t M, int64_t N, tp_dtype_t odt, hipStream_t stream) {
    if (p > MAXP) return TP_ERR_SHAPE;
    PtrPack pk;
    int vec = ((uintptr_t)Y % 16 == 0) ? 1 : 0;
    for (int r = 0; r < p; ++r) {
        pk.p[r] = partials[r];
        if ((uintptr_t)partials[r] % 16 != 0) vec = 0;
    }
    for (int r = p; r < MAXP; ++r) pk.p[r] = nullptr;
    if (M * N == 0) return TP_OK;
    if (pdt == TP_DTYPE_BF16 && odt == TP_DTYPE_BF16) return sum_typed<bf16, bf16>(pk, p, b, Y, M, N, vec, stream);
    if (pdt == TP_DTYPE_BF16 && odt == TP_DTYPE_F32) return sum_typed<bf16, float>(pk, p, b, Y, M, N, vec, stream);
    if (pdt == TP_DTYPE_F32 && odt == TP_DTYPE_BF16) return sum_typed<float, bf16>(pk, p, b, Y, M, N, vec, stream);
    return sum_typed<float, float>(pk, p, b, Y, M, N, vec, stream);
}

tp_status_t launch_concat(const void* const* shards, int p, const int64_t* seg, int nseg, void* Y, int64_t M,
                          size_t elem, hipStream_t stream) {
    if (p > MAXP || nseg > MAXSEG) return TP_ERR_SHAPE;
    int64_t S = 0;
    bool vec = ((uintptr_t)Y % 16 == 0);
    for (int j = 0; j < nseg; ++j) {
        if ((seg[j] * (int64_t)elem) % 16 != 0) vec = false;
        S += seg[j];
    }
    for (int r = 0; r < p; ++r)
        if ((uintptr_t)shards[r] % 16 != 0) vec = false;
    if (M * S == 0) return TP_OK;
    const int64_t unit = vec ? 16 / (int64_t)elem : 1;
    ConcatArgs a;
    for (int r = 0; r < MAXP; ++r) a.src[r] = r < p ? shards[r] : nullptr;
    int64_t off = 0;
    for (int j = 0; j < MAXSEG; ++j) {
        a.seg[j] = j < nseg ? seg[j] / unit : 1;
        a.segoff[j] = j < nseg ? off : 0;
        if (j < nseg) off += seg[j] / unit;
    }
    a.nseg = nseg;
    a.p = p;
    a.S = S / unit;
    const unsigned grid = grid_for(M * a.S * p);
    if (vec) {
        hipLaunchKernelGGL((concat_kernel<Unit16>), dim3(grid), dim3(256), 0, stream, a, static_cast<Unit16*>(Y), M);
    } else if (elem == 2) {
        hipLaunchKernelGGL((concat_kernel<uint16_t>), dim3(grid), dim3(256), 0, stream, a, static_cast<uint16_t*>(Y),
                           M);
    } else {
        hipLaunchKernelGGL((concat_kernel<uint32_t>), dim3(grid), dim3(256), 0, stream, a, static_cast<uint32_t*>(Y),
                           M);
    }
    return hip_status();
}

tp_status_t launch_copy2d(const void* src, int64_t lds, void* dst, int64_t ldd, int64_t rows, int64_t cols,
                          size_t elem, hipStream_t stream) {
    if (rows * cols == 0) return TP_OK;
    const bool vec = (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0 && (cols * (int64_t)elem) % 16 == 0 &&
                     (lds * (int64_t)elem) % 16 == 0 && (ldd * (int64_t)elem) % 16 == 0;
    if (vec) {
        const int64_t u = 16 / (int64_t)elem;
        hipLaunchKernelGGL((copy2d_kernel<Unit16>), dim3(grid_for(rows * cols / u)), dim3(256), 0, stream,
                           static_cast<const Unit16*>(src), lds / u, static_cast<Unit16*>(dst), ldd / u, rows,
                           cols / u);
    } else if (elem == 2) {
        hipLaunchKernelGGL((copy2d_kernel<uint16_t>), dim3(grid_for(rows * cols)), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(src), lds, static_cast<uint16_t*>(dst), ldd, rows, cols);
    } else {
        hipLaunchKernelGGL((copy2d_kernel<uint32_t>), dim3(grid_for(rows * cols)), dim3(256), 0, stream,
                           static_cast<const uint32_t*>(src), lds, static_cast<uint32_t*>(dst), ldd, rows, cols);
    }
    return hip_status();
}

tp_status_t launch_fill_u32(unsigned* p, size_t n, unsigned v, hipStream_t stream) {
    if (n == 0) return TP_OK;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for((int64_t)n)), dim3(256), 0, stream, p, n, v);
    return hip_status();
}

}  // namespace tp
