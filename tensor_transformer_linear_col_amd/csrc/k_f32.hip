// fp32 shard GEMM on the vector ALUs: Y = X W^T (+ b), or the SwiGLU pair, all fp32.
//
// This is the full-precision path (the simulation on the "Tensor parallel serving"
// page runs the split in fp32). gfx950 has no fp32 matrix-core rate worth the
// layout work here, and this path is not the performance path, so it is a plain
// LDS-tiled FMA kernel: a 64 x 64 output tile per 256-thread workgroup, 4 x 4
// outputs per thread, K staged 16 at a time. Any sizes and strides; no alignment.
#include "tp_internal.h"

namespace tp {
namespace {

struct F32Params {
    const float* X;
    int64_t ldx;
    const float* W0;
    const float* W1;
    const float* b0;
    const float* b1;
    float* Y;
    int64_t ldy;
    int M, N, K;
    int gelu;  // 1: y = gelu(g) for plain products
};

constexpr int T64 = 64, KB = 16;

template <bool SWIGLU, bool BIAS>
__global__ __launch_bounds__(256) void f32_kernel(F32Params p) {
    __shared__ float ws0[KB][T64 + 4];
    __shared__ float ws1[SWIGLU ? KB : 1][T64 + 4];
    __shared__ float xs[KB][T64 + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15;  // token sub-tile
    const int ty = tid >> 4;  // feature sub-tile
    const int n0 = blockIdx.x * T64, m0 = blockIdx.y * T64;

    float acc0[4][4] = {}, acc1[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += KB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * 256;
            const int r = e >> 4, kk = e & 15;
            const int n = n0 + r, m = m0 + r, k = k0 + kk;
            const bool kok = k < p.K;
            ws0[kk][r] = (kok && n < p.N) ? p.W0[(int64_t)n * p.K + k] : 0.f;
            if (SWIGLU) ws1[kk][r] = (kok && n < p.N) ? p.W1[(int64_t)n * p.K + k] : 0.f;
            xs[kk][r] = (kok && m < p.M) ? p.X[(int64_t)m * p.ldx + k] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            float a[4], b[4], x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = ws0[kk][ty * 4 + i];
                if (SWIGLU) b[i] = ws1[kk][ty * 4 + i];
                x[i] = xs[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc0[i][j] = fmaf(a[i], x[j], acc0[i][j]);
                    if (SWIGLU) acc1[i][j] = fmaf(b[i], x[j], acc1[i][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = n0 + ty * 4 + i;
        if (n >= p.N) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + tx * 4 + j;
            if (m >= p.M) continue;
            float g = acc0[i][j];
            if (BIAS) g += p.b0[n];
            float y = p.gelu ? 0.5f * g * (1.f + erff(g * 0.70710678118654752f)) : g;
            if (SWIGLU) {
                float u = acc1[i][j];
                if (BIAS) u += p.b1[n];
                y = g / (1.f + expf(-g)) * u;
            }
            p.Y[(int64_t)m * p.ldy + n] = y;
        }
    }
}

}  // namespace

tp_status_t launch_f32(const LinearDesc& d, const Ctx& c) {
    if (c.planning()) return TP_OK;  // no work space
    const hipStream_t stream = c.stream;
    F32Params p;
    p.X = static_cast<const float*>(d.X);
    p.ldx = d.ldx;
    p.W0 = static_cast<const float*>(d.W0);
    p.W1 = static_cast<const float*>(d.W1);
    p.b0 = static_cast<const float*>(d.b0);
    p.b1 = static_cast<const float*>(d.b1);
    p.Y = static_cast<float*>(d.Y);
    p.gelu = d.gelu ? 1 : 0;
    p.ldy = d.ldy;
    p.M = (int)d.M;
    p.N = (int)d.N;
    p.K = (int)d.K;
    const dim3 grid((unsigned)ceil_div(d.N, T64), (unsigned)ceil_div(d.M, T64));
    const bool bias = d.b0 != nullptr;
    if (d.swiglu) {
        if (bias) hipLaunchKernelGGL((f32_kernel<true, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((f32_kernel<true, false>), grid, dim3(256), 0, stream, p);
    } else {
        if (bias) hipLaunchKernelGGL((f32_kernel<false, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((f32_kernel<false, false>), grid, dim3(256), 0, stream, p);
    }
    return hip_status();
}

}  // namespace tp
