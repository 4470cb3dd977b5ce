// Few-token shard products (1 to 4 tokens): Y = X W^T (+ b), or the SwiGLU pair.
//
// With 1-4 tokens a shard product is a stream of the weight shard from HBM ("What is
// tensor parallelism?", section "Why it helps when serving": at decode time each GPU's
// weight traffic is only its own shard), and its fixed costs decide how close the stream
// comes to the memory's rate. This kernel keeps them small:
//   * one workgroup per CU, each owning a contiguous range of output features whose sizes
//     differ by at most one feature, so every CU streams the same number of bytes and no
//     output is split across workgroups (no partial sums travel between workgroups);
//   * inside a workgroup every wave takes an equal contiguous range of K of every row of the
//     range, so the waves stay balanced whatever K is;
//   * each wave keeps D rows' loads in flight (16 bytes per lane per load, a 1 KB
//     contiguous run per wave) in a register ring while it multiplies the oldest row;
//   * the multiply runs on the VALU's bf16 dot product (v_dot2c_f32_bf16: two bf16
//     products added to an fp32 sum, straight from the packed 16-byte loads); with a
//     handful of tokens this is far below the VALU rate. The token chunks a wave needs
//     stay in registers, as loaded, for the whole kernel;
//   * the partial dot products are reduced in a fixed order: across the 64 lanes of a wave
//     by recursive halving (each lane ends with the total of one value), across the waves
//     through LDS in wave order; then bias, SwiGLU or GELU, one rounding, the store.
// Results are therefore bitwise reproducible.
#include <algorithm>
#include <type_traits>

#include "tp_epilogue.h"

namespace tp {
namespace {

constexpr int kGvWaves = 8;           // waves per workgroup
constexpr int kGvThreads = kGvWaves * 64;
constexpr int kGvValues = 64;         // partial values per lane and pass (rows x tokens), padded

struct GemvParams {
    const bf16* X;
    int64_t ldx;
    const bf16* W0;
    const bf16* W1;
    OutDesc o;
    int M, N, K;
    int P;   // workgroups
    int Kw;  // K elements per wave (a multiple of 8)
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + sum_e w[e] * x[e] over 8 consecutive elements, as four bf16 pair products in order.
__device__ __forceinline__ float dot8(const bf16x8& w, const bf16x8& x, float acc) {
#pragma unroll
    for (int e = 0; e < 8; e += 2)
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w[e], w[e + 1]}, bf16x2{x[e], x[e + 1]}, acc, false);
    return acc;
}

// MT: token count bound (1, 2 or 4); J: 512-wide K chunks per row and wave; D: rows in flight.
template <int MT, int J, int ACT, bool BIAS, typename OutT>
__global__ __launch_bounds__(kGvThreads) void gemv_kernel(GemvParams p) {
    constexpr bool SWIGLU = ACT == kActSwiglu;
    constexpr int NR = SWIGLU ? 2 : 1;             // weight rows per output feature
    constexpr int RROWS = kGvValues / MT;          // weight rows per pass
    constexpr int FEAT = RROWS / NR;               // output features per pass
    constexpr int D = J == 1 ? 16 : (J == 2 ? 6 : 3);  // rows in flight per wave (measured)
    static_assert(RROWS * MT == kGvValues, "a pass fills the 64 partial values");

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int f0 = (int)((int64_t)blockIdx.x * p.N / p.P);
    const int f1 = (int)((int64_t)(blockIdx.x + 1) * p.N / p.P);

    // This wave's K range [kb, ke); lane l of chunk j reads elements kb + 512 j + 8 l .. +7.
    const int kb = w * p.Kw;
    const int ke = min(p.K, kb + p.Kw);
    bool kin[J];
    int koff[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        koff[j] = kb + 512 * j + 8 * lane;
        kin[j] = koff[j] < ke;
    }

    // The token chunks of this wave, for the whole kernel.
    bf16x8 xv[J][MT];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            bf16x8 v = {};
            if (kin[j] && m < p.M) v = *reinterpret_cast<const bf16x8*>(p.X + (int64_t)m * p.ldx + koff[j]);
            xv[j][m] = v;
        }

    __shared__ float red[kGvWaves][kGvValues];

    for (int fb = f0; fb < f1; fb += FEAT) {
        const int nf = min(FEAT, f1 - fb);
        const int nrows = nf * NR;
        // Row r of the pass: feature fb + r / NR of the gate (r % NR == 0) or up weight.
        auto row_ptr = [&](int r) -> const bf16* {
            const int f = fb + r / NR;
            return (SWIGLU && (r % NR) ? p.W1 : p.W0) + (int64_t)f * p.K;
        };
        float acc[RROWS][MT];
#pragma unroll
        for (int r = 0; r < RROWS; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

        bf16x8 ring[D][J];
        auto issue = [&](int r, int slot) {
            const bf16* wr = row_ptr(r);
#pragma unroll
            for (int j = 0; j < J; ++j) {
                bf16x8 v = {};
                if (kin[j]) v = *reinterpret_cast<const bf16x8*>(wr + koff[j]);
                ring[slot][j] = v;
            }
        };
#pragma unroll
        for (int r = 0; r < D; ++r)
            if (r < nrows) issue(r, r);
#pragma unroll
        for (int r = 0; r < RROWS; ++r) {
            if (r < nrows) {
                const int slot = r % D;
#pragma unroll
                for (int j = 0; j < J; ++j)
#pragma unroll
                    for (int m = 0; m < MT; ++m) acc[r][m] = dot8(ring[slot][j], xv[j][m], acc[r][m]);
                if (r + D < nrows) issue(r + D, slot);
            }
        }

        // Lane reduction by recursive halving: at the step of width h lanes exchange the
        // half of their values the partner keeps, so after 6 steps lane l holds the wave's
        // total of value v(l) (v = r * MT + m), with v(l) fixed by the lane's bits.
        float v[kGvValues];
#pragma unroll
        for (int r = 0; r < RROWS; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) v[r * MT + m] = acc[r][m];
        int idx = 0;
#pragma unroll
        for (int h = kGvValues / 2, b = 32; h >= 1; h /= 2, b /= 2) {
            const bool hi = (lane & b) != 0;
#pragma unroll
            for (int i = 0; i < h; ++i) {
                const float send = hi ? v[i] : v[i + h];
                const float keep = hi ? v[i + h] : v[i];
                v[i] = keep + __shfl_xor(send, b, 64);
            }
            idx += hi ? h : 0;
        }
        red[w][idx] = v[0];
        __syncthreads();
        // Sum over the waves in wave order, then the epilogue: thread t takes feature
        // q = t / MT of the pass and token m = t % MT.
        if (threadIdx.x < FEAT * MT) {
            const int q = threadIdx.x / MT, m = threadIdx.x % MT;
            if (q < nf && m < p.M) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int ww = 0; ww < kGvWaves; ++ww) {
                    g += red[ww][(q * NR) * MT + m];
                    if (SWIGLU) u += red[ww][(q * NR + 1) * MT + m];
                }
                const int n = fb + q;
                float a = g, c = u;
                if (BIAS) {
                    a += (float)p.o.b0[n];
                    if (SWIGLU) c += (float)p.o.b1[n];
                }
                const float y = SWIGLU ? a / (1.f + expf(-a)) * c : (ACT == kActGelu ? gelu_erf(a) : a);
                reinterpret_cast<OutT*>(p.o.Y)[(int64_t)m * p.o.ldy + n] = (OutT)y;
            }
        }
        __syncthreads();  // red is reused by the next pass
    }
}

}  // namespace

int gemv_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

namespace {

template <int MT, int J, int ACT, bool BIAS, typename OutT>
tp_status_t run_gv(const LinearDesc& d, const Ctx& c, int kw) {
    if (c.planning()) return TP_OK;  // no work space
    GemvParams p;
    p.X = static_cast<const bf16*>(d.X);
    p.ldx = d.ldx;
    p.W0 = static_cast<const bf16*>(d.W0);
    p.W1 = static_cast<const bf16*>(d.W1);
    p.o.Y = d.Y;
    p.o.ldy = d.ldy;
    p.o.M = (int)d.M;
    p.o.N = (int)d.N;
    p.o.b0 = static_cast<const bf16*>(d.b0);
    p.o.b1 = static_cast<const bf16*>(d.b1);
    p.o.vec_store = 0;
    p.o.vec16 = 0;
    p.M = (int)d.M;
    p.N = (int)d.N;
    p.K = (int)d.K;
    p.P = (int)std::min<int64_t>(d.N, gemv_cus());
    p.Kw = kw;
    hipLaunchKernelGGL((gemv_kernel<MT, J, ACT, BIAS, OutT>), dim3((unsigned)p.P), dim3(kGvThreads), 0, c.stream, p);
    return hip_status();
}

template <int MT, int J, int ACT>
tp_status_t run_gv_out(const LinearDesc& d, const Ctx& c, int kw) {
    const bool bias = d.b0 != nullptr;
    if (d.out_dtype == TP_DTYPE_F32) {
        if constexpr (ACT == kActNone) {
            if (!bias) return run_gv<MT, J, ACT, false, float>(d, c, kw);
        }
        return TP_ERR_DTYPE;  // fp32 outputs are the row partials: no bias, no activation
    }
    return bias ? run_gv<MT, J, ACT, true, bf16>(d, c, kw) : run_gv<MT, J, ACT, false, bf16>(d, c, kw);
}

template <int MT, int ACT>
tp_status_t run_gv_j(const LinearDesc& d, const Ctx& c, int kw, int j) {
    switch (j) {
        case 1: return run_gv_out<MT, 1, ACT>(d, c, kw);
        case 2: return run_gv_out<MT, 2, ACT>(d, c, kw);
        case 4: return run_gv_out<MT, 4, ACT>(d, c, kw);
        default: return TP_ERR_SHAPE;
    }
}

template <int ACT>
tp_status_t run_gv_m(const LinearDesc& d, const Ctx& c, int kw, int j) {
    if (d.M == 1) return run_gv_j<1, ACT>(d, c, kw, j);
    if (d.M == 2) return run_gv_j<2, ACT>(d, c, kw, j);
    return run_gv_j<4, ACT>(d, c, kw, j);
}

}  // namespace

// K elements per wave: an equal share of K in whole 16-byte units; J = 512-wide chunks.
int gemv_chunks(int64_t K, int* kw_out) {
    const int64_t kw = (K + 8 * kGvWaves - 1) / (8 * kGvWaves) * 8;
    const int64_t j = (kw + 511) / 512;
    if (kw_out) *kw_out = (int)kw;
    return j <= 1 ? 1 : (j <= 2 ? 2 : (j <= 4 ? 4 : 0));
}

tp_status_t launch_gemv(const LinearDesc& d, const Ctx& c) {
    if (d.M < 1 || d.M > 4) return TP_ERR_SHAPE;
    int kw = 0;
    const int j = gemv_chunks(d.K, &kw);
    if (j == 0) return TP_ERR_SHAPE;
    if (d.swiglu) return run_gv_m<kActSwiglu>(d, c, kw, j);
    if (d.gelu) return run_gv_m<kActGelu>(d, c, kw, j);
    return run_gv_m<kActNone>(d, c, kw, j);
}

}  // namespace tp
