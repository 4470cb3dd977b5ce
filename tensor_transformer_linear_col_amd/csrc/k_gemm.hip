// Prefill-shaped shard GEMM (M > 64 tokens): Y = X W^T (+ b), or the SwiGLU pair.
//
// At prefill sizes the shard product is bound by the matrix cores. The kernel:
//   * computes a TN x TM output tile per workgroup (TN weight rows x TM tokens) on
//     v_mfma_f32_32x32x16_bf16, the weight block as the A operand and the token
//     block as the B operand, so each lane ends with 4 consecutive output
//     features of one token (an 8-byte bf16 store);
//   * stages 64-wide K slices of both operands through LDS, double buffered: the
//     global loads of slice k+1 are in flight (in registers) while the matrix
//     cores consume slice k, and one barrier per slice separates the buffers;
//   * stores each 128-byte LDS row as 8 chunks of 16 bytes placed at chunk
//     c ^ (row & 7), so both the row-wise stores and the column-wise MFMA operand
//     reads hit 8 distinct bank groups;
//   * for SwiGLU keeps the gate rows and the up rows of the same intermediate
//     features in one tile, so the epilogue has both sums in registers;
//   * orders tiles so that the workgroups resident on one XCD (the hardware deals
//     workgroup ids round-robin over the 8 XCDs) work on a compact block of
//     tiles and share weight and token panels in that XCD's L2.
// The K reduction of every output happens inside one workgroup in a fixed order,
// so results are bitwise reproducible.
//
// MFMA 32x32x16 operand mapping (lane l, l32 = l % 32, lh = l / 32):
//   A: lane l holds W[n0 + l32][k0 + 8*lh .. +7];  B: lane l holds X[m0 + l32][k0 + 8*lh .. +7]
//   D: register e of lane l holds D[n0 + 8*(e/4) + 4*lh + e%4][m0 + l32]
#include "tp_epilogue.h"

namespace tp {
namespace {

constexpr int BK = 64;  // K slice per stage: one 128-byte LDS row per operand row

struct GemmParams {
    const bf16* X;
    int64_t ldx;
    const bf16* W0;
    const bf16* W1;
    OutDesc o;
    int M, N, K;
    int tiles_n, tiles_m;
};

__device__ __forceinline__ bf16x8 ld8g(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Logical tile index of workgroup b: XCD-major when the tile count allows, then
// grouped GW weight-row tiles at a time so resident tiles share panels.
__device__ __forceinline__ void tile_of(int b, int tiles_n, int tiles_m, int& tn, int& tm) {
    constexpr int XCDS = 8, GW = 4;
    const int T = tiles_n * tiles_m;
    const int L = (T % XCDS == 0) ? (b % XCDS) * (T / XCDS) + b / XCDS : b;
    const int per_group = GW * tiles_m;
    const int grp = L / per_group;
    const int first = grp * GW;
    const int gw = min(GW, tiles_n - first);
    const int rem = L - grp * per_group;
    tn = first + rem % gw;
    tm = rem / gw;
}

template <int TN, int TM, int WAVES_N, int WAVES_M, bool SWIGLU, bool BIAS, typename OutT>
__global__ __launch_bounds__(WAVES_N* WAVES_M * 64) void gemm_kernel(GemmParams p) {
    constexpr int NT = WAVES_N * WAVES_M * 64;
    constexpr int WN = TN / WAVES_N;           // output features per wave
    constexpr int WM = TM / WAVES_M;           // tokens per wave
    constexpr int BN = WN / 32, BM = WM / 32;  // 32x32 blocks per wave
    constexpr int NA = SWIGLU ? 2 * BN : BN;   // A-operand blocks (gate then up)
    constexpr int WROWS = SWIGLU ? 2 * TN : TN;
    constexpr int ROWS = WROWS + TM;  // LDS rows per stage
    constexpr int CHUNKS = ROWS * 8;  // 16-byte chunks per stage
    constexpr int LPT = CHUNKS / NT;  // chunks per thread per stage
    static_assert(WN % 32 == 0 && WM % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(CHUNKS % NT == 0, "stage must split evenly over the threads");

    __shared__ __attribute__((aligned(16))) bf16 lds[2][ROWS * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % WAVES_N, wm = wave / WAVES_N;
    const int l32 = lane & 31, lh = lane >> 5;

    int tn, tm;
    tile_of(blockIdx.x, p.tiles_n, p.tiles_m, tn, tm);
    const int n0 = tn * TN, m0 = tm * TM;

    // This thread's global chunks. Rows past N / tokens past M are clamped to the
    // last valid row; their products land in outputs that are never stored.
    const bf16* src[LPT];
    int kcol[LPT];
    int dst[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int q = tid + i * NT;
        const int row = q >> 3, c = q & 7;
        if (row < WROWS) {
            const bool up = SWIGLU && row >= TN;
            const int n = min(n0 + (up ? row - TN : row), p.N - 1);
            src[i] = (up ? p.W1 : p.W0) + (int64_t)n * p.K + c * 8;
        } else {
            const int m = min(m0 + row - WROWS, p.M - 1);
            src[i] = p.X + (int64_t)m * p.ldx + c * 8;
        }
        kcol[i] = c * 8;
        dst[i] = row * BK + ((c ^ (row & 7)) * 8);
    }

    const int KT = (p.K + BK - 1) / BK;
    bf16x8 pre[LPT];
    const bf16x8 zero = {};
    auto load_stage = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < LPT; ++i) pre[i] = (k0 + kcol[i] < p.K) ? ld8g(src[i] + k0) : zero;
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) *reinterpret_cast<bf16x8*>(&lds[buf][dst[i]]) = pre[i];
    };

    floatx16 acc[NA][BM];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < BM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // LDS rows read by this lane for each A / B block.
    int arow[NA], brow[BM];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const bool up = SWIGLU && i >= BN;
        arow[i] = (up ? TN : 0) + wn * WN + (up ? i - BN : i) * 32 + l32;
    }
#pragma unroll
    for (int j = 0; j < BM; ++j) brow[j] = WROWS + wm * WM + j * 32 + l32;

    auto compute = [&](int buf) {
        const bf16* s = lds[buf];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = 2 * ks + lh;
            bf16x8 af[NA], bfr[BM];
#pragma unroll
            for (int i = 0; i < NA; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(&s[arow[i] * BK + ((c ^ (arow[i] & 7)) * 8)]);
#pragma unroll
            for (int j = 0; j < BM; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&s[brow[j] * BK + ((c ^ (brow[j] & 7)) * 8)]);
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int j = 0; j < BM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more) load_stage(kt + 1);
        compute(kt & 1);
        if (more) store_stage((kt + 1) & 1);
        __syncthreads();
    }

    // Epilogue: 4 consecutive features per (block, group of 4 registers).
#pragma unroll
    for (int i = 0; i < BN; ++i)
#pragma unroll
        for (int j = 0; j < BM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float gv[4], uv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gv[e] = acc[i][j][4 * q + e];
                    uv[e] = SWIGLU ? acc[i + (SWIGLU ? BN : 0)][j][4 * q + e] : 0.f;
                }
                const int n_base = n0 + wn * WN + i * 32 + 8 * q + 4 * lh;
                const int m = m0 + wm * WM + j * 32 + l32;
                epilogue4<SWIGLU, BIAS, OutT>(p.o, n_base, m, gv, uv);
            }
}

template <int TN, int TM, int WAVES_N, int WAVES_M, bool SWIGLU, bool BIAS, typename OutT>
tp_status_t run(const LinearDesc& d, hipStream_t stream) {
    GemmParams p;
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
    p.o.vec_store = vec_store_ok<OutT>(d.Y, d.ldy);
    p.M = (int)d.M;
    p.N = (int)d.N;
    p.K = (int)d.K;
    p.tiles_n = (int)ceil_div(d.N, TN);
    p.tiles_m = (int)ceil_div(d.M, TM);
    const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m;
    hipLaunchKernelGGL((gemm_kernel<TN, TM, WAVES_N, WAVES_M, SWIGLU, BIAS, OutT>), dim3((unsigned)tiles),
                       dim3(WAVES_N * WAVES_M * 64), 0, stream, p);
    return hip_status();
}

template <int TN, int TM, int WAVES_N, int WAVES_M, bool SWIGLU>
tp_status_t run_bias(const LinearDesc& d, hipStream_t stream) {
    const bool bias = d.b0 != nullptr;
    if (d.out_dtype == TP_DTYPE_BF16)
        return bias ? run<TN, TM, WAVES_N, WAVES_M, SWIGLU, true, bf16>(d, stream)
                    : run<TN, TM, WAVES_N, WAVES_M, SWIGLU, false, bf16>(d, stream);
    return bias ? run<TN, TM, WAVES_N, WAVES_M, SWIGLU, true, float>(d, stream)
                : run<TN, TM, WAVES_N, WAVES_M, SWIGLU, false, float>(d, stream);
}

}  // namespace

tp_status_t launch_gemm(const LinearDesc& d, hipStream_t stream) {
    int cus = 256;
    {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
    }
    // Large tiles (256 x 256, one workgroup per CU) when they fill the chip, else
    // 128 x 128 tiles (two workgroups per CU).
    if (d.swiglu) {
        const int64_t big = ceil_div(d.N, 128) * ceil_div(d.M, 256);
        if (big >= cus) return run_bias<128, 256, 2, 4, true>(d, stream);
        return run_bias<64, 128, 2, 2, true>(d, stream);
    }
    const int64_t big = ceil_div(d.N, 256) * ceil_div(d.M, 256);
    if (big >= cus) return run_bias<256, 256, 2, 4, false>(d, stream);
    return run_bias<128, 128, 2, 2, false>(d, stream);
}

}  // namespace tp
