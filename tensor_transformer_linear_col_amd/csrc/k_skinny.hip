// Decode-shaped shard GEMM (M <= 64 tokens): Y = X W^T (+ b), or the SwiGLU pair.
//
// At decode sizes the product is bound by streaming the weight shard from HBM
// ("What is tensor parallelism?", section "Why it helps when serving": every GPU
// reads its own slice of the weights). The kernel therefore:
//   * reads every weight byte exactly once with 16-byte loads, keeping several
//     loads per lane in flight (register ping-pong between K chunks);
//   * does the multiply on MFMA (v_mfma_f32_16x16x32_bf16): the weight tile is the
//     A operand (16 rows of W), the token tile is the B operand (up to 16 tokens),
//     so one MFMA consumes a 16 x 32 weight block whatever M is;
//   * splits K three ways: across the 4 lane groups of a wave (inside the MFMA),
//     across the waves of a workgroup (interleaved chunks, reduced through LDS in
//     wave order) and, when the shard has too few 16-row groups to fill the chip,
//     across workgroups (fp32 partial tiles in a work space; the last workgroup
//     to arrive at a tile sums the partials in split order and runs the epilogue).
// Every reduction has a fixed order, so results are bitwise reproducible.
//
// MFMA 16x16x32 operand mapping used here (lane l, l16 = l % 16, lg = l / 16):
//   A (weights): lane l holds W[n0 + l16][k0 + 8*lg .. +7]
//   B (tokens):  lane l holds X[m0 + l16][k0 + 8*lg .. +7]
//   D:           lane l holds D[n0 + 4*lg + e][m0 + l16], e = 0..3
// A and B use the same K placement, so the dot products are exact whatever order
// the unit reduces K in.
#include <algorithm>

#include "tp_epilogue.h"

#ifndef TP_SKINNY_WG_PER_CU
#define TP_SKINNY_WG_PER_CU 1
#endif
#ifndef TP_SKINNY_U1
#define TP_SKINNY_U1 4
#endif

namespace tp {
namespace {

struct SkinnyParams {
    const bf16* X;
    int64_t ldx;
    const bf16* W0;
    const bf16* W1;
    OutDesc o;
    int M, N, K;
    int kchunk;  // K range of one workgroup split (multiple of 32)
    int S;       // number of workgroup splits along K
    float* ws;
    unsigned* counters;
};

__device__ __forceinline__ bf16x8 ld8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// MT: 16-token tiles; RT: 16-row weight tiles per wave (SwiGLU: RT/2 gate + RT/2 up);
// NW: waves per workgroup; U: 32-wide K steps per chunk.
template <int MT, int RT, int NW, int U, bool SWIGLU, bool BIAS, typename OutT>
__global__ __launch_bounds__(NW * 64) void skinny_kernel(SkinnyParams p) {
    constexpr int RH = SWIGLU ? RT / 2 : RT;  // output row tiles
    constexpr int KS = 32 * U;                // K elements per chunk
    constexpr int TILEF = RT * MT * 4 * 64;   // floats of one workgroup's partial tile
    static_assert(!SWIGLU || RT % 2 == 0, "SwiGLU pairs gate and up tiles");

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int g = blockIdx.x / p.S;
    const int s = blockIdx.x - g * p.S;
    const int kb = s * p.kchunk;
    const int ke = min(p.K, kb + p.kchunk);

    // Row pointers. Rows past N / tokens past M are clamped to the last valid row:
    // their products are computed but never stored.
    const bf16* wrow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const bool up = SWIGLU && t >= RH;
        const int tt = up ? t - RH : t;
        const int n = min(g * 16 * RH + tt * 16 + l16, p.N - 1);
        wrow[t] = (up ? p.W1 : p.W0) + (int64_t)n * p.K + 8 * lg;
    }
    const bf16* xrow[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int m = min(j * 16 + l16, p.M - 1);
        xrow[j] = p.X + (int64_t)m * p.ldx + 8 * lg;
    }

    floatx4 acc[RT][MT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[t][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    bf16x8 wa[U][RT], xa[U][MT], wb[U][RT], xb[U][MT];

    auto load_full = [&](bf16x8 (&wf)[U][RT], bf16x8 (&xf)[U][MT], int k0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int t = 0; t < RT; ++t) wf[u][t] = ld8(wrow[t] + k0 + 32 * u);
#pragma unroll
            for (int j = 0; j < MT; ++j) xf[u][j] = ld8(xrow[j] + k0 + 32 * u);
        }
    };
    auto mma = [&](bf16x8 (&wf)[U][RT], bf16x8 (&xf)[U][MT]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int j = 0; j < MT; ++j)
                    acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][t], xf[u][j], acc[t][j], 0, 0, 0);
    };

    const int step = NW * KS;
    int kc = kb + w * KS;
    if (kc + KS <= ke) {
        load_full(wa, xa, kc);
        for (;;) {
            int kn = kc + step;
            if (kn + KS > ke) { mma(wa, xa); kc = kn; break; }
            load_full(wb, xb, kn);
            mma(wa, xa);
            kc = kn;
            kn = kc + step;
            if (kn + KS > ke) { mma(wb, xb); kc = kn; break; }
            load_full(wa, xa, kn);
            mma(wb, xb);
            kc = kn;
        }
    }
    if (kc < ke) {  // at most one partial chunk per wave; pieces past ke are zero
        const bf16x8 zero = {};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = kc + 32 * u + 8 * lg < ke;
#pragma unroll
            for (int t = 0; t < RT; ++t) wa[u][t] = ok ? ld8(wrow[t] + kc + 32 * u) : zero;
#pragma unroll
            for (int j = 0; j < MT; ++j) xa[u][j] = ok ? ld8(xrow[j] + kc + 32 * u) : zero;
        }
        mma(wa, xa);
    }

    // Reduce the waves' partial tiles in wave order.
    __shared__ float red[NW * TILEF];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < MT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[(((w * RT + t) * MT + j) * 4 + e) * 64 + lane] = acc[t][j][e];
    __syncthreads();

    constexpr int Q = RH * MT * 64;  // entries of 4 consecutive output rows
    float* wsg = p.S > 1 ? p.ws + (int64_t)g * p.S * TILEF : nullptr;
    for (int q = threadIdx.x; q < Q; q += NW * 64) {
        const int ln = q & 63;
        const int tj = q >> 6;
        const int j = tj % MT, t = tj / MT;
        float gv[4], uv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a = 0.f, c = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                a += red[(((ww * RT + t) * MT + j) * 4 + e) * 64 + ln];
                if (SWIGLU) c += red[(((ww * RT + t + RH) * MT + j) * 4 + e) * 64 + ln];
            }
            gv[e] = a;
            uv[e] = c;
        }
        if (p.S == 1) {
            epilogue4<SWIGLU, BIAS, OutT>(p.o, g * 16 * RH + t * 16 + 4 * (ln >> 4), j * 16 + (ln & 15), gv, uv);
        } else {
            float* dst = wsg + (int64_t)s * TILEF;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                __hip_atomic_store(dst + ((t * MT + j) * 4 + e) * 64 + ln, gv[e], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (SWIGLU)
                    __hip_atomic_store(dst + (((t + RH) * MT + j) * 4 + e) * 64 + ln, uv[e], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (p.S == 1) return;

    // Cross-workgroup split-K: the last workgroup to arrive at row group g sums the
    // S partial tiles in split order and finishes the tile.
    //
    // The partial tiles move only through device-scope atomic stores and loads, which
    // are coherent across the XCDs' separate L2 caches by themselves (they are issued
    // with the sc1 bit). So no device-scope fence is used: on gfx950 such a fence
    // writes back and invalidates the whole L2 of the XCD, once per workgroup, which
    // would serialise the kernel. Ordering comes from waiting until this thread's
    // partial stores have completed before the arrival counter is incremented; the
    // last workgroup issues its loads only after its increment has returned.
    __shared__ unsigned is_last;
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt = expcnt = lgkmcnt = 0: stores acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(p.counters + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = (prev == (unsigned)(p.S - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (!is_last) return;
    for (int q = threadIdx.x; q < Q; q += NW * 64) {
        const int ln = q & 63;
        const int tj = q >> 6;
        const int j = tj % MT, t = tj / MT;
        float gv[4], uv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a = 0.f, c = 0.f;
            for (int ss = 0; ss < p.S; ++ss) {
                const float* src = wsg + (int64_t)ss * TILEF;
                a += __hip_atomic_load(src + ((t * MT + j) * 4 + e) * 64 + ln, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                if (SWIGLU)
                    c += __hip_atomic_load(src + (((t + RH) * MT + j) * 4 + e) * 64 + ln, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
            gv[e] = a;
            uv[e] = c;
        }
        epilogue4<SWIGLU, BIAS, OutT>(p.o, g * 16 * RH + t * 16 + 4 * (ln >> 4), j * 16 + (ln & 15), gv, uv);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(p.counters + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int MT, int RT, int NW, int U, bool SWIGLU, bool BIAS, typename OutT>
tp_status_t run(const LinearDesc& d, hipStream_t stream) {
    constexpr int RH = SWIGLU ? RT / 2 : RT;
    constexpr int KS = 32 * U;
    constexpr int TILEF = RT * MT * 4 * 64;
    SkinnyParams p;
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

    // Work decomposition: G row groups of 16*RH outputs. K is split across
    // workgroups only when there are fewer row groups than CUs (measured: longer
    // per-wave streams beat a second workgroup per CU once every CU has one).
    const int64_t G = ceil_div(d.N, 16 * RH);
    const int64_t target = TP_SKINNY_WG_PER_CU * (int64_t)device_cus();
    int64_t S = ceil_div(target, G);
    const int64_t smax = std::max<int64_t>(1, d.K / (NW * KS));
    S = std::min<int64_t>(std::max<int64_t>(S, 1), std::min<int64_t>(smax, 64));
    int64_t kchunk = ceil_div(ceil_div(d.K, S), KS) * KS;
    S = ceil_div(d.K, kchunk);
    p.kchunk = (int)kchunk;
    p.S = (int)S;
    p.ws = nullptr;
    p.counters = nullptr;
    if (S > 1) {
        Workspace ws;
        tp_status_t st = get_workspace(stream, (size_t)(G * S * TILEF), (size_t)G, &ws);
        if (st != TP_OK) return st;
        p.ws = ws.partials;
        p.counters = ws.counters;
    }
    hipLaunchKernelGGL((skinny_kernel<MT, RT, NW, U, SWIGLU, BIAS, OutT>), dim3((unsigned)(G * S)),
                       dim3(NW * 64), 0, stream, p);
    return hip_status();
}

template <int MT, int RT, int NW, int U, bool SWIGLU>
tp_status_t run_bias(const LinearDesc& d, hipStream_t stream) {
    const bool bias = d.b0 != nullptr;
    if (d.out_dtype == TP_DTYPE_BF16)
        return bias ? run<MT, RT, NW, U, SWIGLU, true, bf16>(d, stream)
                    : run<MT, RT, NW, U, SWIGLU, false, bf16>(d, stream);
    return bias ? run<MT, RT, NW, U, SWIGLU, true, float>(d, stream)
                : run<MT, RT, NW, U, SWIGLU, false, float>(d, stream);
}

}  // namespace

tp_status_t launch_skinny(const LinearDesc& d, hipStream_t stream) {
    const int mt = (int)ceil_div(d.M, 16);
    if (d.swiglu) {
        switch (mt) {
            case 1: return run_bias<1, 2, 8, TP_SKINNY_U1, true>(d, stream);
            case 2: return run_bias<2, 2, 4, 2, true>(d, stream);
            case 3: return run_bias<3, 2, 4, 2, true>(d, stream);
            case 4: return run_bias<4, 4, 4, 1, true>(d, stream);
            default: return TP_ERR_SHAPE;
        }
    }
    switch (mt) {
        case 1: return run_bias<1, 1, 8, TP_SKINNY_U1, false>(d, stream);
        case 2: return run_bias<2, 2, 4, 2, false>(d, stream);
        case 3: return run_bias<3, 2, 4, 2, false>(d, stream);
        case 4: return run_bias<4, 4, 4, 1, false>(d, stream);
        default: return TP_ERR_SHAPE;
    }
}

}  // namespace tp
