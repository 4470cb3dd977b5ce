// Decode-shaped shard GEMM (M <= 64 tokens): Y = X W^T (+ b), or the SwiGLU pair.
//
// At decode sizes the product is bound by streaming the weight shard from HBM
// ("What is tensor parallelism?", section "Why it helps when serving": each GPU's
// weight traffic is only its own shard). The kernel therefore:
//   * reads every weight byte exactly once with 16-byte loads, keeping several
//     loads per lane in flight (register ping-pong between K chunks);
//   * does the multiply on MFMA (v_mfma_f32_16x16x32_bf16): the weight tile is the
//     A operand (16 rows of W), the token tile is the B operand (up to 16 tokens),
//     so one MFMA consumes a 16 x 32 weight block whatever M is;
//   * splits a row group's K across the 4 lane groups of a wave (inside the MFMA),
//     across the waves of a workgroup (interleaved pieces, reduced through LDS in
//     wave order) and across workgroups (fp32 partial tiles in a work space; the
//     last workgroup to arrive at the row group sums the partials in K order and
//     runs the epilogue);
//   * hands out the work as the list of (row group, K chunk) units, row group major,
//     cut into one contiguous range per workgroup. With one unit per workgroup this
//     is a plain split-K grid; with one workgroup per CU and equal ranges (used for
//     the 33-64 token tiles, whose register footprint allows one workgroup per CU, and
//     for long SwiGLU weight streams) every CU streams the same number of bytes
//     whatever the shard's shape.
// Every reduction has a fixed order, so results are bitwise reproducible.
//
// MFMA 16x16x32 operand mapping used here (lane l, l16 = l % 16, lg = l / 16):
//   A (weights): lane l holds W[n0 + l16][k0 + 8*lg .. +7]
//   B (tokens):  lane l holds X[m0 + l16][k0 + 8*lg .. +7]
//   D:           lane l holds D[n0 + 4*lg + e][m0 + l16], e = 0..3
// A and B use the same K placement, so the dot products are exact whatever order
// the unit reduces K in.
#include <algorithm>
#include <type_traits>

#include "tp_epilogue.h"

namespace tp {
namespace {

// Tile choices, each measured on the decode shards (70B TP=4, 7B TP=2):
constexpr int kWgPerCu = 1;    // split-K grid target: workgroups per CU
constexpr int kU1 = 4;         // 32-wide K steps per piece, one token tile, plain products
constexpr int kU4 = 2;         // 32-wide K steps per piece, four token tiles
constexpr int kTwoRowsM = 5;   // from this many tokens, two row tiles per wave (plain)
constexpr int kPairTilesM = 3; // from this many tokens, 2 gate + 2 up tiles per wave (SwiGLU)

struct SkinnyParams {
    const bf16* X;
    int64_t ldx;
    const bf16* W0;
    const bf16* W1;
    OutDesc o;
    int M, N, K;
    int C;       // K chunks per row group
    int CK;      // K elements per chunk
    int64_t U;   // units: row groups x C
    int P;       // workgroups (the grid)
    float* ws;   // two partial tiles per workgroup (its first and its last row group)
    unsigned* counters;  // one per row group; zero between launches
};

// First unit of workgroup w's range, and the workgroup that owns unit u.
__device__ __forceinline__ int64_t range_begin(int64_t w, int64_t U, int64_t P) { return w * U / P; }
__device__ __forceinline__ int64_t owner_of(int64_t u, int64_t U, int64_t P) { return ((u + 1) * P - 1) / U; }

__device__ __forceinline__ bf16x8 ld8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// MT: 16-token tiles; RT: 16-row weight tiles per wave (SwiGLU: RT/2 gate + RT/2 up);
// NW: waves per workgroup; U: 32-wide K steps per piece; PERSIST: ranges of many
// units (else exactly one unit per workgroup).
template <int MT, int RT, int NW, int U, bool PERSIST, int ACT, bool BIAS, typename OutT>
__global__ __launch_bounds__(NW * 64) void skinny_kernel(SkinnyParams p) {
    constexpr bool SWIGLU = ACT == kActSwiglu;
    constexpr int RH = SWIGLU ? RT / 2 : RT;  // output row tiles
    constexpr int KS = 32 * U;                // K elements per piece
    constexpr int TILEF = RT * MT * 4 * 64;   // floats of one workgroup's partial tile
    constexpr int Q = RH * MT * 64;           // entries of 4 consecutive output rows
    static_assert(!SWIGLU || RT % 2 == 0, "SwiGLU pairs gate and up tiles");

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int64_t u0 = PERSIST ? range_begin(blockIdx.x, p.U, p.P) : blockIdx.x;
    const int64_t u1 = PERSIST ? range_begin(blockIdx.x + 1, p.U, p.P) : u0 + 1;

    // Token rows past M are clamped to the last valid row: their products are
    // computed but never stored.
    const bf16* xrow[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int m = min(j * 16 + l16, p.M - 1);
        xrow[j] = p.X + (int64_t)m * p.ldx + 8 * lg;
    }

    __shared__ float red[NW * TILEF];
    __shared__ unsigned is_last;

    for (int64_t u = u0; u < u1;) {
        const int g = (int)(u / p.C);
        const int c0 = (int)(u - (int64_t)g * p.C);
        const int64_t uend = min(u1, (int64_t)(g + 1) * p.C);
        const int c1 = (int)(uend - (int64_t)g * p.C);
        const bool whole = c0 == 0 && c1 == p.C;
        const int kb = c0 * p.CK;
        const int ke = min(p.K, c1 * p.CK);

        // Weight rows past N are clamped like the token rows.
        const bf16* wrow[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const bool up = SWIGLU && t >= RH;
            const int tt = up ? t - RH : t;
            const int n = min(g * 16 * RH + tt * 16 + l16, p.N - 1);
            wrow[t] = (up ? p.W1 : p.W0) + (int64_t)n * p.K + 8 * lg;
        }

        floatx4 acc[RT][MT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int j = 0; j < MT; ++j) acc[t][j] = floatx4{0.f, 0.f, 0.f, 0.f};

        bf16x8 wa[U][RT], xa[U][MT], wb[U][RT], xb[U][MT];
        auto load_full = [&](bf16x8 (&wf)[U][RT], bf16x8 (&xf)[U][MT], int k0) {
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
#pragma unroll
                for (int t = 0; t < RT; ++t) wf[uu][t] = ld8(wrow[t] + k0 + 32 * uu);
#pragma unroll
                for (int j = 0; j < MT; ++j) xf[uu][j] = ld8(xrow[j] + k0 + 32 * uu);
            }
        };
        auto mma = [&](bf16x8 (&wf)[U][RT], bf16x8 (&xf)[U][MT]) {
#pragma unroll
            for (int uu = 0; uu < U; ++uu)
#pragma unroll
                for (int t = 0; t < RT; ++t)
#pragma unroll
                    for (int j = 0; j < MT; ++j)
                        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[uu][t], xf[uu][j], acc[t][j], 0, 0, 0);
        };

        // This wave's pieces: kb + w*KS, then every NW*KS, with register ping-pong so
        // one piece is in flight while the previous one is multiplied. The scheduling
        // barriers keep every load of the next piece ahead of the first wait for the
        // current one.
        const int step = NW * KS;
        int kc = kb + w * KS;
        if (kc + KS <= ke) {
            load_full(wa, xa, kc);
            for (;;) {
                int kn = kc + step;
                if (kn + KS > ke) { mma(wa, xa); kc = kn; break; }
                load_full(wb, xb, kn);
                __builtin_amdgcn_sched_barrier(0);
                mma(wa, xa);
                kc = kn;
                kn = kc + step;
                if (kn + KS > ke) { mma(wb, xb); kc = kn; break; }
                load_full(wa, xa, kn);
                __builtin_amdgcn_sched_barrier(0);
                mma(wb, xb);
                kc = kn;
            }
        }
        if (kc < ke) {  // at most one partial piece per wave; K past ke reads as zero
            const bf16x8 zero = {};
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                const bool ok = kc + 32 * uu + 8 * lg < ke;
#pragma unroll
                for (int t = 0; t < RT; ++t) wa[uu][t] = ok ? ld8(wrow[t] + kc + 32 * uu) : zero;
#pragma unroll
                for (int j = 0; j < MT; ++j) xa[uu][j] = ok ? ld8(xrow[j] + kc + 32 * uu) : zero;
            }
            mma(wa, xa);
        }

        // Reduce the waves' partial tiles in wave order.
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int j = 0; j < MT; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[(((w * RT + t) * MT + j) * 4 + e) * 64 + lane] = acc[t][j][e];
        __syncthreads();

        // A cut row group leaves its partial tile in this workgroup's slot: slot 0
        // for the first row group of the range, slot 1 for the last.
        float* mine = p.ws + ((int64_t)blockIdx.x * 2 + (u == u0 ? 0 : 1)) * TILEF;
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
            if (whole) {
                epilogue4<ACT, BIAS, OutT>(p.o, g * 16 * RH + t * 16 + 4 * (ln >> 4), j * 16 + (ln & 15), gv, uv);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    __hip_atomic_store(mine + ((t * MT + j) * 4 + e) * 64 + ln, gv[e], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    if (SWIGLU)
                        __hip_atomic_store(mine + (((t + RH) * MT + j) * 4 + e) * 64 + ln, uv[e], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if (!whole) {
            // The partial tiles move only through device-scope atomic stores and loads,
            // which are coherent across the XCDs' separate L2 caches by themselves (they
            // are issued with the sc1 bit). So no device-scope fence is used: on gfx950
            // such a fence writes back and invalidates the whole L2 of the XCD, which
            // would serialise the kernel. Ordering comes from waiting until this
            // thread's partial stores have completed before the arrival counter is
            // incremented; the last workgroup issues its loads only after its
            // increment has returned.
            const int64_t wfirst = PERSIST ? owner_of((int64_t)g * p.C, p.U, p.P) : (int64_t)g * p.C;
            const int64_t wlast = PERSIST ? owner_of((int64_t)(g + 1) * p.C - 1, p.U, p.P) : (int64_t)(g + 1) * p.C - 1;
            __builtin_amdgcn_s_waitcnt(0);  // vmcnt = expcnt = lgkmcnt = 0: stores acknowledged
            __syncthreads();
            if (threadIdx.x == 0) {
                const unsigned prev =
                    __hip_atomic_fetch_add(p.counters + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                is_last = (prev == (unsigned)(wlast - wfirst)) ? 1u : 0u;
            }
            __syncthreads();
            if (is_last) {
                // Sum the row group's partial tiles in K order, i.e. in workgroup order.
                for (int q = threadIdx.x; q < Q; q += NW * 64) {
                    const int ln = q & 63;
                    const int tj = q >> 6;
                    const int j = tj % MT, t = tj / MT;
                    // NB contributors' loads in flight at a time (clamped indices past the
                    // last are loaded and not added), summed in workgroup order.
                    constexpr int NB = MT * RT >= 8 ? 1 : (SWIGLU ? 2 : 4);  // register budget
                    float gv[4] = {0.f, 0.f, 0.f, 0.f}, uv[4] = {0.f, 0.f, 0.f, 0.f};
                    for (int64_t ob = wfirst; ob <= wlast; ob += NB) {
                        float xg[NB][4], xu[NB][4];
#pragma unroll
                        for (int b = 0; b < NB; ++b) {
                            const int64_t ow = min(ob + b, wlast);
                            const bool first = !PERSIST || range_begin(ow, p.U, p.P) / p.C == g;
                            const float* src = p.ws + (ow * 2 + (first ? 0 : 1)) * TILEF;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                xg[b][e] = __hip_atomic_load(src + ((t * MT + j) * 4 + e) * 64 + ln, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                                xu[b][e] = SWIGLU ? __hip_atomic_load(src + (((t + RH) * MT + j) * 4 + e) * 64 + ln,
                                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                  : 0.f;
                            }
                        }
#pragma unroll
                        for (int b = 0; b < NB; ++b)
                            if (ob + b <= wlast)
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    gv[e] += xg[b][e];
                                    uv[e] += xu[b][e];
                                }
                    }
                    epilogue4<ACT, BIAS, OutT>(p.o, g * 16 * RH + t * 16 + 4 * (ln >> 4), j * 16 + (ln & 15), gv,
                                                  uv);
                }
                if (threadIdx.x == 0)
                    __hip_atomic_store(p.counters + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();  // red and is_last are reused by the next row group
        u = uend;
    }
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

// whole_k: never split K across workgroups (one workgroup per row group).
template <int MT, int RT, int NW, int U, bool PERSIST, int ACT, bool BIAS, typename OutT>
tp_status_t run(const LinearDesc& d, const Ctx& c, bool whole_k = false) {
    constexpr int RH = ACT == kActSwiglu ? RT / 2 : RT;
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
    p.o.vec16 = vec16_ok<OutT>(d.Y, d.ldy);
    p.M = (int)d.M;
    p.N = (int)d.N;
    p.K = (int)d.K;

    // Work decomposition: G row groups of 16*RH outputs, each cut into C chunks of K.
    //  * Persistent (PERSIST): chunks of NW*KS elements, one workgroup per CU, equal
    //    contiguous ranges of units.
    //  * Otherwise one unit per workgroup: K is split across workgroups only when
    //    there are fewer row groups than CUs (measured: longer per-wave streams beat
    //    a second workgroup per CU once every CU has one).
    const int64_t G = ceil_div(d.N, 16 * RH);
    int64_t C, CK, P;
    if (PERSIST) {
        CK = (int64_t)NW * KS;
        C = ceil_div(d.K, CK);
        P = std::min<int64_t>(G * C, (int64_t)device_cus());
    } else {
        const int64_t target = kWgPerCu * (int64_t)device_cus();
        int64_t S = whole_k ? 1 : ceil_div(target, G);
        const int64_t smax = std::max<int64_t>(1, d.K / (NW * KS));
        S = std::min<int64_t>(std::max<int64_t>(S, 1), std::min<int64_t>(smax, 64));
        CK = ceil_div(ceil_div(d.K, S), KS) * KS;
        C = ceil_div(d.K, CK);
        P = G * C;
    }
    p.C = (int)C;
    p.CK = (int)CK;
    p.U = G * C;
    p.P = (int)P;
    p.ws = nullptr;
    p.counters = nullptr;
    if (P != G) {  // some row group is cut: partial tiles and arrival counters
        const WsNeed need{(size_t)(P * 2 * TILEF), (size_t)G};
        if (c.planning()) {
            c.need->merge(need);
            return TP_OK;
        }
        if (!c.ws || !c.ws->covers(need)) return TP_ERR_WORKSPACE;
        p.ws = c.ws->partials;
        p.counters = c.ws->counters;
    } else if (c.planning()) {
        return TP_OK;
    }
    hipLaunchKernelGGL((skinny_kernel<MT, RT, NW, U, PERSIST, ACT, BIAS, OutT>), dim3((unsigned)P),
                       dim3(NW * 64), 0, c.stream, p);
    return hip_status();
}

template <int MT, int RT, int NW, int U, bool PERSIST, int ACT>
tp_status_t run_bias(const LinearDesc& d, const Ctx& c, bool whole_k = false) {
    const bool bias = d.b0 != nullptr;
    if (d.out_dtype == TP_DTYPE_BF16)
        return bias ? run<MT, RT, NW, U, PERSIST, ACT, true, bf16>(d, c, whole_k)
                    : run<MT, RT, NW, U, PERSIST, ACT, false, bf16>(d, c, whole_k);
    return bias ? run<MT, RT, NW, U, PERSIST, ACT, true, float>(d, c, whole_k)
                : run<MT, RT, NW, U, PERSIST, ACT, false, float>(d, c, whole_k);
}

}  // namespace

tp_status_t launch_skinny(const LinearDesc& d, const Ctx& c) {
    const int mt = (int)ceil_div(d.M, 16);
    if (d.swiglu) {
        switch (mt) {
            case 1:
                // From kPairTilesM tokens on, two gate and two up tiles per wave halve the token
                // reloads, which then cost more than the shorter weight stream per wave. Only
                // where those 32-output row groups by themselves occupy at least 80% of the CUs:
                // K is then not split, as the cross-workgroup reduction of a split costs more
                // than the reloads saved (measured on the 70B and 7B FFN shards).
                if (d.M >= kPairTilesM && ceil_div(d.N, 32) * 5 >= (int64_t)device_cus() * 4)
                    return run_bias<1, 4, 8, 2, false, kActSwiglu>(d, c, true);
                // A long weight stream (>= 640 KB per CU) is dealt in equal ranges, one workgroup
                // per CU: one workgroup per row group leaves some CUs two row groups and others
                // one (measured: 70B TP=4 at 1 token 51.4 -> 48 us; the 7B TP=2 shard, 352 KB per
                // CU, is faster with one workgroup per row group).
                if (4 * d.N * d.K >= (int64_t)device_cus() * (640 << 10))
                    return run_bias<1, 2, 8, kU1, true, kActSwiglu>(d, c);
                // Shorter streams: two 32-wide K steps per piece (measured: 7B TP=2 gate/up at 1
                // token 25.2 -> 24.2 us; four steps stay best for the plain products).
                return run_bias<1, 2, 8, 2, false, kActSwiglu>(d, c);
            case 2:  // the same choice for two token tiles (measured: 70B TP=4 at 32 tokens 68 -> 61 us)
                if (ceil_div(d.N, 32) * 5 >= (int64_t)device_cus() * 4)
                    return run_bias<2, 4, 8, 2, false, kActSwiglu>(d, c, true);
                return run_bias<2, 2, 4, 2, false, kActSwiglu>(d, c);
            case 3:  // three token tiles run as four: 1 + 1 tiles per wave reload tokens more than the
                     // padded rows cost (measured: 70B TP=4 at 48 tokens 79 -> 63 us, 7B TP=2 42 -> 35 us)
                return run_bias<4, 4, 4, kU4, true, kActSwiglu>(d, c);
            case 4: return run_bias<4, 4, 4, kU4, true, kActSwiglu>(d, c);
            default: return TP_ERR_SHAPE;
        }
    }
    auto plain = [&](auto act) -> tp_status_t {
        constexpr int A = decltype(act)::value;
        switch (mt) {
            case 1:
                // From kTwoRowsM tokens on, two row tiles per token load halve the token
                // reloads (measured: 70B TP=4 down at 16 tokens 34 -> 26 us).
                if (d.M >= kTwoRowsM) return run_bias<1, 2, 8, 2, false, A>(d, c);
                return run_bias<1, 1, 8, kU1, false, A>(d, c);
            case 2: return run_bias<2, 2, 4, 2, false, A>(d, c);
            case 3: return run_bias<3, 2, 4, 2, false, A>(d, c);
            case 4: return run_bias<4, 4, 4, kU4, true, A>(d, c);
            default: return TP_ERR_SHAPE;
        }
    };
    return d.gelu ? plain(std::integral_constant<int, kActGelu>{}) : plain(std::integral_constant<int, kActNone>{});
}

}  // namespace tp
