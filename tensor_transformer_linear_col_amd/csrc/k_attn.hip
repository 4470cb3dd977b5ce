// Head-local attention core of one shard: A_r = [O_0 | O_1 | ...] with
//   O_h = softmax(Q_h K_g^T / sqrt(d), causal mask) V_g,  g = h / (hq / hk),
// read straight out of the shard's QKV_r ([M, (hq + 2 hk) d], segments Q | K | V).
// Heads go to different GPUs ("What is tensor parallelism?", section "How a layer is
// split"), so the core needs nothing from other shards; its formula is not on the
// pages (scaled dot-product attention, causal, grouped-query: a reading).
//
// One workgroup = 4 waves = 128 query rows of one query head; each wave owns 32
// queries. Keys and values stream through LDS 32 at a time (the next block is
// prefetched into registers while the current one is used); all four waves share
// each block. Per block and wave:
//   S^T = K Q^T on MFMA 32x32x16 bf16 (A = 32 keys from LDS, B = the wave's 32 queries,
//       held in registers for the whole loop), so each lane holds 16 scores of one
//       query: register e <-> key 8*(e/4) + 4*lh + e%4 (lh = lane / 32);
//   online softmax per query in the log2 domain (running max m, running sum l; the
//       two lane halves sharing a query exchange their maxima);
//   O^T += V^T P^T on MFMA, P^T straight from the score registers as the B operand.
//       An MFMA reduces its 16 K positions in any order, so B may hold a lane's keys
//       as they come; the A operand (V^T, stored transposed in LDS) supplies the same
//       keys at the same positions: lane half lh, step s: keys 16s + 4lh + {0..3},
//       then 16s + 8 + 4lh + {0..3}.
// O^T registers hold one query per lane, so the rescale by exp2(m_old - m_new) and
// the final 1/l are per-lane scalars. Softmax and accumulation are fp32; A_r is
// rounded once to bf16.
#include <type_traits>

#include "tp_internal.h"

namespace tp {
namespace {

struct AttnParams {
    const bf16* qkv;  // [M, ldq]
    int64_t ldq;
    bf16* out;        // [M, lda]
    int64_t lda;
    int M, hq, hk;
    float scale_log2;  // log2(e) / sqrt(d)
};

constexpr int QB = 128;  // queries per workgroup (4 waves x 32)
constexpr int KB = 32;   // keys per block

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int KP = D * 2 + 16;        // K tile row pitch (bytes): 16-byte pad
    constexpr int VP = KB * 2 + 8;        // V^T tile row pitch (bytes): 8-byte pad
    constexpr int NC = D / 16;            // 16-wide d chunks (MFMA K steps of S)
    constexpr int NB = D / 32;            // 32-row d blocks of O^T
    constexpr int CH = KB * D / 8 / 256;  // 16-byte chunks of K (and of V) per thread per block
    __shared__ __attribute__((aligned(16))) char ks[KB * KP];
    __shared__ __attribute__((aligned(16))) char vts[D * VP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const int nqb = (p.M + QB - 1) / QB;
    // The longest (causal) query blocks first.
    const int h = blockIdx.x % p.hq;
    const int qblk = CAUSAL ? nqb - 1 - (int)(blockIdx.x / p.hq) : (int)(blockIdx.x / p.hq);
    const int g = h / (p.hq / p.hk);
    const int q0 = qblk * QB, qw = q0 + wave * 32;
    const int qi = qw + l32;  // this lane's query
    const bf16* Q = p.qkv + (int64_t)h * D;
    const bf16* K = p.qkv + (int64_t)(p.hq + g) * D;
    const bf16* V = p.qkv + (int64_t)(p.hq + p.hk + g) * D;

    // The wave's queries as the B operand of S^T: chunk c holds d 16c + 8lh .. +7.
    bf16x8 qf[NC];
    {
        const bf16* qrow = Q + (int64_t)min(qi, p.M - 1) * p.ldq + 8 * lh;
#pragma unroll
        for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c);
    }

    floatx16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // Key blocks: all keys of the sequence, or (causal) those up to the block's last query.
    const int kend = CAUSAL ? min(p.M, q0 + QB) : p.M;
    const int nkb = (kend + KB - 1) / KB;
    const int wave_kend = CAUSAL ? min(p.M, qw + 32) : p.M;  // this wave needs keys < wave_kend

    // Global -> register prefetch of one block: thread chunk i covers key (t + 256 i) / (D/8),
    // d offset 8 * ((t + 256 i) % (D/8)). Keys past M are clamped (masked below).
    bf16x8 kr[CH], vr[CH];
    auto fetch = [&](int kb) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + 256 * i;
            const int key = min(kb * KB + c / (D / 8), p.M - 1);
            const int64_t off = (int64_t)key * p.ldq + 8 * (c % (D / 8));
            kr[i] = *reinterpret_cast<const bf16x8*>(K + off);
            vr[i] = *reinterpret_cast<const bf16x8*>(V + off);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + 256 * i;
            const int key = c / (D / 8), d0 = 8 * (c % (D / 8));
            *reinterpret_cast<bf16x8*>(ks + key * KP + d0 * 2) = kr[i];
#pragma unroll
            for (int e = 0; e < 8; ++e) *reinterpret_cast<bf16*>(vts + (d0 + e) * VP + key * 2) = vr[i][e];
        }
    };

    if (nkb > 0) fetch(0);
    for (int kb = 0; kb < nkb; ++kb) {
        __syncthreads();  // every wave is done with the previous block's tiles
        stage();
        __syncthreads();
        if (kb + 1 < nkb) fetch(kb + 1);
        const int k0 = kb * KB;
        if (k0 >= wave_kend) continue;  // uniform per wave: past this wave's last query

        // S^T = K Q^T
        floatx16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + l32 * KP + (16 * c + 8 * lh) * 2);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s, 0, 0, 0);
        }

        // Mask (keys past M; causal: keys after the query), scale, online softmax.
        float t[16];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = k0 + 8 * (e / 4) + 4 * lh + (e % 4);
            const bool ok = key < p.M && (!CAUSAL || key <= qi);
            t[e] = ok ? s[e] * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, t[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        // A query with no valid key yet (m_new = -inf) keeps zeros; exp2(-inf) = 0.
        const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
        bf16x8 pf[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float pe = m_new == -INFINITY ? 0.f : exp2f(t[e] - m_new);
            l_run += pe;
            pf[e / 8][e % 8] = (bf16)pe;
        }
        m_run = m_new;

        // O^T += V^T P^T
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const char* row = vts + (32 * b + l32) * VP;
                const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + (16 * st + 4 * lh) * 2);
                const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + (16 * st + 8 + 4 * lh) * 2);
                const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st], acc[b], 0, 0, 0);
            }
    }

    // O = O^T / l for this lane's query; 4 consecutive d per store.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qi >= p.M) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16* orow = p.out + (int64_t)qi * p.lda + (int64_t)h * D;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bf16x4 v = {(bf16)(acc[b][4 * q] * inv), (bf16)(acc[b][4 * q + 1] * inv),
                              (bf16)(acc[b][4 * q + 2] * inv), (bf16)(acc[b][4 * q + 3] * inv)};
            *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * q + 4 * lh) = v;
        }
}

template <int D, bool CAUSAL>
tp_status_t run_attn(const AttnParams& p, hipStream_t stream) {
    const int nqb = (p.M + QB - 1) / QB;
    hipLaunchKernelGGL((attn_kernel<D, CAUSAL>), dim3((unsigned)(nqb * p.hq)), dim3(256), 0, stream, p);
    return hip_status();
}

}  // namespace

tp_status_t launch_attn_core(const void* qkv, int64_t ldq, void* out, int64_t lda, int64_t M, int hq, int hk, int d,
                             bool causal, hipStream_t stream) {
    AttnParams p;
    p.qkv = static_cast<const bf16*>(qkv);
    p.ldq = ldq;
    p.out = static_cast<bf16*>(out);
    p.lda = lda;
    p.M = (int)M;
    p.hq = hq;
    p.hk = hk;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
    if (d == 128) return causal ? run_attn<128, true>(p, stream) : run_attn<128, false>(p, stream);
    if (d == 64) return causal ? run_attn<64, true>(p, stream) : run_attn<64, false>(p, stream);
    return TP_ERR_SHAPE;
}

}  // namespace tp
