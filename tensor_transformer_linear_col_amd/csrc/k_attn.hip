// Head-local attention core of one shard: A_r = [O_0 | O_1 | ...] with
//   O_h = softmax(Q_h K_g^T / sqrt(d), causal mask) V_g,  g = h / (hq / hk),
// read straight out of the shard's QKV_r ([M, (hq + 2 hk) d], segments Q | K | V).
// Heads go to different GPUs ("What is tensor parallelism?", section "How a layer is
// split"), so the core needs nothing from other shards; its formula is not on the
// pages (scaled dot-product attention, causal, grouped-query: a reading).
//
// One workgroup = 8 waves = 128 query rows of one query head. Waves w and w + 4 own the
// same 32 queries and split every 64-key block between them (keys 0..31 and 32..63 of
// the block), each with its own running maximum, sum and output accumulators; the two
// halves are merged once at the end. Two waves per SIMD let one wave's softmax run
// while the other's MFMAs do. Keys and values stream through LDS 64 at a time,
// double-buffered: the next block is fetched into registers while the current one is
// used and written to the other LDS buffer afterwards, so one barrier per block
// suffices; all eight waves share each block. Per block and wave:
//   S^T = K Q^T on MFMA 32x32x16 bf16 (A = the wave's 32 keys from LDS, B = its 32
//       queries, held in registers for the whole loop), so each lane holds 16 scores of
//       one query: register e <-> key 8*(e/4) + 4*lh + e%4 of the half (lh = lane / 32);
//   online softmax per query in the log2 domain, with the running maximum m raised
//       only when a score exceeds it by more than 2^8 (then the accumulators are
//       rescaled); below that the unnormalised weights stay <= 256, well inside fp32
//       and bf16 range, and the final division by l makes the result independent of
//       which m was used;
//   O^T += V^T P^T on MFMA, P^T straight from the score registers as the B operand.
//       An MFMA reduces its 16 K positions in any order, so B holds a lane's keys as
//       they come: lane half lh, step s: keys 16s + 4lh + {0..3}, then
//       16s + 8 + 4lh + {0..3}. V^T is stored transposed in LDS with the keys of each
//       16-key run in that order (4-key groups 0, 2, 1, 3), so the A operand is one
//       16-byte read per lane.
// The causal mask and the sequence-end mask are applied only on blocks that need them.
// O^T registers hold one query per lane, so the rescale, the merge and the final 1/l
// are per-lane scalars. Softmax and accumulation are fp32; A_r is rounded once to bf16.
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
    // Causal balance: the units (head, query block) of the query blocks >= qsplit are
    // cut in two key ranges handled by two workgroups (nsu such units); each leaves its
    // unnormalised partial in ws, and the second to arrive merges and stores.
    int qsplit, nsu;
    float* ws;
    unsigned* counters;
};

constexpr int KB = 64;   // keys per block

// 16 bytes at byte offset voff + soff of a raw buffer descriptor over [base, base + bytes):
// reads past the end return zeros instead of faulting. The descriptor type exists only for
// the GPU target, so the body is compiled in the device pass alone.
__device__ __forceinline__ bf16x8 load16(const void* base, uint32_t bytes, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0));
#else
    return bf16x8{};
#endif
}

// Storage position of key k of a block in the transposed V tile (see above).
__device__ __forceinline__ int vpos(int k) {
    const int g = (k >> 2) & 3;
    return (k & ~15) | ((((g & 1) << 1) | (g >> 1)) << 2) | (k & 3);
}

template <int D, bool CAUSAL, int WQ>
__global__ __launch_bounds__(128 * WQ, 2) void attn_kernel(AttnParams p) {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int QB = 32 * WQ;            // queries per workgroup
    constexpr int NT = 128 * WQ;           // threads: WQ query slices x 2 key halves
    constexpr int KP = D * 2 + 16;         // K tile row pitch (bytes): 16-byte pad
    constexpr int VP = KB * 2 + 16;        // V^T tile row pitch (bytes): 16-byte pad
    constexpr int KT = KB * KP;            // K tile bytes
    constexpr int STG = KT + D * VP;       // one buffer: K tile, then V^T tile
    constexpr int NC = D / 16;             // 16-wide d chunks (MFMA K steps of S)
    constexpr int NB = D / 32;             // 32-row d blocks of O^T
    constexpr int CK = KB * D / 8 / NT;    // 16-byte chunks of K per thread per block (2 or 1)
    constexpr int R = CK;                  // keys per thread in the V transpose
    constexpr int NKG = KB / R;            // key groups of the V transpose
    static_assert(CK >= 1 && NKG * (D / 8) == NT, "staging covers the tile");
    // LDS: two block buffers; after the loop the same bytes hold the merge data.
    constexpr int MERGEB = WQ * 64 * (NB * 16 + 2) * 4;
    constexpr int LDSB = 2 * STG > MERGEB ? 2 * STG : MERGEB;
    __shared__ __attribute__((aligned(16))) char lds[LDSB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wq = wave % WQ, kh = wave / WQ;  // query slice, key half
    const int l32 = lane & 31, lh = lane >> 5;
    const int nqb = (p.M + QB - 1) / QB;
    // Workgroup -> (head, query block, key range). The halves of the split units come
    // first, then the whole units, each from the longest (causal) query block down.
    int h, qblk, part = -1, unit = 0;
    if ((int)blockIdx.x < 2 * p.nsu) {
        const int b = blockIdx.x;
        h = b % p.hq;
        part = (b / p.hq) % 2;
        qblk = nqb - 1 - b / (2 * p.hq);
        unit = (nqb - 1 - qblk) * p.hq + h;
    } else {
        const int b = blockIdx.x - 2 * p.nsu;
        h = b % p.hq;
        qblk = p.qsplit - 1 - b / p.hq;
    }
    const int g = h / (p.hq / p.hk);
    const int q0 = qblk * QB, qw = q0 + wq * 32;
    const int qi = qw + l32;  // this lane's query
    const bf16* Q = p.qkv + (int64_t)h * D;
    const bf16* K = p.qkv + (int64_t)(p.hq + g) * D;
    const bf16* V = p.qkv + (int64_t)(p.hq + p.hk + g) * D;
    const float c = p.scale_log2;
    const float thr = 8.f / c;  // raw-score margin before m is raised

    // The wave's queries as the B operand of S^T: chunk j holds d 16j + 8lh .. +7.
    bf16x8 qf[NC];
    {
        const bf16* qrow = Q + (int64_t)min(qi, p.M - 1) * p.ldq + 8 * lh;
#pragma unroll
        for (int j = 0; j < NC; ++j) qf[j] = *reinterpret_cast<const bf16x8*>(qrow + 16 * j);
        // Consume the loads here: otherwise the wait for them lands inside the key loop,
        // where the in-order load counter would also wait for the next block's prefetch.
#pragma unroll
        for (int j = 0; j < NC; ++j) asm volatile("" ::"v"(qf[j]));
    }

    floatx16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // Key blocks: all keys of the sequence, or (causal) those up to the block's last query.
    const int kend = CAUSAL ? min(p.M, q0 + QB) : p.M;
    const int nkb_all = (kend + KB - 1) / KB;
    const int kb0 = part == 1 ? nkb_all / 2 : 0;
    const int nkb = part == 0 ? nkb_all / 2 : nkb_all;  // this workgroup's blocks: [kb0, nkb)
    const int wave_kend = CAUSAL ? min(p.M, qw + 32) : p.M;  // this wave needs keys < wave_kend

    // Global -> registers through buffer loads whose bound is the end of the last key (or
    // value) row, so keys past M read as zeros (they are masked below) and the per-thread
    // offsets are fixed: only the block's scalar row offset changes.
    // K: chunk i of thread t is key (t + NT i) / (D/8), d offset 8 * ((t + NT i) % (D/8))
    // (rows read whole). V (threads t < NVT): keys 2*kg, 2*kg + 1 (kg = t % NKG) at
    // d 8*dv .. 8*dv+7 (dv = t / NKG), ready to be written transposed.
    const int kg = tid % NKG, dv = tid / NKG;
    const uint32_t kv_bytes = (uint32_t)(((int64_t)(p.M - 1) * p.ldq + D) * 2);
    uint32_t koff[CK], voff[R];
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const int ch = tid + NT * i;
        koff[i] = (uint32_t)(((ch / (D / 8)) * p.ldq + 8 * (ch % (D / 8))) * 2);
    }
#pragma unroll
    for (int j = 0; j < R; ++j) voff[j] = (uint32_t)(((R * kg + j) * p.ldq + 8 * dv) * 2);
    bf16x8 kr[CK], vr[R];
    auto fetch = [&](int kb) {
        const uint32_t soff = (uint32_t)(kb * KB * p.ldq * 2);
#pragma unroll
        for (int i = 0; i < CK; ++i) kr[i] = load16(K, kv_bytes, koff[i], soff);
#pragma unroll
        for (int j = 0; j < R; ++j) vr[j] = load16(V, kv_bytes, voff[j], soff);
    };
    auto stage = [&](char* buf) {
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            const int ch = tid + NT * i;
            *reinterpret_cast<bf16x8*>(buf + (ch / (D / 8)) * KP + (ch % (D / 8)) * 16) = kr[i];
        }
        char* vt = buf + KT + vpos(R * kg) * 2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (R == 4) {
                const bf16x4 w = {vr[0][e], vr[1][e], vr[2][e], vr[3][e]};
                *reinterpret_cast<bf16x4*>(vt + (8 * dv + e) * VP) = w;
            } else if constexpr (R == 2) {
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const bf16x2 w = {vr[0][e], vr[1][e]};
                *reinterpret_cast<bf16x2*>(vt + (8 * dv + e) * VP) = w;
            } else {
                *reinterpret_cast<bf16*>(vt + (8 * dv + e) * VP) = vr[0][e];
            }
        }
    };

    if (kb0 < nkb) {
        fetch(kb0);
        stage(lds + (kb0 & 1) * STG);
        __syncthreads();
        if (kb0 + 1 < nkb) fetch(kb0 + 1);
    }
    for (int kb = kb0; kb < nkb; ++kb) {
        const char* ks = lds + (kb & 1) * STG;
        const char* vts = ks + KT;
        const int k0 = kb * KB + 32 * kh;  // this wave's 32 keys
        if (k0 < wave_kend) {  // uniform per wave: past this wave's last query otherwise
            // S^T = K Q^T; all K fragments are read first so the LDS latency overlaps.
            bf16x8 kf[NC];
#pragma unroll
            for (int j = 0; j < NC; ++j)
                kf[j] = *reinterpret_cast<const bf16x8*>(ks + (32 * kh + l32) * KP + (16 * j + 8 * lh) * 2);
            floatx16 s;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
            for (int j = 0; j < NC; ++j) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf[j], s, 0, 0, 0);

            // The V^T fragments do not depend on the weights: read them now so their LDS
            // latency hides under the softmax.
            bf16x8 vf[2][NB];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    vf[st][b] = *reinterpret_cast<const bf16x8*>(vts + (32 * b + l32) * VP + (32 * kh + 16 * st + 8 * lh) * 2);

            // Masks (keys past M; causal: keys after the query), only where a key can fail them.
            if (k0 + 32 > p.M || (CAUSAL && k0 + 31 > qw)) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = k0 + 8 * (e / 4) + 4 * lh + (e % 4);
                    const bool ok = key < p.M && (!CAUSAL || key <= qi);
                    s[e] = ok ? s[e] : -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // Raise m (and rescale) only when some query's maximum grew past the margin.
            if (__any(mx > m_run + thr)) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
                l_run *= alpha;
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
                m_run = m_new;
            }
            // A query with no valid key yet (m = -inf) gets weights exp2(-inf) = 0.
            const float nm = m_run == -INFINITY ? 0.f : -m_run * c;
            bf16x8 pf[2];
            float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short dependency chains
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(s[e], c, nm));
                ls[e % 4] += pe;
                pf[e / 8][e % 8] = (bf16)pe;
            }
            l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

            // O^T += V^T P^T
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st][b], pf[st], acc[b], 0, 0, 0);
        }
        if (kb + 1 < nkb) {
            // The other buffer was last read in the previous block, which every wave
            // finished before the previous barrier.
            stage(lds + ((kb + 1) & 1) * STG);
            __syncthreads();
            if (kb + 2 < nkb) fetch(kb + 2);
        }
    }

    // Merge the two key halves: wave w + WQ leaves (m, l, O^T) in LDS, wave w combines.
    // Lane order in the merge area: [wave slice][register][lane], conflict-free.
    constexpr int NR = NB * 16 + 2;  // floats per lane: O^T, m, l
    l_run += __shfl_xor(l_run, 32);
    __syncthreads();  // every wave is done with the block buffers
    float* mg = reinterpret_cast<float*>(lds) + wq * 64 * NR;
    if (kh == 1) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) mg[(b * 16 + e) * 64 + lane] = acc[b][e];
        mg[NB * 16 * 64 + lane] = m_run;
        mg[(NB * 16 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    // (m, l, O^T) of two partial results over disjoint keys -> one. A part that saw no
    // valid key has m = -inf and l = 0: weight 0. Symmetric in its two operands (products
    // rounded separately, no fused multiply-add), so the result does not depend on which is
    // "this" one, i.e. on which workgroup of a split unit arrives last.
    auto merge = [&](float m2, float l2, auto&& other) {
#pragma clang fp contract(off)
        const float mm = fmaxf(m_run, m2);
        const float a1 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - mm) * c);
        const float a2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m2 - mm) * c);
        l_run = l_run * a1 + l2 * a2;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[b][e] = acc[b][e] * a1 + other(b * 16 + e) * a2;
        m_run = mm;
    };
    if (kh == 0)
        merge(mg[NB * 16 * 64 + lane], mg[(NB * 16 + 1) * 64 + lane], [&](int r) { return mg[r * 64 + lane]; });

    if (part >= 0) {
        // Split unit: leave this half's partial in its slot, then the second workgroup to
        // arrive merges the two. The partials move only through device-scope atomic
        // stores and loads, coherent across the XCDs' L2 caches by themselves; waiting for
        // the stores before the arrival counter is incremented orders them.
        __shared__ unsigned is_last;
        float* slot = p.ws + ((int64_t)unit * 2 + part) * (WQ * 64 * NR) + wq * 64 * NR;
        if (kh == 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    __hip_atomic_store(slot + (b * 16 + e) * 64 + lane, acc[b][e], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(slot + NB * 16 * 64 + lane, m_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(slot + (NB * 16 + 1) * 64 + lane, l_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);  // vmcnt = expcnt = lgkmcnt = 0: stores acknowledged
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = __hip_atomic_fetch_add(p.counters + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            is_last = prev == 1u ? 1u : 0u;
            if (prev == 1u) __hip_atomic_store(p.counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!is_last) return;
        const float* other = p.ws + ((int64_t)unit * 2 + (1 - part)) * (WQ * 64 * NR) + wq * 64 * NR;
        auto ld = [&](int r) { return __hip_atomic_load(other + r * 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        if (kh == 0) merge(ld(NB * 16), ld(NB * 16 + 1), ld);
    }
    if (kh == 1 || qi >= p.M) return;

    // O = O^T / l for this lane's query; 4 consecutive d per store.
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
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

constexpr int kWQ = 4;  // query slices per workgroup: 128 queries, 8 waves

template <int D, bool CAUSAL>
tp_status_t run_attn(AttnParams p, hipStream_t stream) {
    constexpr int QB = 32 * kWQ;
    const int nqb = (p.M + QB - 1) / QB;
    // Causal: a query block's work grows with its index. Cutting the upper half of the
    // blocks in two key ranges bounds every workgroup's share by about the longest
    // whole block's half, so the grid drains evenly.
    p.qsplit = CAUSAL && nqb >= 4 ? nqb / 2 : nqb;
    p.nsu = (nqb - p.qsplit) * p.hq;
    p.ws = nullptr;
    p.counters = nullptr;
    if (p.nsu > 0) {
        Workspace ws;
        const tp_status_t st = get_workspace(stream, (size_t)p.nsu * 2 * kWQ * 64 * (D / 2 + 2), (size_t)p.nsu, &ws);
        if (st != TP_OK) return st;
        p.ws = ws.partials;
        p.counters = ws.counters;
    }
    hipLaunchKernelGGL((attn_kernel<D, CAUSAL, kWQ>), dim3((unsigned)(2 * p.nsu + p.qsplit * p.hq)), dim3(128 * kWQ), 0,
                       stream, p);
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
    // Buffer offsets are 32-bit: the K and V column blocks must lie within 2 GiB.
    if (M * ldq * 2 >= (int64_t(1) << 31)) return TP_ERR_SHAPE;
    if (d == 128) return causal ? run_attn<128, true>(p, stream) : run_attn<128, false>(p, stream);
    if (d == 64) return causal ? run_attn<64, true>(p, stream) : run_attn<64, false>(p, stream);
    return TP_ERR_SHAPE;
}

}  // namespace tp
