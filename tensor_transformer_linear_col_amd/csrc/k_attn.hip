// Head-local attention core of one shard: A_r = [O_0 | O_1 | ...] with
//   O_h = softmax(Q_h K_g^T / sqrt(d), causal mask) V_g,  g = h / (hq / hk),
// read straight out of the shard's QKV_r ([M, (hq + 2 hk) d], segments Q | K | V), or,
// for a decode step, with K and V from the shard's cache (the new tokens at the end).
// Heads go to different GPUs ("What is tensor parallelism?", section "How a layer is
// split"), so the core needs nothing from other shards; its formula is not on the
// pages (scaled dot-product attention, causal, grouped-query: a reading).
//
// One workgroup = 8 waves = 128 query rows: 128 tokens of one query head (prefill), or
// (token, head) pairs of one KV group (decode: the group's heads share every K/V block).
// The keys of long query blocks are cut into ranges of their own workgroups whose
// partial results are merged afterwards (by the last to arrive, or by a merge kernel).
// Waves w and w + 4 own the
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
#include <algorithm>
#include <vector>
#include <type_traits>

#include "tp_internal.h"

namespace tp {
namespace {

struct AttnParams {
    const bf16* q;  // query rows: token i, head h at q + i * ldq + h * d
    const bf16* k;  // key rows: position t of KV head g at k + t * ldk + g * d
    const bf16* v;  // value rows: position t of KV head g at v + t * ldv + g * d
    bf16* out;      // A: token i, head h at out + i * lda + h * d
    int64_t ldq, ldk, ldv, lda;
    int M;     // query tokens, at positions pos0 .. pos0 + M - 1
    int Nk;    // keys (positions 0 .. Nk - 1)
    int pos0;  // position of query token 0 (Nk - M)
    int hq, hk;
    float scale_log2;  // log2(e) / sqrt(d)
    // A workgroup holds 128 query rows of one query block: PACK = false, 128 tokens of one
    // query head; PACK = true (few tokens, e.g. decode), rows = (token, head) pairs of one
    // KV group, row r = token r / Gq, head g * Gq + r % Gq (Gq = hq / hk), so the group's
    // query heads share every K/V block. The keys of a query block (nkb blocks of 64)
    // are cut in ceil(nkb / L) near-equal ranges, one workgroup each (L = 0: no cut);
    // each leaves its unnormalised partial in ws, and the last of a query block to
    // arrive merges them in range order and stores.
    // With PACK the ranges leave their partials with plain stores and attn_merge_kernel, the
    // next launch, merges them: O^T rows at ws[slot][row][d], (m, l) at ws[ml_off + (slot *
    // 128 + row) * 2].
    int L;
    float* ws;          // partial slots: (slot of the range) * (heads or KV groups) + head or group
    unsigned* counters; // one arrival counter per (query block, head) (without PACK)
    int64_t ml_off;
    // Without PACK and with cut blocks: the workgroups' (query block, range) pairs, largest
    // range first (entry = 4 * block + range; heads are the minor index of blockIdx), so
    // the hardware's in-order dispatch schedules the longest work first. nord = 0: the
    // order of the scalar walk below.
    int nord;
    unsigned short ord[768];
};

constexpr int KB = 64;  // keys per block

// 16 bytes at byte offset off of a raw buffer descriptor over [base, base + bytes): a lane
// whose offset lies past the end reads zeros instead of touching memory (the bound check
// covers the per-lane offset, so the whole offset is passed there). The descriptor type
// exists only for the GPU target, so the body is compiled in the device pass alone.
__device__ __forceinline__ bf16x8 load16(const void* base, uint32_t bytes, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
#else
    return bf16x8{};
#endif
}

// Max and sum of a value over the two lane halves that hold one query (lanes i and i ^ 32):
// one cross-half swap of the register (lanes 0..31 then hold the upper half's values and
// the others the lower half's) instead of an LDS permute. Both halves get the same bits.
__device__ __forceinline__ float halves_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Storage position of key k of a block in the transposed V tile (see above).
__device__ __forceinline__ int vpos(int k) {
    const int g = (k >> 2) & 3;
    return (k & ~15) | ((((g & 1) << 1) | (g >> 1)) << 2) | (k & 3);
}

template <int D, bool CAUSAL, bool PACK, int WQ>
__global__ __launch_bounds__(128 * WQ, 2) void attn_kernel(AttnParams p) {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int QB = 32 * WQ;            // query rows per workgroup
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
    constexpr int NR = NB * 16 + 2;        // floats per lane of a partial: O^T, m, l
    // LDS: two block buffers; after the loop the same bytes hold the merge data.
    constexpr int MERGEB = WQ * 64 * NR * 4;
    constexpr int LDSB = 2 * STG > MERGEB ? 2 * STG : MERGEB;
    __shared__ __attribute__((aligned(16))) char lds[LDSB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wq = wave % WQ, kh = wave / WQ;  // query slice, key half
    const int l32 = lane & 31, lh = lane >> 5;
    const int gq = p.hq / p.hk;                       // query heads per KV head
    const int HM = PACK ? p.hk : p.hq;                // workgroups per query block
    const int rows = PACK ? p.M * gq : p.M;           // query rows of one workgroup column
    const int nqb = (rows + QB - 1) / QB;
    // Last query token of query block b and the keys it needs.
    auto last_tok = [&](int b) { return PACK ? min(p.M - 1, ((b + 1) * QB - 1) / gq) : min(p.M - 1, (b + 1) * QB - 1); };
    auto kend_of = [&](int b) { return CAUSAL ? min(p.Nk, p.pos0 + last_tok(b) + 1) : p.Nk; };

    // Workgroup -> (head or KV group, query block, key range): blockIdx = piece * HM + hm.
    // With an order table the piece is ord[blockIdx / HM] (slots: four per query block);
    // otherwise pieces are enumerated from the last (longest, when causal) query block down
    // and, within one, in key order (base = the slot of this query block's first piece).
    const int hm = blockIdx.x % HM;
    int qblk, np = 1, part = 0, base = 0;
    if (!PACK && p.nord > 0) {
        const int e = p.ord[blockIdx.x / HM];
        qblk = e >> 2;
        part = e & 3;
        np = (kend_of(qblk) - 1) / KB / p.L + 1;  // ceil(nkb / L)
        base = 4 * qblk;                           // partial slots: four per query block
    } else {
        int b = blockIdx.x / HM;
        if (p.L > 0) {
            // A scalar walk over the query blocks; its length grows like L, i.e. like the
            // work of every piece, so its share stays small.
            for (qblk = nqb - 1;; --qblk) {
                np = ((kend_of(qblk) - 1) / KB + p.L) / p.L;  // ceil(nkb / L)
                if (b < np) break;
                b -= np;
                base += np;
            }
            part = b;
        } else {
            qblk = nqb - 1 - b;
        }
    }
    const int g = PACK ? hm : hm / gq;  // KV head
    const int row = qblk * QB + wq * 32 + l32;         // this lane's query row
    const int qi = PACK ? row / gq : row;              // its token
    const int h = PACK ? g * gq + row % gq : hm;       // its query head
    const int qpos = p.pos0 + qi;                      // its position
    // This wave's last token (rows past the end count as the last token).
    const int wlast = PACK ? min(p.M - 1, (qblk * QB + wq * 32 + 31) / gq) : min(p.M - 1, qblk * QB + wq * 32 + 31);
    const int wfirst = PACK ? (qblk * QB + wq * 32) / gq : qblk * QB + wq * 32;
    const bf16* K = p.k + (int64_t)g * D;
    const bf16* V = p.v + (int64_t)g * D;
    const float c = p.scale_log2;
    const float thr = 8.f / c;  // raw-score margin before m is raised

    // The wave's queries as the B operand of S^T: chunk j holds d 16j + 8lh .. +7.
    bf16x8 qf[NC];
    {
        const bf16* qrow = p.q + (int64_t)min(qi, p.M - 1) * p.ldq + (int64_t)h * D + 8 * lh;
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

    // Key blocks: all keys, or (causal) those up to the block's last query.
    const int nkb_all = (kend_of(qblk) + KB - 1) / KB;
    const int kb0 = part * nkb_all / np;
    const int nkb = (part + 1) * nkb_all / np;  // this workgroup's blocks: [kb0, nkb)
    // This wave needs keys < wave_kend; a wave whose rows all lie past the last token needs none.
    const int wave_kend = wfirst >= p.M ? 0 : CAUSAL ? min(p.Nk, p.pos0 + wlast + 1) : p.Nk;

    // Global -> registers through buffer loads whose bound is the end of the last key (or
    // value) row, so keys past Nk read as zeros (they are masked below) and never touch
    // memory past the operand; the per-thread offsets are fixed, plus the block's row offset.
    // K: chunk i of thread t is key (t + NT i) / (D/8), d offset 8 * ((t + NT i) % (D/8))
    // (rows read whole). V: thread t holds keys R*kg .. R*kg+R-1 (kg = t % NKG) at
    // d 8*dv .. 8*dv+7 (dv = t / NKG), ready to be written transposed.
    const int kg = tid % NKG, dv = tid / NKG;
    const uint32_t k_bytes = (uint32_t)(((int64_t)(p.Nk - 1) * p.ldk + D) * 2);
    const uint32_t v_bytes = (uint32_t)(((int64_t)(p.Nk - 1) * p.ldv + D) * 2);
    uint32_t koff[CK], voff[R];
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const int ch = tid + NT * i;
        koff[i] = (uint32_t)(((ch / (D / 8)) * p.ldk + 8 * (ch % (D / 8))) * 2);
    }
#pragma unroll
    for (int j = 0; j < R; ++j) voff[j] = (uint32_t)(((R * kg + j) * p.ldv + 8 * dv) * 2);
    bf16x8 kr[CK], vr[R];
    auto fetch = [&](int kb) {
        const uint32_t ko = (uint32_t)(kb * KB * p.ldk * 2), vo = (uint32_t)(kb * KB * p.ldv * 2);
#pragma unroll
        for (int i = 0; i < CK; ++i) kr[i] = load16(K, k_bytes, koff[i] + ko);
#pragma unroll
        for (int j = 0; j < R; ++j) vr[j] = load16(V, v_bytes, voff[j] + vo);
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

            // Masks (keys past Nk; causal: keys after the query's position), only where a key
            // can fail them.
            if (k0 + 32 > p.Nk || (CAUSAL && k0 + 31 > p.pos0 + wfirst)) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = k0 + 8 * (e / 4) + 4 * lh + (e % 4);
                    const bool ok = key < p.Nk && (!CAUSAL || key <= qpos);
                    s[e] = ok ? s[e] : -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
            mx = halves_max(mx);
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
    l_run = halves_sum(l_run);
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
    // valid key has m = -inf and l = 0: weight 0.
    auto merge = [&](float m2, float l2, auto&& other) {
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

    if (PACK && np > 1) {
        // Decode: this range's partial goes out with plain stores; attn_merge_kernel merges
        // all ranges of the query block at once (a kernel boundary orders the two).
        if (kh == 0 && wfirst < p.M) {
            const int64_t sl = (int64_t)(base + part) * HM + hm;
            const int r = wq * 32 + l32;
            float* o = p.ws + (sl * QB + r) * D;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<floatx4*>(o + 32 * b + 8 * q + 4 * lh) =
                        floatx4{acc[b][4 * q], acc[b][4 * q + 1], acc[b][4 * q + 2], acc[b][4 * q + 3]};
            if (lh == 0) {
                p.ws[p.ml_off + (sl * QB + r) * 2] = m_run;
                p.ws[p.ml_off + (sl * QB + r) * 2 + 1] = l_run;
            }
        }
        return;
    }
    if (np > 1) {
        // Cut query block: leave this range's partial in the workgroup's slot; the last
        // workgroup of the block to arrive merges all of them in key order (so the result
        // does not depend on the arrival order). The partials move only through
        // device-scope atomic stores and loads, coherent across the XCDs' L2 caches by
        // themselves; waiting for the stores before the arrival counter is incremented
        // orders them.
        __shared__ unsigned is_last;
        auto slot = [&](int part_) { return p.ws + ((int64_t)(base + part_) * HM + hm) * (WQ * 64 * NR) + wq * 64 * NR; };
        const int unit = (nqb - 1 - qblk) * HM + hm;
        if (kh == 0) {
            float* mine = slot(part);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    __hip_atomic_store(mine + (b * 16 + e) * 64 + lane, acc[b][e], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(mine + NB * 16 * 64 + lane, m_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(mine + (NB * 16 + 1) * 64 + lane, l_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);  // vmcnt = expcnt = lgkmcnt = 0: stores acknowledged
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = __hip_atomic_fetch_add(p.counters + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            is_last = prev == (unsigned)(np - 1) ? 1u : 0u;
            if (is_last) __hip_atomic_store(p.counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!is_last) return;
        if (kh == 0) {
            auto ld = [&](const float* src, int r) {
                return __hip_atomic_load(src + r * 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            };
            const float* s0 = slot(0);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[b][e] = ld(s0, b * 16 + e);
            m_run = ld(s0, NB * 16);
            l_run = ld(s0, NB * 16 + 1);
            for (int q = 1; q < np; ++q) {
                const float* sq = slot(q);
                merge(ld(sq, NB * 16), ld(sq, NB * 16 + 1), [&](int r) { return ld(sq, r); });
            }
        }
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

constexpr int kWQ = 4;  // query slices per workgroup: 128 query rows, 8 waves

// Merge of the key ranges of cut packed query blocks: one workgroup per (query block, KV
// head, row); thread (j, d4) takes the ranges q = j, j + 8, ... (independent loads, all in
// flight at once) for 4 consecutive d, merging them online in that order; the 8 partial
// results then meet through LDS in j order. Fixed order throughout, one division by the
// merged sum, one rounding.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p, int nqb) {
    constexpr int QB = 32 * kWQ, NJ = 256 / (D / 4);  // range lanes: 8 (D = 128) or 16 (D = 64)
    __shared__ float sm[NJ], sl_[NJ];
    __shared__ floatx4 so[NJ][D / 4];
    const int gq = p.hq / p.hk, HM = p.hk;
    const int d4 = threadIdx.x % (D / 4), j = threadIdx.x / (D / 4);
    const int row = blockIdx.x % QB;
    const int u = blockIdx.x / QB;
    const int hm = u % HM, qblk = nqb - 1 - u / HM;
    const int grow = qblk * QB + row;
    const int tok = grow / gq, h = hm * gq + grow % gq;
    if (tok >= p.M) return;  // uniform per workgroup
    auto np_of = [&](int b) {
        const int last = min(p.M - 1, ((b + 1) * QB - 1) / gq);
        return ((min(p.Nk, p.pos0 + last + 1) - 1) / KB + p.L) / p.L;
    };
    int base = 0;
    for (int b = nqb - 1; b > qblk; --b) base += np_of(b);
    const int np = np_of(qblk);
    if (np <= 1) return;  // an uncut query block stored its own result
    const float c = p.scale_log2;
    // Merge (m2, l2, o2) into (m, l, o); a part that saw no valid key (m = -inf, l = 0) has weight 0.
    auto merge = [&](float& m, float& l, floatx4& o, float m2, float l2, const floatx4& o2) {
        const float mn = fmaxf(m, m2);
        const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * c);
        const float w = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m2 - mn) * c);
        l = l * a + l2 * w;
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = o[t] * a + o2[t] * w;
        m = mn;
    };
    float m = -INFINITY, l = 0.f;
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int q = j; q < np; q += NJ) {
        const int64_t sl = (int64_t)(base + q) * HM + hm;
        merge(m, l, o, p.ws[p.ml_off + (sl * QB + row) * 2], p.ws[p.ml_off + (sl * QB + row) * 2 + 1],
              *reinterpret_cast<const floatx4*>(p.ws + (sl * QB + row) * D + 4 * d4));
    }
    if (d4 == 0) {
        sm[j] = m;
        sl_[j] = l;
    }
    so[j][d4] = o;
    __syncthreads();
    if (j != 0) return;
    for (int jj = 1; jj < NJ; ++jj) merge(m, l, o, sm[jj], sl_[jj], so[jj][d4]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const bf16x4 v = {(bf16)(o[0] * inv), (bf16)(o[1] * inv), (bf16)(o[2] * inv), (bf16)(o[3] * inv)};
    *reinterpret_cast<bf16x4*>(p.out + (int64_t)tok * p.lda + (int64_t)h * D + 4 * d4) = v;
}

// Appends M new tokens' K and V rows (QKV columns hq*d.. and (hq+hk)*d.., hk*d wide each) to
// the caches at row T, in 16-byte units: one grid-stride pass over both copies.
__global__ __launch_bounds__(256) void append_kv_kernel(const bf16* qkv, int64_t ldq, int64_t koff, int64_t voff,
                                                        bf16* kc, bf16* vc, int64_t ldkv, int64_t T, int64_t M) {
    const int64_t per_row = ldkv / 8;  // 16-byte units per cache row
    const int64_t total = 2 * M * per_row;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t which = i / (M * per_row), j = i - which * M * per_row;
        const int64_t r = j / per_row, u = j - r * per_row;
        const bf16* src = qkv + r * ldq + (which ? voff : koff) + 8 * u;
        bf16* dst = (which ? vc : kc) + (T + r) * ldkv + 8 * u;
        *reinterpret_cast<bf16x8*>(dst) = *reinterpret_cast<const bf16x8*>(src);
    }
}

int device_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
        return n;
    return 256;
}

template <int D, bool CAUSAL, bool PACK>
tp_status_t run_attn(AttnParams p, hipStream_t stream) {
    constexpr int QB = 32 * kWQ;
    const int gq = p.hq / p.hk;
    const int HM = PACK ? p.hk : p.hq;
    const int rows = PACK ? p.M * gq : p.M;
    const int nqb = (rows + QB - 1) / QB;
    auto kend_of = [&](int b) {
        const int last = PACK ? std::min(p.M - 1, ((b + 1) * QB - 1) / gq) : std::min(p.M - 1, (b + 1) * QB - 1);
        return CAUSAL ? std::min(p.Nk, p.pos0 + last + 1) : p.Nk;
    };
    // Cutting keys: causal prefill, where a query block's work grows with its index, cuts
    // every block into ranges of at most a third of the longest, which bounds every
    // workgroup's share (the ranges then run largest first, see ord); few query blocks
    // (decode) cut their keys so that the grid has about one workgroup per CU.
    const int nkb_max = (kend_of(nqb - 1) + KB - 1) / KB;
    p.L = 0;
    if (PACK) {
        // About one workgroup per CU, at most 128 ranges per query block (the merge reads
        // up to 16 ranges per thread).
        const int want = std::min(128, std::max(1, (device_cu_count() + nqb * HM - 1) / (nqb * HM)));
        p.L = std::max(1, (nkb_max + want - 1) / want);
        if (p.L >= nkb_max) p.L = 0;
    } else if (CAUSAL && nqb >= 4) {
        p.L = (nkb_max + 2) / 3;  // at most 3 ranges (measured: 2 and 4 ranges are slower)
    }
    p.ws = nullptr;
    p.counters = nullptr;
    int64_t pieces = nqb;
    if (p.L > 0) {
        pieces = 0;
        for (int b = 0; b < nqb; ++b) pieces += ((kend_of(b) - 1) / KB + p.L) / p.L;
        // Partials: without PACK one slot of WQ x 64 lanes x (D/2 + 2) floats per workgroup;
        // with PACK 128 rows x (D + 2) floats.
        const int64_t slots = PACK ? pieces : std::max<int64_t>(pieces, 4 * (int64_t)nqb);
        const size_t floats = (size_t)(slots * HM) * (PACK ? QB * (D + 2) : kWQ * 64 * (D / 2 + 2));
        Workspace ws;
        const tp_status_t st = get_workspace(stream, floats, (size_t)nqb * HM, &ws);
        if (st != TP_OK) return st;
        p.ws = ws.partials;
        p.counters = ws.counters;
        p.ml_off = (int64_t)pieces * HM * QB * D;
    }
    // Causal prefill: largest ranges first (a cut block's halves are about half as long as
    // an uncut block of the same index, so the plain walk would queue long uncut blocks
    // behind short halves).
    p.nord = 0;
    if (!PACK && p.L > 0 && pieces <= (int64_t)(sizeof(p.ord) / sizeof(p.ord[0]))) {
        struct Piece { int size, e; };
        std::vector<Piece> v;
        for (int b = nqb - 1; b >= 0; --b) {
            const int nkb = (kend_of(b) - 1) / KB + 1;
            const int np = (nkb - 1) / p.L + 1;
            for (int q = 0; q < np; ++q) v.push_back({(q + 1) * nkb / np - q * nkb / np, 4 * b + q});
        }
        std::stable_sort(v.begin(), v.end(), [](const Piece& a, const Piece& b) { return a.size > b.size; });
        for (size_t i = 0; i < v.size(); ++i) p.ord[i] = (unsigned short)v[i].e;
        p.nord = (int)v.size();
    }
    hipLaunchKernelGGL((attn_kernel<D, CAUSAL, PACK, kWQ>), dim3((unsigned)(pieces * HM)), dim3(128 * kWQ), 0,
                       stream, p);
    if (PACK && p.L > 0) {
        const tp_status_t st = hip_status();
        if (st != TP_OK) return st;
        hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)(nqb * HM * QB)), dim3(256), 0, stream, p, nqb);
    }
    return hip_status();
}

template <bool PACK>
tp_status_t run_attn_d(const AttnParams& p, int d, bool causal, hipStream_t stream) {
    if (d == 128) return causal ? run_attn<128, true, PACK>(p, stream) : run_attn<128, false, PACK>(p, stream);
    if (d == 64) return causal ? run_attn<64, true, PACK>(p, stream) : run_attn<64, false, PACK>(p, stream);
    return TP_ERR_SHAPE;
}

}  // namespace

tp_status_t launch_attn_core(const void* qkv, int64_t ldq, void* out, int64_t lda, int64_t M, int hq, int hk, int d,
                             bool causal, hipStream_t stream) {
    // Buffer offsets are 32-bit: the K and V column blocks must lie within 2 GiB.
    if (M * ldq * 2 >= (int64_t(1) << 31)) return TP_ERR_SHAPE;
    AttnParams p;
    const bf16* base = static_cast<const bf16*>(qkv);
    p.q = base;
    p.k = base + (int64_t)hq * d;
    p.v = base + (int64_t)(hq + hk) * d;
    p.out = static_cast<bf16*>(out);
    p.ldq = p.ldk = p.ldv = ldq;
    p.lda = lda;
    p.M = p.Nk = (int)M;
    p.pos0 = 0;
    p.hq = hq;
    p.hk = hk;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
    return run_attn_d<false>(p, d, causal, stream);
}

tp_status_t launch_attn_decode(const void* qkv, int64_t ldq, void* kc, void* vc, int64_t ldkv, int64_t cache_len,
                               void* out, int64_t lda, int64_t M, int hq, int hk, int d, hipStream_t stream) {
    const int64_t n_keys = cache_len + M;
    if (n_keys * ldkv * 2 >= (int64_t(1) << 31)) return TP_ERR_SHAPE;
    const int64_t units = 2 * M * (ldkv / 8);
    const unsigned grid = (unsigned)std::min<int64_t>((units + 255) / 256, 4096);
    hipLaunchKernelGGL(append_kv_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const bf16*>(qkv), ldq,
                       (int64_t)hq * d, (int64_t)(hq + hk) * d, static_cast<bf16*>(kc), static_cast<bf16*>(vc), ldkv,
                       cache_len, M);
    const tp_status_t st = hip_status();
    if (st != TP_OK) return st;
    AttnParams p;
    p.q = static_cast<const bf16*>(qkv);
    p.k = static_cast<const bf16*>(kc);
    p.v = static_cast<const bf16*>(vc);
    p.out = static_cast<bf16*>(out);
    p.ldq = ldq;
    p.ldk = p.ldv = ldkv;
    p.lda = lda;
    p.M = (int)M;
    p.Nk = (int)n_keys;
    p.pos0 = (int)cache_len;
    p.hq = hq;
    p.hk = hk;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
    return run_attn_d<true>(p, d, true, stream);
}

}  // namespace tp
