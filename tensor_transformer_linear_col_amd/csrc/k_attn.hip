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
// double-buffered, by DMA (buffer loads that write LDS directly, no registers): the next
// block is requested into the other buffer right after the barrier that frees it and
// lands while the current one is used, so one barrier per block suffices; all eight
// waves share each block. K and V rows sit in LDS as loaded (one row per key), their
// 16-byte chunks XOR-swizzled by row so that the fragment reads below hit distinct
// banks. Per block and wave:
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
//       16s + 8 + 4lh + {0..3}. The A operand (one head-dim row of V^T per lane, those
//       8 keys) comes from V's key rows through gfx950's LDS transpose read: within
//       each 16-lane group, output lane 4a + b receives element b of the 8 bytes read
//       by lanes a, a + 4, a + 8 and a + 12. With source lane 4r + a pointing at key
//       r of a 4-key run, head-dim columns 4a .. 4a + 3 of a 16-column group, output
//       lane i gets column i of the group across the 4 keys; two such reads per
//       fragment give the 8 keys above.
// The causal mask and the sequence-end mask are applied only on blocks that need them.
// O^T registers hold one query per lane, so the rescale, the merge and the final 1/l
// are per-lane scalars. Softmax and accumulation are fp32; each weight P is rounded to
// bf16 where it becomes the P*V product's MFMA operand (the normaliser l sums the fp32
// weights), and A_r is rounded once to bf16.
#include <algorithm>
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
    // query heads share every K/V block.
    // PACK: the keys of a query block (nkb blocks of 64) are cut in ceil(nkb / L) near-equal
    // ranges, one workgroup each (L = 0: no cut); each leaves its unnormalised partial with
    // plain stores and attn_merge_kernel, the next launch, merges them: O^T rows at
    // ws[slot][row][d], (m, l) at ws[ml_off + (slot * 128 + row) * 2].
    // Without PACK, L > 0: the same cut, one workgroup per range; a query block's ranges
    // leave their unnormalised partials in ws and the last of them to arrive merges them in
    // key order. With an order table the workgroups take the ranges largest first (entry =
    // 4 * block + range, heads the minor index of blockIdx), so the hardware's in-order
    // dispatch approximates longest-processing-time scheduling.
    // Without PACK, nwg > 0: the work is U key blocks in a fixed order (head-major; within a
    // head the query blocks in pairs nqb - 1, 0, nqb - 2, 1, ..., each in key order), and
    // workgroup i takes the contiguous run [i U / nwg, (i + 1) U / nwg): every workgroup the
    // same work, one per CU. A query block split between workgroups is merged as above.
    int L;
    int U, nwg;
    float* ws;          // partial slots: (slot of the range) * (heads or KV groups) + head or group
    unsigned* counters; // one arrival counter per (query block, head) (without PACK)
    int64_t ml_off;
    int nord;
    unsigned short ord[768];
};

constexpr int KB = 64;  // keys per block

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

// 8 bytes from LDS through the transpose read (see the header).
__device__ __forceinline__ bf16x4 ld_tr(const char* a) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                          (__attribute__((address_space(3))) v4i16*)(const_cast<char*>(a))));
#else
    return bf16x4{};
#endif
}

// s_waitcnt immediates: vmcnt(n) (n < 16) and lgkmcnt(0); lgkmcnt(0) alone.
constexpr unsigned kLgkm0Vm(int n) { return (unsigned)(n | (0x7 << 4)); }
constexpr unsigned kLgkm0 = 0xC07F;

template <int D, bool CAUSAL, bool PACK, int WQ>
__global__ __launch_bounds__(128 * WQ, 2) void attn_kernel(AttnParams p) {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int QB = 32 * WQ;            // query rows per workgroup
    constexpr int NT = 128 * WQ;           // threads: WQ query slices x 2 key halves
    constexpr int ROWB = D * 2;            // bytes per K or V row in LDS
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;          // rows per DMA instruction (64 lanes x 16 bytes)
    constexpr int TILE = KB * ROWB;        // K or V tile bytes
    constexpr int STG = 2 * TILE;          // one buffer: K tile, then V tile
    constexpr int NC = D / 16;             // 16-wide d chunks (MFMA K steps of S)
    constexpr int NB = D / 32;             // 32-row d blocks of O^T
    constexpr int IPW = KB / RPI / (2 * WQ);  // DMA instructions per wave, operand and block
    static_assert(IPW >= 1 && IPW * RPI * 2 * WQ == KB, "the waves' DMAs cover a tile");
    constexpr int NR = NB * 16 + 2;        // floats per lane of a partial: O^T, m, l
    // LDS: two block buffers and the merge area, separate objects so that the compiler
    // can tell a DMA into one buffer from reads of the other (it would otherwise wait for
    // every DMA in flight before each read). One workgroup per CU either way (registers).
    constexpr int MERGEB = WQ * 64 * NR * 4;
    __shared__ __attribute__((aligned(1024))) char buf0[STG];
    __shared__ __attribute__((aligned(1024))) char buf1[STG];
    __shared__ __attribute__((aligned(16))) char mgs[MERGEB];
    __shared__ unsigned is_last;

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

    auto nkb_of = [&](int b) { return (kend_of(b) + KB - 1) / KB; };

    // One piece of work: key blocks [kb0, nkb) of query block qblk for head (or KV group)
    // hm; part `part` of the np parts of that query block, whose partial slots start at base.
    auto piece = [&](const int hm, const int qblk, const int np, const int part, const int base, const int kb0,
                     const int nkb) {
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
    }

    floatx16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // This wave needs keys < wave_kend; a wave whose rows all lie past the last token needs none.
    const int wave_kend = wfirst >= p.M ? 0 : CAUSAL ? min(p.Nk, p.pos0 + wlast + 1) : p.Nk;

    // Chunk c of row r of a K or V tile sits at chunk position c ^ swz(r), chosen for 64
    // banks of 4 bytes: the K fragment reads (one chunk of 16 consecutive rows per 256 bytes
    // served) and the transpose reads (64 bytes of each of 4 consecutive rows per 32 lanes)
    // then touch every bank once. 16 chunks a row (a row spans all banks): swz takes 16
    // distinct values over 16 rows, and the 4 rows of a run fall in distinct 64-byte groups.
    // 8 chunks a row (two rows share the banks): the same over rows of equal parity.
    auto swz = [](int r) {
        return CPR >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    };

    // DMA: wave w fills rows w * IPW * RPI .. of both tiles, instruction j the RPI rows from
    // row0(j) = (w * IPW + j) * RPI into 1 KB of LDS; lane i writes chunk position i % CPR
    // of row row0(j) + i / CPR, so it fetches the chunk that belongs there. Rows past the
    // last key repeat the last key's row (finite values; those keys are masked).
    const int wrow0 = wave * IPW * RPI;
    int drow[IPW], dcol[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
        drow[j] = wrow0 + j * RPI + lane / CPR;
        dcol[j] = ((lane % CPR) ^ swz(drow[j])) * 8;
    }
    auto dma = [&](int kb, char* buf) {
#if defined(__HIP_DEVICE_COMPILE__)
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16*>(K), (short)0, (int)(((int64_t)(p.Nk - 1) * p.ldk + D) * 2), 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16*>(V), (short)0, (int)(((int64_t)(p.Nk - 1) * p.ldv + D) * 2), 0x00020000);
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int t = min(kb * KB + drow[j], p.Nk - 1);
            char* l = buf + (wrow0 + j * RPI) * ROWB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)l, 16,
                                                     (uint32_t)((t * p.ldk + dcol[j]) * 2), 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(l + TILE), 16,
                                                     (uint32_t)((t * p.ldv + dcol[j]) * 2), 0, 0, 0);
        }
#endif
    };
    // Every wave's DMAs issued so far have landed (vm) and its LDS reads are done; then the
    // waves meet. The waits are explicit (a full fence would add its own), and the signal
    // fences keep the compiler from moving memory accesses across.
    auto block_barrier = [&](bool vm) {
        if (vm)
            __builtin_amdgcn_s_waitcnt(kLgkm0Vm(0));
        else
            __builtin_amdgcn_s_waitcnt(kLgkm0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // Fragment offsets. K: row 32 kh + l32, chunk 2 j + lh. V (transpose read, O^T block b,
    // step st): lane group g = lane / 16 covers head-dim columns 32 b + 16 (g % 2) .. +15
    // and, as source, its lane s = lane % 16 points at key 32 kh + 16 st + 4 (g / 2) + s / 4
    // (+ 8 for the second read), columns 32 b + 16 (g % 2) + 4 (s % 4) .. +3.
    const int krow = (32 * kh + l32) * ROWB, ksw = swz(l32);
    const int g16 = lane >> 4, s16 = lane & 15;
    const int vr1 = 32 * kh + 4 * (g16 >> 1) + (s16 >> 2), vr2 = vr1 + 8;
    int voff1[NB], voff2[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int c = 4 * b + 2 * (g16 & 1) + ((s16 & 3) >> 1);
        voff1[b] = vr1 * ROWB + ((c ^ swz(vr1)) << 4) + (s16 & 1) * 8;
        voff2[b] = vr2 * ROWB + ((c ^ swz(vr2)) << 4) + (s16 & 1) * 8;
    }

    // Block kb is in `cur`, block kb + 1 in the other buffer (in flight); after the barrier
    // that ends block kb, block kb + 2 goes into `cur`. Every wait for DMAs is unconditional
    // and waits for all of them (with both first blocks in flight and a wait for the older
    // one only, the compiler split the tests of kb0 + 1 < nkb into separate branches, saw a
    // path with no wait and waited for every DMA before the loop's reads), and each loop
    // trip runs both buffers' steps, so on every path the compiler sees a buffer's DMAs
    // retired before that buffer's next reads and adds no waits of its own.
    auto step = [&](int kb, char* cur) {
        const char* ks = cur;
        const char* vs = cur + TILE;
        const int k0 = kb * KB + 32 * kh;  // this wave's 32 keys
        if (k0 < wave_kend) {  // uniform per wave: past this wave's last query otherwise
            // S^T = K Q^T; all K fragments are read first so the LDS latency overlaps.
            bf16x8 kf[NC];
#pragma unroll
            for (int j = 0; j < NC; ++j)
                kf[j] = *reinterpret_cast<const bf16x8*>(ks + krow + (((2 * j + lh) ^ ksw) << 4));
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
                for (int b = 0; b < NB; ++b) {
                    const bf16x4 lo = ld_tr(vs + st * 16 * ROWB + voff1[b]);
                    const bf16x4 hi = ld_tr(vs + st * 16 * ROWB + voff2[b]);
                    vf[st][b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }

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
        block_barrier(true);  // block kb + 1 is in; `cur` is free
        if (kb + 2 < nkb) dma(kb + 2, cur);
    };
    if (kb0 < nkb) {
        // The queries and the first two blocks are in flight together; one unconditional
        // wait covers all of them (so the wait for the queries does not land inside the key
        // loop, where the in-order load counter would also wait for the next prefetch).
        dma(kb0, buf0);
        if (kb0 + 1 < nkb) dma(kb0 + 1, buf1);
#pragma unroll
        for (int j = 0; j < NC; ++j) asm volatile("" ::"v"(qf[j]));
        block_barrier(true);
    }
    int kb = kb0;
    for (; kb + 1 < nkb; kb += 2) {
        step(kb, buf0);
        step(kb + 1, buf1);
    }
    if (kb < nkb) step(kb, buf0);

    // Merge the two key halves: wave w + WQ leaves (m, l, O^T) in LDS, wave w combines.
    // Lane order in the merge area: [wave slice][register][lane], conflict-free.
    l_run = halves_sum(l_run);
    float* mg = reinterpret_cast<float*>(mgs) + wq * 64 * NR;
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
    };

    if (!PACK && p.nwg > 0) {
        // This workgroup's run of the work order, one piece per query block it touches.
        const int i = blockIdx.x;
        const int u0 = (int)((int64_t)i * p.U / p.nwg), u1 = (int)((int64_t)(i + 1) * p.U / p.nwg);
        const int Uh = p.U / HM;
        // The workgroup whose run holds unit x.
        auto wg_of = [&](int x) { return (int)(((int64_t)(x + 1) * p.nwg + p.U - 1) / p.U) - 1; };
        for (int u = u0; u < u1;) {
            const int hm = u / Uh;
            int r = u - hm * Uh, o = 0, qb, n;
            for (;; ++o) {
                qb = (o & 1) ? o / 2 : nqb - 1 - o / 2;
                n = nkb_of(qb);
                if (r < n) break;
                r -= n;
            }
            const int first = wg_of(u - r);
            const int np = wg_of(u - r + n - 1) - first + 1;
            const int kb1 = min(n, r + (u1 - u));
            if (u != u0) __syncthreads();  // the previous piece is done with LDS
            piece(hm, qb, np, i - first, 4 * qb, r, kb1);
            u += kb1 - r;
        }
    } else {
        // Workgroup -> (head or KV group, query block, key range): blockIdx = range * HM + hm;
        // the range is ord[blockIdx / HM], or, without a table, ranges are enumerated from
        // the last query block down and, within one, in key order (base = the slot of this
        // query block's first range).
        const int hm = blockIdx.x % HM;
        int b = blockIdx.x / HM, qblk, np = 1, base = 0;
        if (!PACK && p.nord > 0) {
            const int e = p.ord[b];
            qblk = e >> 2;
            b = e & 3;
            np = (nkb_of(qblk) - 1 + p.L) / p.L;
            base = 4 * qblk;  // partial slots: four per query block
        } else if (p.L > 0) {
            // A scalar walk over the query blocks; its length grows like L, i.e. like the
            // work of every range, so its share stays small.
            for (qblk = nqb - 1;; --qblk) {
                np = (nkb_of(qblk) - 1 + p.L) / p.L;  // ceil(nkb / L)
                if (b < np) break;
                b -= np;
                base += np;
            }
        } else {
            qblk = nqb - 1 - b;
            b = 0;
        }
        const int n = nkb_of(qblk);
        piece(hm, qblk, np, b, base, b * n / np, (b + 1) * n / np);
    }
}

constexpr int kWQ = 4;  // query slices per workgroup: 128 query rows, 8 waves

// Merge of the key ranges of cut packed query blocks: one workgroup per (query block, KV
// head, row); thread (j, d4) takes the ranges q = j, j + 8, ... (independent loads, all in
// flight at once) for 4 consecutive d, merging them online in that order; the 8 partial
// results then meet through LDS in j order. Fixed order throughout, one division by the
// merged sum, and the output rounded once to bf16 (the ranges' weights were rounded to bf16
// where they entered their P*V products).
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
tp_status_t run_attn(AttnParams p, const Ctx& c) {
    constexpr int QB = 32 * kWQ;
    const int gq = p.hq / p.hk;
    const int HM = PACK ? p.hk : p.hq;
    const int rows = PACK ? p.M * gq : p.M;
    const int nqb = (rows + QB - 1) / QB;
    auto kend_of = [&](int b) {
        const int last = PACK ? std::min(p.M - 1, ((b + 1) * QB - 1) / gq) : std::min(p.M - 1, (b + 1) * QB - 1);
        return CAUSAL ? std::min(p.Nk, p.pos0 + last + 1) : p.Nk;
    };
    // Cutting keys. Decode (PACK): few query blocks, whose keys are cut so that the grid has
    // about one workgroup per CU. Prefill (no PACK), causal (a query block's work grows with
    // its index) or with too few query blocks to fill the chip: every query block is cut into
    // ranges of at most L key blocks; if those ranges fit in one wave of resident workgroups
    // they run as they are, otherwise the work order is cut into equal runs, one per resident
    // workgroup slot (a second wave would leave the chip idle behind its longest ranges).
    const int nkb_max = (kend_of(nqb - 1) + KB - 1) / KB;
    const int cus = device_cu_count();
    // Resident workgroups per CU, from the kernel's registers and LDS against a CDNA4 CU:
    // 512 VGPRs per SIMD lane (allocated in steps of 8), four SIMDs, 160 KB of LDS.
    static const int occ = [] {
        hipFuncAttributes a;
        if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(attn_kernel<D, CAUSAL, PACK, kWQ>)) != hipSuccess ||
            a.numRegs <= 0)
            return 1;
        const int vgprs = (a.numRegs + 7) / 8 * 8;
        const int waves_per_simd = std::min(8, 512 / vgprs);
        const int by_regs = 4 * waves_per_simd / (2 * kWQ);  // 2 kWQ waves per workgroup
        const int by_lds = a.sharedSizeBytes > 0 ? (int)(160 * 1024 / a.sharedSizeBytes) : by_regs;
        return std::max(1, std::min(by_regs, by_lds));
    }();
    const int64_t slots_max = (int64_t)cus * occ;  // resident workgroups
    p.L = 0;
    p.U = 0;
    p.nwg = 0;
    p.nord = 0;
    int64_t grid = (int64_t)nqb * HM;
    int64_t slots = 0;  // partial slots per head or KV group
    if (PACK) {
        // About one workgroup per CU, at most 128 ranges per query block (the merge reads
        // up to 16 ranges per thread).
        const int want = std::min(128, std::max(1, (cus + nqb * HM - 1) / (nqb * HM)));
        p.L = std::max(1, (nkb_max + want - 1) / want);
        if (p.L >= nkb_max) p.L = 0;
        if (p.L > 0) {
            int64_t ranges = 0;
            for (int b = 0; b < nqb; ++b) ranges += ((kend_of(b) - 1) / KB + p.L) / p.L;
            grid = ranges * HM;
            slots = ranges;
            p.ml_off = ranges * HM * QB * D;
        }
    } else {
        int L = 0;
        if (CAUSAL && nqb >= 4)
            L = (nkb_max + 2) / 3;  // at most 3 ranges (measured: 2 and 4 ranges are slower)
        else if (2 * grid <= slots_max && nkb_max >= 2) {
            const int k = (int)std::min<int64_t>(4, slots_max / grid);  // ranges per query block
            L = (nkb_max + k - 1) / k;
        }
        if (L > 0 && L < nkb_max) {
            int64_t ranges = 0, U = 0;
            for (int b = 0; b < nqb; ++b) {
                const int n = (kend_of(b) + KB - 1) / KB;
                ranges += (n - 1 + L) / L;
                U += n;
            }
            U *= HM;
            // Equal runs of at least a third of the longest query block, so a query block
            // touches at most 4 runs (its partial slots). Only with one resident workgroup per
            // CU: with two, ranges in largest-first order keep both busy better (measured, head
            // size 64: 52.5 us against 56.0 us for equal runs at 4096 tokens, 16 heads).
            const int64_t nwg = std::min<int64_t>(slots_max, U / ((nkb_max + 2) / 3));
            if (occ == 1 && ranges * HM > slots_max && nwg > 1 && U < (int64_t(1) << 30)) {
                p.U = (int)U;
                p.nwg = (int)nwg;
                grid = nwg;
                slots = 4 * (int64_t)nqb;
            } else {
                p.L = L;
                grid = ranges * HM;
                slots = ranges;
                if (ranges <= (int64_t)(sizeof(p.ord) / sizeof(p.ord[0]))) {
                    // Largest ranges first (a cut block's ranges are shorter than an uncut
                    // block of the same index, so the plain walk would queue long uncut blocks
                    // behind short ranges); four slots per query block.
                    struct Piece { int size, e; };
                    Piece v[sizeof(p.ord) / sizeof(p.ord[0])];
                    int nv = 0;
                    for (int b = nqb - 1; b >= 0; --b) {
                        const int n = (kend_of(b) + KB - 1) / KB;
                        const int np = (n - 1 + L) / L;
                        for (int q = 0; q < np; ++q) v[nv++] = {(q + 1) * n / np - q * n / np, 4 * b + q};
                    }
                    std::stable_sort(v, v + nv, [](const Piece& a, const Piece& b) { return a.size > b.size; });
                    for (int i = 0; i < nv; ++i) p.ord[i] = (unsigned short)v[i].e;
                    p.nord = nv;
                    slots = 4 * (int64_t)nqb;
                }
            }
        }
    }
    p.ws = nullptr;
    p.counters = nullptr;
    if (slots > 0) {
        // Partials: without PACK one slot of WQ x 64 lanes x (D/2 + 2) floats per workgroup;
        // with PACK 128 rows x (D + 2) floats.
        const size_t floats = (size_t)(slots * HM) * (PACK ? QB * (D + 2) : kWQ * 64 * (D / 2 + 2));
        const WsNeed need{floats, (size_t)nqb * HM};
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
    hipLaunchKernelGGL((attn_kernel<D, CAUSAL, PACK, kWQ>), dim3((unsigned)grid), dim3(128 * kWQ), 0, c.stream, p);
    if (PACK && p.L > 0) {
        const tp_status_t st = hip_status();
        if (st != TP_OK) return st;
        hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)(nqb * HM * QB)), dim3(256), 0, c.stream, p, nqb);
    }
    return hip_status();
}

template <bool PACK>
tp_status_t run_attn_d(const AttnParams& p, int d, bool causal, const Ctx& c) {
    if (d == 128) return causal ? run_attn<128, true, PACK>(p, c) : run_attn<128, false, PACK>(p, c);
    if (d == 64) return causal ? run_attn<64, true, PACK>(p, c) : run_attn<64, false, PACK>(p, c);
    return TP_ERR_SHAPE;
}

}  // namespace

tp_status_t launch_attn_core(const void* qkv, int64_t ldq, void* out, int64_t lda, int64_t M, int hq, int hk, int d,
                             bool causal, const Ctx& c) {
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
    return run_attn_d<false>(p, d, causal, c);
}

tp_status_t launch_attn_decode(const void* qkv, int64_t ldq, void* kc, void* vc, int64_t ldkv, int64_t cache_len,
                               void* out, int64_t lda, int64_t M, int hq, int hk, int d, const Ctx& c) {
    const int64_t n_keys = cache_len + M;
    if (n_keys * ldkv * 2 >= (int64_t(1) << 31)) return TP_ERR_SHAPE;
    if (!c.planning()) {  // (the plan below covers the attention launches)
        const int64_t units = 2 * M * (ldkv / 8);
        const unsigned grid = (unsigned)std::min<int64_t>((units + 255) / 256, 4096);
        hipLaunchKernelGGL(append_kv_kernel, dim3(grid), dim3(256), 0, c.stream, static_cast<const bf16*>(qkv), ldq,
                           (int64_t)hq * d, (int64_t)(hq + hk) * d, static_cast<bf16*>(kc), static_cast<bf16*>(vc),
                           ldkv, cache_len, M);
        const tp_status_t st = hip_status();
        if (st != TP_OK) return st;
    }
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
    return run_attn_d<true>(p, d, true, c);
}

}  // namespace tp
