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
//     c ^ ((row >> 1) & 7): gfx950 serves a 16-byte-per-lane LDS access 16 lanes
//     (256 bytes, all 64 banks) at a time, and with this placement both the
//     row-wise stores (2 rows x 8 chunks) and the MFMA operand reads (16
//     consecutive rows, one chunk each) cover 16 distinct 16-byte bank groups;
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
#include <algorithm>
#include <type_traits>

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
    // Split-K remainder (LDS-DMA kernel only): the first F tiles run whole, one per
    // workgroup; each of the remaining tiles is cut into S equal K ranges, one per
    // workgroup, whose fp32 partials meet in ws.
    int F, S;
    float* ws;  // one fp32 partial tile per split workgroup
};

__device__ __forceinline__ bf16x8 ld8g(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Workgroup b's logical index: the hardware deals workgroups to the 8 XCDs in
// turn, so logical neighbours are put on one XCD (when n divides evenly) and share
// that XCD's L2.
__device__ __forceinline__ int xcd_major(int b, int n) {
    constexpr int XCDS = 8;
    return (n % XCDS == 0) ? (b % XCDS) * (n / XCDS) + b / XCDS : b;
}

// Tile of logical index L: grouped GW weight-row tiles at a time so consecutive
// tiles share panels.
__device__ __forceinline__ void tile_coords(int L, int tiles_n, int tiles_m, int& tn, int& tm) {
    constexpr int GW = 4;
    const int per_group = GW * tiles_m;
    const int grp = L / per_group;
    const int first = grp * GW;
    const int gw = min(GW, tiles_n - first);
    const int rem = L - grp * per_group;
    tn = first + rem % gw;
    tm = rem / gw;
}

// Tile of workgroup b when every workgroup takes one tile.
__device__ __forceinline__ void tile_of(int b, int tiles_n, int tiles_m, int& tn, int& tm) {
    tile_coords(xcd_major(b, tiles_n * tiles_m), tiles_n, tiles_m, tn, tm);
}

template <int TN, int TM, int WAVES_N, int WAVES_M, int ACT, bool BIAS, bool KTAIL, typename OutT>
__global__ __launch_bounds__(WAVES_N* WAVES_M * 64)
__attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_kernel(GemmParams p) {
    constexpr bool SWIGLU = ACT == kActSwiglu;
    constexpr int NT = WAVES_N * WAVES_M * 64;
    constexpr int WN = TN / WAVES_N;           // output features per wave
    constexpr int WM = TM / WAVES_M;           // tokens per wave
    constexpr int BN = WN / 32, BM = WM / 32;  // 32x32 blocks per wave
    constexpr int NA = SWIGLU ? 2 * BN : BN;   // A-operand blocks (gate then up)
    constexpr int WROWS = SWIGLU ? 2 * TN : TN;
    constexpr int ROWS = WROWS + TM;  // LDS rows per stage
    constexpr int RSTEP = NT / 8;     // rows covered by one round of 16-byte chunk loads
    constexpr int LW = WROWS / RSTEP, LX = TM / RSTEP, LPT = LW + LX;
    static_assert(WN % 32 == 0 && WM % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(WROWS % RSTEP == 0 && TM % RSTEP == 0 && TN % RSTEP == 0, "rounds must not straddle operands");
    static_assert(RSTEP % 16 == 0, "the LDS swizzle must repeat every round");

    __shared__ __attribute__((aligned(16))) bf16 lds[2][ROWS * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % WAVES_N, wm = wave / WAVES_N;
    const int l32 = lane & 31, lh = lane >> 5;

    int tn, tm;
    tile_of(blockIdx.x, p.tiles_n, p.tiles_m, tn, tm);
    const int n0 = tn * TN, m0 = tm * TM;

    // Global side: thread t loads chunk c = t % 8 of rows t / 8 + i * RSTEP. Rows past
    // N / tokens past M are clamped to the last valid row; their products land in
    // outputs that are never stored. Offsets are bytes from the operand's base
    // (each operand is below 4 GiB, checked on the host).
    const int c = tid & 7, r0 = tid >> 3;
    uint32_t off[LPT];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int row = r0 + i * RSTEP;
        const bool up = SWIGLU && row >= TN;
        const int n = min(n0 + (up ? row - TN : row), p.N - 1);
        off[i] = (uint32_t)(((int64_t)n * p.K + c * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < LX; ++i) {
        const int m = min(m0 + r0 + i * RSTEP, p.M - 1);
        off[LW + i] = (uint32_t)(((int64_t)m * p.ldx + c * 8) * 2);
    }
    // LDS side: row r0 + i*RSTEP, chunk c stored at c ^ ((row >> 1) & 7); the swizzle
    // term is the same for every round because RSTEP is a multiple of 16.
    const int dst0 = r0 * BK + ((c ^ ((r0 >> 1) & 7)) * 8);

    const char* w0b = reinterpret_cast<const char*>(p.W0);
    const char* w1b = reinterpret_cast<const char*>(SWIGLU ? p.W1 : p.W0);
    const char* xb = reinterpret_cast<const char*>(p.X);
    const int KT = (p.K + BK - 1) / BK;
    auto load_stage = [&](int kt, bf16x8 (&pre)[LPT]) {
        const int64_t kb = (int64_t)kt * BK * 2;
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const char* base = i < LW ? ((SWIGLU && i * RSTEP >= TN) ? w1b : w0b) : xb;
            const char* a = base + kb + off[i];
            if (KTAIL) a -= (kt * BK + c * 8 >= p.K) ? kb : 0;  // past K: re-read column 0, zeroed below
            pre[i] = *reinterpret_cast<const bf16x8*>(a);
        }
    };
    auto store_stage = [&](int kt, int buf, bf16x8 (&pre)[LPT]) {
        const bool ok = !KTAIL || kt * BK + c * 8 < p.K;
        const bf16x8 zero = {};
#pragma unroll
        for (int i = 0; i < LPT; ++i)
            *reinterpret_cast<bf16x8*>(&lds[buf][dst0 + i * RSTEP * BK]) = ok ? pre[i] : zero;
    };

    floatx16 acc[NA][BM];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < BM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // MFMA operand reads. Every block starts on a multiple of 32 rows, so the swizzle
    // term of this lane's row is (l32 >> 1) & 7 for all of them.
    const int sw = (l32 >> 1) & 7;
    const int lrow = l32 * BK;
    int arow[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const bool up = SWIGLU && i >= BN;
        arow[i] = ((up ? TN : 0) + wn * WN + (up ? i - BN : i) * 32) * BK;
    }
    const int brow0 = (WROWS + wm * WM) * BK;
    auto read_frags = [&](const bf16* s, int ks, bf16x8 (&af)[NA], bf16x8 (&bfr)[BM]) {
        const int kx = (((2 * ks + lh) ^ sw) * 8) + lrow;
#pragma unroll
        for (int i = 0; i < NA; ++i) af[i] = *reinterpret_cast<const bf16x8*>(&s[arow[i] + kx]);
#pragma unroll
        for (int j = 0; j < BM; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(&s[brow0 + j * 32 * BK + kx]);
    };
    auto mfmas = [&](bf16x8 (&af)[NA], bf16x8 (&bfr)[BM]) {
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < BM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    // The fragments of sub-step ks+1 are requested before the MFMAs of sub-step ks are
    // issued; the scheduling barriers keep the compiler from sinking those reads next
    // to their use, which would expose the LDS latency with one wave per SIMD.
    auto compute = [&](int buf) {
        const bf16* s = lds[buf];
        bf16x8 fa0[NA], fb0[BM], fa1[NA], fb1[BM];
        read_frags(s, 0, fa0, fb0);
        read_frags(s, 1, fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(s, 2, fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(s, 3, fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fa1, fb1);
    };

    bf16x8 pre[LPT];
    load_stage(0, pre);
    store_stage(0, 0, pre);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more) load_stage(kt + 1, pre);
        compute(kt & 1);
        if (more) store_stage(kt + 1, (kt + 1) & 1, pre);
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
                epilogue4<ACT, BIAS, OutT>(p.o, n_base, m, gv, uv);
                __builtin_amdgcn_sched_barrier(0);  // keep bias loads next to their use
            }
}

// ---------------------------------------------------------------------------------
// Large-tile kernel with direct global -> LDS loads.
//
// gfx950's buffer_load_dwordx4 ... lds writes each lane's 16 bytes straight into
// LDS (at a wave-uniform LDS address + 16 * lane), so staging needs no registers and
// the LDS ring can hold several BK-wide K slices while the matrix cores consume
// one. Holding more than one slice in registers would not fit next to each wave's
// accumulator tile.
//
// LDS row = BK bf16 = CPR chunks of 16 bytes. gfx950 serves a 16-byte-per-lane
// LDS access 16 lanes (256 bytes, 64 banks) at a time; chunk c of row r is stored
// at position c ^ ((r / RPW) % CPR), RPW = rows per 256-byte window, so the 16
// rows read by an MFMA operand access (one chunk each) hit 16 distinct 16-byte
// bank groups. A DMA instruction fills 64 / CPR consecutive rows (1 KB), each lane
// fetching the chunk that belongs at its position.
//
// Synchronisation is explicit: before slice k+1 is read, each wave has drained its
// LDS reads of slice k and waited until its own DMA for slice k+1 has landed
// (vmcnt: DMA completes in order), and all waves meet at s_barrier. Only then is
// slice k + STAGES requested, into slice k's buffer.
// ---------------------------------------------------------------------------------
// Slice width and ring depth, measured: 64-wide slices in a 2 x 64 KB ring beat 32-wide
// slices in 4- or 5-deep rings (gate/up of the 70B TP=8 shard at 4096 tokens: 408 us vs
// 425 / 435 us), whose extra barriers cost more than the deeper prefetch saves.
constexpr int DBK = 64;      // K slice per stage
constexpr int DSTAGES = 2;   // LDS ring depth
constexpr int kSpread = 2;   // MFMA sub-steps over which a slice's refill DMAs are spread

constexpr unsigned vmcnt_wait(int n) {  // s_waitcnt immediate: vmcnt(n), no other wait
    return (unsigned)((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
constexpr unsigned kLgkm0 = 0xC07F;     // s_waitcnt immediate: lgkmcnt(0) only

// Wait until at most min(ahead, A) * IPW of this wave's vector memory instructions are in
// flight (the DMAs of the slices requested after the one needed next).
template <int IPW, int A>
__device__ __forceinline__ void wait_ahead(int ahead) {
    if constexpr (A > 0) {
        static_assert(A * IPW < 64, "vmcnt has 6 bits");
        if (ahead >= A) {
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(A * IPW));
            return;
        }
        wait_ahead<IPW, A - 1>(ahead);
    } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    }
}

// One wave's DMA of a stage: IPW instructions of 1 KB each into consecutive LDS
// blocks, through a raw buffer descriptor of the operand (bounds = its byte size).
// The descriptor type exists only for the GPU target, so the body is compiled in
// the device pass alone (the host pass only needs the kernel's launch stub).
// Instructions j0 <= j < j1 only; callers pass bounds that are constants once their
// loops are unrolled, so the selection costs nothing.
template <int IPW>
__device__ __forceinline__ void dma_rows(const void* base, uint32_t bytes, const uint32_t (&goff)[IPW], uint32_t koff,
                                         char* l, int j0 = 0, int j1 = IPW) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
#pragma unroll
    for (int j = 0; j < IPW; ++j)
        if (j >= j0 && j < j1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(l + j * 1024), 16,
                                                     goff[j], koff, 0, 0);
#endif
}

// SK: split-K remainder. Workgroups below F take one whole tile each; the others
// take one of the S equal K ranges of a remaining tile and leave an fp32 partial
// tile, which splitk_reduce_kernel sums in K order and finishes.
// Workgroups that run side by side on one XCD hold neighbouring tiles at the same K
// range, so their panels are shared in that XCD's L2 (a stream-K split, whose
// workgroups sit at different K offsets, forfeits that sharing).
template <int TN, int TM, int WAVES_N, int WAVES_M, int ACT, bool BIAS, bool SK, typename OutT>
__global__ __launch_bounds__(WAVES_N* WAVES_M * 64) void gemm_dtl_kernel(GemmParams p) {
    constexpr bool SWIGLU = ACT == kActSwiglu;
    constexpr int NWAVES = WAVES_N * WAVES_M;
    constexpr int NT = NWAVES * 64;
    constexpr int WN = TN / WAVES_N, WM = TM / WAVES_M;
    constexpr int BN = WN / 32, BM = WM / 32;
    constexpr int NA = SWIGLU ? 2 * BN : BN;
    constexpr int WROWS = SWIGLU ? 2 * TN : TN;
    constexpr int ROWS = WROWS + TM;
    constexpr int ROWB = DBK * 2;             // bytes per LDS row
    constexpr int CPR = DBK / 8;              // 16-byte chunks per row
    constexpr int RPW = 256 / ROWB;           // rows per 256-byte bank window
    constexpr int RPI = 64 / CPR;             // rows per DMA instruction
    constexpr int STAGEB = ROWS * ROWB;
    constexpr int IPW = ROWS / RPI / NWAVES;  // DMA instructions per wave per stage
    constexpr int KS = DBK / 16;              // MFMA sub-steps per slice
    static_assert(DBK == 32 || DBK == 64, "slice width");
    static_assert(KS % 2 == 0, "sub-steps alternate between two fragment sets");
    static_assert(WN % 32 == 0 && WM % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(ROWS % (RPI * NWAVES) == 0, "each wave fills whole DMA row groups");
    static_assert(TN % (IPW * RPI) == 0 && WROWS % (IPW * RPI) == 0, "a wave's rows come from one operand");
    static_assert(32 % (RPW * CPR) == 0, "swizzle period divides a 32-row block");

    // The LDS ring, which also stages a plain bf16 output tile (rows padded by 16
    // bytes) so the tile leaves in whole 16-byte runs of each output row.
    constexpr int OPITCH = TN * 2 + 16;
    constexpr int OBYTES = SWIGLU ? 0 : TM * OPITCH;
    constexpr int LDSB = DSTAGES * STAGEB > OBYTES ? DSTAGES * STAGEB : OBYTES;
    __shared__ __attribute__((aligned(1024))) char lds_raw[LDSB];
    auto lds = reinterpret_cast<char (*)[STAGEB]>(lds_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // The wave index is uniform; saying so keeps the DMA base address and the LDS
    // destination (M0) in scalar registers, so each DMA is one instruction with a
    // 32-bit per-lane offset instead of a 64-bit vector address computation.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WAVES_N, wm = wave / WAVES_N;
    const int l32 = lane & 31, lh = lane >> 5;

    // This wave's DMA rows: wrow0 + j * RPI + lane / CPR, all from one operand, read
    // through a buffer descriptor of that operand (scalar base and size, 32-bit
    // per-lane offsets, the K slice's offset as the scalar offset).
    const int wrow0 = wave * IPW * RPI;
    const bool wop = wrow0 < WROWS;
    const bool wup = SWIGLU && wop && wrow0 >= TN;
    const void* obase = wop ? (wup ? (const void*)p.W1 : (const void*)p.W0) : (const void*)p.X;
    const int64_t obytes = wop ? (int64_t)p.N * p.K * 2 : (int64_t)(p.M - 1) * p.ldx * 2 + (int64_t)p.K * 2;
    uint32_t goff[IPW];
    auto set_rows = [&](int n0, int m0) {
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int row = wrow0 + j * RPI + lane / CPR;
            const int c = (lane % CPR) ^ ((row / RPW) % CPR);  // the chunk that belongs at this lane's position
            if (wop) {
                const bool up = SWIGLU && row >= TN;
                const int n = min(n0 + (up ? row - TN : row), p.N - 1);
                goff[j] = (uint32_t)(((int64_t)n * p.K + c * 8) * 2);
            } else {
                const int m = min(m0 + row - WROWS, p.M - 1);
                goff[j] = (uint32_t)(((int64_t)m * p.ldx + c * 8) * 2);
            }
        }
    };
    const int KT = p.K / DBK;

    floatx16 acc[NA][BM];

    // Operand reads: every block starts on a multiple of 32 rows, so this lane's
    // swizzle term is (l32 / RPW) % CPR for all of them.
    const int sw = (l32 / RPW) % CPR;
    int arow[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const bool up = SWIGLU && i >= BN;
        arow[i] = ((up ? TN : 0) + wn * WN + (up ? i - BN : i) * 32) * ROWB;
    }
    const int brow0 = (WROWS + wm * WM) * ROWB;
    auto read_frags = [&](const char* s, int ks, bf16x8 (&af)[NA], bf16x8 (&bfr)[BM]) {
        const int kx = l32 * ROWB + (((2 * ks + lh) ^ sw) * 16);
#pragma unroll
        for (int i = 0; i < NA; ++i) af[i] = *reinterpret_cast<const bf16x8*>(s + arow[i] + kx);
#pragma unroll
        for (int j = 0; j < BM; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(s + brow0 + j * 32 * ROWB + kx);
    };
    auto mfmas = [&](bf16x8 (&af)[NA], bf16x8 (&bfr)[BM]) {
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < BM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    // Wait until this wave's DMA for the next slice has landed (`ahead` slices were
    // requested after it), then meet the other waves.
    auto sync_slice = [&](int ahead) {
        static_assert(DSTAGES <= 5, "waits below cover up to 4 slices ahead");
        if (ahead >= 4) __builtin_amdgcn_s_waitcnt(vmcnt_wait(4 * IPW));
        else if (ahead == 3) __builtin_amdgcn_s_waitcnt(vmcnt_wait(3 * IPW));
        else if (ahead == 2) __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * IPW));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_wait(IPW));
        else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));  // also for a slice past the end
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // Per sub-step: request the next fragments and run this sub-step's MFMAs, each
    // fragment read issued right behind an MFMA so the matrix cores never wait on the
    // LDS queue. Before the last sub-step of slice k, synchronise on slice k+1. The
    // buffer slice k-1 left free is refilled (with slice k-1+STAGES) during the first
    // NSPREAD sub-steps of slice k, one DMA behind every few MFMAs. Whether a slice
    // refills is a template flag, so no branch splits a sub-step and the interleaving
    // below holds for every slice.
    constexpr int NSPREAD = kSpread;
    // The refill DMAs must all be issued before the last sub-step's wait for the next slice.
    static_assert(NSPREAD >= 1 && NSPREAD < KS && IPW % NSPREAD == 0, "DMA spread");
    constexpr int NMF = NA * BM;                 // MFMAs per sub-step
    constexpr int NRD = NA + BM;                 // fragment reads per sub-step
    constexpr int DPS = IPW / NSPREAD;           // DMA instructions per spread sub-step
    static_assert(NRD <= NMF, "one fragment read per MFMA");
    // DMAs that find no MFMA after the reads go behind the last one.
    constexpr int DTAIL = NRD + DPS > NMF ? NRD + DPS - NMF : 0;
    bf16x8 fa0[NA], fb0[BM], fa1[NA], fb1[BM];

    // acc = the product over K slices kt0 .. kt0+nkt-1 of the tile whose rows goff holds.
    auto compute = [&](int kt0, int nkt) {
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < BM; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        // Prologue: every buffer requested; sub-step 0 of the first slice read.
        for (int st = 0; st < DSTAGES && st < nkt; ++st)
            dma_rows<IPW>(obase, (uint32_t)obytes, goff, (uint32_t)((kt0 + st) * DBK * 2), &lds[st][wrow0 * ROWB]);
        sync_slice(min(nkt - 1, DSTAGES - 1));
        read_frags(lds[0], 0, fa0, fb0);
        // lgkmcnt has 4 bits: with two batches of reads outstanding the compiler could
        // only wait for zero. Each batch is therefore drained (it had a whole MFMA
        // phase to land, so this does not stall) before the next one is issued.
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        auto slice = [&](int kt, auto refill_tag) {
            constexpr bool REFILL = decltype(refill_tag)::value;
            const char* s = lds[kt % DSTAGES];
            const uint32_t rkoff = (uint32_t)((kt0 + kt - 1 + DSTAGES) * DBK * 2);
            char* rl = &lds[(kt + DSTAGES - 1) % DSTAGES][wrow0 * ROWB];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bool even = (ks & 1) == 0;
                if (ks + 1 == KS) {
                    // On the last slice this synchronises once more and reads a buffer
                    // nobody uses any more, so every slice takes the same path.
                    sync_slice(min(nkt - 2 - kt, DSTAGES - 2));
                    __builtin_amdgcn_sched_barrier(0);
                }
                const char* src = ks + 1 < KS ? s : lds[(kt + 1) % DSTAGES];
                const int nks = ks + 1 < KS ? ks + 1 : 0;
                if (even) read_frags(src, nks, fa1, fb1);  // KS is even: sets alternate 0, 1, 0, 1
                else read_frags(src, nks, fa0, fb0);
                if (REFILL && ks < NSPREAD)
                    dma_rows<IPW>(obase, (uint32_t)obytes, goff, rkoff, rl, ks * DPS, (ks + 1) * DPS);
                if (even) mfmas(fa0, fb0);
                else mfmas(fa1, fb1);
                // The DMAs write LDS, so the compiler keeps every fragment read ahead of
                // them: reads go behind the first MFMAs, DMAs behind the following ones.
#pragma unroll
                for (int q = 0; q < NMF; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    else if (REFILL && ks < NSPREAD && q - NRD < DPS)
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one DMA
                }
                if (REFILL && ks < NSPREAD && DTAIL > 0) __builtin_amdgcn_sched_group_barrier(0x020, DTAIL, 0);
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(kLgkm0);
            }
        };
        slice(0, std::false_type{});  // the prologue filled every buffer
        int kt = 1;
        for (; kt + DSTAGES - 1 < nkt; ++kt) slice(kt, std::true_type{});
        for (; kt < nkt; ++kt) slice(kt, std::false_type{});
    };

    auto store_tile = [&](int n0, int m0) {
        // Measured: staging pays for plain tiles (256 B of each output row per wave
        // and block row otherwise goes out 8 bytes at a time) but not for SwiGLU
        // ones, whose epilogue arithmetic then sits between two barriers.
        if (!SWIGLU && std::is_same<OutT, bf16>::value && p.o.vec16) {
            // Every wave is past its last LDS read of the ring.
            __syncthreads();
#pragma unroll
            for (int i = 0; i < BN; ++i)
#pragma unroll
                for (int j = 0; j < BM; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float gv[4], uv[4], y[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            gv[e] = acc[i][j][4 * q + e];
                            uv[e] = SWIGLU ? acc[i + (SWIGLU ? BN : 0)][j][4 * q + e] : 0.f;
                        }
                        const int nl = wn * WN + i * 32 + 8 * q + 4 * lh;
                        const int ml = wm * WM + j * 32 + l32;
                        epilogue_vals4<ACT, BIAS>(p.o, n0 + nl, gv, uv, y);
                        const bf16x4 v = {(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
                        *reinterpret_cast<bf16x4*>(lds_raw + ml * OPITCH + nl * 2) = v;
                    }
            __syncthreads();
            // Each pass writes NT/CPRW whole rows of the tile, 16 bytes per thread.
            constexpr int CPRW = TN * 2 / 16;  // 16-byte chunks per output row
            constexpr int RPP = NT / CPRW;
            static_assert(NT % CPRW == 0 && TM % RPP == 0, "whole rows per pass");
            const int c = tid % CPRW;
            const int n = n0 + c * 8;
#pragma unroll 4
            for (int r0 = 0; r0 < TM; r0 += RPP) {
                const int row = r0 + tid / CPRW;
                const int m = m0 + row;
                if (m >= p.o.M) continue;
                const bf16x8 v = *reinterpret_cast<const bf16x8*>(lds_raw + row * OPITCH + c * 16);
                bf16* dst = reinterpret_cast<bf16*>(p.o.Y) + (int64_t)m * p.o.ldy + n;
                if (n + 8 <= p.o.N) {
                    *reinterpret_cast<bf16x8*>(dst) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < p.o.N) dst[e] = v[e];
                }
            }
            return;
        }
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
                    epilogue4<ACT, BIAS, OutT>(p.o, n_base, m, gv, uv);
                    __builtin_amdgcn_sched_barrier(0);
                }
    };

    if (!SK) {
        int tn, tm;
        tile_of(blockIdx.x, p.tiles_n, p.tiles_m, tn, tm);
        set_rows(tn * TN, tm * TM);
        compute(0, KT);
        store_tile(tn * TN, tm * TM);
        return;
    }

    // Split tiles: piece q (XCD-major) is K range sp of split tile r. Its fp32
    // partial tile goes to slot q of the work space as float4 groups [group][thread],
    // so every 16-byte store covers contiguous memory; splitk_reduce_kernel, the next
    // launch on the stream, sums the pieces.
    constexpr int NG = NA * BM * 4;  // float4 groups per thread
    const int R = p.tiles_n * p.tiles_m - p.F;
    int tn, tm;
    if ((int)blockIdx.x < p.F) {
        tile_coords(xcd_major(blockIdx.x, p.F), p.tiles_n, p.tiles_m, tn, tm);
        set_rows(tn * TN, tm * TM);
        compute(0, KT);
        store_tile(tn * TN, tm * TM);
        return;
    }
    const int q = xcd_major((int)blockIdx.x - p.F, R * p.S);
    const int sp = q / R, r = q - sp * R;
    const int kt0 = (int)((int64_t)sp * KT / p.S), kt1 = (int)((int64_t)(sp + 1) * KT / p.S);
    tile_coords(p.F + r, p.tiles_n, p.tiles_m, tn, tm);
    set_rows(tn * TN, tm * TM);
    compute(kt0, kt1 - kt0);
    floatx4* dst = reinterpret_cast<floatx4*>(p.ws) + (int64_t)q * NG * NT + tid;
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < BM; ++j)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                dst[((i * BM + j) * 4 + qq) * NT] = floatx4{acc[i][j][4 * qq], acc[i][j][4 * qq + 1],
                                                          acc[i][j][4 * qq + 2], acc[i][j][4 * qq + 3]};
}

// One float4 per lane from base + voff + soff (voff a lane register, soff uniform),
// through a raw buffer descriptor of `bytes` bytes (device pass only, as dma_rows).
__device__ __forceinline__ floatx4 load_f4(const void* base, uint32_t bytes, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0));
#else
    return floatx4{};
#endif
}

// The S pieces of each split tile, summed in K order, then the tile's epilogue.
// Workgroup (r, i, j) takes 32x32 block (i, j) of every wave's part of split tile r,
// with the thread layout of the GEMM kernel, so thread tid reads exactly the float4
// groups it would have held. S is a compile-time count so that every piece's loads are
// in flight together: one memory round trip per workgroup.
template <int TN, int TM, int WAVES_N, int WAVES_M, int ACT, bool BIAS, typename OutT, int S>
__global__ __launch_bounds__(WAVES_N* WAVES_M * 64) void splitk_reduce_kernel(GemmParams p) {
    constexpr bool SWIGLU = ACT == kActSwiglu;
    constexpr int NWAVES = WAVES_N * WAVES_M, NT = NWAVES * 64;
    constexpr int WN = TN / WAVES_N, WM = TM / WAVES_M;
    constexpr int BN = WN / 32, BM = WM / 32;
    constexpr int NA = SWIGLU ? 2 * BN : BN;
    constexpr int NG = NA * BM * 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WAVES_N, wm = wave / WAVES_N;
    const int l32 = lane & 31, lh = lane >> 5;
    const int R = p.tiles_n * p.tiles_m - p.F;
    const int j = (int)blockIdx.x % BM, ri = (int)blockIdx.x / BM;
    const int r = ri / BN, i = ri - r * BN;
    int tn, tm;
    tile_coords(p.F + r, p.tiles_n, p.tiles_m, tn, tm);
    // The tile's partials, read through a buffer descriptor: one lane offset register
    // for every load and the piece and group as a scalar offset (a 64-bit address per
    // load in flight would take the registers the loads need). All offsets are below
    // the descriptor's bound, the end of the tile's last piece.
    const floatx4* src = reinterpret_cast<const floatx4*>(p.ws) + (int64_t)r * NG * NT;
    const int64_t piece = (int64_t)R * NG * NT;  // float4s between pieces of one tile
    const uint32_t src_bytes = (uint32_t)(((S - 1) * piece + NG * NT) * (int64_t)sizeof(floatx4));
    const uint32_t lane_off = (uint32_t)tid * sizeof(floatx4);
    // Block (row block a, column block j): every piece's four float4 groups loaded, then
    // summed in K order (the gate and up blocks of a SwiGLU tile one after the other).
    auto sum_block = [&](int a, floatx4 (&out)[4]) {
        floatx4 x[S][4];
#pragma unroll
        for (int sp = 0; sp < S; ++sp)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                x[sp][qq] = load_f4(src, src_bytes, lane_off,
                                    (uint32_t)((sp * piece + ((a * BM + j) * 4 + qq) * NT) * (int64_t)sizeof(floatx4)));
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            out[qq] = x[0][qq];
#pragma unroll
            for (int sp = 1; sp < S; ++sp) out[qq] += x[sp][qq];
        }
    };
    {
        floatx4 g[4], u[4];
        sum_block(i, g);
        // The up block's loads stay behind the gate sums (hoisted, they overflow the 128
        // registers a thread of a 1024-thread workgroup has).
        if (SWIGLU) __builtin_amdgcn_sched_barrier(0);
        if (SWIGLU) sum_block(i + (SWIGLU ? BN : 0), u);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            float gv[4], uv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gv[e] = g[qq][e];
                uv[e] = SWIGLU ? u[qq][e] : 0.f;
            }
            const int n_base = tn * TN + wn * WN + i * 32 + 8 * qq + 4 * lh;
            const int m = tm * TM + wm * WM + j * 32 + l32;
            epilogue4<ACT, BIAS, OutT>(p.o, n_base, m, gv, uv);
        }
    }
}

// ---------------------------------------------------------------------------------
// Products on 16-row MFMA blocks: v_mfma_f32_16x16x32_bf16, TN x TM tiles of 4 waves
// with (TN/2) x (TM/2) outputs each (plain products; the SwiGLU pair at up to 64 tokens).
//
// 32-row blocks leave no good layout for a product whose 256 x 256 tiles do not fill
// whole waves of CUs: the 70B TP=8 QKV shard (1280 features x 4096 tokens) has 80 such
// tiles, which run as split-K pieces plus a reduce pass. With 16-row blocks the tile
// can be 160 features x 128 tokens: 256 tiles, one per CU, each over the whole K, with
// 80 x 64 outputs per wave (5 x 4 blocks: 9 fragment reads per 20 MFMAs). With weights cold
// from HBM it runs 90.6 us against 93.4 us for the split-K pieces and their reduce. With
// fewer tokens the same tiles are cut into the S equal K ranges that fill the chip (SK):
// fp32 partial tiles summed in K order by splitk16_reduce_kernel, the next launch on the
// stream (2048 tokens: 2 ranges, a third of the partials of 256 x 256 tiles in 6).
//
// The same kernel takes up to 64 tokens as one 64-token tile (SK): 128-feature tiles (96
// SwiGLU pairs), each cut into K ranges the same way, a 4-deep DMA ring so that every CU
// keeps its weight stream in flight; or whole-K tiles of 32 pairs in a 10-deep ring. The
// tokens are staged once per slice for the 4 waves (the decode kernel's waves each reload
// them from L2).
//
// Operand staging as in gemm_dtl_kernel: K slices of 64 by LDS DMA into a ring of
// STAGES buffers; the weight rows are dealt to the first W0 waves, the token rows to
// the others, each wave an equal run of whole DMA rows. A wave whose run is shorter than
// its IPW instructions issues the rest past the operand's bounds, where the buffer
// descriptor's range check drops them, so every wave waits on the same counts.
//
// MFMA 16x16x32 operand mapping (lane l, l16 = l % 16, lq = l / 16):
//   A: lane l holds W[n0 + l16][k0 + 8*lq .. +7];  B: lane l holds X[m0 + l16][k0 + 8*lq .. +7]
//   D: register e of lane l holds D[n0 + 4*lq + e][m0 + l16]
// ---------------------------------------------------------------------------------
template <int TN, int TM, bool SW = false>
struct Dtl16Shape {
    static constexpr int NWAVES = 4, NT = 256;
    static constexpr int WN = TN / 2, WM = TM / 2;   // outputs per wave (2 x 2 waves)
    static constexpr int NA = WN / 16, BM = WM / 16;  // 16-row blocks per wave (of each weight operand)
    static constexpr int NAT = SW ? 2 * NA : NA;      // A blocks per wave: gate blocks, then up blocks
    static constexpr int NG = NAT * BM;               // float4 accumulator groups per thread
    static constexpr int NOPW = SW ? 2 : 1;           // weight operands (SwiGLU: gate and up)
    static constexpr int ROWB = DBK * 2, CPR = DBK / 8, RPW = 256 / ROWB, RPI = 64 / CPR;
    // Rows per wave of an operand of r rows over w waves, or 0 when they do not split into
    // whole DMA instructions that fit ipw.
    static constexpr int run(int r, int w, int ipw) { return (r % w == 0 && (r / w) % RPI == 0 && r / w <= ipw * RPI) ? r / w : 0; }
    static constexpr int fit(int ipw) {  // waves per weight operand for ipw instructions per wave, 0 if none fits
        for (int w0 = 1; NOPW * w0 < NWAVES; ++w0)
            if (run(TN, w0, ipw) && run(TM, NWAVES - NOPW * w0, ipw)) return w0;
        return 0;
    }
    static constexpr int ipw_min() {
        int i = ((NOPW * TN + TM) / RPI + NWAVES - 1) / NWAVES;
        while (fit(i) == 0) ++i;
        return i;
    }
    static constexpr int IPW = ipw_min();                  // DMA instructions per wave and slice
    static constexpr int RPWV = IPW * RPI;                 // LDS rows per wave
    static constexpr int W0 = fit(IPW);                    // waves loading each weight operand's rows
    static constexpr int RW = TN / W0, RX = TM / (NWAVES - NOPW * W0);  // operand rows per wave
    static constexpr int UPB = W0 * RPWV;                  // first LDS row of the up weights (SwiGLU)
    static constexpr int XB = NOPW * W0 * RPWV;            // first LDS row of the tokens
    static constexpr int ROWS = NWAVES * RPWV;             // LDS rows per stage
    static_assert(IPW < 32, "DMA instructions per wave");
    static_assert(WN % 16 == 0 && WM % 16 == 0, "whole blocks");
};

// The LDS row of operand row t of a tile: weight rows t in the first W0 waves' runs (the up
// weights of the SwiGLU pair the same after UPB), token rows after XB.
template <typename Sh>
__device__ __forceinline__ int dtl16_wrow(int t) { return (t / Sh::RW) * Sh::RPWV + t % Sh::RW; }
template <typename Sh>
__device__ __forceinline__ int dtl16_xrow(int t) { return Sh::XB + (t / Sh::RX) * Sh::RPWV + t % Sh::RX; }

template <int TN, int TM, int STAGES, int ACT, bool BIAS, bool SK, typename OutT>
__global__ __launch_bounds__(256) void gemm_dtl16_kernel(GemmParams p) {
    constexpr bool SW = ACT == kActSwiglu;
    using Sh = Dtl16Shape<TN, TM, SW>;
    constexpr int NA = Sh::NA, NAT = Sh::NAT, BM = Sh::BM, WN = Sh::WN, WM = Sh::WM, NT = Sh::NT;
    constexpr int ROWB = Sh::ROWB, CPR = Sh::CPR, RPW = Sh::RPW, RPI = Sh::RPI, IPW = Sh::IPW, RPWV = Sh::RPWV;
    constexpr int STAGEB = Sh::ROWS * ROWB;
    constexpr int KS = DBK / 32;  // MFMA sub-steps per slice
    static_assert(KS == 2, "two sub-steps per slice alternate the fragment sets");
    __shared__ __attribute__((aligned(1024))) char lds_raw[STAGES * STAGEB];
    auto lds = reinterpret_cast<char (*)[STAGEB]>(lds_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int l16 = lane & 15, lq = lane >> 4;

    // Tile and K range: one whole tile per workgroup, or (SK) piece q = K range sp of tile
    // r, pieces side by side on one XCD holding neighbouring tiles at the same K range.
    const int KTALL = p.K / DBK;
    int tn, tm, kt0 = 0, KT = KTALL, q = 0;
    if (SK) {
        const int R = p.tiles_n * p.tiles_m;
        q = xcd_major((int)blockIdx.x, R * p.S);
        const int sp = q / R, r = q - sp * R;
        kt0 = (int)((int64_t)sp * KTALL / p.S);
        KT = (int)((int64_t)(sp + 1) * KTALL / p.S) - kt0;
        tile_coords(r, p.tiles_n, p.tiles_m, tn, tm);
    } else {
        tile_of(blockIdx.x, p.tiles_n, p.tiles_m, tn, tm);
    }
    const int n0 = tn * TN, m0 = tm * TM;

    // This wave's DMA rows: operand rows t0 + j*RPI + lane/CPR into LDS rows
    // wave*RPWV + j*RPI + lane/CPR; chunk c of LDS row r sits at c ^ ((r / RPW) % CPR).
    const bool wop = wave < Sh::NOPW * Sh::W0;
    const bool wup = SW && wave >= Sh::W0 && wop;
    const int orun = wop ? Sh::RW : Sh::RX;
    const int t0 = (wop ? (wup ? wave - Sh::W0 : wave) : wave - Sh::NOPW * Sh::W0) * orun;
    const void* obase = wop ? (wup ? (const void*)p.W1 : (const void*)p.W0) : (const void*)p.X;
    const int64_t obytes = wop ? (int64_t)p.N * p.K * 2 : (int64_t)(p.M - 1) * p.ldx * 2 + (int64_t)p.K * 2;
    uint32_t goff[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
        const int lr = j * RPI + lane / CPR;
        const int row = wave * RPWV + lr;
        const int c = (lane % CPR) ^ ((row / RPW) % CPR);
        const int t = t0 + lr;
        if (j * RPI >= orun) {
            goff[j] = (uint32_t)obytes;  // past the wave's run: dropped by the range check
        } else if (wop) {
            goff[j] = (uint32_t)(((int64_t)min(n0 + t, p.N - 1) * p.K + c * 8) * 2);
        } else {
            goff[j] = (uint32_t)(((int64_t)min(m0 + t, p.M - 1) * p.ldx + c * 8) * 2);
        }
    }

    // Fragment reads: block i of this lane is weight row wn*WN + 16 i + l16 (SwiGLU: blocks
    // NA + i the up rows of the same features) and block j token row wm*WM + 16 j + l16, at
    // their LDS rows; every 16-row block lies in one wave's run
    // and starts on a multiple of 16 LDS rows, so the swizzle term is (l16 / RPW) % CPR for
    // all of them. Sub-step ks takes chunk 4 ks + lq.
    static_assert(Sh::RW % 16 == 0 && Sh::RX % 16 == 0 && RPWV % 16 == 0, "16-row blocks stay in one run");
    const int sw = (l16 / RPW) % CPR;
    int arow[NAT], brow[BM];
#pragma unroll
    for (int i = 0; i < NAT; ++i)
        arow[i] = ((i < NA ? 0 : Sh::UPB) + dtl16_wrow<Sh>(wn * WN + 16 * (i % NA) + l16)) * ROWB;
#pragma unroll
    for (int j = 0; j < BM; ++j) brow[j] = dtl16_xrow<Sh>(wm * WM + 16 * j + l16) * ROWB;
    floatx4 acc[NAT][BM];
#pragma unroll
    for (int i = 0; i < NAT; ++i)
#pragma unroll
        for (int j = 0; j < BM; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto read_frags = [&](const char* s, int ks, bf16x8 (&af)[NAT], bf16x8 (&bfr)[BM]) {
        const int kx = ((4 * ks + lq) ^ sw) * 16;
#pragma unroll
        for (int i = 0; i < NAT; ++i) af[i] = *reinterpret_cast<const bf16x8*>(s + arow[i] + kx);
#pragma unroll
        for (int j = 0; j < BM; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(s + brow[j] + kx);
    };
    auto mfmas = [&](bf16x8 (&af)[NAT], bf16x8 (&bfr)[BM]) {
#pragma unroll
        for (int i = 0; i < NAT; ++i)
#pragma unroll
            for (int j = 0; j < BM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    auto sync_slice = [&](int ahead) {
        wait_ahead<IPW, STAGES - 1>(ahead);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    constexpr int NMF = NAT * BM, NRD = NAT + BM;
    // Reads and refill DMAs that find no MFMA to follow go behind the last one.
    constexpr int RTAIL = NRD > NMF ? NRD - NMF : 0;
    constexpr int DTAIL = NRD + IPW > NMF ? (NRD > NMF ? IPW : NRD + IPW - NMF) : 0;
    bf16x8 fa0[NAT], fb0[BM], fa1[NAT], fb1[BM];

    // Prologue: every buffer requested; sub-step 0 of the first slice read.
    for (int st = 0; st < STAGES && st < KT; ++st)
        dma_rows<IPW>(obase, (uint32_t)obytes, goff, (uint32_t)((kt0 + st) * DBK * 2), &lds[st][wave * RPWV * ROWB]);
    sync_slice(min(KT - 1, STAGES - 1));
    read_frags(lds[0], 0, fa0, fb0);
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    // Slice kt: sub-step 0 reads sub-step 1's fragments and refills the buffer slice kt-1
    // left free (with slice kt-1+STAGES) behind its MFMAs; sub-step 1 synchronises on
    // slice kt+1 and reads its sub-step 0.
    auto slice = [&](int kt, auto refill_tag) {
        constexpr bool REFILL = decltype(refill_tag)::value;
        const char* s = lds[kt % STAGES];
        read_frags(s, 1, fa1, fb1);
        if (REFILL)
            dma_rows<IPW>(obase, (uint32_t)obytes, goff, (uint32_t)((kt0 + kt - 1 + STAGES) * DBK * 2),
                          &lds[(kt + STAGES - 1) % STAGES][wave * RPWV * ROWB]);
        mfmas(fa0, fb0);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            else if (REFILL && q - NRD < IPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one DMA
        }
        if (RTAIL > 0) __builtin_amdgcn_sched_group_barrier(0x100, RTAIL, 0);
        if (REFILL && DTAIL > 0) __builtin_amdgcn_sched_group_barrier(0x020, DTAIL, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        // On the last slice this synchronises once more and reads a buffer nobody uses any
        // more, so every slice takes the same path.
        sync_slice(min(KT - 2 - kt, STAGES - 2));
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds[(kt + 1) % STAGES], 0, fa0, fb0);
        mfmas(fa1, fb1);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (RTAIL > 0) __builtin_amdgcn_sched_group_barrier(0x100, RTAIL, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
    };
    int kt = 0;
    for (; kt == 0 && kt < KT; ++kt) slice(kt, std::false_type{});  // the prologue filled every buffer
    for (; kt + STAGES - 1 < KT; ++kt) slice(kt, std::true_type{});
    for (; kt < KT; ++kt) slice(kt, std::false_type{});

    if (SK) {
        // The fp32 partial tile as float4 groups [group][thread], every store contiguous.
        floatx4* dst = reinterpret_cast<floatx4*>(p.ws) + (int64_t)q * Sh::NG * NT + tid;
#pragma unroll
        for (int i = 0; i < NAT; ++i)
#pragma unroll
            for (int j = 0; j < BM; ++j) dst[(i * BM + j) * NT] = acc[i][j];
        return;
    }
    // Epilogue: register e of block (i, j) holds feature wn*WN + 16 i + 4 lq + e of token
    // wm*WM + 16 j + l16 (SwiGLU: its up sum in block (NA + i, j)); bias, activation, one
    // rounding, 4 consecutive outputs per store.
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < BM; ++j) {
            float gv[4], uv[4] = {};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gv[e] = acc[i][j][e];
                if (SW) uv[e] = acc[(i + NA) % NAT][j][e];
            }
            const int n_base = n0 + wn * WN + 16 * i + 4 * lq;
            const int m = m0 + wm * WM + 16 * j + l16;
            epilogue4<ACT, BIAS, OutT>(p.o, n_base, m, gv, uv);
            __builtin_amdgcn_sched_barrier(0);
        }
}

// The S pieces of every tile of gemm_dtl16_kernel<SK>, summed in K order, then the
// epilogue. Workgroup (r, g) takes float4 group g of every thread of tile r, so thread
// tid reads exactly the group it would have held; S is a compile-time count so that
// every piece's load is in flight before the first add.
template <int TN, int TM, int ACT, bool BIAS, typename OutT, int S>
__global__ __launch_bounds__(256) void splitk16_reduce_kernel(GemmParams p) {
    constexpr bool SW = ACT == kActSwiglu;
    using Sh = Dtl16Shape<TN, TM, SW>;
    constexpr int NT = Sh::NT, NG = Sh::NG, BM = Sh::BM, NA = Sh::NA;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int l16 = lane & 15, lq = lane >> 4;
    const int R = p.tiles_n * p.tiles_m;
    // Workgroup (r, g), g < NA * BM: the output group (i, j) (SwiGLU: with its up group
    // (NA + i, j)).
    const int g = (int)blockIdx.x % (NA * BM), r = (int)blockIdx.x / (NA * BM);
    const int i = g / BM, j = g % BM;
    int tn, tm;
    tile_coords(r, p.tiles_n, p.tiles_m, tn, tm);
    const floatx4* src = reinterpret_cast<const floatx4*>(p.ws) + (int64_t)r * NG * NT + tid;
    const int64_t piece = (int64_t)R * NG * NT;  // float4s between pieces of one tile
    constexpr int NS = SW ? 2 : 1;
    floatx4 x[NS][S];
#pragma unroll
    for (int h = 0; h < NS; ++h)
#pragma unroll
        for (int sp = 0; sp < S; ++sp) x[h][sp] = src[sp * piece + (int64_t)((h * NA + i) * BM + j) * NT];
    float gv[4], uv[4] = {};
#pragma unroll
    for (int h = 0; h < NS; ++h) {
        floatx4 s = x[h][0];
#pragma unroll
        for (int sp = 1; sp < S; ++sp) s += x[h][sp];
#pragma unroll
        for (int e = 0; e < 4; ++e) (h == 0 ? gv : uv)[e] = s[e];
    }
    const int n_base = tn * TN + wn * Sh::WN + 16 * i + 4 * lq;
    const int m = tm * TM + wm * Sh::WM + 16 * j + l16;
    epilogue4<ACT, BIAS, OutT>(p.o, n_base, m, gv, uv);
}

GemmParams dtl16_params(const LinearDesc& d, int TN, int TM, bool vec_store, bool vec16) {
    GemmParams p{};
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
    p.o.vec_store = vec_store;
    p.o.vec16 = vec16;
    p.M = (int)d.M;
    p.N = (int)d.N;
    p.K = (int)d.K;
    p.tiles_n = (int)ceil_div(d.N, TN);
    p.tiles_m = (int)ceil_div(d.M, TM);
    return p;
}

template <int TN, int TM, bool BIAS, typename OutT>
tp_status_t run_dtl16(const LinearDesc& d, const Ctx& c) {
    if (c.planning()) return TP_OK;  // no work space
    GemmParams p = dtl16_params(d, TN, TM, vec_store_ok<OutT>(d.Y, d.ldy), vec16_ok<OutT>(d.Y, d.ldy));
    const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m;
    // A 4-deep ring (4 x 40 KB, all of a CU's LDS): with the weights cold from HBM, as in the
    // layer, the QKV shard at 4096 tokens takes 90.6 us against 96.8 us with 3 buffers.
    hipLaunchKernelGGL((gemm_dtl16_kernel<TN, TM, 4, kActNone, BIAS, false, OutT>), dim3((unsigned)tiles), dim3(256),
                       0, c.stream, p);
    return hip_status();
}

template <int TN, int TM>
tp_status_t run_dtl16_bias(const LinearDesc& d, const Ctx& c) {
    const bool bias = d.b0 != nullptr;
    if (d.out_dtype == TP_DTYPE_BF16)
        return bias ? run_dtl16<TN, TM, true, bf16>(d, c) : run_dtl16<TN, TM, false, bf16>(d, c);
    return bias ? run_dtl16<TN, TM, true, float>(d, c) : run_dtl16<TN, TM, false, float>(d, c);
}

// Ring depth of the decode tiles: 4 slices of 32 KB (128 x 64 tiles; a fifth measured no
// faster), 3 of 48 KB (96 SwiGLU pairs x 64 tokens), else as many as the LDS holds, at most 10
// (32 pairs x 64 tokens: 10 x 16 KB).
template <int TN, int TM, bool SW>
constexpr int dtl16_decode_stages() {
    constexpr int b = Dtl16Shape<TN, TM, SW>::ROWS * Dtl16Shape<TN, TM, SW>::ROWB;
    return b >= 32 * 1024 ? ((160 * 1024) / b < 4 ? (160 * 1024) / b : 4) : ((160 * 1024) / b > 10 ? 10 : (160 * 1024) / b);
}

// Up to 64 tokens: every tile cut into S K ranges (S pieces per tile fill at most one wave of
// CUs, each at least 4 slices, S <= 16), then the reduce pass; S = 1 runs whole tiles.
template <int TN, int TM, int ACT, bool BIAS, typename OutT, int S>
tp_status_t run_dtl16_split_s(GemmParams p, int64_t tiles, const Ctx& c) {
    using Sh = Dtl16Shape<TN, TM, ACT == kActSwiglu>;
    constexpr int ST = dtl16_decode_stages<TN, TM, ACT == kActSwiglu>();
    hipLaunchKernelGGL((gemm_dtl16_kernel<TN, TM, ST, ACT, BIAS, true, OutT>), dim3((unsigned)(tiles * S)), dim3(256), 0,
                       c.stream, p);
    const tp_status_t st = hip_status();
    if (st != TP_OK) return st;
    hipLaunchKernelGGL((splitk16_reduce_kernel<TN, TM, ACT, BIAS, OutT, S>), dim3((unsigned)(tiles * Sh::NA * Sh::BM)),
                       dim3(256), 0, c.stream, p);
    return hip_status();
}

template <int TN, int TM, int ACT, bool BIAS, typename OutT>
tp_status_t run_dtl16_split(const LinearDesc& d, int cus, const Ctx& c) {
    GemmParams p = dtl16_params(d, TN, TM, vec_store_ok<OutT>(d.Y, d.ldy), vec16_ok<OutT>(d.Y, d.ldy));
    const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m;
    const int64_t kt = d.K / DBK;
    const int S = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)cus / tiles, kt / 4, 16}));
    if (S == 1) {  // the tiles alone fill the chip: whole K per workgroup, no partials
        if (c.planning()) return TP_OK;
        constexpr int ST = dtl16_decode_stages<TN, TM, ACT == kActSwiglu>();
        hipLaunchKernelGGL((gemm_dtl16_kernel<TN, TM, ST, ACT, BIAS, false, OutT>), dim3((unsigned)tiles), dim3(256), 0,
                           c.stream, p);
        return hip_status();
    }
    // S > 1 only when tiles * S <= cus: at most cus fp32 partial tiles.
    const WsNeed need{(size_t)(tiles * S * Dtl16Shape<TN, TM, ACT == kActSwiglu>::NG * 1024), 0};
    if (c.planning()) {
        c.need->merge(need);
        return TP_OK;
    }
    if (!c.ws || !c.ws->covers(need)) return TP_ERR_WORKSPACE;
    p.S = S;
    p.ws = c.ws->partials;
    switch (S) {
        case 2: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 2>(p, tiles, c);
        case 3: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 3>(p, tiles, c);
        case 4: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 4>(p, tiles, c);
        case 5: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 5>(p, tiles, c);
        case 6: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 6>(p, tiles, c);
        case 7: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 7>(p, tiles, c);
        case 8: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 8>(p, tiles, c);
        case 9: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 9>(p, tiles, c);
        case 10: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 10>(p, tiles, c);
        case 11: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 11>(p, tiles, c);
        case 12: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 12>(p, tiles, c);
        case 13: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 13>(p, tiles, c);
        case 14: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 14>(p, tiles, c);
        case 15: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 15>(p, tiles, c);
        default: return run_dtl16_split_s<TN, TM, ACT, BIAS, OutT, 16>(p, tiles, c);
    }
}

template <int TN, int TM, int ACT>
tp_status_t run_dtl16_split_bias(const LinearDesc& d, int cus, const Ctx& c) {
    const bool bias = d.b0 != nullptr;
    if (d.out_dtype == TP_DTYPE_BF16)
        return bias ? run_dtl16_split<TN, TM, ACT, true, bf16>(d, cus, c)
                    : run_dtl16_split<TN, TM, ACT, false, bf16>(d, cus, c);
    return bias ? run_dtl16_split<TN, TM, ACT, true, float>(d, cus, c)
                : run_dtl16_split<TN, TM, ACT, false, float>(d, cus, c);
}

template <int TN, int TM, int WAVES_N, int WAVES_M, int ACT, bool BIAS, typename OutT>
tp_status_t run_dtl(const LinearDesc& d, int cus, const Ctx& c) {
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
    p.o.vec16 = vec16_ok<OutT>(d.Y, d.ldy);
    p.M = (int)d.M;
    p.N = (int)d.N;
    p.K = (int)d.K;
    p.tiles_n = (int)ceil_div(d.N, TN);
    p.tiles_m = (int)ceil_div(d.M, TM);
    p.F = 0;
    p.S = 0;
    p.ws = nullptr;
    const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m;
    constexpr unsigned NT = WAVES_N * WAVES_M * 64;
    // One tile per workgroup when whole waves of tiles fill the chip to 90 %. Else
    // the whole waves stay one tile per workgroup and the R remaining tiles are cut
    // into S K ranges, S (at least 8 slices each) chosen so the pieces
    // take the least time on `cus` CUs: ceil(R*S / cus) / S tile times. A split is
    // only taken where it saves at least a third of a tile time: the partials cost
    // a pass of their own.
    const int64_t kt = d.K / DBK;
    const int64_t F = tiles / cus * cus, R = tiles - F;
    int S = 1;
    if (R > 0 && tiles * 10 < ceil_div(tiles, (int64_t)cus) * cus * 9) {
        double best = 2.0 / 3.0;
        // Up to 8 ranges for plain products, 4 for the SwiGLU pair (twice the partials).
        for (int s = 2; s <= (ACT == kActSwiglu ? 4 : 8) && kt / s >= 8; ++s) {
            const double tm = (double)ceil_div(R * s, (int64_t)cus) / s;
            if (tm < best - 1e-9) { best = tm; S = s; }
        }
    }
    if (S == 1) {
        if (c.planning()) return TP_OK;
        hipLaunchKernelGGL((gemm_dtl_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, false, OutT>), dim3((unsigned)tiles),
                           dim3(NT), 0, c.stream, p);
        return hip_status();
    }
    constexpr int64_t TILEF = (int64_t)TN * (ACT == kActSwiglu ? 2 : 1) * TM;  // floats of a partial tile
    const WsNeed need{(size_t)(R * S * TILEF), 0};
    if (c.planning()) {
        c.need->merge(need);
        return TP_OK;
    }
    if (!c.ws || !c.ws->covers(need)) return TP_ERR_WORKSPACE;
    p.F = (int)F;
    p.S = S;
    p.ws = c.ws->partials;
    hipLaunchKernelGGL((gemm_dtl_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, true, OutT>),
                       dim3((unsigned)(F + R * S)), dim3(NT), 0, c.stream, p);
    const tp_status_t st = hip_status();
    if (st != TP_OK) return st;
    constexpr int BN = TN / WAVES_N / 32, BM = TM / WAVES_M / 32;
    const dim3 rgrid((unsigned)(R * BN * BM));
    if (S == 2)
        hipLaunchKernelGGL((splitk_reduce_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, OutT, 2>), rgrid, dim3(NT), 0,
                           c.stream, p);
    else if (S == 3)
        hipLaunchKernelGGL((splitk_reduce_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, OutT, 3>), rgrid, dim3(NT), 0,
                           c.stream, p);
    else if (S == 4)
        hipLaunchKernelGGL((splitk_reduce_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, OutT, 4>), rgrid, dim3(NT), 0,
                           c.stream, p);
    else if constexpr (ACT != kActSwiglu) {
        if (S == 5)
            hipLaunchKernelGGL((splitk_reduce_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, OutT, 5>), rgrid, dim3(NT), 0,
                               c.stream, p);
        else if (S == 6)
            hipLaunchKernelGGL((splitk_reduce_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, OutT, 6>), rgrid, dim3(NT), 0,
                               c.stream, p);
        else if (S == 7)
            hipLaunchKernelGGL((splitk_reduce_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, OutT, 7>), rgrid, dim3(NT), 0,
                               c.stream, p);
        else
            hipLaunchKernelGGL((splitk_reduce_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, OutT, 8>), rgrid, dim3(NT), 0,
                               c.stream, p);
    }
    return hip_status();
}

template <int TN, int TM, int WAVES_N, int WAVES_M, int ACT>
tp_status_t run_dtl_bias(const LinearDesc& d, int cus, const Ctx& c) {
    const bool bias = d.b0 != nullptr;
    if (d.out_dtype == TP_DTYPE_BF16)
        return bias ? run_dtl<TN, TM, WAVES_N, WAVES_M, ACT, true, bf16>(d, cus, c)
                    : run_dtl<TN, TM, WAVES_N, WAVES_M, ACT, false, bf16>(d, cus, c);
    return bias ? run_dtl<TN, TM, WAVES_N, WAVES_M, ACT, true, float>(d, cus, c)
                : run_dtl<TN, TM, WAVES_N, WAVES_M, ACT, false, float>(d, cus, c);
}

template <int TN, int TM, int WAVES_N, int WAVES_M, int ACT, bool BIAS, bool KTAIL, typename OutT>
tp_status_t run(const LinearDesc& d, const Ctx& c) {
    if (c.planning()) return TP_OK;  // no work space
    const hipStream_t stream = c.stream;
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
    p.o.vec16 = vec16_ok<OutT>(d.Y, d.ldy);
    p.M = (int)d.M;
    p.N = (int)d.N;
    p.K = (int)d.K;
    p.tiles_n = (int)ceil_div(d.N, TN);
    p.tiles_m = (int)ceil_div(d.M, TM);
    const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m;
    hipLaunchKernelGGL((gemm_kernel<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, KTAIL, OutT>), dim3((unsigned)tiles),
                       dim3(WAVES_N * WAVES_M * 64), 0, stream, p);
    return hip_status();
}

template <int TN, int TM, int WAVES_N, int WAVES_M, int ACT, bool BIAS, bool KTAIL>
tp_status_t run_out(const LinearDesc& d, const Ctx& c) {
    return d.out_dtype == TP_DTYPE_BF16 ? run<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, KTAIL, bf16>(d, c)
                                        : run<TN, TM, WAVES_N, WAVES_M, ACT, BIAS, KTAIL, float>(d, c);
}

template <int TN, int TM, int WAVES_N, int WAVES_M, int ACT>
tp_status_t run_bias(const LinearDesc& d, const Ctx& c) {
    const bool bias = d.b0 != nullptr;
    const bool ktail = d.K % BK != 0;
    if (bias)
        return ktail ? run_out<TN, TM, WAVES_N, WAVES_M, ACT, true, true>(d, c)
                     : run_out<TN, TM, WAVES_N, WAVES_M, ACT, true, false>(d, c);
    return ktail ? run_out<TN, TM, WAVES_N, WAVES_M, ACT, false, true>(d, c)
                 : run_out<TN, TM, WAVES_N, WAVES_M, ACT, false, false>(d, c);
}

}  // namespace

namespace {
int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        return n;
    return 256;
}

// A SwiGLU pair of 17-48 tokens whose 32-pair tiles fill 80-100 % of the CUs: whole-K tiles
// of 32 pairs x 64 tokens in a 10-deep ring, no partials (70B TP=4 gate/up at 32 tokens: 52.9 ->
// 48.2 us). At 64 tokens, and for plain products, no faster or slower. At 1-16 tokens the
// gain depends on the box (4-16 tokens 5-12 % faster on one, equal on another, and at one token
// 47.4 -> 50.0 us): the decode kernel keeps those.
bool swiglu_pairs32(const LinearDesc& d, int cus) {
    const int64_t t32 = ceil_div(d.N, 32);
    return d.swiglu && d.M > 16 && d.M <= 48 && t32 * 10 >= (int64_t)cus * 8 && t32 <= cus;
}
}  // namespace

bool gemm_takes_decode(const LinearDesc& d) {
    if (d.M > 64 || d.gelu || d.K % DBK != 0 || d.K < 2048) return false;
    return d.M > (d.swiglu ? 16 : 20);
}

tp_status_t launch_gemm(const LinearDesc& d, const Ctx& c) {
    // Byte offsets inside an operand are 32-bit.
    if ((int64_t)d.N * d.K * 2 >= (int64_t(1) << 32) || (int64_t)d.M * d.ldx * 2 >= (int64_t(1) << 32))
        return TP_ERR_SHAPE;
    const int cus = device_cus();
    // Large tiles (256 x 256, or 128 x 256 with the SwiGLU pair, one workgroup per CU)
    // when they fill the chip; with K a whole number of slices they run on the LDS-DMA
    // kernel with 8 waves of 128 x 64 outputs (SwiGLU: 16 waves of 32 pairs x 64), so a
    // SIMD holds 2 (4) waves and one's MFMAs cover another's waits on the DMA and L2
    // misses (measured in the layer step, where each shard's weights come cold from
    // HBM: 907 -> 992 TFLOP/s over 4 waves of 128 x 128); the DMA kernel also takes
    // fewer tiles than CUs, split in K, once each CU gets at least 16 slices of work, or,
    // for plain products with K >= 2048, 8 slices, or with K >= 4096 whenever 128 x 128
    // tiles would leave half the CUs idle (measured on the 70B QKV shard at 1024 / 512
    // tokens: 89 / 95 us on 80 / 40 register-staged 128 x 128 tiles, 42 / 40 us split; that
    // shard now takes the 160 x 128 tiles, which come first for plain products whose tiles,
    // whole or cut in K, fill the chip). Short K stays off the split: its pieces cannot pay
    // for the partials (O shard at 1024 tokens, K = 1024: 28 us as 512 register-staged
    // tiles, 47 us split). Otherwise register-staged 256 x 256 or 128 x 128 tiles.
    const bool dma = d.K % DBK == 0;
    const int64_t kt = d.K / DBK;
    // Decode shapes that gemm_takes_decode accepts: 64-token tiles of 128 features (SwiGLU: 96
    // pairs; 7B TP=2 gate/up at 64 tokens 25.4 -> 24.1 us against 64 pairs, whose 86 tiles x 2
    // K ranges filled 172 CUs) per piece, K cut so that the pieces fill the chip, or whole-K
    // tiles of 32 pairs.
    if (d.M <= 64) {
        if (!gemm_takes_decode(d)) return TP_ERR_SHAPE;  // the decode kernels' shapes
        if (swiglu_pairs32(d, cus)) return run_dtl16_split_bias<32, 64, kActSwiglu>(d, cus, c);
        if (d.swiglu) return run_dtl16_split_bias<96, 64, kActSwiglu>(d, cus, c);
        return run_dtl16_split_bias<128, 64, kActNone>(d, cus, c);
    }
    if (d.swiglu) {
        const int64_t big = ceil_div(d.N, 128) * ceil_div(d.M, 256);
        if (dma && (big >= cus || big * kt >= 16 * (int64_t)cus))
            return run_dtl_bias<128, 256, 4, 4, kActSwiglu>(d, cus, c);
        if (big >= cus) return run_bias<128, 256, 2, 2, kActSwiglu>(d, c);
        return run_bias<64, 128, 2, 2, kActSwiglu>(d, c);
    }
    const int64_t big = ceil_div(d.N, 256) * ceil_div(d.M, 256);
    auto plain = [&](auto act) -> tp_status_t {
        constexpr int A = decltype(act)::value;
        const int64_t small = ceil_div(d.N, 128) * ceil_div(d.M, 128);
        // Fewer 256 x 256 tiles than CUs, but whole waves of 160 x 128 tiles (filled to 90 %)
        // and a long K: one tile per workgroup on 16-row MFMA blocks instead of K ranges and
        // a reduce pass (the 70B TP=8 QKV shard at 4096 tokens: 256 tiles).
        const int64_t t16 = ceil_div(d.N, 160) * ceil_div(d.M, 128);
        if (dma && A == kActNone && big < cus && kt >= 32 && t16 >= cus &&
            t16 * 10 >= ceil_div(t16, (int64_t)cus) * cus * 9)
            return run_dtl16_bias<160, 128>(d, c);
        // Fewer: each tile cut into the S K ranges (at most 16, each >= 4 slices) that fill the
        // chip to 90 %, summed by the reduce pass; 70B TP=8 QKV shard against 256 x 256 tiles cut
        // in K: 2048 tokens 61.2 -> 55.1 us (2 ranges), 1024 42.2 -> 33.0 (4), 512 38.0 -> 23.2 (8).
        const int64_t s16 = std::max<int64_t>(1, std::min<int64_t>({(int64_t)cus / std::max<int64_t>(t16, 1), kt / 4, 16}));
        if (dma && A == kActNone && big < cus && kt >= 32 && t16 < cus && t16 * s16 * 10 >= (int64_t)cus * 9)
            return run_dtl16_split_bias<160, 128, kActNone>(d, cus, c);
        if (dma && (big >= cus || big * kt >= 16 * (int64_t)cus || (kt >= 32 && big * kt >= 8 * (int64_t)cus) ||
                    (kt >= 64 && 2 * small <= cus)))
            return run_dtl_bias<256, 256, 2, 4, A>(d, cus, c);
        if (big >= cus) return run_bias<256, 256, 2, 2, A>(d, c);
        return run_bias<128, 128, 2, 2, A>(d, c);
    };
    return d.gelu ? plain(std::integral_constant<int, kActGelu>{}) : plain(std::integral_constant<int, kActNone>{});
}

}  // namespace tp
