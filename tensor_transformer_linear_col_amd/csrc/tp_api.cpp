// C ABI of the tensor-parallel shard library: host-side validation, then kernel
// launches on the caller's stream. See include/tp_linear.h for the contract.
#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "tp_internal.h"

using namespace tp;

namespace {

constexpr int32_t kMaxTP = 64;
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

bool dtype_ok(tp_dtype_t d) { return d == TP_DTYPE_F32 || d == TP_DTYPE_BF16; }
size_t elem_size(tp_dtype_t d) { return d == TP_DTYPE_F32 ? 4 : 2; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// bf16 operands are read with 16-byte loads: base and row stride must allow it.
tp_status_t check_vec_operand(const void* p, int64_t ld_elems, tp_dtype_t dt) {
    if (dt != TP_DTYPE_BF16) return TP_OK;
    if (!aligned16(p) || (ld_elems * 2) % 16 != 0) return TP_ERR_ALIGN;
    return TP_OK;
}

tp_status_t check_dims(int64_t M, std::initializer_list<int64_t> pos) {
    if (M < 0 || M > kMaxDim) return TP_ERR_SHAPE;
    for (int64_t v : pos)
        if (v <= 0 || v > kMaxDim) return TP_ERR_SHAPE;
    return TP_OK;
}


tp_status_t launch_linear(const LinearDesc& d, const Ctx& c) {
    if (d.M == 0) return TP_OK;
    if (d.in_dtype == TP_DTYPE_F32) return launch_f32(d, c);
    // 1-4 tokens with fewer 16-feature row groups than CUs: the MFMA decode kernel would cut
    // K across workgroups (a partial-sum hand-off of several memory round trips at the end);
    // the GEMV kernel splits the features one by one instead (70B QKV shard at TP=8 and one
    // token: 10.3 -> 8.4 us). With enough row groups the MFMA kernel stays faster.
    if (d.M <= 4 && gemv_chunks(d.K, nullptr) != 0 && ceil_div(d.N, 16) < gemv_cus()) return launch_gemv(d, c);
    // Decode shapes with the tokens staged once per workgroup in LDS, shared by its waves,
    // instead of reloaded by every wave of the decode kernel (gemm_takes_decode: 17-64 tokens
    // of a SwiGLU pair, 21-64 of a plain product, K >= 2048; 70B TP=4 at 64 tokens: gate/up
    // 64.4 -> 49.9 us, down 40.0 -> 28.6 us). Fewer tokens and short K stay on the decode kernel.
    if (d.M <= 64 && gemm_takes_decode(d)) return launch_gemm(d, c);
    if (d.M <= 64) return launch_skinny(d, c);
    return launch_gemm(d, c);
}

// KV heads a shard holds: G/p when p divides G; one (replicated on p/G consecutive
// shards) when p is a multiple of G; 0 (invalid) otherwise.
int64_t kv_heads_per_shard(int64_t n_kv_heads, int64_t p) {
    if (n_kv_heads % p == 0) return n_kv_heads / p;
    if (p % n_kv_heads == 0) return 1;
    return 0;
}

// ---- work space: reserved by the caller, one per (device, stream) -------------------
struct WsEntry {
    void* base = nullptr;
    size_t partial_floats = 0;
    size_t counters = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, WsEntry> g_ws;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Dry run (tp_plan_begin .. tp_plan_end) of this host thread: calls validate and
// record the largest work space any of them needs, and enqueue nothing.
thread_local bool t_planning = false;
thread_local WsNeed t_plan;

Workspace view_of(const WsEntry& e) {
    Workspace w;
    w.counters = static_cast<unsigned*>(e.base);
    w.n_counters = e.counters;
    w.partials = reinterpret_cast<float*>(static_cast<char*>(e.base) + round_up(e.counters * sizeof(unsigned), 256));
    w.partial_floats = e.partial_floats;
    return w;
}

// The reserved work space of the current device and `stream`, if it covers `need`.
tp_status_t find_workspace(hipStream_t stream, const WsNeed& need, Workspace* out) {
    *out = Workspace{};
    if (need.empty()) return TP_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TP_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto it = g_ws.find({dev, stream});
    if (it == g_ws.end() || it->second.base == nullptr) return TP_ERR_WORKSPACE;
    *out = view_of(it->second);
    return out->covers(need) ? TP_OK : TP_ERR_WORKSPACE;
}

// Runs an entry point's launches: first all of them in plan mode (every check, the
// work space they need; nothing enqueued), then, unless this thread is planning, all
// of them for real. So a call that fails enqueues nothing.
template <typename Body>
tp_status_t planned(hipStream_t stream, Body&& body) {
    WsNeed need;
    const Ctx plan{stream, nullptr, &need};
    TP_TRY(body(plan));
    if (t_planning) {
        t_plan.merge(need);
        return TP_OK;
    }
    Workspace ws;
    TP_TRY(find_workspace(stream, need, &ws));
    const Ctx go{stream, &ws, nullptr};
    return body(go);
}

// Validation shared by tp_mlp_shard and its allocation-free variant.
tp_status_t mlp_descs(const void* X, const void* Wg_r, const void* Wu_r, const void* bg_r, const void* bu_r,
                      const void* Wd_r, void* H_r, void* P_r, int64_t M, int64_t hidden, int64_t intermediate,
                      int32_t tp_size, tp_dtype_t dtype, tp_dtype_t partial_dtype, LinearDesc* up, LinearDesc* down) {
    if (!X || !Wg_r || !Wu_r || !H_r) return TP_ERR_NULL;
    if (P_r && !Wd_r) return TP_ERR_NULL;
    if ((bg_r == nullptr) != (bu_r == nullptr)) return TP_ERR_NULL;
    if (!dtype_ok(dtype) || !dtype_ok(partial_dtype)) return TP_ERR_DTYPE;
    if (dtype == TP_DTYPE_F32 && partial_dtype != TP_DTYPE_F32) return TP_ERR_DTYPE;
    TP_TRY(check_dims(M, {hidden, intermediate}));
    if (tp_size < 1 || tp_size > kMaxTP) return TP_ERR_SHAPE;
    if (intermediate % tp_size != 0) return TP_ERR_INDIVISIBLE;
    const int64_t i = intermediate / tp_size;
    TP_TRY(check_vec_operand(X, hidden, dtype));
    TP_TRY(check_vec_operand(Wg_r, hidden, dtype));
    TP_TRY(check_vec_operand(Wu_r, hidden, dtype));
    if (P_r) {
        TP_TRY(check_vec_operand(H_r, i, dtype));
        TP_TRY(check_vec_operand(Wd_r, i, dtype));
    }
    *up = LinearDesc{X, hidden, Wg_r, Wu_r, bg_r, bu_r, H_r, i, M, i, hidden, dtype, dtype, true};
    *down = LinearDesc{H_r, i, Wd_r, nullptr, nullptr, nullptr, P_r, hidden, M, hidden, i, dtype, partial_dtype, false};
    return TP_OK;
}

// ---- scratch of the allocation-free entry point --------------------------------------
// A fixed device array, one copy per GPU the library runs on, held until the process ends:
// the arrival counters first, then the fp32 partial sums. In host code the array's name is
// only a stand-in; its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchCounters = size_t(1) << 16;
constexpr size_t kScratchPartialBytes = size_t(16) << 20;
constexpr size_t kScratchCounterBytes = kScratchCounters * sizeof(unsigned);
static __device__ __align__(256) unsigned char scratch[kScratchCounterBytes + kScratchPartialBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

tp_status_t scratch_of_current_device(Workspace* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TP_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TP_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    char* base = static_cast<char*>(g_scratch_ptr[dev]);
    out->counters = reinterpret_cast<unsigned*>(base);
    out->n_counters = kScratchCounters;
    out->partials = reinterpret_cast<float*>(base + kScratchCounterBytes);
    out->partial_floats = kScratchPartialBytes / sizeof(float);
    return TP_OK;
}

}  // namespace

extern "C" {

const char* tp_status_string(tp_status_t s) {
    switch (s) {
        case TP_OK: return "TP_OK";
        case TP_ERR_NULL: return "TP_ERR_NULL: a required pointer is NULL";
        case TP_ERR_SHAPE: return "TP_ERR_SHAPE: invalid size, stride, tp_size or rank";
        case TP_ERR_INDIVISIBLE: return "TP_ERR_INDIVISIBLE: a split size is not divisible by tp_size";
        case TP_ERR_DTYPE: return "TP_ERR_DTYPE: unsupported dtype combination";
        case TP_ERR_ALIGN: return "TP_ERR_ALIGN: a bf16 operand or its row stride is not 16-byte aligned";
        case TP_ERR_HIP: return "TP_ERR_HIP: the HIP runtime reported an error";
        case TP_ERR_WORKSPACE:
            return "TP_ERR_WORKSPACE: the work space reserved for this device and stream is too small "
                   "(size it with tp_plan_begin/tp_plan_end, reserve it with tp_workspace_reserve)";
    }
    return "unknown tp_status_t";
}

tp_status_t tp_linear_col(const void* X, const void* W_r, const void* b_r, void* Y_r, int64_t M,
                          int64_t in_features, int64_t out_features, int32_t tp_size, tp_dtype_t dtype,
                          void* stream) {
    if (!X || !W_r || !Y_r) return TP_ERR_NULL;
    if (!dtype_ok(dtype)) return TP_ERR_DTYPE;
    TP_TRY(check_dims(M, {in_features, out_features}));
    if (tp_size < 1 || tp_size > kMaxTP) return TP_ERR_SHAPE;
    if (out_features % tp_size != 0) return TP_ERR_INDIVISIBLE;
    const int64_t n = out_features / tp_size;
    TP_TRY(check_vec_operand(X, in_features, dtype));
    TP_TRY(check_vec_operand(W_r, in_features, dtype));
    const LinearDesc d{X, in_features, W_r, nullptr, b_r, nullptr, Y_r, n, M, n, in_features, dtype, dtype, false};
    return planned(static_cast<hipStream_t>(stream), [&](const Ctx& c) { return launch_linear(d, c); });
}

tp_status_t tp_linear_row_partial(const void* X_r, int64_t ldx, const void* W_r, void* P_r, int64_t M,
                                  int64_t in_features, int64_t out_features, int32_t tp_size, tp_dtype_t dtype,
                                  tp_dtype_t partial_dtype, void* stream) {
    if (!X_r || !W_r || !P_r) return TP_ERR_NULL;
    if (!dtype_ok(dtype) || !dtype_ok(partial_dtype)) return TP_ERR_DTYPE;
    if (dtype == TP_DTYPE_F32 && partial_dtype != TP_DTYPE_F32) return TP_ERR_DTYPE;
    TP_TRY(check_dims(M, {in_features, out_features}));
    if (tp_size < 1 || tp_size > kMaxTP) return TP_ERR_SHAPE;
    if (in_features % tp_size != 0) return TP_ERR_INDIVISIBLE;
    const int64_t k = in_features / tp_size;
    if (ldx < k) return TP_ERR_SHAPE;
    TP_TRY(check_vec_operand(X_r, ldx, dtype));
    TP_TRY(check_vec_operand(W_r, k, dtype));
    const LinearDesc d{X_r, ldx, W_r, nullptr, nullptr, nullptr, P_r, out_features, M, out_features, k, dtype,
                       partial_dtype, false};
    return planned(static_cast<hipStream_t>(stream), [&](const Ctx& c) { return launch_linear(d, c); });
}

tp_status_t tp_mlp_shard(const void* X, const void* Wg_r, const void* Wu_r, const void* bg_r, const void* bu_r,
                         const void* Wd_r, void* H_r, void* P_r, int64_t M, int64_t hidden, int64_t intermediate,
                         int32_t tp_size, tp_dtype_t dtype, tp_dtype_t partial_dtype, void* stream) {
    LinearDesc up, down;
    TP_TRY(mlp_descs(X, Wg_r, Wu_r, bg_r, bu_r, Wd_r, H_r, P_r, M, hidden, intermediate, tp_size, dtype,
                     partial_dtype, &up, &down));
    return planned(static_cast<hipStream_t>(stream), [&](const Ctx& c) {
        TP_TRY(launch_linear(up, c));
        return P_r ? launch_linear(down, c) : TP_OK;
    });
}

tp_status_t tp_mlp_shard_noalloc(const void* X, const void* Wg_r, const void* Wu_r, const void* bg_r,
                                 const void* bu_r, const void* Wd_r, void* H_r, void* P_r, int64_t M, int64_t hidden,
                                 int64_t intermediate, int32_t tp_size, tp_dtype_t dtype, tp_dtype_t partial_dtype,
                                 void* stream) {
    LinearDesc up, down;
    TP_TRY(mlp_descs(X, Wg_r, Wu_r, bg_r, bu_r, Wd_r, H_r, P_r, M, hidden, intermediate, tp_size, dtype,
                     partial_dtype, &up, &down));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    auto body = [&](const Ctx& c) {
        TP_TRY(launch_linear(up, c));
        return P_r ? launch_linear(down, c) : TP_OK;
    };
    WsNeed need;
    TP_TRY(body(Ctx{s, nullptr, &need}));
    if (need.partial_floats * sizeof(float) > kScratchPartialBytes || need.counters > kScratchCounters)
        return TP_ERR_WORKSPACE;
    if (t_planning) return TP_OK;  // it needs no reserved work space
    Workspace ws;
    if (!need.empty()) {
        TP_TRY(scratch_of_current_device(&ws));
        // The array keeps the previous call's contents: the counters this call uses start at zero.
        if (need.counters) TP_TRY(launch_fill_u32(ws.counters, need.counters, 0u, s));
    }
    return body(Ctx{s, &ws, nullptr});
}

tp_status_t tp_ffn_gelu_shard(const void* X, const void* W1_r, const void* b1_r, const void* W2_r, void* H_r,
                              void* P_r, int64_t M, int64_t hidden, int64_t intermediate, int32_t tp_size,
                              tp_dtype_t dtype, tp_dtype_t partial_dtype, void* stream) {
    if (!X || !W1_r || !H_r) return TP_ERR_NULL;
    if (P_r && !W2_r) return TP_ERR_NULL;
    if (!dtype_ok(dtype) || !dtype_ok(partial_dtype)) return TP_ERR_DTYPE;
    if (dtype == TP_DTYPE_F32 && partial_dtype != TP_DTYPE_F32) return TP_ERR_DTYPE;
    TP_TRY(check_dims(M, {hidden, intermediate}));
    if (tp_size < 1 || tp_size > kMaxTP) return TP_ERR_SHAPE;
    if (intermediate % tp_size != 0) return TP_ERR_INDIVISIBLE;
    const int64_t i = intermediate / tp_size;
    TP_TRY(check_vec_operand(X, hidden, dtype));
    TP_TRY(check_vec_operand(W1_r, hidden, dtype));
    if (P_r) {
        TP_TRY(check_vec_operand(H_r, i, dtype));
        TP_TRY(check_vec_operand(W2_r, i, dtype));
    }
    const LinearDesc up{X, hidden, W1_r, nullptr, b1_r, nullptr, H_r, i, M, i, hidden, dtype, dtype, false, true};
    const LinearDesc down{H_r, i, W2_r, nullptr, nullptr, nullptr, P_r, hidden, M, hidden, i, dtype, partial_dtype, false};
    return planned(static_cast<hipStream_t>(stream), [&](const Ctx& c) {
        TP_TRY(launch_linear(up, c));
        return P_r ? launch_linear(down, c) : TP_OK;
    });
}

tp_status_t tp_attn_proj_shard(const void* X, const void* Wqkv_r, const void* bqkv_r, void* QKV_r, const void* A_r,
                               const void* Wo_r, void* P_r, int64_t M, int64_t hidden, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t tp_size, tp_dtype_t dtype,
                               tp_dtype_t partial_dtype, void* stream) {
    if (QKV_r && (!X || !Wqkv_r)) return TP_ERR_NULL;
    if (P_r && (!A_r || !Wo_r)) return TP_ERR_NULL;
    if (!dtype_ok(dtype) || !dtype_ok(partial_dtype)) return TP_ERR_DTYPE;
    if (dtype == TP_DTYPE_F32 && partial_dtype != TP_DTYPE_F32) return TP_ERR_DTYPE;
    TP_TRY(check_dims(M, {hidden, n_heads, n_kv_heads, head_dim}));
    if (tp_size < 1 || tp_size > kMaxTP) return TP_ERR_SHAPE;
    if (n_heads % tp_size != 0 || kv_heads_per_shard(n_kv_heads, tp_size) == 0) return TP_ERR_INDIVISIBLE;
    const int64_t hq = n_heads / tp_size, hk = kv_heads_per_shard(n_kv_heads, tp_size);
    const int64_t nqkv = (hq + 2 * hk) * head_dim;
    const int64_t ka = hq * head_dim;
    if (nqkv > kMaxDim) return TP_ERR_SHAPE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (QKV_r) {
        TP_TRY(check_vec_operand(X, hidden, dtype));
        TP_TRY(check_vec_operand(Wqkv_r, hidden, dtype));
    }
    if (P_r) {
        TP_TRY(check_vec_operand(A_r, ka, dtype));
        TP_TRY(check_vec_operand(Wo_r, ka, dtype));
    }
    const LinearDesc q{X, hidden, Wqkv_r, nullptr, bqkv_r, nullptr, QKV_r, nqkv, M, nqkv, hidden, dtype, dtype, false};
    const LinearDesc o{A_r, ka, Wo_r, nullptr, nullptr, nullptr, P_r, hidden, M, hidden, ka, dtype, partial_dtype, false};
    return planned(s, [&](const Ctx& c) {
        if (QKV_r) TP_TRY(launch_linear(q, c));
        return P_r ? launch_linear(o, c) : TP_OK;
    });
}

tp_status_t tp_attn_core_shard(const void* QKV_r, void* A_r, int64_t M, int32_t n_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t tp_size, int32_t causal, tp_dtype_t dtype, void* stream) {
    if (!QKV_r || !A_r) return TP_ERR_NULL;
    if (dtype != TP_DTYPE_BF16) return TP_ERR_DTYPE;
    TP_TRY(check_dims(M, {n_heads, n_kv_heads}));
    if (tp_size < 1 || tp_size > kMaxTP) return TP_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return TP_ERR_SHAPE;
    if (n_heads % tp_size != 0 || kv_heads_per_shard(n_kv_heads, tp_size) == 0) return TP_ERR_INDIVISIBLE;
    const int64_t hq = n_heads / tp_size, hk = kv_heads_per_shard(n_kv_heads, tp_size);
    if (hq % hk != 0) return TP_ERR_INDIVISIBLE;  // query heads grouped evenly over the KV heads
    const int64_t ldq = (hq + 2 * hk) * head_dim, lda = hq * head_dim;
    TP_TRY(check_vec_operand(QKV_r, ldq, dtype));
    TP_TRY(check_vec_operand(A_r, lda, dtype));
    if (M == 0) return TP_OK;
    return planned(static_cast<hipStream_t>(stream), [&](const Ctx& c) {
        return launch_attn_core(QKV_r, ldq, A_r, lda, M, (int)hq, (int)hk, head_dim, causal != 0, c);
    });
}

tp_status_t tp_attn_decode_shard(const void* QKV_r, void* K_cache_r, void* V_cache_r, int64_t cache_len,
                                 int64_t capacity, void* A_r, int64_t M, int32_t n_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t tp_size, tp_dtype_t dtype, void* stream) {
    if (!QKV_r || !K_cache_r || !V_cache_r || !A_r) return TP_ERR_NULL;
    if (dtype != TP_DTYPE_BF16) return TP_ERR_DTYPE;
    TP_TRY(check_dims(M, {n_heads, n_kv_heads}));
    if (tp_size < 1 || tp_size > kMaxTP) return TP_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return TP_ERR_SHAPE;
    if (cache_len < 0 || capacity < 0 || capacity > kMaxDim || cache_len + M > capacity) return TP_ERR_SHAPE;
    if (n_heads % tp_size != 0 || kv_heads_per_shard(n_kv_heads, tp_size) == 0) return TP_ERR_INDIVISIBLE;
    const int64_t hq = n_heads / tp_size, hk = kv_heads_per_shard(n_kv_heads, tp_size);
    if (hq % hk != 0) return TP_ERR_INDIVISIBLE;
    const int64_t ldq = (hq + 2 * hk) * head_dim, ldkv = hk * head_dim, lda = hq * head_dim;
    TP_TRY(check_vec_operand(QKV_r, ldq, dtype));
    TP_TRY(check_vec_operand(K_cache_r, ldkv, dtype));
    TP_TRY(check_vec_operand(V_cache_r, ldkv, dtype));
    TP_TRY(check_vec_operand(A_r, lda, dtype));
    // The kernel addresses the used part of a cache with 32-bit byte offsets.
    if ((cache_len + M) * ldkv * 2 >= (int64_t(1) << 31)) return TP_ERR_SHAPE;
    if (M == 0) return TP_OK;
    return planned(static_cast<hipStream_t>(stream), [&](const Ctx& c) {
        return launch_attn_decode(QKV_r, ldq, K_cache_r, V_cache_r, ldkv, cache_len, A_r, lda, M, (int)hq, (int)hk,
                                  head_dim, c);
    });
}

tp_status_t tp_combine_concat(const void* const* shards, int32_t tp_size, const int64_t* seg_widths, int32_t nseg,
                              void* Y, int64_t M, tp_dtype_t dtype, void* stream) {
    if (!shards || !seg_widths || !Y) return TP_ERR_NULL;
    if (!dtype_ok(dtype)) return TP_ERR_DTYPE;
    if (tp_size < 1 || tp_size > kMaxTP || nseg < 1 || nseg > 8 || M < 0 || M > kMaxDim) return TP_ERR_SHAPE;
    for (int32_t r = 0; r < tp_size; ++r)
        if (!shards[r]) return TP_ERR_NULL;
    for (int32_t j = 0; j < nseg; ++j)
        if (seg_widths[j] <= 0 || seg_widths[j] > kMaxDim) return TP_ERR_SHAPE;
    if (t_planning) return TP_OK;
    return launch_concat(shards, tp_size, seg_widths, nseg, Y, M, elem_size(dtype), static_cast<hipStream_t>(stream));
}

tp_status_t tp_combine_sum(const void* const* partials, int32_t tp_size, tp_dtype_t partial_dtype, const void* b,
                           void* Y, int64_t M, int64_t N, tp_dtype_t out_dtype, void* stream) {
    if (!partials || !Y) return TP_ERR_NULL;
    if (!dtype_ok(partial_dtype) || !dtype_ok(out_dtype)) return TP_ERR_DTYPE;
    TP_TRY(check_dims(M, {N}));
    if (tp_size < 1 || tp_size > kMaxTP) return TP_ERR_SHAPE;
    for (int32_t r = 0; r < tp_size; ++r)
        if (!partials[r]) return TP_ERR_NULL;
    if (t_planning) return TP_OK;
    return launch_combine_sum(partials, tp_size, partial_dtype, b, Y, M, N, out_dtype,
                              static_cast<hipStream_t>(stream));
}

tp_status_t tp_shard_weight(const void* W, int64_t out_features, int64_t in_features, int32_t tp_size, int32_t rank,
                            int32_t axis, void* W_r, tp_dtype_t dtype, void* stream) {
    if (!W || !W_r) return TP_ERR_NULL;
    if (!dtype_ok(dtype)) return TP_ERR_DTYPE;
    TP_TRY(check_dims(0, {out_features, in_features}));
    if (tp_size < 1 || tp_size > kMaxTP || rank < 0 || rank >= tp_size || (axis != 0 && axis != 1))
        return TP_ERR_SHAPE;
    if ((axis == 0 ? out_features : in_features) % tp_size != 0) return TP_ERR_INDIVISIBLE;
    if (t_planning) return TP_OK;
    const size_t es = elem_size(dtype);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (axis == 0) {
        const int64_t rows = out_features / tp_size;
        const char* src = static_cast<const char*>(W) + (size_t)(rank * rows) * in_features * es;
        return launch_copy2d(src, in_features, W_r, in_features, rows, in_features, es, s);
    }
    const int64_t cols = in_features / tp_size;
    const char* src = static_cast<const char*>(W) + (size_t)(rank * cols) * es;
    return launch_copy2d(src, in_features, W_r, cols, out_features, cols, es, s);
}

tp_status_t tp_shard_weight_block(const void* W, int64_t out_features, int64_t in_features, int32_t axis,
                                  int64_t start, int64_t width, void* W_r, tp_dtype_t dtype, void* stream) {
    if (!W || !W_r) return TP_ERR_NULL;
    if (!dtype_ok(dtype)) return TP_ERR_DTYPE;
    TP_TRY(check_dims(0, {out_features, in_features}));
    if ((axis != 0 && axis != 1) || start < 0 || width <= 0) return TP_ERR_SHAPE;
    const int64_t n = axis == 0 ? out_features : in_features;
    if (start + width > n) return TP_ERR_SHAPE;
    if (t_planning) return TP_OK;
    const size_t es = elem_size(dtype);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (axis == 0) {
        const char* src = static_cast<const char*>(W) + (size_t)start * in_features * es;
        return launch_copy2d(src, in_features, W_r, in_features, width, in_features, es, s);
    }
    const char* src = static_cast<const char*>(W) + (size_t)start * es;
    return launch_copy2d(src, in_features, W_r, width, out_features, width, es, s);
}

tp_status_t tp_combine_concat_v(const void* const* shards, int32_t n_shards, const int64_t* widths, void* Y, int64_t M,
                                tp_dtype_t dtype, void* stream) {
    if (!shards || !widths || !Y) return TP_ERR_NULL;
    if (!dtype_ok(dtype)) return TP_ERR_DTYPE;
    if (n_shards < 1 || n_shards > kMaxTP || M < 0 || M > kMaxDim) return TP_ERR_SHAPE;
    int64_t total = 0;
    for (int32_t r = 0; r < n_shards; ++r) {
        if (!shards[r]) return TP_ERR_NULL;
        if (widths[r] <= 0 || widths[r] > kMaxDim) return TP_ERR_SHAPE;
        total += widths[r];
    }
    if (total > kMaxDim) return TP_ERR_SHAPE;
    if (M == 0 || t_planning) return TP_OK;
    const size_t es = elem_size(dtype);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t col = 0;
    for (int32_t r = 0; r < n_shards; ++r) {
        TP_TRY(launch_copy2d(shards[r], widths[r], static_cast<char*>(Y) + (size_t)col * es, total, M, widths[r], es, s));
        col += widths[r];
    }
    return TP_OK;
}

tp_status_t tp_shard_qkv(const void* Wqkv, int64_t in_features, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                         int32_t tp_size, int32_t rank, void* Wqkv_r, tp_dtype_t dtype, void* stream) {
    if (!Wqkv || !Wqkv_r) return TP_ERR_NULL;
    if (!dtype_ok(dtype)) return TP_ERR_DTYPE;
    TP_TRY(check_dims(0, {in_features, n_heads, n_kv_heads, head_dim}));
    if (tp_size < 1 || tp_size > kMaxTP || rank < 0 || rank >= tp_size) return TP_ERR_SHAPE;
    if (n_heads % tp_size != 0 || kv_heads_per_shard(n_kv_heads, tp_size) == 0) return TP_ERR_INDIVISIBLE;
    if (t_planning) return TP_OK;
    const size_t es = elem_size(dtype);
    const int64_t d = head_dim, hq = n_heads / tp_size, hk = kv_heads_per_shard(n_kv_heads, tp_size);
    // First KV head of the shard: rank*hk when p divides G, else rank*G/p (replicated).
    const int64_t kv0 = (n_kv_heads % tp_size == 0) ? rank * hk : (int64_t)rank * n_kv_heads / tp_size;
    const int64_t src_rows[3] = {rank * hq * d, (n_heads + kv0) * d, (n_heads + n_kv_heads + kv0) * d};
    const int64_t nrows[3] = {hq * d, hk * d, hk * d};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t dst_row = 0;
    for (int j = 0; j < 3; ++j) {
        const char* src = static_cast<const char*>(Wqkv) + (size_t)src_rows[j] * in_features * es;
        char* dst = static_cast<char*>(Wqkv_r) + (size_t)dst_row * in_features * es;
        TP_TRY(launch_copy2d(src, in_features, dst, in_features, nrows[j], in_features, es, s));
        dst_row += nrows[j];
    }
    return TP_OK;
}

tp_status_t tp_workspace_reserve(void* stream, size_t partial_bytes, size_t n_counters) {
    if (t_planning) return TP_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TP_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    WsEntry& e = g_ws[{dev, s}];
    const size_t want_f = std::max(e.partial_floats, round_up(partial_bytes, 256) / sizeof(float));
    const size_t want_c = std::max(e.counters, round_up(std::max<size_t>(n_counters, 1), 64));
    if (e.base && e.partial_floats >= want_f && e.counters >= want_c) return TP_OK;
    if (e.base) {
        // Work still queued on this stream may use the old space.
        if (hipStreamSynchronize(s) != hipSuccess) return TP_ERR_HIP;
        if (hipFree(e.base) != hipSuccess) return TP_ERR_HIP;
        e = WsEntry{};
    }
    void* p = nullptr;
    if (hipMalloc(&p, round_up(want_c * sizeof(unsigned), 256) + want_f * sizeof(float)) != hipSuccess)
        return TP_ERR_HIP;
    e.base = p;
    e.partial_floats = want_f;
    e.counters = want_c;
    // Counters start at zero; every launch that uses one leaves it at zero.
    return launch_fill_u32(static_cast<unsigned*>(p), want_c, 0u, s);
}

tp_status_t tp_workspace_reserved(void* stream, size_t* partial_bytes, size_t* n_counters) {
    if (!partial_bytes || !n_counters) return TP_ERR_NULL;
    *partial_bytes = 0;
    *n_counters = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TP_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto it = g_ws.find({dev, static_cast<hipStream_t>(stream)});
    if (it != g_ws.end() && it->second.base) {
        *partial_bytes = it->second.partial_floats * sizeof(float);
        *n_counters = it->second.counters;
    }
    return TP_OK;
}

tp_status_t tp_plan_begin(void) {
    t_planning = true;
    t_plan = WsNeed{};
    return TP_OK;
}

tp_status_t tp_plan_end(size_t* partial_bytes, size_t* n_counters) {
    const WsNeed n = t_plan;
    t_planning = false;
    t_plan = WsNeed{};
    if (partial_bytes) *partial_bytes = n.partial_floats * sizeof(float);
    if (n_counters) *n_counters = n.counters;
    return TP_OK;
}

tp_status_t tp_release_workspaces(void) {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    tp_status_t st = TP_OK;
    for (auto& kv : g_ws) {
        if (kv.second.base) {
            int prev = 0;
            if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(kv.first.first) != hipSuccess) {
                st = TP_ERR_HIP;
                continue;
            }
            if (hipStreamSynchronize(kv.first.second) != hipSuccess || hipFree(kv.second.base) != hipSuccess)
                st = TP_ERR_HIP;
            if (hipSetDevice(prev) != hipSuccess) st = TP_ERR_HIP;
        }
    }
    g_ws.clear();
    return st;
}

}  // extern "C"
