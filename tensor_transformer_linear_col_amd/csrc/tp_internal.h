// Internal declarations shared by the host dispatcher and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_linear.h"

namespace tp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// One linear product Y = X W0^T (+ b0), or the SwiGLU pair
// Y = silu(X W0^T + b0) * (X W1^T + b1), with W0/W1 stored [N, K] contiguous.
struct LinearDesc {
    const void* X;   // [M, K], row stride ldx (elements)
    int64_t ldx;
    const void* W0;  // [N, K]
    const void* W1;  // [N, K] (SwiGLU up weights) or nullptr
    const void* b0;  // [N] or nullptr
    const void* b1;  // [N] or nullptr
    void* Y;         // [M, N], row stride ldy
    int64_t ldy;
    int64_t M, N, K;
    tp_dtype_t in_dtype;   // dtype of X, W, b
    tp_dtype_t out_dtype;  // dtype of Y
    bool swiglu;
    bool gelu = false;  // plain products only: y = gelu(XW^T + b), erf form
};

// Work space of the kernels that split a reduction across workgroups: fp32 partial
// sums and arrival counters (every counter is zero between launches: the last
// workgroup to arrive resets its own).
struct WsNeed {
    size_t partial_floats = 0;
    size_t counters = 0;
    void merge(const WsNeed& o) {
        if (o.partial_floats > partial_floats) partial_floats = o.partial_floats;
        if (o.counters > counters) counters = o.counters;
    }
    bool empty() const { return partial_floats == 0 && counters == 0; }
};

struct Workspace {
    float* partials = nullptr;
    size_t partial_floats = 0;
    unsigned* counters = nullptr;
    size_t n_counters = 0;
    bool covers(const WsNeed& n) const { return partial_floats >= n.partial_floats && n_counters >= n.counters; }
};

// How a launcher is called. Plan mode (need != nullptr): check everything that could
// make the launch fail and record the work space it needs, enqueue nothing. Launch
// mode (need == nullptr): enqueue on `stream`, taking scratch memory from *ws, which the
// caller has sized from the plan.
struct Ctx {
    hipStream_t stream;
    const Workspace* ws;
    WsNeed* need;
    bool planning() const { return need != nullptr; }
};

// Kernel launchers (the C ABI layer has validated the arguments).
tp_status_t launch_skinny(const LinearDesc& d, const Ctx& c);
// 1-4 tokens: one workgroup per CU over balanced feature ranges, no cross-workgroup sums.
tp_status_t launch_gemv(const LinearDesc& d, const Ctx& c);
// 512-wide K chunks per wave of launch_gemv for K (1, 2 or 4; 0 when K is too long for it),
// and the K elements per wave.
int gemv_chunks(int64_t K, int* kw_out);
// Compute units of the current device (256 when it cannot be read).
int gemv_cus();
tp_status_t launch_gemm(const LinearDesc& d, const Ctx& c);
// Decode shapes (M <= 64) that launch_gemm takes on LDS-staged tiles instead of the decode
// kernels: 17-64 tokens of a SwiGLU pair, 21-64 of a plain product, K >= 2048 and a multiple
// of 64.
bool gemm_takes_decode(const LinearDesc& d);
tp_status_t launch_f32(const LinearDesc& d, const Ctx& c);
// Head-local attention core: out[M, hq*d] (row stride lda) from qkv[M, (hq+2hk)*d] (row stride ldq).
tp_status_t launch_attn_core(const void* qkv, int64_t ldq, void* out, int64_t lda, int64_t M, int hq, int hk, int d,
                             bool causal, const Ctx& c);
// One decode step: appends the M new tokens' K and V rows of qkv[M, ldq] (Q segment first) to
// the caches kc/vc[.., ldkv] at row cache_len, then attention of the new tokens (positions
// cache_len ..) over cache_len + M keys, causal; out[M, hq*d] (row stride lda).
tp_status_t launch_attn_decode(const void* qkv, int64_t ldq, void* kc, void* vc, int64_t ldkv, int64_t cache_len,
                               void* out, int64_t lda, int64_t M, int hq, int hk, int d, const Ctx& c);

tp_status_t launch_combine_sum(const void* const* partials, int p, tp_dtype_t pdt, const void* b,
                               void* Y, int64_t M, int64_t N, tp_dtype_t odt, hipStream_t stream);
tp_status_t launch_concat(const void* const* shards, int p, const int64_t* seg, int nseg, void* Y,
                          int64_t M, size_t elem, hipStream_t stream);
// dst[r, c] = src[r * lds + c] for r < rows, c < cols (element size elem bytes), dst ld = ldd.
tp_status_t launch_copy2d(const void* src, int64_t lds, void* dst, int64_t ldd, int64_t rows,
                          int64_t cols, size_t elem, hipStream_t stream);
tp_status_t launch_fill_u32(unsigned* p, size_t n, unsigned v, hipStream_t stream);

#define TP_TRY(expr)                    \
    do {                                \
        const tp_status_t st_ = (expr); \
        if (st_ != TP_OK) return st_;   \
    } while (0)

inline tp_status_t hip_status() {
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_HIP;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace tp
