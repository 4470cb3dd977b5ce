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

// Split-K work space: fp32 partial tiles and per-tile arrival counters.
struct Workspace {
    float* partials;
    unsigned* counters;
};

// Returns the work space for the current device and `stream`, at least the given sizes.
tp_status_t get_workspace(hipStream_t stream, size_t partial_floats, size_t n_counters,
                          Workspace* out);

// Kernel launchers (each validates nothing: the C ABI layer has done it).
tp_status_t launch_skinny(const LinearDesc& d, hipStream_t stream);
tp_status_t launch_gemm(const LinearDesc& d, hipStream_t stream);
tp_status_t launch_f32(const LinearDesc& d, hipStream_t stream);
// Head-local attention core: out[M, hq*d] (row stride lda) from qkv[M, (hq+2hk)*d] (row stride ldq).
tp_status_t launch_attn_core(const void* qkv, int64_t ldq, void* out, int64_t lda, int64_t M, int hq, int hk, int d,
                             bool causal, hipStream_t stream);
// One decode step: appends the M new tokens' K and V rows of qkv[M, ldq] (Q segment first) to
// the caches kc/vc[.., ldkv] at row cache_len, then attention of the new tokens (positions
// cache_len ..) over cache_len + M keys, causal; out[M, hq*d] (row stride lda).
tp_status_t launch_attn_decode(const void* qkv, int64_t ldq, void* kc, void* vc, int64_t ldkv, int64_t cache_len,
                               void* out, int64_t lda, int64_t M, int hq, int hk, int d, hipStream_t stream);

tp_status_t launch_combine_sum(const void* const* partials, int p, tp_dtype_t pdt, const void* b,
                               void* Y, int64_t M, int64_t N, tp_dtype_t odt, hipStream_t stream);
tp_status_t launch_concat(const void* const* shards, int p, const int64_t* seg, int nseg, void* Y,
                          int64_t M, size_t elem, hipStream_t stream);
// dst[r, c] = src[r * lds + c] for r < rows, c < cols (element size elem bytes), dst ld = ldd.
tp_status_t launch_copy2d(const void* src, int64_t lds, void* dst, int64_t ldd, int64_t rows,
                          int64_t cols, size_t elem, hipStream_t stream);
tp_status_t launch_fill_u32(unsigned* p, size_t n, unsigned v, hipStream_t stream);

inline tp_status_t hip_status() {
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_HIP;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace tp
