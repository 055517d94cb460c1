// Argument checks of the C ABI (internal).  Pure C++: no HIP call happens
// before a check fails, so every error path is testable without a GPU.
#pragma once

#include <math.h>
#include <stdint.h>

#include "nrs.h"

namespace nrs {

// Widest norm rows: 16 waves x 8 chunks of 16 bytes per thread (65536 bf16 or
// 32768 fp32 elements), the widest shape of the row kernel.
constexpr int64_t kMaxHiddenBytes = (int64_t)16 * 64 * 8 * 16;
constexpr int kMaxHeadDim = 512;
// Row and token counts reach the kernels as 32-bit values and grid sizes.
constexpr int64_t kMaxRows = ((int64_t)1 << 31) - 1;
constexpr int64_t kMaxHeads = 1 << 16;

inline int elem_size(int dtype) { return dtype == NRS_F32 ? 4 : 2; }
inline bool known_dtype(int dtype) { return dtype == NRS_F32 || dtype == NRS_BF16; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool stride_ok(int64_t stride, int dtype) { return (stride * elem_size(dtype)) % 16 == 0; }
inline int vec_of(int dtype) { return 16 / elem_size(dtype); }

inline int check_rmsnorm(const void *y, const void *x, const void *gamma, int64_t rows,
                         int64_t hidden, int64_t x_stride, int64_t y_stride, float eps,
                         int dtype) {
    if (!known_dtype(dtype)) return NRS_ERR_DTYPE;
    if (rows < 0 || rows > kMaxRows || hidden <= 0 || hidden % vec_of(dtype) != 0 ||
        hidden * elem_size(dtype) > kMaxHiddenBytes)
        return NRS_ERR_SHAPE;
    if (!(eps >= 0.0f) || isinf(eps)) return NRS_ERR_ARG;
    if (rows == 0) return NRS_OK;
    if (x_stride < hidden || y_stride < hidden) return NRS_ERR_SHAPE;
    if (!y || !x || !gamma) return NRS_ERR_NULL;
    if (!aligned16(y) || !aligned16(x) || !aligned16(gamma) || !stride_ok(x_stride, dtype) ||
        !stride_ok(y_stride, dtype))
        return NRS_ERR_ALIGN;
    return NRS_OK;
}

inline int check_add_rmsnorm(const void *y, const void *residual_out, const void *x,
                             const void *residual, const void *gamma, int64_t rows,
                             int64_t hidden, float eps, int dtype) {
    int st = check_rmsnorm(y, x, gamma, rows, hidden, hidden, hidden, eps, dtype);
    if (st != NRS_OK || rows == 0) return st;
    if (!residual_out || !residual) return NRS_ERR_NULL;
    if (!aligned16(residual_out) || !aligned16(residual)) return NRS_ERR_ALIGN;
    return NRS_OK;
}

inline int check_layernorm(const void *y, const void *x, const void *gamma, const void *beta,
                           int64_t rows, int64_t hidden, int64_t x_stride, int64_t y_stride,
                           float eps, int dtype) {
    int st = check_rmsnorm(y, x, gamma, rows, hidden, x_stride, y_stride, eps, dtype);
    if (st != NRS_OK || rows == 0) return st;
    if (beta && !aligned16(beta)) return NRS_ERR_ALIGN;
    return NRS_OK;
}

inline int check_add_layernorm(const void *y, const void *residual_out, const void *x,
                               const void *residual, const void *gamma, const void *beta,
                               int64_t rows, int64_t hidden, float eps, int dtype) {
    int st = check_add_rmsnorm(y, residual_out, x, residual, gamma, rows, hidden, eps, dtype);
    if (st != NRS_OK || rows == 0) return st;
    if (beta && !aligned16(beta)) return NRS_ERR_ALIGN;
    return NRS_OK;
}

inline int check_mrope(const void *q, const void *k, const int32_t *pos, int64_t pos_stride,
                       int64_t tokens, int32_t n_q, int32_t n_kv, int32_t head_dim,
                       int64_t q_stride, int64_t k_stride, int32_t sec_t, int32_t sec_h,
                       int32_t sec_w, double theta, int dtype) {
    if (!known_dtype(dtype)) return NRS_ERR_DTYPE;
    if (tokens < 0 || tokens > kMaxRows || n_q < 0 || n_kv < 0 || (int64_t)n_q + n_kv > kMaxHeads)
        return NRS_ERR_SHAPE;
    if (head_dim <= 0 || head_dim > kMaxHeadDim || head_dim % (2 * vec_of(dtype)) != 0)
        return NRS_ERR_SHAPE;
    if (sec_t < 0 || sec_h < 0 || sec_w < 0 || (int64_t)sec_t + sec_h + sec_w != head_dim / 2)
        return NRS_ERR_SECTIONS;
    if (!(theta > 0.0) || isinf(theta)) return NRS_ERR_ARG;
    if (tokens == 0 || n_q + n_kv == 0) return NRS_OK;
    if (pos_stride < tokens) return NRS_ERR_SHAPE;
    if ((n_q > 0 && q_stride < (int64_t)n_q * head_dim) ||
        (n_kv > 0 && k_stride < (int64_t)n_kv * head_dim))
        return NRS_ERR_SHAPE;
    if (!pos || (n_q > 0 && !q) || (n_kv > 0 && !k)) return NRS_ERR_NULL;
    if (((uintptr_t)pos & 3u) != 0) return NRS_ERR_ALIGN;
    if ((n_q > 0 && (!aligned16(q) || !stride_ok(q_stride, dtype))) ||
        (n_kv > 0 && (!aligned16(k) || !stride_ok(k_stride, dtype))))
        return NRS_ERR_ALIGN;
    return NRS_OK;
}

inline int check_mrope_kv(const void *q, const void *k, const void *v, const int32_t *pos,
                          int64_t pos_stride, int64_t tokens, int32_t n_q, int32_t n_kv,
                          int32_t head_dim, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                          int32_t sec_t, int32_t sec_h, int32_t sec_w, double theta,
                          const void *k_cache, const void *v_cache, const int32_t *seq_idx,
                          const int32_t *slot, int64_t n_seqs, int64_t max_seq, int dtype) {
    int st = check_mrope(q, k, pos, pos_stride, tokens, n_q, n_kv, head_dim, q_stride, k_stride,
                         sec_t, sec_h, sec_w, theta, dtype);
    if (st != NRS_OK) return st;
    if (n_seqs <= 0 || max_seq <= 0 || max_seq > ((int64_t)1 << 36)) return NRS_ERR_SHAPE;
    // cache elements n_seqs * n_kv * max_seq * head_dim must fit in 62 bits
    if (n_kv > 0 && n_seqs > ((int64_t)1 << 62) / ((int64_t)n_kv * max_seq * head_dim))
        return NRS_ERR_SHAPE;
    if (tokens == 0 || n_q + n_kv == 0) return NRS_OK;
    if (n_kv > 0 && v_stride < (int64_t)n_kv * head_dim) return NRS_ERR_SHAPE;
    if (n_kv > 0 && (!v || !k_cache || !v_cache || !seq_idx || !slot)) return NRS_ERR_NULL;
    if (n_kv > 0 && (!aligned16(v) || !stride_ok(v_stride, dtype) || !aligned16(k_cache) ||
                     !aligned16(v_cache) || ((uintptr_t)seq_idx & 3u) || ((uintptr_t)slot & 3u)))
        return NRS_ERR_ALIGN;
    return NRS_OK;
}

inline int check_swiglu(const void *out, const void *gate_up, int64_t rows, int64_t inter,
                        int64_t gate_up_stride, int64_t out_stride, int dtype) {
    if (!known_dtype(dtype)) return NRS_ERR_DTYPE;
    if (rows < 0 || rows > kMaxRows || inter <= 0 || inter % vec_of(dtype) != 0 ||
        inter / vec_of(dtype) >= (1 << 30))
        return NRS_ERR_SHAPE;
    if (rows == 0) return NRS_OK;
    if (gate_up_stride < 2 * inter || out_stride < inter) return NRS_ERR_SHAPE;
    if (!out || !gate_up) return NRS_ERR_NULL;
    if (!aligned16(out) || !aligned16(gate_up) || !stride_ok(gate_up_stride, dtype) ||
        !stride_ok(out_stride, dtype))
        return NRS_ERR_ALIGN;
    return NRS_OK;
}

constexpr int64_t kMaxLinearIn = 1 << 20;
constexpr int64_t kMaxLinearOut = (int64_t)1 << 31;

inline int check_rmsnorm_linear(const void *out, const void *x, const void *w, int64_t rows,
                                int64_t n_in, int64_t n_out, int64_t x_stride, int64_t w_stride,
                                int64_t out_stride, float eps, int dtype) {
    if (!known_dtype(dtype)) return NRS_ERR_DTYPE;
    if (rows < 0 || rows > kMaxRows || n_in <= 0 || n_in % vec_of(dtype) != 0 ||
        n_in > kMaxLinearIn || n_out <= 0 ||
        n_out >= kMaxLinearOut)
        return NRS_ERR_SHAPE;
    if (!(eps >= 0.0f) || isinf(eps)) return NRS_ERR_ARG;
    if (rows == 0) return NRS_OK;
    if (x_stride < n_in || w_stride < n_in || out_stride < n_out) return NRS_ERR_SHAPE;
    if (!out || !x || !w) return NRS_ERR_NULL;
    // out is written element by element: element alignment and any stride suffice
    if (((uintptr_t)out & (uintptr_t)(elem_size(dtype) - 1)) != 0 || !aligned16(x) ||
        !aligned16(w) || !stride_ok(x_stride, dtype) || !stride_ok(w_stride, dtype))
        return NRS_ERR_ALIGN;
    return NRS_OK;
}

constexpr int kMaxTopK = 1024;

inline int check_topk_sample(const int32_t *token, const void *probs, const void *logits,
                             int64_t rows, int64_t vocab, int64_t row_stride, int64_t probs_stride,
                             float temperature, int32_t top_k, const float *u, int dtype) {
    if (!known_dtype(dtype)) return NRS_ERR_DTYPE;
    if (rows < 0 || rows > kMaxRows || vocab <= 0 || vocab % vec_of(dtype) != 0 ||
        vocab >= ((int64_t)1 << 31))
        return NRS_ERR_SHAPE;
    if (top_k < 1 || top_k > kMaxTopK || top_k > vocab) return NRS_ERR_ARG;
    if (!(temperature > 0.0f) || isinf(temperature)) return NRS_ERR_ARG;
    if (rows == 0) return NRS_OK;
    if (row_stride < vocab || (probs && probs_stride < vocab)) return NRS_ERR_SHAPE;
    if (!token || !logits || !u) return NRS_ERR_NULL;
    if (!aligned16(logits) || !stride_ok(row_stride, dtype) || ((uintptr_t)token & 3u) ||
        ((uintptr_t)u & 3u) || (probs && (!aligned16(probs) || !stride_ok(probs_stride, dtype))))
        return NRS_ERR_ALIGN;
    return NRS_OK;
}

// Longest row of a row-granular read (one workgroup walks the row).
constexpr int64_t kMaxReadRowBytes = (int64_t)1 << 30;

inline bool row_size_ok(int64_t row_bytes) {
    const int64_t k = row_bytes >> 10;
    return row_bytes % 1024 == 0 &&
           (k == 1 || k == 2 || k == 3 || k == 4 || k == 6 || k == 8 || k == 12 || k == 16);
}

inline int check_stream_probe(const void *d0, const void *d1, const void *s0, const void *s1,
                              int32_t n_read, int32_t n_write, int64_t bytes, int64_t row_bytes,
                              int32_t variant) {
    if (n_read < 0 || n_read > 2 || n_write < 0 || n_write > 2 || n_read + n_write == 0 ||
        variant < 0 || variant > 3)
        return NRS_ERR_ARG;
    // rows: a row-granular copy (n_read == n_write) or a row-granular read
    // (one source, no destination)
    const bool row_read = row_bytes != 0 && n_read == 1 && n_write == 0;
    if (row_bytes != 0 && ((n_read != n_write && !row_read) || n_read == 0 || variant > 1))
        return NRS_ERR_ARG;
    if (bytes < 0 || bytes % 16 != 0 || bytes / 16 > kMaxRows * 64) return NRS_ERR_SHAPE;
    if (row_bytes < 0) return NRS_ERR_SHAPE;
    if (row_read && (row_bytes % 16 != 0 || row_bytes > kMaxReadRowBytes ||
                     bytes % row_bytes != 0 || bytes / row_bytes > kMaxRows))
        return NRS_ERR_SHAPE;
    if (row_bytes != 0 && !row_read && (!row_size_ok(row_bytes) || bytes % row_bytes != 0))
        return NRS_ERR_SHAPE;
    if (bytes == 0) return NRS_OK;
    const void *p[4] = {s0, s1, d0, d1};
    const bool used[4] = {n_read >= 1, n_read >= 2, n_write >= 1, n_write >= 2};
    for (int i = 0; i < 4; ++i) {
        if (!used[i]) continue;
        if (!p[i]) return NRS_ERR_NULL;
        if (!aligned16(p[i])) return NRS_ERR_ALIGN;
    }
    return NRS_OK;
}

}  // namespace nrs
