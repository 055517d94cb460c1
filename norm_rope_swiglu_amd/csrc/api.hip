// C-ABI entry points of libnrs: validate on the host, then enqueue.
// The declarations, with argument meaning and error behaviour, are in nrs.h.
#include <math.h>

#include <new>

#include "kernels.hpp"
#include "nrs.h"
#include "validate.hpp"

#define NRS_API extern "C" __attribute__((visibility("default")))

namespace nrs {

__global__ void empty_kernel() {}

hipError_t launch_empty(hipStream_t stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError();
}

}  // namespace nrs

struct nrs_graph_s {
    hipGraph_t graph;
    hipGraphExec_t exec;
    int nodes;
};

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return NRS_OK;
    g_last_hip = (int)e;
    return NRS_ERR_HIP;
}

nrs::mrope_freqs make_freqs(int head_dim, double theta) {
    nrs::mrope_freqs f;
    for (int j = 0; j < nrs::kMaxHalf; ++j)
        f.w[j] = j < head_dim / 2 ? pow(theta, -2.0 * (double)j / (double)head_dim) : 0.0;
    return f;
}

// Drop an error left by an earlier, unrelated HIP call on this thread so
// that the check after our launch reports our launch only.
void clear_stale_error() { (void)hipGetLastError(); }

// Record the launches made by `body(stream)` into a graph.
template <typename F>
int record_graph(nrs_graph *out, F &&body) {
    if (!out) return NRS_ERR_NULL;
    *out = nullptr;
    clear_stale_error();
    hipStream_t s = nullptr;
    int st = hip_status(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    if (st != NRS_OK) return st;
    st = hip_status(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    if (st != NRS_OK) {
        (void)hipStreamDestroy(s);
        return st;
    }
    int body_st = body(s);
    hipGraph_t g = nullptr;
    st = hip_status(hipStreamEndCapture(s, &g));
    (void)hipStreamDestroy(s);
    if (body_st != NRS_OK || st != NRS_OK) {
        if (g) (void)hipGraphDestroy(g);
        return body_st != NRS_OK ? body_st : st;
    }
    hipGraphExec_t ex = nullptr;
    st = hip_status(hipGraphInstantiate(&ex, g, nullptr, nullptr, 0));
    if (st != NRS_OK) {
        (void)hipGraphDestroy(g);
        return st;
    }
    size_t n = 0;
    st = hip_status(hipGraphGetNodes(g, nullptr, &n));
    if (st != NRS_OK) {
        (void)hipGraphExecDestroy(ex);
        (void)hipGraphDestroy(g);
        return st;
    }
    nrs_graph h = new (std::nothrow) nrs_graph_s{g, ex, (int)n};
    if (!h) {
        (void)hipGraphExecDestroy(ex);
        (void)hipGraphDestroy(g);
        return NRS_ERR_ARG;
    }
    *out = h;
    return NRS_OK;
}

}  // namespace

NRS_API int nrs_abi_version(void) { return NRS_ABI_VERSION; }

NRS_API const char *nrs_status_string(int status) {
    switch (status) {
        case NRS_OK: return "ok";
        case NRS_ERR_NULL: return "a required pointer is NULL";
        case NRS_ERR_SHAPE: return "unsupported or inconsistent size or stride";
        case NRS_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case NRS_ERR_DTYPE: return "unknown dtype";
        case NRS_ERR_SECTIONS: return "M-RoPE sections must be >= 0 and sum to head_dim / 2";
        case NRS_ERR_ARG: return "invalid scalar argument";
        case NRS_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

NRS_API int nrs_last_hip_error(void) { return g_last_hip; }

NRS_API int nrs_rmsnorm(void *y, const void *x, const void *gamma, int64_t rows, int64_t hidden,
                        int64_t x_stride, int64_t y_stride, float eps, int dtype, void *stream) {
    int st = nrs::check_rmsnorm(y, x, gamma, rows, hidden, x_stride, y_stride, eps, dtype);
    if (st != NRS_OK || rows == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_rmsnorm(y, x, gamma, rows, hidden, x_stride, y_stride, eps,
                                          dtype, (hipStream_t)stream));
}

NRS_API int nrs_add_rmsnorm(void *y, void *residual_out, const void *x, const void *residual,
                            const void *gamma, int64_t rows, int64_t hidden, float eps, int dtype,
                            void *stream) {
    int st = nrs::check_add_rmsnorm(y, residual_out, x, residual, gamma, rows, hidden, eps, dtype);
    if (st != NRS_OK || rows == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_add_rmsnorm(y, residual_out, x, residual, gamma, rows, hidden,
                                              eps, dtype, (hipStream_t)stream));
}

NRS_API int nrs_layernorm(void *y, const void *x, const void *gamma, const void *beta,
                          int64_t rows, int64_t hidden, int64_t x_stride, int64_t y_stride,
                          float eps, int dtype, void *stream) {
    int st = nrs::check_layernorm(y, x, gamma, beta, rows, hidden, x_stride, y_stride, eps, dtype);
    if (st != NRS_OK || rows == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_layernorm(y, x, gamma, beta, rows, hidden, x_stride, y_stride,
                                            eps, dtype, (hipStream_t)stream));
}

NRS_API int nrs_add_layernorm(void *y, void *residual_out, const void *x, const void *residual,
                              const void *gamma, const void *beta, int64_t rows, int64_t hidden,
                              float eps, int dtype, void *stream) {
    int st = nrs::check_add_layernorm(y, residual_out, x, residual, gamma, beta, rows, hidden, eps,
                                      dtype);
    if (st != NRS_OK || rows == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_add_layernorm(y, residual_out, x, residual, gamma, beta, rows,
                                                hidden, eps, dtype, (hipStream_t)stream));
}

NRS_API int nrs_rmsnorm_linear(void *out, const void *x, const void *w, int64_t rows,
                               int64_t in_features, int64_t out_features, int64_t x_stride,
                               int64_t w_stride, int64_t out_stride, float eps, int dtype,
                               void *stream) {
    int st = nrs::check_rmsnorm_linear(out, x, w, rows, in_features, out_features, x_stride,
                                       w_stride, out_stride, eps, dtype);
    if (st != NRS_OK || rows == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_rmsnorm_linear(out, x, w, rows, in_features, out_features,
                                                 x_stride, w_stride, out_stride, eps, dtype,
                                                 (hipStream_t)stream));
}

NRS_API int nrs_mrope(void *q, void *k, const int32_t *pos, int64_t pos_stride, int64_t tokens,
                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      int64_t q_token_stride, int64_t k_token_stride, int32_t sec_t, int32_t sec_h,
                      int32_t sec_w, double theta, int dtype, void *stream) {
    int st = nrs::check_mrope(q, k, pos, pos_stride, tokens, n_q_heads, n_kv_heads, head_dim,
                              q_token_stride, k_token_stride, sec_t, sec_h, sec_w, theta, dtype);
    if (st != NRS_OK || tokens == 0 || n_q_heads + n_kv_heads == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_mrope(q, k, pos, pos_stride, tokens, n_q_heads, n_kv_heads,
                                        head_dim, q_token_stride, k_token_stride, sec_t, sec_h,
                                        make_freqs(head_dim, theta), dtype, (hipStream_t)stream));
}

NRS_API int nrs_mrope_kv_append(void *q, const void *k, const void *v, const int32_t *pos,
                                int64_t pos_stride, int64_t tokens, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim, int64_t q_token_stride,
                                int64_t k_token_stride, int64_t v_token_stride, int32_t sec_t,
                                int32_t sec_h, int32_t sec_w, double theta, void *k_cache,
                                void *v_cache, const int32_t *seq_idx, const int32_t *slot,
                                int64_t n_seqs, int64_t max_seq, int dtype, void *stream) {
    int st = nrs::check_mrope_kv(q, k, v, pos, pos_stride, tokens, n_q_heads, n_kv_heads, head_dim,
                                 q_token_stride, k_token_stride, v_token_stride, sec_t, sec_h,
                                 sec_w, theta, k_cache, v_cache, seq_idx, slot, n_seqs, max_seq,
                                 dtype);
    if (st != NRS_OK || tokens == 0 || n_q_heads + n_kv_heads == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_mrope_kv(q, k, v, pos, pos_stride, tokens, n_q_heads, n_kv_heads,
                                           head_dim, q_token_stride, k_token_stride,
                                           v_token_stride, sec_t, sec_h,
                                           make_freqs(head_dim, theta), k_cache, v_cache, seq_idx,
                                           slot, n_seqs, max_seq, dtype, (hipStream_t)stream));
}

NRS_API int nrs_swiglu(void *out, const void *gate_up, int64_t rows, int64_t inter,
                       int64_t gate_up_stride, int64_t out_stride, int dtype, void *stream) {
    int st = nrs::check_swiglu(out, gate_up, rows, inter, gate_up_stride, out_stride, dtype);
    if (st != NRS_OK || rows == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_swiglu(out, gate_up, rows, inter, gate_up_stride, out_stride,
                                         dtype, (hipStream_t)stream));
}

NRS_API int nrs_softmax_topk_sample(int32_t *token, void *probs, const void *logits, int64_t rows,
                                    int64_t vocab, int64_t row_stride, int64_t probs_stride,
                                    float temperature, int32_t top_k, const float *u, int dtype,
                                    void *stream) {
    int st = nrs::check_topk_sample(token, probs, logits, rows, vocab, row_stride, probs_stride,
                                    temperature, top_k, u, dtype);
    if (st != NRS_OK || rows == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_topk_sample(token, probs, logits, rows, vocab, row_stride,
                                              probs_stride, temperature, top_k, u, dtype,
                                              (hipStream_t)stream));
}

NRS_API int nrs_decode_graph_create(nrs_graph *out, const nrs_decode_shape *shape,
                                    const nrs_decode_layer *layers, int32_t n_layers) {
    if (!out || !shape || (n_layers > 0 && !layers)) return NRS_ERR_NULL;
    if (n_layers <= 0) return NRS_ERR_ARG;
    const nrs_decode_shape S = *shape;
    const int64_t T = S.tokens, H = S.hidden, I = S.inter, D = S.head_dim;
    if (T <= 0) return NRS_ERR_SHAPE;
    for (int32_t l = 0; l < n_layers; ++l) {
        const nrs_decode_layer &L = layers[l];
        int st = nrs::check_add_rmsnorm(L.in_y, L.in_residual_out, L.in_x, L.in_residual,
                                        L.in_gamma, T, H, S.eps, S.dtype);
        if (st == NRS_OK)
            st = nrs::check_mrope(L.q, L.k, S.pos, S.pos_stride, T, S.n_q_heads, S.n_kv_heads,
                                  S.head_dim, S.n_q_heads * D, S.n_kv_heads * D, S.sec_t,
                                  S.sec_h, S.sec_w, S.theta, S.dtype);
        if (st == NRS_OK && L.post_x)
            st = nrs::check_add_rmsnorm(L.post_y, L.post_residual_out, L.post_x,
                                        L.post_residual, L.post_gamma, T, H, S.eps, S.dtype);
        if (st == NRS_OK)
            st = nrs::check_swiglu(L.act_out, L.gate_up, T, I, 2 * I, I, S.dtype);
        if (st != NRS_OK) return st;
    }
    const nrs::mrope_freqs fr = make_freqs(S.head_dim, S.theta);
    return record_graph(out, [&](hipStream_t s) -> int {
        for (int32_t l = 0; l < n_layers; ++l) {
            const nrs_decode_layer &L = layers[l];
            int st = hip_status(nrs::launch_add_rmsnorm(L.in_y, L.in_residual_out, L.in_x,
                                                        L.in_residual, L.in_gamma, T, H, S.eps,
                                                        S.dtype, s));
            if (st == NRS_OK && S.n_q_heads + S.n_kv_heads > 0)
                st = hip_status(nrs::launch_mrope(L.q, L.k, S.pos, S.pos_stride, T, S.n_q_heads,
                                                  S.n_kv_heads, S.head_dim, S.n_q_heads * D,
                                                  S.n_kv_heads * D, S.sec_t, S.sec_h, fr,
                                                  S.dtype, s));
            if (st == NRS_OK && L.post_x)
                st = hip_status(nrs::launch_add_rmsnorm(L.post_y, L.post_residual_out, L.post_x,
                                                        L.post_residual, L.post_gamma, T, H,
                                                        S.eps, S.dtype, s));
            if (st == NRS_OK)
                st = hip_status(nrs::launch_swiglu(L.act_out, L.gate_up, T, I, 2 * I, I, S.dtype, s));
            if (st != NRS_OK) return st;
        }
        return NRS_OK;
    });
}

NRS_API int nrs_null_graph_create(nrs_graph *out, int32_t n_nodes) {
    if (!out) return NRS_ERR_NULL;
    if (n_nodes <= 0) return NRS_ERR_ARG;
    return record_graph(out, [&](hipStream_t s) -> int {
        for (int32_t i = 0; i < n_nodes; ++i) {
            int st = hip_status(nrs::launch_empty(s));
            if (st != NRS_OK) return st;
        }
        return NRS_OK;
    });
}

NRS_API int nrs_stream_probe(void *dst0, void *dst1, const void *src0, const void *src1,
                             int32_t n_read, int32_t n_write, int64_t bytes, int64_t row_bytes,
                             int32_t variant, void *stream) {
    int st = nrs::check_stream_probe(dst0, dst1, src0, src1, n_read, n_write, bytes, row_bytes,
                                     variant);
    if (st != NRS_OK || bytes == 0) return st;
    clear_stale_error();
    return hip_status(nrs::launch_stream_probe(dst0, dst1, src0, src1, n_read, n_write, bytes,
                                               row_bytes, variant, (hipStream_t)stream));
}

NRS_API int nrs_graph_node_count(nrs_graph g) {
    if (!g) return NRS_ERR_NULL;
    return g->nodes;
}

NRS_API int nrs_graph_launch(nrs_graph g, void *stream) {
    if (!g) return NRS_ERR_NULL;
    clear_stale_error();
    return hip_status(hipGraphLaunch(g->exec, (hipStream_t)stream));
}

NRS_API int nrs_graph_destroy(nrs_graph g) {
    if (!g) return NRS_OK;
    int st = hip_status(hipGraphExecDestroy(g->exec));
    int st2 = hip_status(hipGraphDestroy(g->graph));
    delete g;
    return st != NRS_OK ? st : st2;
}
