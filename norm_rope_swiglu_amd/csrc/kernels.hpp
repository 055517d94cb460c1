// Kernel launchers of libnrs (internal).  Each enqueues on `stream` and
// returns hipGetLastError(); arguments are assumed validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nrs {

// Largest supported head_dim / 2 (frequency pairs per head).
constexpr int kMaxHalf = 256;

// Per-pair frequencies theta^(-2j/D), computed on the host in fp64 and passed
// by value (2 KiB of kernel arguments).
struct mrope_freqs {
    double w[kMaxHalf];
};

hipError_t launch_rmsnorm(void *y, const void *x, const void *gamma, int64_t rows, int64_t hidden,
                          int64_t x_stride, int64_t y_stride, float eps, int dtype,
                          hipStream_t stream);
hipError_t launch_add_rmsnorm(void *y, void *residual_out, const void *x, const void *residual,
                              const void *gamma, int64_t rows, int64_t hidden, float eps,
                              int dtype, hipStream_t stream);
hipError_t launch_layernorm(void *y, const void *x, const void *gamma, const void *beta,
                            int64_t rows, int64_t hidden, int64_t x_stride, int64_t y_stride,
                            float eps, int dtype, hipStream_t stream);
hipError_t launch_add_layernorm(void *y, void *residual_out, const void *x, const void *residual,
                                const void *gamma, const void *beta, int64_t rows, int64_t hidden,
                                float eps, int dtype, hipStream_t stream);
hipError_t launch_mrope(void *q, void *k, const int32_t *pos, int64_t pos_stride, int64_t tokens,
                        int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t q_stride,
                        int64_t k_stride, int32_t sec_t, int32_t sec_h, const mrope_freqs &fr,
                        int dtype, hipStream_t stream);
hipError_t launch_mrope_kv(void *q, const void *k, const void *v, const int32_t *pos,
                           int64_t pos_stride, int64_t tokens, int32_t n_q, int32_t n_kv,
                           int32_t head_dim, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                           int32_t sec_t, int32_t sec_h, const mrope_freqs &fr, void *k_cache,
                           void *v_cache, const int32_t *seq_idx, const int32_t *slot,
                           int64_t n_seqs, int64_t max_seq, int dtype, hipStream_t stream);
hipError_t launch_swiglu(void *out, const void *gate_up, int64_t rows, int64_t inter,
                         int64_t gu_stride, int64_t out_stride, int dtype, hipStream_t stream);
hipError_t launch_topk_sample(int32_t *token, void *probs, const void *logits, int64_t rows,
                              int64_t vocab, int64_t row_stride, int64_t probs_stride,
                              float temperature, int32_t top_k, const float *u, int dtype,
                              hipStream_t stream);
hipError_t launch_rmsnorm_linear(void *out, const void *x, const void *w, int64_t rows,
                                 int64_t n_in, int64_t n_out, int64_t x_stride, int64_t w_stride,
                                 int64_t out_stride, float eps, int dtype, hipStream_t stream);
hipError_t launch_empty(hipStream_t stream);
hipError_t launch_stream_probe(void *d0, void *d1, const void *s0, const void *s1, int n_read,
                               int n_write, int64_t bytes, int64_t row_bytes, int variant,
                               hipStream_t stream);

}  // namespace nrs
