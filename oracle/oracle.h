/*
 * fp64 CPU oracle (test infrastructure only; see oracle.c for the sources).
 * Inputs are stored fp32 or bf16 arrays; results are unrounded doubles in
 * dense row-major layout.  No function checks its arguments.
 */
#ifndef NRS_ORACLE_H
#define NRS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_MAX_HALF = 1024 };

void oracle_round(void *out, const double *r, int64_t n, int dtype);
void oracle_widen(double *out, const void *in, int64_t n, int dtype);

/* y[rows][hidden] (double) from x rows of stride x_stride, gamma[hidden]. */
void oracle_rmsnorm(double *y, const void *x, const void *gamma, int64_t rows,
                    int64_t hidden, int64_t x_stride, double eps, int dtype);

/* residual_out (stored dtype) and y (double), all [rows][hidden] contiguous. */
void oracle_add_rmsnorm(double *y, void *residual_out, const void *x,
                        const void *residual, const void *gamma, int64_t rows,
                        int64_t hidden, double eps, int dtype);

/* y[rows][hidden] (double); beta[hidden] may be NULL. */
void oracle_layernorm(double *y, const void *x, const void *gamma, const void *beta,
                      int64_t rows, int64_t hidden, int64_t x_stride, double eps, int dtype);

/* residual_out (stored dtype) and y (double), all [rows][hidden] contiguous. */
void oracle_add_layernorm(double *y, void *residual_out, const void *x,
                          const void *residual, const void *gamma, const void *beta,
                          int64_t rows, int64_t hidden, double eps, int dtype);

/* out[rows][n_out] (double) from x rows of stride x_stride and w[n_out] rows
 * of stride w_stride (each n_in long). */
void oracle_rmsnorm_linear(double *out, const void *x, const void *w, int64_t rows,
                           int64_t n_in, int64_t n_out, int64_t x_stride, int64_t w_stride,
                           double eps, int dtype);

/* q_out[tokens][n_q][D], k_out[tokens][n_kv][D] (double); pos[3][pos_stride]. */
void oracle_mrope(double *q_out, double *k_out, const void *q, const void *k,
                  const int32_t *pos, int64_t pos_stride, int64_t tokens, int n_q_heads,
                  int n_kv_heads, int head_dim, int64_t q_token_stride,
                  int64_t k_token_stride, int sec_t, int sec_h, int sec_w, double theta,
                  int dtype);

/* q_out[tokens][n_q][D] (double); rotated k into k_cache_out and v into
 * v_cache, both [n_seqs][n_kv][max_seq][D]; seq_idx/slot[tokens]. */
void oracle_mrope_kv_append(double *q_out, double *k_cache_out, void *v_cache,
                            const void *q, const void *k, const void *v,
                            const int32_t *pos, int64_t pos_stride, int64_t tokens, int n_q_heads,
                            int n_kv_heads, int head_dim, int64_t q_token_stride,
                            int64_t k_token_stride, int64_t v_token_stride, int sec_t, int sec_h,
                            int sec_w, double theta, const int32_t *seq_idx, const int32_t *slot,
                            int64_t n_seqs, int64_t max_seq, int dtype);

/* token[rows]; probs[rows][vocab] (double, may be NULL); kept/cdf [rows][top_k]
 * (may be NULL); u[rows] uniforms in [0, 1). */
void oracle_softmax_topk_sample(int32_t *token, double *probs, int64_t *kept, double *cdf,
                                const void *logits, int64_t rows, int64_t vocab,
                                int64_t row_stride, double temperature, int64_t top_k,
                                const float *u, int dtype);

/* out[rows][inter] (double) from gate_up rows [gate | up] of stride gate_up_stride. */
void oracle_swiglu(double *out, const void *gate_up, int64_t rows, int64_t inter,
                   int64_t gate_up_stride, int dtype);

#ifdef __cplusplus
}
#endif
#endif
