/*
 * fp64 CPU oracle for the per-token decoder-layer ops (RMSNorm, the fused
 * residual add + RMSNorm, M-RoPE, SwiGLU) and the ops built beside them
 * (M-RoPE + KV-cache append, softmax + top-k sampling, LayerNorm, RMSNorm +
 * Linear).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library; it is plain C99 + libm,
 * deliberately slow and written to be checked against the pages by eye.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "Optimising autoregressive speech models" (research.convozen.ai),
 *        section 09 "LayerNorm -> RMSNorm": "What it is" gives the RMSNorm
 *        formula, "How to swap" the eager module (mean over the last axis,
 *        eps inside the root, weight applied last, eps default 1e-6).
 *   [P2] "Open Source: Triton-Kernel-Fusion beschleunigt die Inferenz von
 *        Qwen3-TTS ..." (de.news.hada.io topic 27742; French and Vietnamese
 *        copies on fr./vi.news.hada.io), part 3: the four fused ops RMSNorm,
 *        M-RoPE, Norm+Residual and SwiGLU, named without formulas.
 *   [P3] forpes.ru post 233929 (Yandex TTS decoder), stage 2 "RoPE": positions
 *        enter Q and K as a rotation in the complex plane.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - Inputs are the stored fp32/bf16 values, widened exactly to double.
 *   - Results are returned unrounded in double; oracle_round() rounds a double
 *     straight to the storage type (RNE) with no fp32 step in between.
 *   - Norm+Residual: h = round_io(x + residual) is stored as residual_out and
 *     the norm sees that rounded h.
 *   - LayerNorm: population variance about the row mean; beta optional; the
 *     fused add variant stores and normalises the rounded h as above.
 *   - RMSNorm + Linear: no gain; weight [n_out][n_in] (torch's Linear layout).
 *   - M-RoPE: half-split pairs (j, j + D/2); pairs [0, s_t) follow the
 *     temporal stream, [s_t, s_t+s_h) the height stream, the rest the width
 *     stream; frequency theta^(-2j/D) as in standard RoPE, same for all
 *     streams; angle = position * frequency in double.
 *   - SwiGLU: gate is the first half of each gate_up row, up the second;
 *     silu(g) = g * sigmoid(g).
 *   - KV-cache append: one cache [n_kv][max_seq][head_dim] per sequence; each
 *     token names its sequence and slot; out-of-range tokens write nothing.
 *   - Softmax + top-k sampling: top_k largest logits (lower index on ties),
 *     renormalised, inverse-CDF sample with a caller-supplied uniform.
 *
 * Parity pins live in the CPU tests (closed forms, invariants, library
 * routines, a hand example); no function here is "parity unpinned".
 */
#include "oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Stored element -> double.  bf16 is the top half of an fp32 bit pattern. */
static double widen(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_F32) {
        return (double)((const float *)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* double -> bf16 bit pattern, round to nearest, ties to even, directly.
 * bf16 keeps 8 significant bits over fp32's exponent range, so a finite
 * value is a multiple of its quantum 2^(e-7) (e = binary exponent, clamped
 * at -126 where the subnormals begin, quantum 2^-133). */
static uint16_t to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) {
        return (uint16_t)(sign | 0x7FC0u);
    }
    double a = fabs(v);
    if (isinf(a)) {
        return (uint16_t)(sign | 0x7F80u);
    }
    if (a == 0.0) {
        return sign;
    }
    int e = ilogb(a);
    if (e < -126) {
        e = -126;
    }
    double quantum = ldexp(1.0, e - 7);
    double r = nearbyint(a / quantum) * quantum; /* default mode: ties to even */
    if (r >= 0x1p128) {
        return (uint16_t)(sign | 0x7F80u);
    }
    float f = (float)r; /* exact: at most 8 significant bits, exponent in range */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

static void put(void *base, int64_t idx, double v, int dtype)
{
    if (dtype == ORACLE_F32) {
        ((float *)base)[idx] = (float)v; /* C conversion: round to nearest even */
    } else {
        ((uint16_t *)base)[idx] = to_bf16(v);
    }
}

void oracle_round(void *out, const double *r, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) {
        put(out, i, r[i], dtype);
    }
}

void oracle_widen(double *out, const void *in, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) {
        out[i] = widen(in, i, dtype);
    }
}

/* [P1] section 09, "What it is": RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps),
 * the mean taken over the hidden (last) axis as in "How to swap". */
void oracle_rmsnorm(double *y, const void *x, const void *gamma, int64_t rows,
                    int64_t hidden, int64_t x_stride, double eps, int dtype)
{
    for (int64_t t = 0; t < rows; ++t) {
        const int64_t base = t * x_stride;
        double sum_sq = 0.0;
        for (int64_t i = 0; i < hidden; ++i) {
            double v = widen(x, base + i, dtype);
            sum_sq += v * v;
        }
        double mean_sq = sum_sq / (double)hidden;
        double root = sqrt(mean_sq + eps);
        for (int64_t i = 0; i < hidden; ++i) {
            y[t * hidden + i] = widen(gamma, i, dtype) * widen(x, base + i, dtype) / root;
        }
    }
}

/* [P2] part 3 "Norm+Residual": the residual add followed by RMSNorm.
 * h = round_io(x + residual) is what the residual stream carries on, so it is
 * written to residual_out; the norm then runs on that stored h. */
void oracle_add_rmsnorm(double *y, void *residual_out, const void *x,
                        const void *residual, const void *gamma, int64_t rows,
                        int64_t hidden, double eps, int dtype)
{
    for (int64_t t = 0; t < rows; ++t) {
        for (int64_t i = 0; i < hidden; ++i) {
            const int64_t at = t * hidden + i;
            put(residual_out, at, widen(x, at, dtype) + widen(residual, at, dtype), dtype);
        }
    }
    oracle_rmsnorm(y, residual_out, gamma, rows, hidden, hidden, eps, dtype);
}

/* [P1] section 09, "What it is": LayerNorm(x) = gamma * (x - mean) /
 * sqrt(variance + eps) + beta over the hidden axis.  The variance is the
 * population variance about the row mean (divided by hidden, as in the
 * torch LayerNorm module the page's swap loop replaces); beta may be NULL
 * (a LayerNorm without bias). */
void oracle_layernorm(double *y, const void *x, const void *gamma, const void *beta,
                      int64_t rows, int64_t hidden, int64_t x_stride, double eps, int dtype)
{
    for (int64_t t = 0; t < rows; ++t) {
        const int64_t row_at = t * x_stride;
        double sum = 0.0;
        for (int64_t i = 0; i < hidden; ++i) {
            sum += widen(x, row_at + i, dtype);
        }
        double mean = sum / (double)hidden;
        double sum_dev_sq = 0.0;
        for (int64_t i = 0; i < hidden; ++i) {
            double d = widen(x, row_at + i, dtype) - mean;
            sum_dev_sq += d * d;
        }
        double variance = sum_dev_sq / (double)hidden;
        double root = sqrt(variance + eps);
        for (int64_t i = 0; i < hidden; ++i) {
            double v = widen(gamma, i, dtype) * (widen(x, row_at + i, dtype) - mean) / root;
            if (beta != NULL) {
                v += widen(beta, i, dtype);
            }
            y[t * hidden + i] = v;
        }
    }
}

/* The residual add followed by LayerNorm, read like "Norm+Residual" ([P2]
 * part 3): h = round_io(x + residual) is stored and normalised. */
void oracle_add_layernorm(double *y, void *residual_out, const void *x,
                          const void *residual, const void *gamma, const void *beta,
                          int64_t rows, int64_t hidden, double eps, int dtype)
{
    for (int64_t t = 0; t < rows; ++t) {
        for (int64_t i = 0; i < hidden; ++i) {
            const int64_t at = t * hidden + i;
            put(residual_out, at, widen(residual, at, dtype) + widen(x, at, dtype), dtype);
        }
    }
    oracle_layernorm(y, residual_out, gamma, beta, rows, hidden, hidden, eps, dtype);
}

/* [P1] "Custom Triton kernels", kernel 1 (fused RMSNorm + Linear): each row
 * is divided by its root-mean-square sqrt(mean(x^2) + eps), written in the
 * listing's sqrt-then-divide form, and multiplied by the weight; no gain is
 * applied (a gain folds into the weight's columns).  The weight is stored as
 * torch's Linear stores it, [n_out][n_in]:
 *   out[m][k] = sum_n (x[m][n] / rms_m) * w[k][n]. */
void oracle_rmsnorm_linear(double *out, const void *x, const void *w, int64_t rows,
                           int64_t n_in, int64_t n_out, int64_t x_stride, int64_t w_stride,
                           double eps, int dtype)
{
    double *xn = malloc((size_t)(n_in > 0 ? n_in : 1) * sizeof *xn);
    for (int64_t m = 0; m < rows; ++m) {
        const int64_t xrow = m * x_stride;
        double sum_sq = 0.0;
        for (int64_t n = 0; n < n_in; ++n) {
            double v = widen(x, xrow + n, dtype);
            sum_sq += v * v;
        }
        double rms = sqrt(sum_sq / (double)n_in + eps);
        for (int64_t n = 0; n < n_in; ++n) {
            xn[n] = widen(x, xrow + n, dtype) / rms;
        }
        for (int64_t k = 0; k < n_out; ++k) {
            double acc = 0.0;
            for (int64_t n = 0; n < n_in; ++n) {
                acc += xn[n] * widen(w, k * w_stride + n, dtype);
            }
            out[m * n_out + k] = acc;
        }
    }
    free(xn);
}

/* Which position stream drives frequency pair j: temporal, height, width. */
static int stream_of_pair(int j, int sec_t, int sec_h)
{
    if (j < sec_t) {
        return 0;
    }
    if (j < sec_t + sec_h) {
        return 1;
    }
    return 2;
}

/* Rotate every (j, j + D/2) pair of `heads` head vectors of one token. */
static void rotate_heads(double *out, const void *v, int64_t base, int heads, int head_dim,
                         const double *c, const double *s, int dtype)
{
    const int half = head_dim / 2;
    for (int h = 0; h < heads; ++h) {
        const int64_t hb = base + (int64_t)h * head_dim;
        for (int j = 0; j < half; ++j) {
            double a = widen(v, hb + j, dtype);
            double b = widen(v, hb + j + half, dtype);
            /* (a + i b) * (cos + i sin) */
            out[h * head_dim + j] = a * c[j] - b * s[j];
            out[h * head_dim + j + half] = b * c[j] + a * s[j];
        }
    }
}

/* [P3] stage 2: RoPE puts the position into Q and K as a rotation in the
 * complex plane; [P2] part 3 names the multimodal variant (M-RoPE), whose
 * three position streams (temporal, height, width) each drive one contiguous
 * section of the frequency pairs.  Output: dense [tokens][heads][head_dim]. */
void oracle_mrope(double *q_out, double *k_out, const void *q, const void *k,
                  const int32_t *pos, int64_t pos_stride, int64_t tokens, int n_q_heads,
                  int n_kv_heads, int head_dim, int64_t q_token_stride,
                  int64_t k_token_stride, int sec_t, int sec_h, int sec_w, double theta,
                  int dtype)
{
    (void)sec_w; /* sec_t + sec_h + sec_w == head_dim / 2; the rest is width */
    const int half = head_dim / 2;
    double c[ORACLE_MAX_HALF], s[ORACLE_MAX_HALF];
    for (int64_t t = 0; t < tokens; ++t) {
        for (int j = 0; j < half; ++j) {
            int stream = stream_of_pair(j, sec_t, sec_h);
            double p = (double)pos[stream * pos_stride + t];
            double freq = pow(theta, -2.0 * (double)j / (double)head_dim);
            double phi = p * freq;
            c[j] = cos(phi);
            s[j] = sin(phi);
        }
        rotate_heads(q_out + t * (int64_t)n_q_heads * head_dim, q, t * q_token_stride,
                     n_q_heads, head_dim, c, s, dtype);
        rotate_heads(k_out + t * (int64_t)n_kv_heads * head_dim, k, t * k_token_stride,
                     n_kv_heads, head_dim, c, s, dtype);
    }
}

/* [P1] "Custom Triton kernels", kernel 3 (KV cache update): each new K, V
 * head vector is written into its cache at [head][position][:], here with one
 * cache of [n_kv][max_seq][head_dim] per sequence, so entry (b, h, s) is at
 * ((b * n_kv + h) * max_seq + s) * head_dim.  Fused with M-RoPE: q is rotated
 * (returned in q_out), k is rotated and the rotated k goes to the k cache (k
 * itself is only read), v is copied unchanged into the v cache.  A token whose
 * sequence index or slot is out of range writes nothing.  k_cache_out holds
 * double values (the caller fills it beforehand); v_cache holds the storage
 * type. */
void oracle_mrope_kv_append(double *q_out, double *k_cache_out, void *v_cache,
                            const void *q, const void *k, const void *v,
                            const int32_t *pos, int64_t pos_stride, int64_t tokens, int n_q_heads,
                            int n_kv_heads, int head_dim, int64_t q_token_stride,
                            int64_t k_token_stride, int64_t v_token_stride, int sec_t, int sec_h,
                            int sec_w, double theta, const int32_t *seq_idx, const int32_t *slot,
                            int64_t n_seqs, int64_t max_seq, int dtype)
{
    double *k_rot = (double *)malloc(sizeof(double) * (size_t)(n_kv_heads > 0 ? n_kv_heads : 1) *
                                     (size_t)head_dim);
    for (int64_t t = 0; t < tokens; ++t) {
        /* rotate this token's q and k with the single-token M-RoPE above */
        const int32_t p3[3] = {pos[t], pos[pos_stride + t], pos[2 * pos_stride + t]};
        oracle_mrope(q_out + t * (int64_t)n_q_heads * head_dim, k_rot,
                     (const char *)q + t * q_token_stride * (dtype == ORACLE_F32 ? 4 : 2),
                     (const char *)k + t * k_token_stride * (dtype == ORACLE_F32 ? 4 : 2), p3, 1, 1,
                     n_q_heads, n_kv_heads, head_dim, 0, 0, sec_t, sec_h, sec_w, theta, dtype);
        const int64_t b = seq_idx[t], s = slot[t];
        if (b < 0 || b >= n_seqs || s < 0 || s >= max_seq) {
            continue;
        }
        for (int h = 0; h < n_kv_heads; ++h) {
            const int64_t at = ((b * n_kv_heads + h) * max_seq + s) * head_dim;
            for (int d = 0; d < head_dim; ++d) {
                k_cache_out[at + d] = k_rot[h * head_dim + d];
                put(v_cache, at + d, widen(v, t * v_token_stride + (int64_t)h * head_dim + d, dtype),
                    dtype);
            }
        }
    }
    free(k_rot);
}

/* Order of two candidates for top-k: larger logit first, lower index on a tie. */
static const double *g_topk_vals;
static int topk_order(const void *a, const void *b)
{
    const int64_t i = *(const int64_t *)a, j = *(const int64_t *)b;
    const double x = g_topk_vals[i], y = g_topk_vals[j];
    if (x > y) {
        return -1;
    }
    if (x < y) {
        return 1;
    }
    return i < j ? -1 : (i > j ? 1 : 0);
}

/* [P1] "Custom Triton kernels", kernel 2 (fused softmax + top-K sampling):
 * probs = softmax(logits / temperature) over the vocabulary (the page divides
 * by the temperature, subtracts the max, exponentiates and normalises; its
 * top-K and sampling steps are cut off).  Reading for the missing steps: keep
 * the top_k largest logits (lower index first on ties), renormalise their
 * probabilities, and return the first kept token, in that order, whose
 * cumulative probability exceeds u[row] (the last kept token if rounding
 * leaves none).  probs (double, [rows][vocab]) may be NULL.  For the parity
 * check, kept[row][top_k] receives the kept tokens in order and cdf[row][top_k]
 * their exact cumulative probabilities (both may be NULL). */
void oracle_softmax_topk_sample(int32_t *token, double *probs, int64_t *kept, double *cdf,
                                const void *logits, int64_t rows, int64_t vocab,
                                int64_t row_stride, double temperature, int64_t top_k,
                                const float *u, int dtype)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)vocab);
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)vocab);
    for (int64_t r = 0; r < rows; ++r) {
        double zmax = -INFINITY;
        for (int64_t i = 0; i < vocab; ++i) {
            z[i] = widen(logits, r * row_stride + i, dtype) / temperature;
            if (z[i] > zmax) {
                zmax = z[i];
            }
        }
        if (probs) {
            double sum = 0.0;
            for (int64_t i = 0; i < vocab; ++i) {
                sum += exp(z[i] - zmax);
            }
            for (int64_t i = 0; i < vocab; ++i) {
                probs[r * vocab + i] = exp(z[i] - zmax) / sum;
            }
        }
        /* rank by the logits themselves: dividing by temperature > 0 keeps the order */
        for (int64_t i = 0; i < vocab; ++i) {
            order[i] = i;
            z[i] = widen(logits, r * row_stride + i, dtype);
        }
        g_topk_vals = z;
        qsort(order, (size_t)vocab, sizeof(int64_t), topk_order);
        const double zt = z[order[0]] / temperature;
        double kept_sum = 0.0;
        for (int64_t j = 0; j < top_k; ++j) {
            kept_sum += exp(z[order[j]] / temperature - zt);
        }
        double cum = 0.0;
        int32_t pick = (int32_t)order[top_k - 1];
        int found = 0;
        for (int64_t j = 0; j < top_k; ++j) {
            cum += exp(z[order[j]] / temperature - zt) / kept_sum;
            if (kept) {
                kept[r * top_k + j] = order[j];
            }
            if (cdf) {
                cdf[r * top_k + j] = cum;
            }
            if (!found && cum > (double)u[r]) {
                pick = (int32_t)order[j];
                found = 1;
            }
        }
        token[r] = pick;
    }
    free(order);
    free(z);
}

/* sigmoid, evaluated so that exp never overflows: 1/(1+e^-g) for g >= 0 and
 * e^g/(1+e^g) for g < 0 (the same function, rearranged). */
static double sigmoid(double g)
{
    if (g >= 0.0) {
        return 1.0 / (1.0 + exp(-g));
    }
    double e = exp(g);
    return e / (1.0 + e);
}

/* [P2] part 3 "SwiGLU": out = silu(gate) * up with silu(g) = g * sigmoid(g);
 * each gate_up row is [gate | up], `inter` elements each. */
void oracle_swiglu(double *out, const void *gate_up, int64_t rows, int64_t inter,
                   int64_t gate_up_stride, int dtype)
{
    for (int64_t t = 0; t < rows; ++t) {
        for (int64_t i = 0; i < inter; ++i) {
            double g = widen(gate_up, t * gate_up_stride + i, dtype);
            double u = widen(gate_up, t * gate_up_stride + inter + i, dtype);
            out[t * inter + i] = g * sigmoid(g) * u;
        }
    }
}
