/*
 * libnrs: fused per-token decoder-layer ops (RMSNorm, residual-add + RMSNorm,
 * M-RoPE, SwiGLU) as hand-written HIP kernels for AMD CDNA4 (gfx950), behind
 * a plain C ABI; beyond them, M-RoPE fused with the KV-cache append, softmax +
 * top-k sampling, LayerNorm, and RMSNorm fused into a Linear.
 *
 * Conventions for every entry point below:
 *   - Tensor pointers are DEVICE pointers; sizes and strides count ELEMENTS;
 *     rows are row-major with unit element stride inside a row.
 *   - dtype is NRS_F32 or NRS_BF16 and applies to every tensor argument of the
 *     call (inputs, weights and outputs); arithmetic is fp32 inside, each
 *     output is rounded once to the storage type, nearest-even.
 *   - The caller owns every buffer; the library allocates nothing per call,
 *     keeps no state between calls and is re-entrant.
 *   - `stream` is a hipStream_t (NULL = the null stream).  A call only
 *     validates its arguments on the host and enqueues kernels on `stream`;
 *     it never synchronises, allocates or copies, so it may be recorded by
 *     hipStreamBeginCapture.  Results are ready when the stream reaches them.
 *   - Errors: a negative nrs_status.  Argument checks run on the host before
 *     any HIP call, so an invalid call touches neither the GPU nor its
 *     buffers.  A zero-sized call (rows or tokens == 0) returns NRS_OK and
 *     launches nothing; rows and tokens above 2^31 - 1 return NRS_ERR_SHAPE.  NRS_ERR_HIP means the launch itself failed;
 *     nrs_last_hip_error() then gives the hipError_t of this thread's call.
 *   - Pointers must be 16-byte aligned and strides must span whole 16-byte
 *     chunks (NRS_ERR_ALIGN otherwise).  Buffers may not overlap except where
 *     an entry point says so.
 *
 * Sources of the operations (web pages, cited by title and section):
 *   [P1] "Optimising autoregressive speech models" (research.convozen.ai),
 *        section 09 "LayerNorm -> RMSNorm", parts "What it is" and "How to swap".
 *   [P2] "Open Source: Triton-Kernel-Fusion beschleunigt die Inferenz von
 *        Qwen3-TTS um bis zu das Fuenffache" (de.news.hada.io topic 27742),
 *        part 3: the four fused ops RMSNorm, M-RoPE, Norm+Residual, SwiGLU,
 *        and the CUDA-graph replay of the decode step ("Hybrid" note).
 *   [P3] forpes.ru post 233929, stage 2 "RoPE": positions enter Q and K as a
 *        rotation in the complex plane.
 */
#ifndef NRS_H
#define NRS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NRS_ABI_VERSION 1

typedef enum { NRS_F32 = 0, NRS_BF16 = 1 } nrs_dtype;

typedef enum {
    NRS_OK = 0,
    NRS_ERR_NULL = -1,     /* a required pointer is NULL */
    NRS_ERR_SHAPE = -2,    /* negative or unsupported size, stride shorter than a row */
    NRS_ERR_ALIGN = -3,    /* pointer not 16-byte aligned, or stride not whole 16-byte chunks */
    NRS_ERR_DTYPE = -4,    /* dtype is neither NRS_F32 nor NRS_BF16 */
    NRS_ERR_SECTIONS = -5, /* M-RoPE sections negative or not summing to head_dim / 2 */
    NRS_ERR_ARG = -6,      /* eps negative/NaN/inf, theta not finite and positive, bad count */
    NRS_ERR_HIP = -7       /* a HIP runtime call failed; see nrs_last_hip_error() */
} nrs_status;

/* NRS_ABI_VERSION of the loaded library. */
int nrs_abi_version(void);

/* Static text for a status code (never NULL). */
const char *nrs_status_string(int status);

/* hipError_t of the last failing HIP call made by this thread inside libnrs
 * (0 if none). */
int nrs_last_hip_error(void);

/*
 * RMSNorm, [P1] section 09 "What it is": y = gamma * x / sqrt(mean(x^2) + eps),
 * the mean over the hidden axis of each row ("How to swap": mean over the
 * last dimension, eps inside the root, the weight applied last).
 *   y[rows][y_stride]  out; x[rows][x_stride]  in; gamma[hidden]  in.
 *   hidden: a multiple of 8 (bf16) or 4 (fp32), at most 65536 bf16 / 32768
 *   fp32 elements; strides >= hidden.
 *   eps: >= 0, finite, used as given (fp32).
 *   y == x (exactly) is allowed.
 */
int nrs_rmsnorm(void *y, const void *x, const void *gamma, int64_t rows, int64_t hidden,
                int64_t x_stride, int64_t y_stride, float eps, int dtype, void *stream);

/*
 * Fused residual add + RMSNorm, [P2] part 3 "Norm+Residual":
 *   h = round(x + residual)   -> residual_out  (the residual stream carried on)
 *   y = RMSNorm(h; gamma, eps)                  (the norm sees the rounded h)
 * in one pass over the rows.  All four [rows][hidden] tensors are contiguous;
 * gamma is [hidden].  Limits on hidden and eps as for nrs_rmsnorm.
 * Exact aliasing y == x and/or residual_out == residual is allowed.
 */
int nrs_add_rmsnorm(void *y, void *residual_out, const void *x, const void *residual,
                    const void *gamma, int64_t rows, int64_t hidden, float eps, int dtype,
                    void *stream);

/*
 * LayerNorm, [P1] section 09 "What it is":
 *   y = gamma * (x - mean) / sqrt(variance + eps) + beta
 * over the hidden axis of each row; variance is the population variance
 * about the row mean (divided by hidden), as in the torch LayerNorm module
 * the section's swap loop replaces.  Arguments as for nrs_rmsnorm, plus
 *   beta[hidden]  in, 16-byte aligned, or NULL for a LayerNorm without bias.
 *   y == x (exactly) is allowed.
 */
int nrs_layernorm(void *y, const void *x, const void *gamma, const void *beta, int64_t rows,
                  int64_t hidden, int64_t x_stride, int64_t y_stride, float eps, int dtype,
                  void *stream);

/*
 * Fused residual add + LayerNorm, "Norm+Residual" ([P2] part 3) with the
 * LayerNorm of [P1] section 09:
 *   h = round(x + residual) -> residual_out;  y = LayerNorm(h; gamma, beta, eps)
 * Layout, limits and aliasing as for nrs_add_rmsnorm; beta may be NULL.
 */
int nrs_add_layernorm(void *y, void *residual_out, const void *x, const void *residual,
                      const void *gamma, const void *beta, int64_t rows, int64_t hidden,
                      float eps, int dtype, void *stream);

/*
 * Fused RMSNorm + Linear, [P1] "Custom Triton kernels", kernel 1: each row
 * is normalised by its root-mean-square and multiplied by the weight in one
 * kernel, with no gain (a gain folds into the weight's columns):
 *   out[m][k] = sum_n (x[m][n] / rms_m) * w[k][n],  rms_m = sqrt(mean_n x[m][n]^2 + eps)
 *   x[rows][x_stride]  in; w[out_features][w_stride]  in (torch's Linear
 *   layout, input index fastest); out[rows][out_stride]  out.
 *   in_features: a multiple of 8 (bf16) or 4 (fp32), at most 2^20;
 *   1 <= out_features < 2^31; strides >= the row widths; eps >= 0, finite.
 *   x and w follow the 16-byte rules above; out needs only element alignment
 *   and any out_stride (it is written element by element).
 * Products are accumulated in fp32 (on the matrix cores, or as bf16 pair dot
 * products for up to 8 bf16 rows) and each row is scaled by 1/rms at the end;
 * the normalised row is never stored.  out must not overlap x or w.
 */
int nrs_rmsnorm_linear(void *out, const void *x, const void *w, int64_t rows, int64_t in_features,
                       int64_t out_features, int64_t x_stride, int64_t w_stride,
                       int64_t out_stride, float eps, int dtype, void *stream);

/*
 * Multimodal rotary position embedding, in place on q and k.  [P3] stage 2:
 * the position enters Q and K as a rotation in the complex plane; [P2] part 3
 * names the multimodal (three-stream) variant.  For token t, every q and k
 * head, and pair j < head_dim/2 of elements (j, j + head_dim/2):
 *   stream s(j) = temporal if j < sec_t, height if j < sec_t + sec_h, else width
 *   phi = pos[s(j)][t] * theta^(-2j/head_dim)
 *   (a, b) -> (a cos phi - b sin phi, b cos phi + a sin phi)
 *   q[tokens][q_token_stride]: n_q_heads heads of head_dim, packed in a token.
 *   k[tokens][k_token_stride]: n_kv_heads heads likewise (may be 0 heads).
 *   pos: int32 [3][pos_stride] (temporal, height, width rows), pos_stride >=
 *   tokens, 4-byte aligned; |pos| < 2^24 keeps the angle exact.
 *   head_dim: a multiple of 16 (bf16) or 8 (fp32), at most 512;
 *   sec_t + sec_h + sec_w == head_dim / 2, each >= 0; theta finite, > 0.
 *   q and k must not overlap (they may sit in one packed qkv buffer).
 */
int nrs_mrope(void *q, void *k, const int32_t *pos, int64_t pos_stride, int64_t tokens,
              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int64_t q_token_stride,
              int64_t k_token_stride, int32_t sec_t, int32_t sec_h, int32_t sec_w, double theta,
              int dtype, void *stream);

/*
 * M-RoPE fused with the KV-cache append.  [P1] "Custom Triton kernels",
 * kernel 3 (KV cache update): the new K and V head vectors of a step are
 * written into the cache at [head][position][:].  Here each of n_seqs
 * sequences owns a cache [n_kv_heads][max_seq][head_dim]:
 *   k_cache, v_cache: [n_seqs][n_kv_heads][max_seq][head_dim], 16-byte aligned.
 *   n_seqs >= 1, 1 <= max_seq <= 2^36.
 *   seq_idx[tokens], slot[tokens]: int32 device arrays; token t goes to
 *     sequence seq_idx[t], position slot[t] of that sequence's cache.  A token
 *     whose index is outside [0, n_seqs) or slot outside [0, max_seq) writes
 *     no cache entry (the device data is not otherwise checked).
 *   q: rotated in place exactly as nrs_mrope does.
 *   k: read only; its rotated values go to k_cache (one trip through memory).
 *   v[tokens][v_token_stride]: read only; copied unchanged to v_cache.
 *   pos, sections, theta, head_dim, strides: as for nrs_mrope.
 * Two tokens naming the same (sequence, slot) race; the caches must not
 * overlap q, k or v.
 */
int nrs_mrope_kv_append(void *q, const void *k, const void *v, const int32_t *pos,
                        int64_t pos_stride, int64_t tokens, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, int64_t q_token_stride, int64_t k_token_stride,
                        int64_t v_token_stride, int32_t sec_t, int32_t sec_h, int32_t sec_w,
                        double theta, void *k_cache, void *v_cache, const int32_t *seq_idx,
                        const int32_t *slot, int64_t n_seqs, int64_t max_seq, int dtype,
                        void *stream);

/*
 * SwiGLU, [P2] part 3: out = silu(gate) * up, silu(g) = g * sigmoid(g).
 *   gate_up[rows][gate_up_stride]: each row is [gate (inter) | up (inter)].
 *   out[rows][out_stride]: inter elements per row.
 *   inter: a multiple of 8 (bf16) or 4 (fp32); gate_up_stride >= 2*inter,
 *   out_stride >= inter.  out must not overlap gate_up.
 */
int nrs_swiglu(void *out, const void *gate_up, int64_t rows, int64_t inter,
               int64_t gate_up_stride, int64_t out_stride, int dtype, void *stream);

/*
 * Fused softmax + top-k sampling over vocabulary logits.  [P1] "Custom Triton
 * kernels", kernel 2: softmax(logits / temperature) then sampling in one
 * pass over the row (the page's sketch stops after the softmax; its top-k and
 * sampling steps are completed as follows).  Per row: keep the top_k largest
 * logits (lower index first on equal logits), renormalise their probabilities,
 * and write to token[row] the first kept index, in that order, whose
 * cumulative probability exceeds u[row] (the last kept index if rounding
 * leaves none).
 *   logits[rows][row_stride]: vocab values per row; vocab a multiple of 8
 *     (bf16) or 4 (fp32), below 2^31.
 *   u[rows]: fp32 uniforms in [0, 1) chosen by the caller (device array).
 *   token[rows]: int32 output.
 *   probs[rows][probs_stride]: optional (NULL: not written) softmax over the
 *     whole row at this temperature, in the logits' type.
 *   top_k: 1..1024 and <= vocab; temperature finite and > 0 (NRS_ERR_ARG).
 * NaN logits give an unspecified token.
 */
int nrs_softmax_topk_sample(int32_t *token, void *probs, const void *logits, int64_t rows,
                            int64_t vocab, int64_t row_stride, int64_t probs_stride,
                            float temperature, int32_t top_k, const float *u, int dtype,
                            void *stream);

/* ---------------------------------------------------------------------------
 * Decode-step graphs.  [P2] part 3 ("Hybrid" note) replays the decode step as
 * a CUDA graph on top of the fused kernels; here the per-layer op set is
 * recorded once into a hipGraph and replayed with a single launch.
 * ------------------------------------------------------------------------- */

typedef struct nrs_graph_s *nrs_graph;

/* Shapes shared by every layer of a decode step. */
typedef struct {
    int64_t tokens;      /* rows per op (sequences x new tokens) */
    int64_t hidden;
    int64_t inter;       /* SwiGLU width; gate_up rows are 2*inter, contiguous */
    int32_t n_q_heads, n_kv_heads, head_dim;
    const int32_t *pos;  /* int32 [3][pos_stride] device pointer */
    int64_t pos_stride;
    int32_t sec_t, sec_h, sec_w;
    double theta;
    float eps;
    int32_t dtype;
} nrs_decode_shape;

/* Device buffers of one layer.  The op order within a layer is
 *   add_rmsnorm(in_*) -> mrope(q, k) -> [add_rmsnorm(post_*)] -> swiglu,
 * the post-attention norm being recorded only when post_x is non-NULL.
 * All tensors are contiguous: [tokens][hidden], q [tokens][n_q][D],
 * k [tokens][n_kv][D], gate_up [tokens][2*inter], act_out [tokens][inter]. */
typedef struct {
    void *in_y, *in_residual_out;
    const void *in_x, *in_residual, *in_gamma;
    void *q, *k;
    void *post_y, *post_residual_out;
    const void *post_x, *post_residual, *post_gamma;
    void *act_out;
    const void *gate_up;
} nrs_decode_layer;

/* Record n_layers layers into a graph.  Buffers are bound at creation: the
 * graph reads and writes exactly these pointers on every launch.  Validates
 * every op first (same errors as the single-op calls); allocates the graph. */
int nrs_decode_graph_create(nrs_graph *out, const nrs_decode_shape *shape,
                            const nrs_decode_layer *layers, int32_t n_layers);

/* Calibration: a graph of n_nodes empty kernels (1 wave each), recorded the
 * same way, giving the per-node launch floor of a replay. */
int nrs_null_graph_create(nrs_graph *out, int32_t n_nodes);

/* Measurement aid (not an op): a streaming kernel that reads n_read (0-2)
 * buffers src0, src1 and writes n_write (0-2) buffers dst0, dst1, each of
 * `bytes` bytes, every 16-byte chunk once, with nontemporal loads (cached
 * accesses when the call moves under 16 MiB in all, as the ops do).
 *   row_bytes == 0: one 16-byte access per thread and buffer; `variant`
 *     picks one of the four patterns that streamed fastest on MI355X: bit 0
 *     set = 256-thread workgroups (else 64), bit 1 set = stores with the
 *     sc1 + nt cache policy (else nontemporal only).  What it writes: dst0 =
 *     src0 XOR src1 (a missing src reads as 0; a counter pattern when
 *     n_read == 0), dst1 = NOT of src0 (NOT of dst0 when n_read == 0); with
 *     n_write == 0 nothing is written.
 *   row_bytes > 0: a row-granular copy, the access pattern of a single-pass
 *     row reduction: whole rows of row_bytes (1, 2, 3, 4, 6, 8, 12 or 16 KiB)
 *     per workgroup, n_read == n_write (1 or 2); variant 0 = one row per
 *     workgroup, one chunk per thread; variant 1 = one wave per row, four
 *     rows per 256-thread workgroup.  It writes dst0 = src0 (XOR src1),
 *     dst1 = NOT of src0; bytes must be a whole number of rows.
 *   row_bytes > 0 with n_read == 1 and n_write == 0: a row-granular read,
 *     the access pattern of the sampler's long rows: one 1024-thread
 *     workgroup per row of row_bytes (a multiple of 16, at most 1 GiB),
 *     thread t reading chunks t, t + 1024, ..., its first 8 together, then
 *     the rest 4 (variant 0) or 8 (variant 1) at a time; nothing is written;
 *     bytes must be a whole number of rows, at most 2^31 - 1 of them.
 * The fastest variant at an op's read/write mix and size is the practical
 * ceiling the op is compared with.
 *   1 <= n_read + n_write; 0 <= variant <= 3 (0-1 with rows), other
 *   combinations NRS_ERR_ARG; bytes >= 0, a multiple of 16; the buffers in
 *   use are 16-byte aligned and must not overlap.  Unused pointers may be
 *   NULL. */
int nrs_stream_probe(void *dst0, void *dst1, const void *src0, const void *src1, int32_t n_read,
                     int32_t n_write, int64_t bytes, int64_t row_bytes, int32_t variant,
                     void *stream);

/* Number of kernel nodes recorded in a graph (>= 0), or a negative status. */
int nrs_graph_node_count(nrs_graph g);

/* Enqueue one replay of the graph on `stream`. */
int nrs_graph_launch(nrs_graph g, void *stream);

/* Release a graph (NULL is a no-op).  The caller must ensure no launch of it
 * is still pending. */
int nrs_graph_destroy(nrs_graph g);

#ifdef __cplusplus
}
#endif

#endif /* NRS_H */
