// RMSNorm, LayerNorm and their fused residual-add variants for gfx950.
//
// RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps), the mean over the hidden
// axis ("Optimising autoregressive speech models", section 09 "LayerNorm ->
// RMSNorm": "What it is" and "How to swap").  LayerNorm(x) = gamma * (x -
// mean) / sqrt(variance + eps) + beta, from the same section; the variance
// is the population variance about the row mean and beta is optional.  The
// fused variants are the "Norm+Residual" op of the qwen3-tts-triton post
// (de.news.hada.io topic 27742, part 3): h = x + residual is rounded to the
// storage type, written as residual_out, and normalised in the same pass.
//
// Layout: a row is split over whole waves of 64 threads, each thread holding
// NCH 16-byte chunks, so every load instruction of a wave reads 1 KiB of
// contiguous HBM and the row stays in VGPRs between the read, the reduction
// and the write: each input byte is read once and each output byte written
// once.  A thread holds one chunk while the row fits in 16 waves (measured
// on MI355X, one 16-byte access per thread per stream in a one-shot grid
// streams faster than threads that walk several chunks or several rows), and
// the wave count follows the row so that no lane idles when the row is a
// multiple of 64 chunks; wider rows give each thread 2, 4 or 8 chunks.
//
// Reduction: DPP row operations plus four readlanes per wave (no LDS, no
// barrier); rows spanning several waves add their wave sums through a few
// bytes of LDS and one barrier.  LayerNorm reduces twice within each wave,
// the mean and then the squared deviations from it, over the registers (an
// exact two-pass variance with no extra HBM traffic), and merges the waves'
// moments through the same single barrier.
// gamma and beta are loaded together with x (they stay in L2 across rows)
// and applied last.
#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

// Sum over aligned groups of SEG lanes (SEG a power of two up to 32): every
// lane of a group ends with its group's sum.
template <int SEG> __device__ inline float seg_sum(float v) {
#pragma unroll
    for (int o = SEG / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// A row is split over WPR waves of 64 threads; each thread holds NCH chunks
// (thread t of the row owns chunks t, t + 64*WPR, ...).  Rows of one wave are
// packed four to a block, wider rows get a block each.  Rows of at most 32
// chunks (SEG < 64, e.g. per-head norms over head_dim) share a wave: each
// takes an aligned group of SEG lanes (the chunk count rounded up to a power
// of two), so a 256-thread block holds 256 / SEG rows and no wave idles on a
// short row.
// LN selects LayerNorm (beta may be null) over RMSNorm.
// ONE: one-wave rows one to a 64-thread block instead of four to a block.
template <typename IO, int WPR, int NCH, bool ADD, bool LN, bool NT, int SEG = 64, bool ONE = false>
__global__ __launch_bounds__(WPR == 1 && !ONE ? 256 : 64 * WPR) void norm_kernel(
    IO *y, IO *res_out, const IO *x, const IO *res, const IO *gamma, const IO *beta,
    int64_t rows, int32_t nchunks, int64_t x_stride, int64_t y_stride, float inv_h, float eps) {
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    static_assert(SEG == 64 || (WPR == 1 && NCH == 1), "short rows take one chunk per lane");
    static_assert(!ONE || (WPR == 1 && SEG == 64), "one row per block: one-wave rows");
    constexpr int TPR = SEG < 64 ? SEG : 64 * WPR;                     // threads per row
    constexpr int RPB = SEG < 64 ? 256 / SEG : (WPR == 1 && !ONE ? 4 : 1);   // rows per block
    __shared__ float partial[LN ? 1 : WPR * RPB];
    __shared__ float4 moments[LN ? WPR * RPB : 1];

    const int wave = threadIdx.x >> 6;
    const int rib = threadIdx.x / TPR;          // row within the block
    const int t = threadIdx.x - rib * TPR;      // thread within the row
    // a row's reduction: its lane group, or the whole wave (and LDS beyond)
    auto row_sum = [](float v) { return SEG < 64 ? seg_sum<SEG < 64 ? SEG : 1>(v) : wave_sum(v); };
    const int64_t row = (int64_t)blockIdx.x * RPB + rib;
    const bool live = row < rows;

    const bool has_beta = LN && beta != nullptr;
    u32x4 xr[NCH], rr[NCH], gr[NCH], br[LN ? NCH : 1];
    // gamma (and beta) before x (and the residual): loads return in order, so
    // waiting for x also covers gamma, and no wait for gamma lands after the
    // residual_out store (stores count in the same vmcnt on gfx950, so such a
    // wait would stall on the store's acknowledgement)
    if constexpr (sizeof(IO) == 4 && NCH >= 4) {
        // fp32 with 4 or 8 chunks per thread: every lane loads, with no
        // branch; lanes past the row's end or past the last row read the last
        // chunk of a real row and zero what they got.  With the loads inside a
        // per-chunk branch (below), these instances merged the chunk arrays
        // into one register vector, waited for each chunk before issuing the
        // next, and at 8 chunks spilled: fp32 H = 5120 add_rmsnorm took 1150 us
        // for 8192 rows, 111 us this way.  (bf16 and fewer chunks compile well
        // with the branch, and measured up to 12% slower without it.)
        const int64_t lrow = live ? row : rows - 1;
        auto chunk_off = [&](int c) {
            const int idx = t + TPR * c;
            return (int64_t)(idx < nchunks ? idx : nchunks - 1) * VEC;
        };
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            gr[c] = load16(gamma + chunk_off(c));
            if (LN) br[c] = has_beta ? load16(beta + chunk_off(c)) : u32x4{0, 0, 0, 0};
        }
        __builtin_amdgcn_sched_barrier(0);   // keeps gamma's loads first
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            xr[c] = load16_policy<NT>(x + lrow * x_stride + chunk_off(c));
            rr[c] = ADD ? load16_policy<NT>(res + lrow * x_stride + chunk_off(c)) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (!(live && t + TPR * c < nchunks)) {
                xr[c] = u32x4{0, 0, 0, 0};
                rr[c] = u32x4{0, 0, 0, 0};
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int idx = t + TPR * c;
            xr[c] = rr[c] = gr[c] = u32x4{0, 0, 0, 0};
            if (LN) br[c] = u32x4{0, 0, 0, 0};
            if (live && idx < nchunks) {
                gr[c] = load16(gamma + (int64_t)idx * VEC);
                if (has_beta) br[c] = load16(beta + (int64_t)idx * VEC);
                xr[c] = load16_policy<NT>(x + row * x_stride + (int64_t)idx * VEC);
                if (ADD) rr[c] = load16_policy<NT>(res + row * x_stride + (int64_t)idx * VEC);
            }
        }
    }

    // RMSNorm: ss = sum of squares.  LayerNorm: ss = sum.
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        float v[VEC];
        T::unpack(xr[c], v);
        if (ADD) {
            float r[VEC];
            T::unpack(rr[c], r);
#pragma unroll
            for (int i = 0; i < VEC; ++i) v[i] += r[i];
            // the stored h: one rounding to the storage type
            xr[c] = T::pack(v);
            T::unpack(xr[c], v);
            const int idx = t + TPR * c;
            if (live && idx < nchunks)
                store16_policy<NT>(res_out + row * y_stride + (int64_t)idx * VEC, xr[c]);
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) ss = LN ? ss + v[i] : __builtin_fmaf(v[i], v[i], ss);
    }
    ss = row_sum(ss);
    float mean = 0.0f;
    if (!LN) {
        if (WPR > 1) {
            if ((threadIdx.x & 63) == 0) partial[wave] = ss;
            __syncthreads();
            ss = 0.0f;
#pragma unroll
            for (int w = 0; w < WPR; ++w) ss += partial[rib * WPR + w];
        }
    } else {
        // LayerNorm moments with one barrier: each wave takes the exact
        // two-pass mean and sum of squared deviations of its own elements
        // (registers only), and the row's waves are then combined by the law of
        // total variance, M2 = sum_w [M2_w + n_w (mean_w - mean)^2], which adds
        // small differences only (no E[x^2] - E[x]^2 cancellation).
        const int wir = wave - rib * WPR;       // wave within the row
        int nw = 0;                             // elements held by this wave
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            nw += SEG < 64 ? nchunks : min(max(nchunks - TPR * c - 64 * wir, 0), 64);
        nw *= VEC;
        const float mw = nw > 0 ? ss / (float)nw : 0.0f;
        float m2 = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (t + TPR * c < nchunks) {        // lanes past the row's end add nothing
                float v[VEC];
                T::unpack(xr[c], v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float d = v[i] - mw;
                    m2 = __builtin_fmaf(d, d, m2);
                }
            }
        }
        m2 = row_sum(m2);
        mean = mw;
        if (WPR > 1) {
            if ((threadIdx.x & 63) == 0) moments[wave] = float4{ss, mw, m2, (float)nw};
            __syncthreads();
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < WPR; ++w) sum += moments[rib * WPR + w].x;
            mean = sum / (float)(nchunks * VEC);
            m2 = 0.0f;
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                const float4 p = moments[rib * WPR + w];
                const float d = p.y - mean;
                m2 += __builtin_fmaf(p.w * d, d, p.z);
            }
        }
        ss = m2;
    }
    if (!live) return;
    const float rs = rsqrtf(__builtin_fmaf(ss, inv_h, eps));
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int idx = t + TPR * c;
        if (idx < nchunks) {
            float v[VEC], g[VEC], o[VEC];
            T::unpack(xr[c], v);
            T::unpack(gr[c], g);
            if (LN) {
                float b[VEC];
                T::unpack(br[c], b);
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    o[i] = has_beta ? __builtin_fmaf((v[i] - mean) * rs, g[i], b[i])
                                    : ((v[i] - mean) * rs) * g[i];
            } else {
#pragma unroll
                for (int i = 0; i < VEC; ++i) o[i] = (v[i] * rs) * g[i];
            }
            store16_policy<NT>(y + row * y_stride + (int64_t)idx * VEC, T::pack(o));
        }
    }
}

namespace {

// Waves per row and chunks per thread: the fewest chunks per thread, from
// min_nch up, whose wave count is 1, 2, 3, 4 or 8.  Measured at 32768 rows on
// MI355X, RMSNorm rows spread over 6 or 16 waves stream 7-10% slower than the
// same rows over 3 or 8 waves with two chunks per thread, and 1-4 or 8 waves
// with one chunk are best.  LayerNorm starts from two chunks per thread: its
// second reduction lengthens each wave's load-reduce-store chain, and with
// one chunk per thread too few bytes stay in flight to cover it (hidden 1024
// to 4096: 16-20% slower than with two).
void norm_shape(int nchunks, int min_nch, int &wpr, int &nch) {
    if (nchunks < 64 * min_nch) min_nch = 1;   // short rows: keep every lane busy
    for (nch = min_nch; nch < 8; nch *= 2) {
        wpr = (nchunks + 64 * nch - 1) / (64 * nch);
        if (wpr <= 4 || wpr == 8) return;
    }
    wpr = (nchunks + 64 * nch - 1) / (64 * nch);
}

// One-wave rows of one 16-byte chunk per lane (1 KiB) in streaming calls go
// one to a 64-thread block, the rest four to a block.  Measured on MI355X
// (32768 rows, bf16 hidden 512, graph-timed, inputs rotated past the cache):
// rmsnorm 12.8 -> 12.3 us, add_rmsnorm 23.1 -> 22.8 us; with 2 or 4 chunks per
// lane, one row per block measured the same or slower.  A 64-thread block per
// 1 KiB piece, consecutive pieces on consecutive XCDs, is the pattern that
// copies fastest on this chip.
template <typename IO, bool ADD, bool LN, int WPR, bool NT>
void launch_shape(IO *y, IO *ro, const IO *x, const IO *r, const IO *g, const IO *b, int64_t rows,
                  int32_t nchunks, int nch, int64_t xs, int64_t ys, float inv_h, float eps,
                  hipStream_t stream) {
    if (WPR == 1 && nch <= 1 && NT) {
        hipLaunchKernelGGL((norm_kernel<IO, 1, 1, ADD, LN, NT, 64, true>), dim3((unsigned)rows),
                           dim3(64), 0, stream, y, ro, x, r, g, b, rows, nchunks, xs, ys, inv_h, eps);
        return;
    }
    constexpr int RPB = WPR == 1 ? 4 : 1;
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(64 * WPR * RPB);
#define NRS_NORM(N)                                                                             \
    hipLaunchKernelGGL((norm_kernel<IO, WPR, N, ADD, LN, NT>), grid, block, 0, stream, y, ro, x, r, \
                       g, b, rows, nchunks, xs, ys, inv_h, eps)
    if (nch <= 1) NRS_NORM(1);
    else if (nch <= 2) NRS_NORM(2);
    else if (nch <= 4) NRS_NORM(4);
    else NRS_NORM(8);
#undef NRS_NORM
}

// Rows of at most 32 chunks: `seg` lanes per row, 256 / seg rows per block.
template <typename IO, bool ADD, bool LN, bool NT>
void launch_short(IO *y, IO *ro, const IO *x, const IO *r, const IO *g, const IO *b, int64_t rows,
                  int32_t nchunks, int seg, int64_t xs, int64_t ys, float inv_h, float eps,
                  hipStream_t stream) {
    const dim3 grid((unsigned)((rows + 256 / seg - 1) / (256 / seg))), block(256);
#define NRS_SHORT(S)                                                                            \
    hipLaunchKernelGGL((norm_kernel<IO, 1, 1, ADD, LN, NT, S>), grid, block, 0, stream, y, ro, x, \
                       r, g, b, rows, nchunks, xs, ys, inv_h, eps)
    switch (seg) {
        case 1: NRS_SHORT(1); break;
        case 2: NRS_SHORT(2); break;
        case 4: NRS_SHORT(4); break;
        case 8: NRS_SHORT(8); break;
        case 16: NRS_SHORT(16); break;
        default: NRS_SHORT(32); break;
    }
#undef NRS_SHORT
}

template <typename IO, bool ADD, bool LN>
hipError_t launch_norm_typed(void *y, void *res_out, const void *x, const void *res,
                             const void *gamma, const void *beta, int64_t rows, int64_t hidden,
                             int64_t x_stride, int64_t y_stride, float eps, hipStream_t stream) {
    constexpr int VEC = io_traits<IO>::VEC;
    const int32_t nchunks = (int32_t)(hidden / VEC);
    const float inv_h = (float)(1.0 / (double)hidden);
    int wpr, nch;
    norm_shape(nchunks, LN ? 2 : 1, wpr, nch);
    IO *Y = (IO *)y, *RO = (IO *)res_out;
    const IO *X = (const IO *)x, *R = (const IO *)res, *G = (const IO *)gamma,
             *B = (const IO *)beta;
    const bool nt = rows * hidden * (long long)sizeof(IO) * (ADD ? 4 : 2) >= kStreamBytes;
    // Streaming-size (>= 16 MiB) calls over rows of 65-256 chunks (bf16 H =
    // 520-2048, fp32 260-1024) take one wave per row and 2 or 4 chunks per
    // thread: each wave keeps more bytes in flight and LayerNorm's moments
    // need no cross-wave step.  Measured on MI355X (graph-timed, inputs
    // rotated past the 256 MB cache): add_rmsnorm at 2048 x 2048 bf16 7.8 ->
    // 7.0 us, add_layernorm 8.4 -> 7.7 us, layernorm at 32768 x 1536 and
    // x 2048 9% and 6% faster; fp32 at 2048 x 1024 12-14% faster with the
    // residual, 6% for layernorm (once its 4-chunk loads lost their branch,
    // above); plain rmsnorm at 32768 rows, bf16 hidden 1024 23.6 -> 22.8 us
    // and hidden 2048 43.1 -> 42.9 us.  Rows of 512 chunks with 8 chunks per
    // thread were 8% slower with a residual, and small calls slower too: with
    // it, the 5-token decode step's 28-layer op set took 183 us instead of
    // 169 (its add_rmsnorm rows on fewer waves and CUs).
    if (nt && nchunks > 64 && nchunks <= 256) {
        wpr = 1;
        nch = nchunks <= 128 ? 2 : 4;
    }
    // plain RMSNorm over rows of 257-512 chunks in calls of at most 32 MiB
    // (the grid covers the chip a few times): 2 waves per row with 4 chunks
    // per thread (measured: 2048 x 4096 7.8 -> 6.6 us; at 32768 rows within
    // 1%, and slower with a residual)
    if (!ADD && !LN && sizeof(IO) == 2 && nt && nchunks > 256 && nchunks <= 512 &&
        rows * hidden * 4 <= (32ll << 20)) {
        wpr = 2;
        nch = 4;
    }
    // fp32 plain RMSNorm and LayerNorm over rows of 257-512 chunks in calls of
    // at most 32 MiB: one wave per row with 8 chunks per thread (measured:
    // 2048 x 2048 rmsnorm 7.6 -> 6.7 us, layernorm 8.6 -> 7.7 us; 3-6% slower
    // at 4096 rows, no better at 32768 rows or with a residual)
    if (!ADD && sizeof(IO) == 4 && nt && nchunks > 256 && nchunks <= 512 &&
        rows * hidden * 8 <= (32ll << 20)) {
        wpr = 1;
        nch = 8;
    }
    // plain LayerNorm over rows of 257-512 chunks: one wave per row with 8
    // chunks per thread (measured: 32768 x 3072 and x 4096 8% and 6% faster
    // than 2-chunk threads over 3-4 waves; with a residual, mixed)
    if (LN && !ADD && sizeof(IO) == 2 && nt && nchunks > 256 && nchunks <= 512) {
        wpr = 1;
        nch = 8;
    }
    if (nchunks <= 32) {
        int seg = 1;
        while (seg < nchunks) seg <<= 1;
        if (nt)
            launch_short<IO, ADD, LN, true>(Y, RO, X, R, G, B, rows, nchunks, seg, x_stride,
                                            y_stride, inv_h, eps, stream);
        else
            launch_short<IO, ADD, LN, false>(Y, RO, X, R, G, B, rows, nchunks, seg, x_stride,
                                             y_stride, inv_h, eps, stream);
        return hipGetLastError();
    }
#define NRS_SHAPE(W)                                                                             \
    (nt ? launch_shape<IO, ADD, LN, W, true>(Y, RO, X, R, G, B, rows, nchunks, nch, x_stride,      \
                                             y_stride, inv_h, eps, stream)                        \
        : launch_shape<IO, ADD, LN, W, false>(Y, RO, X, R, G, B, rows, nchunks, nch, x_stride,     \
                                              y_stride, inv_h, eps, stream))
    switch (wpr) {
        case 1: NRS_SHAPE(1); break;
        case 2: NRS_SHAPE(2); break;
        case 3: NRS_SHAPE(3); break;
        case 4: NRS_SHAPE(4); break;
        case 8: NRS_SHAPE(8); break;
        default: NRS_SHAPE(16); break;
    }
#undef NRS_SHAPE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(void *y, const void *x, const void *gamma, int64_t rows, int64_t hidden,
                          int64_t x_stride, int64_t y_stride, float eps, int dtype,
                          hipStream_t stream) {
    if (dtype == 0)
        return launch_norm_typed<float, false, false>(y, nullptr, x, nullptr, gamma, nullptr, rows,
                                                      hidden, x_stride, y_stride, eps, stream);
    return launch_norm_typed<__bf16, false, false>(y, nullptr, x, nullptr, gamma, nullptr, rows,
                                                   hidden, x_stride, y_stride, eps, stream);
}

hipError_t launch_add_rmsnorm(void *y, void *residual_out, const void *x, const void *residual,
                              const void *gamma, int64_t rows, int64_t hidden, float eps,
                              int dtype, hipStream_t stream) {
    if (dtype == 0)
        return launch_norm_typed<float, true, false>(y, residual_out, x, residual, gamma, nullptr,
                                                     rows, hidden, hidden, hidden, eps, stream);
    return launch_norm_typed<__bf16, true, false>(y, residual_out, x, residual, gamma, nullptr,
                                                  rows, hidden, hidden, hidden, eps, stream);
}

hipError_t launch_layernorm(void *y, const void *x, const void *gamma, const void *beta,
                            int64_t rows, int64_t hidden, int64_t x_stride, int64_t y_stride,
                            float eps, int dtype, hipStream_t stream) {
    if (dtype == 0)
        return launch_norm_typed<float, false, true>(y, nullptr, x, nullptr, gamma, beta, rows,
                                                     hidden, x_stride, y_stride, eps, stream);
    return launch_norm_typed<__bf16, false, true>(y, nullptr, x, nullptr, gamma, beta, rows,
                                                  hidden, x_stride, y_stride, eps, stream);
}

hipError_t launch_add_layernorm(void *y, void *residual_out, const void *x, const void *residual,
                                const void *gamma, const void *beta, int64_t rows, int64_t hidden,
                                float eps, int dtype, hipStream_t stream) {
    if (dtype == 0)
        return launch_norm_typed<float, true, true>(y, residual_out, x, residual, gamma, beta,
                                                    rows, hidden, hidden, hidden, eps, stream);
    return launch_norm_typed<__bf16, true, true>(y, residual_out, x, residual, gamma, beta, rows,
                                                 hidden, hidden, hidden, eps, stream);
}

}  // namespace nrs
