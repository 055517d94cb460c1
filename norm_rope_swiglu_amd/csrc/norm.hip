// RMSNorm and fused residual-add + RMSNorm for gfx950.
//
// RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps), the mean over the hidden
// axis ("Optimising autoregressive speech models", section 09 "LayerNorm ->
// RMSNorm": "What it is" and "How to swap").  The fused variant is the
// "Norm+Residual" op of the qwen3-tts-triton post (de.news.hada.io topic
// 27742, part 3): h = x + residual is rounded to the storage type, written
// as residual_out, and normalised in the same pass.
//
// Layout: one wave64 owns one row.  Lane l holds chunks l, l+64, l+128, ...
// of 16 bytes each, so every load instruction of a wave reads 1 KiB of
// contiguous HBM; the whole row stays in VGPRs between the read, the
// reduction and the write, so each input byte is read once and each output
// byte written once.  The sum of squares is reduced with DPP row operations
// plus four readlanes (no LDS, no barrier).  gamma is read once per wave and
// kept in registers while the wave walks its rows; the next row's loads are
// issued before the current row is reduced and written.
//
// Rows wider than 16 chunks per lane (more than 8192 bf16 / 4096 fp32
// elements) go to a block-per-row kernel: each of 512 threads holds up to 16
// chunks and the per-wave partial sums meet in 32 bytes of LDS.
#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

template <typename IO, int NCH, bool ADD>
__global__ __launch_bounds__(256) void norm_wave_kernel(
    IO *y, IO *res_out, const IO *x, const IO *res, const IO *gamma, int64_t rows,
    int32_t nchunks, int64_t x_stride, int64_t y_stride, float inv_h, float eps) {
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= rows) return;

    u32x4 graw[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int idx = lane + 64 * c;
        graw[c] = idx < nchunks ? load16(gamma + (int64_t)idx * VEC) : u32x4{0, 0, 0, 0};
    }

    u32x4 xa[NCH], ra[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int idx = lane + 64 * c;
        xa[c] = u32x4{0, 0, 0, 0};
        ra[c] = u32x4{0, 0, 0, 0};
        if (idx < nchunks) {
            xa[c] = load16_stream(x + row * x_stride + (int64_t)idx * VEC);
            if (ADD) ra[c] = load16_stream(res + row * x_stride + (int64_t)idx * VEC);
        }
    }

    while (true) {
        const int64_t next = row + nwaves;
        u32x4 xb[NCH], rb[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int idx = lane + 64 * c;
            xb[c] = u32x4{0, 0, 0, 0};
            rb[c] = u32x4{0, 0, 0, 0};
            if (next < rows && idx < nchunks) {
                xb[c] = load16_stream(x + next * x_stride + (int64_t)idx * VEC);
                if (ADD) rb[c] = load16_stream(res + next * x_stride + (int64_t)idx * VEC);
            }
        }

        float v[NCH][VEC];
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            T::unpack(xa[c], v[c]);
            if (ADD) {
                float r[VEC];
                T::unpack(ra[c], r);
#pragma unroll
                for (int i = 0; i < VEC; ++i) v[c][i] = T::round_trip(v[c][i] + r[i]);
            }
#pragma unroll
            for (int i = 0; i < VEC; ++i) ss = __builtin_fmaf(v[c][i], v[c][i], ss);
        }
        if (ADD) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int idx = lane + 64 * c;
                if (idx < nchunks)
                    store16_stream(res_out + row * y_stride + (int64_t)idx * VEC, T::pack(v[c]));
            }
        }
        ss = wave_sum(ss);
        const float rs = rsqrtf(__builtin_fmaf(ss, inv_h, eps));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int idx = lane + 64 * c;
            float g[VEC], o[VEC];
            T::unpack(graw[c], g);
#pragma unroll
            for (int i = 0; i < VEC; ++i) o[i] = (v[c][i] * rs) * g[i];
            if (idx < nchunks) store16_stream(y + row * y_stride + (int64_t)idx * VEC, T::pack(o));
        }

        if (next >= rows) break;
        row = next;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            xa[c] = xb[c];
            ra[c] = rb[c];
        }
    }
}

constexpr int BLOCK_ROW_THREADS = 512;

template <typename IO, int NCH, bool ADD>
__global__ __launch_bounds__(BLOCK_ROW_THREADS) void norm_block_kernel(
    IO *y, IO *res_out, const IO *x, const IO *res, const IO *gamma, int64_t rows,
    int32_t nchunks, int64_t x_stride, int64_t y_stride, float inv_h, float eps) {
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    constexpr int NW = BLOCK_ROW_THREADS / 64;
    __shared__ float partial[NW];
    const int tid = threadIdx.x;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        float v[NCH][VEC];
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int idx = tid + BLOCK_ROW_THREADS * c;
            u32x4 xr = u32x4{0, 0, 0, 0}, rr = u32x4{0, 0, 0, 0};
            if (idx < nchunks) {
                xr = load16_stream(x + row * x_stride + (int64_t)idx * VEC);
                if (ADD) rr = load16_stream(res + row * x_stride + (int64_t)idx * VEC);
            }
            T::unpack(xr, v[c]);
            if (ADD) {
                float r[VEC];
                T::unpack(rr, r);
#pragma unroll
                for (int i = 0; i < VEC; ++i) v[c][i] = T::round_trip(v[c][i] + r[i]);
                if (idx < nchunks)
                    store16_stream(res_out + row * y_stride + (int64_t)idx * VEC, T::pack(v[c]));
            }
#pragma unroll
            for (int i = 0; i < VEC; ++i) ss = __builtin_fmaf(v[c][i], v[c][i], ss);
        }
        ss = wave_sum(ss);
        if ((tid & 63) == 0) partial[tid >> 6] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += partial[w];
        __syncthreads();  // partial[] is rewritten by the next row
        const float rs = rsqrtf(__builtin_fmaf(tot, inv_h, eps));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int idx = tid + BLOCK_ROW_THREADS * c;
            if (idx < nchunks) {
                float g[VEC], o[VEC];
                T::unpack(load16(gamma + (int64_t)idx * VEC), g);
#pragma unroll
                for (int i = 0; i < VEC; ++i) o[i] = (v[c][i] * rs) * g[i];
                store16_stream(y + row * y_stride + (int64_t)idx * VEC, T::pack(o));
            }
        }
    }
}

namespace {

template <typename IO, bool ADD>
hipError_t launch_norm_typed(void *y, void *res_out, const void *x, const void *res,
                             const void *gamma, int64_t rows, int64_t hidden, int64_t x_stride,
                             int64_t y_stride, float eps, hipStream_t stream) {
    constexpr int VEC = io_traits<IO>::VEC;
    const int32_t nchunks = (int32_t)(hidden / VEC);
    const int per_lane = (nchunks + 63) / 64;
    const float inv_h = (float)(1.0 / (double)hidden);
    IO *Y = (IO *)y, *RO = (IO *)res_out;
    const IO *X = (const IO *)x, *R = (const IO *)res, *G = (const IO *)gamma;

    if (per_lane <= 16) {
        const int64_t waves_per_block = 4;
        int64_t blocks = (rows + waves_per_block - 1) / waves_per_block;
        if (blocks > kMaxResidentBlocks) blocks = kMaxResidentBlocks;
        const dim3 grid((unsigned)blocks), block(256);
#define NRS_NORM_WAVE(N)                                                                        \
    hipLaunchKernelGGL((norm_wave_kernel<IO, N, ADD>), grid, block, 0, stream, Y, RO, X, R, G, \
                       rows, nchunks, x_stride, y_stride, inv_h, eps)
        if (per_lane <= 1) NRS_NORM_WAVE(1);
        else if (per_lane <= 2) NRS_NORM_WAVE(2);
        else if (per_lane <= 3) NRS_NORM_WAVE(3);
        else if (per_lane <= 4) NRS_NORM_WAVE(4);
        else if (per_lane <= 6) NRS_NORM_WAVE(6);
        else if (per_lane <= 8) NRS_NORM_WAVE(8);
        else if (per_lane <= 12) NRS_NORM_WAVE(12);
        else NRS_NORM_WAVE(16);
#undef NRS_NORM_WAVE
    } else {
        const int per_thread = (nchunks + BLOCK_ROW_THREADS - 1) / BLOCK_ROW_THREADS;
        int64_t blocks = rows < kMaxResidentBlocks ? rows : kMaxResidentBlocks;
        const dim3 grid((unsigned)blocks), block(BLOCK_ROW_THREADS);
#define NRS_NORM_BLOCK(N)                                                                        \
    hipLaunchKernelGGL((norm_block_kernel<IO, N, ADD>), grid, block, 0, stream, Y, RO, X, R, G, \
                       rows, nchunks, x_stride, y_stride, inv_h, eps)
        if (per_thread <= 4) NRS_NORM_BLOCK(4);
        else if (per_thread <= 8) NRS_NORM_BLOCK(8);
        else NRS_NORM_BLOCK(16);
#undef NRS_NORM_BLOCK
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(void *y, const void *x, const void *gamma, int64_t rows, int64_t hidden,
                          int64_t x_stride, int64_t y_stride, float eps, int dtype,
                          hipStream_t stream) {
    if (dtype == 0)
        return launch_norm_typed<float, false>(y, nullptr, x, nullptr, gamma, rows, hidden,
                                               x_stride, y_stride, eps, stream);
    return launch_norm_typed<__bf16, false>(y, nullptr, x, nullptr, gamma, rows, hidden, x_stride,
                                            y_stride, eps, stream);
}

hipError_t launch_add_rmsnorm(void *y, void *residual_out, const void *x, const void *residual,
                              const void *gamma, int64_t rows, int64_t hidden, float eps,
                              int dtype, hipStream_t stream) {
    if (dtype == 0)
        return launch_norm_typed<float, true>(y, residual_out, x, residual, gamma, rows, hidden,
                                              hidden, hidden, eps, stream);
    return launch_norm_typed<__bf16, true>(y, residual_out, x, residual, gamma, rows, hidden,
                                           hidden, hidden, eps, stream);
}

}  // namespace nrs
