// Fused RMSNorm + Linear for gfx950.
//
// out[m][k] = sum_n (x[m][n] / rms_m) * w[k][n],  rms_m = sqrt(mean_n x[m][n]^2 + eps)
// ("Optimising autoregressive speech models", "Custom Triton kernels",
// kernel 1: the row is normalised and multiplied by the weight in one kernel,
// with no gain; a gain folds into the weight's columns).  w is [n_out][n_in]
// as torch's Linear stores it.
//
// Since 1/rms_m is one scalar per row, it commutes with the product: the
// kernel multiplies the stored x rows (bf16 or fp32, unrounded by any
// normalisation) by w on the matrix cores with fp32 accumulation, takes
// sum_n x^2 from the same operand registers, and scales each output row by
// rsqrt(sum_n x^2 / n_in + eps) at the end.  The normalised row never
// exists in memory.
//
// With few rows the product is bound by streaming w from HBM once (2 bytes
// per weight, 2 * rows flops per weight).  A workgroup owns 16 output
// columns; its S waves split the input dimension, each streaming 16-byte
// chunks of its 16 weight rows as the B operand of a 16x16 MFMA tile while
// x supplies the A operand (one tile per 16 rows, up to MT = 4 tiles sharing
// every weight load).  The waves' partial tiles and partial sums of squares
// meet once in LDS.  Weights are read with ordinary cached loads: measured on
// MI355X, nontemporal loads of this 16-rows-per-instruction pattern were up
// to 10% slower.
//
// With many rows (bf16) it is a GEMM bound by the matrix cores: 256 x 256
// output tiles of eight waves of 64 x 128 each when the problem has enough of
// them to fill the chip, 128 x 128 tiles of four 64 x 64 waves otherwise,
// operands staged through
// double-buffered, swizzled LDS 64 inputs at a time, and the row sums of squares taken
// from the A fragments as the tiles stream through.
#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One step of a 16x16 output tile over 4 * VEC inputs.  Lane (r, g) = (lane %
// 16, lane / 16) supplies a 16-byte chunk of A row r and of B column r, both
// starting at input g * VEC of the step; the tile's reduction runs over every
// (g, element) pair, so A and B need only agree on that order.
template <typename IO> struct mfma_step;

template <> struct mfma_step<__bf16> {
    // v_mfma_f32_16x16x32_bf16: A[r][8g + i] and B[8g + i][r], i < 8.
    __device__ static inline f32x4 run(const u32x4 &a, const u32x4 &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <> struct mfma_step<float> {
    // four v_mfma_f32_16x16x4_f32; instruction j reduces over element j of
    // every lane group's chunk
    __device__ static inline f32x4 run(const u32x4 &a, const u32x4 &b, f32x4 c) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, (unsigned)a[j]),
                                                     __builtin_bit_cast(float, (unsigned)b[j]), c,
                                                     0, 0, 0);
        return c;
    }
};

}  // namespace

// Output element D[row][col] of a 16x16 tile sits in lane col + 16 * (row / 4),
// element row % 4 (the MFMA accumulator layout).
template <typename IO, int MT, int S>
__global__ __launch_bounds__(64 * S) void rmsnorm_linear_kernel(
    IO *out, const IO *x, const IO *w, int32_t rows, int32_t n_in, int64_t n_out,
    int64_t x_stride, int64_t w_stride, int64_t out_stride, float inv_n, float eps) {
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    constexpr int SN = 4 * VEC;                       // inputs one wave consumes per step
    // steps whose loads are in flight together (measured: 4 beat 8 once the
    // grid no longer fits the chip in one round, and lose nothing below that)
    constexpr int U = MT == 1 ? 4 : 2;
    __shared__ f32x4 part[S][MT][64];
    __shared__ float sq_part[S][MT][16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int64_t col = (int64_t)blockIdx.x * 16 + r;   // weight row this lane streams
    const bool col_ok = col < n_out;
    const IO *wp = w + (col_ok ? col : 0) * w_stride + g * VEC;
    const IO *xp[MT];
    bool row_ok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int m = t * 16 + r;
        row_ok[t] = m < rows;
        xp[t] = x + (int64_t)(row_ok[t] ? m : 0) * x_stride + g * VEC;
    }

    // this wave's share of the input steps
    const int nsteps = (n_in + SN - 1) / SN;
    const int s0 = (int)((int64_t)wave * nsteps / S), s1 = (int)((int64_t)(wave + 1) * nsteps / S);

    f32x4 acc[MT];
    float ssq[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        ssq[t] = 0.0f;
    }
    const u32x4 zero = {0, 0, 0, 0};
    for (int s = s0; s < s1; s += U) {
        u32x4 b[U], a[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int off = (s + u) * SN;             // step start; this lane reads off + g*VEC
            const bool in = s + u < s1 && off + g * VEC < n_in;  // n_in is whole chunks
            b[u] = in && col_ok ? load16(wp + off) : zero;
#pragma unroll
            for (int t = 0; t < MT; ++t) a[u][t] = in && row_ok[t] ? load16(xp[t] + off) : zero;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                float v[VEC];
                T::unpack(a[u][t], v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) ssq[t] = __builtin_fmaf(v[i], v[i], ssq[t]);
                acc[t] = mfma_step<IO>::run(a[u][t], b[u], acc[t]);
            }
        }
    }

    // sum of squares of row t*16 + r: add the four lane groups, then the waves
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        ssq[t] += __shfl_xor(ssq[t], 16);
        ssq[t] += __shfl_xor(ssq[t], 32);
        part[wave][t][lane] = acc[t];
        if (g == 0) sq_part[wave][t][r] = ssq[t];
    }
    __syncthreads();

    // epilogue: add the waves' tiles, scale each row by its reciprocal rms
    const float *pf = reinterpret_cast<const float *>(&part[0][0][0]);
    for (int e = threadIdx.x; e < MT * 256; e += 64 * S) {
        const int t = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const int m = t * 16 + rr;
        const int64_t oc = (int64_t)blockIdx.x * 16 + cc;
        if (m >= rows || oc >= n_out) continue;
        const int src = (cc + 16 * (rr >> 2)) * 4 + (rr & 3);  // float index within a tile
        float sum = 0.0f, sq = 0.0f;
#pragma unroll
        for (int wv = 0; wv < S; ++wv) {
            sum += pf[(wv * MT + t) * 256 + src];
            sq += sq_part[wv][t][rr];
        }
        const float rs = rsqrtf(__builtin_fmaf(sq, inv_n, eps));
        out[(int64_t)m * out_stride + oc] = (IO)(sum * rs);
    }
}

// ---------------------------------------------------------------- many rows (GEMM)

constexpr int kGBK = 64;                // inputs per LDS stage: one 128-byte LDS row per tile row

// LDS element offset of 16-byte chunk c (0..7) of tile row `row`.  The chunk's
// slot is XOR-swizzled by bits 1..3 of the row, so both access patterns fill
// all 64 banks once per 16 lanes: a fragment load (16 consecutive rows, one
// chunk) and a staging store (two rows, all eight chunks).  Against 144-byte
// padded rows it removes the staging stores' bank conflicts and 18 KiB of
// LDS; measured speed is the same to within run-to-run spread.
__device__ inline int lds_at(int row, int c) { return row * kGBK + ((c ^ ((row >> 1) & 7)) << 3); }

// One workgroup of WM x WN waves computes a (16 WM TM) x (16 WN TN) tile of
// out; wave (wm, wn) owns TM x TN MFMA tiles of 16 x 16, so every 16-byte
// fragment read from LDS feeds TN (A) or TM (B) matrix-core steps.  Each
// stage every thread moves 16-byte chunks of x and w from HBM into registers
// while the waves multiply the stage already in LDS; then it writes them to
// the other LDS buffer and all meet at one barrier.
template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(64 * WM * WN) void rmsnorm_linear_gemm_kernel(
    __bf16 *out, const __bf16 *x, const __bf16 *w, int32_t rows, int32_t n_in, int64_t n_out,
    int64_t x_stride, int64_t w_stride, int64_t out_stride, float inv_n, float eps,
    uint32_t mblocks, uint32_t nblocks) {
    constexpr int kGBM = 16 * WM * TM, kGBN = 16 * WN * TN;
    constexpr int kGThreads = 64 * WM * WN;
    constexpr int kGTM = TM, kGTN = TN;
    static_assert(kGBM == kGBN, "one staging map serves both operands");
    constexpr int kGChunks = kGBM * kGBK / 8 / kGThreads;   // 16-byte chunks per thread per operand
    __shared__ __attribute__((aligned(16))) __bf16 As[2][kGBM * kGBK];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][kGBN * kGBK];
    __shared__ float row_ss[kGBM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wm = wave / WN, wn = wave % WN;
    // consecutive tiles of one XCD share a weight tile and walk down the rows
    const uint32_t b = xcd_contiguous(blockIdx.x, mblocks * nblocks);
    const int64_t m0 = (int64_t)(b % mblocks) * kGBM, c0 = (int64_t)(b / mblocks) * kGBN;
    const int nstages = (n_in + kGBK - 1) / kGBK;
    const u32x4 zero = {0, 0, 0, 0};

    // staging map: chunk q = tid + threads * j is row q / 8, inputs 8 (q % 8) .. + 7
    u32x4 ra[kGChunks], rb[kGChunks];
    auto gload = [&](int st) {
#pragma unroll
        for (int j = 0; j < kGChunks; ++j) {
            const int q = tid + kGThreads * j, row = q >> 3, n = st * kGBK + (q & 7) * 8;
            const bool nin = n < n_in;                      // n_in is whole chunks
            ra[j] = nin && m0 + row < rows ? load16(x + (m0 + row) * x_stride + n) : zero;
            rb[j] = nin && c0 + row < n_out ? load16(w + (c0 + row) * w_stride + n) : zero;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kGChunks; ++j) {
            const int q = tid + kGThreads * j, at = lds_at(q >> 3, q & 7);
            *reinterpret_cast<u32x4 *>(&As[buf][at]) = ra[j];
            *reinterpret_cast<u32x4 *>(&Bs[buf][at]) = rb[j];
        }
    };

    f32x4 acc[kGTM][kGTN];
    float ssq[kGTM];
#pragma unroll
    for (int i = 0; i < kGTM; ++i) {
        ssq[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < kGTN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    gload(0);
    lstore(0);
    __syncthreads();
    for (int st = 0; st < nstages; ++st) {
        const int buf = st & 1;
        if (st + 1 < nstages) gload(st + 1);
#pragma unroll
        for (int kk = 0; kk < kGBK; kk += 32) {
            u32x4 af[kGTM], bf[kGTN];
#pragma unroll
            for (int t = 0; t < kGTM; ++t)
                af[t] = *reinterpret_cast<const u32x4 *>(
                    &As[buf][lds_at(wm * 16 * kGTM + t * 16 + r, (kk >> 3) + g)]);
#pragma unroll
            for (int t = 0; t < kGTN; ++t)
                bf[t] = *reinterpret_cast<const u32x4 *>(
                    &Bs[buf][lds_at(wn * 16 * kGTN + t * 16 + r, (kk >> 3) + g)]);
            if (wn == 0) {   // one wave per row band takes the rows' sums of squares
#pragma unroll
                for (int t = 0; t < kGTM; ++t) {
                    float v[8];
                    io_traits<__bf16>::unpack(af[t], v);
#pragma unroll
                    for (int i = 0; i < 8; ++i) ssq[t] = __builtin_fmaf(v[i], v[i], ssq[t]);
                }
            }
#pragma unroll
            for (int tm = 0; tm < kGTM; ++tm)
#pragma unroll
                for (int tn = 0; tn < kGTN; ++tn)
                    acc[tm][tn] = mfma_step<__bf16>::run(af[tm], bf[tn], acc[tm][tn]);
        }
        if (st + 1 < nstages) lstore(buf ^ 1);
        __syncthreads();
    }

    if (wn == 0) {
#pragma unroll
        for (int t = 0; t < kGTM; ++t) {
            float s2 = ssq[t];
            s2 += __shfl_xor(s2, 16);
            s2 += __shfl_xor(s2, 32);
            if (g == 0) row_ss[wm * 16 * kGTM + t * 16 + r] = s2;
        }
    }
    __syncthreads();
#pragma unroll
    for (int tm = 0; tm < kGTM; ++tm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wm * 16 * kGTM + tm * 16 + 4 * g + i;   // accumulator layout
            const int64_t gm = m0 + row;
            if (gm >= rows) continue;
            const float rs = rsqrtf(__builtin_fmaf(row_ss[row], inv_n, eps));
#pragma unroll
            for (int tn = 0; tn < kGTN; ++tn) {
                const int64_t gc = c0 + wn * 16 * kGTN + tn * 16 + r;
                if (gc < n_out) out[gm * out_stride + gc] = (__bf16)(acc[tm][tn][i] * rs);
            }
        }
    }
}

namespace {

constexpr int kSplit = 8;      // waves per workgroup (splitting the input dimension)
constexpr int kMaxTileRows = 64;

template <typename IO>
void launch_chunk(IO *out, const IO *x, const IO *w, int32_t rows, int32_t n_in, int64_t n_out,
                  int64_t xs, int64_t ws, int64_t os, float inv_n, float eps, hipStream_t stream) {
    const dim3 grid((unsigned)((n_out + 15) / 16)), block(64 * kSplit);
#define NRS_LIN(MT)                                                                          \
    hipLaunchKernelGGL((rmsnorm_linear_kernel<IO, MT, kSplit>), grid, block, 0, stream, out,     \
                       x, w, rows, n_in, n_out, xs, ws, os, inv_n, eps)
    if (rows <= 16) NRS_LIN(1);
    else if (rows <= 32) NRS_LIN(2);
    else NRS_LIN(4);
#undef NRS_LIN
}

template <typename IO>
hipError_t launch_typed(void *out, const void *x, const void *w, int64_t rows, int64_t n_in,
                        int64_t n_out, int64_t xs, int64_t ws, int64_t os, float eps,
                        hipStream_t stream) {
    const float inv_n = (float)(1.0 / (double)n_in);
    if (sizeof(IO) == 2 && rows > kMaxTileRows) {
        // 256 x 256 tiles read half the operand bytes per flop of 128 x 128
        // ones but need enough of them to give every CU one
        const int64_t big = ((rows + 255) / 256) * ((n_out + 255) / 256);
        const int tile = big >= 256 ? 256 : 128;
        const uint32_t nblocks = (uint32_t)((n_out + tile - 1) / tile);
        // rows per launch: whole tiles, and a grid below 2^31 workgroups
        const int64_t max_mblocks = (((int64_t)1 << 31) - 1) / nblocks;
        for (int64_t r0 = 0; r0 < rows; r0 += max_mblocks * tile) {
            const int64_t rr = rows - r0 < max_mblocks * tile ? rows - r0 : max_mblocks * tile;
            const uint32_t mblocks = (uint32_t)((rr + tile - 1) / tile);
            __bf16 *o = (__bf16 *)out + r0 * os;
            const __bf16 *xx = (const __bf16 *)x + r0 * xs;
            if (tile == 256)
                hipLaunchKernelGGL((rmsnorm_linear_gemm_kernel<4, 2, 4, 8>),
                                   dim3(mblocks * nblocks), dim3(512), 0, stream, o, xx,
                                   (const __bf16 *)w, (int32_t)rr, (int32_t)n_in, n_out, xs, ws,
                                   os, inv_n, eps, mblocks, nblocks);
            else
                hipLaunchKernelGGL((rmsnorm_linear_gemm_kernel<2, 2, 4, 4>),
                                   dim3(mblocks * nblocks), dim3(256), 0, stream, o, xx,
                                   (const __bf16 *)w, (int32_t)rr, (int32_t)n_in, n_out, xs, ws,
                                   os, inv_n, eps, mblocks, nblocks);
        }
        return hipGetLastError();
    }
    // fp32 rows beyond one launch's 64 are taken 64 at a time (each pass streams w again)
    for (int64_t m0 = 0; m0 < rows; m0 += kMaxTileRows) {
        const int32_t mr = (int32_t)(rows - m0 < kMaxTileRows ? rows - m0 : kMaxTileRows);
        IO *o = (IO *)out + m0 * os;
        const IO *xx = (const IO *)x + m0 * xs;
        launch_chunk<IO>(o, xx, (const IO *)w, mr, (int32_t)n_in, n_out, xs, ws, os, inv_n, eps,
                         stream);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_linear(void *out, const void *x, const void *w, int64_t rows,
                                 int64_t n_in, int64_t n_out, int64_t x_stride, int64_t w_stride,
                                 int64_t out_stride, float eps, int dtype, hipStream_t stream) {
    if (dtype == 0)
        return launch_typed<float>(out, x, w, rows, n_in, n_out, x_stride, w_stride, out_stride,
                                   eps, stream);
    return launch_typed<__bf16>(out, x, w, rows, n_in, n_out, x_stride, w_stride, out_stride, eps,
                                stream);
}

}  // namespace nrs
