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
// per weight, 2 * rows flops per weight).  Up to 8 bf16 rows take plain dot
// products, one weight row per wave at a time in whole lines (the GEMV
// kernel below).  Otherwise a workgroup owns 16 output
// columns; its S waves split the input dimension, each streaming 16-byte
// chunks of its 16 weight rows as the B operand of a 16x16 MFMA tile while
// x supplies the A operand (one tile per 16 rows, up to MT = 4 tiles sharing
// every weight load).  The waves' partial tiles and partial sums of squares
// meet once in LDS.  Weights are read with ordinary cached loads: measured on
// MI355X, nontemporal loads of this 16-rows-per-instruction pattern were up
// to 10% slower.
//
// With many rows (bf16) it is a GEMM bound by the matrix cores: 256 x 256
// output tiles when the problem has enough of them to fill the chip, else
// 256 x 128; eight waves per tile in two groups that take turns between
// multiplying and reading LDS; operands loaded straight into a three-slot LDS
// ring; the row sums of squares taken from the A fragments as the tiles
// stream through (details above the kernel).
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// ---------------------------------------------------------------- decode rows (bf16 GEMV)
//
// Up to 8 bf16 rows whose x fits 32 KiB: plain dot products instead of
// matrix-core tiles.  A 16x16 tile's B operand makes every load instruction
// read 64 bytes from each of 16 weight rows, half of each 128-byte line;
// here a wave owns kGemvRowsPerWave weight rows and lane l takes their
// 16-byte chunks l, l + 64, ..., so every load instruction reads 1 KiB of
// one weight row, whole lines, and the loads of all the wave's rows are in
// flight together.  The block stages the x rows in LDS once (their sums of
// squares come from that copy); the products are v_dot2_f32_bf16 on bf16
// pairs accumulating in fp32, and each lane's partial sums are added across
// the wave.  Measured on MI355X (graph of 28 calls with distinct weights,
// 5 x 2048): 12288 outputs 13.8 -> 11.9 us against the tile kernel, 4096
// outputs 6.6 -> 6.2 us; the weights are read nontemporal (this pattern ran
// 5-11% faster so, unlike the tiles' 16-row one), and two rows per wave beat
// one and four.
//
// A lane holds CPL chunks of each of its weight rows per pass; rows wider
// than 64 * CPL chunks (CPL = 8: more than 4096 inputs) take NP passes, the
// next pass's weight loads issued before this pass's products.
constexpr int kGemvRowsPerWave = 2;
constexpr int kGemvWaves = 4;           // waves per block (kGemvWavesWide for wide outputs)
// Every block stages all x rows in LDS, so the grid re-reads x from L2 once
// per block.  Wide outputs take blocks of 8 waves, half the blocks: measured
// on MI355X (graph of 28 calls with distinct weights) 5 x 2048 -> 12288
// 12.25 -> 11.9 us, while 5 x 2048 -> 4096 (one block per CU with 8 waves)
// went 6.2 -> 6.3 us and keeps 4.
constexpr int kGemvWavesWide = 8;
constexpr int64_t kGemvWideOut = 8192;   // outputs from which blocks are wide
constexpr int kGemvMaxXChunks = 2048;   // rows x chunks of x staged in LDS: 32 KiB
constexpr int kGemvMaxPasses = 4;       // 64 lanes x 8 chunks x 4 passes = kGemvMaxXChunks

template <int M, int CPL, int NP, int W>
__global__ __launch_bounds__(64 * W) void rmsnorm_gemv_kernel(
    __bf16 *out, const __bf16 *x, const __bf16 *w, int32_t nchunks, int64_t n_out,
    int64_t x_stride, int64_t w_stride, int64_t out_stride, fastdiv div_nchunks, float inv_n,
    float eps) {
    constexpr int RPW = kGemvRowsPerWave;
    constexpr int NTH = 64 * W;
    // x chunks each thread stages: M * nchunks <= M * 64 * CPL * NP <= NTH * XPT
    constexpr int XPT = (M * CPL * NP + W - 1) / W;
    static_assert(NP == 1 || CPL == 8, "only 8-chunk lanes take several passes");
    static_assert(NP <= kGemvMaxPasses, "a row fits kGemvMaxXChunks");
    extern __shared__ u32x4 xs[];            // [M][nchunks]
    __shared__ float rs[M];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const u32x4 zero = {0, 0, 0, 0};
    const int nx = M * nchunks;

    // 1. loads, all branch-free (indices clamped, the extra lanes' data
    //    dropped below): this thread's x chunks first, then the wave's weight
    //    chunks of the first pass, so the x stores to LDS wait for x alone
    u32x4 xv[XPT];
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
        const int e = min((int)threadIdx.x + NTH * k, nx - 1);
        const int m = (int)div((uint32_t)e, div_nchunks), c = e - m * nchunks;
        xv[k] = load16(x + (int64_t)m * x_stride + c * 8);
    }
    const int64_t row0 = ((int64_t)blockIdx.x * W + wave) * RPW;   // the wave's first weight row
    u32x4 wv[NP > 1 ? 2 : 1][RPW][CPL];   // this pass's chunks and the next pass's loads
    auto load_w = [&](int p, int buf) {
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int64_t n = min(row0 + j, n_out - 1);
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                wv[buf][j][i] = load16_stream(
                    w + n * w_stride + (int64_t)min(lane + 64 * (i + CPL * p), nchunks - 1) * 8);
        }
    };
    load_w(0, 0);
    // (threads past the end store the last chunk again, the value it holds:
    // no branch, so no wait beyond x's own loads)
#pragma unroll
    for (int k = 0; k < XPT; ++k) xs[min((int)threadIdx.x + NTH * k, nx - 1)] = xv[k];
    __syncthreads();

    // 2. each row's 1 / rms from the staged copy (wave w takes rows w, w + W, ...)
#pragma unroll
    for (int m = wave; m < M; m += W) {
        float sq = 0.0f;
        for (int c = lane; c < nchunks; c += 64) {
            const u32x4 v = xs[m * nchunks + c];
#pragma unroll
            for (int p = 0; p < 4; ++p)
                sq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (unsigned)v[p]),
                                                     __builtin_bit_cast(bf16x2, (unsigned)v[p]), sq, false);
        }
        sq = wave_sum(sq);
        if (lane == 0) rs[m] = rsqrtf(__builtin_fmaf(sq, inv_n, eps));
    }

    // 3. per pass: the next pass's weight loads, then the products (chunk c
    //    of every weight row meets chunk c of every x row); then the wave
    //    sums, and lane m stores row m's output
    float acc[RPW][M];
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int buf = p & 1;
        if (p + 1 < NP) load_w(p + 1, buf ^ 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * (i + CPL * p);
            const bool live = c < nchunks;
            const int cc = live ? c : nchunks - 1;
#pragma unroll
            for (int j = 0; j < RPW; ++j)
                if (!live) wv[buf][j][i] = zero;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4 xa = xs[m * nchunks + cc];
#pragma unroll
                for (int j = 0; j < RPW; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[j][m] = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2, (unsigned)xa[q]),
                            __builtin_bit_cast(bf16x2, (unsigned)wv[buf][j][i][q]), acc[j][m], false);
            }
        }
    }
    __syncthreads();   // rs is written (uniform: every thread takes it)
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        const int64_t n = row0 + j;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float sum = wave_sum(acc[j][m]);
            if (lane == m && n < n_out) out[(int64_t)m * out_stride + n] = (__bf16)(sum * rs[m]);
        }
    }
}

// ---------------------------------------------------------------- many rows (GEMM)
//
// A 256-row tile of x against BN weight rows, BK inputs per stage, eight
// waves in two groups of four.  Group h owns tile rows [128 h, 128 h + 128);
// its waves split them 2 x 2, so each wave holds a 64 x BN/2 block of 16 x 16
// accumulators.  Each SIMD runs one wave of each group, and the groups take
// turns: while one multiplies the stage it holds in registers, the other
// reads its next stage's fragments from LDS and issues the loads of a later
// stage, and one workgroup barrier separates the turns.  Measured on MI355X,
// a wave reads LDS at ~40 B/clk on its own and the CU at ~240 B/clk with
// eight waves, while 16-byte LDS stores peak at ~78 B/clk.  So the operands
// reach LDS by buffer loads that write LDS directly (no register staging and
// no LDS store instructions), into a ring of three stage slots held as
// separate arrays.  The compiler then orders each fragment read only after
// the loads into its own slot.

// Where a tile row's 16-byte chunks sit in a stage slot whose rows are CPR
// chunks long.  A fragment read takes one chunk from each of 16 consecutive
// tile rows (g = lane / 16 picks the chunk); a 1 KiB load fills 1 KiB of LDS
// in lane order.  Both must spread over every bank.  128-byte rows (CPR 8)
// keep the tile's row order and store chunk c at slot c ^ ((row / 2) % 8).
// With 64-byte rows (CPR 4) an in-row swizzle alone left every fragment read
// two-way conflicted on MI355X (SQ_LDS_BANK_CONFLICT: four cycles on each
// ds_read_b128, against none with 128-byte rows): within an aligned block of
// 16 rows, the LDS row of tile row r is gemm_pos(r), which gives the rows that
// a read serves together different 64-byte quarters of a 256-byte bank line,
// and chunk c sits at slot c ^ ((r / 2) % 4).
template <int CPR> __device__ inline int gemm_swizzle(int row) {
    if constexpr (CPR == 8) return (row >> 1) & 7;
    else return (row >> 1) & 3;
}
// LDS row, within its aligned block of 16, of tile row r (0..15), and back
template <int CPR> __device__ inline int gemm_pos(int r) {
    if constexpr (CPR == 8) return r;
    else return (r & 1) | (((r >> 3) & 1) << 1) | (((r >> 1) & 3) << 2);
}
template <int CPR> __device__ inline int gemm_row_of(int p) {
    if constexpr (CPR == 8) return p;
    else return (p & 1) | (((p >> 2) & 3) << 1) | (((p >> 1) & 1) << 3);
}
template <int CPR> __device__ inline int gemm_at(int row, int c) {
    return ((row & ~15) + gemm_pos<CPR>(row & 15)) * CPR * 8 + ((c ^ gemm_swizzle<CPR>(row)) << 3);
}

// s_waitcnt with vmcnt = N and the other counters at their maximum
template <int N> __device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ inline void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// a workgroup barrier that waits for nothing itself (the waits before it are
// explicit), and that the compiler does not move memory accesses across
__device__ inline void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// one 16-byte load per lane from buffer r at voff + soff, lane l writing
// bytes [16 l, 16 l + 16) after lds (wave-uniform)
__device__ inline void load_to_lds(__amdgpu_buffer_rsrc_t r, __bf16 *lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
}

constexpr int kGemmRows = 256;           // x rows per tile
constexpr int kGemmGroupRows = 4;        // row tiles per group of the tile order

template <int BN, int BK>
__global__ __launch_bounds__(512, 1) void rmsnorm_linear_gemm_kernel(
    __bf16 *out, const __bf16 *x, const __bf16 *w, int32_t rows, int32_t n_in, int64_t n_out,
    int64_t x_stride, int64_t w_stride, int64_t out_stride, float inv_n, float eps,
    uint32_t mblocks, uint32_t nblocks) {
    constexpr int BM = kGemmRows, TM = 4, TN = BN / 32, KS = BK / 32, CPR = BK / 8;
    constexpr int RPK = 64 / CPR;                         // tile rows per 1 KiB load
    constexpr int NA = (BM / 2) / RPK / 4, NB = (BN / 2) / RPK / 4;   // loads per wave per stage
    constexpr int NL = NA + NB;
    static_assert(NA * RPK * 4 == BM / 2 && NB * RPK * 4 == BN / 2, "loads split evenly");
    static_assert(CPR == 8 || RPK == 16, "64-byte rows: loads cover whole 16-row blocks");
    constexpr int D = 2;                                  // stages in flight ahead of the one read
    __shared__ __attribute__((aligned(16))) __bf16 A0[BM * BK], A1[BM * BK], A2[BM * BK];
    __shared__ __attribute__((aligned(16))) __bf16 B0[BN * BK], B1[BN * BK], B2[BN * BK];
    __shared__ float row_ss[BM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
    const int grp = wave >> 2, wig = wave & 3, wm = wig >> 1, wn = wig & 1;
    const int r = lane & 15, g = lane >> 4;
    // each XCD runs consecutive tiles together; they are taken in groups of
    // kGemmGroupRows row tiles across all column tiles, so the tiles in
    // flight on one XCD share row and column tiles in its L2
    constexpr uint32_t GM = kGemmGroupRows;
    const uint32_t b = xcd_contiguous(blockIdx.x, mblocks * nblocks);
    const uint32_t gid = b / (GM * nblocks), first = gid * GM;
    const uint32_t gsz = mblocks - first < GM ? mblocks - first : GM;
    const uint32_t within = b - gid * GM * nblocks;
    const int64_t m0 = (int64_t)(first + within % gsz) * BM, c0 = (int64_t)(within / gsz) * BN;
    const int nst = (n_in + BK - 1) / BK;

    // buffers based at the tile's first row and covering only its rows inside
    // the matrix, so loads of rows past the end read zeros
    const int a_rows = (int)(rows - m0 < BM ? rows - m0 : BM);
    const int b_rows = (int)(n_out - c0 < BN ? n_out - c0 : BN);
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + m0 * x_stride), 0, (int)((int64_t)a_rows * x_stride * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w + c0 * w_stride), 0, (int)((int64_t)b_rows * w_stride * 2), 0x00020000);
    constexpr uint32_t kOut = 0x80000000u;    // beyond any buffer here: reads as zeros

    // this wave's loads.  Load j covers RPK tile rows; lane l fills LDS slot l
    // of that 1 KiB block, i.e. LDS row base + l / CPR, stored chunk l % CPR,
    // which holds tile row lr = base + gemm_row_of(l / CPR) (a load starts on
    // a 16-row boundary, or covers 8 rows of 128 bytes) and its input chunk
    // (l % CPR) ^ swizzle(lr).
    uint32_t offa[NA], offb[NB];
    int cla[NA], clb[NB];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int lr = grp * (BM / 2) + (wig * NA + j) * RPK + gemm_row_of<CPR>(lane / CPR);
        cla[j] = ((lane % CPR) ^ gemm_swizzle<CPR>(lr)) * 8;
        offa[j] = (uint32_t)(lr * (int)x_stride + cla[j]) * 2u;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int lr = grp * (BN / 2) + (wig * NB + j) * RPK + gemm_row_of<CPR>(lane / CPR);
        clb[j] = ((lane % CPR) ^ gemm_swizzle<CPR>(lr)) * 8;
        offb[j] = (uint32_t)(lr * (int)w_stride + clb[j]) * 2u;
    }
    // stage st of this wave's share into a slot; only the last stage can
    // reach past n_in, and its lanes beyond it read zeros
    auto issue = [&](auto steady, int st, auto &As, auto &Bs) {
        const int k0 = st * BK;
        const bool tail = !decltype(steady)::value && k0 + BK > n_in;
#pragma unroll
        for (int j = 0; j < NA; ++j)
            load_to_lds(ar, &As[(grp * (BM / 2) + (wig * NA + j) * RPK) * BK],
                        tail && k0 + cla[j] >= n_in ? kOut : offa[j], k0 * 2);
#pragma unroll
        for (int j = 0; j < NB; ++j)
            load_to_lds(br, &Bs[(grp * (BN / 2) + (wig * NB + j) * RPK) * BK],
                        tail && k0 + clb[j] >= n_in ? kOut : offb[j], k0 * 2);
    };

    f32x4 acc[TM][TN];
    float ssq0 = 0.0f, ssq1 = 0.0f;     // sums of squares of rows t = 2 wn, 2 wn + 1
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int arow = grp * (BM / 2) + wm * 64 + r, brow = wn * (BN / 2) + r;

    // one stage: the fragment turn, a barrier, the multiply turn, a barrier
    auto body = [&](auto steady, int st, const auto &As, const auto &Bs, auto &An, auto &Bn) {
        // stage st + D into the slot stage st - 1 used, which every wave has
        // finished reading (its reads completed before the last barrier).
        // Issued before this stage's fragment reads, which read another slot
        // (measured: 2-7% faster than issuing after them).
        const bool more = decltype(steady)::value || st + D < nst;
        if (more) issue(steady, st + D, An, Bn);
        u32x4 af[KS][TM], bf[KS][TN];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
                af[ks][t] = *reinterpret_cast<const u32x4 *>(&As[gemm_at<CPR>(arow + t * 16, ks * 4 + g)]);
#pragma unroll
            for (int t = 0; t < TN; ++t)
                bf[ks][t] = *reinterpret_cast<const u32x4 *>(&Bs[gemm_at<CPR>(brow + t * 16, ks * 4 + g)]);
        }
        wait_lgkmcnt0();
        // this wave's share of stage st + 1 must have landed before the
        // barrier after which the other group reads it
        if (more) wait_vmcnt<(D - 1) * NL>();
        else wait_vmcnt<0>();
        bare_barrier();
        // the fragments pass through an empty asm so that no multiply is
        // hoisted above the barrier
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(af[ks][t]));
#pragma unroll
            for (int t = 0; t < TN; ++t) asm volatile("" : "+v"(bf[ks][t]));
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            {   // sums of squares: the two waves of a row band take two A fragments each
                const u32x4 a0 = wn ? af[ks][2] : af[ks][0], a1 = wn ? af[ks][3] : af[ks][1];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ssq0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (unsigned)a0[i]),
                                                           __builtin_bit_cast(bf16x2, (unsigned)a0[i]), ssq0, false);
                    ssq1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (unsigned)a1[i]),
                                                           __builtin_bit_cast(bf16x2, (unsigned)a1[i]), ssq1, false);
                }
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = mfma_step<__bf16>::run(af[ks][tm], bf[ks][tn], acc[tm][tn]);
        }
        __builtin_amdgcn_sched_barrier(0);
        bare_barrier();
    };

    // prologue: stages 0 and 1 in flight, stage 0 landed and visible; then
    // group 1 passes one extra barrier so the groups run a turn apart
    issue(std::false_type{}, 0, A0, B0);
    if (nst > 1) issue(std::false_type{}, 1, A1, B1);
    if (nst > 1) wait_vmcnt<NL>();
    else wait_vmcnt<0>();
    bare_barrier();
    if (grp) bare_barrier();
    // steady state: every stage loads the one D ahead, with no branches
    // between the ring's slots (a branch there would cost the compiler its
    // per-slot ordering of loads and reads); every stage it loads lies wholly
    // inside n_in
    const int nfull = n_in / BK;
    int st = 0;
    for (; st + 3 + D <= nfull; st += 3) {
        body(std::true_type{}, st, A0, B0, A2, B2);
        body(std::true_type{}, st + 1, A1, B1, A0, B0);
        body(std::true_type{}, st + 2, A2, B2, A1, B1);
    }
    for (; st < nst; st += 3) {
        body(std::false_type{}, st, A0, B0, A2, B2);
        if (st + 1 < nst) body(std::false_type{}, st + 1, A1, B1, A0, B0);
        if (st + 2 < nst) body(std::false_type{}, st + 2, A2, B2, A1, B1);
    }
    if (!grp) bare_barrier();    // both groups have now passed the same number

    // sums of squares over the four lane groups, then one row each in LDS
    ssq0 += __shfl_xor(ssq0, 16);
    ssq0 += __shfl_xor(ssq0, 32);
    ssq1 += __shfl_xor(ssq1, 16);
    ssq1 += __shfl_xor(ssq1, 32);
    if (g == 0) {
        row_ss[arow + 2 * wn * 16] = ssq0;
        row_ss[arow + (2 * wn + 1) * 16] = ssq1;
    }
    __syncthreads();
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = grp * (BM / 2) + wm * 64 + tm * 16 + 4 * g + i;   // accumulator layout
            const int64_t gm = m0 + row;
            if (gm >= rows) continue;
            const float rs = rsqrtf(__builtin_fmaf(row_ss[row], inv_n, eps));
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int64_t gc = c0 + wn * (BN / 2) + tn * 16 + r;
                if (gc < n_out) out[gm * out_stride + gc] = (__bf16)(acc[tm][tn][i] * rs);
            }
        }
    }
}

namespace {

constexpr int kSplit = 8;      // waves per workgroup (splitting the input dimension)
constexpr int kMaxTileRows = 64;
// the tiled path addresses a tile's rows with 32-bit byte offsets
constexpr int64_t kMaxGemmStride = (int64_t)1 << 22;

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

// bf16, many rows: 256 x 256 tiles (32 inputs per stage) when they give every
// CU one, else 256 x 128 (64 inputs per stage)
hipError_t launch_gemm(void *out, const void *x, const void *w, int64_t rows, int64_t n_in,
                       int64_t n_out, int64_t xs, int64_t ws, int64_t os, float inv_n, float eps,
                       hipStream_t stream) {
    const int64_t big = ((rows + kGemmRows - 1) / kGemmRows) * ((n_out + 255) / 256);
    const int tile = big >= 256 ? 256 : 128;
    const uint32_t nblocks = (uint32_t)((n_out + tile - 1) / tile);
    // rows per launch: whole tiles, and a grid below 2^31 workgroups
    const int64_t max_mblocks = (((int64_t)1 << 31) - 1) / nblocks;
    for (int64_t r0 = 0; r0 < rows; r0 += max_mblocks * kGemmRows) {
        const int64_t rr = rows - r0 < max_mblocks * kGemmRows ? rows - r0 : max_mblocks * kGemmRows;
        const uint32_t mblocks = (uint32_t)((rr + kGemmRows - 1) / kGemmRows);
        __bf16 *o = (__bf16 *)out + r0 * os;
        const __bf16 *xx = (const __bf16 *)x + r0 * xs;
        if (tile == 256)
            hipLaunchKernelGGL((rmsnorm_linear_gemm_kernel<256, 32>), dim3(mblocks * nblocks), dim3(512),
                               0, stream, o, xx, (const __bf16 *)w, (int32_t)rr, (int32_t)n_in, n_out,
                               xs, ws, os, inv_n, eps, mblocks, nblocks);
        else
            hipLaunchKernelGGL((rmsnorm_linear_gemm_kernel<128, 64>), dim3(mblocks * nblocks), dim3(512),
                               0, stream, o, xx, (const __bf16 *)w, (int32_t)rr, (int32_t)n_in, n_out,
                               xs, ws, os, inv_n, eps, mblocks, nblocks);
    }
    return hipGetLastError();
}

// bf16, at most 8 rows whose x fits kGemvMaxXChunks: the GEMV kernel.  Lanes
// take 1, 2, 4 or 8 chunks of a weight row per pass; rows of more than 512
// chunks (only 1-3 rows fit kGemvMaxXChunks then) take 2-4 passes of 8.
hipError_t launch_gemv(void *out, const void *x, const void *w, int64_t rows, int64_t n_in,
                       int64_t n_out, int64_t xs, int64_t ws, int64_t os, float inv_n, float eps,
                       hipStream_t stream) {
    const int32_t nchunks = (int32_t)(n_in / 8);
    const int cpl = nchunks <= 64 ? 1 : nchunks <= 128 ? 2 : nchunks <= 256 ? 4 : 8;
    const int np = (nchunks + 64 * cpl - 1) / (64 * cpl);
    // wide blocks where measured faster: 4 chunks per lane (1032-2048 inputs)
    const bool wide = cpl == 4 && np == 1 && n_out >= kGemvWideOut;
    const int waves = wide ? kGemvWavesWide : kGemvWaves;
    const int64_t per_block = waves * kGemvRowsPerWave;
    const dim3 grid((unsigned)((n_out + per_block - 1) / per_block)), block(64 * waves);
    const size_t lds = (size_t)rows * nchunks * sizeof(u32x4);
    const fastdiv dn = make_fastdiv((uint32_t)nchunks);
#define NRS_GEMV_W(M, C, P, W)                                                                   \
    hipLaunchKernelGGL((rmsnorm_gemv_kernel<M, C, P, W>), grid, block, lds, stream,              \
                       (__bf16 *)out, (const __bf16 *)x, (const __bf16 *)w, nchunks, n_out, xs,  \
                       ws, os, dn, inv_n, eps)
#define NRS_GEMV(M, C, P) NRS_GEMV_W(M, C, P, kGemvWaves)
#define NRS_GEMV_M(C, W)                                                                         \
    switch (rows) {                                                                              \
        case 1: NRS_GEMV_W(1, C, 1, W); break;                                                   \
        case 2: NRS_GEMV_W(2, C, 1, W); break;                                                   \
        case 3: NRS_GEMV_W(3, C, 1, W); break;                                                   \
        case 4: NRS_GEMV_W(4, C, 1, W); break;                                                   \
        case 5: NRS_GEMV_W(5, C, 1, W); break;                                                   \
        case 6: NRS_GEMV_W(6, C, 1, W); break;                                                   \
        case 7: NRS_GEMV_W(7, C, 1, W); break;                                                   \
        default: NRS_GEMV_W(8, C, 1, W); break;                                                  \
    }
    if (np > 1) {
        // rows * nchunks <= kGemvMaxXChunks: 2 passes (513-1024 chunks) take
        // 1-3 rows, 3 and 4 passes (more than 1024 chunks) one row
        if (rows == 1) {
            if (np == 2) NRS_GEMV(1, 8, 2);
            else if (np == 3) NRS_GEMV(1, 8, 3);
            else NRS_GEMV(1, 8, 4);
        } else if (rows == 2) {
            NRS_GEMV(2, 8, 2);
        } else {
            NRS_GEMV(3, 8, 2);
        }
    } else if (cpl == 1) NRS_GEMV_M(1, kGemvWaves)
    else if (cpl == 2) NRS_GEMV_M(2, kGemvWaves)
    else if (cpl == 4 && wide) NRS_GEMV_M(4, kGemvWavesWide)
    else if (cpl == 4) NRS_GEMV_M(4, kGemvWaves)
    else NRS_GEMV_M(8, kGemvWaves)
#undef NRS_GEMV_M
#undef NRS_GEMV
#undef NRS_GEMV_W
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_typed(void *out, const void *x, const void *w, int64_t rows, int64_t n_in,
                        int64_t n_out, int64_t xs, int64_t ws, int64_t os, float eps,
                        hipStream_t stream) {
    const float inv_n = (float)(1.0 / (double)n_in);
    if (sizeof(IO) == 2 && rows <= 8 && rows * (n_in / 8) <= kGemvMaxXChunks)
        return launch_gemv(out, x, w, rows, n_in, n_out, xs, ws, os, inv_n, eps, stream);
    if (sizeof(IO) == 2 && rows > kMaxTileRows && xs < kMaxGemmStride && ws < kMaxGemmStride)
        return launch_gemm(out, x, w, rows, n_in, n_out, xs, ws, os, inv_n, eps, stream);
    // fp32 rows (and bf16 rows of very long strides) beyond one launch's 64
    // are taken 64 at a time (each pass streams w again)
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
