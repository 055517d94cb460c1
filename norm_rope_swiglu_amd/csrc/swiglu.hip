// SwiGLU over a packed gate_up buffer, gfx950.
//
// out = silu(gate) * up with silu(g) = g * sigmoid(g), the "SwiGLU" op of the
// qwen3-tts-triton post (de.news.hada.io topic 27742, part 3).  Each gate_up
// row holds [gate | up], `inter` elements each; out rows hold `inter`.
//
// Elementwise streaming: one thread per 16-byte output chunk, reading the
// matching gate and up chunks, in 64-thread workgroups taken in order (so
// consecutive 1 KiB pieces of the output go to consecutive XCDs); measured on
// MI355X, one access per thread per stream in a one-shot grid streams faster
// than threads that loop over several chunks, and 64-thread workgroups in
// order beat 256-thread ones with each XCD walking one contiguous eighth of
// the chunks by 3-7% (graph-timed, inputs rotated past the cache: 32768 x 6144
// bf16 184.0 -> 178.7 us, 2048 x 6144 14.6 -> 13.7 us, 32768 x 1536 48.3 ->
// 46.8 us; 128- and 512-thread workgroups fell in between).  Chunk -> (row,
// column) uses a multiply-high division by the fixed chunks-per-row.
//
// Numerics: sigmoid(g) = 1/(1 + e^-g) is safe while e^-g stays finite
// (g >= -80); there e^-g comes from the hardware base-2 exponential on an
// exactly split exponent (exp_neg below).  Below that, silu(g) * up can still be a normal fp32 number
// (e.g. g = -95, up = 1e3 gives ~5e-37) while e^g itself is subnormal or 0,
// so the product is formed on a scaled exponent: g * e^(g + 64) * up, then
// times e^-64 (twice for g < -150), so precision is lost at most in the last
// rounding.  Below g = -214 the exact result is under 1e-54 for any finite
// fp32 up and rounds to a signed zero.
#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

namespace {
constexpr int kThreads = 64;
constexpr float kExpM64 = 1.60381089054863785e-28f;  // e^-64

__device__ inline float silu_mul_tail(float g, float u) {
    if (g >= -150.0f) return ((g * expf(g + 64.0f)) * u) * kExpM64;
    if (g >= -214.0f) return (((g * expf(g + 128.0f)) * u) * kExpM64) * kExpM64;
    return __builtin_copysignf(0.0f, -u);
}

__device__ inline float silu_mul(float g, float u) {
    if (__builtin_expect(g < -80.0f, 0)) return silu_mul_tail(g, u);
    const float e = expf(-g);
    return (g * __builtin_amdgcn_rcpf(1.0f + e)) * u;
}

// e^-g for -80 <= g <= 100 on the hardware base-2 exponential: -g * log2(e)
// is formed as its fp32 value x plus the rounding error r, which one FMA
// recovers exactly (the error-free product of Dekker and Ogita-Rump-Oishi),
// plus -g times the part of log2(e) below fp32; then
// e^-g = 2^x * 2^r ~= 2^x * (1 + r ln 2).  |x| <= 116, so |r| < 2^-17 and the
// dropped terms of 2^r are below 2^-35 relative.  The caller clamps g at 100
// (e^-100 vanishes next to 1, and an infinite gate would make r NaN; a NaN
// gate still makes the product NaN through the factor g).
constexpr float kLog2E = 1.44269502163f;      // log2(e) rounded to fp32
constexpr float kLog2ELo = 1.92596303e-08f;   // log2(e) - kLog2E
constexpr float kLn2 = 0.693147182f;
__device__ inline float exp_neg(float g) {
    const float x = -g * kLog2E;
    const float r = __builtin_fmaf(-g, kLog2E, -x) + (-g) * kLog2ELo;
    const float p = __builtin_amdgcn_exp2f(x);
    return __builtin_fmaf(p, r * kLn2, p);
}

// silu(g) * u over a chunk.  A chunk whose gates are all >= -80 (the usual
// case) takes exp_neg and one reciprocal per element, with no per-element
// branch; any lower gate sends the whole chunk through silu_mul.  In bf16
// the chunk's eight products take 128 vector instructions instead of about
// 190 plus a branch per element; measured on MI355X (graph-timed, inputs
// rotated past the cache) 2048 x 6144 13.78 -> 13.49 us, 32768 x 1536
// 47.8 -> 47.0 us, and the 32768-token calls at H >= 2048, which stream at
// their bandwidth ceiling, unchanged.
template <int VEC> __device__ inline void silu_mul_chunk(const float *g, const float *u, float *o) {
    // g < -80 exactly when g's bits, as an unsigned integer, exceed those of
    // -80 (negative values order by magnitude above every positive pattern);
    // negative NaNs and -inf land there too, and silu_mul handles them
    uint32_t gmax = 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) gmax = max(gmax, __builtin_bit_cast(uint32_t, g[e]));
    if (__builtin_expect(gmax > 0xC2A00000u, 0)) {   // -80.0f
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = silu_mul(g[e], u[e]);
        return;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const float en = exp_neg(__builtin_amdgcn_fmed3f(g[e], -100.0f, 100.0f));
        o[e] = (g[e] * __builtin_amdgcn_rcpf(1.0f + en)) * u[e];
    }
}
}  // namespace

template <typename IO, bool NT>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(IO *out, const IO *gate_up,
                                                          int32_t total, int32_t cpr,
                                                          fastdiv div_cpr, int64_t inter,
                                                          int64_t gu_stride, int64_t out_stride) {
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    const int32_t ci = (int32_t)blockIdx.x * kThreads + threadIdx.x;
    if (ci >= total) return;
    const int32_t r = (int32_t)div((uint32_t)ci, div_cpr);
    const int32_t col = ci - r * cpr;
    const IO *g = gate_up + (int64_t)r * gu_stride + (int64_t)col * VEC;
    const u32x4 graw = load16_policy<NT>(g);
    const u32x4 uraw = load16_policy<NT>(g + inter);
    float gv[VEC], uv[VEC], o[VEC];
    T::unpack(graw, gv);
    T::unpack(uraw, uv);
    silu_mul_chunk<VEC>(gv, uv, o);
    store16_policy<NT>(out + (int64_t)r * out_stride + (int64_t)col * VEC, T::pack(o));
}

hipError_t launch_swiglu(void *out, const void *gate_up, int64_t rows, int64_t inter,
                         int64_t gu_stride, int64_t out_stride, int dtype, hipStream_t stream) {
    const int vec = dtype == 0 ? 4 : 8;
    const int64_t cpr = inter / vec;
    const size_t esz = dtype == 0 ? 4 : 2;
    // launch in row slabs so every chunk index of a launch fits in 31 bits
    const int64_t max_rows = ((int64_t)1 << 30) / cpr;
    hipError_t err = hipSuccess;
    for (int64_t r0 = 0; r0 < rows && err == hipSuccess; r0 += max_rows) {
        const int64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
        const int32_t total = (int32_t)(nr * cpr);
        const bool nt = 3 * nr * inter * (long long)esz >= kStreamBytes;
        // (small calls are latency-bound and take the same narrow blocks,
        // which spread them over more CUs: measured at the 5-token decode
        // step, 64-thread blocks shorten the kernel by ~0.07 us against 256)
        const int64_t blocks = (total + kThreads - 1) / kThreads;
        const fastdiv dv = make_fastdiv((uint32_t)cpr);
        const char *gu = (const char *)gate_up + r0 * gu_stride * esz;
        char *o = (char *)out + r0 * out_stride * esz;
        const dim3 grid((unsigned)blocks), block(kThreads);
#define NRS_SWIGLU(IO, NT)                                                                        \
    hipLaunchKernelGGL((swiglu_kernel<IO, NT>), grid, block, 0, stream, (IO *)o, (const IO *)gu, \
                       total, (int32_t)cpr, dv, inter, gu_stride, out_stride)
        if (dtype == 0) {
            if (nt) NRS_SWIGLU(float, true);
            else NRS_SWIGLU(float, false);
        } else {
            if (nt) NRS_SWIGLU(__bf16, true);
            else NRS_SWIGLU(__bf16, false);
        }
#undef NRS_SWIGLU
        err = hipGetLastError();
    }
    return err;
}

}  // namespace nrs
