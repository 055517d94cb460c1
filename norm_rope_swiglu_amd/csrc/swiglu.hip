// SwiGLU over a packed gate_up buffer, gfx950.
//
// out = silu(gate) * up with silu(g) = g * sigmoid(g), the "SwiGLU" op of the
// qwen3-tts-triton post (de.news.hada.io topic 27742, part 3).  Each gate_up
// row holds [gate | up], `inter` elements each; out rows hold `inter`.
//
// Elementwise streaming: one thread per 16-byte output chunk, reading the
// matching gate and up chunks; measured on MI355X, one access per thread per
// stream in a one-shot grid streams faster than threads that loop over
// several chunks.  Each XCD takes one contiguous eighth of the chunks
// (measured ~1.6% faster than the round-robin interleave; the norms and
// M-RoPE measured faster interleaved).  Chunk -> (row, column) uses a
// multiply-high division by the fixed chunks-per-row.
//
// Numerics: sigmoid(g) = 1/(1 + e^-g) is safe while e^-g stays finite
// (g >= -80).  Below that, silu(g) * up can still be a normal fp32 number
// (e.g. g = -95, up = 1e3 gives ~5e-37) while e^g itself is subnormal or 0,
// so the product is formed on a scaled exponent: g * e^(g + 64) * up, then
// times e^-64 (twice for g < -150), so precision is lost at most in the last
// rounding.  Below g = -214 the exact result is under 1e-54 for any finite
// fp32 up and rounds to a signed zero.
#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

namespace {
constexpr int kThreads = 256;
constexpr int kSmallThreads = 64;   // block size of calls below kStreamBytes
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
}  // namespace

template <typename IO, bool NT>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(IO *out, const IO *gate_up,
                                                          int32_t total, int32_t cpr,
                                                          fastdiv div_cpr, int64_t inter,
                                                          int64_t gu_stride, int64_t out_stride) {
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    const int32_t ci = (int32_t)xcd_contiguous(blockIdx.x, gridDim.x) * (int32_t)blockDim.x + threadIdx.x;
    if (ci >= total) return;
    const int32_t r = (int32_t)div((uint32_t)ci, div_cpr);
    const int32_t col = ci - r * cpr;
    const IO *g = gate_up + (int64_t)r * gu_stride + (int64_t)col * VEC;
    const u32x4 graw = load16_policy<NT>(g);
    const u32x4 uraw = load16_policy<NT>(g + inter);
    float gv[VEC], uv[VEC], o[VEC];
    T::unpack(graw, gv);
    T::unpack(uraw, uv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = silu_mul(gv[e], uv[e]);
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
        // small calls are latency-bound: narrow blocks spread them over more
        // CUs (measured at the 5-token decode step: 64-thread blocks shorten
        // the kernel by ~0.07 us; more chunks per thread lengthen it)
        const int bt = nt ? kThreads : kSmallThreads;
        const int64_t blocks = (total + bt - 1) / bt;
        const fastdiv dv = make_fastdiv((uint32_t)cpr);
        const char *gu = (const char *)gate_up + r0 * gu_stride * esz;
        char *o = (char *)out + r0 * out_stride * esz;
        const dim3 grid((unsigned)blocks), block(bt);
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
