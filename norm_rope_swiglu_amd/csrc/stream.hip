// Streaming calibration kernels: the practical HBM ceilings the ops are
// measured against.  A kernel reads n_read (0-2) buffers and writes n_write
// (0-2) buffers of the same length, each element once, one 16-byte access
// per thread per buffer in a one-shot grid.  Four patterns are built, the
// ones that streamed fastest on MI355X among those measured (threads moving
// 2, 4 or 8 chunks each copied at 5.8-6.25 TB/s against 6.6-6.7 for one):
//   variant bit 0: 256-thread workgroups (else 64).  At 1 GiB per buffer, 64
//     threads copy fastest (6.70 TB/s against 6.61 with 256 and 6.33 with
//     1024) and are best for the 2-read mixes, while a read-only or
//     write-only kernel of 64-thread groups is limited by the workgroup
//     dispatch rate (about 4.8 TB/s against 7.0 with 256 threads);
//   variant bit 1: stores with the sc1 + nt cache policy through a buffer
//     resource (else nontemporal only).  At 1 GiB this wrote at 7.0 TB/s
//     against 6.7, and copied about 1% faster; in the ops it gained at most
//     1% on large calls and cost up to 10% on 17 MB ones, so the ops keep
//     nontemporal stores.
// Loads are nontemporal; calls that move under kStreamBytes in all use cached
// accesses, as the ops do.  The ceiling of a read/write mix and size is the
// fastest of the four.  With a row size, the copy is row-granular instead
// (stream_rows_kernel): the ceiling of the norms' access pattern; with a row
// size and no writes it reads whole rows one workgroup each
// (stream_rowread_kernel): the ceiling of the sampler's access pattern.
//
// This is a measurement aid, not an op of the pages: it gives the copy (1
// read, 1 write), read-only, write-only, 2-read-1-write (SwiGLU's mix) and
// 2-read-2-write (the fused residual add's mix) rates at any size, so each
// op's rate can be compared with kernels that do nothing but move the same
// bytes ("Optimising autoregressive speech models", "Custom Triton kernels":
// profile first to find the actual bottleneck).
#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

namespace {

constexpr int kPolicySc1Nt = 2 | 16;   // buffer-instruction cache policy bits: nt | sc1

// Stores through a buffer resource based at the workgroup's first chunk (a
// workgroup-uniform base, 32-bit offsets), so they can carry the sc1 + nt
// policy, which a plain pointer store cannot express.
struct out_window {
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ explicit out_window(void *base)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(base, 0, -1, 0x00020000)) {}
    __device__ void store(uint32_t off, const u32x4 &v) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)off, 0, kPolicySc1Nt);
    }
};

template <int NR, int NW, int BS, bool NT, bool SC1>
__global__ __launch_bounds__(BS) void stream_kernel(u32x4 *d0, u32x4 *d1, const u32x4 *s0,
                                                    const u32x4 *s1, int64_t n) {
    const int64_t i0 = (int64_t)blockIdx.x * BS;
    const int64_t i = i0 + threadIdx.x;
    if (i >= n) return;
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (NR >= 1) a = load16_policy<NT>(s0 + i);
    if (NR >= 2) b = load16_policy<NT>(s1 + i);
    u32x4 v;
    if (NR == 0) v = u32x4{(unsigned)i, (unsigned)(i >> 32), 0x5A5A5A5Au, 0xA5A5A5A5u};
    else v = a ^ b;
    if (NW == 0) {
        // read-only: an empty asm statement consumes the loaded values, so
        // the loads are issued and waited for and nothing is written (a
        // store under a never-taken branch let the compiler move the loads
        // into that branch, and nothing was read)
        asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
        return;
    }
    const u32x4 v1 = NR >= 1 ? ~a : ~v;
    if constexpr (NT && SC1) {
        const uint32_t off = threadIdx.x * 16u;
        out_window(d0 + i0).store(off, v);
        if (NW >= 2) out_window(d1 + i0).store(off, v1);
    } else {
        store16_policy<NT>(d0 + i, v);
        if (NW >= 2) store16_policy<NT>(d1 + i, v1);
    }
}

// Row-granular copies: whole rows of KIB KiB per workgroup, the access
// pattern of a single-pass row reduction (a row's elements must meet in one
// workgroup).  WAVE = false: one row per workgroup of KIB waves, one chunk
// per thread (the norms' layout for rows of up to 16 waves); WAVE = true: one
// wave per row, KIB chunks per lane (lane l takes chunks l, l + 64, ...),
// four rows to a 256-thread workgroup (the norms' layout for one-wave rows).
template <int NR, int NW, int KIB, bool WAVE, bool NT>
__global__ __launch_bounds__(WAVE ? 256 : 64 * KIB) void stream_rows_kernel(
    u32x4 *d0, u32x4 *d1, const u32x4 *s0, const u32x4 *s1, int64_t rows) {
    static_assert(NR >= 1 && NR == NW, "row copies move 1 or 2 streams each way");
    constexpr int CPR = 64 * KIB;                       // chunks per row
    constexpr int NCH = WAVE ? KIB : 1;                 // chunks per thread
    const int64_t row = WAVE ? (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6) : (int64_t)blockIdx.x;
    if (row >= rows) return;
    const int t = WAVE ? (threadIdx.x & 63) : threadIdx.x;
    u32x4 a[NCH], b[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t i = row * CPR + t + 64 * c;
        a[c] = load16_policy<NT>(s0 + i);
        if (NR >= 2) b[c] = load16_policy<NT>(s1 + i);
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t i = row * CPR + t + 64 * c;
        store16_policy<NT>(d0 + i, NR >= 2 ? a[c] ^ b[c] : a[c]);
        if (NW >= 2) store16_policy<NT>(d1 + i, ~a[c]);
    }
}

// Row-granular reads: one 1024-thread workgroup per row of `cpr` 16-byte
// chunks, thread t reading chunks t, t + 1024, ...: its first 8 issued
// together, then the rest B at a time, every batch folded into a running XOR
// that an empty asm statement consumes (nothing is written).  The access
// pattern of the sampler's long rows, which are read once by one workgroup
// each while the row's selection runs.
template <int B, bool NT>
__global__ __launch_bounds__(1024) void stream_rowread_kernel(const u32x4 *s0, int64_t cpr) {
    constexpr int kHold = 8;
    const u32x4 *p = s0 + (int64_t)blockIdx.x * cpr;
    const int64_t t = threadIdx.x;
    u32x4 acc = {0, 0, 0, 0};
    u32x4 h[kHold];
#pragma unroll
    for (int i = 0; i < kHold; ++i) {
        const int64_t c = t + 1024 * i;
        h[i] = c < cpr ? load16_policy<NT>(p + c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kHold; ++i) acc ^= h[i];
    for (int64_t c = t + 1024 * kHold; c < cpr; c += 1024 * B) {
        u32x4 b[B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int64_t cc = c + 1024 * i;
            b[i] = cc < cpr ? load16_policy<NT>(p + cc) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < B; ++i) acc ^= b[i];
    }
    asm volatile("" ::"v"(acc[0]), "v"(acc[1]), "v"(acc[2]), "v"(acc[3]));
}

template <int NR, int KIB, bool NT>
void launch_rows_kib(void *d0, void *d1, const void *s0, const void *s1, int64_t rows, bool wave,
                     hipStream_t stream) {
    if (wave)
        hipLaunchKernelGGL((stream_rows_kernel<NR, NR, KIB, true, NT>), dim3((unsigned)((rows + 3) / 4)),
                           dim3(256), 0, stream, (u32x4 *)d0, (u32x4 *)d1, (const u32x4 *)s0,
                           (const u32x4 *)s1, rows);
    else
        hipLaunchKernelGGL((stream_rows_kernel<NR, NR, KIB, false, NT>), dim3((unsigned)rows),
                           dim3(64 * KIB), 0, stream, (u32x4 *)d0, (u32x4 *)d1, (const u32x4 *)s0,
                           (const u32x4 *)s1, rows);
}

template <int NR, bool NT>
void launch_rows(void *d0, void *d1, const void *s0, const void *s1, int64_t rows, int kib,
                 bool wave, hipStream_t stream) {
    switch (kib) {
        case 1: launch_rows_kib<NR, 1, NT>(d0, d1, s0, s1, rows, wave, stream); break;
        case 2: launch_rows_kib<NR, 2, NT>(d0, d1, s0, s1, rows, wave, stream); break;
        case 3: launch_rows_kib<NR, 3, NT>(d0, d1, s0, s1, rows, wave, stream); break;
        case 4: launch_rows_kib<NR, 4, NT>(d0, d1, s0, s1, rows, wave, stream); break;
        case 6: launch_rows_kib<NR, 6, NT>(d0, d1, s0, s1, rows, wave, stream); break;
        case 8: launch_rows_kib<NR, 8, NT>(d0, d1, s0, s1, rows, wave, stream); break;
        case 12: launch_rows_kib<NR, 12, NT>(d0, d1, s0, s1, rows, wave, stream); break;
        default: launch_rows_kib<NR, 16, NT>(d0, d1, s0, s1, rows, wave, stream); break;
    }
}

template <int NR, int NW>
void launch_mix(void *d0, void *d1, const void *s0, const void *s1, int64_t n, bool nt,
                int variant, hipStream_t stream) {
    const int bs = (variant & 1) ? 256 : 64;
    const dim3 grid((unsigned)((n + bs - 1) / bs)), block(bs);
#define NRS_STREAM(BS, NT, SC1)                                                                  \
    hipLaunchKernelGGL((stream_kernel<NR, NW, BS, NT, SC1>), grid, block, 0, stream, (u32x4 *)d0, \
                       (u32x4 *)d1, (const u32x4 *)s0, (const u32x4 *)s1, n)
    if (!nt) {
        if (bs == 64) NRS_STREAM(64, false, false);
        else NRS_STREAM(256, false, false);
    } else if (variant & 2) {
        if (bs == 64) NRS_STREAM(64, true, true);
        else NRS_STREAM(256, true, true);
    } else {
        if (bs == 64) NRS_STREAM(64, true, false);
        else NRS_STREAM(256, true, false);
    }
#undef NRS_STREAM
}

}  // namespace

hipError_t launch_stream_probe(void *d0, void *d1, const void *s0, const void *s1, int n_read,
                               int n_write, int64_t bytes, int64_t row_bytes, int variant,
                               hipStream_t stream) {
    const int64_t n = bytes / 16;
    const bool nt = bytes * (n_read + n_write) >= kStreamBytes;
    if (row_bytes > 0 && n_write == 0) {
        // row-granular read: variant 0 streams the rest of a row 4 chunks per
        // thread at a time (the sampler's batches), variant 1 8 at a time
        const int64_t rows = bytes / row_bytes, cpr = row_bytes / 16;
        const dim3 grid((unsigned)rows), block(1024);
#define NRS_ROWREAD(B, NT)                                                                        \
    hipLaunchKernelGGL((stream_rowread_kernel<B, NT>), grid, block, 0, stream,                    \
                       (const u32x4 *)s0, cpr)
        if (variant == 0) {
            if (nt) NRS_ROWREAD(4, true);
            else NRS_ROWREAD(4, false);
        } else {
            if (nt) NRS_ROWREAD(8, true);
            else NRS_ROWREAD(8, false);
        }
#undef NRS_ROWREAD
        return hipGetLastError();
    }
    if (row_bytes > 0) {
        const int64_t rows = bytes / row_bytes;
        const int kib = (int)(row_bytes >> 10);
        const bool wave = variant & 1;
        if (n_read == 1) {
            if (nt) launch_rows<1, true>(d0, d1, s0, s1, rows, kib, wave, stream);
            else launch_rows<1, false>(d0, d1, s0, s1, rows, kib, wave, stream);
        } else {
            if (nt) launch_rows<2, true>(d0, d1, s0, s1, rows, kib, wave, stream);
            else launch_rows<2, false>(d0, d1, s0, s1, rows, kib, wave, stream);
        }
        return hipGetLastError();
    }
    switch (n_read * 3 + n_write) {
        case 1: launch_mix<0, 1>(d0, d1, s0, s1, n, nt, variant, stream); break;
        case 2: launch_mix<0, 2>(d0, d1, s0, s1, n, nt, variant, stream); break;
        case 3: launch_mix<1, 0>(d0, d1, s0, s1, n, nt, variant, stream); break;
        case 4: launch_mix<1, 1>(d0, d1, s0, s1, n, nt, variant, stream); break;
        case 5: launch_mix<1, 2>(d0, d1, s0, s1, n, nt, variant, stream); break;
        case 6: launch_mix<2, 0>(d0, d1, s0, s1, n, nt, variant, stream); break;
        case 7: launch_mix<2, 1>(d0, d1, s0, s1, n, nt, variant, stream); break;
        default: launch_mix<2, 2>(d0, d1, s0, s1, n, nt, variant, stream); break;
    }
    return hipGetLastError();
}

}  // namespace nrs
