// Device-side helpers shared by the CDNA4 (gfx950) kernels of libnrs.
//
// Storage types are fp32 and bf16; all arithmetic is fp32.  Every global
// access is a 16-byte vector (4 fp32 or 8 bf16 lanes of one "chunk"), so a
// wave64 moves 1 KiB per load instruction.  bf16 results are rounded to
// nearest-even by v_cvt_pk_bf16_f32; fp32 denormals are kept (the kernels are
// built in the default IEEE denormal mode).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nrs {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One 16-byte chunk of a storage type, unpacked to VEC floats.
template <typename IO> struct io_traits;

template <> struct io_traits<float> {
    static constexpr int VEC = 4;
    __device__ static inline void unpack(const u32x4 &raw, float (&v)[VEC]) {
        // bit-cast an rvalue copy: bit-casting the vector-element lvalue
        // itself reads element 0 whatever the index
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(float, (unsigned)raw[i]);
    }
    __device__ static inline u32x4 pack(const float (&v)[VEC]) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(unsigned, v[i]);
        return r;
    }
    // Round an fp32 value to the storage type and back (identity for fp32).
    __device__ static inline float round_trip(float x) { return x; }
};

template <> struct io_traits<__bf16> {
    static constexpr int VEC = 8;
    __device__ static inline void unpack(const u32x4 &raw, float (&v)[VEC]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, raw[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, raw[i] & 0xFFFF0000u);
        }
    }
    __device__ static inline u32x4 pack(const float (&v)[VEC]) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2 p = {v[2 * i], v[2 * i + 1]};
            r[i] = __builtin_bit_cast(unsigned, __builtin_convertvector(p, bf16x2));
        }
        return r;
    }
    __device__ static inline float round_trip(float x) {
        f32x2 p = {x, 0.0f};
        unsigned b = __builtin_bit_cast(unsigned, __builtin_convertvector(p, bf16x2));
        return __builtin_bit_cast(float, b << 16);
    }
};

__device__ inline u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ inline void store16(void *p, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Loads of data touched exactly once: the "nontemporal" hint streams them
// past the caches instead of evicting reusable lines.
__device__ inline u32x4 load16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ inline void store16_stream(void *p, const u32x4 &v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Access policy of a launch: NT streams data that is touched once (large
// calls: read and written once, nothing gained by caching it); otherwise the
// data goes through the caches (small, latency-bound calls whose inputs were
// just written by the producing op and are still cache-resident).
template <bool NT> __device__ inline u32x4 load16_policy(const void *p) {
    if constexpr (NT) return load16_stream(p);
    else return load16(p);
}

template <bool NT> __device__ inline void store16_policy(void *p, const u32x4 &v) {
    if constexpr (NT) store16_stream(p, v);
    else store16(p, v);
}

// Calls that move fewer bytes than this run with cached accesses.
constexpr long long kStreamBytes = 16ll << 20;

// DPP move of a float across lanes of a 16-lane row (bound_ctrl: lanes with
// no source read 0, which never happens for the patterns used here).
template <int CTRL> __device__ inline float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; every lane receives the same total.
// Butterfly inside each 16-lane row (xor 1, xor 2, then mirrors that pair
// lane i with 7-i and 15-i), then the four row sums are read as scalars.
// No LDS and no barrier.
__device__ inline float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    const int b = __builtin_bit_cast(int, v);
    float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// Inclusive prefix over the 64 lanes of a wave (lane order), with DPP only:
// within each 16-lane row, lane i adds lanes i-1, i-2 and i-3, then (lanes
// 4..15) the running sum 4 back, then (lanes 8..15) 8 back; rows 1 and 3 add
// the last lane of the row before them (row_bcast:15), rows 2 and 3 add lane
// 31 (row_bcast:31).  Lanes a step does not write, and sources before the
// start of a row, contribute 0.  Checked on MI355X against sequential sums.
template <int CTRL, int ROWS, int BANKS> __device__ inline int dpp_or0(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, BANKS, true);
}
template <typename V> __device__ inline V wave_incl_scan(V v) {
    auto bits = [](V x) { return __builtin_bit_cast(int, x); };
    auto val = [](int b) { return __builtin_bit_cast(V, b); };
    V x = v + val(dpp_or0<0x111, 0xF, 0xF>(bits(v)));   // row_shr:1
    x += val(dpp_or0<0x112, 0xF, 0xF>(bits(v)));         // row_shr:2
    x += val(dpp_or0<0x113, 0xF, 0xF>(bits(v)));         // row_shr:3
    x += val(dpp_or0<0x114, 0xF, 0xE>(bits(x)));         // row_shr:4, lanes 4..15
    x += val(dpp_or0<0x118, 0xF, 0xC>(bits(x)));         // row_shr:8, lanes 8..15
    x += val(dpp_or0<0x142, 0xA, 0xF>(bits(x)));         // row_bcast:15 into rows 1, 3
    x += val(dpp_or0<0x143, 0xC, 0xF>(bits(x)));         // row_bcast:31 into rows 2, 3
    return x;
}

// Division of 0 <= n < 2^31 by a fixed 1 <= d < 2^31 with a multiply-high
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994: the round-up variant with a 33-bit multiplier,
// its top bit folded into the final add).
struct fastdiv {
    uint32_t d, m, s;
};

inline fastdiv make_fastdiv(uint32_t d) {
    fastdiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
    return f;
}

__device__ inline uint32_t div(uint32_t n, const fastdiv &f) {
    uint32_t hi = __umulhi(n, f.m);
    return (hi + n) >> f.s;
}

// Workgroups are dispatched to the 8 XCDs of an MI355X round-robin (block b
// runs on XCD b % 8).  This remaps block indices so that each XCD walks one
// contiguous eighth of the index range; blocks past the last multiple of 8
// keep their index.
__device__ inline uint32_t xcd_contiguous(uint32_t b, uint32_t nb) {
    const uint32_t per = nb / 8;
    if (b >= per * 8) return b;
    return (b % 8) * per + b / 8;
}

}  // namespace nrs
