// Fused softmax + top-k sampling over vocabulary logits, gfx950.
//
// "Optimising autoregressive speech models", "Custom Triton kernels", kernel 2:
// decoding ends with softmax then sampling, and fusing them saves a full
// write and re-read of the vocabulary row.  The page's sketch divides the
// logits by the temperature, subtracts the max, exponentiates and normalises;
// its top-k and sampling steps are cut off.  Completed here as: keep the
// top_k largest logits (lower index first on ties), renormalise their
// probabilities, and return the first kept token, in that order, whose
// cumulative probability exceeds the caller's uniform u[row] (the last kept
// token if rounding leaves none).  The full softmax row is written only when
// asked for.
//
// One 1024-thread workgroup per row:
//   1. radix select of the k-th largest logit on monotone 32-bit keys, 8 bits
//      per pass for register-held rows and 12 for streamed ones (bf16 keys
//      vary in 16 bits, fp32 in 32), histograms in LDS, stopping as soon as
//      everything above the selected bin plus the bin fits the 1024-entry
//      gather buffer;
//   2. one pass gathers every logit in or above the selected bin (the
//      histogram counts them) when they fit; only tie runs longer than the
//      buffer take an ordered compaction (a block-wide prefix count per 1024
//      chunks keeps the lowest-index ties);
//   3. a sort of the gathered entries by (logit descending, index ascending):
//      up to 256 entries, each entry's rank counted by several threads over
//      slices of the entries, then each entry moved to its rank; beyond, a
//      bitonic network in LDS;
//   4. exp((l - l_max) / T) per kept entry, an inclusive scan (one wave's lane
//      shuffles when top_k <= 64, else block-wide), and the first entry whose
//      prefix exceeds u * total.
// Rows of up to 8 16-byte chunks per thread (65536 bf16 or 32768 fp32
// logits) are read from HBM once, into registers, as order keys, and every
// pass runs over the registers (token-only calls with top_k <= 128 over rows
// of at least 1024 chunks take the bounded filter described next instead,
// with the whole row held).  (At 20 chunks per thread the registers spill
// and the kernel ran slower than streaming the row.)  Longer rows, when only
// the token is asked for, are read once too: the first 8 chunks per thread
// are held as loaded, each thread's largest logit is found with packed
// compares, a lower bound for the row's top_k-th largest is taken from those
// maxima (the waves sort theirs across the lanes; the bound is the top_k-th
// largest of every wave's first 8 or 16), and one pass over the held part and
// the streamed rest tests the loaded values against it and keeps, as keys,
// every logit at or above it (about 2.5 top_k of them), which step 3 sorts.  Such a row falls back to the passes above,
// re-reading it, only when the kept logits overflow the 1024-entry buffer
// (top_k near 1024, or a row whose logits rise along it), or when the softmax
// output is asked for.
#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;  // chunks in flight per thread in the passes over the row
// Radix digit and histogram replicas: rows streamed from memory take 12-bit
// digits (4096 bins, 4 replicas), so the first pass usually narrows the
// candidates enough to skip the rest and one read of the row is saved;
// register-held rows take 8-bit digits (256 bins, 32 replicas; 8 when each
// thread holds one chunk), whose smaller histograms cost less to clear and scan
// than an extra pass over registers.  Measured on MI355X: at one chunk per
// thread (rows up to 8192 bf16) 8 replicas cut a 5 x 3072 call from 8.6 to
// 8.1 us; with more chunks per thread, or flat rows, fewer replicas lose more to
// atomics on the same bins than they save.
constexpr int kHistWords = 16384;
// up to this many kept entries are ranked by counting; more by a bitonic
// network (counting grows as entries squared over the 1024 threads)
constexpr int kRankMax = 256;
// rows filtered against a bound take it from the waves' leading thread
// maxima up to this top_k (a radix select over all the maxima beyond)
constexpr int kLeadTopK = 128;
// the template value of the kernel for rows longer than its held part
constexpr int kLongRow = -9;

// Order-preserving map of an fp32 value to uint32 (larger value, larger key);
// -0 is folded onto +0 so equal values have equal keys.
__device__ inline uint32_t key_of(float f) {
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline float value_of(uint32_t k) {
    const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __builtin_bit_cast(float, b);
}

// Rows are held as order keys: an fp32 chunk as four 32-bit keys, a bf16
// chunk as eight 16-bit keys (the high half of the fp32 key; its low half
// follows from the sign), two to a word, so a chunk keeps its 16 bytes.
template <typename IO> struct keys;

template <> struct keys<float> {
    __device__ static inline u32x4 from_raw(const u32x4 &raw) {
        u32x4 k;
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = key_of(__builtin_bit_cast(float, (unsigned)raw[i]));
        return k;
    }
    __device__ static inline uint32_t at(const u32x4 &k, int e) { return k[e]; }
    // the largest full key of a chunk
    __device__ static inline uint32_t chunk_max(const u32x4 &k) {
        const uint32_t a = k[0] > k[1] ? k[0] : k[1], b = k[2] > k[3] ? k[2] : k[3];
        return a > b ? a : b;
    }
    __device__ static inline uint32_t max2(uint32_t a, uint32_t b) { return a > b ? a : b; }
    __device__ static inline uint32_t full(uint32_t m) { return m; }
    // bit e set when element e's key is at least `bound` (a full key)
    __device__ static inline uint32_t mask_ge(const u32x4 &k, uint32_t bound) {
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) m |= (k[e] >= bound ? 1u : 0u) << e;
        return m;
    }
};

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

template <> struct keys<__bf16> {
    __device__ static inline uint32_t key16(uint32_t h) {
        if (h == 0x8000u) h = 0u;                       // -0 onto +0
        return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
    }
    __device__ static inline u32x4 from_raw(const u32x4 &raw) {
        u32x4 k;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            k[i] = key16(raw[i] & 0xFFFFu) | (key16(raw[i] >> 16) << 16);
        return k;
    }
    __device__ static inline uint32_t at(const u32x4 &k, int e) {
        const uint32_t h = (k[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        return (h << 16) | ((h & 0x8000u) ? 0u : 0xFFFFu);   // the full fp32 key
    }
    // per-half maxima of two words of keys, and the largest 16-bit key of a
    // chunk (as its full key by full())
    __device__ static inline uint32_t max2(uint32_t a, uint32_t b) {
        const us2 m = __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b));
        return __builtin_bit_cast(uint32_t, m);
    }
    __device__ static inline uint32_t chunk_max(const u32x4 &k) {
        const uint32_t w = max2(max2(k[0], k[1]), max2(k[2], k[3]));
        return full(w);
    }
    __device__ static inline uint32_t full(uint32_t w) {
        const uint32_t lo = w & 0xFFFFu, hi = w >> 16, h = lo > hi ? lo : hi;
        return (h << 16) | ((h & 0x8000u) ? 0u : 0xFFFFu);
    }
    // bit e set when element e's key is at least `bound`, a full key whose
    // low 16 bits are zero (so comparing the 16-bit keys decides it)
    __device__ static inline uint32_t mask_ge(const u32x4 &k, uint32_t bound) {
        const uint32_t b16 = bound >> 16;
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m |= ((k[i] & 0xFFFFu) >= b16 ? 1u : 0u) << (2 * i);
            m |= ((k[i] >> 16) >= b16 ? 1u : 0u) << (2 * i + 1);
        }
        return m;
    }
};

// Exclusive prefix over the block (thread order) of a small int, and the total.
__device__ inline int block_exclusive_scan(int v, int *wave_tot, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int t = wave_tot[w];
        if (w < wave) before += t;
        total += t;
    }
    __syncthreads();
    return before + incl - v;
}

// Inclusive prefix sum over the block (thread order) of a float.
__device__ inline float block_inclusive_scan(float v, float *wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float incl = wave_incl_scan(v);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    float before = 0.0f;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    __syncthreads();
    return before + incl;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// v from lane ^ J (J a power of two below 64): DPP moves within a 16-lane
// row (quad permutes for 1 and 2, the row shifted up or down by 4, the row
// rotated by 8), ds_swizzle within 32 lanes for 16, a lane permute for 32.
template <int J> __device__ inline uint32_t lane_xor(uint32_t v) {
    const int iv = (int)v;
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(iv, iv, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(iv, iv, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    } else if constexpr (J == 4) {
        const int up = __builtin_amdgcn_update_dpp(iv, iv, 0x104, 0xF, 0xF, false);   // row_shl:4: lane + 4
        const int dn = __builtin_amdgcn_update_dpp(iv, iv, 0x114, 0xF, 0xF, false);   // row_shr:4: lane - 4
        return (uint32_t)((threadIdx.x & 4) ? dn : up);
    } else if constexpr (J == 8) {
        return (uint32_t)__builtin_amdgcn_update_dpp(iv, iv, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (J == 16) {
        return (uint32_t)__builtin_amdgcn_ds_swizzle(iv, (16 << 10) | 0x1F);           // xor 16 in 32
    } else {
        return (uint32_t)__shfl_xor(iv, J, 64);
    }
}

// A bitonic network across the lanes: compare-exchange of lanes (lane,
// lane ^ J); in a block of SIZE lanes to be sorted descending the lower lane
// keeps the larger key.
template <int SIZE, int J> __device__ inline uint32_t bitonic_step(uint32_t v, int lane) {
    const uint32_t o = lane_xor<J>(v);
    const bool keep_max = ((lane & J) == 0) == ((lane & SIZE) == 0);
    return keep_max ? (v > o ? v : o) : (v < o ? v : o);
}
template <int SIZE, int J> __device__ inline uint32_t bitonic_merge(uint32_t v, int lane) {
    v = bitonic_step<SIZE, J>(v, lane);
    if constexpr (J > 1) return bitonic_merge<SIZE, J / 2>(v, lane);
    else return v;
}
template <int SIZE> __device__ inline uint32_t bitonic_sort(uint32_t v, int lane) {
    if constexpr (SIZE > 2) v = bitonic_sort<SIZE / 2>(v, lane);
    return bitonic_merge<SIZE, SIZE / 2>(v, lane);
}

// The wave's 64 keys sorted across the lanes, descending (lane 0 the largest).
__device__ inline uint32_t wave_sort_desc(uint32_t v) {
    return bitonic_sort<64>(v, threadIdx.x & 63);
}

// A workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight (__syncthreads also waits for every one of them).
__device__ inline void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// max(v, v of lane ^ J).  The partner's value is read before the compare:
// a cross-lane read inside a branch (as a conditional operator evaluates its
// arms) would read lanes the branch has switched off.
template <int J> __device__ inline uint32_t max_xor(uint32_t v) {
    const uint32_t o = lane_xor<J>(v);
    return v > o ? v : o;
}

// The largest of the wave's 64 keys, in every lane.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
    v = max_xor<1>(v);
    v = max_xor<2>(v);
    v = max_xor<4>(v);
    v = max_xor<8>(v);
    const int b = (int)v;
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane(b, 0), r1 = (uint32_t)__builtin_amdgcn_readlane(b, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane(b, 32), r3 = (uint32_t)__builtin_amdgcn_readlane(b, 48);
    const uint32_t a = r0 > r1 ? r0 : r1, c = r2 > r3 ? r2 : r3;
    return a > c ? a : c;
}

// The full order key of one bf16 pattern h (as keys<__bf16>::at gives it).
__device__ inline uint32_t bf16_full_key(uint32_t h) {
    const uint32_t k = keys<__bf16>::key16(h);
    return (k << 16) | ((k & 0x8000u) ? 0u : 0xFFFFu);
}

// The order key of entry e of a chunk as loaded.
template <typename IO> __device__ inline uint32_t raw_key(const u32x4 &raw, int e) {
    if constexpr (sizeof(IO) == 2) return bf16_full_key((raw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    else return key_of(__builtin_bit_cast(float, (unsigned)raw[e]));
}

// The largest logit of the first n of N chunks as loaded, as an order key,
// with no per-entry key: bf16 patterns compare as signed 16-bit integers in
// value order while a non-negative one exists, and among negative ones the
// least unsigned pattern is the largest value (packed max and min, two
// patterns an op); fp32 takes the float max.  n >= 1.
template <typename IO, int N> __device__ inline uint32_t max_key_raw(const u32x4 (&c)[N], int n) {
    if constexpr (sizeof(IO) == 2) {
        s16x2 mx = {(short)-32768, (short)-32768};
        us2 mn = {(unsigned short)0xFFFF, (unsigned short)0xFFFF};
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if (j < n) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(s16x2, (unsigned)c[j][i]));
                    mn = __builtin_elementwise_min(mn, __builtin_bit_cast(us2, (unsigned)c[j][i]));
                }
            }
        }
        const int hmax = mx.x > mx.y ? mx.x : mx.y;
        return bf16_full_key(hmax >= 0 ? (uint32_t)hmax : (uint32_t)(mn.x < mn.y ? mn.x : mn.y));
    } else {
        float m = -__builtin_huge_valf();
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if (j < n) {
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, __builtin_bit_cast(float, (unsigned)c[j][i]));
            }
        }
        return key_of(m);
    }
}

// A bound on order keys tested on chunks as loaded.  A bound above zero and
// finite (the usual case) is compared with the loaded values: bf16 patterns
// as signed 16-bit integers (negative patterns fall below it) by a saturating
// packed subtract, whose sign bit is set where an entry falls below; fp32 as
// floats.  Any other bound is compared on order keys.
template <typename IO> struct RawBound {
    uint32_t key, hb;
    float bval;
    bool fast;
    // k is the same in every lane: held in a scalar register, so the choice
    // between the two tests is a uniform branch (as a per-lane value the
    // compiler evaluated both tests for every chunk)
    __device__ explicit RawBound(uint32_t k)
        : key((uint32_t)__builtin_amdgcn_readfirstlane((int)k)), hb(0u), bval(0.0f) {
        k = key;
        if constexpr (sizeof(IO) == 2) {
            hb = (k >> 16) & 0x7FFFu;   // a bf16 key's low 16 bits follow its sign
            fast = (k & 0x80000000u) && hb != 0u;
        } else {
            const uint32_t mag = k & 0x7FFFFFFFu;
            fast = (k & 0x80000000u) && mag - 1u < 0x7F800000u;
            bval = __builtin_bit_cast(float, mag);
        }
    }
    // whether any entry of the chunk is at or above the bound
    __device__ bool any(const u32x4 &raw) const {
        if (fast) {
            if constexpr (sizeof(IO) == 2) {
                const s16x2 b2 = {(short)hb, (short)hb};
                uint32_t all = 0xFFFFFFFFu;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    all &= __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(
                                                             __builtin_bit_cast(s16x2, (unsigned)raw[i]), b2));
                return (all & 0x80008000u) != 0x80008000u;
            } else {
                bool p = false;
#pragma unroll
                for (int i = 0; i < 4; ++i) p |= __builtin_bit_cast(float, (unsigned)raw[i]) >= bval;
                return p;
            }
        }
        return keys<IO>::chunk_max(keys<IO>::from_raw(raw)) >= key;
    }
    // bit e set when entry e is at or above the bound
    __device__ uint32_t mask(const u32x4 &raw) const {
        if (fast) {
            uint32_t m = 0u;
            if constexpr (sizeof(IO) == 2) {
                const s16x2 b2 = {(short)hb, (short)hb};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t d = ~__builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(
                                                                         __builtin_bit_cast(s16x2, (unsigned)raw[i]), b2));
                    m |= ((d >> 15) & 1u) << (2 * i);
                    m |= (d >> 31) << (2 * i + 1);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) m |= (__builtin_bit_cast(float, (unsigned)raw[i]) >= bval ? 1u : 0u) << i;
            }
            return m;
        }
        return keys<IO>::mask_ge(keys<IO>::from_raw(raw), key);
    }
};
}  // namespace

// The workgroup's LDS, shared by a row's first attempt and its fallback.
struct SampleShared {
    // bin-major: the replicas of a bin sit on kRep consecutive banks
    uint32_t hist[kHistWords];
    uint32_t wtot[4];
    uint32_t sel[3];            // selected digit, count above it, count equal
    int iscan[kWaves];
    float fscan[kWaves];
    alignas(16) uint32_t ckey[kThreads];   // kept entries: key, index
    alignas(16) int32_t cidx[kThreads];
    float csum[kThreads];       // prefix sums of the kept weights
    int32_t rank_of[kThreads];  // ranks of the kept entries (up to kRankMax)
    alignas(16) uint32_t lead[kThreads / 4];   // the waves' largest thread maxima
    uint32_t n_gt, lead_bound;
    int32_t pick;
};

// One row.  CPT > 0: thread t holds the row's chunks t, t + 1024, ... (at
// most CPT of them) in registers; CPT == 0: every pass streams the row from
// memory.  CPT < 0 (token only): the row's first chunks are held, the
// whole row if CPT > kLongRow (-CPT chunks per thread), else 8 * 1024 of
// them, and selected as a row of their own; their k-th largest key is a lower bound for the whole row's, so one
// pass over the rest of the row appends every key at or above it to the kept
// entries, and the sort of all of them gives the row's top k.  The row is read
// once.  If the kept entries overflow the buffer (a row whose later logits
// run higher, for instance), it returns false having written nothing, and the
// row is then selected again as CPT == 0.  Otherwise it returns true.
template <typename IO, int CPT>
__device__ __attribute__((always_inline)) bool sample_row(
    SampleShared &sh, int32_t *token, IO *probs, const IO *logits, int64_t vocab,
    int64_t row_stride, int64_t probs_stride, float inv_temp, int32_t top_k, const float *u) {
    using K = keys<IO>;
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    constexpr bool FILTER = CPT < 0;
    // CPT == kLongRow: a row longer than its held part (8 chunks per thread,
    // every one in the row); other negative CPT: the whole row held, -CPT
    // chunks per thread, the last round possibly partial
    constexpr bool LONG = CPT == kLongRow;
    constexpr int HC = LONG ? 8 : (FILTER ? -CPT : CPT);   // chunks held per thread
    constexpr int kDigitBits = HC > 0 ? 8 : 12;
    // (the select over the threads' maxima counts one key per thread)
    constexpr int kRep = FILTER ? 4 : (HC == 1 ? 8 : (HC > 0 ? 32 : 4));
    static_assert((kRep << kDigitBits) <= kHistWords, "histogram fits");
    uint32_t *hist = sh.hist, *wtot = sh.wtot, *sel = sh.sel, *ckey = sh.ckey;
    int *iscan = sh.iscan;
    float *fscan = sh.fscan, *csum = sh.csum;
    int32_t *cidx = sh.cidx, *rank_of = sh.rank_of;
    uint32_t &n_gt = sh.n_gt;
    int32_t &pick = sh.pick;

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const IO *x = logits + row * row_stride;
    const int64_t nchunks = vocab / VEC;
    // chunks the select and gather run over: the whole row, or its held part
    const int64_t nheld = FILTER ? (nchunks < (int64_t)HC * kThreads ? nchunks : (int64_t)HC * kThreads)
                                 : nchunks;

    // the row's source: keys in registers (loaded here, all at once) or
    // memory (converted to keys as each pass reads it)
    u32x4 held[HC > 0 ? HC : 1];
    // FILTER: the rest of the row streams in batches of kUnroll chunks per
    // thread, the next batch in flight while one is filtered; the first batch
    // is issued with the held part.  These loads take no branch (an index past
    // the row reads its last chunk, skipped by the filter), so the compiler
    // waits for each batch alone rather than for every load in flight.
    // Measured on MI355X (256 x 151936 bf16, 23.6 us as written): issuing the
    // second batch with the held part too made the call 24.7 us, every batch
    // at once (six chunks per thread) 25.7 us, and issuing the first two only
    // once a wave's held part had landed 25.1 us: the held part, which the
    // bound waits for, lands later.
    constexpr int FB = FILTER ? kUnroll : 1;
    u32x4 sa[FB], sb[FB];
    auto load_batch = [&](u32x4 (&buf)[FB], int64_t c0) {
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            const int64_t c = c0 + (int64_t)j * kThreads;
            buf[j] = load16(x + (c < nchunks ? c : nchunks - 1) * VEC);
        }
    };
    if constexpr (FILTER) {
#pragma unroll
        for (int j = 0; j < HC; ++j) {
            const int64_t c = tid + (int64_t)j * kThreads;   // (no branch: a chunk past the
            held[j] = load16(x + (LONG || c < nchunks ? c : nchunks - 1) * VEC);   // row re-reads its last)
        }
        load_batch(sa, nheld + tid);
    } else if constexpr (HC > 0) {
#pragma unroll
        for (int j = 0; j < HC; ++j) {
            const int64_t c = tid + (int64_t)j * kThreads;
            if (c < nheld) held[j] = load16(x + c * VEC);
        }
    }
    // (a row filtered against a bound keeps its chunks as loaded: keys are
    // formed only for the entries it keeps)
    if constexpr (HC > 0 && !FILTER) {
#pragma unroll
        for (int j = 0; j < HC; ++j) held[j] = K::from_raw(held[j]);
    }
    // Marks the held keys as rewritten (an empty asm statement that emits no
    // instruction), so each pass re-derives per-element keys from them instead
    // of the compiler keeping every pass's unpacked keys alive in registers.
    auto opaque = [&]() {
        if constexpr (HC > 0) {
#pragma unroll
            for (int j = 0; j < HC; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(held[j][i]));
        }
    };
    // f(c, keys) for every chunk c this thread owns, in increasing c
    auto for_chunks = [&](auto &&f) {
        if constexpr (HC > 0) {
#pragma unroll
            for (int j = 0; j < HC; ++j) {
                const int64_t c = tid + (int64_t)j * kThreads;
                if (c < nheld) f(c, held[j]);
            }
        } else {
            for (int64_t c0 = tid; c0 < nchunks; c0 += kUnroll * kThreads) {
                u32x4 raw[kUnroll];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) {
                    const int64_t c = c0 + j * kThreads;
                    if (c < nchunks) raw[j] = load16(x + c * VEC);
                }
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) {
                    const int64_t c = c0 + j * kThreads;
                    if (c < nchunks) f(c, K::from_raw(raw[j]));
                }
            }
        }
    };

    // 1. radix select: find the top_k-th largest key, kDigitBits at a time from
    //    the top (streamed bf16 keys: 12 + 4 bits; fp32: 12 + 12 + 8).  The
    //    remaining digits are left to the sort once every key above the
    //    selected bin plus the bin itself fits the counting sort (256), or, for a
    //    streamed row (CPT == 0: a long row that fell back), the 1024-entry
    //    gather buffer (with 12-bit digits this usually happens after the first
    //    pass, so such a row is read twice: once counted, once gathered).  The
    //    histograms keep replicas (indexed by lane) so lanes counting the same
    //    bin, common with peaky logits, split over several addresses.
    constexpr int kKeyBits = sizeof(IO) == 4 ? 32 : 16;   // bits that vary in a key
    // FILTER: the select runs over one key per thread, the largest it holds.
    // These are distinct entries of the row, so the top_k-th largest of them
    // is at most the row's top_k-th largest: every kept entry lies at or
    // above it.  With top_k well below the thread count, the row's largest
    // entries mostly sit in different threads, and the bound is nearly the
    // row's own top_k-th largest.  (Up to top_k = kLeadTopK the bound comes
    // from the waves' sorted maxima instead, below.)
    uint32_t mkey = 0;
    if constexpr (FILTER) {
        // the held chunks that lie in the row (at least one: such rows have at
        // least one chunk per thread)
        const int64_t nv = LONG ? HC : (nchunks - tid + kThreads - 1) / kThreads;
        mkey = max_key_raw<IO, HC>(held, nv < HC ? (int)nv : HC);
    }
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)top_k;
    const uint32_t rep = tid & (kRep - 1);
    bool fits = false;
    constexpr int kPasses = (kKeyBits + kDigitBits - 1) / kDigitBits;
    // FILTER, top_k <= kLeadTopK: the bound is instead the top_k-th largest
    // of the waves' m largest thread maxima (m = 8, or 16 past top_k = 64),
    // the waves sorting their maxima across the lanes; ranked by counting
    // over those 16 * m keys.  They are distinct entries of the row too, and
    // with the row's largest entries spread over the threads, the waves'
    // first eight or sixteen hold nearly all that matter: on rows of 151,936
    // normally distributed logits, top_k = 50, it keeps 118.6 entries on
    // average against 118.1 for the exact top_k-th of all 1024 maxima.  One
    // sort in registers and two barriers that leave the streamed batch in
    // flight, in place of a radix select's passes (which waited for it).
    const bool lead = FILTER && top_k <= kLeadTopK;   // uniform
    if (lead) {
        const int lane = tid & 63, wave = tid >> 6;
        const int m = top_k <= 64 ? 8 : 16;
        const uint32_t srt = wave_sort_desc(mkey);
        if (lane < m) sh.lead[wave * m + lane] = srt;
        if (tid == 0) sh.lead_bound = 0u;
        lds_sync();   // the streamed batch stays in flight
        const int na = kWaves * m;
        uint32_t cand = 0u;
        if (tid < na) {
            const uint32_t a = sh.lead[tid];
            int ge = 0;
            for (int j = 0; j < na; j += 4) {
                const u32x4 q = *reinterpret_cast<const u32x4 *>(&sh.lead[j]);
#pragma unroll
                for (int e = 0; e < 4; ++e) ge += q[e] >= a ? 1 : 0;
            }
            cand = ge >= top_k ? a : 0u;   // the bound: the largest such key
        }
        if (wave * 64 < na) {
            cand = wave_max_u32(cand);
            if (lane == 0) atomicMax(&sh.lead_bound, cand);
        }
        lds_sync();
        prefix = sh.lead_bound;
    }
    if (!lead) {
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        // digit bits [shift, top): constants once the loop is unrolled
        const int top = 32 - pass * kDigitBits;
        const int bits = top - (32 - kKeyBits) < kDigitBits ? top - (32 - kKeyBits) : kDigitBits;
        const int shift = top - bits;
        const uint32_t nb = 1u << bits;
        for (int i = tid; i < (int)nb * kRep; i += kThreads) hist[i] = 0;
        opaque();
        __syncthreads();
        if constexpr (FILTER) {
            if ((mkey & pmask) == prefix) atomicAdd(&hist[((mkey >> shift) & (nb - 1)) * kRep + rep], 1u);
        } else {
            for_chunks([&](int64_t, const u32x4 &kc) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const uint32_t key = K::at(kc, e);
                    if ((key & pmask) == prefix)
                        atomicAdd(&hist[((key >> shift) & (nb - 1)) * kRep + rep], 1u);
                }
            });
        }
        __syncthreads();
        if (nb <= 256) {
            // thread t < nb sums digit nb-1-t (rotating the replica index keeps
            // a wave's lanes on different banks); an inclusive scan over t then
            // counts the candidates with digit >= nb-1-t: per wave first, then,
            // after a barrier every thread reaches, across the (at most four) waves
            const uint32_t d = nb - 1 - (uint32_t)(tid & 255);
            uint32_t h = 0, incl = 0;
            if (tid < (int)nb) {
#pragma unroll
                for (int r = 0; r < kRep; ++r) h += hist[d * kRep + ((r + tid) & (kRep - 1))];
                incl = wave_incl_scan(h);
                if ((tid & 63) == 63) wtot[tid >> 6] = incl;
            }
            __syncthreads();
            if (tid < (int)nb) {
                for (int w2 = 0; w2 < (tid >> 6); ++w2) incl += wtot[w2];
                if (incl - h < need && need <= incl) {   // the need-th largest has digit d
                    sel[0] = d;
                    sel[1] = incl - h;
                    sel[2] = h;
                }
            }
        } else {
            // thread t sums bins nb-1-t*bpt .. nb-bpt-t*bpt (largest digits
            // first); a block scan finds the thread whose bins hold the need-th
            // largest key, which then walks its bins
            const int bpt = (int)nb / kThreads;
            uint32_t hsum = 0;
            for (int j = 0; j < bpt; ++j) {
                const uint32_t d = nb - 1 - (uint32_t)(tid * bpt + j);
#pragma unroll
                for (int r = 0; r < kRep; ++r) hsum += hist[d * kRep + ((r + tid) & (kRep - 1))];
            }
            int total;
            const uint32_t before = (uint32_t)block_exclusive_scan((int)hsum, iscan, total);
            if (before < need && need <= before + hsum) {
                uint32_t above = before;
                for (int j = 0; j < bpt; ++j) {
                    const uint32_t d = nb - 1 - (uint32_t)(tid * bpt + j);
                    uint32_t h = 0;
#pragma unroll
                    for (int r = 0; r < kRep; ++r) h += hist[d * kRep + r];
                    if (above < need && need <= above + h) {
                        sel[0] = d;
                        sel[1] = above;
                        sel[2] = h;
                        break;
                    }
                    above += h;
                }
            }
        }
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= (nb - 1) << shift;
        need -= sel[1];
        // the candidates left (the same in every thread): stop early when the
        // counting sort takes them (kRankMax; measured on MI355X, this skips
        // the second pass over a 5 x 3072 row and beats the extra pass), or,
        // for a streamed row, when they fit the buffer (a read of the row
        // saved outweighs the larger sort); after the last digit, whenever
        // they fit the buffer
        const int cand = (top_k - (int)need) + (int)sel[2];
        const bool last = shift == 32 - kKeyBits;
        fits = cand <= kThreads;
        // the bound from the threads' maxima filters the whole row: it stops
        // only once few keys beyond the k needed share the selected bin
        const bool stop = last || (FILTER ? cand <= top_k + (top_k >> 3) + 8
                                          : (cand <= kRankMax || (HC == 0 && fits)));
        __syncthreads();                                        // sel is rewritten next pass
        if (stop) break;
    }
    }   // !lead
    // keys below the selected digits are either left to the sort (fits) or
    // fixed (bf16: the low 16 bits follow the sign), so one representative
    // key decides the comparisons
    const uint32_t kth = prefix;
    const uint32_t kth_mask = pmask;
    const int n_above = top_k - (int)need;   // keys strictly above kth
    const int n_tied = (int)sel[2];          // keys equal to kth under kth_mask

    // 2. gather the kept entries.  When everything above kth and every tie at
    //    kth fits the 1024-entry buffer, one pass appends them all in any
    //    order and the sort below ranks the ties by index; otherwise an
    //    ordered compaction keeps exactly the lowest-index `need` ties.
    if (tid == 0) n_gt = 0;
    __syncthreads();
    const bool gather_all = fits;
    int n_kept = gather_all ? n_above + n_tied : top_k;   // entries to sort
    if constexpr (FILTER) {
        // every entry of the row at or above the bound (a key passes exactly
        // when key >= kth: the bound's bits below its digits are zero, or, from
        // the waves' leading maxima, it is a key itself): the held part, then
        // the streamed rest, both tested as loaded (RawBound), and a chunk's
        // bit mask of its passing entries formed only when one passes.  A wave
        // adds its lanes' counts with one scan and reserves their slots with
        // one LDS atomic, and each lane then writes its entries, as keys, in
        // order.  (An atomic per passing entry, behind a branch per entry, took
        // about 4x as long; forming every entry's key before the test spent
        // about 12 vector operations per logit.)
        const int lane = tid & 63;
        const RawBound<IO> bnd(kth);
        auto append = [&](const uint32_t *masks, const u32x4 *raws, const int64_t *cs, int n) {
            int cnt = 0;
            for (int j = 0; j < n; ++j) cnt += __builtin_popcount(masks[j]);
            const int incl = wave_incl_scan(cnt);
            const int wave_total = __shfl(incl, 63, 64);
            if (wave_total == 0) return;                 // uniform over the wave
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&n_gt, (uint32_t)wave_total);
            base = (uint32_t)__shfl((int)base, 0, 64);
            uint32_t pos = base + (uint32_t)(incl - cnt);
            for (int j = 0; j < n; ++j) {
                uint32_t m = masks[j];
                while (m) {
                    const int e = __builtin_ctz(m);
                    m &= m - 1;
                    if (pos < (uint32_t)kThreads) {
                        ckey[pos] = raw_key<IO>(raws[j], e);
                        cidx[pos] = (int32_t)(cs[j] * VEC + e);
                    }
                    ++pos;
                }
            }
        };
        {
            uint32_t masks[HC];
            int64_t cs[HC];
#pragma unroll
            for (int j = 0; j < HC; ++j) {
                cs[j] = tid + (int64_t)j * kThreads;
                masks[j] = ((LONG || cs[j] < nchunks) && bnd.any(held[j])) ? bnd.mask(held[j]) : 0u;
            }
            append(masks, held, cs, HC);
        }
        auto filter_batch = [&](const u32x4 (&buf)[FB], int64_t c0) {
            uint32_t masks[FB];
            int64_t cs[FB];
#pragma unroll
            for (int j = 0; j < FB; ++j) {
                cs[j] = c0 + (int64_t)j * kThreads;
                masks[j] = (cs[j] < nchunks && bnd.any(buf[j])) ? bnd.mask(buf[j]) : 0u;
            }
            append(masks, buf, cs, FB);
        };
        // uniform trip count: every thread passes the same loads
        constexpr int64_t kB = (int64_t)FB * kThreads;   // chunks per batch
        // (the first two batches were issued with the held part)
        for (int64_t base = nheld; base < nchunks; base += 2 * kB) {
            if (base + kB < nchunks) load_batch(sb, base + kB + tid);
            filter_batch(sa, base + tid);
            if (base + 2 * kB < nchunks) load_batch(sa, base + 2 * kB + tid);
            if (base + kB < nchunks) filter_batch(sb, base + kB + tid);
        }
        __syncthreads();
        const uint32_t total = n_gt;
        if (total > (uint32_t)kThreads) {   // uniform: the buffer overflowed
            __syncthreads();                // every thread has read n_gt
            return false;
        }
        n_kept = (int)total;                // all of them are sorted; the first top_k are kept
    } else if (gather_all) {
        opaque();
        for_chunks([&](int64_t c, const u32x4 &kc) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t full = K::at(kc, e);
                if ((full & kth_mask) >= kth) {
                    const uint32_t at = atomicAdd(&n_gt, 1u);
                    ckey[at] = full;
                    cidx[at] = (int32_t)(c * VEC + e);
                }
            }
        });
    } else {
    int eq_taken = 0;
    opaque();
    // one block-wide step per 1024 chunks, so ties are ranked in index order
    auto compact = [&](int64_t base, const u32x4 &kc) {
        const int64_t c = base + tid;
        int n_eq = 0;
        if (c < nchunks) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t full = K::at(kc, e), key = full & kth_mask;
                if (key > kth) {
                    const uint32_t at = atomicAdd(&n_gt, 1u);
                    ckey[at] = full;
                    cidx[at] = (int32_t)(c * VEC + e);
                } else if (key == kth) {
                    ++n_eq;
                }
            }
        }
        int chunk_total;
        int r = eq_taken + block_exclusive_scan(n_eq, iscan, chunk_total);
        if (c < nchunks && n_eq > 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t full = K::at(kc, e);
                if ((full & kth_mask) == kth) {
                    if (r < (int)need) {
                        ckey[n_above + r] = full;
                        cidx[n_above + r] = (int32_t)(c * VEC + e);
                    }
                    ++r;
                }
            }
        }
        eq_taken += chunk_total;
    };
    if constexpr (HC > 0) {
#pragma unroll
        for (int j = 0; j < HC; ++j) {
            if ((int64_t)j * kThreads >= nheld) break;   // uniform: every thread stops together
            compact((int64_t)j * kThreads, held[j]);
        }
    } else {
        for (int64_t base = 0; base < nchunks; base += kThreads) {
            const int64_t c = base + tid;
            compact(base, c < nchunks ? K::from_raw(load16(x + c * VEC)) : u32x4{0, 0, 0, 0});
        }
    }
    }   // ordered compaction
    __syncthreads();

    // 3. sort of the kept entries: logit descending, index ascending.
    if (n_kept <= kRankMax) {
        // up to kRankMax entries: every entry's rank is counted by several
        // threads, each over one slice of the entries (thread t takes entry
        // t % n_kept and slice t / n_kept), the slices' counts meet in LDS,
        // and each entry then moves to its rank.  Measured on MI355X at
        // 256 x 151936 this replaced a bitonic network of ~28 barrier steps.
        const int per = kThreads / n_kept;                 // threads per entry (>= 1)
        // slices of whole 16-byte groups of entries; the last group is padded
        // with entries that rank after every real one
        const int npad = (n_kept + 3) & ~3;
        const int len = (((n_kept + per - 1) / per) + 3) & ~3;
        if (tid < n_kept) rank_of[tid] = 0;
        if (tid >= n_kept && tid < npad) {
            ckey[tid] = 0u;
            cidx[tid] = 0x7FFFFFFF;
        }
        __syncthreads();
        const uint32_t my_k = tid < n_kept ? ckey[tid] : 0u;
        const int32_t my_ix = tid < n_kept ? cidx[tid] : 0;
        if (tid < per * n_kept) {
            const int e = tid % n_kept, sl = tid / n_kept;
            const uint32_t ke = ckey[e];
            const int32_t ie = cidx[e];
            const int j1 = (sl + 1) * len < npad ? (sl + 1) * len : npad;
            int before = 0;
            for (int j = sl * len; j < j1; j += 4) {
                const u32x4 kj = *reinterpret_cast<const u32x4 *>(&ckey[j]);
                const u32x4 ij = *reinterpret_cast<const u32x4 *>(&cidx[j]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    before += (kj[q] > ke || (kj[q] == ke && (int32_t)ij[q] < ie)) ? 1 : 0;
            }
            if (before) atomicAdd(&rank_of[e], before);
        }
        __syncthreads();
        if (tid < n_kept) {
            const int r = rank_of[tid];
            ckey[r] = my_k;
            cidx[r] = my_ix;
        }
        __syncthreads();
    } else {
        // more entries: a bitonic network in LDS, a barrier per step
        int n = 64;
        while (n < n_kept) n <<= 1;
        if (tid >= n_kept && tid < n) {
            ckey[tid] = 0u;          // below every real key
            cidx[tid] = 0x7FFFFFFF;
        }
        __syncthreads();
        for (int size = 2; size <= n; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                if (tid < n) {
                    const int other = tid ^ stride;
                    if (other > tid) {
                        const uint32_t ka = ckey[tid], kb = ckey[other];
                        const int32_t ia = cidx[tid], ib = cidx[other];
                        const bool a_first = ka > kb || (ka == kb && ia < ib);
                        const bool up = (tid & size) == 0;
                        if (up != a_first) {
                            ckey[tid] = kb;
                            ckey[other] = ka;
                            cidx[tid] = ib;
                            cidx[other] = ia;
                        }
                    }
                }
                __syncthreads();
            }
        }
    }

    // 4. renormalised weights of the kept entries, prefix sums, inverse CDF:
    //    the first kept entry whose prefix exceeds u * total (the last one if
    //    rounding leaves u * total at or above the last prefix)
    const float lmax = value_of(ckey[0]);
    if (top_k <= 64) {
        // one wave holds every kept entry: lane shuffles and a ballot, no
        // block barrier (measured: 6.6 -> 5.9 us for a 5 x 3072 call)
        if (tid < 64) {
            const float w = tid < top_k ? expf((value_of(ckey[tid]) - lmax) * inv_temp) : 0.0f;
            const float cum = wave_incl_scan(w);
            const float total = __shfl(cum, top_k - 1, 64);
            const float thr = u[row] * total;
            const uint64_t m = __ballot(tid < top_k && cum > thr);
            if (tid == 0) token[row] = cidx[m ? __ffsll((unsigned long long)m) - 1 : top_k - 1];
        }
    } else {
        const float w = tid < top_k ? expf((value_of(ckey[tid]) - lmax) * inv_temp) : 0.0f;
        const float cum = block_inclusive_scan(w, fscan);
        csum[tid] = cum;
        if (tid == 0) pick = -1;
        __syncthreads();
        const float thr = u[row] * csum[top_k - 1];
        const float before = tid > 0 ? csum[tid - 1] : 0.0f;
        if (tid < top_k && cum > thr && (tid == 0 || before <= thr)) pick = cidx[tid];
        __syncthreads();
        if (tid == 0) token[row] = pick >= 0 ? pick : cidx[top_k - 1];
    }

    // optional full softmax row (never asked of a row filtered against a
    // bound, which keeps its chunks as loaded)
    if (!FILTER && probs) {
        opaque();
        float part = 0.0f;
        for_chunks([&](int64_t, const u32x4 &kc) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) part += expf((value_of(K::at(kc, e)) - lmax) * inv_temp);
        });
        part = wave_sum(part);
        if ((tid & 63) == 0) fscan[tid >> 6] = part;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) tot += fscan[wv];
        const float inv = 1.0f / tot;
        IO *p = probs + row * probs_stride;
        for_chunks([&](int64_t c, const u32x4 &kc) {
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = expf((value_of(K::at(kc, e)) - lmax) * inv_temp) * inv;
            store16(p + c * VEC, T::pack(o));
        });
    }
    return true;
}

template <typename IO, int CPT>
__global__ __launch_bounds__(kThreads) void topk_sample_kernel(
    int32_t *token, IO *probs, const IO *logits, int64_t vocab, int64_t row_stride,
    int64_t probs_stride, float inv_temp, int32_t top_k, const float *u) {
    __shared__ SampleShared sh;
    // the softmax output needs passes over the whole row anyway
    if (CPT >= 0 || probs == nullptr) {
        if (sample_row<IO, CPT>(sh, token, probs, logits, vocab, row_stride, probs_stride, inv_temp,
                                top_k, u))
            return;
    }
    if constexpr (CPT < 0)
        sample_row<IO, 0>(sh, token, probs, logits, vocab, row_stride, probs_stride, inv_temp,
                          top_k, u);
}

namespace {

template <typename IO, int CPT>
void launch_cpt(int32_t *token, void *probs, const void *logits, int64_t rows, int64_t vocab,
                int64_t row_stride, int64_t probs_stride, float inv_temp, int32_t top_k,
                const float *u, hipStream_t stream) {
    hipLaunchKernelGGL((topk_sample_kernel<IO, CPT>), dim3((unsigned)rows), dim3(kThreads), 0,
                       stream, token, (IO *)probs, (const IO *)logits, vocab, row_stride,
                       probs_stride, inv_temp, top_k, u);
}

template <typename IO>
void launch_typed(int32_t *token, void *probs, const void *logits, int64_t rows, int64_t vocab,
                  int64_t row_stride, int64_t probs_stride, float inv_temp, int32_t top_k,
                  const float *u, hipStream_t stream) {
    const int64_t nchunks = vocab / io_traits<IO>::VEC;
    const int64_t per_thread = (nchunks + kThreads - 1) / kThreads;
    // Token-only calls with top_k <= kLeadTopK over rows of at least one chunk
    // per thread are filtered against a bound (the long rows' path, with the
    // whole row held): measured on MI355X (graph-timed, inputs rotated past
    // the cache), 256 x 32000 bf16 11.9 -> 10.8 us, 256 x 65536 bf16 20.1 ->
    // 14.9 us.  Shorter rows keep the radix select over their held keys (too
    // few thread maxima for the bound).
    const bool bound = probs == nullptr && top_k <= kLeadTopK && nchunks >= kThreads;
#define NRS_TS(C) launch_cpt<IO, C>(token, probs, logits, rows, vocab, row_stride, probs_stride, \
                                    inv_temp, top_k, u, stream)
    if (per_thread <= 1) { if (bound) NRS_TS(-1); else NRS_TS(1); }
    else if (per_thread <= 2) { if (bound) NRS_TS(-2); else NRS_TS(2); }
    else if (per_thread <= 4) { if (bound) NRS_TS(-4); else NRS_TS(4); }
    else if (per_thread <= 8) { if (bound) NRS_TS(-8); else NRS_TS(8); }
    else NRS_TS(kLongRow);
#undef NRS_TS
}

}  // namespace

hipError_t launch_topk_sample(int32_t *token, void *probs, const void *logits, int64_t rows,
                              int64_t vocab, int64_t row_stride, int64_t probs_stride,
                              float temperature, int32_t top_k, const float *u, int dtype,
                              hipStream_t stream) {
    const float inv_temp = (float)(1.0 / (double)temperature);
    if (dtype == 0)
        launch_typed<float>(token, probs, logits, rows, vocab, row_stride, probs_stride, inv_temp,
                            top_k, u, stream);
    else
        launch_typed<__bf16>(token, probs, logits, rows, vocab, row_stride, probs_stride, inv_temp,
                             top_k, u, stream);
    return hipGetLastError();
}

}  // namespace nrs
