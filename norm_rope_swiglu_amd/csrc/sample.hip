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
// pass runs over the registers; longer rows are re-read (from the caches) by
// each pass.  (At 20 chunks per thread the registers spill and the kernel
// ran slower than streaming the row.)
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
    static constexpr int VEC = 4;
    __device__ static inline u32x4 from_raw(const u32x4 &raw) {
        u32x4 k;
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = key_of(__builtin_bit_cast(float, (unsigned)raw[i]));
        return k;
    }
    __device__ static inline uint32_t at(const u32x4 &k, int e) { return k[e]; }
};

template <> struct keys<__bf16> {
    static constexpr int VEC = 8;
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
}  // namespace

// CPT > 0: thread t holds the row's chunks t, t + 1024, ... (at most CPT of
// them) in registers; CPT == 0: every pass streams the row from memory.
template <typename IO, int CPT>
__global__ __launch_bounds__(kThreads) void topk_sample_kernel(
    int32_t *token, IO *probs, const IO *logits, int64_t vocab, int64_t row_stride,
    int64_t probs_stride, float inv_temp, int32_t top_k, const float *u) {
    using K = keys<IO>;
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    constexpr int kDigitBits = CPT > 0 ? 8 : 12;
    constexpr int kRep = CPT == 1 ? 8 : (CPT > 0 ? 32 : 4);
    static_assert((kRep << kDigitBits) <= kHistWords, "histogram fits");
    // bin-major: the replicas of a bin sit on kRep consecutive banks
    __shared__ uint32_t hist[kHistWords];
    __shared__ uint32_t wtot[4];
    __shared__ uint32_t sel[3];            // selected digit, count above it, count equal
    __shared__ int iscan[kWaves];
    __shared__ float fscan[kWaves];
    __shared__ __attribute__((aligned(16))) uint32_t ckey[kThreads];   // kept entries: key, index
    __shared__ __attribute__((aligned(16))) int32_t cidx[kThreads];
    __shared__ float csum[kThreads];       // prefix sums of the kept weights
    __shared__ int32_t rank_of[kThreads];  // ranks of the kept entries (up to kRankMax)
    __shared__ uint32_t n_gt;
    __shared__ int32_t pick;

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const IO *x = logits + row * row_stride;
    const int64_t nchunks = vocab / VEC;

    // the row's source: keys in registers (loaded here, all at once) or
    // memory (converted to keys as each pass reads it)
    u32x4 held[CPT > 0 ? CPT : 1];
    if constexpr (CPT > 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int64_t c = tid + (int64_t)j * kThreads;
            if (c < nchunks) held[j] = load16(x + c * VEC);
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) held[j] = K::from_raw(held[j]);
    }
    // Marks the held keys as rewritten (an empty asm statement that emits no
    // instruction), so each pass re-derives per-element keys from them instead
    // of the compiler keeping every pass's unpacked keys alive in registers.
    auto opaque = [&]() {
        if constexpr (CPT > 0) {
#pragma unroll
            for (int j = 0; j < CPT; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(held[j][i]));
        }
    };
    // f(c, keys) for every chunk c this thread owns, in increasing c
    auto for_chunks = [&](auto &&f) {
        if constexpr (CPT > 0) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int64_t c = tid + (int64_t)j * kThreads;
                if (c < nchunks) f(c, held[j]);
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
    //    streamed row, the 1024-entry gather buffer (with 12-bit digits this
    //    usually happens after the first pass, so a streamed row is read twice:
    //    once counted, once gathered).  The
    //    histograms keep replicas (indexed by lane) so lanes counting the same
    //    bin, common with peaky logits, split over several addresses.
    constexpr int kKeyBits = sizeof(IO) == 4 ? 32 : 16;   // bits that vary in a key
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)top_k;
    const uint32_t rep = tid & (kRep - 1);
    bool fits = false;
    constexpr int kPasses = (kKeyBits + kDigitBits - 1) / kDigitBits;
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
        for_chunks([&](int64_t, const u32x4 &kc) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t key = K::at(kc, e);
                if ((key & pmask) == prefix)
                    atomicAdd(&hist[((key >> shift) & (nb - 1)) * kRep + rep], 1u);
            }
        });
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
        const bool stop = last || cand <= kRankMax || (CPT == 0 && fits);
        __syncthreads();                                        // sel is rewritten next pass
        if (stop) break;
    }
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
    const int n_kept = gather_all ? n_above + n_tied : top_k;   // entries to sort
    if (gather_all) {
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
    if constexpr (CPT > 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            if ((int64_t)j * kThreads >= nchunks) break;   // uniform: every thread stops together
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

    // optional full softmax row
    if (probs) {
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
    const int64_t per_thread = (vocab / io_traits<IO>::VEC + kThreads - 1) / kThreads;
#define NRS_TS(C) launch_cpt<IO, C>(token, probs, logits, rows, vocab, row_stride, probs_stride, \
                                    inv_temp, top_k, u, stream)
    if (per_thread <= 1) NRS_TS(1);
    else if (per_thread <= 2) NRS_TS(2);
    else if (per_thread <= 4) NRS_TS(4);
    else if (per_thread <= 8) NRS_TS(8);
    else NRS_TS(0);
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
