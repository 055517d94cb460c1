// Multimodal rotary position embedding (M-RoPE), in place on q and k, gfx950.
//
// RoPE puts the position into Q and K as a rotation in the complex plane
// (forpes.ru post 233929, stage 2 "RoPE"); the multimodal variant named in the
// qwen3-tts-triton post (de.news.hada.io topic 27742, part 3) drives the
// frequency pairs from three position streams.  Pair j of a head couples
// elements j and j + D/2; pairs [0, s_t) follow the temporal stream,
// [s_t, s_t + s_h) the height stream and the rest the width stream; pair j
// turns by p * theta^(-2j/D).
//
// Structure: a block owns `tpb` consecutive tokens and one thread per
// (token, head, chunk) item; every item reads 16 bytes from each half of its
// head (elements j..j+VEC-1 and j+D/2..), rotates them and writes them back
// to the same place.  Each item owns its elements, so the in-place update has
// no read/write hazard.  The item's two loads are issued first, then the
// block builds its angle table (its position loads queue behind the item
// loads; loading the positions first measured no faster):
//   for every (token, pair) of the block the angle p * w_j is formed in fp64
//   (w_j computed on the host in fp64) and converted to turns, the nearest
//   whole turn is removed in fp64, and only the reduced fraction, |t| <= 1/2,
//   is rounded to fp32 for the hardware v_sin_f32 / v_cos_f32 (which take
//   turns).  The (cos, sin) table lives in LDS: one evaluation per token and
//   pair, shared by all n_q + n_kv heads of the token.
// q and k are addressed with their own token strides, so they may sit inside
// a packed qkv projection output.  mrope_wave_kernel below gives each 64-lane
// workgroup 64 consecutive chunks instead, one per lane, with the pair
// partner from another lane and a per-wave table; launch_mrope picks between
// the two by shape (measured).
#include "device.hpp"
#include "kernels.hpp"

namespace nrs {

namespace {
constexpr double kInvTwoPi = 0.15915494309189533577;  // 1 / (2 pi), fp64
constexpr int kMaxThreads = 1024;
// chunks in flight per thread in mrope_kv_narrow_kernel: two for streaming calls,
// one for small (latency-bound) calls, which spread over more threads instead
template <bool NT> constexpr int narrow_per_thread() { return NT ? 2 : 1; }
}  // namespace

// (cos, sin) of the angle p * w (w = w_j from the host in fp64): the product
// formed in fp64, converted to turns, the nearest whole turn removed in fp64
// (exact), and the fraction, |t| <= 1/2, rounded to fp32 for the hardware
// v_sin_f32 / v_cos_f32, which take turns: measured max abs error 1.3e-7 over
// [-1/2, 1/2) on MI355X.  Every kernel here forms its angles with this, so
// they all give the same bits.
__device__ inline f32x2 angle_cs(int32_t p, double w) {
    const double turns = ((double)p * w) * kInvTwoPi;
    const float t = (float)(turns - __builtin_rint(turns));
    return f32x2{__builtin_amdgcn_cosf(t), __builtin_amdgcn_sinf(t)};
}

// (cos, sin) of every (token, pair) of the block's tokens into LDS.
__device__ inline void build_angle_table(f32x2 *table, const int32_t *pos, int64_t pos_stride,
                                         int64_t tok0, int ntok, int half, int32_t sec_t,
                                         int32_t sec_th, const fastdiv &div_half,
                                         const mrope_freqs &fr) {
    const int n_ang = ntok * half;
    for (int e = threadIdx.x; e < n_ang; e += blockDim.x) {
        const int tl = (int)div((uint32_t)e, div_half);
        const int j = e - tl * half;
        const int s = j < sec_t ? 0 : (j < sec_th ? 1 : 2);
        table[e] = angle_cs(pos[s * pos_stride + tok0 + tl], fr.w[j]);
    }
}

// The frequencies w_j of a kernel whose first argument is its mrope_freqs,
// through an opaque global pointer to the kernel-argument segment: read as
// the struct, the compiler treats them as invariant and may move their loads
// behind the data loads (and taking the struct's address copies it to
// scratch).
typedef const __attribute__((address_space(1))) double gdouble;
__device__ inline gdouble *kernarg_freqs() {
    const void *ka = (const void *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ka));
    return (gdouble *)ka;
}

// Position and frequency of (cos, sin) entry e of the block's tokens (token
// tok0 + e / half, pair e % half).
__device__ inline void angle_input(int e, const int32_t *pos, int64_t pos_stride, int64_t tok0,
                                   int half, int32_t sec_t, int32_t sec_th,
                                   const fastdiv &div_half, gdouble *wg, int32_t &p, double &w) {
    const int tl = (int)div((uint32_t)e, div_half);
    const int j = e - tl * half;
    const int s = j < sec_t ? 0 : (j < sec_th ? 1 : 2);
    p = pos[s * pos_stride + tok0 + tl];
    w = wg[j];
}

// The block's table when each thread loaded the inputs of its first two
// entries (tid and tid + blockDim) ahead of its data: those two are formed
// outside any loop (a loop that may load made the compiler wait for every
// load, the data too, on entry), further entries load their own.
__device__ inline void build_angle_table_from(f32x2 *table, int n_ang, int32_t p0, double w0,
                                              int32_t p1, double w1, const int32_t *pos,
                                              int64_t pos_stride, int64_t tok0, int half,
                                              int32_t sec_t, int32_t sec_th,
                                              const fastdiv &div_half, gdouble *wg) {
    const int tid = threadIdx.x, nth = blockDim.x;
    if (tid < n_ang) table[tid] = angle_cs(p0, w0);
    if (tid + nth < n_ang) table[tid + nth] = angle_cs(p1, w1);
    for (int e = tid + 2 * nth; e < n_ang; e += nth) {
        int32_t p;
        double w;
        angle_input(e, pos, pos_stride, tok0, half, sec_t, sec_th, div_half, wg, p, w);
        table[e] = angle_cs(p, w);
    }
}

// Rotate one item: VEC pairs (a from the first half, b from the second).
template <typename IO>
__device__ inline void rotate_chunks(const f32x2 *tab, const u32x4 &lo, const u32x4 &hi,
                                     u32x4 &rlo, u32x4 &rhi) {
    using T = io_traits<IO>;
    constexpr int VEC = T::VEC;
    float a[VEC], b[VEC], ra[VEC], rb[VEC];
    T::unpack(lo, a);
    T::unpack(hi, b);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const f32x2 t = tab[e];
        ra[e] = __builtin_fmaf(a[e], t.x, -(b[e] * t.y));
        rb[e] = __builtin_fmaf(b[e], t.x, a[e] * t.y);
    }
    rlo = T::pack(ra);
    rhi = T::pack(rb);
}

template <typename IO, bool NT>
__global__ __launch_bounds__(kMaxThreads) void mrope_kernel(
    [[maybe_unused]] mrope_freqs fr, IO *q, IO *k, const int32_t *pos, int64_t pos_stride,
    int64_t tokens, int32_t n_q, int32_t head_dim, int64_t q_stride, int64_t k_stride,
    int32_t sec_t, int32_t sec_th, int32_t tpb, int32_t per_tok, int32_t cph, fastdiv div_half,
    fastdiv div_q_ipt, fastdiv div_k_ipt, fastdiv div_cph) {
    constexpr int VEC = io_traits<IO>::VEC;
    extern __shared__ f32x2 table[];  // [tpb][half] = (cos, sin)
    const int half = head_dim >> 1;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int64_t tok0 = (int64_t)blockIdx.x * tpb;
    const int ntok = (int)((tokens - tok0) < tpb ? (tokens - tok0) : tpb);
    const int items = ntok * per_tok;

    // where item i lives, and its slot in the table: the block's q items
    // first (token-major, so consecutive tokens' q rows are walked in one
    // run), then its k items
    const int q_items = ntok * n_q * cph;
    // the fastdiv fields by value: selecting between the two structs made the
    // compiler load the chosen one from the kernel arguments per lane, and
    // wait for it, before the data loads below
    const uint32_t qm = div_q_ipt.m, qs = div_q_ipt.s, km = div_k_ipt.m, ks = div_k_ipt.s;
    auto locate = [&](int i, int &tab) -> IO * {
        const bool is_q = i < q_items;
        const int j = is_q ? i : i - q_items;
        const int hpt = is_q ? n_q : per_tok / cph - n_q;   // heads per token
        const uint32_t m = is_q ? qm : km, sh = is_q ? qs : ks;
        const int tl = (int)((__umulhi((uint32_t)j, m) + (uint32_t)j) >> sh);
        const int rem = j - tl * hpt * cph;
        const int head = (int)div((uint32_t)rem, div_cph);
        const int c = rem - head * cph;
        const int64_t tok = tok0 + tl;
        IO *p = is_q ? q + tok * q_stride : k + tok * k_stride;
        tab = tl * half + c * VEC;
        return p + (int64_t)head * head_dim + c * VEC;
    };
    auto rotate_store = [&](IO *p, int tab, const u32x4 &lo, const u32x4 &hi) {
        u32x4 rlo, rhi;
        rotate_chunks<IO>(table + tab, lo, hi, rlo, rhi);
        store16_policy<NT>(p, rlo);
        store16_policy<NT>(p + half, rhi);
    };

    // 0. the position and frequency of this thread's first two (cos, sin)
    //    entries, loaded before its data: loads complete in order, so loaded
    //    after the data they would make the table, and the block barrier
    //    behind it, wait for this thread's data as well
    gdouble *const wg = kernarg_freqs();
    const int n_ang = ntok * half;
    int32_t pe0, pe1;
    double we0, we1;
    angle_input(tid < n_ang ? tid : 0, pos, pos_stride, tok0, half, sec_t, sec_th, div_half, wg,
                pe0, we0);   // (no branch: entry 0 always exists)
    angle_input(tid + nthreads < n_ang ? tid + nthreads : 0, pos, pos_stride, tok0, half, sec_t,
                sec_th, div_half, wg, pe1, we1);
    __builtin_amdgcn_sched_barrier(0);

    // 1. this thread's first item: its data loads, with no branch (a thread
    //    past the block's items re-reads its last item and stores nothing),
    //    so the table below waits for the position loads alone
    const bool has0 = tid < items;
    int tab0 = 0;
    IO *const p0 = locate(has0 ? tid : items - 1, tab0);
    const u32x4 lo0 = load16_policy<NT>(p0);
    const u32x4 hi0 = load16_policy<NT>(p0 + half);
    __builtin_amdgcn_sched_barrier(0);
    // (the positions are used from here on only, or the compiler converts
    // them before issuing the data loads, waiting for them there)
    asm volatile("" : "+v"(pe0), "+v"(pe1), "+v"(we0), "+v"(we1));

    // 2. the block's angle table
    build_angle_table_from(table, n_ang, pe0, we0, pe1, we1, pos, pos_stride, tok0, half, sec_t,
                           sec_th, div_half, wg);
    __syncthreads();

    // 3. rotate; blocks with more items than threads loop over the rest
    if (has0) rotate_store(p0, tab0, lo0, hi0);
    for (int i = tid + nthreads; i < items; i += nthreads) {
        int tab;
        IO *p = locate(i, tab);
        const u32x4 lo = load16_policy<NT>(p);
        const u32x4 hi = load16_policy<NT>(p + half);
        rotate_store(p, tab, lo, hi);
    }
}

// One 64-lane workgroup per 64 consecutive 16-byte chunks of q (or of k) in
// token-major order, one chunk per lane.  Measured on MI355X, a copy moving
// one 1 KiB piece per 64-thread workgroup, consecutive pieces going to
// consecutive XCDs, streams faster than any pattern that hands an XCD 2 KiB
// or more at a time (134 MB per buffer: 81% of 8 TB/s against 77%); the
// token-blocked kernels above hand each workgroup whole tokens.  So here a
// wave is the unit: a lane's pair partner (head_dim / 2 elements on) sits
// CPH lanes away in the same wave and arrives by a lane swizzle (chunk
// groups of a head are 2 * CPH lanes, aligned, since a wave starts at a
// multiple of 64 chunks and a token holds whole heads), and the wave builds
// the (cos, sin) entries of its own tokens in its own LDS slice with
// angle_cs (so the results are those of the kernels above, bit for bit).  A
// wave's chunks never mix q and k: k's waves start on a fresh wave.  Chunk
// indices are 32-bit: the launcher splits the tokens into slabs.
template <typename IO, bool NT, int CPH>
__global__ __launch_bounds__(64) void mrope_wave_kernel(
    [[maybe_unused]] mrope_freqs fr, IO *q, IO *k, const int32_t *pos, int64_t pos_stride, int32_t tokens,
    int32_t half, int64_t q_stride, int64_t k_stride, int32_t sec_t, int32_t sec_th,
    int32_t q_cpt, int32_t k_cpt, int32_t q_waves, fastdiv div_q_cpt, fastdiv div_k_cpt,
    fastdiv div_half) {
    constexpr int VEC = io_traits<IO>::VEC;
    constexpr int CPHEAD = 2 * CPH;
    static_assert(CPH >= 1 && CPH <= 32 && (CPH & (CPH - 1)) == 0, "chunks per half-head");
    using T = io_traits<IO>;
    extern __shared__ f32x2 table[];   // [tokens of this wave][half] = (cos, sin)
    const int lane = threadIdx.x;
    const bool is_q = (int32_t)blockIdx.x < q_waves;
    const int32_t cpt = is_q ? q_cpt : k_cpt;
    const fastdiv dv = is_q ? div_q_cpt : div_k_cpt;    // by value: a select, no stack copy
    IO *const base = is_q ? q : k;
    const int64_t stride = is_q ? q_stride : k_stride;
    const int32_t n = tokens * cpt;                         // chunks of this tensor
    const int32_t c0 = ((int32_t)blockIdx.x - (is_q ? 0 : q_waves)) * 64;

    // 1. the position and frequency of this lane's first (cos, sin) entry,
    //    then this lane's chunk: the table is built while the chunk is in
    //    flight (loads complete in order, so position loads issued after the
    //    data would wait for it)
    const int32_t t_first = (int32_t)div((uint32_t)c0, dv);
    const int32_t t_last = (int32_t)div((uint32_t)min(c0 + 63, n - 1), dv);
    const int n_ang = (t_last - t_first + 1) * half;   // entries of the wave's tokens
    // the frequencies through the kernel-argument pointer (kernarg_freqs):
    // read as fr.w[j], the compiler sank the first load behind the data load
    gdouble *const wg = kernarg_freqs();
    auto entry = [&](int e, int32_t &p_out, double &w_out) {
        const int tt = (int)div((uint32_t)e, div_half);
        const int j = e - tt * half;
        const int s = j < sec_t ? 0 : (j < sec_th ? 1 : 2);
        p_out = pos[s * pos_stride + t_first + tt];
        w_out = wg[j];
    };
    int32_t p0;
    double w0;
    entry(lane < n_ang ? lane : 0, p0, w0);   // no branch: entry 0 always exists
    __builtin_amdgcn_sched_barrier(0);
    // no branch around the load (a lane past the end re-reads the last chunk
    // and stores nothing), so the table below waits for its own loads only
    const int32_t c = min(c0 + lane, n - 1);
    const int32_t tl = (int32_t)div((uint32_t)c, dv);
    const int32_t rem = c - tl * cpt;                        // chunk within the token's heads
    const int cc = rem & (CPHEAD - 1);                       // chunk within the head
    IO *const p = base + (int64_t)tl * stride + (int64_t)rem * VEC;
    const u32x4 own = load16_policy<NT>(p);
    __builtin_amdgcn_sched_barrier(0);
    // the first entry's position and frequency are used from here on only:
    // without this the compiler converted the position to fp64 before issuing
    // the data load (waiting for the position load there)
    asm volatile("" : "+v"(p0), "+v"(w0));

    // 2. the (cos, sin) entries of the wave's tokens [t_first, t_last]
    for (int e = lane; e < n_ang; e += 64) {
        int32_t pe = p0;
        double we = w0;
        if (e != lane) entry(e, pe, we);
        table[e] = angle_cs(pe, we);
    }
    __syncthreads();   // one wave: orders its own LDS writes before the reads

    // 3. the partner half-chunk from lane ^ CPH, rotate, store
    u32x4 other;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (CPH < 32)
            other[e] = (unsigned)__builtin_amdgcn_ds_swizzle((int)own[e], (CPH << 10) | 0x1F);
        else
            other[e] = (unsigned)__shfl_xor((int)own[e], 32, 64);
    }
    if (c0 + lane >= n) return;
    const bool upper = cc >= CPH;
    const f32x2 *tab = table + (tl - t_first) * half + (cc & (CPH - 1)) * VEC;
    float a[VEC], b[VEC], o[VEC];
    T::unpack(own, a);
    T::unpack(other, b);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const f32x2 cs = tab[e];
        // lower half: a cos - b sin; upper half (own = b, other = a): b cos + a sin
        o[e] = upper ? __builtin_fmaf(a[e], cs.x, b[e] * cs.y)
                     : __builtin_fmaf(a[e], cs.x, -(b[e] * cs.y));
    }
    store16_policy<NT>(p, T::pack(o));
}

// M-RoPE fused with the KV-cache append ("Optimising autoregressive speech
// models", "Custom Triton kernels", kernel 3: each new K, V head vector goes
// to its cache at [head][position][:]).  Here every sequence owns a cache
// [n_kv][max_seq][head_dim] and each token names its sequence and slot.  q is
// rotated in place; k is rotated straight into the k cache (k itself is only
// read, so the rotated k makes a single trip to memory); v is copied into the
// v cache.  Items are ordered q, then k, then v per block, two 16-byte chunks
// (a pair-half each) per item.  All loads are issued before the angle table
// is built, the data first and the token's sequence index and slot after it,
// so no load waits on another (with the slot read first, the data loads had
// to wait for it).  A token whose sequence index or slot is out of range
// writes no cache entry.
template <typename IO, bool NT>
__global__ __launch_bounds__(kMaxThreads) void mrope_kv_kernel(
    IO *q, const IO *k, const IO *v, const int32_t *pos, int64_t pos_stride, int64_t tokens,
    int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t q_stride, int64_t k_stride,
    int64_t v_stride, int32_t sec_t, int32_t sec_th, int32_t tpb, int32_t cph, fastdiv div_half,
    fastdiv div_q_ipt, fastdiv div_kv_ipt, fastdiv div_cph, IO *k_cache, IO *v_cache,
    const int32_t *seq_idx, const int32_t *slot, int64_t n_seqs, int64_t max_seq,
    mrope_freqs fr) {
    constexpr int VEC = io_traits<IO>::VEC;
    extern __shared__ f32x2 table[];  // [tpb][half] = (cos, sin)
    const int half = head_dim >> 1;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int64_t tok0 = (int64_t)blockIdx.x * tpb;
    const int ntok = (int)((tokens - tok0) < tpb ? (tokens - tok0) : tpb);
    const int q_items = ntok * n_q * cph;
    const int kv_items = ntok * n_kv * cph;
    const int items = q_items + 2 * kv_items;

    // item i -> its source (elements j.. of the pair-halves), kind (0 q, 1 k,
    // 2 v), token, head and chunk; the fastdiv fields are taken by value
    // (selecting between structs by address put one on the stack)
    const uint32_t qm = div_q_ipt.m, qs = div_q_ipt.s, kvm = div_kv_ipt.m, kvs = div_kv_ipt.s;
    auto locate = [&](int i, int &kind, int64_t &tok, int &head, int &c) -> const IO * {
        kind = i < q_items ? 0 : (i < q_items + kv_items ? 1 : 2);
        const uint32_t j = (uint32_t)(kind == 0 ? i : (kind == 1 ? i - q_items : i - q_items - kv_items));
        const uint32_t m = kind == 0 ? qm : kvm, sh = kind == 0 ? qs : kvs;
        const int tl = (int)((__umulhi(j, m) + j) >> sh);
        const int rem = (int)j - tl * (kind == 0 ? n_q : n_kv) * cph;
        head = (int)div((uint32_t)rem, div_cph);
        c = rem - head * cph;
        tok = tok0 + tl;
        const int64_t off = (int64_t)head * head_dim + c * VEC;
        return (kind == 0 ? q + tok * q_stride : (kind == 1 ? k + tok * k_stride : v + tok * v_stride)) + off;
    };
    // destination of an item once its token's sequence index and slot are in
    // (nullptr: out of range, nothing written)
    auto dest = [&](const IO *src, int kind, int head, int c, int64_t b, int64_t s) -> IO * {
        if (kind == 0) return const_cast<IO *>(src);
        if (b < 0 || b >= n_seqs || s < 0 || s >= max_seq) return nullptr;
        return (kind == 1 ? k_cache : v_cache) + ((b * n_kv + head) * max_seq + s) * head_dim + c * VEC;
    };
    auto finish = [&](IO *dst, int tab, bool rotate, const u32x4 &lo, const u32x4 &hi) {
        u32x4 olo = lo, ohi = hi;
        if (rotate) rotate_chunks<IO>(table + tab, lo, hi, olo, ohi);
        store16_policy<NT>(dst, olo);
        store16_policy<NT>(dst + half, ohi);
    };

    // 1. this thread's first item: its two loads (a token's k and v exist
    //    whatever its cache slot), then its token's sequence index and slot,
    //    with no wait between them
    const IO *s0 = nullptr;
    int kind0 = 0, head0 = 0, c0 = 0;
    int64_t t0 = tok0;
    u32x4 lo0 = u32x4{0, 0, 0, 0}, hi0 = u32x4{0, 0, 0, 0};
    if (tid < items) {
        s0 = locate(tid, kind0, t0, head0, c0);
        lo0 = load16_policy<NT>(s0);
        hi0 = load16_policy<NT>(s0 + half);
    }
    const int64_t b0 = seq_idx[t0], sl0 = slot[t0];   // t0 = tok0 for idle threads: no branch

    // 2. the block's angle table (here the position loads follow the data:
    //    loading them first, as mrope_kernel does, measured no faster at
    //    32768 tokens x 16 q / 8 kv heads of 128)
    build_angle_table(table, pos, pos_stride, tok0, ntok, half, sec_t, sec_th, div_half, fr);
    __syncthreads();

    // 3. rotate or copy; blocks with more items than threads loop over the rest
    if (s0) {
        IO *d0 = dest(s0, kind0, head0, c0, b0, sl0);
        if (d0) finish(d0, (int)(t0 - tok0) * half + c0 * VEC, kind0 != 2, lo0, hi0);
    }
    for (int i = tid + nthreads; i < items; i += nthreads) {
        int kind, head, c;
        int64_t tok;
        const IO *src = locate(i, kind, tok, head, c);
        const u32x4 lo = load16_policy<NT>(src);
        const u32x4 hi = load16_policy<NT>(src + half);
        IO *dst = dest(src, kind, head, c, seq_idx[tok], slot[tok]);
        if (dst) finish(dst, (int)(tok - tok0) * half + c * VEC, kind != 2, lo, hi);
    }
}

// The KV-cache append for half-heads under a cache line: a chunk-per-lane
// layout (consecutive lanes, consecutive 16-byte chunks; the pair partner by
// ds_swizzle) over the items of mrope_kv_kernel:
// q chunks rotated in place, k chunks rotated into the k cache, v chunks
// copied into the v cache, in that order per block.  A token whose sequence
// index or slot is out of range writes no cache chunk.
template <typename IO, bool NT, int CPH>
__global__ __launch_bounds__(kMaxThreads) void mrope_kv_narrow_kernel(
    IO *q, const IO *k, const IO *v, const int32_t *pos, int64_t pos_stride, int64_t tokens,
    int32_t n_kv, int32_t head_dim, int64_t q_stride, int64_t k_stride, int64_t v_stride,
    int32_t sec_t, int32_t sec_th, int32_t tpb, int32_t q_cpt, int32_t kv_cpt, fastdiv div_half,
    fastdiv div_q_cpt, fastdiv div_kv_cpt, IO *k_cache, IO *v_cache, const int32_t *seq_idx,
    const int32_t *slot, int64_t n_seqs, int64_t max_seq, mrope_freqs fr) {
    constexpr int VEC = io_traits<IO>::VEC;
    constexpr int CPHEAD = 2 * CPH;                          // chunks per head
    constexpr int kSwz = (CPH << 10) | 0x1F;                 // bitmask mode: lane xor CPH
    static_assert(CPH == 1 || CPH == 2 || CPH == 4, "a head's chunk group must tile a wave");
    using T = io_traits<IO>;
    extern __shared__ f32x2 table[];  // [tpb][half] = (cos, sin)
    const int half = head_dim >> 1;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;   // a multiple of 64
    const int64_t tok0 = (int64_t)blockIdx.x * tpb;
    const int ntok = (int)((tokens - tok0) < tpb ? (tokens - tok0) : tpb);
    const int q_items = ntok * q_cpt;
    const int kv_items = ntok * kv_cpt;
    const int items = q_items + 2 * kv_items;

    // item i -> its source chunk, kind (0 q, 1 k, 2 v), token, chunk within
    // the token's heads, table slot and half; the fastdiv fields are taken by
    // value (selecting between the two structs by address put one on the stack)
    const uint32_t qm = div_q_cpt.m, qs = div_q_cpt.s, kvm = div_kv_cpt.m, kvs = div_kv_cpt.s;
    auto locate = [&](int i, int &kind, int64_t &tok, int &rem, int &tab, bool &upper) -> const IO * {
        kind = i < q_items ? 0 : (i < q_items + kv_items ? 1 : 2);
        const uint32_t j = (uint32_t)(kind == 0 ? i : (kind == 1 ? i - q_items : i - q_items - kv_items));
        const uint32_t m = kind == 0 ? qm : kvm, sh = kind == 0 ? qs : kvs;
        const int tl = (int)((__umulhi(j, m) + j) >> sh);
        rem = (int)j - tl * (kind == 0 ? q_cpt : kv_cpt);
        const int cc = rem & (CPHEAD - 1);                       // chunk within the head
        tok = tok0 + tl;
        upper = cc >= CPH;
        tab = tl * half + (cc & (CPH - 1)) * VEC;
        return kind == 0 ? q + tok * q_stride + (int64_t)rem * VEC
                         : (kind == 1 ? k + tok * k_stride : v + tok * v_stride) + (int64_t)rem * VEC;
    };
    // every lane of the wave runs this (the swizzle reads other lanes); dst
    // nullptr stores nothing
    auto finish = [&](IO *dst, int tab, bool upper, bool rotate, const u32x4 &own) {
        u32x4 other;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            other[e] = (unsigned)__builtin_amdgcn_ds_swizzle((int)own[e], kSwz);
        if (!dst) return;
        u32x4 out = own;
        if (rotate) {
            float a[VEC], b[VEC], o[VEC];
            T::unpack(own, a);
            T::unpack(other, b);
            const f32x2 *t = table + tab;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const f32x2 cs = t[e];
                o[e] = upper ? __builtin_fmaf(a[e], cs.x, b[e] * cs.y)
                             : __builtin_fmaf(a[e], cs.x, -(b[e] * cs.y));
            }
            out = T::pack(o);
        }
        store16_policy<NT>(dst, out);
    };

    // rounds of U chunks per thread: every source chunk is loaded (a token's
    // k and v exist whatever its cache slot), then the sequence index and slot
    // of the k and v chunks, so no load waits on another before the table
    constexpr int U = narrow_per_thread<NT>();
    for (int base = 0; base < items; base += U * nthreads) {
        const IO *src[U];
        int kind[U], rem[U], tab[U];
        int64_t tok[U], sb[U], ss[U];
        bool up[U];
        u32x4 val[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * nthreads + tid;
            src[u] = nullptr;
            kind[u] = rem[u] = tab[u] = 0;
            tok[u] = tok0;
            up[u] = false;
            val[u] = u32x4{0, 0, 0, 0};
            if (i < items) {
                src[u] = locate(i, kind[u], tok[u], rem[u], tab[u], up[u]);
                val[u] = load16_policy<NT>(src[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {   // unconditional (tok0 stands in for idle lanes): no branch
            sb[u] = seq_idx[tok[u]];    // between the loads, so all of them are in flight together
            ss[u] = slot[tok[u]];
        }
        if (base == 0) {   // uniform: every thread takes the barrier
            build_angle_table(table, pos, pos_stride, tok0, ntok, half, sec_t, sec_th, div_half,
                              fr);
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            IO *dst = nullptr;
            if (src[u]) {
                if (kind[u] == 0) {
                    dst = const_cast<IO *>(src[u]);
                } else if (sb[u] >= 0 && sb[u] < n_seqs && ss[u] >= 0 && ss[u] < max_seq) {
                    const int head = rem[u] / CPHEAD, cc = rem[u] & (CPHEAD - 1);
                    dst = (kind[u] == 1 ? k_cache : v_cache) +
                          ((sb[u] * n_kv + head) * max_seq + ss[u]) * head_dim + cc * VEC;
                }
            }
            finish(dst, tab[u], up[u], kind[u] != 2, val[u]);
        }
    }
}

hipError_t launch_mrope_kv(void *q, const void *k, const void *v, const int32_t *pos,
                           int64_t pos_stride, int64_t tokens, int32_t n_q, int32_t n_kv,
                           int32_t head_dim, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                           int32_t sec_t, int32_t sec_h, const mrope_freqs &fr, void *k_cache,
                           void *v_cache, const int32_t *seq_idx, const int32_t *slot,
                           int64_t n_seqs, int64_t max_seq, int dtype, hipStream_t stream) {
    const int half = head_dim / 2;
    const int vec = dtype == 0 ? 4 : 8;
    const int cph = half / vec;
    const int per_tok = (n_q + 2 * n_kv) * cph;
    const bool nt = tokens * (long long)(2 * n_q + 4 * n_kv) * head_dim * (dtype == 0 ? 4 : 2) >=
                    kStreamBytes;
    if (cph == 1 || cph == 2 || cph == 4) {
        // half-heads under a cache line: mrope_kv_narrow_kernel, two chunks
        // per thread (a block's width apart) in streaming calls, one in small
        // ones, and about 512 threads' worth of whole tokens per block
        const int cpt = 2 * per_tok;
        const int u = nt ? narrow_per_thread<true>() : narrow_per_thread<false>();
        int tpb = nt ? 512 * u / cpt : 1;
        if (tpb < 1) tpb = 1;
        const int per_block = (tpb * cpt + u - 1) / u;
        int threads = ((per_block + 63) / 64) * 64;
        if (threads > kMaxThreads) threads = kMaxThreads;
        const int64_t blocks = (tokens + tpb - 1) / tpb;
        const size_t lds = (size_t)tpb * half * sizeof(f32x2);
        const int q_cpt = 2 * n_q * cph, kv_cpt = 2 * n_kv * cph;
        const fastdiv dh = make_fastdiv((uint32_t)half),
                      dq = make_fastdiv((uint32_t)(q_cpt > 0 ? q_cpt : 1)),
                      dkv = make_fastdiv((uint32_t)(kv_cpt > 0 ? kv_cpt : 1));
        const dim3 grid((unsigned)blocks), block(threads);
#define NRS_KV_NARROW(IO, NT, C)                                                                 \
    hipLaunchKernelGGL((mrope_kv_narrow_kernel<IO, NT, C>), grid, block, lds, stream, (IO *)q,   \
                       (const IO *)k, (const IO *)v, pos, pos_stride, tokens, n_kv, head_dim,    \
                       q_stride, k_stride, v_stride, sec_t, sec_t + sec_h, tpb, q_cpt, kv_cpt,   \
                       dh, dq, dkv, (IO *)k_cache, (IO *)v_cache, seq_idx, slot, n_seqs,         \
                       max_seq, fr)
#define NRS_KV_NARROW_C(IO, NT)                                                                  \
    do {                                                                                         \
        if (cph == 1) NRS_KV_NARROW(IO, NT, 1);                                                  \
        else if (cph == 2) NRS_KV_NARROW(IO, NT, 2);                                             \
        else NRS_KV_NARROW(IO, NT, 4);                                                           \
    } while (0)
        if (dtype == 0) {
            if (nt) NRS_KV_NARROW_C(float, true);
            else NRS_KV_NARROW_C(float, false);
        } else {
            if (nt) NRS_KV_NARROW_C(__bf16, true);
            else NRS_KV_NARROW_C(__bf16, false);
        }
#undef NRS_KV_NARROW_C
#undef NRS_KV_NARROW
        return hipGetLastError();
    }
    // as for M-RoPE, small calls take one token per block (measured at the
    // 5-token decode step: 2.77 -> 2.55 us per call), and tokens of at most 64
    // items aim at ~256 threads (H = 512 bf16 at 32768 tokens: 7% faster).
    // Tokens of 65-256 items aim at 1024 threads, so each kv head's cache rows
    // are written 4 slots (1 KiB) at a time instead of 2: measured at 32768
    // tokens, bf16 head_dim 128, H = 2048 89.3 -> 86.8 us, H = 1024 the same
    // (47.3 -> 47.1 us); H = 4096 (512 items a token) 2% slower with 2 tokens
    // a block, and 8 tokens a block (a second pass over the items) slower at
    // every width.
    int tpb = nt ? (per_tok <= 64 ? 256 : (per_tok <= 256 ? 1024 : 512)) / per_tok : 1;
    if (tpb < 1) tpb = 1;
    int threads = ((tpb * per_tok + 63) / 64) * 64;
    if (threads > kMaxThreads) threads = kMaxThreads;
    const int64_t blocks = (tokens + tpb - 1) / tpb;
    const size_t lds = (size_t)tpb * half * sizeof(f32x2);
    const int q_ipt = n_q * cph, kv_ipt = n_kv * cph;
    const fastdiv dh = make_fastdiv((uint32_t)half),
                  dq = make_fastdiv((uint32_t)(q_ipt > 0 ? q_ipt : 1)),
                  dkv = make_fastdiv((uint32_t)(kv_ipt > 0 ? kv_ipt : 1)),
                  dc = make_fastdiv((uint32_t)cph);
    const dim3 grid((unsigned)blocks), block(threads);
#define NRS_MROPE_KV(IO, NT)                                                                    \
    hipLaunchKernelGGL((mrope_kv_kernel<IO, NT>), grid, block, lds, stream, (IO *)q,            \
                       (const IO *)k, (const IO *)v, pos, pos_stride, tokens, n_q, n_kv,         \
                       head_dim, q_stride, k_stride, v_stride, sec_t, sec_t + sec_h, tpb, cph,   \
                       dh, dq, dkv, dc, (IO *)k_cache, (IO *)v_cache, seq_idx, slot, n_seqs,     \
                       max_seq, fr)
    if (dtype == 0) {
        if (nt) NRS_MROPE_KV(float, true);
        else NRS_MROPE_KV(float, false);
    } else {
        if (nt) NRS_MROPE_KV(__bf16, true);
        else NRS_MROPE_KV(__bf16, false);
    }
#undef NRS_MROPE_KV
    return hipGetLastError();
}

namespace {

// mrope_wave_kernel over token slabs whose chunk counts fit 31 bits; heads of
// 2 * cph chunks, cph a power of two up to 32.
template <typename IO, bool NT>
void launch_mrope_wave(IO *q, IO *k, const int32_t *pos, int64_t pos_stride, int64_t tokens,
                       int32_t n_q, int32_t n_kv, int32_t half, int cph, int64_t q_stride,
                       int64_t k_stride, int32_t sec_t, int32_t sec_th, const mrope_freqs &fr,
                       hipStream_t stream) {
    const int32_t q_cpt = 2 * n_q * cph, k_cpt = 2 * n_kv * cph;
    const int32_t max_cpt = q_cpt > k_cpt ? q_cpt : k_cpt;
    const int32_t min_cpt = q_cpt == 0 ? k_cpt : (k_cpt == 0 ? q_cpt : (q_cpt < k_cpt ? q_cpt : k_cpt));
    // a wave's 64 chunks touch at most 63 / cpt + 2 tokens
    const size_t lds = (size_t)(63 / min_cpt + 2) * half * sizeof(f32x2);
    const int64_t slab = ((int64_t)1 << 30) / max_cpt;
    const fastdiv dq = make_fastdiv((uint32_t)(q_cpt > 0 ? q_cpt : 1)),
                  dk = make_fastdiv((uint32_t)(k_cpt > 0 ? k_cpt : 1)),
                  dh = make_fastdiv((uint32_t)half);
    for (int64_t t0 = 0; t0 < tokens; t0 += slab) {
        const int32_t nt = (int32_t)(tokens - t0 < slab ? tokens - t0 : slab);
        const int32_t q_waves = (int32_t)(((int64_t)nt * q_cpt + 63) / 64);
        const int32_t k_waves = (int32_t)(((int64_t)nt * k_cpt + 63) / 64);
        const dim3 grid((unsigned)(q_waves + k_waves)), block(64);
#define NRS_MROPE_WAVE(C)                                                                         \
    hipLaunchKernelGGL((mrope_wave_kernel<IO, NT, C>), grid, block, lds, stream, fr,             \
                       q + t0 * q_stride, k + t0 * k_stride, pos + t0, pos_stride, nt, half,     \
                       q_stride, k_stride, sec_t, sec_th, q_cpt, k_cpt, q_waves, dq, dk, dh)
        switch (cph) {
            case 1: NRS_MROPE_WAVE(1); break;
            case 2: NRS_MROPE_WAVE(2); break;
            case 4: NRS_MROPE_WAVE(4); break;
            case 8: NRS_MROPE_WAVE(8); break;
            case 16: NRS_MROPE_WAVE(16); break;
            default: NRS_MROPE_WAVE(32); break;
        }
#undef NRS_MROPE_WAVE
    }
}

}  // namespace

hipError_t launch_mrope(void *q, void *k, const int32_t *pos, int64_t pos_stride, int64_t tokens,
                        int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t q_stride,
                        int64_t k_stride, int32_t sec_t, int32_t sec_h, const mrope_freqs &fr,
                        int dtype, hipStream_t stream) {
    const int half = head_dim / 2;
    const int vec = dtype == 0 ? 4 : 8;
    const int cph = half / vec;
    const int per_tok = (n_q + n_kv) * cph;
    const bool nt = 2 * tokens * (long long)(n_q + n_kv) * head_dim * (dtype == 0 ? 4 : 2) >=
                    kStreamBytes;
    // One wave per 64 chunks (mrope_wave_kernel) where its pairing works (a
    // power-of-two number of chunks per half-head, a head within 64 lanes)
    // and it measured faster: fp32, half-heads of 1, 2 or 4 chunks (bf16
    // head_dim <= 64), and small calls.  Measured against the token-blocked
    // kernels on one MI355X (graph-timed, inputs rotated past the cache, 32768
    // tokens): fp32 head_dim 64 and 128 2-5% faster at hidden 512-4096, bf16
    // head_dim 64 2-6% faster; the 5-token decode op set (28 layers) 169.8 ->
    // 165.8 us per replay.  Streaming bf16 calls with head_dim 128 were 1-5%
    // slower with it (also with two chunks per lane) and keep mrope_kernel,
    // as do fp32 head_dim 512 and half-heads of 3, 5, 6 or 7 chunks.
    const bool pow2 = (cph & (cph - 1)) == 0 && cph <= 32;
    if (pow2 && (dtype == 0 || cph <= 4 || !nt)) {
        if (dtype == 0) {
            if (nt) launch_mrope_wave<float, true>((float *)q, (float *)k, pos, pos_stride, tokens, n_q, n_kv, half, cph, q_stride, k_stride, sec_t, sec_t + sec_h, fr, stream);
            else launch_mrope_wave<float, false>((float *)q, (float *)k, pos, pos_stride, tokens, n_q, n_kv, half, cph, q_stride, k_stride, sec_t, sec_t + sec_h, fr, stream);
        } else {
            if (nt) launch_mrope_wave<__bf16, true>((__bf16 *)q, (__bf16 *)k, pos, pos_stride, tokens, n_q, n_kv, half, cph, q_stride, k_stride, sec_t, sec_t + sec_h, fr, stream);
            else launch_mrope_wave<__bf16, false>((__bf16 *)q, (__bf16 *)k, pos, pos_stride, tokens, n_q, n_kv, half, cph, q_stride, k_stride, sec_t, sec_t + sec_h, fr, stream);
        }
        return hipGetLastError();
    }
    // about 512 items (threads) per block, whole tokens only; one item per
    // thread unless a single token has more than kMaxThreads items.  Small
    // (latency-bound) calls take one token per block: measured at the 5-token
    // decode step, spreading the tokens over more CUs shortens the kernel by
    // ~0.16 us.
    // tokens of at most 64 items (e.g. 4 q + 2 kv heads of 128 in bf16) aim at
    // ~256 threads a block: measured at 32768 tokens, H = 512 bf16 5% faster
    // than ~512 (4 tokens a block instead of 8)
    int tpb = nt ? (per_tok <= 64 ? 256 : 512) / per_tok : 1;
    if (tpb < 1) tpb = 1;
    // the most tokens up to that whose items fill whole waves (measured at
    // 32768 tokens: H = 512 and 1024 bf16 2.5% faster with 8 and 4 tokens a
    // block than with 10 and 5, which leave half a wave idle)
    for (int t = tpb; t >= 1; --t) {
        if ((t * per_tok) % 64 == 0) {
            tpb = t;
            break;
        }
    }
    int threads = ((tpb * per_tok + 63) / 64) * 64;
    if (threads > kMaxThreads) threads = kMaxThreads;
    const int64_t blocks = (tokens + tpb - 1) / tpb;
    const size_t lds = (size_t)tpb * half * sizeof(f32x2);
    // items per token of q and of k (a count of 0 never reaches a division)
    const int q_ipt = n_q * cph, k_ipt = n_kv * cph;
    const fastdiv dh = make_fastdiv((uint32_t)half),
                  dq = make_fastdiv((uint32_t)(q_ipt > 0 ? q_ipt : 1)),
                  dk = make_fastdiv((uint32_t)(k_ipt > 0 ? k_ipt : 1)), dc = make_fastdiv((uint32_t)cph);
    const dim3 grid((unsigned)blocks), block(threads);
#define NRS_MROPE(IO, NT)                                                                        \
    hipLaunchKernelGGL((mrope_kernel<IO, NT>), grid, block, lds, stream, fr, (IO *)q, (IO *)k,   \
                       pos, pos_stride, tokens, n_q, head_dim, q_stride, k_stride, sec_t,        \
                       sec_t + sec_h, tpb, per_tok, cph, dh, dq, dk, dc)
    if (dtype == 0) {
        if (nt) NRS_MROPE(float, true);
        else NRS_MROPE(float, false);
    } else {
        if (nt) NRS_MROPE(__bf16, true);
        else NRS_MROPE(__bf16, false);
    }
#undef NRS_MROPE
    return hipGetLastError();
}

}  // namespace nrs
