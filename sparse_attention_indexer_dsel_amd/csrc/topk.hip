// Row-wise top-k for gfx950: radix select over order-preserving keys with a
// candidate filter, then a stable (column-ordered) compaction.
//
// What is computed (DeepSelect tutorial, "Sheshisa Imisebenzi ye-PyTorch TopK
// nge-DeepSelect": basic usage, variable-length rows, NaN handling): for each
// row the c = min(k, n) largest entries of the valid prefix x[0:n), n the
// clamped per-row exclusive end; equal values keep column order, NaN ranks
// above +inf, -0 equals +0; the selected columns are written in ascending
// order, short rows padded with -1 / -inf; a per-row flag reports NaN in rows
// longer than k.
//
// How (this file's design, not the pages'):
//   * a key is the value's bits mapped to an unsigned integer whose order is
//     the ranking order (sign-magnitude -> offset binary, so -0 and +0 meet;
//     every NaN -> the largest key); bf16 keys are formed two per VGPR with
//     packed 16-bit integer ops;
//   * pass A streams the workgroup's columns from HBM with coalesced 16-byte
//     loads, several in flight per thread, and histograms an 11-bit first
//     digit in LDS; it keeps nothing in VGPRs, so many workgroups fit on a
//     compute unit and hide the load latency;
//   * pass B re-reads the columns from cache, each thread a contiguous
//     segment held in VGPRs; the bin holding the k-th largest key fixes a
//     threshold T1 and only the C candidates with key >= T1 (about k plus
//     one bin) are compacted, in column order, into an LDS list (one
//     workgroup scan);
//   * the rest of the radix select (5 more bits for bf16, 11+10 for fp32)
//     and the output run on that short list: every key > T plus the first
//     `need` keys == T in column order, written in column order in rounds
//     of 256 so the stores coalesce; the output is ascending by
//     construction and no sort is run;
//   * a row too long for one workgroup, or too few rows to fill the GPU, is
//     split over G workgroups: their pass-A histograms meet in a per-row
//     workspace slot (device-scope relaxed atomics and one rendezvous); each
//     stages its candidates there and the last workgroup to finish runs the
//     exact selection for the row;
//   * if a row's candidate list would not fit (massive ties at the
//     threshold), the radix select finishes over the segments in VGPRs
//     instead (slower, same result).
#include "dsel_internal.h"

namespace dsel {
namespace {

constexpr int NT = kTopkThreads;
constexpr int NWAVE = NT / 64;
constexpr int UNROLL_A = 4;  // pass-A 16-byte loads in flight per thread
constexpr uint32_t kSpinLimit = 1u << 22;

// Hide a value from the optimiser so a comparison repeated after a
// workgroup scan is recomputed instead of keeping one lane mask per element
// alive across it (which spills scalar registers).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// The thread index, opaque: a persistent workgroup walking rows must not
// have the many per-thread constants derived from it hoisted out of its row
// loop and pinned in VGPRs; recomputing them costs a few ALU ops per row.
__device__ __forceinline__ int tid() { return (int)opaque(threadIdx.x); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

// bf16: two keys per 32-bit word (element 0 in the low half).
struct Bf16Key {
    using raw_t = uint16_t;
    static constexpr int VEC = 8;  // elements per 16-byte load
    static constexpr int EPW = 2;  // elements per key word
    static constexpr int NPASS = 2;
    static constexpr int SH1 = 5;  // first digit = key >> 5 (11 bits)
    static constexpr uint32_t NEG_INF = 0xFF80u;
    __device__ static int digit(int pass) { return pass == 0 ? 11 : 5; }
    // offset binary of both halves: 0x8000 +/- magnitude (packed int16 ops);
    // magmax collects the largest magnitude bits for the NaN probe
    __device__ static uint32_t keyword(uint32_t w, uint32_t &magmax) {
        const u16x2 mag = as_u16x2(w & 0x7FFF7FFFu);
        magmax = as_u32(__builtin_elementwise_max(as_u16x2(magmax), mag));
        const u16x2 s = __builtin_bit_cast(u16x2, __builtin_bit_cast(s16x2, as_u16x2(w)) >> (short)15);
        return as_u32((mag ^ s) - s) ^ 0x80008000u;
    }
    __device__ static bool probe_nan(uint32_t m) {
        return (m & 0xFFFFu) > 0x7F80u || (m >> 16) > 0x7F80u;
    }
    // a NaN's key lies above +inf's (0xFF80) or below -inf's (0x0080); send it
    // to the top.  Key 0 marks an empty slot and stays.
    __device__ static uint32_t fix_nan_half(uint32_t h) {
        return (h > 0xFF80u || (h != 0u && h < 0x0080u)) ? 0xFFFFu : h;
    }
    __device__ static uint32_t fix_nan_word(uint32_t kw) {
        return fix_nan_half(kw & 0xFFFFu) | (fix_nan_half(kw >> 16) << 16);
    }
    __device__ static uint32_t elem(uint32_t kw, int h) { return h ? (kw >> 16) : (kw & 0xFFFFu); }
    __device__ static uint32_t clear_elem(uint32_t kw, int h) {
        return h ? (kw & 0x0000FFFFu) : (kw & 0xFFFF0000u);
    }
};

struct F32Key {
    using raw_t = uint32_t;
    static constexpr int VEC = 4;
    static constexpr int EPW = 1;
    static constexpr int NPASS = 3;
    static constexpr int SH1 = 21;
    static constexpr uint32_t NEG_INF = 0xFF800000u;
    __device__ static int digit(int pass) { return pass == 2 ? 10 : 11; }
    __device__ static uint32_t keyword(uint32_t w, uint32_t &magmax) {
        const uint32_t mag = w & 0x7FFFFFFFu;
        magmax = max(magmax, mag);
        const uint32_t s = (uint32_t)((int32_t)w >> 31);
        return ((mag ^ s) - s) + 0x80000000u;
    }
    __device__ static bool probe_nan(uint32_t m) { return m > 0x7F800000u; }
    __device__ static uint32_t fix_nan_word(uint32_t kw) {
        return (kw > 0xFF800000u || (kw != 0u && kw < 0x00800000u)) ? 0xFFFFFFFFu : kw;
    }
    __device__ static uint32_t elem(uint32_t kw, int) { return kw; }
    __device__ static uint32_t clear_elem(uint32_t, int) { return 0u; }
};

// Inclusive prefix sum over a wave64 with DPP row shifts and row broadcasts.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
}

// Inclusive prefix sum over the workgroup in thread order; *total receives
// the workgroup's sum.
__device__ uint32_t block_incl_scan(uint32_t x, uint32_t *s_red, uint32_t *total = nullptr) {
    const int t = tid();
    const uint32_t w = wave_incl_scan(x);
    if ((t & 63) == 63) s_red[t >> 6] = w;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) {
        const uint32_t v = s_red[i];
        off += (i < (t >> 6)) ? v : 0u;
        tot += v;
    }
    __syncthreads();
    if (total) *total = tot;
    return w + off;
}

__device__ uint32_t block_sum(uint32_t x, uint32_t *s_red) {
    const uint32_t w = wave_sum(x);
    if ((tid() & 63) == 0) s_red[tid() >> 6] = w;
    __syncthreads();
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) tot += s_red[i];
    __syncthreads();
    return tot;
}

struct Digit {
    uint32_t v;      // boundary digit
    uint32_t above;  // count in digits above it
    uint32_t cnt;    // count in the boundary digit
};

// Scan a histogram from its top bin down and find the digit holding the
// need-th largest element (need >= 1 and the histogram holds >= need).
__device__ Digit find_digit(const uint32_t *hist, int nb, uint32_t need, uint32_t *s_red,
                            uint32_t *s_out) {
    const int t = tid();
    const int bpt = nb > NT ? nb / NT : 1;
    const int nact = nb / bpt;
    const int top = nb - t * bpt;  // exclusive upper bin of this thread
    uint32_t local = 0;
    if (t < nact)
        for (int i = 1; i <= bpt; ++i) local += hist[top - i];
    const uint32_t incl = block_incl_scan(local, s_red);
    const uint32_t excl = incl - local;
    if (t < nact && excl < need && need <= incl) {
        uint32_t acc = excl;
        for (int i = 1; i <= bpt; ++i) {
            const uint32_t h = hist[top - i];
            if (acc + h >= need) {
                s_out[0] = (uint32_t)(top - i);
                s_out[1] = acc;
                s_out[2] = h;
                break;
            }
            acc += h;
        }
    }
    __syncthreads();
    const Digit d{s_out[0], s_out[1], s_out[2]};
    __syncthreads();
    return d;
}

// Cross-workgroup data moves only through device-scope relaxed atomics (no
// cache-wide fences); ordering comes from waiting for this workgroup's
// outstanding memory operations before it signals.
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain_memory() { __builtin_amdgcn_s_waitcnt(0); }


// Rendezvous of the G workgroups of one row.  `ctr` counts arrivals over the
// whole launch; the m-th rendezvous completes at m*G.  The wait is bounded:
// past the spin limit the workgroup records an error bit and goes on, so
// every wave always exits.
__device__ void row_rendezvous(uint32_t *ctr, uint32_t target, uint32_t *err) {
    drain_memory();
    __syncthreads();
    if (tid() == 0) {
        add_agent(ctr, 1u);
        uint32_t spins = 0;
        while (ld_agent(ctr) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

template <class K>
__device__ __forceinline__ void emit(const TopkArgs &a, int64_t row, uint32_t pos, int64_t col,
                                     const typename K::raw_t *xr) {
    if (pos >= (uint32_t)a.k) return;  // never write past the row's k slots
    if (a.idx64)
        reinterpret_cast<int64_t *>(a.out_idx)[row * a.idx_stride + pos] = col;
    else
        reinterpret_cast<int32_t *>(a.out_idx)[row * a.idx_stride + pos] = (int32_t)col;
    if (a.ret_val)
        reinterpret_cast<typename K::raw_t *>(a.out_val)[row * a.val_stride + pos] = xr[col];
}

// Rows with n <= k: columns 0..n-1 in order, then padding.  Workgroup c of G
// writes slots [c*S, (c+1)*S) with S = ceil(k / G).
template <class K>
__device__ void write_short_row(const TopkArgs &a, int64_t row, int64_t n, int c, int G,
                                const typename K::raw_t *xr) {
    const int S = (a.k + G - 1) / G;
    const int s0 = c * S;
    const int s1 = min(a.k, s0 + S);
    if (!a.idx64 && !a.ret_val && (a.idx_stride & 3) == 0 && (s0 & 3) == 0) {
        // index-only int32: four slots per 16-byte store
        int32_t *o = reinterpret_cast<int32_t *>(a.out_idx) + row * a.idx_stride;
        const int nv = (s1 - s0) >> 2;
        for (int v = tid(); v < nv; v += NT) {
            const int s = s0 + 4 * v;
            int4 q;
            q.x = s < n ? s : -1;
            q.y = s + 1 < n ? s + 1 : -1;
            q.z = s + 2 < n ? s + 2 : -1;
            q.w = s + 3 < n ? s + 3 : -1;
            *reinterpret_cast<int4 *>(o + s) = q;
        }
        for (int s = s0 + 4 * nv + tid(); s < s1; s += NT) o[s] = s < n ? s : -1;
    } else {
        for (int s = s0 + tid(); s < s1; s += NT) {
            const bool in = s < n;
            if (a.idx64)
                reinterpret_cast<int64_t *>(a.out_idx)[row * a.idx_stride + s] = in ? (int64_t)s : -1;
            else
                reinterpret_cast<int32_t *>(a.out_idx)[row * a.idx_stride + s] = in ? s : -1;
            if (a.ret_val)
                reinterpret_cast<typename K::raw_t *>(a.out_val)[row * a.val_stride + s] =
                    in ? xr[s] : (typename K::raw_t)K::NEG_INF;
        }
    }
    if (c == 0 && tid() == 0 && a.nan_flag) a.nan_flag[row] = 0;
}

// Range-checked view of one row's first `end` columns for raw buffer loads:
// bytes at or past the (dword-rounded) end read as zero without touching
// memory, so every 16-byte load is unconditional.  The rounding keeps a
// partly valid dword whole; the element past the end is cleared by the
// caller (clear_tail).
template <class K>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_view(const typename K::raw_t *xr, int64_t end) {
    const int64_t bytes = end > 0 ? ((end * (int64_t)sizeof(typename K::raw_t) + 3) & ~(int64_t)3) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<typename K::raw_t *>(xr), (short)0,
                                             (int)bytes, 0x00020000);
}

// 16 bytes of raw values at column p of a row view.
template <class K>
__device__ __forceinline__ uint4 load_vec(__amdgpu_buffer_rsrc_t view, int64_t p) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
        view, (unsigned)(p * (int64_t)sizeof(typename K::raw_t)), 0u, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Keys of one 16-byte vector; NaNs sent to the top key.  Returns true if the
// vector held a NaN.
template <class K>
__device__ __forceinline__ bool keys_of(uint4 v, uint32_t *kw) {
    uint32_t m = 0;
    kw[0] = K::keyword(v.x, m);
    kw[1] = K::keyword(v.y, m);
    kw[2] = K::keyword(v.z, m);
    kw[3] = K::keyword(v.w, m);
    const bool nan = K::probe_nan(m);
    if (nan) {
#pragma unroll
        for (int q = 0; q < 4; ++q) kw[q] = K::fix_nan_word(kw[q]);
    }
    return nan;
}

// Give the elements at and past `valid` (0..VEC) the empty-slot key 0.
template <class K>
__device__ __forceinline__ void clear_tail(uint32_t *kw, int valid) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < K::EPW; ++h)
            kw[q] = (q * K::EPW + h >= valid) ? K::clear_elem(kw[q], h) : kw[q];
}

// Histogram the first digit of every element of a key word.
template <class K>
__device__ __forceinline__ void hist_add(uint32_t *hist, uint32_t kw) {
#pragma unroll
    for (int h = 0; h < K::EPW; ++h) atomicAdd(&hist[K::elem(kw, h) >> K::SH1], 1u);
}

// Same, with empty slots (key 0) sent to this lane's spare bin past the
// histogram so they neither count nor collide.
template <class K>
__device__ __forceinline__ void hist_add_masked(uint32_t *hist, uint32_t kw, uint32_t spare) {
#pragma unroll
    for (int h = 0; h < K::EPW; ++h) {
        const uint32_t key = K::elem(kw, h);
        atomicAdd(&hist[key ? (key >> K::SH1) : spare], 1u);
    }
}

// Pass A of a split row: stream columns [lo, hi) with coalesced 16-byte loads
// (UNROLL_A per thread in flight) and histogram the first digit.  Returns
// whether this thread saw a NaN.
template <class K>
__device__ uint32_t first_digit_histogram(const typename K::raw_t *xr, int64_t lo, int64_t hi,
                                          uint32_t *hist) {
    constexpr int VEC = K::VEC, U = UNROLL_A;
    const int t = tid();
    const uint32_t spare = kBins + (t & 63);
    const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, hi);
    const int64_t span = (int64_t)NT * VEC;  // columns per workgroup-wide load
    const int64_t len = hi > lo ? hi - lo : 0;
    const int64_t full = len / span;         // loads valid for every thread
    uint32_t nan = 0;
    int64_t j = 0;
    for (; j + U <= full; j += U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = load_vec<K>(view, lo + (j + u) * span + (int64_t)t * VEC);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            uint32_t kw[4];
            nan |= keys_of<K>(v[u], kw) ? 1u : 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) hist_add<K>(hist, kw[q]);
        }
    }
    for (; j < full; ++j) {
        uint32_t kw[4];
        nan |= keys_of<K>(load_vec<K>(view, lo + j * span + (int64_t)t * VEC), kw) ? 1u : 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) hist_add<K>(hist, kw[q]);
    }
    if (full * span < len) {  // the last, partly valid load
        const int64_t p = lo + full * span + (int64_t)t * VEC;
        uint32_t kw[4];
        nan |= keys_of<K>(load_vec<K>(view, p), kw) ? 1u : 0u;
        const int64_t valid = hi - p;
        clear_tail<K>(kw, valid < 0 ? 0 : (valid > VEC ? VEC : (int)valid));
#pragma unroll
        for (int q = 0; q < 4; ++q) hist_add_masked<K>(hist, kw[q], spare);
    }
    return nan;
}

// Pass B load of a split row: this thread's contiguous segment [s0, s1) (at
// most SL vectors) into VGPRs as keys; slots past s1 get key 0.
template <class K, int SL>
__device__ __forceinline__ void load_segment(const typename K::raw_t *xr, int64_t s0, int64_t s1,
                                             uint32_t (&kw)[SL * 4]) {
    constexpr int VEC = K::VEC;
    const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, s1);
    uint4 v[SL];
#pragma unroll
    for (int j = 0; j < SL; ++j) v[j] = load_vec<K>(view, s0 + (int64_t)j * VEC);
#pragma unroll
    for (int j = 0; j < SL; ++j) {
        keys_of<K>(v[j], &kw[4 * j]);
        const int64_t valid = s1 - (s0 + (int64_t)j * VEC);
        clear_tail<K>(&kw[4 * j], valid < 0 ? 0 : (valid > VEC ? VEC : (int)valid));
    }
}

// Finish a row from its candidate list (entries (key, column) in column
// order; every key's first digit is >= d1.v): resolve the remaining digits
// of the boundary key among the candidates in the boundary bin, then write
// the selection in column order, NT candidates per round so stores coalesce.
template <class K>
__device__ void select_and_write(const TopkArgs &a, int64_t row, const uint2 *ent, uint32_t C,
                                 Digit d1, uint32_t *s_hist, uint32_t *s_red, uint32_t *s_out,
                                 const typename K::raw_t *xr) {
    const int t = tid();
    uint32_t need = (uint32_t)a.k - d1.above;
    uint32_t P = d1.v;
    int s = K::SH1;
    if (d1.cnt != need) {
#pragma unroll 1
        for (int pass = 1; pass < K::NPASS; ++pass) {
            const int d = K::digit(pass);
            const int sh = s - d;
            const uint32_t dmask = (1u << d) - 1u;
            const int nb = 1 << d;
            for (int b = t; b < nb; b += NT) s_hist[b] = 0;
            __syncthreads();
            for (uint32_t i = t; i < C; i += NT) {
                const uint32_t key = ent[i].x;
                if ((key >> s) == P) atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
            }
            __syncthreads();
            const Digit dg = find_digit(s_hist, nb, need, s_red, s_out);
            need -= dg.above;
            P = (P << d) | dg.v;
            s = sh;
            if (dg.cnt == need) break;
        }
    }
    // every candidate whose top bits (key >> s) exceed P is taken, plus the
    // first `need` equal to P
    uint32_t g0 = 0, q0 = 0;
    for (uint32_t r0 = 0; r0 < C; r0 += NT) {
        const uint32_t i = r0 + t;
        const bool in = i < C;
        const uint2 e = in ? ent[i] : make_uint2(0u, 0u);
        const uint32_t pre = e.x >> s;
        const bool gt = in && pre > P;
        const bool eq = in && pre == P;
        const uint32_t mine = (gt ? 1u : 0u) | (eq ? 0x10000u : 0u);
        uint32_t tot;
        const uint32_t ex = block_incl_scan(mine, s_red, &tot) - mine;
        const uint32_t gb = g0 + (ex & 0xFFFFu), qb = q0 + (ex >> 16);
        if (gt)
            emit<K>(a, row, gb + min(qb, need), e.y, xr);
        else if (eq && qb < need)
            emit<K>(a, row, gb + qb, e.y, xr);
        g0 += tot & 0xFFFFu;
        q0 += tot >> 16;
    }
}

// Compact the candidates (key >= T1) of a thread's contiguous key segment
// into ent[pos ..] in column order; every element is written once, the
// non-candidates to this lane's spare slot past the list, so the loop has
// no branches.
template <class K, int W>
__device__ __forceinline__ void compact_segment(const uint32_t (&kw)[W], uint32_t T1, uint32_t pos,
                                                uint32_t col0, uint32_t spare, uint2 *ent) {
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
        for (int h = 0; h < K::EPW; ++h) {
            const uint32_t key = K::elem(kw[w], h);
            const bool cand = key >= T1;
            ent[cand ? pos : spare] = make_uint2(key, col0 + w * K::EPW + h);
            pos += cand ? 1u : 0u;
        }
}

template <class K, int MAXL>
__global__ __launch_bounds__(NT) void topk_rows_split(const TopkArgs a) {
    using raw_t = typename K::raw_t;
    constexpr int VEC = K::VEC;
    constexpr int EPW = K::EPW;
    constexpr int SL = MAXL / VEC;  // 16-byte vectors in one thread's segment
    constexpr int W = SL * 4;       // key words in one thread's segment
    static_assert(MAXL % VEC == 0, "segment must hold whole vectors");

    extern __shared__ uint2 s_ent[];  // candidate list (cap entries) + one spare per lane
    __shared__ uint32_t s_hist[kBins + 64];
    __shared__ uint32_t s_red[NWAVE];
    __shared__ uint32_t s_out[8];

    const int t = tid();
    const int G = a.G;
    const int c = (int)(blockIdx.x % (unsigned)G);
    const int64_t lrow = (int64_t)(blockIdx.x / (unsigned)G);
    const int64_t row = a.row0 + lrow;
    if (row >= a.rows) return;  // uniform over the row's workgroups

    int64_t n = a.cols;
    if (a.row_end) {
        const int64_t e = a.row_end[row];
        n = e < 0 ? 0 : (e > a.cols ? a.cols : e);
    }
    const raw_t *xr = reinterpret_cast<const raw_t *>(a.x) + row * a.x_stride;
    if (n <= a.k) {
        write_short_row<K>(a, row, n, c, G, xr);
        return;
    }

    const uint32_t cap = (uint32_t)a.cap;
    uint32_t *slot = a.ws + kHeaderWords + lrow * a.slot_words;
    uint32_t *err = a.ws;
    uint32_t *ghist = slot + kSlotHeadWords;
    uint32_t *gcnt = ghist + kMaxPasses * kBins;
    uint32_t *stage_key = gcnt + 4 * G;
    uint32_t *stage_col = stage_key + cap;

    // this workgroup's columns [lo, hi), and this thread's segment [s0, s1)
    const int64_t lo = (int64_t)c * a.chunk;
    const int64_t hi = min(lo + a.chunk, n);
    const int64_t len = hi > lo ? hi - lo : 0;
    const int64_t L = ((len + NT - 1) / NT + VEC - 1) / VEC * VEC;  // <= MAXL
    const int64_t s0 = lo + (int64_t)t * L;
    const int64_t s1 = min(s0 + L, hi);

    // ---- pass A: first-digit histogram (HBM, coalesced) ---------------------
    for (int b = t; b < kBins + 64; b += NT) s_hist[b] = 0;
    __syncthreads();
    const uint32_t thread_nan = first_digit_histogram<K>(xr, lo, hi, s_hist);
    const uint32_t block_nan = __syncthreads_or((int)thread_nan) ? 1u : 0u;

    // ---- pass B load: this thread's segment into VGPRs (from cache); the
    // loads are in flight across the rendezvous
    uint32_t kw[W];
    load_segment<K, SL>(xr, s0, s1, kw);

    uint32_t nren = 0;
    for (int b = t; b < kBins; b += NT) {
        const uint32_t h = s_hist[b];
        if (h) add_agent(ghist + b, h);
    }
    row_rendezvous(slot, (++nren) * (uint32_t)G, err);
    for (int b = t; b < kBins; b += NT) s_hist[b] = ld_agent(ghist + b);
    __syncthreads();
    const Digit d1 = find_digit(s_hist, kBins, (uint32_t)a.k, s_red, s_out);
    const uint32_t C = d1.above + d1.cnt;

    if (C <= cap) {
        // ---- compaction of the candidates (key >= T1) in column order -------
        const uint32_t T1 = d1.v << K::SH1;
        uint32_t cnt = 0;
#pragma unroll
        for (int w = 0; w < W; ++w)
#pragma unroll
            for (int h = 0; h < EPW; ++h) cnt += K::elem(kw[w], h) >= T1 ? 1u : 0u;
        uint32_t run;
        const uint32_t pos = block_incl_scan(cnt, s_red, &run) - cnt;
#pragma unroll
        for (int w = 0; w < W; ++w) kw[w] = opaque(kw[w]);
        compact_segment<K, W>(kw, opaque(T1), pos, (uint32_t)(s0 - lo), cap + (t & 63), s_ent);
        __syncthreads();
        // run == this workgroup's candidate count

        // ---- stage candidates; the last workgroup finishes the row ----------
        if (t == 0) s_out[4] = add_agent(slot + 2, run);
        __syncthreads();
        const uint32_t off = s_out[4];
        for (uint32_t i = t; i < run; i += NT) {
            st_agent(stage_key + off + i, s_ent[i].x);
            st_agent(stage_col + off + i, s_ent[i].y + (uint32_t)lo);
        }
        if (t == 0) {
            st_agent(gcnt + 4 * c + 0, off);
            st_agent(gcnt + 4 * c + 1, run);
            st_agent(gcnt + 4 * c + 2, block_nan);
        }
        drain_memory();
        __syncthreads();
        if (t == 0) s_out[3] = (add_agent(slot + 1, 1u) == (uint32_t)G - 1u) ? 1u : 0u;
        __syncthreads();
        if (!s_out[3]) return;

        // Last workgroup: every other one has staged its candidates.  Pull
        // them into LDS in workgroup order (= column order).
        uint32_t nn = 0;
        for (int i = t; i < G; i += NT) nn |= ld_agent(gcnt + 4 * i + 2);
        const uint32_t row_nan = __syncthreads_or((int)nn) ? 1u : 0u;
        // destination offsets (exclusive prefix of the counts) in s_hist[0, G),
        // source offsets in s_hist[kMaxSplit, kMaxSplit + G)
        uint32_t base = 0;
        for (int i0 = 0; i0 < G; i0 += NT) {
            const int i = i0 + t;
            const uint32_t cnt_i = i < G ? ld_agent(gcnt + 4 * i + 1) : 0u;
            uint32_t tot;
            const uint32_t incl = block_incl_scan(cnt_i, s_red, &tot);
            if (i < G) {
                s_hist[i] = base + incl - cnt_i;
                s_hist[kMaxSplit + i] = ld_agent(gcnt + 4 * i + 0);
            }
            base += tot;
        }
        __syncthreads();
        for (uint32_t idx = t; idx < C; idx += NT) {
            int lo_b = 0, hi_b = G - 1;  // last workgroup whose range starts at or before idx
            while (lo_b < hi_b) {
                const int mid = (lo_b + hi_b + 1) >> 1;
                if (s_hist[mid] <= idx)
                    lo_b = mid;
                else
                    hi_b = mid - 1;
            }
            const uint32_t src = s_hist[kMaxSplit + lo_b] + (idx - s_hist[lo_b]);
            s_ent[idx] = make_uint2(ld_agent(stage_key + src), ld_agent(stage_col + src));
        }
        __syncthreads();
        select_and_write<K>(a, row, s_ent, C, d1, s_hist, s_red, s_out, xr);
        if (t == 0 && a.nan_flag) a.nan_flag[row] = (uint8_t)row_nan;
        // return the slot to zero for the next call
        for (int b = t; b < kBins; b += NT) st_agent(ghist + b, 0u);
        for (uint32_t i = t; i < C; i += NT) {
            st_agent(stage_key + i, 0u);
            st_agent(stage_col + i, 0u);
        }
        for (int i = t; i < 4 * G; i += NT) st_agent(gcnt + i, 0u);
        drain_memory();
        __syncthreads();
        if (t == 0) {
            st_agent(slot + 0, 0u);
            st_agent(slot + 1, 0u);
            st_agent(slot + 2, 0u);
        }
        return;
    }

    // ---- fallback: too many candidates.  Finish the radix select by
    // re-streaming this thread's segment from cache for each pass, so the
    // rare path costs no extra VGPRs for the common one.
    const __amdgpu_buffer_rsrc_t seg_view = row_view<K>(xr, s1);
    uint32_t need = (uint32_t)a.k - d1.above;
    uint32_t P = d1.v;
    int s = K::SH1;
    if (d1.cnt != need) {
#pragma unroll 1
        for (int pass = 1; pass < K::NPASS; ++pass) {
            const int d = K::digit(pass);
            const int sh = s - d;
            const uint32_t dmask = (1u << d) - 1u;
            const int nb = 1 << d;
            for (int b = t; b < nb; b += NT) s_hist[b] = 0;
            __syncthreads();
#pragma unroll 1
            for (int64_t p = s0; p < s1; p += VEC) {
                uint32_t w4[4];
                keys_of<K>(load_vec<K>(seg_view, p), w4);
                clear_tail<K>(w4, p + VEC > s1 ? (int)(s1 - p) : VEC);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) {
                        const uint32_t kk = K::elem(w4[q], h);
                        if ((kk >> s) == P) atomicAdd(&s_hist[(kk >> sh) & dmask], 1u);
                    }
            }
            __syncthreads();
            uint32_t *g = ghist + pass * kBins;
            for (int b = t; b < nb; b += NT) {
                const uint32_t h = s_hist[b];
                if (h) add_agent(g + b, h);
            }
            row_rendezvous(slot, (++nren) * (uint32_t)G, err);
            for (int b = t; b < nb; b += NT) s_hist[b] = ld_agent(g + b);
            __syncthreads();
            const Digit dg = find_digit(s_hist, nb, need, s_red, s_out);
            need -= dg.above;
            P = (P << d) | dg.v;
            s = sh;
            if (dg.cnt == need) break;  // the boundary bin is taken whole
        }
    }

    // stable compaction over the segment: count, scan, then write in order
    uint32_t g = 0, q = 0;
#pragma unroll 1
    for (int64_t p = s0; p < s1; p += VEC) {
        uint32_t w4[4];
        keys_of<K>(load_vec<K>(seg_view, p), w4);
        clear_tail<K>(w4, p + VEC > s1 ? (int)(s1 - p) : VEC);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t pre = K::elem(w4[qq], h) >> s;
                g += pre > P ? 1u : 0u;
                q += pre == P ? 1u : 0u;
            }
    }
    const uint32_t mine = g | (q << 16);
    uint32_t tot;
    const uint32_t ex = block_incl_scan(mine, s_red, &tot) - mine;

    if (t == 0) {
        st_agent(gcnt + 4 * c + 0, tot & 0xFFFFu);
        st_agent(gcnt + 4 * c + 1, tot >> 16);
        st_agent(gcnt + 4 * c + 2, block_nan);
    }
    row_rendezvous(slot, (++nren) * (uint32_t)G, err);
    uint32_t gg = 0, qq = 0, nn = 0;
    for (int i = t; i < G; i += NT) {
        if (i < c) {
            gg += ld_agent(gcnt + 4 * i + 0);
            qq += ld_agent(gcnt + 4 * i + 1);
        }
        nn |= ld_agent(gcnt + 4 * i + 2);
    }
    const uint32_t gt0 = block_sum(gg, s_red);
    const uint32_t eq0 = block_sum(qq, s_red);
    const uint32_t row_nan = __syncthreads_or((int)nn) ? 1u : 0u;
    {
        uint32_t gb = gt0 + (ex & 0xFFFFu);
        uint32_t qb = eq0 + (ex >> 16);
#pragma unroll 1
        for (int64_t p = s0; p < s1; p += VEC) {
            uint32_t w4[4];
            keys_of<K>(load_vec<K>(seg_view, p), w4);
            clear_tail<K>(w4, p + VEC > s1 ? (int)(s1 - p) : VEC);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int h = 0; h < EPW; ++h) {
                    const uint32_t pre = K::elem(w4[q4], h) >> s;
                    const int64_t col = p + q4 * EPW + h;
                    if (pre > P) {
                        emit<K>(a, row, gb + min(qb, need), col, xr);
                        ++gb;
                    } else if (pre == P) {
                        if (qb < need) emit<K>(a, row, gb + qb, col, xr);
                        ++qb;
                    }
                }
        }
    }
    if (c == 0 && t == 0 && a.nan_flag) a.nan_flag[row] = (uint8_t)row_nan;

    // Leave the slot zeroed for the next call (whose slot layout may differ):
    // every workgroup has read the histograms before the last rendezvous, so
    // each clears a share now; the last workgroup out, once every workgroup
    // has read the counts, clears them and resets the counters.
    constexpr int HW = kMaxPasses * kBins;
    const int per = (HW + G - 1) / G;
    const int z0 = c * per, z1 = min(HW, z0 + per);
    for (int i = z0 + t; i < z1; i += NT) st_agent(ghist + i, 0u);
    drain_memory();
    __syncthreads();
    if (t == 0) s_out[3] = (add_agent(slot + 1, 1u) == (uint32_t)G - 1u) ? 1u : 0u;
    __syncthreads();
    if (s_out[3]) {
        for (int i = t; i < 4 * G; i += NT) st_agent(gcnt + i, 0u);
        drain_memory();
        __syncthreads();
        if (t == 0) {
            st_agent(slot + 0, 0u);
            st_agent(slot + 1, 0u);
        }
    }
}

// ---------------------------------------------------------------------------
// Whole rows: one workgroup per row, persistent and software-pipelined.
// ---------------------------------------------------------------------------

// Issue the loads of one row's first NT*EPT columns (columns at or past n
// read as zero).
template <class K, int LOADS>
__device__ __forceinline__ void prefetch_row(const typename K::raw_t *xr, int64_t n,
                                             uint4 (&v)[LOADS]) {
    const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, n);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) v[j] = load_vec<K>(view, (int64_t)(j * NT + tid()) * K::VEC);
}

// Slow path of a whole row (candidates exceed the LDS list): finish the radix
// select by re-streaming the row from cache; the compaction walks the
// coalesced layout one load at a time with a workgroup scan per load.
template <class K, int LOADS>
__device__ void select_row_streaming(const TopkArgs &a, int64_t row, int64_t n, Digit d1,
                                     const typename K::raw_t *xr, uint32_t *s_hist,
                                     uint32_t *s_red, uint32_t *s_out) {
    constexpr int VEC = K::VEC, EPW = K::EPW;
    const int t = tid();
    const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, n);
    uint32_t need = (uint32_t)a.k - d1.above;
    uint32_t P = d1.v;
    int s = K::SH1;
    if (d1.cnt != need) {
#pragma unroll 1
        for (int pass = 1; pass < K::NPASS; ++pass) {
            const int d = K::digit(pass);
            const int sh = s - d;
            const uint32_t dmask = (1u << d) - 1u;
            const int nb = 1 << d;
            for (int b = t; b < nb; b += NT) s_hist[b] = 0;
            __syncthreads();
#pragma unroll 1
            for (int j = 0; j < LOADS; ++j) {
                const int64_t p = (int64_t)(j * NT + t) * VEC;
                if (p >= n) continue;
                uint32_t w4[4];
                keys_of<K>(load_vec<K>(view, p), w4);
                clear_tail<K>(w4, p + VEC > n ? (int)(n - p) : VEC);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) {
                        const uint32_t kk = K::elem(w4[q], h);
                        if ((kk >> s) == P) atomicAdd(&s_hist[(kk >> sh) & dmask], 1u);
                    }
            }
            __syncthreads();
            const Digit dg = find_digit(s_hist, nb, need, s_red, s_out);
            need -= dg.above;
            P = (P << d) | dg.v;
            s = sh;
            if (dg.cnt == need) break;
        }
    }
    uint32_t gb = 0, qb = 0;  // taken-above and equal counts before the current load
#pragma unroll 1
    for (int j = 0; j < LOADS; ++j) {
        const int64_t p = (int64_t)(j * NT + t) * VEC;
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        if (p < n) {
            keys_of<K>(load_vec<K>(view, p), w4);
            clear_tail<K>(w4, p + VEC > n ? (int)(n - p) : VEC);
        }
        uint32_t g = 0, q = 0;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t pre = K::elem(w4[qq], h) >> s;
                g += pre > P ? 1u : 0u;
                q += pre == P ? 1u : 0u;
            }
        const uint32_t mine = g | (q << 16);
        uint32_t tot;
        const uint32_t ex = block_incl_scan(mine, s_red, &tot) - mine;
        uint32_t g1 = gb + (ex & 0xFFFFu), q1 = qb + (ex >> 16);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t pre = K::elem(w4[qq], h) >> s;
                const int64_t col = p + qq * EPW + h;
                if (pre > P) {
                    emit<K>(a, row, g1 + min(q1, need), col, xr);
                    ++g1;
                } else if (pre == P) {
                    if (q1 < need) emit<K>(a, row, g1 + q1, col, xr);
                    ++q1;
                }
            }
        gb += tot & 0xFFFFu;
        qb += tot >> 16;
    }
}

// Shared memory of the whole-row kernel (the histogram has one spare bin per
// lane past kBins).
template <int LP>
struct RowLds {
    uint32_t hist[kBins + 64];
    uint32_t wtot[LP * NWAVE];
    uint32_t red[NWAVE];
    uint32_t out[8];
};

// One row of valid length n > k whose raw 16-byte vectors are in buf
// (coalesced layout: load j of thread t holds columns (j*NT + t)*VEC ..).
template <class K, int LOADS>
__device__ __forceinline__ void select_row(const TopkArgs &a, int64_t row, int64_t n,
                                           const uint4 (&buf)[LOADS],
                                           RowLds<(LOADS + 1) / 2> &L, uint2 *ent) {
    using raw_t = typename K::raw_t;
    constexpr int VEC = K::VEC;
    constexpr int EPW = K::EPW;
    constexpr int W = LOADS * 4;
    constexpr int LP = (LOADS + 1) / 2;
    constexpr int SPAN = NT * VEC;  // columns per workgroup-wide load
    const int t = tid();
    const int lane = t & 63, wid = t >> 6;
    const uint32_t cap = (uint32_t)a.cap;
    const raw_t *xr = reinterpret_cast<const raw_t *>(a.x) + row * a.x_stride;
    const int ni = (int)n;
    const int full = ni / SPAN;                 // loads valid for every thread
    const int any = (ni + SPAN - 1) / SPAN;     // loads holding some valid column

    // ---- keys, NaN probe, first-digit histogram -----------------------------
    uint32_t kw[W];
    uint32_t nan = 0;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) nan |= keys_of<K>(buf[j], &kw[4 * j]) ? 1u : 0u;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if (j >= full) {
            const int valid = ni - (j * NT + t) * VEC;
            clear_tail<K>(&kw[4 * j], valid < 0 ? 0 : (valid > VEC ? VEC : valid));
        }
    }
    for (int b = t; b < kBins + 64; b += NT) L.hist[b] = 0;
    const uint32_t block_nan = __syncthreads_or((int)nan) ? 1u : 0u;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if (j < full) {
#pragma unroll
            for (int q = 0; q < 4; ++q) hist_add<K>(L.hist, kw[4 * j + q]);
        } else if (j < any) {
#pragma unroll
            for (int q = 0; q < 4; ++q) hist_add_masked<K>(L.hist, kw[4 * j + q], kBins + lane);
        }
    }
    __syncthreads();
    const Digit d1 = find_digit(L.hist, kBins, (uint32_t)a.k, L.red, L.out);
    const uint32_t C = d1.above + d1.cnt;

    if (C <= cap) {
        // ---- candidates (key >= T1) to LDS in column order ------------------
        const uint32_t T1 = d1.v << K::SH1;
        uint32_t pk[LP];
#pragma unroll
        for (int i = 0; i < LP; ++i) pk[i] = 0;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            if (j < any) {
                uint32_t m = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) m += K::elem(kw[4 * j + q], h) >= T1 ? 1u : 0u;
                pk[j >> 1] |= m << ((j & 1) * 16);
            }
        }
        uint32_t ex[LP];
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const uint32_t incl = wave_incl_scan(pk[i]);
            ex[i] = incl - pk[i];
            if (lane == 63) L.wtot[i * NWAVE + wid] = incl;
        }
        __syncthreads();
        const uint32_t T1w = opaque(T1);
#pragma unroll
        for (int w = 0; w < W; ++w) kw[w] = opaque(kw[w]);
        const uint32_t spare = cap + lane;
        uint32_t run = 0;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            if (j < any) {
                const int i = j >> 1, sh = (j & 1) * 16;
                uint32_t tot = 0, before = 0;
#pragma unroll
                for (int w = 0; w < NWAVE; ++w) {
                    const uint32_t v = (L.wtot[i * NWAVE + w] >> sh) & 0xFFFFu;
                    tot += v;
                    before += (w < wid) ? v : 0u;
                }
                uint32_t pos = run + before + ((ex[i] >> sh) & 0xFFFFu);
                run += tot;
                const uint32_t p = (uint32_t)(j * NT + t) * VEC;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) {
                        const uint32_t key = K::elem(kw[4 * j + q], h);
                        const bool cand = key >= T1w;
                        ent[cand ? pos : spare] = make_uint2(key, p + q * EPW + h);
                        pos += cand ? 1u : 0u;
                    }
            }
        }
        __syncthreads();
        select_and_write<K>(a, row, ent, C, d1, L.hist, L.red, L.out, xr);
    } else {
        select_row_streaming<K, LOADS>(a, row, n, d1, xr, L.hist, L.red, L.out);
    }
    if (t == 0 && a.nan_flag) a.nan_flag[row] = (uint8_t)block_nan;
}

__device__ __forceinline__ int64_t valid_length(const TopkArgs &a, int64_t row) {
    int64_t n = a.cols;
    if (a.row_end) {
        const int64_t e = a.row_end[row];
        n = e < 0 ? 0 : (e > a.cols ? a.cols : e);
    }
    return n;
}

// A workgroup walks rows blockIdx.x, blockIdx.x + gridDim.x, ...: while it
// selects from one row (keys in VGPRs), the 16-byte loads of its next row are
// already in flight into a second register buffer, and the row after that
// has its row_end read, so neither latency sits between two rows.
template <class K, int EPT>
__global__ __launch_bounds__(NT) void topk_rows_pipelined(const TopkArgs a) {
    using raw_t = typename K::raw_t;
    constexpr int LOADS = EPT / K::VEC;
    static_assert(EPT % K::VEC == 0, "EPT must be a multiple of the vector width");
    extern __shared__ uint2 s_ent[];  // candidate list (cap entries) + one spare per lane
    __shared__ RowLds<(LOADS + 1) / 2> L;

    const int64_t stride = gridDim.x;
    const raw_t *x = reinterpret_cast<const raw_t *>(a.x);
    int64_t row = a.row0 + blockIdx.x;
    if (row >= a.rows) return;
    int64_t n = valid_length(a, row);
    int64_t n2 = row + stride < a.rows ? valid_length(a, row + stride) : 0;
    uint4 cur[LOADS], nxt[LOADS];
    if (n > a.k) prefetch_row<K, LOADS>(x + row * a.x_stride, n, cur);

#pragma unroll 1
    for (; row < a.rows; row += stride) {
        const int64_t row2 = row + stride;
        if (row2 < a.rows && n2 > a.k) prefetch_row<K, LOADS>(x + row2 * a.x_stride, n2, nxt);
        const int64_t n3 = row2 + stride < a.rows ? valid_length(a, row2 + stride) : 0;
        if (n <= a.k)
            write_short_row<K>(a, row, n, 0, 1, x + row * a.x_stride);
        else
            select_row<K, LOADS>(a, row, n, cur, L, s_ent);
        __syncthreads();  // LDS is reused by the next row
        // the next row's vectors had this whole row's work to arrive
#pragma unroll
        for (int j = 0; j < LOADS; ++j) cur[j] = nxt[j];
        n = n2;
        n2 = n3;
    }
}

template <class K, int MAXL, bool SPLIT>
const void *kptr() {
    if (SPLIT) return reinterpret_cast<const void *>(&topk_rows_split<K, MAXL>);
    return reinterpret_cast<const void *>(&topk_rows_pipelined<K, MAXL>);
}

template <class K, bool SPLIT>
const void *pick(int maxl) {
    switch (maxl) {
        case 8: return kptr<K, 8, SPLIT>();
        case 16: return kptr<K, 16, SPLIT>();
        case 32: return kptr<K, 32, SPLIT>();
        case 64: return kptr<K, 64, SPLIT>();
        default: return nullptr;
    }
}

}  // namespace

// Split rows: topk_rows_split (maxl = longest per-thread segment).  Whole
// rows: topk_rows_pipelined (maxl = columns per thread).
const void *topk_kernel_ptr(int dtype, int maxl, bool split) {
    if (dtype == 0) return split ? pick<Bf16Key, true>(maxl) : pick<Bf16Key, false>(maxl);
    return split ? pick<F32Key, true>(maxl) : pick<F32Key, false>(maxl);
}

// Candidate entries (key, column) plus one spare entry per lane.
size_t topk_dyn_lds(int dtype, int64_t cap) {
    (void)dtype;
    return (size_t)(cap + 64) * sizeof(uint2);
}

hipError_t launch_topk(int dtype, int maxl, bool split, const TopkArgs &a, unsigned grid,
                       hipStream_t stream) {
    const void *fn = topk_kernel_ptr(dtype, maxl, split);
    if (!fn) return hipErrorInvalidValue;
    TopkArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(NT), args, topk_dyn_lds(dtype, a.cap), stream);
}

}  // namespace dsel
