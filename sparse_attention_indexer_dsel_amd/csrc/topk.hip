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
//   * a workgroup (4 wave64s) holds up to 256 x 64 keys of one row in VGPRs,
//     read once from HBM with 16-byte loads; bf16 keys stay packed two per
//     VGPR and are formed with packed 16-bit integer ops;
//   * a key is the value's bits mapped to an unsigned integer whose order is
//     the ranking order (sign-magnitude -> offset binary, so -0 and +0 meet;
//     every NaN -> the largest key);
//   * pass 1 histograms an 11-bit first digit in LDS; the bin holding the
//     k-th largest key fixes a threshold T1, and only the C candidates with
//     key >= T1 (about k plus one bin) are compacted, in column order, into
//     an LDS list;
//   * the rest of the radix select (5 more bits for bf16, 11+10 for fp32)
//     and the output run on that short list: every key > T plus the first
//     `need` keys == T in column order, written in column order, so the
//     output is ascending by construction and no sort is run;
//   * a row too long for one workgroup, or too few rows to fill the GPU, is
//     split over G workgroups: their pass-1 histograms meet in a per-row
//     workspace slot (device-scope relaxed atomics and one rendezvous); each
//     stages its candidates there and the last workgroup to finish runs the
//     exact selection for the row;
//   * if a row's candidate list would not fit (massive ties at the
//     threshold), the whole radix select runs over the keys in VGPRs
//     instead (slower, same result).
#include "dsel_internal.h"

namespace dsel {
namespace {

constexpr int NT = kTopkThreads;
constexpr int NWAVE = NT / 64;
constexpr uint32_t kSpinLimit = 1u << 22;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

// bf16: two keys per 32-bit word (element 0 in the low half).
struct Bf16Key {
    using raw_t = uint16_t;
    using ckey_t = uint16_t;
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
    __device__ static uint32_t raw_word(const raw_t *xr, int64_t p, int64_t hi) {
        const uint32_t lo = (p < hi) ? (uint32_t)xr[p] : 0u;
        const uint32_t up = (p + 1 < hi) ? (uint32_t)xr[p + 1] : 0u;
        return lo | (up << 16);
    }
};

struct F32Key {
    using raw_t = uint32_t;
    using ckey_t = uint32_t;
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
    __device__ static uint32_t raw_word(const raw_t *xr, int64_t p, int64_t hi) {
        return (p < hi) ? xr[p] : 0u;
    }
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

// Inclusive prefix sum over the workgroup in thread order.
__device__ uint32_t block_incl_scan(uint32_t x, uint32_t *s_red) {
    const int t = threadIdx.x;
    const uint32_t w = wave_incl_scan(x);
    if ((t & 63) == 63) s_red[t >> 6] = w;
    __syncthreads();
    uint32_t off = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) off += (i < (t >> 6)) ? s_red[i] : 0u;
    __syncthreads();
    return w + off;
}

__device__ uint32_t block_sum(uint32_t x, uint32_t *s_red) {
    const uint32_t w = wave_sum(x);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = w;
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
    const int t = threadIdx.x;
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
    if (threadIdx.x == 0) {
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
        for (int v = (int)threadIdx.x; v < nv; v += NT) {
            const int s = s0 + 4 * v;
            int4 q;
            q.x = s < n ? s : -1;
            q.y = s + 1 < n ? s + 1 : -1;
            q.z = s + 2 < n ? s + 2 : -1;
            q.w = s + 3 < n ? s + 3 : -1;
            *reinterpret_cast<int4 *>(o + s) = q;
        }
        for (int s = s0 + 4 * nv + (int)threadIdx.x; s < s1; s += NT) o[s] = s < n ? s : -1;
    } else {
        for (int s = s0 + (int)threadIdx.x; s < s1; s += NT) {
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
    if (c == 0 && threadIdx.x == 0 && a.nan_flag) a.nan_flag[row] = 0;
}

// Finish a row from its candidate list (keys ck, columns cc, in column order;
// every candidate's first digit is >= d1.v): resolve the remaining digits of
// the boundary key among the candidates in the boundary bin, then write the
// selection in column order.
template <class K>
__device__ void select_and_write(const TopkArgs &a, int64_t row, const typename K::ckey_t *ck,
                                 const uint32_t *cc, uint32_t C, Digit d1, uint32_t *s_hist,
                                 uint32_t *s_red, uint32_t *s_out, const typename K::raw_t *xr) {
    const int t = threadIdx.x;
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
                const uint32_t key = ck[i];
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
    // every candidate whose top KEY_BITS-s bits exceed P is taken, plus the
    // first `need` equal to P
    const uint32_t S = (C + NT - 1) / NT;
    const uint32_t i0 = min(C, t * S), i1 = min(C, i0 + S);
    uint32_t g = 0, q = 0;
    for (uint32_t i = i0; i < i1; ++i) {
        const uint32_t pre = (uint32_t)ck[i] >> s;
        g += pre > P ? 1u : 0u;
        q += pre == P ? 1u : 0u;
    }
    const uint32_t mine = g | (q << 16);
    const uint32_t ex = block_incl_scan(mine, s_red) - mine;
    uint32_t gb = ex & 0xFFFFu, qb = ex >> 16;
    for (uint32_t i = i0; i < i1; ++i) {
        const uint32_t pre = (uint32_t)ck[i] >> s;
        if (pre > P) {
            emit<K>(a, row, gb + min(qb, need), cc[i], xr);
            ++gb;
        } else if (pre == P) {
            if (qb < need) emit<K>(a, row, gb + qb, cc[i], xr);
            ++qb;
        }
    }
}

template <class K, int EPT, bool SPLIT>
__global__ __launch_bounds__(NT) void topk_rows_kernel(const TopkArgs a) {
    using raw_t = typename K::raw_t;
    using ckey_t = typename K::ckey_t;
    constexpr int VEC = K::VEC;
    constexpr int EPW = K::EPW;
    constexpr int LOADS = EPT / VEC;
    constexpr int W = LOADS * 4;  // key words per thread
    constexpr int LP = (LOADS + 1) / 2;
    static_assert(EPT % VEC == 0, "EPT must be a multiple of the vector width");

    extern __shared__ uint32_t s_dyn[];  // candidate list: keys, then columns
    __shared__ uint32_t s_hist[kBins];
    __shared__ uint32_t s_wtot[LP * NWAVE];
    __shared__ uint32_t s_red[NWAVE];
    __shared__ uint32_t s_out[8];

    const int t = threadIdx.x;
    const int lane = t & 63, wid = t >> 6;
    const int G = SPLIT ? a.G : 1;
    const int c = SPLIT ? (int)(blockIdx.x % (unsigned)G) : 0;
    const int64_t lrow = SPLIT ? (int64_t)(blockIdx.x / (unsigned)G) : (int64_t)blockIdx.x;
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
    ckey_t *ck = reinterpret_cast<ckey_t *>(s_dyn);
    uint32_t *cc = s_dyn + (cap * sizeof(ckey_t) + 3) / 4;

    uint32_t *slot = SPLIT ? a.ws + kHeaderWords + lrow * a.slot_words : nullptr;
    uint32_t *err = a.ws;
    uint32_t *ghist = SPLIT ? slot + kSlotHeadWords : nullptr;
    uint32_t *gcnt = SPLIT ? ghist + kMaxPasses * kBins : nullptr;
    uint32_t *stage_key = SPLIT ? gcnt + 4 * G : nullptr;
    uint32_t *stage_col = SPLIT ? stage_key + cap : nullptr;

    const int64_t lo = SPLIT ? (int64_t)c * a.chunk : 0;
    const int64_t hi = SPLIT ? min(lo + a.chunk, n) : n;

    // ---- load once: keys in VGPRs, NaN probe --------------------------------
    uint32_t kw[W];
    uint32_t magmax = 0;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int64_t p = lo + (int64_t)(j * NT + t) * VEC;
        if (p + VEC <= hi) {
            const uint4 v = *reinterpret_cast<const uint4 *>(xr + p);
            kw[4 * j + 0] = K::keyword(v.x, magmax);
            kw[4 * j + 1] = K::keyword(v.y, magmax);
            kw[4 * j + 2] = K::keyword(v.z, magmax);
            kw[4 * j + 3] = K::keyword(v.w, magmax);
        } else if (p < hi) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t pe = p + q * EPW;
                uint32_t k = K::keyword(K::raw_word(xr, pe, hi), magmax);
#pragma unroll
                for (int h = 0; h < EPW; ++h)
                    if (pe + h >= hi) k = K::clear_elem(k, h);  // empty slot: key 0
                kw[4 * j + q] = k;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) kw[4 * j + q] = 0u;
        }
    }
    const bool thread_nan = K::probe_nan(magmax);
    if (thread_nan) {
#pragma unroll
        for (int w = 0; w < W; ++w) kw[w] = K::fix_nan_word(kw[w]);
    }
    const uint32_t block_nan = __syncthreads_or((int)thread_nan) ? 1u : 0u;

    // ---- pass 1: first-digit histogram --------------------------------------
    for (int b = t; b < kBins; b += NT) s_hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if (lo + (int64_t)(j * NT + t) * VEC >= hi) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int h = 0; h < EPW; ++h) atomicAdd(&s_hist[K::elem(kw[4 * j + q], h) >> K::SH1], 1u);
    }
    __syncthreads();
    uint32_t nren = 0;
    if (SPLIT) {
        for (int b = t; b < kBins; b += NT) {
            const uint32_t h = s_hist[b];
            if (h) add_agent(ghist + b, h);
        }
        row_rendezvous(slot, (++nren) * (uint32_t)G, err);
        for (int b = t; b < kBins; b += NT) s_hist[b] = ld_agent(ghist + b);
        __syncthreads();
    }
    const Digit d1 = find_digit(s_hist, kBins, (uint32_t)a.k, s_red, s_out);
    const uint32_t C = d1.above + d1.cnt;

    if (C <= cap) {
        // ---- compaction of the candidates (key >= T1) in column order -------
        const uint32_t T1 = d1.v << K::SH1;
        uint32_t pk[LP];
#pragma unroll
        for (int i = 0; i < LP; ++i) pk[i] = 0;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            uint32_t m = 0;
            if (lo + (int64_t)(j * NT + t) * VEC < hi) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) m += K::elem(kw[4 * j + q], h) >= T1 ? 1u : 0u;
            }
            pk[j >> 1] |= m << ((j & 1) * 16);
        }
        uint32_t ex[LP];
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const uint32_t incl = wave_incl_scan(pk[i]);
            ex[i] = incl - pk[i];
            if (lane == 63) s_wtot[i * NWAVE + wid] = incl;
        }
        __syncthreads();
        uint32_t run = 0;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int i = j >> 1, sh = (j & 1) * 16;
            uint32_t tot = 0, before = 0;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) {
                const uint32_t v = (s_wtot[i * NWAVE + w] >> sh) & 0xFFFFu;
                tot += v;
                before += (w < wid) ? v : 0u;
            }
            uint32_t pos = run + before + ((ex[i] >> sh) & 0xFFFFu);
            run += tot;
            const int64_t p = lo + (int64_t)(j * NT + t) * VEC;
            if (p < hi) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) {
                        const uint32_t key = K::elem(kw[4 * j + q], h);
                        if (key >= T1) {
                            ck[pos] = (ckey_t)key;
                            cc[pos] = (uint32_t)(p - lo) + q * EPW + h;
                            ++pos;
                        }
                    }
            }
        }
        __syncthreads();
        // run == this workgroup's candidate count

        if (!SPLIT) {
            select_and_write<K>(a, row, ck, cc, C, d1, s_hist, s_red, s_out, xr);
            if (t == 0 && a.nan_flag) a.nan_flag[row] = (uint8_t)block_nan;
            return;
        }

        // ---- split row: stage candidates; the last workgroup finishes -------
        if (t == 0) s_out[4] = add_agent(slot + 2, run);
        __syncthreads();
        const uint32_t off = s_out[4];
        for (uint32_t i = t; i < run; i += NT) {
            st_agent(stage_key + off + i, ck[i]);
            st_agent(stage_col + off + i, cc[i] + (uint32_t)lo);
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
            const uint32_t cnt = i < G ? ld_agent(gcnt + 4 * i + 1) : 0u;
            const uint32_t incl = block_incl_scan(cnt, s_red);
            if (i < G) {
                s_hist[i] = base + incl - cnt;
                s_hist[kMaxSplit + i] = ld_agent(gcnt + 4 * i + 0);
            }
            if (t == NT - 1) s_out[5] = incl;
            __syncthreads();
            base += s_out[5];
            __syncthreads();
        }
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
            ck[idx] = (ckey_t)ld_agent(stage_key + src);
            cc[idx] = ld_agent(stage_col + src);
        }
        __syncthreads();
        select_and_write<K>(a, row, ck, cc, C, d1, s_hist, s_red, s_out, xr);
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

    // ---- fallback: too many candidates; finish the radix select in VGPRs ----
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
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                if (lo + (int64_t)(j * NT + t) * VEC >= hi) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) {
                        const uint32_t kk = K::elem(kw[4 * j + q], h);
                        if ((kk >> s) == P) atomicAdd(&s_hist[(kk >> sh) & dmask], 1u);
                    }
            }
            __syncthreads();
            if (SPLIT) {
                uint32_t *g = ghist + pass * kBins;
                for (int b = t; b < nb; b += NT) {
                    const uint32_t h = s_hist[b];
                    if (h) add_agent(g + b, h);
                }
                row_rendezvous(slot, (++nren) * (uint32_t)G, err);
                for (int b = t; b < nb; b += NT) s_hist[b] = ld_agent(g + b);
                __syncthreads();
            }
            const Digit dg = find_digit(s_hist, nb, need, s_red, s_out);
            need -= dg.above;
            P = (P << d) | dg.v;
            s = sh;
            if (dg.cnt == need) break;  // the boundary bin is taken whole
        }
    }

    // stable compaction straight from the VGPRs
    uint32_t cnt[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        uint32_t g = 0, q2 = 0;
        if (lo + (int64_t)(j * NT + t) * VEC < hi) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int h = 0; h < EPW; ++h) {
                    const uint32_t pre = K::elem(kw[4 * j + q], h) >> s;
                    g += pre > P ? 1u : 0u;
                    q2 += pre == P ? 1u : 0u;
                }
        }
        cnt[j] = g | (q2 << 16);
    }
    uint32_t basev[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const uint32_t incl = wave_incl_scan(cnt[j]);
        basev[j] = incl - cnt[j];
        if (lane == 63) s_hist[j * NWAVE + wid] = incl;  // s_hist is free here
    }
    __syncthreads();
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
            const uint32_t v = s_hist[j * NWAVE + w];
            tot += v;
            before += (w < wid) ? v : 0u;
        }
        basev[j] += run + before;
        run += tot;
    }
    __syncthreads();

    uint32_t gt0 = 0, eq0 = 0, row_nan = block_nan;
    if (SPLIT) {
        if (t == 0) {
            st_agent(gcnt + 4 * c + 0, run & 0xFFFFu);
            st_agent(gcnt + 4 * c + 1, run >> 16);
            st_agent(gcnt + 4 * c + 2, block_nan);
        }
        row_rendezvous(slot, (++nren) * (uint32_t)G, err);
        uint32_t g = 0, q = 0, nn = 0;
        for (int i = t; i < G; i += NT) {
            if (i < c) {
                g += ld_agent(gcnt + 4 * i + 0);
                q += ld_agent(gcnt + 4 * i + 1);
            }
            nn |= ld_agent(gcnt + 4 * i + 2);
        }
        gt0 = block_sum(g, s_red);
        eq0 = block_sum(q, s_red);
        row_nan = __syncthreads_or((int)nn) ? 1u : 0u;
    }

#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int64_t p = lo + (int64_t)(j * NT + t) * VEC;
        if (p >= hi) continue;
        uint32_t g = gt0 + (basev[j] & 0xFFFFu);
        uint32_t q2 = eq0 + (basev[j] >> 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t pre = K::elem(kw[4 * j + q], h) >> s;
                const int64_t col = p + q * EPW + h;
                if (pre > P) {
                    emit<K>(a, row, g + min(q2, need), col, xr);
                    ++g;
                } else if (pre == P) {
                    if (q2 < need) emit<K>(a, row, g + q2, col, xr);
                    ++q2;
                }
            }
    }
    if (c == 0 && t == 0 && a.nan_flag) a.nan_flag[row] = (uint8_t)row_nan;

    if (SPLIT) {
        // Leave the slot zeroed for the next call (whose slot layout may
        // differ): every workgroup has read the histograms before the last
        // rendezvous, so each clears a share now; the last workgroup out,
        // once every workgroup has read the counts, clears them and resets
        // the counters.
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
}

template <class K, int EPT, bool SPLIT>
const void *kptr() {
    return reinterpret_cast<const void *>(&topk_rows_kernel<K, EPT, SPLIT>);
}

template <bool SPLIT>
const void *pick_bf16(int ept) {
    switch (ept) {
        case 8: return kptr<Bf16Key, 8, SPLIT>();
        case 16: return kptr<Bf16Key, 16, SPLIT>();
        case 32: return kptr<Bf16Key, 32, SPLIT>();
        case 64: return kptr<Bf16Key, 64, SPLIT>();
        default: return nullptr;
    }
}

template <bool SPLIT>
const void *pick_f32(int ept) {
    switch (ept) {
        case 4: return kptr<F32Key, 4, SPLIT>();
        case 8: return kptr<F32Key, 8, SPLIT>();
        case 16: return kptr<F32Key, 16, SPLIT>();
        case 32: return kptr<F32Key, 32, SPLIT>();
        case 64: return kptr<F32Key, 64, SPLIT>();
        default: return nullptr;
    }
}

}  // namespace

const void *topk_kernel_ptr(int dtype, int ept, bool split) {
    if (dtype == 0) return split ? pick_bf16<true>(ept) : pick_bf16<false>(ept);
    return split ? pick_f32<true>(ept) : pick_f32<false>(ept);
}

size_t topk_dyn_lds(int dtype, int64_t cap) {
    const size_t ksz = dtype == 0 ? 2 : 4;
    return ((size_t)cap * ksz + 3) / 4 * 4 + (size_t)cap * 4;
}

hipError_t launch_topk(int dtype, int ept, bool split, const TopkArgs &a, unsigned grid,
                       hipStream_t stream) {
    const void *fn = topk_kernel_ptr(dtype, ept, split);
    if (!fn) return hipErrorInvalidValue;
    TopkArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(NT), args, topk_dyn_lds(dtype, a.cap), stream);
}

}  // namespace dsel
