// Row-wise top-k for gfx950: radix select over order-preserving keys with a
// candidate filter, then a stable (column-ordered) compaction.
//
// What is computed (DeepSelect tutorial, "Sheshisa Imisebenzi ye-PyTorch TopK
// nge-DeepSelect": basic usage, variable-length rows, NaN handling): for each
// row the c = min(k, n) largest entries of the valid prefix x[0:n), n the
// clamped per-row exclusive end; equal values keep column order, NaN ranks
// above +inf, -0 equals +0; the selected columns are written in ascending
// order (or, on request, by value), short rows padded with the fill index
// and value (-1 / -inf unless the call gives others); a per-row flag reports
// NaN in rows longer than k.
//
// How (this file's design, not the pages'):
//   * a key is the value's bits mapped to an unsigned integer whose order is
//     the ranking order (sign-magnitude -> offset binary, so -0 and +0 meet;
//     every NaN -> the largest key); bf16 keys are formed two per VGPR with
//     packed 16-bit integer ops.  The map is invertible except at the +-0
//     and NaN keys, so a selected value is rebuilt from its key and only
//     those two keys re-read the row;
//   * a workgroup holds its columns in VGPRs in the coalesced layout (load j
//     of thread t holds the 16 bytes at column (j*NT + t)*VEC of its range),
//     all loads issued at once; it histograms an 11-bit first digit in LDS;
//   * the bin holding the k-th largest key fixes a threshold T1; only the C
//     candidates with key >= T1 (about k plus one bin) are compacted, in
//     column order, into an LDS list (bf16: one word per entry, key << 16 |
//     column; fp32: key and column words side by side);
//   * the rest of the radix select (5 more bits for bf16, 11+10 for fp32)
//     runs on that short list; the selection, every key > T plus the first
//     `need` keys == T in column order, is written in column order: each
//     thread owns a contiguous run of the list and one workgroup scan gives
//     its ranks.  The output is ascending by construction; no sort is run;
//   * a workgroup holding at most two loads per thread with dense candidates
//     skips the list: the later passes and the write work on its VGPRs;
//   * rows of at most 2048 columns take one wave each: the keys in VGPRs, a
//     per-wave LDS histogram and wave scans only, so no row waits on a
//     workgroup barrier and four rows run side by side per workgroup;
//   * rows longer than one workgroup holds (16384 columns) are split over G
//     workgroups, each holding one chunk.  bf16 rows first try the one
//     exchange: each workgroup lists its keys from the floor of its own
//     top-k bin (the row's k-th largest key cannot lie below it), publishes
//     their suffix counts, and one rendezvous gives every workgroup the exact
//     threshold and its starting ranks.  Otherwise (and for fp32) the
//     histograms meet in a per-row workspace slot (device-scope relaxed
//     atomics and a rendezvous per radix pass); each workgroup lists its own
//     candidates; the last pass also carries each workgroup's counts, which
//     give every workgroup the ranks of the chunks before its own.  Either
//     way each workgroup writes its part of the row's output;
//   * if a candidate list would not fit (massive ties at the threshold), the
//     radix select finishes over the range re-read from cache (slower, same
//     result);
//   * value order (sorted_index 2) is a separate pass after the select: one
//     workgroup per row sorts its (key, column) pairs with a stable radix
//     sort in LDS, largest value first, equal values by ascending column.
#include "dsel_internal.h"

namespace dsel {
namespace {

// Phase stamps, compiled only into the instrumented build (DSEL_PHASE_STAMPS,
// built and read by sparse_attention_indexer_dsel_amd/phase_stamps.py): when
// one thread reaches a phase boundary it records the 100 MHz real-time clock
// in slot (unit, i) of a device array, where a unit is a row (one-wave and
// whole rows) or a workgroup (split fp32 rows).  The stamp does not wait for
// the thread's memory operations (a wait would hold back the loads' overlap
// with the work), so it marks when the boundary's instructions issue; a
// phase that ends in a workgroup barrier ends when every wave has reached
// it.  The product build compiles every stamp to nothing.
#ifdef DSEL_PHASE_STAMPS
constexpr int kStampUnits = 4096, kStampsPerUnit = 24;
__device__ unsigned long long g_stamps[kStampUnits * kStampsPerUnit];
__device__ __forceinline__ void stamp_at(bool who, int64_t unit, int i) {
    const unsigned long long t = __builtin_amdgcn_s_memrealtime();
    if (who && unit >= 0 && unit < kStampUnits) g_stamps[unit * kStampsPerUnit + i] = t;
}
__device__ __forceinline__ void stamp_value(bool who, int64_t unit, int i, unsigned long long v) {
    if (who && unit >= 0 && unit < kStampUnits) g_stamps[unit * kStampsPerUnit + i] = v;
}
#define DSEL_STAMP(who, unit, i) stamp_at((who), (unit), (i))
#define DSEL_STAMP_VALUE(who, unit, i, v) stamp_value((who), (unit), (i), (v))
#else
#define DSEL_STAMP(who, unit, i) ((void)0)
#define DSEL_STAMP_VALUE(who, unit, i, v) ((void)0)
#endif

constexpr int NT = kTopkThreads;
constexpr int NWAVE = NT / 64;

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
    static constexpr bool PACK = true;  // list entry = key << 16 | column
    __device__ static int digit(int pass) { return pass == 0 ? 11 : 5; }
    static constexpr int digit_last() { return 5; }
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
    // raw word with the elements at and past `valid` (0..2 in this word) zeroed
    __device__ static uint32_t keep_raw(uint32_t w, int valid) {
        return valid >= 2 ? w : (valid == 1 ? (w & 0xFFFFu) : 0u);
    }
    // keys whose value cannot be rebuilt: +-0 and NaN
    __device__ static bool ambiguous(uint32_t key) { return key == 0x8000u || key == 0xFFFFu; }
    __device__ static uint32_t value_bits(uint32_t key) {
        return key >= 0x8000u ? key - 0x8000u : (0x8000u - key) | 0x8000u;
    }
};

struct F32Key {
    using raw_t = uint32_t;
    static constexpr int VEC = 4;
    static constexpr int EPW = 1;
    static constexpr int NPASS = 3;
    static constexpr int SH1 = 21;
    static constexpr bool PACK = false;  // list entry = (key, column) in two arrays
    __device__ static int digit(int pass) { return pass == 2 ? 10 : 11; }
    static constexpr int digit_last() { return 10; }
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
    __device__ static uint32_t keep_raw(uint32_t w, int valid) { return valid >= 1 ? w : 0u; }
    __device__ static bool ambiguous(uint32_t key) {
        return key == 0x80000000u || key == 0xFFFFFFFFu;
    }
    __device__ static uint32_t value_bits(uint32_t key) {
        return key >= 0x80000000u ? key - 0x80000000u : (0x80000000u - key) | 0x80000000u;
    }
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

// Inclusive prefix sum within each 16-lane row of the wave.
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    return x;
}

__device__ __forceinline__ uint32_t rdlane(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Lanes below this one whose bit is set in a wave mask.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

// Inclusive prefix sum over the workgroup in thread order, and the
// workgroup's total.
struct Scan {
    uint32_t incl, total;
};

__device__ Scan block_scan(uint32_t x, uint32_t *s_red) {
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
    return Scan{w + off, tot};
}

// block_scan of two values at once (one pair of barriers); s_red2 holds
// 2 * NWAVE words.
struct Scan2 {
    uint32_t incl0, incl1, total0, total1;
};

__device__ Scan2 block_scan2(uint32_t x0, uint32_t x1, uint32_t *s_red2) {
    const int t = tid();
    const uint32_t w0 = wave_incl_scan(x0), w1 = wave_incl_scan(x1);
    if ((t & 63) == 63) {
        s_red2[t >> 6] = w0;
        s_red2[NWAVE + (t >> 6)] = w1;
    }
    __syncthreads();
    Scan2 r{w0, w1, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) {
        const uint32_t v0 = s_red2[i], v1 = s_red2[NWAVE + i];
        r.incl0 += (i < (t >> 6)) ? v0 : 0u;
        r.incl1 += (i < (t >> 6)) ? v1 : 0u;
        r.total0 += v0;
        r.total1 += v1;
    }
    __syncthreads();
    return r;
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
    const uint32_t incl = block_scan(local, s_red).incl;
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

// find_digit for histograms of at least NT bins (nb = NT * bpt, bpt <= 16,
// a multiple of 4) whose bins each pack two counts: all elements in the low
// 16 bits, a subset of them in the high 16 (every sum stays below 2^16).
// Each thread sums its bpt bins with 16-byte reads, one workgroup scan finds
// the thread holding the need-th largest element (by the low counts), and
// every wave then resolves the bin among that thread's bpt bins with one
// 16-lane scan (no serial walk).  The Digit's `above` and `cnt` keep both
// halves: above & 0xFFFF elements lie in higher digits, above >> 16 of them
// in the subset, and likewise for cnt in the digit itself.
__device__ Digit find_digit_fast(const uint32_t *hist, int nb, uint32_t need, uint32_t *s_red,
                                 uint32_t *s_out) {
    const int t = tid();
    const int lane = t & 63;
    const int bpt = nb / NT;
    const int top = nb - t * bpt;  // exclusive upper bin of this thread
    uint32_t local = 0;
    for (int i = 0; i < bpt; i += 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(hist + top - bpt + i);
        local += (q.x + q.y) + (q.z + q.w);
    }
    const uint32_t incl = block_scan(local, s_red).incl;
    const uint32_t excl = incl - local;
    if ((excl & 0xFFFFu) < need && need <= (incl & 0xFFFFu)) {
        s_out[0] = (uint32_t)t;
        s_out[1] = excl;
    }
    __syncthreads();
    const int T = (int)s_out[0];
    const uint32_t ex = s_out[1];
    const int topT = nb - T * bpt;
    const int bin = topT - 1 - (lane & 15);  // descending over the thread's bins
    const uint32_t h = (lane & 15) < bpt ? hist[bin] : 0u;
    const uint32_t cum = ex + row16_incl_scan(h);
    const int L = (int)__builtin_ctzll(__ballot(lane < bpt && (cum & 0xFFFFu) >= need));
    const Digit d{rdlane((uint32_t)bin, L), rdlane(cum - h, L), rdlane(h, L)};
    __syncthreads();  // s_out may be rewritten by the next search
    return d;
}

// Order this wave's LDS accesses (one wave's LDS operations execute in
// order; this keeps the compiler from moving them across phases).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave's search of a 1024-bin histogram for the bin holding the need-th
// largest key (bins counted from the top; the histogram holds at least
// `need` keys): 16 bins per lane with 16-byte reads, one wave scan for the
// lane, one 16-lane scan for the bin (no serial walk).
__device__ __forceinline__ Digit wave_find1024(const uint32_t *hist, uint32_t need, int lane) {
    const uint4 *h4 = reinterpret_cast<const uint4 *>(hist + (1024 - 16) - 16 * lane);
    const uint4 a0 = h4[0], a1 = h4[1], a2 = h4[2], a3 = h4[3];
    const uint32_t local = (a0.x + a0.y + a0.z + a0.w) + (a1.x + a1.y + a1.z + a1.w) +
                           (a2.x + a2.y + a2.z + a2.w) + (a3.x + a3.y + a3.z + a3.w);
    const uint32_t incl = wave_incl_scan(local);
    const int L = (int)__builtin_ctzll(__ballot(incl >= need));
    const uint32_t above = rdlane(incl - local, L);
    // lane i of each row of 16 takes bin 1023 - 16 L - i (descending)
    const int bin = (1024 - 1) - 16 * L - (lane & 15);
    const uint32_t h = hist[bin];
    const uint32_t cum = above + row16_incl_scan(h);
    const int L2 = (int)__builtin_ctzll(__ballot(lane < 16 && cum >= need));
    return Digit{rdlane((uint32_t)bin, L2), rdlane(cum - h, L2), rdlane(h, L2)};
}

// Workgroup search of a 4096-bin histogram for the bin holding the need-th
// largest key, with bank-conflict-free reads: thread t reads the 16 bytes at
// bins 1024 i + 4 t (i < 4; consecutive lanes, consecutive 16 bytes), each
// quad of lanes sums its 16-bin group (DPP), the 256 group sums go through
// LDS (s_grp, 256 words), one workgroup scan over the groups from the top
// finds the group, and one 16-lane scan of its bins finds the bin.
__device__ Digit find_digit_4096(const uint32_t *hist, uint32_t need, uint32_t *s_grp,
                                 uint32_t *s_red, uint32_t *s_out) {
    const int t = tid();
    const int lane = t & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 q = *reinterpret_cast<const uint4 *>(hist + 1024 * i + 4 * t);
        uint32_t v = (q.x + q.y) + (q.z + q.w);
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
        if ((t & 3) == 0) s_grp[64 * i + (t >> 2)] = v;  // group (1024 i + 4 t) / 16
    }
    __syncthreads();
    const uint32_t local = s_grp[255 - t];  // thread t: group 255 - t (from the top)
    const uint32_t incl = block_scan(local, s_red).incl;
    const uint32_t excl = incl - local;
    if (excl < need && need <= incl) {
        s_out[0] = (uint32_t)t;
        s_out[1] = excl;
    }
    __syncthreads();
    const int g = 255 - (int)s_out[0];
    const uint32_t ex = s_out[1];
    const int bin = 16 * g + 15 - (lane & 15);  // descending over the group's bins
    const uint32_t h = hist[bin];
    const uint32_t cum = ex + row16_incl_scan(h);
    const int L = (int)__builtin_ctzll(__ballot(lane < 16 && cum >= need));
    const Digit d{rdlane((uint32_t)bin, L), rdlane(cum - h, L), rdlane(h, L)};
    __syncthreads();  // s_out and s_grp may be rewritten by the next search
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
// past `limit` polls the workgroup records kErrRendezvous in workspace word
// 0 (`err`) and goes on, so every wave always exits; the row's output is
// then undefined and the host learns of it from dsel_topk_check.
//
// Ordering: a workgroup's data for its peers is written with agent-scope
// atomic stores or adds (they bypass the compute unit's L1 and land in L2,
// the agent's point of coherence); the s_waitcnt(0) before the arrival add
// waits until every one of them is acknowledged, so they are visible in L2
// before the arrival is.  A peer that has seen the target count reads with
// agent-scope atomic loads, which also go to L2 and so never return a stale
// L1 line.  No cache-wide release or acquire fence is needed (on gfx950 an
// agent-scope fence writes back and invalidates the whole L2 per workgroup).
__device__ void row_rendezvous(uint32_t *ctr, uint32_t target, uint32_t *err, uint32_t limit) {
    drain_memory();
    __syncthreads();
    if (tid() == 0) {
        add_agent(ctr, 1u);
        uint32_t spins = 0;
        while (ld_agent(ctr) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > limit) {
                __hip_atomic_fetch_or(err, kErrRendezvous, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// Publish this workgroup's histogram bins [0, nb) into a row's global
// histogram (nonzero bins only).
__device__ __forceinline__ void merge_histogram(const uint32_t *hist, uint32_t *ghist, int nb) {
    for (int b = tid(); b < nb; b += NT) {
        const uint32_t h = hist[b];
        if (h) add_agent(ghist + b, h);
    }
}

// Read a row's global histogram bins [0, nb) (nb <= kBins) into LDS, all
// loads in flight at once.
__device__ __forceinline__ void fetch_histogram(const uint32_t *ghist, uint32_t *hist, int nb) {
    constexpr int R = kBins / NT;
    uint32_t v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int b = i * NT + tid();
        v[i] = b < nb ? ld_agent(ghist + b) : 0u;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int b = i * NT + tid();
        if (b < nb) hist[b] = v[i];
    }
}

// Publish a workgroup's counts at the last radix pass, given its histogram
// of that pass's digit (nb bins) and `above`, its keys above the current
// prefix: word j of dst (j in [0, nb]) = above + its keys at the prefix
// whose digit is >= j.  Once the digit v is known, words v+1 and v are the
// chunk's taken-above count and (by difference) its count at the boundary.
__device__ __forceinline__ void publish_suffix(const uint32_t *hist, int nb, uint32_t above,
                                               uint32_t *dst, uint32_t *s_red) {
    const int t = tid();
    const int bpt = nb > NT ? nb / NT : 1;
    const int nact = nb / bpt;
    const int top = nb - t * bpt;  // exclusive upper bin of this thread
    uint32_t local = 0;
    if (t < nact)
        for (int i = 1; i <= bpt; ++i) local += hist[top - i];
    uint32_t acc = above + block_scan(local, s_red).incl - local;
    if (t < nact)
        for (int i = 1; i <= bpt; ++i) {
            acc += hist[top - i];
            st_agent(dst + top - i, acc);
        }
    if (t == 0) st_agent(dst + nb, above);
}

// A row's output slots, resolved once per row (uniform: held in SGPRs).
struct RowOut {
    char *idx;  // the row's index slots
    char *val;  // the row's value slots, or nullptr without values
    uint32_t k;
    int idx64;
};

template <class K>
__device__ __forceinline__ RowOut row_out(const TopkArgs &a, int64_t row) {
    RowOut o;
    o.idx = reinterpret_cast<char *>(a.out_idx) + row * a.idx_stride * (a.idx64 ? 8 : 4);
    o.val = a.ret_val ? reinterpret_cast<char *>(a.out_val) +
                            row * a.val_stride * (int64_t)sizeof(typename K::raw_t)
                      : nullptr;
    o.k = (uint32_t)a.k;
    o.idx64 = a.idx64;
    return o;
}

// 16 bytes of output with the non-temporal hint: the outputs are written
// once and not read back by the select.
__device__ __forceinline__ void store16_nt(void *p, uint4 v) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t *>(p));
}

// Output slot `pos`: its column, and (with values) the value bits.
// NTS: with the non-temporal hint.  The whole-row kernel's writers take it
// (measured faster, though its scattered 4-byte stores then leave L2 as
// partial lines: 2.5x the write bytes); its instance that fuses the gather,
// whose workers read the positions back at once, and the split rows' writes
// (a few slots per workgroup, measured slower with it) do not.
template <bool NTS = false, class T>
__device__ __forceinline__ void store_out(T *p, T v) {
    if constexpr (NTS) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool NTS = false>
__device__ __forceinline__ void store_index(const RowOut &o, uint32_t pos, uint32_t col) {
    if (pos >= o.k) return;  // never write past the row's k slots
    if (o.idx64)
        store_out<NTS>(reinterpret_cast<int64_t *>(o.idx) + pos, (int64_t)col);
    else
        store_out<NTS>(reinterpret_cast<int32_t *>(o.idx) + pos, (int32_t)col);
}

template <class K, bool NTS = false>
__device__ __forceinline__ void store_value(const RowOut &o, uint32_t pos, uint32_t bits) {
    if (pos >= o.k) return;
    store_out<NTS>(reinterpret_cast<typename K::raw_t *>(o.val) + pos, (typename K::raw_t)bits);
}

// One selected element: its column at output slot `pos`, and its value,
// rebuilt from the key (read back from the row only for +-0 and NaN keys,
// whose bits the key does not determine).
template <class K, bool NTS = false>
__device__ __forceinline__ void emit(const RowOut &o, uint32_t pos, uint32_t col, uint32_t key,
                                     const typename K::raw_t *xr) {
    store_index<NTS>(o, pos, col);
    if (o.val)
        store_value<K, NTS>(o, pos, K::ambiguous(key) ? (uint32_t)xr[col] : K::value_bits(key));
}

// Range-checked view of one row's first `end` columns for raw buffer loads:
// bytes at or past the (dword-rounded) end read as zero without touching
// memory, so every 16-byte load is unconditional.  The rounding keeps a
// partly valid dword whole; the element past the end is masked by the
// caller before it is looked at.
template <class K>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_view(const typename K::raw_t *xr, int64_t end) {
    const int64_t bytes = end > 0 ? ((end * (int64_t)sizeof(typename K::raw_t) + 3) & ~(int64_t)3) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<typename K::raw_t *>(xr), (short)0,
                                             (int)bytes, 0x00020000);
}

// 16 bytes of raw values at column p of a row view.  NTL: with the
// non-temporal hint (cache policy bit nt), for the whole-row and split
// kernels, which read each value once (a streaming read of 66 MB measured
// 7% faster with it); the slow paths' re-reads of a range and the one-wave
// kernels (measured slower with it) use the default policy.
template <class K, bool NTL = true>
__device__ __forceinline__ uint4 load_vec(__amdgpu_buffer_rsrc_t view, int64_t p) {
    constexpr int kNonTemporal = 2;  // the nt bit of a buffer load's cache policy
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
        view, (unsigned)(p * (int64_t)sizeof(typename K::raw_t)), 0u, NTL ? kNonTemporal : 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Short rows (n <= k) hold columns 0..n-1 in order, then padding (the fill
// index and fill value bits the call gives).
//
// The value slots [s0, s1) of a short row, `me` of `nthr` threads sharing
// them: range-checked 16-byte loads over the aligned middle (an element-wise
// load then store waits for every earlier store, since the vector memory
// counter counts stores too), element-wise ends.
template <class K>
__device__ __forceinline__ void write_short_values(typename K::raw_t *ov, typename K::raw_t fill,
                                                   int64_t n, int s0, int s1,
                                                   const typename K::raw_t *xr, int me, int nthr) {
    using raw_t = typename K::raw_t;
    constexpr int VEC = K::VEC;  // elements per 16 bytes
    const int vb = min(s1, (s0 + VEC - 1) / VEC * VEC);
    const int ve = max(vb, s1 / VEC * VEC);
    for (int s = s0 + me; s < vb; s += nthr) ov[s] = s < n ? xr[s] : fill;
    const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, n);
    for (int s = vb + VEC * me; s < ve; s += VEC * nthr) {
        uint4 q = load_vec<K>(view, s);  // bytes past the row end read as zero
        raw_t e[VEC];
        __builtin_memcpy(e, &q, 16);
#pragma unroll
        for (int i = 0; i < VEC; ++i) e[i] = s + i < n ? e[i] : fill;
        __builtin_memcpy(&q, e, 16);
        store16_nt(ov + s, q);
    }
    for (int s = ve + me; s < s1; s += nthr) ov[s] = s < n ? xr[s] : fill;
}

// The index slots [s0, s1) of a short row (int32 in 16-byte stores) and its
// NaN flag.
__device__ __forceinline__ void write_short_idx(const TopkArgs &a, int64_t row, int64_t n, int c,
                                                int s0, int s1, int me, int nthr) {
    if (!a.idx64 && (s0 & 3) == 0) {
        // int32: four slots per 16-byte store
        int32_t *o = reinterpret_cast<int32_t *>(a.out_idx) + row * a.idx_stride;
        const int fill = (int)a.idx_fill;
        const int nv = (s1 - s0) >> 2;
        for (int v = me; v < nv; v += nthr) {
            const int s = s0 + 4 * v;
            int4 q;
            q.x = s < n ? s : fill;
            q.y = s + 1 < n ? s + 1 : fill;
            q.z = s + 2 < n ? s + 2 : fill;
            q.w = s + 3 < n ? s + 3 : fill;
            store16_nt(o + s, make_uint4((uint32_t)q.x, (uint32_t)q.y, (uint32_t)q.z, (uint32_t)q.w));
        }
        for (int s = s0 + 4 * nv + me; s < s1; s += nthr) o[s] = s < n ? s : fill;
    } else {
        for (int s = s0 + me; s < s1; s += nthr) {
            if (a.idx64)
                reinterpret_cast<int64_t *>(a.out_idx)[row * a.idx_stride + s] =
                    s < n ? (int64_t)s : a.idx_fill;
            else
                reinterpret_cast<int32_t *>(a.out_idx)[row * a.idx_stride + s] =
                    s < n ? s : (int32_t)a.idx_fill;
        }
    }
    if (c == 0 && me == 0 && a.nan_flag) a.nan_flag[row] = 0;
}

// One wave's short-row values (slots [0, k)), kept out of line: inlined into
// the one-wave kernel the copy would cost that kernel a wave per SIMD.
template <class K>
__device__ __attribute__((noinline)) void write_short_values_wave(typename K::raw_t *ov,
                                                                  typename K::raw_t fill,
                                                                  int64_t n, int k,
                                                                  const typename K::raw_t *xr,
                                                                  int lane) {
    write_short_values<K>(ov, fill, n, 0, k, xr, lane, 64);
}

// A whole short row, index and value stores in one element-wise loop
// (index-only int32 rows take 16-byte stores).  Workgroup c of G writes
// slots [c*S, (c+1)*S) with S = ceil(k / G); `me` of `nthr` threads (a
// workgroup's, or one wave's lanes) share them.  The whole-row and split
// kernels and the index-only one-wave kernel keep this form: the two writers
// above measured no faster there and moved those kernels' code enough to slow
// their long rows by 1 to 4%.
template <class K>
__device__ __forceinline__ void write_short_row(const TopkArgs &a, int64_t row, int64_t n, int c, int G,
                                const typename K::raw_t *xr, int me = tid(),
                                int nthr = NT) {
    const int S = (a.k + G - 1) / G;
    const int s0 = c * S;
    const int s1 = min(a.k, s0 + S);
    if (!a.idx64 && !a.ret_val && (a.idx_stride & 3) == 0 && (s0 & 3) == 0) {
        // index-only int32: four slots per 16-byte store
        int32_t *o = reinterpret_cast<int32_t *>(a.out_idx) + row * a.idx_stride;
        const int fill = (int)a.idx_fill;
        const int nv = (s1 - s0) >> 2;
        for (int v = me; v < nv; v += nthr) {
            const int s = s0 + 4 * v;
            int4 q;
            q.x = s < n ? s : fill;
            q.y = s + 1 < n ? s + 1 : fill;
            q.z = s + 2 < n ? s + 2 : fill;
            q.w = s + 3 < n ? s + 3 : fill;
            store16_nt(o + s, make_uint4((uint32_t)q.x, (uint32_t)q.y, (uint32_t)q.z, (uint32_t)q.w));
        }
        for (int s = s0 + 4 * nv + me; s < s1; s += nthr) o[s] = s < n ? s : fill;
    } else {
        for (int s = s0 + me; s < s1; s += nthr) {
            const bool in = s < n;
            if (a.idx64)
                reinterpret_cast<int64_t *>(a.out_idx)[row * a.idx_stride + s] =
                    in ? (int64_t)s : a.idx_fill;
            else
                reinterpret_cast<int32_t *>(a.out_idx)[row * a.idx_stride + s] =
                    in ? s : (int32_t)a.idx_fill;
            if (a.ret_val)
                reinterpret_cast<typename K::raw_t *>(a.out_val)[row * a.val_stride + s] =
                    in ? xr[s] : (typename K::raw_t)a.val_fill;
        }
    }
    if (c == 0 && me == 0 && a.nan_flag) a.nan_flag[row] = 0;
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

// Keys of a workgroup's loads in the coalesced layout (load j of thread t
// holds the VEC columns from (j*TW + t)*VEC of a range of `len` columns; TW
// is NT, or 64 for one wave's lanes).
// Columns at or past len get key 0 and are not probed for NaN; loads wholly
// past len are not transformed at all.  Returns whether this thread saw a
// NaN.
// PER_VECTOR: the NaN fix-up branch per 16-byte vector instead of once over
// every load (the fused gather's whole-row kernel keeps its registers that
// way).
template <class K, int LOADS, int TW = NT, bool PER_VECTOR = false>
__device__ __forceinline__ uint32_t keys_of_loads(const uint4 (&v)[LOADS], int len,
                                                  uint32_t (&kw)[LOADS * 4], int me = tid()) {
    constexpr int VEC = K::VEC, EPW = K::EPW;
    const int full = len / (TW * VEC);  // loads valid for every thread (uniform)
    const int any = (len + TW * VEC - 1) / (TW * VEC);
    uint32_t m = 0;  // NaN probe over every load: one branch, taken only with a NaN
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if (j >= any) {
#pragma unroll
            for (int q = 0; q < 4; ++q) kw[4 * j + q] = 0u;
            continue;
        }
        uint4 x = v[j];
        int valid = VEC;
        if (j >= full) {
            valid = len - (j * TW + me) * VEC;
            valid = valid < 0 ? 0 : (valid > VEC ? VEC : valid);
            x.x = K::keep_raw(x.x, valid);
            x.y = K::keep_raw(x.y, valid - EPW);
            x.z = K::keep_raw(x.z, valid - 2 * EPW);
            x.w = K::keep_raw(x.w, valid - 3 * EPW);
        }
        if constexpr (PER_VECTOR) {
            m |= keys_of<K>(x, &kw[4 * j]) ? 1u : 0u;
        } else {
            kw[4 * j] = K::keyword(x.x, m);
            kw[4 * j + 1] = K::keyword(x.y, m);
            kw[4 * j + 2] = K::keyword(x.z, m);
            kw[4 * j + 3] = K::keyword(x.w, m);
        }
        if (j >= full) clear_tail<K>(&kw[4 * j], valid);
    }
    if constexpr (PER_VECTOR) return m;
    const bool nan = K::probe_nan(m);
    if (nan) {
#pragma unroll
        for (int w = 0; w < LOADS * 4; ++w) kw[w] = K::fix_nan_word(kw[w]);
    }
    return nan ? 1u : 0u;
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

// First-digit histogram of a workgroup's keys (hist zeroed, kBins + 64 bins).
template <class K, int LOADS>
__device__ __forceinline__ void first_digit_histogram(const uint32_t (&kw)[LOADS * 4], int len,
                                                      uint32_t *hist) {
    constexpr int SPAN = NT * K::VEC;
    const int full = len / SPAN, any = (len + SPAN - 1) / SPAN;
    const uint32_t spare = kBins + (tid() & 63);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if (j < full) {
#pragma unroll
            for (int q = 0; q < 4; ++q) hist_add<K>(hist, kw[4 * j + q]);
        } else if (j < any) {
#pragma unroll
            for (int q = 0; q < 4; ++q) hist_add_masked<K>(hist, kw[4 * j + q], spare);
        }
    }
}

// A candidate list in LDS, cap entries plus one spare entry per lane.  A
// bf16 entry is one word, key << 16 | column (columns of a workgroup's range
// are below 2^16); an fp32 entry is two words, key then column.  Either way
// an entry sits at one address (the column at immediate offset 4), so a
// compaction store needs no per-element address arithmetic beyond one
// select.
struct List {
    uint32_t *w;
};

template <class K>
__device__ __forceinline__ List list_of(uint32_t *s_dyn) {
    return List{s_dyn};
}

// Words per entry.
template <class K>
__host__ __device__ constexpr uint32_t list_words() {
    return K::PACK ? 1u : 2u;
}

// Store an entry at p (an entry slot of a list).
template <class K>
__device__ __forceinline__ void list_store(uint32_t *p, uint32_t key, uint32_t col) {
    if constexpr (K::PACK) {
        p[0] = (key << 16) | col;
    } else {
        p[0] = key;
        p[1] = col;
    }
}

template <class K>
__device__ __forceinline__ uint32_t list_key(List ent, uint32_t i) {
    if constexpr (K::PACK) return ent.w[i] >> 16;
    return ent.w[2 * i];
}

// (key, column) of entry i
template <class K>
__device__ __forceinline__ uint2 list_entry(List ent, uint32_t i) {
    if constexpr (K::PACK) {
        const uint32_t e = ent.w[i];
        return make_uint2(e >> 16, e & 0xFFFFu);
    }
    return *reinterpret_cast<const uint2 *>(ent.w + 2 * i);
}

// Compact the candidates (key >= T1, T1 > 0) of a workgroup's keys into
// ent[0, run) in column order (entry = (key, column within the range));
// returns run.
// Every element is written once, the non-candidates to this lane's spare
// entry (entry cap + lane), so the loop has no branches.  CHECKED: when more
// than `cap` qualify nothing is written (the count is still returned).  wtot
// holds LP*NWAVE words, base LOADS*NWAVE + 1: one wave turns the per-(load,
// wave) counts into list offsets once, so each load costs a thread one LDS
// read.
// RAWF (fp32 only): kw holds raw float bits and T1 the bits of a float; the
// candidates are the elements x >= T1 as floats (-0 == +0; a NaN, the filler
// of columns past len, never qualifies).
template <class K, int LOADS, bool CHECKED = false, bool RAWF = false>
__device__ __forceinline__ uint32_t compact_candidates(uint32_t (&kw)[LOADS * 4], int len,
                                                       uint32_t T1, uint32_t *wtot,
                                                       uint32_t *base, List ent, uint32_t cap) {
    static_assert(!RAWF || !K::PACK, "raw float candidates: 32-bit elements");
    auto qualifies = [](uint32_t key, uint32_t t1) {
        if constexpr (RAWF) return __uint_as_float(key) >= __uint_as_float(t1);
        return key >= t1;
    };
    constexpr int VEC = K::VEC, EPW = K::EPW, LP = (LOADS + 1) / 2, SPAN = NT * VEC;
    const int t = tid();
    const int lane = t & 63, wid = t >> 6;
    const int any = (len + SPAN - 1) / SPAN;
    // per-load counts, two loads per word (each count <= 512 per wave)
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
                for (int h = 0; h < EPW; ++h) m += qualifies(K::elem(kw[4 * j + q], h), T1) ? 1u : 0u;
            pk[j >> 1] |= m << ((j & 1) * 16);
        }
    }
    uint32_t ex[LP];
#pragma unroll
    for (int i = 0; i < LP; ++i) {
        const uint32_t incl = wave_incl_scan(pk[i]);
        ex[i] = incl - pk[i];
        if (lane == 63) wtot[i * NWAVE + wid] = incl;
    }
    __syncthreads();
    // wave 0: exclusive prefix of the (load, wave) counts in column order
    // (load-major), two entries per lane
    constexpr int NE = LOADS * NWAVE;
    static_assert(NE <= 128, "two (load, wave) entries per lane of one wave");
    if (wid == 0) {
        uint32_t c[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = 2 * lane + u, j = e / NWAVE, w = e % NWAVE;
            c[u] = e < NE ? (wtot[(j >> 1) * NWAVE + w] >> ((j & 1) * 16)) & 0xFFFFu : 0u;
        }
        const uint32_t pair = c[0] + c[1];
        const uint32_t incl = wave_incl_scan(pair);
        if (2 * lane < NE) base[2 * lane] = incl - pair;
        if (2 * lane + 1 < NE) base[2 * lane + 1] = incl - c[1];
        if (lane == 63) base[NE] = incl;
    }
    __syncthreads();
    const uint32_t total = base[NE];
    if (CHECKED && total > cap) return total;  // uniform
    const uint32_t T1w = opaque(T1);
#pragma unroll
    for (int w = 0; w < LOADS * 4; ++w) kw[w] = opaque(kw[w]);
    constexpr uint32_t WPE = list_words<K>();
    uint32_t *const spare = ent.w + WPE * (cap + lane);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if (j < any) {
            const int i = j >> 1, sh = (j & 1) * 16;
            // slot of this thread's next candidate of this load
            uint32_t *next = ent.w + WPE * (base[j * NWAVE + wid] + ((ex[i] >> sh) & 0xFFFFu));
            const uint32_t p = (uint32_t)(j * NT + t) * VEC;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int h = 0; h < EPW; ++h) {
                    const uint32_t key = K::elem(kw[4 * j + q], h);
                    const bool cand = qualifies(key, T1w);
                    list_store<K>(cand ? next : spare, key, p + q * EPW + h);
                    next += cand ? WPE : 0u;
                }
        }
    }
    __syncthreads();
    return total;
}

// The boundary of a selection: every key whose top bits (key >> s) exceed P
// is taken, plus the first `need` (in column order) whose top bits equal P.
struct Bound {
    uint32_t P;
    int s;
    uint32_t need;
};

// Histogram of the next digit ((key >> sh) & dmask) of the list entries
// whose top bits (key >> s) equal P (hist zeroed).  Reads are unconditional
// (clamped index, masked result) so several are in flight.
template <class K>
__device__ __forceinline__ void list_refine_histogram(List ent, uint32_t C, uint32_t P, int s,
                                                      int sh, uint32_t dmask, uint32_t *hist) {
    constexpr int U = 4;
    for (uint32_t i0 = 0; i0 < C; i0 += U * NT) {
        uint32_t key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = i0 + u * NT + tid();
            const uint32_t kk = list_key<K>(ent, i < C ? i : 0u);
            key[u] = i < C ? kk : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (key[u] && (key[u] >> s) == P) atomicAdd(&hist[(key[u] >> sh) & dmask], 1u);
    }
}

// The radix passes after the first digit d1, within one workgroup: each
// zeroes the pass's bins, has fill(P, s, sh, dmask) histogram the next digit
// ((key >> sh) & dmask) of the keys whose top bits (key >> s) equal P, and
// finds the digit holding the need-th key.  They stop early when a boundary
// bin is taken whole.
template <class K, class Fill>
__device__ __forceinline__ Bound refine_passes(Digit d1, uint32_t k, uint32_t *s_hist,
                                               uint32_t *s_red, uint32_t *s_out, Fill fill) {
    const int t = tid();
    Bound b{d1.v, K::SH1, k - d1.above};
    if (d1.cnt == b.need) return b;  // the boundary bin is taken whole
#pragma unroll 1
    for (int pass = 1; pass < K::NPASS; ++pass) {
        const int d = K::digit(pass);
        const int sh = b.s - d;
        const int nb = 1 << d;
        for (int i = t; i < nb; i += NT) s_hist[i] = 0;
        __syncthreads();
        fill(b.P, b.s, sh, (1u << d) - 1u);
        __syncthreads();
        const Digit dg = find_digit(s_hist, nb, b.need, s_red, s_out);
        b.need -= dg.above;
        b.P = (b.P << d) | dg.v;
        b.s = sh;
        if (dg.cnt == b.need) break;
    }
    return b;
}

// Resolve the digits after the first among the candidate list's entries
// (every entry's first digit is >= d1.v).
template <class K>
__device__ Bound refine_on_list(List ent, uint32_t C, Digit d1, uint32_t k,
                                uint32_t *s_hist, uint32_t *s_red, uint32_t *s_out) {
    return refine_passes<K>(d1, k, s_hist, s_red, s_out,
                            [&](uint32_t P, int s, int sh, uint32_t dmask) {
                                list_refine_histogram<K>(ent, C, P, s, sh, dmask, s_hist);
                            });
}

// This workgroup's list totals: entries taken above the boundary (top bits >
// P) and entries at it (== P), packed (equal << 16 | above).
template <class K>
__device__ uint32_t list_counts(List ent, uint32_t C, Bound b, uint32_t *s_red) {
    uint32_t g = 0, q = 0;
    for (uint32_t i0 = 0; i0 < C; i0 += NT) {
        const uint32_t i = i0 + tid();
        const uint32_t kk = list_key<K>(ent, i < C ? i : 0u);
        const uint32_t key = i < C ? kk : 0u;
        g += (key && (key >> b.s) > b.P) ? 1u : 0u;
        q += (key && (key >> b.s) == b.P) ? 1u : 0u;
    }
    return block_scan(g | (q << 16), s_red).total;
}

// Write the selection from a column-ordered candidate list whose columns are
// relative to col0; gt0 / eq0 are the taken-above and equal counts of the
// row's columns before the list's.  Thread t owns the contiguous entries
// [t*E, (t+1)*E) (E = ceil(C / NT)): it counts them, one workgroup scan
// gives its starting ranks, and it writes them.  Values are rebuilt from
// keys, so the write loop issues no loads (a load there would make every
// store wait for the ones before it); the rare +-0 / NaN keys get their bits
// from the row in a third pass, run only when some thread holds one.
template <class K, bool NTS = false>
__device__ __forceinline__ void write_from_list(const TopkArgs &a, int64_t row, List ent,
                                                uint32_t C, Bound b, uint32_t *s_red,
                                                const typename K::raw_t *xr, uint32_t gt0 = 0,
                                                uint32_t eq0 = 0, uint32_t col0 = 0) {
    constexpr int U = 4;
    const RowOut o = row_out<K>(a, row);
    const uint32_t E = (C + NT - 1) / NT;
    const uint32_t i0 = (uint32_t)tid() * E;
    const uint32_t i1 = min(C, i0 + E);
    // entry i of this thread's range, read unconditionally (clamped, then
    // masked) so several reads can be in flight
    auto entry = [&](uint32_t i) {
        const uint2 e = list_entry<K>(ent, i < i1 ? i : 0u);
        return i < i1 ? e : make_uint2(0u, 0u);
    };
    uint32_t g = 0, q = 0, amb = 0;
    for (uint32_t i = i0; i < i0 + E; i += U) {
        uint32_t key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) key[u] = entry(i + u).x;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t pre = key[u] >> b.s;
            const bool gt = key[u] && pre > b.P, eq = key[u] && pre == b.P;
            g += gt ? 1u : 0u;
            q += eq ? 1u : 0u;
            amb |= ((gt || eq) && K::ambiguous(key[u])) ? 1u : 0u;
        }
    }
    // packed (equal << 16 | above): above < 2^12 and equal <= C < 2^16
    const uint32_t mine = g | (q << 16);
    const uint32_t ex = block_scan(mine, s_red).incl - mine;
    const uint32_t gb0 = gt0 + (ex & 0xFFFFu), qb0 = eq0 + (ex >> 16);
    uint32_t gb = gb0, qb = qb0;
    for (uint32_t i = i0; i < i0 + E; i += U) {
        uint2 e[U];
#pragma unroll
        for (int u = 0; u < U; ++u) e[u] = entry(i + u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t pre = e[u].x >> b.s;
            if (e[u].x && pre > b.P) {
                const uint32_t pos = gb + min(qb, b.need);
                store_index<NTS>(o, pos, e[u].y + col0);
                if (o.val) store_value<K, NTS>(o, pos, K::value_bits(e[u].x));
                ++gb;
            } else if (e[u].x && pre == b.P) {
                if (qb < b.need) {
                    store_index<NTS>(o, gb + qb, e[u].y + col0);
                    if (o.val) store_value<K, NTS>(o, gb + qb, K::value_bits(e[u].x));
                }
                ++qb;
            }
        }
    }
    if (!(o.val && __syncthreads_or((int)amb))) return;
    gb = gb0;
    qb = qb0;
    for (uint32_t i = i0; i < i1; ++i) {
        const uint2 e = entry(i);
        const uint32_t pre = e.x >> b.s;
        if (e.x && pre > b.P) {
            if (K::ambiguous(e.x))
                store_value<K, NTS>(o, gb + min(qb, b.need), (uint32_t)xr[e.y + col0]);
            ++gb;
        } else if (e.x && pre == b.P) {
            if (qb < b.need && K::ambiguous(e.x))
                store_value<K, NTS>(o, gb + qb, (uint32_t)xr[e.y + col0]);
            ++qb;
        }
    }
}

// A row's output slots as range-checked buffer views: a store at offset
// kDrop (past every view's end) is dropped, so a store loop needs no branch.
struct RowViews {
    __amdgpu_buffer_rsrc_t idx, val;
    int idx64, has_val;
};
constexpr uint32_t kDrop = 0x80000000u;

template <class K>
__device__ __forceinline__ RowViews row_views(const TopkArgs &a, int64_t row) {
    RowViews v;
    const int isz = a.idx64 ? 8 : 4;
    v.idx = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<char *>(a.out_idx) + row * a.idx_stride * isz, (short)0, a.k * isz,
        0x00020000);
    v.val = __builtin_amdgcn_make_buffer_rsrc(
        a.ret_val ? reinterpret_cast<char *>(a.out_val) +
                        row * a.val_stride * (int64_t)sizeof(typename K::raw_t)
                  : reinterpret_cast<char *>(a.out_idx),
        (short)0, a.ret_val ? a.k * (int)sizeof(typename K::raw_t) : 0, 0x00020000);
    v.idx64 = a.idx64;
    v.has_val = a.ret_val;
    return v;
}

// Slot `pos` (or nothing, when !take): the value bits.
template <class K>
__device__ __forceinline__ void view_store_value(const RowViews &v, bool take, uint32_t pos,
                                                 uint32_t bits) {
    if constexpr (sizeof(typename K::raw_t) == 2)
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bits, v.val, take ? pos * 2u : kDrop,
                                              0u, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(bits, v.val, take ? pos * 4u : kDrop, 0u, 0);
}

// Slot `pos` (or nothing, when !take): the column, and the value bits.
template <class K>
__device__ __forceinline__ void view_store(const RowViews &v, bool take, uint32_t pos, uint32_t col,
                                           uint32_t bits) {
    if (v.idx64) {
        const uint64_t c = col;
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, c), v.idx,
            take ? pos * 8u : kDrop, 0u, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(col, v.idx, take ? pos * 4u : kDrop, 0u, 0);
    }
    if (v.has_val) view_store_value<K>(v, take, pos, bits);
}

// Write the selection from a column-ordered list when the boundary is an
// exact key T: every entry with key > T, and the first `need` (in column
// order, counting the eq0 before the list) with key == T.  Same ranks as
// write_from_list.  The workgroup's selected entries fill one contiguous run
// of output slots; when the run fits `stage` (kStageSlots slots: columns,
// then 16-bit values), each thread puts its entries there by rank and the
// run is copied out with consecutive stores (a list holds many more entries
// than it selects, so stores straight from the list would scatter a few
// lanes over many store instructions).  The stage takes kStageSlots column
// words then kStageSlots keys (16 or 32 bits).
constexpr uint32_t kStageSlots = 1024;

template <class K>
__device__ __forceinline__ void write_exact(const TopkArgs &a, int64_t row, List ent, uint32_t C,
                                            uint32_t T, uint32_t need, uint32_t gt0, uint32_t eq0,
                                            uint32_t col0, uint32_t *s_red, uint32_t *stage,
                                            const typename K::raw_t *xr) {
    using skey_t = typename K::raw_t;  // a key has the width of its value
    constexpr int U = 4;
    const RowOut o = row_out<K>(a, row);
    const RowViews v = row_views<K>(a, row);
    const uint32_t E = (C + NT - 1) / NT;
    const uint32_t i0 = (uint32_t)tid() * E;
    const uint32_t i1 = min(C, i0 + E);
    auto entry = [&](uint32_t i) {
        const uint2 e = list_entry<K>(ent, i < i1 ? i : 0u);
        return i < i1 ? e : make_uint2(0u, 0u);
    };
    uint32_t g = 0, q = 0;
    for (uint32_t i = i0; i < i0 + E; i += U) {
        uint32_t key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) key[u] = entry(i + u).x;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            g += key[u] > T ? 1u : 0u;
            q += key[u] == T ? 1u : 0u;
        }
    }
    const uint32_t mine = g | (q << 16);
    const Scan sc = block_scan(mine, s_red);
    const uint32_t ex = sc.incl - mine;
    const uint32_t gb0 = gt0 + (ex & 0xFFFFu), qb0 = eq0 + (ex >> 16);
    // this workgroup's run of slots [p0, p1)
    const uint32_t p0 = gt0 + min(eq0, need);
    const uint32_t p1 = gt0 + (sc.total & 0xFFFFu) + min(eq0 + (sc.total >> 16), need);
    uint32_t gb = gb0, qb = qb0;
    if (p1 - p0 <= kStageSlots) {
        // columns and keys by rank; no global access in this loop (a load
        // here would make each iteration wait for every outstanding one)
        uint32_t *s_col = stage;
        skey_t *s_key = reinterpret_cast<skey_t *>(stage + kStageSlots);
        for (uint32_t i = i0; i < i0 + E; i += U) {
            uint2 e[U];
#pragma unroll
            for (int u = 0; u < U; ++u) e[u] = entry(i + u);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool gt = e[u].x > T, eq = e[u].x == T;
                const uint32_t pos = gt ? gb + min(qb, need) : gb + qb;
                if (gt || (eq && qb < need)) {
                    s_col[pos - p0] = e[u].y + col0;
                    s_key[pos - p0] = (skey_t)e[u].x;
                }
                gb += gt ? 1u : 0u;
                qb += eq ? 1u : 0u;
            }
        }
        __syncthreads();
        uint32_t amb = 0;
        for (uint32_t j = (uint32_t)tid(); j < p1 - p0; j += NT) {
            const uint32_t key = s_key[j];
            store_index(o, p0 + j, s_col[j]);
            if (o.val) store_value<K>(o, p0 + j, K::value_bits(key));
            amb |= K::ambiguous(key) ? 1u : 0u;
        }
        // +-0 (and NaN) keys: the value bits come from the row (the same
        // thread rewrites the same slot, so this store lands last)
        if (o.val && __syncthreads_or((int)amb))
            for (uint32_t j = (uint32_t)tid(); j < p1 - p0; j += NT)
                if (K::ambiguous(s_key[j])) store_value<K>(o, p0 + j, (uint32_t)xr[s_col[j]]);
        return;
    }
    uint32_t amb = 0;
    for (uint32_t i = i0; i < i0 + E; i += U) {
        uint2 e[U];
#pragma unroll
        for (int u = 0; u < U; ++u) e[u] = entry(i + u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool gt = e[u].x > T, eq = e[u].x == T;
            const bool take = gt || (eq && qb < need);
            const uint32_t pos = gt ? gb + min(qb, need) : gb + qb;
            view_store<K>(v, take, pos, e[u].y + col0, K::value_bits(e[u].x));
            amb |= (take && K::ambiguous(e[u].x)) ? 1u : 0u;
            gb += gt ? 1u : 0u;
            qb += eq ? 1u : 0u;
        }
    }
    if (!(o.val && __syncthreads_or((int)amb))) return;
    // +-0 (and NaN) keys: the value bits come from the row
    gb = gb0;
    qb = qb0;
    for (uint32_t i = i0; i < i1; ++i) {
        const uint2 e = entry(i);
        const bool gt = e.x > T, eq = e.x == T;
        const uint32_t pos = gt ? gb + min(qb, need) : gb + qb;
        if ((gt || (eq && qb < need)) && K::ambiguous(e.x))
            store_value<K>(o, pos, (uint32_t)xr[e.y + col0]);
        gb += gt ? 1u : 0u;
        qb += eq ? 1u : 0u;
    }
}

// ---- slow path: the candidate list would not fit (massive ties at the
// threshold).  The radix select finishes over the range's keys re-read from
// cache one load at a time, so the rare path adds no VGPRs to the common one.

// Keys of load j of a range of `len` columns starting at column `base` of a
// row view (coalesced layout; columns at or past len get key 0).
template <class K>
__device__ __forceinline__ void reload_keys(__amdgpu_buffer_rsrc_t view, int64_t base, int len,
                                            int j, uint32_t (&w4)[4]) {
    constexpr int VEC = K::VEC, EPW = K::EPW;
    const int p = (j * NT + tid()) * VEC;
    uint4 x = load_vec<K, false>(view, base + p);
    int valid = len - p;
    valid = valid < 0 ? 0 : (valid > VEC ? VEC : valid);
    x.x = K::keep_raw(x.x, valid);
    x.y = K::keep_raw(x.y, valid - EPW);
    x.z = K::keep_raw(x.z, valid - 2 * EPW);
    x.w = K::keep_raw(x.w, valid - 3 * EPW);
    keys_of<K>(x, w4);
    clear_tail<K>(w4, valid);
}

// Refine-pass histogram: the next digit ((key >> sh) & dmask) of every key
// whose top bits (key >> s) equal P.
template <class K>
__device__ void refine_histogram_stream(__amdgpu_buffer_rsrc_t view, int64_t base, int len,
                                        uint32_t P, int s, int sh, uint32_t dmask,
                                        uint32_t *hist) {
    const int loads = (len + NT * K::VEC - 1) / (NT * K::VEC);
#pragma unroll 1
    for (int j = 0; j < loads; ++j) {
        uint32_t w4[4];
        reload_keys<K>(view, base, len, j, w4);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int h = 0; h < K::EPW; ++h) {
                const uint32_t key = K::elem(w4[q], h);
                if (key && (key >> s) == P) atomicAdd(&hist[(key >> sh) & dmask], 1u);
            }
    }
}

// First-digit histogram of the range's keys re-read from cache (columns at
// or past len go to this lane's spare bin).
template <class K>
__device__ void first_digit_histogram_stream(__amdgpu_buffer_rsrc_t view, int64_t base, int len,
                                             uint32_t *hist) {
    const int loads = (len + NT * K::VEC - 1) / (NT * K::VEC);
    const uint32_t spare = kBins + (uint32_t)(tid() & 63);
#pragma unroll 1
    for (int j = 0; j < loads; ++j) {
        uint32_t w4[4];
        reload_keys<K>(view, base, len, j, w4);
#pragma unroll
        for (int q = 0; q < 4; ++q) hist_add_masked<K>(hist, w4[q], spare);
    }
}

// Counts of taken-above (top bits > P) and equal (== P) keys in four key
// words, packed (equal << 16 | above).
template <class K>
__device__ __forceinline__ uint32_t load_counts(const uint32_t (&w4)[4], Bound b) {
    uint32_t g = 0, q = 0;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int h = 0; h < K::EPW; ++h) {
            const uint32_t key = K::elem(w4[qq], h);
            const uint32_t pre = key >> b.s;
            g += (key && pre > b.P) ? 1u : 0u;
            q += (key && pre == b.P) ? 1u : 0u;
        }
    return g | (q << 16);
}

// This thread's packed counts over the whole range.
template <class K>
__device__ uint32_t range_counts(__amdgpu_buffer_rsrc_t view, int64_t base, int len, Bound b) {
    const int loads = (len + NT * K::VEC - 1) / (NT * K::VEC);
    uint32_t mine = 0;
#pragma unroll 1
    for (int j = 0; j < loads; ++j) {
        uint32_t w4[4];
        reload_keys<K>(view, base, len, j, w4);
        mine += load_counts<K>(w4, b);
    }
    return mine;
}

// Write the selection of the range (columns base + ...).  gt0 / eq0 are the
// taken-above and equal counts of the columns before the range; each load is
// one workgroup scan.
template <class K, bool NTS = false>
__device__ __forceinline__ void write_from_stream(const TopkArgs &a, int64_t row,
                                                  __amdgpu_buffer_rsrc_t view, int64_t base,
                                                  int len, Bound b, uint32_t gt0, uint32_t eq0,
                                                  uint32_t *s_red, const typename K::raw_t *xr) {
    const RowOut o = row_out<K>(a, row);
    constexpr int VEC = K::VEC, EPW = K::EPW;
    const int loads = (len + NT * VEC - 1) / (NT * VEC);
    uint32_t gb = gt0, qb = eq0;
#pragma unroll 1
    for (int j = 0; j < loads; ++j) {
        uint32_t w4[4];
        reload_keys<K>(view, base, len, j, w4);
        const uint32_t mine = load_counts<K>(w4, b);
        const Scan sc = block_scan(mine, s_red);
        const uint32_t ex = sc.incl - mine, tot = sc.total;
        uint32_t g1 = gb + (ex & 0xFFFFu), q1 = qb + (ex >> 16);
        const uint32_t p = (uint32_t)(base + (int64_t)(j * NT + tid()) * VEC);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t key = K::elem(w4[qq], h);
                const uint32_t pre = key >> b.s;
                const uint32_t col = p + qq * EPW + h;
                if (key && pre > b.P) {
                    emit<K, NTS>(o, g1 + min(q1, b.need), col, key, xr);
                    ++g1;
                } else if (key && pre == b.P) {
                    if (q1 < b.need) emit<K, NTS>(o, g1 + q1, col, key, xr);
                    ++q1;
                }
            }
        gb += tot & 0xFFFFu;
        qb += tot >> 16;
    }
}

// ---- small ranges (at most two 16-byte loads per thread): no candidate
// list.  The later radix passes and the ranked write work straight from the
// keys in VGPRs, one workgroup scan per load, which costs less than listing
// and re-reading the candidates when each thread holds a few elements.

// Refine-pass histogram of keys held in VGPRs: the next digit of every key
// whose top bits (key >> s) equal P.
template <class K, int LOADS>
__device__ __forceinline__ void refine_histogram_regs(const uint32_t (&kw)[LOADS * 4], uint32_t P,
                                                      int s, int sh, uint32_t dmask,
                                                      uint32_t *hist) {
#pragma unroll
    for (int w = 0; w < LOADS * 4; ++w)
#pragma unroll
        for (int h = 0; h < K::EPW; ++h) {
            const uint32_t key = K::elem(kw[w], h);
            if (key && (key >> s) == P) atomicAdd(&hist[(key >> sh) & dmask], 1u);
        }
}

// This thread's (equal << 16 | above) counts over its keys.
template <class K, int LOADS>
__device__ __forceinline__ uint32_t counts_regs(const uint32_t (&kw)[LOADS * 4], Bound b) {
    uint32_t g = 0, q = 0;
#pragma unroll
    for (int w = 0; w < LOADS * 4; ++w)
#pragma unroll
        for (int h = 0; h < K::EPW; ++h) {
            const uint32_t key = K::elem(kw[w], h);
            const uint32_t pre = key >> b.s;
            g += (key && pre > b.P) ? 1u : 0u;
            q += (key && pre == b.P) ? 1u : 0u;
        }
    return g | (q << 16);
}

// Write the selection from keys held in VGPRs (coalesced layout: this
// range's columns base + (j*NT + t)*VEC + ..., the range a view of the row);
// gt0 / eq0 are the taken-above and equal counts of the row's columns before
// the range.  Values are rebuilt from keys, so the loop issues no loads (a
// load there would make every store wait for the ones before it); if a +-0
// or NaN key was taken, whose bits the key does not determine, the range is
// written again from the row.
template <class K, int LOADS, bool NTS = false>
__device__ __forceinline__ void write_from_regs(const TopkArgs &a, int64_t row,
                                                const uint32_t (&kw)[LOADS * 4], int len, Bound b,
                                                uint32_t gt0, uint32_t eq0,
                                                __amdgpu_buffer_rsrc_t view, int64_t base,
                                                uint32_t *s_red, const typename K::raw_t *xr) {
    constexpr int VEC = K::VEC, EPW = K::EPW, SPAN = NT * VEC;
    const RowOut o = row_out<K>(a, row);
    const int t = tid();
    const int any = (len + SPAN - 1) / SPAN;
    uint32_t gb = gt0, qb = eq0, amb = 0;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if (j < any) {
            const uint32_t mine = counts_regs<K, 1>(
                *reinterpret_cast<const uint32_t(*)[4]>(&kw[4 * j]), b);
            const Scan sc = block_scan(mine, s_red);
            uint32_t g1 = gb + ((sc.incl - mine) & 0xFFFFu), q1 = qb + ((sc.incl - mine) >> 16);
            const uint32_t p = (uint32_t)(base + (int64_t)(j * NT + t) * VEC);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int h = 0; h < EPW; ++h) {
                    const uint32_t key = K::elem(kw[4 * j + qq], h);
                    const uint32_t pre = key >> b.s;
                    const bool gt = key && pre > b.P, eq = key && pre == b.P;
                    const bool take = gt || (eq && q1 < b.need);
                    const uint32_t pos = gt ? g1 + min(q1, b.need) : g1 + q1;
                    if (take) {
                        store_index<NTS>(o, pos, p + qq * EPW + h);
                        if (o.val) store_value<K, NTS>(o, pos, K::value_bits(key));
                        amb |= K::ambiguous(key) ? 1u : 0u;
                    }
                    g1 += gt ? 1u : 0u;
                    q1 += eq ? 1u : 0u;
                }
            gb += sc.total & 0xFFFFu;
            qb += sc.total >> 16;
        }
    }
    if (o.val && __syncthreads_or((int)amb))
        write_from_stream<K, NTS>(a, row, view, base, len, b, gt0, eq0, s_red, xr);
}

__device__ __forceinline__ int64_t valid_length(const TopkArgs &a, int64_t row) {
    int64_t n = a.cols;
    if (a.row_end) {
        const int64_t e = a.row_end[row];
        n = e < 0 ? 0 : (e > a.cols ? a.cols : e);
    }
    return n;
}

// Dynamic LDS of the top-k kernels: the first-digit histogram (kBins bins
// plus one spare bin per lane) at word 0, and the candidate list from word
// list_base.  For bf16 the later radix pass needs only 32 bins, so the list
// overlays the histogram once the first digit is found (the histogram is
// dead by then); fp32's later passes need the full histogram beside it.
template <class K>
__host__ __device__ constexpr uint32_t list_base() {
    return K::NPASS == 2 ? 64u : (uint32_t)(kBins + 64);
}

// Split rows keep the list past the histogram for either key type: the
// one-exchange select builds its list before the row's boundary is known
// and then needs the histogram's space for the exchanged counts.
__host__ __device__ constexpr uint32_t split_list_base() { return (uint32_t)(kBins + 64); }

// Static LDS of the top-k kernels (LOADS 16-byte loads per thread).
template <int LOADS>
struct TopkShared {
    uint32_t wtot[(LOADS + 1) / 2 * NWAVE];  // compaction: per-wave counts
    uint32_t base[LOADS * NWAVE + 1];        // compaction: list offsets
    uint32_t red[NWAVE];
    uint32_t out[8];
};

// The kernels' view of their LDS.
struct TopkLds {
    uint32_t *hist;
    uint32_t *wtot;
    uint32_t *base;
    uint32_t *red;
    uint32_t *out;
};

// ---------------------------------------------------------------------------
// One-exchange select of a split bf16 row (G <= kOneMaxSplit workgroups).
//
// Let b_c be the first-digit bin of chunk c's own k-th largest key.  The
// row holds at least k keys at or above that bin (chunk c's own top k), so
// the row's k-th largest key T lies in a bin >= b_c, for every chunk c with
// at least k keys.  Each workgroup therefore lists its keys from the floor
// of b_c (its own top k plus that bin), histograms them over the 512 keys
// from the floor, and publishes the suffix counts: word j = its keys >=
// floor + j.  After one rendezvous every workgroup reads every header and
// the counts at bin boundaries, finds T's bin B (the largest bin whose keys
// at or above it number >= k), reads every chunk's 33 counts around B, and
// gets T, the count `need` still to take at T, and the keys above / equal to
// T in the chunks before its own: all it needs to write its part.
//
// The exchange holds when every chunk's list fits, every chunk's keys from
// its floor span at most 512 keys, some chunk has >= k keys, and no shorter
// chunk's floor lies above the full chunks' highest floor.  Otherwise (ties,
// NaN, spikes, short chunks) the caller runs the multi-pass select; every
// workgroup reads the same headers, so the choice is uniform over the row.
//
// LDS: hist[0, 512) the fine histogram; after the rendezvous hist[512, 576)
// the headers and hist[576, 1600) the counts at bin boundaries, then
// hist[0, 33 G) the counts around B.  The list lies past the histogram.
// ---------------------------------------------------------------------------
struct OneResult {
    bool ok;
    bool nan;           // some chunk of the row holds a NaN
    Bound b;
    uint32_t gt0, eq0;  // keys above / at T in the chunks before this one
    uint32_t run;       // this workgroup's list length
};

// Sum over the lanes of one wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
    return x;
}

template <class K, int LOADS>
__device__ OneResult one_exchange(const TopkArgs &a, int c, int G, int len,
                                  uint32_t (&kw)[LOADS * 4], bool blk_nan, const TopkLds &L,
                                  List ent, uint32_t cap, uint32_t *area, uint32_t *slot,
                                  uint32_t *err) {
    static_assert(K::PACK && K::SH1 == 5, "one exchange: 16-bit keys, 32 keys per first-digit bin");
    static_assert(kOneKeys == 2 * NT, "two fine bins per thread");
    static_assert(kOneHdr == kOneKeys / 32 && kOneFine > kOneHdr, "area: boundary counts, header, counts");
    constexpr int NBIN = kOneKeys / 32;  // first-digit bins a chunk's region may span
    const int t = tid();
    const int lane = t & 63;
    const uint32_t k = (uint32_t)a.k;
    OneResult r{};

    // ---- this chunk's floor bin b_c and its list of keys from the floor ----
    uint32_t bc = 0, full = 0, ok = 1, run = 0;
    if (len > 0) {
        const uint32_t need = len >= (int)k ? k : (uint32_t)len;
        bc = find_digit(L.hist, kBins, need, L.red, L.out).v;
        full = len >= (int)k ? 1u : 0u;
        run = compact_candidates<K, LOADS, true>(kw, len, bc << K::SH1, L.wtot, L.base, ent, cap);
        ok = run <= cap ? 1u : 0u;  // uniform
    }
    // ---- fine histogram of the list over the 512 keys from the floor -------
    uint32_t *fh = L.hist;  // the first-digit histogram is dead
    fh[t] = 0;
    fh[t + NT] = 0;
    __syncthreads();
    const uint32_t lo = bc << K::SH1;
    uint32_t over = 0;
    if (ok)
        for (uint32_t i = (uint32_t)t; i < run; i += NT) {
            const uint32_t off = list_key<K>(ent, i) - lo;
            if (off < (uint32_t)kOneKeys)
                atomicAdd(&fh[off], 1u);
            else
                over = 1;
        }
    if (__syncthreads_or((int)over)) ok = 0;
    // (Polling these words instead of a rendezvous counter was measured
    // slower: every workgroup's loads of the same few lines queue at one
    // memory channel.)
    // The header records nz, the number of counts from the floor that are
    // nonzero; only those are stored, and a reader takes every count at or
    // past nz as zero (the area is not cleared between calls).
    uint32_t *mine = area + (int64_t)c * kOneWords;
    uint32_t nz = 0;
    if (ok) {
        // suffix counts from the top: thread t owns keys top-1, top-2
        const int top = kOneKeys - 2 * t;
        const uint32_t h1 = fh[top - 1], h0 = fh[top - 2];
        const uint32_t incl = block_scan(h1 + h0, L.red).incl;
        if (incl - h0) st_agent(mine + kOneFine + (top - 1), incl - h0);
        if (incl) st_agent(mine + kOneFine + (top - 2), incl);
        // and the counts at bin boundaries (key 32 j) side by side
        if (incl && ((top - 2) & 31) == 0) st_agent(mine + ((top - 2) >> 5), incl);
        // words [0, nz) hold nonzero counts: nz = highest nonzero key + 1
        const uint32_t last = h1 ? (uint32_t)top : (h0 ? (uint32_t)top - 1u : 0u);
        const uint32_t wm = wave_max_u32(last);
        if (lane == 0) L.red[t >> 6] = wm;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) nz = max(nz, L.red[w]);
    }
    if (t == 0)
        st_agent(mine + kOneHdr,
                 bc | (full << 16) | (ok << 17) | (blk_nan ? 1u << 18 : 0u) | (nz << 20));
    row_rendezvous(slot, (uint32_t)G, err, a.spin_limit);

    // ---- every chunk's header and counts at its bin boundaries -------------
    uint32_t *s_hdr = L.hist + kOneKeys;       // [64]
    uint32_t *s_cs = L.hist + kOneKeys + 64;   // [64][NBIN]
    {
        constexpr int PER = NBIN + 1;
        constexpr int R1 = (kOneMaxSplit * PER + NT - 1) / NT;
        const int total = G * PER;
        uint32_t v[R1];
#pragma unroll
        for (int q = 0; q < R1; ++q) {
            const int i = q * NT + t;
            const int ii = i < total ? i : 0;
            const int cc = ii / PER, j = ii % PER;
            v[q] = ld_agent(area + (int64_t)cc * kOneWords + j);  // j == NBIN: the header
        }
#pragma unroll
        for (int q = 0; q < R1; ++q) {
            const int i = q * NT + t;
            if (i < total) {
                const int cc = i / PER, j = i % PER;
                if (j == NBIN)
                    s_hdr[cc] = v[q];
                else
                    s_cs[cc * NBIN + j] = v[q];
            }
        }
    }
    __syncthreads();
    // every wave finds B on its own (no barrier to share it): lane = chunk
    const uint32_t h = lane < G ? s_hdr[lane] : (1u << 17);
    const uint32_t hb = h & 0x7FFu, hfull = (h >> 16) & 1u, hok = (h >> 17) & 1u;
    r.nan = __ballot(((h >> 18) & 1u) != 0u) != 0ull;
    const uint32_t maxb = wave_max_u32(hfull ? hb : 0u);
    const bool any_full = __ballot(hfull != 0u) != 0ull;
    const bool fits = __ballot(!hok || (!hfull && hb > maxb)) == 0ull;
    if (!(any_full && fits)) {
        r.ok = false;
        __syncthreads();  // the caller reuses the histogram's space
        return r;
    }
    // keys at or above bin maxb + j, j < 16: lane = j + 16 * (chunk group)
    uint32_t part = 0;
    {
        // chunks lane>>4, +4, ...: four header reads, then four count reads,
        // in flight together
        constexpr int M = 4;
        const int j = lane & (NBIN - 1);
#pragma unroll 1
        for (int c0 = lane >> 4; c0 < G; c0 += 4 * M) {
            uint32_t hbv[M], cv[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int cc = c0 + 4 * m;
                hbv[m] = s_hdr[cc < G ? cc : 0];
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int cc = c0 + 4 * m;
                const uint32_t idx = maxb + (uint32_t)j - (hbv[m] & 0x7FFu);
                const uint32_t nzc = (hbv[m] >> 20) & 0x3FFu;
                cv[m] = s_cs[(cc < G ? cc : 0) * NBIN + (idx < (uint32_t)NBIN ? idx : 0u)];
                cv[m] = (cc < G && idx < (uint32_t)NBIN && 32u * idx < nzc) ? cv[m] : 0u;
            }
#pragma unroll
            for (int m = 0; m < M; ++m) part += cv[m];
        }
        part += (uint32_t)__shfl_xor((int)part, 16);
        part += (uint32_t)__shfl_xor((int)part, 32);
    }
    const uint64_t geb = __ballot(lane < NBIN && part >= k);
    const uint32_t B = maxb + (uint32_t)__popcll(geb) - 1u;
    // ---- every chunk's counts at the 33 keys from B's floor ----------------
    {
        constexpr int PER = 33;
        constexpr int R2 = (kOneMaxSplit * PER + NT - 1) / NT;
        const int total = G * PER;
        // word index of each of this thread's counts (past the 512 keys: 0)
        uint32_t idx[R2], nzv[R2];
#pragma unroll
        for (int q = 0; q < R2; ++q) {
            const int i = q * NT + t;
            const int ii = i < total ? i : 0;
            const uint32_t hh = s_hdr[ii / PER];
            idx[q] = 32u * (B - (hh & 0x7FFu)) + (uint32_t)(ii % PER);
            nzv[q] = min((hh >> 20) & 0x3FFu, (uint32_t)kOneKeys);  // (a header is never past it)
        }
        uint32_t v[R2];
#pragma unroll
        for (int q = 0; q < R2; ++q) {
            const int i = q * NT + t;
            const int ii = i < total ? i : 0;
            v[q] = ld_agent(area + (int64_t)(ii / PER) * kOneWords + kOneFine +
                            (idx[q] < nzv[q] ? idx[q] : 0u));
        }
        __syncthreads();  // every wave is done with the headers and boundary counts
#pragma unroll
        for (int q = 0; q < R2; ++q) {
            const int i = q * NT + t;
            if (i < total) L.hist[i] = idx[q] < nzv[q] ? v[q] : 0u;
        }
    }
    __syncthreads();
    // keys >= B's floor + j over the row (lanes 0..32), then T = floor + j*
    uint32_t gf = 0;
    if (lane <= 32) {
#pragma unroll 8
        for (int cc = 0; cc < G; ++cc) gf += L.hist[cc * 33 + lane];
    }
    // (js >= 0 whenever the rendezvous completed; the guard keeps every LDS
    // index in range after one that gave up)
    const uint32_t nge = (uint32_t)__popcll(__ballot(lane <= 32 && gf >= k));
    const uint32_t js = nge ? min(nge - 1u, 31u) : 0u;
    const uint32_t above = (uint32_t)__shfl((int)gf, (int)js + 1);
    // keys above / at T in the chunks before this one: lane = chunk
    const uint32_t s1 = lane < c ? L.hist[lane * 33 + js + 1] : 0u;
    const uint32_t s0 = lane < c ? L.hist[lane * 33 + js] : 0u;
    r.gt0 = wave_sum(s1);
    r.eq0 = wave_sum(s0 - s1);
    r.b = Bound{(B << K::SH1) | js, 0, k - above};
    r.run = run;
    r.ok = true;
    __syncthreads();  // the exchanged counts are read; the caller may reuse the space
    return r;
}

// The window exchange places a chunk's window from one load in kWxSample:
// only those loads' keys go into the 12-bit histogram (a quarter of the LDS
// atomics of a full one).  Every count the exchange relies on comes from the
// chunk's exact list of candidates.
constexpr int kWxSample = 4;

// Columns of a chunk of len columns that the sampled loads cover.
template <int LOADS>
__device__ __forceinline__ uint32_t wx_sample_len(int len) {
    constexpr int SPAN = NT * 4;
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < LOADS; j += kWxSample) {
        const int r = len - j * SPAN;
        s += r <= 0 ? 0u : (r >= SPAN ? (uint32_t)SPAN : (uint32_t)r);
    }
    return s;
}

// ---------------------------------------------------------------------------
// Window exchange of a split fp32 row (G <= kOneMaxSplit workgroups, one
// rendezvous).
//
// Chunk c estimates the row's boundary bin (12-bit first digit) from its
// own keys: the bin b_c of its q_c-th largest key, q_c = ceil(k len_c / n),
// the row's selected share of its own keys.  It lists its keys from bin
// b_c - 1 up (column order, LDS), publishes the keys of the window
// [b_c - 1, b_c + 1], each bin at a fixed place of its area, their counts,
// and its count above the window.  After one rendezvous every workgroup reads the G headers.  For a
// bin B inside every non-empty chunk's window the row's count of keys at or
// above B is known exactly (above-window counts plus window counts from B
// up), so the boundary bin B1 (the highest bin whose count reaches k) is
// found when it lies in all windows.  The keys of bin B1 of every chunk are
// gathered into LDS; the (k - count above B1)-th largest of them is the
// row's k-th largest key T (two local radix passes over the low 20 bits).
// The chunks' counts above and at T follow, and each workgroup writes its
// part of the output from its list as in the bf16 exchange.
//
// The exchange holds when no chunk holds a NaN, every chunk's list and
// window bins fit, the windows of the non-empty chunks meet and hold the
// boundary, and the row's keys in B1 fit the gather buffer.  Otherwise (NaN
// rows, skewed or short chunks, heavy ties) the row runs the multi-pass
// select; every workgroup reads the same headers, so the choice is uniform
// over the row.  Until the list is made the chunk's values stay raw floats:
// the list takes every value at or above the float whose key is wlo << 20
// (float compares order the values as their keys do, with -0 == +0, and
// only NaN compares unordered, which is why a NaN chunk places no window),
// and its entries become keys in the pass that counts the window.
//
// Area of a workgroup: word 0 = lo | hi << 12 | ok << 24 | empty << 25 |
// nan << 26 (the window bins [lo, hi]), word 1 = keys above the window,
// words 2..4 = keys in bins lo, lo+1, lo+2, then the window keys from word
// kWxHdr, bin lo + w at kWxHdr + w kWxBinCap (at most kWxBinCap keys a bin,
// in no particular order).
// LDS after the rendezvous (the histogram's space): gathered keys [0, 2048),
// the local radix histogram [2048, 3072), per-chunk words [3072, 3202) (two
// arrays of G + 1 <= 65: segment starts, offsets).
// The local histograms count each key twice in one word: once in the low
// half, and once in the high half when it comes from a chunk before this
// workgroup's, so the digit searches also give this workgroup's counts of
// earlier keys above and at T.
// ---------------------------------------------------------------------------
// fp32 key of one value: 0x80000000 + magnitude (positive), 0x80000000 -
// magnitude (negative), so -0 and +0 meet: (x ^ (s | 0x80000000)) - s with
// s the sign spread over the word.  A NaN lands above +inf's key
// (0xFF800000) or below -inf's (0x00800000) and is moved to the top apart.
__device__ __forceinline__ uint32_t f32_key(uint32_t x) {
    const uint32_t s = (uint32_t)((int32_t)x >> 31);
    return (x ^ (s | 0x80000000u)) - s;
}

// The bits of the smallest float whose key is at least T (T a multiple of
// 2^20, at most +inf's key): keys from 0x80000000 up are +0 .. +inf, keys
// below are the negative floats by falling magnitude, and keys at or below
// -inf's hold only NaNs, so -inf stands for them.
__device__ __forceinline__ uint32_t f32_floor_bits(uint32_t T) {
    if (T >= 0x80000000u) return T - 0x80000000u;
    const uint32_t m = 0x80000000u - T;
    return m >= 0x7F800000u ? 0xFF800000u : (0x80000000u | m);
}

struct WxResult {
    bool ok, nan;
    uint32_t T, need, gt0, eq0, run;
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }

template <class K, int LOADS>
__device__ __forceinline__ WxResult window_exchange(const TopkArgs &a, int c, int G, int len, int64_t n,
                                    uint32_t (&kw)[LOADS * 4], bool blk_nan, const TopkLds &L,
                                    List ent, uint32_t cap, uint32_t *area, uint32_t *slot,
                                    uint32_t *err) {
    static_assert(!K::PACK, "window exchange: 32-bit keys");
    constexpr int SH = 20;                 // 12-bit first digit
    constexpr uint32_t GAT = 0, SEL = 2048, CHK = 3072;
    const int t = tid();
    const int lane = t & 63;
    const uint32_t k = (uint32_t)a.k;
    WxResult r{};

    // ---- this chunk: window, counts, list -----------------------------------
    uint32_t wlo = 0, whi = 0, above = 0, cw0 = 0, cw1 = 0, cw2 = 0, ok = 1, run = 0;
    const bool empty = len <= 0;
    if (!empty && blk_nan) {
        ok = 0;  // a NaN in the chunk: the row takes the multi-pass select
    } else if (!empty) {
        // q: the chunk's share of k; qs: the same share of the sample
        uint64_t q = ((uint64_t)k * (uint64_t)len + (uint64_t)n - 1) / (uint64_t)n;
        q = q < 1 ? 1 : (q > (uint64_t)len ? (uint64_t)len : q);
        const uint32_t slen = wx_sample_len<LOADS>(len);
        uint64_t qs = (q * slen + (uint64_t)len - 1) / (uint64_t)len;
        qs = qs < 1 ? 1 : (qs > slen ? slen : qs);
        const Digit d = find_digit_4096(L.hist, (uint32_t)qs, ent.w + 2 * (cap + 64), L.red, L.out);
        DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 8);
        wlo = d.v > 0 ? d.v - 1 : 0;
        whi = d.v < (uint32_t)kWxBins - 1 ? d.v + 1 : d.v;
        // the list: every value whose key is T1 = max(wlo << SH, 1) or more
        // (kw and the list hold raw float bits until the pass below)
        run = compact_candidates<K, LOADS, true, true>(kw, len, f32_floor_bits(max(wlo << SH, 1u)),
                                                       L.wtot, L.base, ent, cap);
        DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 9);
        if (run > cap) {
            ok = 0;  // uniform
        } else {
            // one pass over the list (it holds every key of bin wlo and up:
            // the rest lie above the window): each entry becomes its key,
            // and a window key takes the next slot of its bin (an LDS
            // counter; the order within a bin does not matter) and is
            // published there at once, bin w of the area at w kWxBinCap
            const uint32_t nwin = whi - wlo + 1u;
            const uint32_t E = (run + NT - 1) / NT;
            const uint32_t i0 = min(run, (uint32_t)t * E), i1 = min(run, i0 + E);
            uint32_t *dst = area + (int64_t)c * kWxWords + kWxHdr;
            for (uint32_t i = i0; i < i1; ++i) {
                const uint32_t key = f32_key(ent.w[2 * i]);  // the entries' keys from here on
                ent.w[2 * i] = key;
                const uint32_t w = (key >> SH) - wlo;
                if (w < nwin) {
                    const uint32_t slot = atomicAdd(&L.out[4 + w], 1u);
                    if (slot < (uint32_t)kWxBinCap) st_agent(dst + w * (uint32_t)kWxBinCap + slot, key);
                }
            }
            __syncthreads();
            cw0 = L.out[4];
            cw1 = L.out[5];
            cw2 = L.out[6];
            above = run - cw0 - cw1 - cw2;
            ok = (cw0 <= (uint32_t)kWxBinCap && cw1 <= (uint32_t)kWxBinCap && cw2 <= (uint32_t)kWxBinCap)
                     ? 1u : 0u;
            DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 14);
        }
    }
    uint32_t *mine = area + (int64_t)c * kWxWords;
    if (t == 0) {
        st_agent(mine + 0, wlo | (whi << 12) | (ok << 24) | (empty ? 1u << 25 : 0u) |
                               (blk_nan ? 1u << 26 : 0u));
        st_agent(mine + 1, above);
        st_agent(mine + 2, cw0);
        st_agent(mine + 3, cw1);
        st_agent(mine + 4, cw2);
    }
    DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 2);
    row_rendezvous(slot, (uint32_t)G, err, a.spin_limit);
    DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 6);

    // ---- every chunk's header: each wave reads them all (lane = chunk) and
    // decides on its own, so no barrier shares them
    const bool in = lane < G;
    uint32_t h0 = 1u << 25, cab = 0, cc0 = 0, cc1 = 0, cc2 = 0;
    if (in) {
        const uint32_t *hl = area + (int64_t)lane * kWxWords;
        h0 = ld_agent(hl);
        cab = ld_agent(hl + 1);
        cc0 = ld_agent(hl + 2);
        cc1 = ld_agent(hl + 3);
        cc2 = ld_agent(hl + 4);
    }
    const uint32_t clo = h0 & 0xFFFu, chi = (h0 >> 12) & 0xFFFu;
    const bool cok = (h0 >> 24) & 1u, cempty = (h0 >> 25) & 1u;
    const bool live = in && !cempty;
    r.nan = __ballot(in && ((h0 >> 26) & 1u)) != 0ull;
    // a header this call wrote always passes these checks; they keep every
    // read below inside its area should a rendezvous have given up
    const bool sane = clo <= chi && chi - clo <= 2u && cc0 <= (uint32_t)kWxBinCap &&
                      cc1 <= (uint32_t)kWxBinCap && cc2 <= (uint32_t)kWxBinCap;
    const bool all_ok = __ballot(live && !(cok && sane)) == 0ull;
    const bool any_live = __ballot(live) != 0ull;
    const uint32_t maxlo = wave_max_u32(live ? clo : 0u);
    const uint32_t minhi = wave_min_u32(live ? chi : 0xFFFFFFFFu);
    // this chunk's keys at or above bin B (B within its window, or one past it)
    auto at_or_above = [&](uint32_t B) -> uint32_t {
        if (!live) return 0u;
        uint32_t v = cab;
        v += clo >= B ? cc0 : 0u;
        v += clo + 1 <= chi && clo + 1 >= B ? cc1 : 0u;
        v += clo + 2 <= chi && clo + 2 >= B ? cc2 : 0u;
        return v;
    };
    bool good = all_ok && any_live && maxlo <= minhi;
    uint32_t B1 = 0;
    if (good) {
        good = wave_sum(at_or_above(minhi + 1)) < k && wave_sum(at_or_above(maxlo)) >= k;
        if (good) {
            B1 = maxlo;
            for (uint32_t B = minhi; B > maxlo; --B)
                if (wave_sum(at_or_above(B)) >= k) {
                    B1 = B;
                    break;
                }
        }
    }
    uint32_t M = 0;
    if (good) {
        const uint32_t w1 = B1 - clo;  // bin B1 in this lane's window (live lanes)
        const uint32_t mc = !live ? 0u : (w1 == 0 ? cc0 : (w1 == 1 ? cc1 : cc2));
        const uint32_t boff = w1 * (uint32_t)kWxBinCap;
        const uint32_t incl = wave_incl_scan(mc);
        M = rdlane(incl, 63);
        good = M <= (uint32_t)kWxGather;
        if (good && t < 64) {  // wave 0 keeps the per-chunk words
            uint32_t *chk = L.hist + CHK;
            if (in) {
                chk[lane] = incl - mc;      // segment start of this chunk's keys in B1
                chk[65 + lane] = boff;      // their offset in its area
            }
            if (lane == 0) chk[G] = M;
        }
    }
    if (!good) {
        r.ok = false;
        __syncthreads();  // the caller reuses the histogram's space
        return r;
    }
    const uint32_t R1 = wave_sum(at_or_above(B1 + 1));
    const uint32_t need1 = k - R1;  // keys to take from bin B1, 1..M
    const uint32_t ab0 = wave_sum(lane < c ? at_or_above(B1 + 1) : 0u);  // earlier chunks, above B1
    uint32_t *sel = L.hist + SEL;
    for (int i = t; i < 1024; i += NT) sel[i] = 0;
    __syncthreads();

    DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 10);
    // ---- gather bin B1's keys of every chunk (NT / G threads per chunk), and
    // histogram their first local digit (key >> 10) & 1023 as they arrive
    {
        const uint32_t *chk = L.hist + CHK;
        const int tpc = NT / G;
        const int cc = t / tpc, r0 = t % tpc;
        if (cc < G) {
            const uint32_t seg = chk[cc], m = chk[cc + 1] - seg;
            const uint32_t *src = area + (int64_t)cc * kWxWords + kWxHdr + chk[65 + cc];
#pragma unroll 1
            for (uint32_t i = (uint32_t)r0; i < m; i += 4u * (uint32_t)tpc) {
                uint32_t v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t ii = i + (uint32_t)(u * tpc);
                    v[u] = ld_agent(src + (ii < m ? ii : 0u));
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t ii = i + (uint32_t)(u * tpc);
                    if (ii < m) {
                        L.hist[GAT + seg + ii] = v[u];
                        atomicAdd(&sel[(v[u] >> 10) & 1023u], cc < c ? 0x10001u : 1u);
                    }
                }
            }
        }
    }
    __syncthreads();
    DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 11);
    // ---- the (need1)-th largest of them: digits (key >> 10) & 1023, then
    // key & 1023, over the workgroup; a key of an earlier chunk (gathered
    // before this chunk's segment) also counts in the high half of its bin
    const uint32_t segc = L.hist[CHK + c];
    const Digit dA = find_digit_fast(sel, 1024, need1, L.red, L.out);
    const uint32_t needA = need1 - (dA.above & 0xFFFFu);
    uint32_t T, needT, gtE, eqE;  // earlier chunks' keys of B1 above T, at T
    if ((dA.cnt & 0xFFFFu) == needA) {
        T = ((B1 << SH) | (dA.v << 10)) - 1u;  // the digit's bin is taken whole
        needT = 0;
        gtE = (dA.above >> 16) + (dA.cnt >> 16);
        eqE = 0;  // (no key at T is taken)
    } else {
        for (int i = t; i < 1024; i += NT) sel[i] = 0;
        __syncthreads();
        for (uint32_t i = (uint32_t)t; i < M; i += NT) {
            const uint32_t key = L.hist[GAT + i];
            if (((key >> 10) & 1023u) == dA.v) atomicAdd(&sel[key & 1023u], i < segc ? 0x10001u : 1u);
        }
        __syncthreads();
        const Digit dB = find_digit_fast(sel, 1024, needA, L.red, L.out);
        T = (B1 << SH) | (dA.v << 10) | dB.v;
        needT = needA - (dB.above & 0xFFFFu);
        gtE = (dA.above >> 16) + (dB.above >> 16);
        eqE = dB.cnt >> 16;
    }
    DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 12);
    r.gt0 = ab0 + gtE;
    r.eq0 = eqE;
    r.T = T;
    r.need = needT;
    r.run = run;
    r.ok = true;
    __syncthreads();  // the gathered keys are read; the caller may reuse the space
    return r;
}

// The multi-pass select of a split row, from each workgroup's first-digit
// histogram in LDS (hist): the histograms meet in the row's workspace slot,
// one rendezvous per radix pass (nren rendezvous of this launch are already
// behind the row), each workgroup writes its own part.  STREAM: the
// workgroup does not hold its keys (the fallback of the fp32 window
// exchange, whose registers are reused), so its passes and its write re-read
// its range from cache.
template <class K, int LOADS, bool STREAM>
__device__ __forceinline__ void split_multipass(const TopkArgs &a, int64_t row, int64_t n, int c,
                                                int G, int len, int64_t lo,
                                                uint32_t (&kw)[LOADS * 4], const TopkLds &L,
                                                List ent, uint32_t cap,
                                                __amdgpu_buffer_rsrc_t view, uint32_t *slot,
                                                uint32_t *err, uint32_t nren,
                                                const typename K::raw_t *xr) {
    const int t = tid();
    uint32_t *ghist = slot + kSlotHeadWords;
    uint32_t *gcnt = ghist + kMaxPasses * kBins;
    constexpr int LASTB = 1 << K::digit_last();  // bins of the last pass
    uint32_t *pub = gcnt + 4 * G;                // G x (LASTB + 1) suffix counts
    // ---- merge the histograms of the row's workgroups ----------------------
    merge_histogram(L.hist, ghist, kBins);
    row_rendezvous(slot, (++nren) * (uint32_t)G, err, a.spin_limit);
    fetch_histogram(ghist, L.hist, kBins);
    __syncthreads();
    const Digit d1 = find_digit(L.hist, kBins, (uint32_t)a.k, L.red, L.out);

    // ---- the rest of the radix select, one rendezvous per pass.  Each
    // workgroup histograms its own keys at the boundary: straight from VGPRs
    // when it holds a few keys per thread and candidates are dense, else from
    // an LDS list of its candidates (key >= T1), else (its candidates do not
    // fit the list: massive ties, or a row whose largest values crowd into
    // one chunk) from its range re-read from cache.  All three take part in
    // the same rendezvous.  In the last pass each workgroup also publishes its
    // suffix counts, so the counts of the chunks before it come with that
    // pass's rendezvous.
    Bound b{d1.v, K::SH1, (uint32_t)a.k - d1.above};
    // dense: at least a quarter of the row are candidates (uniform over it)
    const bool regs = !STREAM && LOADS <= 2 && 4 * (int64_t)(d1.above + d1.cnt) >= n;
    uint32_t run = 0;
    bool listed = false;
    if constexpr (!STREAM) {
        if (!regs) {
            run = compact_candidates<K, LOADS, true>(kw, len, d1.v << K::SH1, L.wtot, L.base, ent,
                                                     cap);
            listed = run <= cap;  // uniform over the workgroup
        }
    }
    // this workgroup's (equal << 16 | above) counts at a bound
    auto local_counts = [&](Bound bb) -> uint32_t {
        if constexpr (!STREAM) {
            if (regs) return block_scan(counts_regs<K, LOADS>(kw, bb), L.red).total;
        }
        if (listed) return list_counts<K>(ent, run, bb, L.red);
        return block_scan(range_counts<K>(view, lo, len, bb), L.red).total;
    };
    bool folded = false;  // the last pass published this workgroup's counts
    auto local_histogram = [&](uint32_t P, int s, int sh, uint32_t dmask) {
        if constexpr (!STREAM) {
            if (regs) {
                refine_histogram_regs<K, LOADS>(kw, P, s, sh, dmask, L.hist);
                return;
            }
        }
        if (listed)
            list_refine_histogram<K>(ent, run, P, s, sh, dmask, L.hist);
        else
            refine_histogram_stream<K>(view, lo, len, P, s, sh, dmask, L.hist);
    };
    if (d1.cnt != b.need) {
#pragma unroll 1
        for (int pass = 1; pass < K::NPASS; ++pass) {
            const int d = K::digit(pass);
            const int sh = b.s - d;
            const int nb = 1 << d;
            for (int i = t; i < nb; i += NT) L.hist[i] = 0;
            __syncthreads();
            local_histogram(b.P, b.s, sh, (1u << d) - 1u);
            __syncthreads();
            if (pass == K::NPASS - 1) {
                publish_suffix(L.hist, nb, local_counts(b) & 0xFFFFu,
                               pub + (int64_t)c * (LASTB + 1), L.red);
                folded = true;
            }
            uint32_t *g = ghist + pass * kBins;
            merge_histogram(L.hist, g, nb);
            row_rendezvous(slot, (++nren) * (uint32_t)G, err, a.spin_limit);
            fetch_histogram(g, L.hist, nb);
            __syncthreads();
            const Digit dg = find_digit(L.hist, nb, b.need, L.red, L.out);
            b.need -= dg.above;
            b.P = (b.P << d) | dg.v;
            b.s = sh;
            if (dg.cnt == b.need) break;  // the boundary bin is taken whole
        }
    }
    // ---- the taken-above and equal counts of the chunks before this one:
    // from the last pass's suffix counts, or (the selection ended at an
    // earlier digit) one more exchange.  Each workgroup then writes its own
    // part of the row's output.
    uint32_t gg = 0, qq = 0;
    if (folded) {
        const uint32_t v = b.P & (uint32_t)(LASTB - 1);
        for (int i = t; i < c; i += NT) {
            const uint32_t *w = pub + (int64_t)i * (LASTB + 1) + v;
            const uint32_t at = ld_agent(w), above = ld_agent(w + 1);
            gg += above;
            qq += at - above;
        }
    } else {
        const uint32_t mine = local_counts(b);
        if (t == 0) {
            st_agent(gcnt + 2 * c + 0, mine & 0xFFFFu);
            st_agent(gcnt + 2 * c + 1, mine >> 16);
        }
        row_rendezvous(slot, (++nren) * (uint32_t)G, err, a.spin_limit);
        for (int i = t; i < c; i += NT) {
            gg += ld_agent(gcnt + 2 * i + 0);
            qq += ld_agent(gcnt + 2 * i + 1);
        }
    }
    const uint32_t gt0 = block_scan(gg, L.red).total;
    const uint32_t eq0 = block_scan(qq, L.red).total;
    if constexpr (!STREAM) {
        if (regs) write_from_regs<K, LOADS>(a, row, kw, len, b, gt0, eq0, view, lo, L.red, xr);
    }
    if (regs)
        ;
    else if (listed)
        write_from_list<K>(a, row, ent, run, b, L.red, xr, gt0, eq0, (uint32_t)lo);
    else
        write_from_stream<K>(a, row, view, lo, len, b, gt0, eq0, L.red, xr);
    // every workgroup's NaN bit was in before the first rendezvous
    if (c == 0 && t == 0 && a.nan_flag) a.nan_flag[row] = ld_agent(slot + 2) ? 1u : 0u;

    // Leave the slot zeroed for the next call (whose slot layout may differ).
    // The histograms of all passes but the last were read before the last
    // rendezvous, so each workgroup clears a share of them now; the last
    // workgroup out, once every workgroup has read what it needs, clears the
    // last pass's histogram, the counts and the counters.  The stores
    // complete before the launch does.
    constexpr int HW = (K::NPASS - 1) * kBins;
    const int per = (HW + G - 1) / G;
    const int z0 = c * per, z1 = min(HW, z0 + per);
    for (int i = z0 + t; i < z1; i += NT) st_agent(ghist + i, 0u);
    __syncthreads();
    if (t == 0) L.out[3] = (add_agent(slot + 1, 1u) == (uint32_t)G - 1u) ? 1u : 0u;
    __syncthreads();
    if (L.out[3]) {
        for (int i = t; i < LASTB; i += NT) st_agent(ghist + HW + i, 0u);
        if (folded)
            for (int i = t; i < G * (LASTB + 1); i += NT) st_agent(pub + i, 0u);
        else
            for (int i = t; i < 2 * G; i += NT) st_agent(gcnt + i, 0u);
        if (t == 0) {
            st_agent(slot + 0, 0u);
            st_agent(slot + 1, 0u);
            st_agent(slot + 2, 0u);
        }
    }
}

// ---------------------------------------------------------------------------
// Split rows: G workgroups per row, workgroup c owning columns
// [c*chunk, (c+1)*chunk) of the valid prefix, held in VGPRs.
// ---------------------------------------------------------------------------
template <class K, int EPT>
__global__ __launch_bounds__(NT) void topk_rows_split(const TopkArgs a) {
    using raw_t = typename K::raw_t;
    constexpr int VEC = K::VEC;
    constexpr int LOADS = EPT / VEC;
    static_assert(EPT % VEC == 0, "EPT must be a multiple of the vector width");

    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];  // histogram, candidate list
    __shared__ TopkShared<LOADS> S;
    const TopkLds L{s_dyn, S.wtot, S.base, S.red, S.out};

    const int t = tid();
    const int G = a.G;
    const int c = (int)(blockIdx.x % (unsigned)G);
    const int64_t lrow = (int64_t)(blockIdx.x / (unsigned)G);
    const int64_t row = a.row0 + lrow;
    if (row >= a.rows) return;  // uniform over the row's workgroups

    const int64_t n = valid_length(a, row);
    const raw_t *xr = reinterpret_cast<const raw_t *>(a.x) + row * a.x_stride;
    if (n <= a.k) {
        write_short_row<K>(a, row, n, c, G, xr);
        return;
    }

    const uint32_t cap = (uint32_t)a.cap;
    const List ent = list_of<K>(s_dyn + split_list_base());
    uint32_t *slot = a.ws + a.slot0 + lrow * a.slot_words;
    uint32_t *err = a.ws;
    uint32_t *ghist = slot + kSlotHeadWords;
    uint32_t *gcnt = ghist + kMaxPasses * kBins;
    constexpr int LASTB = 1 << K::digit_last();  // bins of the last pass
    uint32_t *pub = gcnt + 4 * G;                // G x (LASTB + 1) suffix counts
    // the row's G exchange areas (bf16), in the region after the header
    uint32_t *one_area = a.ws + kHeaderWords + lrow * G * kOneWords;

    // ---- this workgroup's columns into VGPRs; first-digit histogram --------
    const int64_t lo = (int64_t)c * a.chunk;
    const int64_t hi = min(lo + a.chunk, n);
    const int len = hi > lo ? (int)(hi - lo) : 0;
    uint32_t kw[LOADS * 4];
    uint32_t nan;
    {
        const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, len ? hi : 0);
        uint4 v[LOADS];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) v[j] = load_vec<K>(view, lo + (int64_t)(j * NT + t) * VEC);
        for (int b = t; b < kBins + 64; b += NT) L.hist[b] = 0;
        nan = keys_of_loads<K, LOADS>(v, len, kw);
    }
    const bool blk_nan = __syncthreads_or((int)nan) != 0;
    constexpr bool ONE = K::PACK && EPT <= kOneMaxEpt;
    // the row's NaN bit, drained by the multi-pass select's first rendezvous
    // (in the one exchange each workgroup's bit travels in its header; if it
    // falls back to the multi-pass select, the bit is set then)
    if ((!ONE || !a.one) && blk_nan && t == 0)
        __hip_atomic_fetch_or(slot + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    first_digit_histogram<K, LOADS>(kw, len, L.hist);
    __syncthreads();
    const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, len ? hi : 0);

    // ---- one exchange (bf16): the whole boundary from one rendezvous -------
    uint32_t nren = 0;
    if constexpr (ONE) {
        if (a.one) {
            const OneResult r = one_exchange<K, LOADS>(a, c, G, len, kw, blk_nan, L, ent, cap,
                                                       one_area, slot, err);
            nren = 1;
            if (r.ok) {
                // every read of the row's shared words is done: depart now, so
                // the returning atomic overlaps the write.  (The address is
                // hidden from uniformity analysis: a uniform atomic is
                // aggregated over the wave and its result waited for at once,
                // which would put a round trip before the write.)
                uint32_t dep = 0;
                if (t == 0) dep = add_agent(slot + 1 + opaque(0u), 1u);
                // the histogram's space (free again) stages the output run
                write_exact<K>(a, row, ent, r.run, r.b.P, r.b.need, r.gt0, r.eq0, (uint32_t)lo,
                               L.red, L.hist, xr);
                if (t == 0) {
                    if (c == 0 && a.nan_flag) a.nan_flag[row] = r.nan ? 1u : 0u;
                    L.out[3] = dep == (uint32_t)G - 1u ? 1u : 0u;
                }
                __syncthreads();
                // last out: every workgroup is past the rendezvous, so the
                // counters go back to zero (the exchanged words need no
                // clearing: a reader trusts only words its header vouches for)
                if (L.out[3] && t == 0) {
                    st_agent(slot + 0, 0u);
                    st_agent(slot + 1, 0u);
                }
                return;
            }
            // the exchange does not hold for this row: set the NaN bit, rebuild
            // the first-digit histogram (its space was reused) and run the
            // radix passes
            if (blk_nan && t == 0)
                __hip_atomic_fetch_or(slot + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int b = t; b < kBins + 64; b += NT) L.hist[b] = 0;
            __syncthreads();
            first_digit_histogram<K, LOADS>(kw, len, L.hist);
            __syncthreads();
        }
    }

    // ---- merge the histograms of the row's workgroups ----------------------
    merge_histogram(L.hist, ghist, kBins);
    row_rendezvous(slot, (++nren) * (uint32_t)G, err, a.spin_limit);
    fetch_histogram(ghist, L.hist, kBins);
    __syncthreads();
    const Digit d1 = find_digit(L.hist, kBins, (uint32_t)a.k, L.red, L.out);

    // ---- the rest of the radix select, one rendezvous per pass.  Each
    // workgroup histograms its own keys at the boundary: straight from VGPRs
    // when it holds a few keys per thread and candidates are dense, else from
    // an LDS list of its candidates (key >= T1), else (its candidates do not
    // fit the list: massive ties, or a row whose largest values crowd into
    // one chunk) from its range re-read from cache.  All three take part in
    // the same rendezvous.  In the last pass each workgroup also publishes its
    // suffix counts, so the counts of the chunks before it come with that
    // pass's rendezvous.
    Bound b{d1.v, K::SH1, (uint32_t)a.k - d1.above};
    // dense: at least a quarter of the row are candidates (uniform over it)
    const bool regs = LOADS <= 2 && 4 * (int64_t)(d1.above + d1.cnt) >= n;
    uint32_t run = 0;
    bool listed = false;
    if (!regs) {
        run = compact_candidates<K, LOADS, true>(kw, len, d1.v << K::SH1, L.wtot, L.base, ent,
                                                 cap);
        listed = run <= cap;  // uniform over the workgroup
    }
    // this workgroup's (equal << 16 | above) counts at a bound
    auto local_counts = [&](Bound bb) -> uint32_t {
        if (regs) return block_scan(counts_regs<K, LOADS>(kw, bb), L.red).total;
        if (listed) return list_counts<K>(ent, run, bb, L.red);
        return block_scan(range_counts<K>(view, lo, len, bb), L.red).total;
    };
    bool folded = false;  // the last pass published this workgroup's counts
    auto local_histogram = [&](uint32_t P, int s, int sh, uint32_t dmask) {
        if (regs)
            refine_histogram_regs<K, LOADS>(kw, P, s, sh, dmask, L.hist);
        else if (listed)
            list_refine_histogram<K>(ent, run, P, s, sh, dmask, L.hist);
        else
            refine_histogram_stream<K>(view, lo, len, P, s, sh, dmask, L.hist);
    };
    if (d1.cnt != b.need) {
#pragma unroll 1
        for (int pass = 1; pass < K::NPASS; ++pass) {
            const int d = K::digit(pass);
            const int sh = b.s - d;
            const int nb = 1 << d;
            for (int i = t; i < nb; i += NT) L.hist[i] = 0;
            __syncthreads();
            local_histogram(b.P, b.s, sh, (1u << d) - 1u);
            __syncthreads();
            if (pass == K::NPASS - 1) {
                publish_suffix(L.hist, nb, local_counts(b) & 0xFFFFu,
                               pub + (int64_t)c * (LASTB + 1), L.red);
                folded = true;
            }
            uint32_t *g = ghist + pass * kBins;
            merge_histogram(L.hist, g, nb);
            row_rendezvous(slot, (++nren) * (uint32_t)G, err, a.spin_limit);
            fetch_histogram(g, L.hist, nb);
            __syncthreads();
            const Digit dg = find_digit(L.hist, nb, b.need, L.red, L.out);
            b.need -= dg.above;
            b.P = (b.P << d) | dg.v;
            b.s = sh;
            if (dg.cnt == b.need) break;  // the boundary bin is taken whole
        }
    }
    // ---- the taken-above and equal counts of the chunks before this one:
    // from the last pass's suffix counts, or (the selection ended at an
    // earlier digit) one more exchange.  Each workgroup then writes its own
    // part of the row's output.
    uint32_t gg = 0, qq = 0;
    if (folded) {
        const uint32_t v = b.P & (uint32_t)(LASTB - 1);
        for (int i = t; i < c; i += NT) {
            const uint32_t *w = pub + (int64_t)i * (LASTB + 1) + v;
            const uint32_t at = ld_agent(w), above = ld_agent(w + 1);
            gg += above;
            qq += at - above;
        }
    } else {
        const uint32_t mine = local_counts(b);
        if (t == 0) {
            st_agent(gcnt + 2 * c + 0, mine & 0xFFFFu);
            st_agent(gcnt + 2 * c + 1, mine >> 16);
        }
        row_rendezvous(slot, (++nren) * (uint32_t)G, err, a.spin_limit);
        for (int i = t; i < c; i += NT) {
            gg += ld_agent(gcnt + 2 * i + 0);
            qq += ld_agent(gcnt + 2 * i + 1);
        }
    }
    const uint32_t gt0 = block_scan(gg, L.red).total;
    const uint32_t eq0 = block_scan(qq, L.red).total;
    if (regs)
        write_from_regs<K, LOADS>(a, row, kw, len, b, gt0, eq0, view, lo, L.red, xr);
    else if (listed)
        write_from_list<K>(a, row, ent, run, b, L.red, xr, gt0, eq0, (uint32_t)lo);
    else
        write_from_stream<K>(a, row, view, lo, len, b, gt0, eq0, L.red, xr);
    // every workgroup's NaN bit was in before the first rendezvous
    if (c == 0 && t == 0 && a.nan_flag) a.nan_flag[row] = ld_agent(slot + 2) ? 1u : 0u;

    // Leave the slot zeroed for the next call (whose slot layout may differ).
    // The histograms of all passes but the last were read before the last
    // rendezvous, so each workgroup clears a share of them now; the last
    // workgroup out, once every workgroup has read what it needs, clears the
    // last pass's histogram, the counts and the counters.  The stores
    // complete before the launch does.
    constexpr int HW = (K::NPASS - 1) * kBins;
    const int per = (HW + G - 1) / G;
    const int z0 = c * per, z1 = min(HW, z0 + per);
    for (int i = z0 + t; i < z1; i += NT) st_agent(ghist + i, 0u);
    __syncthreads();
    if (t == 0) L.out[3] = (add_agent(slot + 1, 1u) == (uint32_t)G - 1u) ? 1u : 0u;
    __syncthreads();
    if (L.out[3]) {
        for (int i = t; i < LASTB; i += NT) st_agent(ghist + HW + i, 0u);
        if (folded)
            for (int i = t; i < G * (LASTB + 1); i += NT) st_agent(pub + i, 0u);
        else
            for (int i = t; i < 2 * G; i += NT) st_agent(gcnt + i, 0u);
        if (t == 0) {
            st_agent(slot + 0, 0u);
            st_agent(slot + 1, 0u);
            st_agent(slot + 2, 0u);
        }
    }
}


// The window exchange's first pass: each 16-byte load kept as four raw
// floats as soon as it arrives (columns at or past len get a NaN, which no
// float compare selects), one load in kWxSample histogrammed by key (12-bit
// first digit; invalid columns into this lane's spare bin), and each valid
// pair of values tested for a NaN.  Returns whether this thread saw a NaN.
constexpr uint32_t kF32Filler = 0x7FFFFFFFu;

template <int LOADS>
__device__ __forceinline__ bool f32_raw_hist12(const uint4 (&v)[LOADS], int len,
                                               uint32_t (&kw)[LOADS * 4], uint32_t *hist) {
    constexpr int VEC = 4, SPAN = NT * VEC;
    const int me = tid();
    const int full = len / SPAN, any = (len + SPAN - 1) / SPAN;
    const uint32_t spare = (uint32_t)kWxBins + (uint32_t)(me & 63);
    bool nan = false;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if (j >= any) {
#pragma unroll
            for (int q = 0; q < 4; ++q) kw[4 * j + q] = kF32Filler;
            continue;
        }
        const uint32_t x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        if (j < full) {
#pragma unroll
            for (int q = 0; q < 4; ++q) kw[4 * j + q] = x[q];
            nan |= __builtin_isunordered(__uint_as_float(x[0]), __uint_as_float(x[1]));
            nan |= __builtin_isunordered(__uint_as_float(x[2]), __uint_as_float(x[3]));
            if (j % kWxSample == 0) {
#pragma unroll
                for (int q = 0; q < 4; ++q) atomicAdd(&hist[f32_key(x[q]) >> 20], 1u);
            }
        } else {
            int valid = len - (j * NT + me) * VEC;
            valid = valid < 0 ? 0 : (valid > VEC ? VEC : valid);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                kw[4 * j + q] = q < valid ? x[q] : kF32Filler;
                nan |= q < valid && __builtin_isnan(__uint_as_float(x[q]));
                if (j % kWxSample == 0) atomicAdd(&hist[q < valid ? (f32_key(x[q]) >> 20) : spare], 1u);
            }
        }
    }
    return nan;
}

// ---------------------------------------------------------------------------
// Split fp32 rows through the window exchange: one rendezvous per row.  The
// rare rows it does not hold for take the multi-pass select on keys re-read
// from cache, so no key stays in VGPRs past the exchange's list.  Same grid,
// workspace layout and output contract as topk_rows_split; the candidate
// list lies past the 12-bit histogram.
// ---------------------------------------------------------------------------
template <int EPT>
__global__ __launch_bounds__(NT) void topk_rows_wx(const TopkArgs a) {
    using K = F32Key;
    using raw_t = typename K::raw_t;
    constexpr int VEC = K::VEC;
    constexpr int LOADS = EPT / VEC;
    static_assert(EPT % VEC == 0, "EPT must be a multiple of the vector width");

    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];  // histogram, candidate list
    __shared__ TopkShared<LOADS> S;
    const TopkLds L{s_dyn, S.wtot, S.base, S.red, S.out};

    const int t = tid();
    const int G = a.G;
    const int c = (int)(blockIdx.x % (unsigned)G);
    const int64_t lrow = (int64_t)(blockIdx.x / (unsigned)G);
    const int64_t row = a.row0 + lrow;
    if (row >= a.rows) return;  // uniform over the row's workgroups
    DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 0);

    const int64_t n = valid_length(a, row);
    const raw_t *xr = reinterpret_cast<const raw_t *>(a.x) + row * a.x_stride;
    if (n <= a.k) {
        write_short_row<K>(a, row, n, c, G, xr);
        return;
    }
    const uint32_t cap = (uint32_t)a.cap;
    const List ent = list_of<K>(s_dyn + (kWxBins + 64));
    uint32_t *slot = a.ws + a.slot0 + lrow * a.slot_words;
    uint32_t *err = a.ws;
    uint32_t *area = a.ws + kHeaderWords + lrow * G * kWxWords;

    const int64_t lo = (int64_t)c * a.chunk;
    const int64_t hi = min(lo + a.chunk, n);
    const int len = hi > lo ? (int)(hi - lo) : 0;
    uint32_t kw[LOADS * 4];  // raw float bits (kF32Filler past the chunk's end)
    uint32_t nan;
    {
        const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, len ? hi : 0);
        uint4 v[LOADS];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) v[j] = load_vec<K>(view, lo + (int64_t)(j * NT + t) * VEC);
        for (int b = t; b < kWxBins + 64; b += NT) L.hist[b] = 0;
        if (t < 3) L.out[4 + t] = 0;  // the window bins' publish counters
        __syncthreads();
        // the 12-bit histogram, filled load by load as the data arrives
        DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 13);
        nan = f32_raw_hist12<LOADS>(v, len, kw, L.hist) ? 1u : 0u;
    }
    // a chunk with a NaN does not place a window: its row takes the
    // multi-pass select
    const bool blk_nan = __syncthreads_or((int)nan) != 0;
    DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 1);
    const WxResult r = window_exchange<K, LOADS>(a, c, G, len, n, kw, blk_nan, L, ent, cap, area,
                                                 slot, err);
    if (r.ok) {
        DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 3);
        // every read of the row's shared words is done: depart now, so the
        // returning atomic overlaps the write
        uint32_t dep = 0;
        if (t == 0) dep = add_agent(slot + 1 + opaque(0u), 1u);
        write_exact<K>(a, row, ent, r.run, r.T, r.need, r.gt0, r.eq0, (uint32_t)lo, L.red, L.hist, xr);
        DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 4);
        if (t == 0) {
            if (c == 0 && a.nan_flag) a.nan_flag[row] = r.nan ? 1u : 0u;
            L.out[3] = dep == (uint32_t)G - 1u ? 1u : 0u;
        }
        __syncthreads();
        DSEL_STAMP((t == 0), (int64_t)blockIdx.x, 5);
        DSEL_STAMP_VALUE((t == 0), (int64_t)blockIdx.x, 7, 1);
        if (L.out[3] && t == 0) {  // last out: the counters back to zero
            st_agent(slot + 0, 0u);
            st_agent(slot + 1, 0u);
        }
        return;
    }
    // the exchange does not hold: the multi-pass select with the row's NaN
    // bit, from an 11-bit histogram of the keys re-read from cache
    if (blk_nan && t == 0)
        __hip_atomic_fetch_or(slot + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, len ? hi : 0);
    for (int b = t; b < kBins + 64; b += NT) L.hist[b] = 0;
    __syncthreads();
    first_digit_histogram_stream<K>(view, lo, len, L.hist);
    __syncthreads();
    split_multipass<K, LOADS, true>(a, row, n, c, G, len, lo, kw, L, ent, cap, view, slot, err, 1u,
                                    xr);
}

// ---------------------------------------------------------------------------
// The gather fused into the select (dsel_topk_gather).  MindSpore hyper-
// parallel PR #1094 (English description and the section on the fix): the
// candidate chain selects each query row's top positions and then gathers
// the compressed keys at them (key[batch_ids, positions], made one
// index_select over batch-offset positions by the fix).  Here the workers
// that selected a row copy its gathered rows right away:
//     out_g[row, j, :] = key_g[row / rows_per_batch, p_j, :]   for j < k,
// p_j the row's j-th selected position (a short row's padding slots carry
// -1).  A position outside [0, len) is clamped into it, or (pad_zero, the
// chain's masked fill) gives a zero row.  NTH threads (me = 0 .. NTH-1)
// share the row's 16-byte vectors, U loads in flight per thread; the output
// is written once and not re-read, so its stores are non-temporal.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Key g's rows of one selected row, by all NTH threads of the workgroup.
// First each slot's position becomes a byte offset in s_off (k words of
// LDS): clamped into the key, or, for a zero-filled slot, an offset past the
// end of a buffer view of the row's batch of the key (32-bit offsets: the
// host fuses only keys whose batch spans less than 2^31 bytes), which reads
// as zero.  Then each 16-byte vector costs an LDS read, a load and a store.
template <int NTH, class Pos>
__device__ __forceinline__ void gather_key_rows(const TopkArgs &a, const GatherKeyArgs &kg,
                                                int64_t row, int me, Pos pos, uint32_t *s_off) {
    // loads in flight per thread (measured: 16 for the 512-thread copy of
    // the one-wave rows' kernel, 8 for whole rows' 256 threads)
    constexpr int U = NTH > 256 ? 16 : 8;
    constexpr uint32_t kOutside = 0x80000000u;  // past every view
    const int64_t b = row / a.fg.rows_per_batch;
    const char *kb = kg.key + b * kg.batch_bytes;
    const int64_t span = (kg.len - 1) * kg.row_bytes + (int64_t)kg.vecs * 16;
    const __amdgpu_buffer_rsrc_t kv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kb), (short)0, (int)span, 0x00020000);
    const uint32_t k = (uint32_t)a.k;
    const int64_t len = kg.len;
    const bool zero = a.fg.pad_zero != 0;
    for (uint32_t j = (uint32_t)me; j < k; j += NTH) {
        const int64_t p = pos(j);
        const bool in = p >= 0 && p < len;
        const int64_t pc = in ? p : (p < 0 ? 0 : len - 1);
        s_off[j] = (zero && !in) ? kOutside : (uint32_t)(pc * kg.row_bytes);
    }
    __syncthreads();
    u32x4 *ob = reinterpret_cast<u32x4 *>(kg.out) + row * (int64_t)k * kg.vecs;
    const uint32_t total = k * (uint32_t)kg.vecs, vecs = (uint32_t)kg.vecs;
    const int l2 = kg.vecs_log2;
#pragma unroll 1
    for (uint32_t i0 = (uint32_t)me; i0 < total; i0 += (uint32_t)(NTH * U)) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = min(i0 + (uint32_t)(u * NTH), total - 1u);
            const uint32_t j = l2 >= 0 ? i >> l2 : i / vecs;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(kv, s_off[j] + (i - j * vecs) * 16u, 0u, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = i0 + (uint32_t)(u * NTH);
            if (i < total) __builtin_nontemporal_store(v[u], ob + i);
        }
    }
    __syncthreads();  // s_off is read: the next key may rewrite it
}

template <int NTH, class Pos>
__device__ __forceinline__ void gather_tail(const TopkArgs &a, int64_t row, int me, Pos pos,
                                            uint32_t *s_off) {
#pragma unroll 1
    for (int g = 0; g < a.fg.n; ++g) gather_key_rows<NTH>(a, a.fg.k[g], row, me, pos, s_off);  // uniform
}

// ---------------------------------------------------------------------------
// Whole rows: one workgroup per row.
// ---------------------------------------------------------------------------

// Issue the loads of one row's first NT*EPT columns (columns at or past n
// read as zero).
template <class K, int LOADS>
__device__ __forceinline__ void load_row(const typename K::raw_t *xr, int64_t n,
                                             uint4 (&v)[LOADS]) {
    const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, n);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) v[j] = load_vec<K>(view, (int64_t)(j * NT + tid()) * K::VEC);
}

// One row of valid length n > k whose raw 16-byte vectors are in buf
// (coalesced layout).  GATHER: the instance that also copies the row's keys.
template <class K, int LOADS, bool GATHER = false>
__device__ __forceinline__ void select_row(const TopkArgs &a, int64_t row, int64_t n,
                                           const uint4 (&buf)[LOADS],
                                           const TopkLds &L, List ent) {
    using raw_t = typename K::raw_t;
    const int t = tid();
    const uint32_t cap = (uint32_t)a.cap;
    const raw_t *xr = reinterpret_cast<const raw_t *>(a.x) + row * a.x_stride;
    const int len = (int)n;

    DSEL_STAMP((t == 0), row, 1);
    uint32_t kw[LOADS * 4];
    const uint32_t nan = keys_of_loads<K, LOADS, NT, GATHER>(buf, len, kw);
    for (int b = t; b < kBins + 64; b += NT) L.hist[b] = 0;
    const uint32_t block_nan = __syncthreads_or((int)nan) ? 1u : 0u;
    DSEL_STAMP((t == 0), row, 2);

    first_digit_histogram<K, LOADS>(kw, len, L.hist);
    __syncthreads();
    DSEL_STAMP((t == 0), row, 3);
    const Digit d1 = find_digit(L.hist, kBins, (uint32_t)a.k, L.red, L.out);
    const uint32_t C = d1.above + d1.cnt;
    DSEL_STAMP((t == 0), row, 4);

    if (LOADS <= 2 && 4 * (int64_t)C >= n) {
        // a few keys per thread and dense candidates: no list
        const Bound b = refine_passes<K>(d1, (uint32_t)a.k, L.hist, L.red, L.out,
                                         [&](uint32_t P, int s, int sh, uint32_t dmask) {
                                             refine_histogram_regs<K, LOADS>(kw, P, s, sh, dmask,
                                                                             L.hist);
                                         });
        write_from_regs<K, LOADS, !GATHER>(a, row, kw, len, b, 0u, 0u, row_view<K>(xr, n), 0, L.red, xr);
    } else if (C <= cap) {
        compact_candidates<K, LOADS>(kw, len, d1.v << K::SH1, L.wtot, L.base, ent, cap);
        DSEL_STAMP((t == 0), row, 5);
        const Bound b = refine_on_list<K>(ent, C, d1, (uint32_t)a.k, L.hist, L.red, L.out);
        DSEL_STAMP((t == 0), row, 6);
        write_from_list<K, !GATHER>(a, row, ent, C, b, L.red, xr);
        DSEL_STAMP((t == 0), row, 7);
    } else {
        // the candidates do not fit the list: the passes re-read the row
        const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, n);
        const Bound b = refine_passes<K>(d1, (uint32_t)a.k, L.hist, L.red, L.out,
                                         [&](uint32_t P, int s, int sh, uint32_t dmask) {
                                             refine_histogram_stream<K>(view, 0, len, P, s, sh,
                                                                        dmask, L.hist);
                                         });
        write_from_stream<K, !GATHER>(a, row, view, 0, len, b, 0u, 0u, L.red, xr);
    }
    if (t == 0 && a.nan_flag) a.nan_flag[row] = (uint8_t)block_nan;
}

// A workgroup walks rows blockIdx.x, blockIdx.x + gridDim.x, ... (one row
// each when the grid covers the rows).  A row's loads are issued when the
// workgroup reaches it; other workgroups on the compute unit hide their
// latency.  Holding only one row in VGPRs keeps more workgroups resident,
// which pays more than double-buffering the next row's loads.
template <class K, int EPT, bool GATHER = false>
__global__ __launch_bounds__(NT) void topk_rows_whole(const TopkArgs a) {
    using raw_t = typename K::raw_t;
    constexpr int LOADS = EPT / K::VEC;
    static_assert(EPT % K::VEC == 0, "EPT must be a multiple of the vector width");
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];  // histogram, candidate list
    __shared__ TopkShared<LOADS> S;
    const TopkLds L{s_dyn, S.wtot, S.base, S.red, S.out};
    const List ent = list_of<K>(s_dyn + list_base<K>());
    const raw_t *x = reinterpret_cast<const raw_t *>(a.x);

    const int64_t R = a.rows - a.row0;
#pragma unroll 1
    for (int64_t t = blockIdx.x; t < R; t += gridDim.x) {
        const int64_t row = a.row0 + taker_row(a.row_order, t, R);
        const int64_t n = valid_length(a, row);
        DSEL_STAMP((tid() == 0), row, 0);
        const raw_t *xr = x + row * a.x_stride;
        if (n <= a.k) {
            write_short_row<K>(a, row, n, 0, 1, xr);
        } else {
            uint4 v[LOADS];
            load_row<K, LOADS>(xr, n, v);
            select_row<K, LOADS, GATHER>(a, row, n, v, L, ent);
        }
        if constexpr (GATHER) {
            // the row's positions, as this workgroup wrote them, into LDS
            // (the select's space is free; it holds at least k words); each
            // thread's stores are acknowledged before the barrier, so the
            // reads after it see them
            drain_memory();
            __syncthreads();
            int32_t *s_pos = reinterpret_cast<int32_t *>(s_dyn);
            const uint32_t *ib = reinterpret_cast<const uint32_t *>(a.out_idx) +
                                 row * a.idx_stride * (a.idx64 ? 2 : 1);
            for (int j = tid(); j < a.k; j += NT) s_pos[j] = (int32_t)ld_agent(ib + (a.idx64 ? 2 * j : j));
            __syncthreads();
            gather_tail<NT>(a, row, tid(), [&](uint32_t j) -> int64_t { return s_pos[j]; },
                            reinterpret_cast<uint32_t *>(s_dyn) + a.k);
        }
        DSEL_STAMP((tid() == 0), row, 8);
        __syncthreads();  // LDS is reused by the next row
    }
}

// ---------------------------------------------------------------------------
// Short rows (at most 64 x EPL columns): one wave per row.  The keys stay in
// VGPRs, each wave has its own LDS histogram and every scan is a wave scan,
// so a row needs no workgroup barrier: four rows run side by side in a
// workgroup, and many more rows are in flight per compute unit than with a
// workgroup per row.
// ---------------------------------------------------------------------------

// Digit plan of the wave kernel: bf16 10 + 6 bits (a 1024-bin first
// histogram, 4 KB per wave), fp32 11 + 11 + 10.
template <class K>
struct WaveDigits;
template <>
struct WaveDigits<Bf16Key> {
    static constexpr int NPASS = 2, HB = 1024, SH1 = 6;
    __device__ static int bits(int pass) { return pass == 0 ? 10 : 6; }
};
template <>
struct WaveDigits<F32Key> {
    static constexpr int NPASS = 3, HB = 2048, SH1 = 21;
    __device__ static int bits(int pass) { return pass == 2 ? 10 : 11; }
};

// LDS words per wave: its histogram and one spare bin per lane.
template <class K>
__host__ __device__ constexpr uint32_t wave_lds_words() {
    return (uint32_t)WaveDigits<K>::HB + 64;
}

// find_digit for one wave: lane l sums the bins [nb - (l+1)*bpt, nb - l*bpt)
// from the top, one wave scan finds the lane holding the need-th largest
// element, and that lane walks its bins.
__device__ __forceinline__ Digit wave_find_digit(const uint32_t *hist, int nb, uint32_t need) {
    const int lane = tid() & 63;
    const int bpt = nb > 64 ? nb / 64 : 1;
    const int nact = nb / bpt;
    const int top = nb - lane * bpt;
    uint32_t local = 0;
    if (lane < nact)
        for (int i = 1; i <= bpt; ++i) local += hist[top - i];
    const uint32_t incl = wave_incl_scan(local);
    const uint32_t excl = incl - local;
    const uint64_t m = __ballot(lane < nact && excl < need && need <= incl);
    const int L = (int)__builtin_ctzll(m);  // uniform; m != 0 when the bins hold >= need
    uint32_t v = 0, above = 0, cnt = 0;
    if (lane == L) {
        uint32_t acc = excl;
        for (int i = 1; i <= bpt; ++i) {
            const uint32_t h = hist[top - i];
            if (acc + h >= need) {
                v = (uint32_t)(top - i);
                above = acc;
                cnt = h;
                break;
            }
            acc += h;
        }
    }
    return Digit{(uint32_t)__builtin_amdgcn_readlane((int)v, L),
                 (uint32_t)__builtin_amdgcn_readlane((int)above, L),
                 (uint32_t)__builtin_amdgcn_readlane((int)cnt, L)};
}

// A row's outputs as range-checked buffer views: a store at an offset past
// the row's k slots is dropped by the hardware, so a lane that takes no
// element stores to kDrop and the write needs no branch.
// Write one wave's row from its keys in VGPRs (coalesced layout, load j of
// lane l at columns (j*64 + l)*VEC...).  First pass (fix = false): indices,
// and values rebuilt from the keys; amb reports whether a +-0 / NaN key was
// taken.  Second pass (fix = true): only those keys' values, from the row.
template <class K, int LPL>
__device__ __forceinline__ void wave_write(const RowViews &o, uint32_t (&kw)[LPL * 4], int len,
                                           Bound b, int lane, const typename K::raw_t *xr,
                                           bool fix, uint32_t &amb) {
    constexpr int VEC = K::VEC, EPW = K::EPW, SPAN = 64 * VEC;
    const int any = (len + SPAN - 1) / SPAN;
    uint32_t G = 0, Q = 0;  // taken-above and equal counts of earlier loads
#pragma unroll
    for (int j = 0; j < LPL; ++j) {
        if (j >= any) continue;
        uint32_t g = 0, q = 0;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t key = K::elem(kw[4 * j + qq], h);
                const uint32_t pre = key >> b.s;
                g += (key && pre > b.P) ? 1u : 0u;
                q += (key && pre == b.P) ? 1u : 0u;
            }
        const uint32_t mine = g | (q << 16);
        const uint32_t incl = wave_incl_scan(mine);
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        uint32_t gb = G + ((incl - mine) & 0xFFFFu), qb = Q + ((incl - mine) >> 16);
        const uint32_t p = (uint32_t)(j * 64 + lane) * VEC;
        // recompute the comparisons below rather than keep a lane mask per
        // element alive across the scan
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) kw[4 * j + qq] = opaque(kw[4 * j + qq]);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t key = K::elem(kw[4 * j + qq], h);
                const uint32_t pre = key >> b.s;
                const bool gt = key && pre > b.P, eq = key && pre == b.P;
                const bool take = gt || (eq && qb < b.need);
                const uint32_t pos = gt ? gb + min(qb, b.need) : gb + qb;
                const uint32_t col = p + qq * EPW + h;
                if (!fix) {
                    view_store<K>(o, take, pos, col, K::value_bits(key));
                    amb |= (take && K::ambiguous(key)) ? 1u : 0u;
                } else if (take && K::ambiguous(key)) {
                    view_store_value<K>(o, true, pos, (uint32_t)xr[col]);
                }
                gb += gt ? 1u : 0u;
                qb += eq ? 1u : 0u;
            }
        G += tot & 0xFFFFu;
        Q += tot >> 16;
    }
}

// Bytes of a row's staged output: k indices, then (16-byte aligned) k values.
__device__ __forceinline__ uint32_t stage_value_offset(const TopkArgs &a) {
    return ((uint32_t)a.k * (a.idx64 ? 8u : 4u) + 15u) & ~15u;
}
template <class K>
__device__ __forceinline__ uint32_t stage_bytes(const TopkArgs &a) {
    return stage_value_offset(a) + (a.ret_val ? (uint32_t)a.k * (uint32_t)sizeof(typename K::raw_t) : 0u);
}

// Copy `bytes` bytes (a multiple of 2) from LDS to a 16-byte aligned global
// row: 16 bytes per lane and store while they last, then words, then a last
// half word.
__device__ __forceinline__ void wave_copy_out(const char *src, char *dst, uint32_t bytes, int lane) {
    const uint32_t full = bytes & ~15u;
    for (uint32_t off = (uint32_t)lane * 16u; off < full; off += 64u * 16u)
        store16_nt(dst + off, *reinterpret_cast<const uint4 *>(src + off));
    const uint32_t words = bytes & ~3u;
    const uint32_t w = full + (uint32_t)lane * 4u;
    if (w < words) *reinterpret_cast<uint32_t *>(dst + w) = *reinterpret_cast<const uint32_t *>(src + w);
    if ((bytes & 2u) && lane == 0)
        *reinterpret_cast<uint16_t *>(dst + words) = *reinterpret_cast<const uint16_t *>(src + words);
}

// Write one wave's row through LDS (the row's k slots fit the wave's LDS
// region): the ranked elements fill the slots in LDS, then the wave copies
// them out with contiguous stores.  Every slot is filled: the row holds more
// than k keys, so exactly k are taken.
template <class K, int LPL>
__device__ __forceinline__ void wave_write_staged(const TopkArgs &a, int64_t row,
                                                  uint32_t (&kw)[LPL * 4], int len, Bound b,
                                                  int lane, const typename K::raw_t *xr,
                                                  char *stage) {
    using raw_t = typename K::raw_t;
    constexpr int VEC = K::VEC, EPW = K::EPW, SPAN = 64 * VEC;
    const int any = (len + SPAN - 1) / SPAN;
    const uint32_t voff = stage_value_offset(a);
    uint32_t G = 0, Q = 0;
#pragma unroll
    for (int j = 0; j < LPL; ++j) {
        if (j >= any) continue;
        uint32_t g = 0, q = 0;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t key = K::elem(kw[4 * j + qq], h);
                const uint32_t pre = key >> b.s;
                g += (key && pre > b.P) ? 1u : 0u;
                q += (key && pre == b.P) ? 1u : 0u;
            }
        const uint32_t mine = g | (q << 16);
        const uint32_t incl = wave_incl_scan(mine);
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        uint32_t gb = G + ((incl - mine) & 0xFFFFu), qb = Q + ((incl - mine) >> 16);
        const uint32_t p = (uint32_t)(j * 64 + lane) * VEC;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) kw[4 * j + qq] = opaque(kw[4 * j + qq]);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int h = 0; h < EPW; ++h) {
                const uint32_t key = K::elem(kw[4 * j + qq], h);
                const uint32_t pre = key >> b.s;
                const bool gt = key && pre > b.P, eq = key && pre == b.P;
                const bool take = gt || (eq && qb < b.need);
                const uint32_t pos = gt ? gb + min(qb, b.need) : gb + qb;
                const uint32_t col = p + qq * EPW + h;
                if (take) {
                    if (a.idx64)
                        reinterpret_cast<uint64_t *>(stage)[pos] = col;
                    else
                        reinterpret_cast<uint32_t *>(stage)[pos] = col;
                    if (a.ret_val)
                        reinterpret_cast<raw_t *>(stage + voff)[pos] =
                            K::ambiguous(key) ? xr[col] : (raw_t)K::value_bits(key);
                }
                gb += gt ? 1u : 0u;
                qb += eq ? 1u : 0u;
            }
        G += tot & 0xFFFFu;
        Q += tot >> 16;
    }
    wave_sync();
    const int isz = a.idx64 ? 8 : 4;
    wave_copy_out(stage, reinterpret_cast<char *>(a.out_idx) + row * a.idx_stride * isz,
                  (uint32_t)a.k * (uint32_t)isz, lane);
    if (a.ret_val)
        wave_copy_out(stage + voff,
                      reinterpret_cast<char *>(a.out_val) + row * a.val_stride * (int64_t)sizeof(raw_t),
                      (uint32_t)a.k * (uint32_t)sizeof(raw_t), lane);
}

// EPL = columns per lane (a multiple of VEC); rows of n <= k are padded.
// RV: the instance for calls that return values (launched only with
// a.ret_val set), whose short rows copy values out of line with 16-byte
// loads; index-only calls take the other instance, which has no call.
template <class K, int EPL, bool RV>
__global__ __launch_bounds__(NT) void topk_rows_wave(const TopkArgs a) {
    using raw_t = typename K::raw_t;
    using D = WaveDigits<K>;
    constexpr int VEC = K::VEC, EPW = K::EPW, LPL = EPL / VEC, SPAN = 64 * VEC;
    static_assert(EPL % VEC == 0, "EPL must be a multiple of the vector width");
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];  // one histogram per wave
    // the wave index, uniform (in an SGPR): the row, its views and the
    // output descriptors are then scalar, not per-lane values
    const int lane = tid() & 63, wid = __builtin_amdgcn_readfirstlane(tid() >> 6);
    uint32_t *hist = s_dyn + wid * wave_lds_words<K>();
    // the row's output is staged in the histogram's space, or, when a launch
    // that returns values gives one, in a region of its own after the
    // histograms (the index-only instance keeps every LDS offset constant)
    char *stage = reinterpret_cast<char *>(hist);
    uint32_t stage_cap = wave_lds_words<K>() * 4u;
    if constexpr (RV) {
        if (a.stage_words) {
            stage = reinterpret_cast<char *>(s_dyn + NWAVE * wave_lds_words<K>() + wid * a.stage_words);
            stage_cap = a.stage_words * 4u;
        }
    }
    const raw_t *x = reinterpret_cast<const raw_t *>(a.x);
    const int64_t step = (int64_t)gridDim.x * NWAVE;

    const int64_t R = a.rows - a.row0;
#pragma unroll 1
    for (int64_t t = (int64_t)blockIdx.x * NWAVE + wid; t < R; t += step) {
        const int64_t row = a.row0 + taker_row(a.row_order, t, R);
        const int64_t n = valid_length(a, row);
        const raw_t *xr = x + row * a.x_stride;
        if (n <= a.k) {
            if constexpr (RV) {
                write_short_idx(a, row, n, 0, 0, a.k, lane, 64);
                write_short_values_wave<K>(reinterpret_cast<raw_t *>(a.out_val) + row * a.val_stride,
                                           (raw_t)a.val_fill, n, a.k, xr, lane);
            } else {
                write_short_row<K>(a, row, n, 0, 1, xr, lane, 64);
            }
            continue;
        }
        const int len = (int)n;
        uint4 v[LPL];
        {
            const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, n);
#pragma unroll
            for (int j = 0; j < LPL; ++j) v[j] = load_vec<K, false>(view, (int64_t)(j * 64 + lane) * VEC);
        }
        wave_sync();  // the previous row's reads of the histogram are done
        for (int i = lane; i < D::HB + 64; i += 64) hist[i] = 0;
        uint32_t kw[LPL * 4];
        const bool row_nan = __ballot(keys_of_loads<K, LPL, 64>(v, len, kw, lane) != 0u) != 0;
        wave_sync();

        // first digit
        const int full = len / SPAN, any = (len + SPAN - 1) / SPAN;
        const uint32_t spare = (uint32_t)D::HB + (uint32_t)lane;
#pragma unroll
        for (int j = 0; j < LPL; ++j)
            if (j < any)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) {
                        const uint32_t key = K::elem(kw[4 * j + q], h);
                        atomicAdd(&hist[(j < full || key) ? (key >> D::SH1) : spare], 1u);
                    }
        wave_sync();
        const Digit d1 = wave_find_digit(hist, D::HB, (uint32_t)a.k);

        // the later digits, from the keys in VGPRs
        Bound b{d1.v, D::SH1, (uint32_t)a.k - d1.above};
        if (d1.cnt != b.need) {
#pragma unroll 1
            for (int pass = 1; pass < D::NPASS; ++pass) {
                const int d = D::bits(pass);
                const int sh = b.s - d;
                const int nb = 1 << d;
                wave_sync();
                for (int i = lane; i < nb; i += 64) hist[i] = 0;
                wave_sync();
#pragma unroll
                for (int w = 0; w < LPL * 4; ++w)
#pragma unroll
                    for (int h = 0; h < EPW; ++h) {
                        const uint32_t key = K::elem(kw[w], h);
                        if (key && (key >> b.s) == b.P)
                            atomicAdd(&hist[(key >> sh) & (uint32_t)(nb - 1)], 1u);
                    }
                wave_sync();
                const Digit dg = wave_find_digit(hist, nb, b.need);
                b.need -= dg.above;
                b.P = (b.P << d) | dg.v;
                b.s = sh;
                if (dg.cnt == b.need) break;
            }
        }

        // the selection in column order: per load, a wave scan of the lanes'
        // (equal << 16 | above) counts gives each lane its ranks.  Values come
        // from the keys, so the stores wait for no load; +-0 / NaN keys get
        // their bits from the row in a second pass, run only if one was taken.
        if (stage_bytes<K>(a) <= stage_cap) {
            wave_sync();  // the histogram is dead: its space may hold the row's slots
            wave_write_staged<K, LPL>(a, row, kw, len, b, lane, xr, stage);
        } else {
            const RowViews o = row_views<K>(a, row);
            uint32_t amb = 0;
            wave_write<K, LPL>(o, kw, len, b, lane, xr, false, amb);
            if (o.has_val && __ballot(amb != 0u))
                wave_write<K, LPL>(o, kw, len, b, lane, xr, true, amb);
        }
        if (lane == 0 && a.nan_flag) a.nan_flag[row] = row_nan ? 1u : 0u;
    }
}

// ---------------------------------------------------------------------------
// bf16 rows of at most 2048 columns: one wave per row on packed 16-bit keys.
//
// A row's keys stay packed two per VGPR (element 2q in the low half of word
// q of a load) from the transform to the write, so the transform, the NaN
// probe and the value rebuild are packed 16-bit operations.  Each load is
// turned into keys and histogrammed (10-bit first digit, 1024 bins) as soon
// as it arrives.  The digit search reads the histogram 16 bins per lane,
// finds the lane holding the k-th key with one wave scan, then resolves the
// bin inside that lane's 16 with one 16-lane scan (no serial walk).  A
// second pass over the 6 low bits (64 bins) of the boundary bin's keys
// gives the exact threshold key T and the number of T-keys to take.
//
// The selection is then a per-element predicate, key > T' (or, when equal
// keys at T are only partly taken, key > T or key == T at a column at or
// before the cut: the column of the last T-key taken, found once per row
// with per-load wave scans), so the write needs one comparison per element:
// per load, a wave scan of the lanes' counts gives each lane its first slot
// in column order.  The slots are filled in LDS and copied out with
// contiguous 16-byte stores (or stored straight to the row when the stage
// does not fit).
// ---------------------------------------------------------------------------
constexpr int W16_BINS = 1024;                    // first digit: key >> 6
constexpr uint32_t W16_WORDS = W16_BINS + 64;     // bins, then one spare bin per lane

// Keys of two bf16 values: 0x8000 + magnitude (positive), 0x8000 -
// magnitude (negative): x ^ (s | 0x8000) - s per half, s the sign spread
// over the half.
__device__ __forceinline__ uint32_t bf16_key2(uint32_t x) {
    const u16x2 s = __builtin_bit_cast(u16x2, __builtin_bit_cast(s16x2, as_u16x2(x)) >> (short)15);
    const uint32_t t = x ^ (as_u32(s) | 0x80008000u);
    return as_u32(as_u16x2(t) - s);
}

// The values of two keys (the inverse map; key 0x8000 gives +0 and the NaN
// key 0xFFFF gives 0xFFFF, so those two keys' bits come from the row).
__device__ __forceinline__ uint32_t bf16_val2(uint32_t key) {
    const u16x2 s = __builtin_bit_cast(
        u16x2, __builtin_bit_cast(s16x2, as_u16x2(key ^ 0x80008000u)) >> (short)15);
    return as_u32(as_u16x2(key) + s) ^ (as_u32(s) | 0x80008000u);
}

__device__ __forceinline__ bool K16ambiguous(uint32_t key) { return key == 0x8000u || key == 0xFFFFu; }

// Packed 16-bit max / min.
__device__ __forceinline__ uint32_t pk_max16(uint32_t a, uint32_t b) {
    return as_u32(__builtin_elementwise_max(as_u16x2(a), as_u16x2(b)));
}
__device__ __forceinline__ uint32_t pk_min16(uint32_t a, uint32_t b) {
    return as_u32(__builtin_elementwise_min(as_u16x2(a), as_u16x2(b)));
}

// Word with the halves at and past `valid` (0..2 in this word) cleared.
__device__ __forceinline__ uint32_t keep_halves(uint32_t w, int valid) {
    return valid >= 2 ? w : (valid == 1 ? (w & 0xFFFFu) : 0u);
}

// The bin of a 1024-bin histogram holding the need-th largest key.
__device__ __forceinline__ Digit w16_find1024(const uint32_t *hist, uint32_t need, int lane) {
    return wave_find1024(hist, need, lane);
}

// The same for a 64-bin histogram.
__device__ __forceinline__ Digit w16_find64(const uint32_t *hist, uint32_t need, int lane) {
    const uint32_t h = hist[63 - lane];
    const uint32_t incl = wave_incl_scan(h);
    const int L = (int)__builtin_ctzll(__ballot(incl >= need));
    return Digit{(uint32_t)(63 - L), rdlane(incl - h, L), rdlane(h, L)};
}

// One wave's selection written in column order.  take(key, col) decides an
// element; emit(pos, col, key_half, val_half) stores a taken one.  (The
// direct-store and value fix-up paths.)
template <int LPL, class Take, class Emit>
__device__ __forceinline__ void w16_write(const uint32_t (&kw)[LPL * 4], int any, int lane,
                                          Take take, Emit emit) {
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < LPL; ++j) {
        if (j >= any) break;
        const uint32_t c0 = (uint32_t)(j * 64 + lane) * 8u;
        uint32_t cnt = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = opaque(kw[4 * j + q]);
            cnt += take(w & 0xFFFFu, c0 + 2 * q) ? 1u : 0u;
            cnt += take(w >> 16, c0 + 2 * q + 1) ? 1u : 0u;
        }
        const uint32_t incl = wave_incl_scan(cnt);
        uint32_t pos = run + incl - cnt;
        run += rdlane(incl, 63);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = opaque(kw[4 * j + q]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t key = h ? (w >> 16) : (w & 0xFFFFu);
                const uint32_t col = c0 + 2 * q + h;
                if (take(key, col)) {
                    emit(pos, col, key);
                    ++pos;
                }
            }
        }
    }
}

// The staged form: every element stores, a taken one at its slot of the
// stage (index, and with RVAL the rebuilt value at voff), the others to a
// per-lane dummy word (no branches and no exec-mask changes per element).
// CUT: equal keys at T are only partly taken (those at columns <= cut).
template <int LPL, bool CUT, bool I64, bool RVAL, bool IDX = true>
__device__ __forceinline__ void w16_stage(const uint32_t (&kw)[LPL * 4], int any, int lane,
                                          uint32_t T, uint32_t cut, char *stage, uint32_t voff,
                                          char *dummy, uint32_t &amb) {
    auto take = [&](uint32_t key, uint32_t col) {
        return CUT ? (key > T || (key == T && col <= cut)) : key > T;
    };
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < LPL; ++j) {
        if (j >= any) break;
        const uint32_t c0 = (uint32_t)(j * 64 + lane) * 8u;
        uint32_t cnt = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = kw[4 * j + q];
            cnt += take(w & 0xFFFFu, c0 + 2 * q) ? 1u : 0u;
            cnt += take(w >> 16, c0 + 2 * q + 1) ? 1u : 0u;
        }
        const uint32_t incl = wave_incl_scan(cnt);
        uint32_t pos = run + incl - cnt;
        run += rdlane(incl, 63);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = opaque(kw[4 * j + q]);
            const uint32_t vw = RVAL ? bf16_val2(w) : 0u;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t key = h ? (w >> 16) : (w & 0xFFFFu);
                const uint32_t col = c0 + 2 * q + h;
                const bool t = take(key, col);
                if constexpr (IDX && I64) {
                    char *p = t ? stage + pos * 8u : dummy;
                    *reinterpret_cast<uint64_t *>(p) = (uint64_t)col;
                } else if constexpr (IDX) {
                    char *p = t ? stage + pos * 4u : dummy;
                    *reinterpret_cast<uint32_t *>(p) = col;
                }
                if constexpr (RVAL) {
                    char *p = t ? stage + voff + pos * 2u : dummy;
                    *reinterpret_cast<uint16_t *>(p) = (uint16_t)(h ? (vw >> 16) : vw);
                    amb |= (t && K16ambiguous(key)) ? 1u : 0u;
                }
                pos += t ? 1u : 0u;
            }
        }
    }
}

// GATHER: workgroups of kGatherWaves waves; each wave selects a row, then
// the whole workgroup copies the gathered keys of its rows one row at a time
// (a row's keys written by many threads at once keep few output streams
// open, which the HBM writes favour over one stream per wave).
template <int LPL, bool RV, bool GATHER = false>
__global__ __launch_bounds__(GATHER ? kGatherWaves * 64 : NT) void topk_rows_wave_bf16(const TopkArgs a) {
    using K = Bf16Key;
    constexpr int SPAN = 64 * 8;  // columns per load over the wave
    constexpr int NW = GATHER ? kGatherWaves : NWAVE;
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];  // one region per wave
    const int wid = __builtin_amdgcn_readfirstlane(tid() >> 6);
    uint32_t *hist = s_dyn + wid * W16_WORDS;
    char *stage = reinterpret_cast<char *>(hist);
    uint32_t stage_cap = W16_WORDS * 4u;
    if constexpr (RV) {
        if (a.stage_words) {
            stage = reinterpret_cast<char *>(s_dyn + NW * W16_WORDS + wid * a.stage_words);
            stage_cap = a.stage_words * 4u;
        }
    }
    // GATHER: each wave's row, valid length and where its positions are
    // (0: a short row's, 1: this wave's stage, 2: the index row in memory)
    __shared__ int64_t g_row[GATHER ? NW : 1], g_n[GATHER ? NW : 1];
    __shared__ int g_mode[GATHER ? NW : 1];
    const uint16_t *x = reinterpret_cast<const uint16_t *>(a.x);
    const int64_t step = (int64_t)gridDim.x * NW;

    const int64_t R = a.rows - a.row0;

#pragma unroll 1
    for (int64_t base = (int64_t)blockIdx.x * NW; base < R; base += step) {  // uniform
      const int64_t t = base + wid;
      if constexpr (GATHER) {
          if (tid() % 64 == 0) g_row[wid] = -1;
      }
      do {  // this wave's row ("continue" ends it)
        if (t >= R) continue;
        const int64_t row = a.row0 + taker_row(a.row_order, t, R);
        // the lane index again, opaque: the per-lane column numbers derived
        // from it must not be hoisted out of the row loop into VGPRs
        const int lane = tid() & 63;
        const uint16_t *xr = x + row * a.x_stride;
        const int64_t n = valid_length(a, row);
        DSEL_STAMP((lane == 0), row, 0);
        DSEL_STAMP_VALUE((lane == 0), row, 7, (unsigned long long)n);
        if (n <= a.k) {
            if constexpr (RV) {
                write_short_idx(a, row, n, 0, 0, a.k, lane, 64);
                write_short_values_wave<K>(reinterpret_cast<uint16_t *>(a.out_val) + row * a.val_stride,
                                           (uint16_t)a.val_fill, n, a.k, xr, lane);
            } else {
                write_short_row<K>(a, row, n, 0, 1, xr, lane, 64);
            }
            DSEL_STAMP((lane == 0), row, 4);
            if constexpr (GATHER) {
                if (lane == 0) {
                    g_row[wid] = row;
                    g_n[wid] = n;
                    g_mode[wid] = 0;
                }
            }
            continue;
        }
        const int len = (int)n;
        const int full = len / SPAN, any = (len + SPAN - 1) / SPAN;  // uniform
        uint4 v[LPL];
        {
            const __amdgpu_buffer_rsrc_t view = row_view<K>(xr, n);
#pragma unroll
            for (int j = 0; j < LPL; ++j)
                if (j < any) v[j] = load_vec<K, false>(view, (int64_t)(j * 64 + lane) * 8);
        }
        wave_sync();  // the previous row's reads of this wave's LDS are done
        {
            uint4 *h4 = reinterpret_cast<uint4 *>(hist);
#pragma unroll
            for (int i = 0; i < W16_BINS / 256; ++i) h4[lane + 64 * i] = make_uint4(0u, 0u, 0u, 0u);
        }
        wave_sync();

        // keys and the first-digit histogram, one load at a time as it arrives
        uint32_t kw[LPL * 4];
        uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
        const uint32_t spare = (uint32_t)W16_BINS + (uint32_t)lane;
#pragma unroll
        for (int j = 0; j < LPL; ++j) {
            if (j >= any) {
#pragma unroll
                for (int q = 0; q < 4; ++q) kw[4 * j + q] = 0u;
                continue;
            }
            uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
            if (j < full) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t kk = bf16_key2(w[q]);
                    kmax = pk_max16(kmax, kk);
                    kmin = pk_min16(kmin, kk);
                    kw[4 * j + q] = kk;
                    atomicAdd(&hist[(kk >> 6) & 0x3FFu], 1u);
                    atomicAdd(&hist[kk >> 22], 1u);
                }
            } else {
                // the row ends in this load: halves at or past it get key 0
                // (raw bits cleared first, so they are never probed)
                int valid = len - (j * 64 + lane) * 8;
                valid = valid < 0 ? 0 : (valid > 8 ? 8 : valid);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t kk = bf16_key2(keep_halves(w[q], valid - 2 * q));
                    kmax = pk_max16(kmax, kk);
                    kmin = pk_min16(kmin, kk);
                    const uint32_t kz = keep_halves(kk, valid - 2 * q);
                    kw[4 * j + q] = kz;
                    const uint32_t lo = kz & 0xFFFFu, hi = kz >> 16;
                    atomicAdd(&hist[lo ? (lo >> 6) : spare], 1u);
                    atomicAdd(&hist[hi ? (hi >> 6) : spare], 1u);
                }
            }
        }
        // a NaN key lies above +inf's (0xFF80) or below -inf's (0x0080)
        const bool row_nan =
            __ballot(max(kmax & 0xFFFFu, kmax >> 16) > 0xFF80u || min(kmin & 0xFFFFu, kmin >> 16) < 0x0080u) != 0ull;
        DSEL_STAMP((lane == 0), row, 1);
        if (row_nan) {
            // rare: every NaN to the top key, and the histogram again
            wave_sync();
            {
                uint4 *h4 = reinterpret_cast<uint4 *>(hist);
#pragma unroll
                for (int i = 0; i < W16_BINS / 256; ++i) h4[lane + 64 * i] = make_uint4(0u, 0u, 0u, 0u);
            }
            wave_sync();
#pragma unroll
            for (int j = 0; j < LPL; ++j) {
                if (j >= any) break;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t kz = K::fix_nan_word(kw[4 * j + q]);
                    kw[4 * j + q] = kz;
                    const uint32_t lo = kz & 0xFFFFu, hi = kz >> 16;
                    atomicAdd(&hist[lo ? (lo >> 6) : spare], 1u);
                    atomicAdd(&hist[hi ? (hi >> 6) : spare], 1u);
                }
            }
        }
        wave_sync();
        const uint32_t k = (uint32_t)a.k;
        const Digit d1 = w16_find1024(hist, k, lane);
        DSEL_STAMP((lane == 0), row, 2);
        // every valid key is at least -inf's 0x0080, so the boundary bin is
        // >= 2 and no empty slot (key 0) is ever counted in it
        uint32_t T, cut = 0xFFFFFFFFu;  // take: key > T, or key == T at a column <= cut
        const uint32_t need1 = k - d1.above;
        if (d1.cnt == need1) {
            T = (d1.v << 6) - 1u;  // the boundary bin is taken whole
        } else {
            wave_sync();
            hist[lane] = 0u;
            wave_sync();
            // every element adds: the boundary bin's keys to their low 6
            // bits' bin, the others to this lane's spare bin (no branches)
            const uint32_t spare2 = 64u + (uint32_t)lane;
#pragma unroll
            for (int j = 0; j < LPL; ++j) {
                if (j >= any) break;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w = kw[4 * j + q];
                    const uint32_t lo = w & 0xFFFFu, hi = w >> 16;
                    atomicAdd(&hist[(lo >> 6) == d1.v ? (lo & 63u) : spare2], 1u);
                    atomicAdd(&hist[(hi >> 6) == d1.v ? (hi & 63u) : spare2], 1u);
                }
            }
            wave_sync();
            const Digit d2 = w16_find64(hist, need1, lane);
            const uint32_t needT = need1 - d2.above;  // T-keys to take, 1..d2.cnt
            T = (d1.v << 6) | d2.v;
            if (needT == d2.cnt) {
                T -= 1u;  // every T-key is taken
            } else {
                // the column of the needT-th T-key in column order
                uint32_t rem = needT;
#pragma unroll
                for (int j = 0; j < LPL; ++j) {
                    if (j >= any) break;
                    uint32_t c = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t w = kw[4 * j + q];
                        c += ((w & 0xFFFFu) == T) ? 1u : 0u;
                        c += ((w >> 16) == T) ? 1u : 0u;
                    }
                    const uint32_t incl = wave_incl_scan(c);
                    const uint32_t tot = rdlane(incl, 63);
                    if (rem <= tot) {
                        const int L = (int)__builtin_ctzll(__ballot(incl >= rem));
                        uint32_t r = rem - rdlane(incl - c, L);
                        uint32_t col = 0;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t w = kw[4 * j + q];
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                const bool eq = (h ? (w >> 16) : (w & 0xFFFFu)) == T;
                                if (eq && r == 1u) col = (uint32_t)(j * 64 + lane) * 8u + 2 * q + h;
                                r -= eq ? 1u : 0u;
                            }
                        }
                        cut = rdlane(col, L);
                        break;
                    }
                    rem -= tot;
                }
            }
        }

        DSEL_STAMP((lane == 0), row, 3);
        // the write
        const bool rv = RV && a.ret_val;  // (the values instance is launched only with values)
        const uint32_t idx_bytes = a.idx64 ? 8u : 4u;
        const uint32_t ibytes = (uint32_t)a.k * idx_bytes;
        // staged when the slots fit the stage; in the histogram's space they
        // must leave its last 256 bytes (the spare bins) to the dummy stores.
        // Without a stage of its own, a row with values stages its indices
        // and then its values there, one after the other ("two").
        bool staged, two = false;
        uint32_t voff;
        if (RV && a.stage_words) {
            voff = (ibytes + 15u) & ~15u;
            staged = voff + (rv ? (uint32_t)a.k * 2u : 0u) <= stage_cap;
        } else {
            staged = ibytes <= (uint32_t)W16_BINS * 4u && (!rv || (uint32_t)a.k * 2u <= (uint32_t)W16_BINS * 4u);
            two = rv && staged;
            voff = two ? 0u : (ibytes + 15u) & ~15u;
        }
        uint32_t amb = 0;
        char *const dummy = reinterpret_cast<char *>(hist + W16_BINS + (lane & ~1));
        if (two) {
            if constexpr (RV) {
                wave_sync();  // the histogram is dead: its space holds the indices
                const bool c = cut != 0xFFFFFFFFu;
                if (a.idx64) {
                    if (c) w16_stage<LPL, true, true, false>(kw, any, lane, T, cut, stage, 0u, dummy, amb);
                    else   w16_stage<LPL, false, true, false>(kw, any, lane, T, cut, stage, 0u, dummy, amb);
                } else {
                    if (c) w16_stage<LPL, true, false, false>(kw, any, lane, T, cut, stage, 0u, dummy, amb);
                    else   w16_stage<LPL, false, false, false>(kw, any, lane, T, cut, stage, 0u, dummy, amb);
                }
                wave_sync();
                wave_copy_out(stage, reinterpret_cast<char *>(a.out_idx) + row * a.idx_stride * (int64_t)idx_bytes,
                              ibytes, lane);
                wave_sync();  // the indices are read out: the values take their place
                if (c) w16_stage<LPL, true, false, true, false>(kw, any, lane, T, cut, stage, 0u, dummy, amb);
                else   w16_stage<LPL, false, false, true, false>(kw, any, lane, T, cut, stage, 0u, dummy, amb);
            }
        } else if (staged) {
            wave_sync();  // the histogram is dead: its space may hold the row's slots
            const bool c = cut != 0xFFFFFFFFu;
            if (rv) {
                if constexpr (RV) {
                    if (a.idx64) {
                        if (c) w16_stage<LPL, true, true, true>(kw, any, lane, T, cut, stage, voff, dummy, amb);
                        else   w16_stage<LPL, false, true, true>(kw, any, lane, T, cut, stage, voff, dummy, amb);
                    } else {
                        if (c) w16_stage<LPL, true, false, true>(kw, any, lane, T, cut, stage, voff, dummy, amb);
                        else   w16_stage<LPL, false, false, true>(kw, any, lane, T, cut, stage, voff, dummy, amb);
                    }
                }
            } else if (a.idx64) {
                if (c) w16_stage<LPL, true, true, false>(kw, any, lane, T, cut, stage, voff, dummy, amb);
                else   w16_stage<LPL, false, true, false>(kw, any, lane, T, cut, stage, voff, dummy, amb);
            } else {
                if (c) w16_stage<LPL, true, false, false>(kw, any, lane, T, cut, stage, voff, dummy, amb);
                else   w16_stage<LPL, false, false, false>(kw, any, lane, T, cut, stage, voff, dummy, amb);
            }
        } else {
            const RowViews o = row_views<K>(a, row);
            auto direct = [&](auto take) {
                w16_write<LPL>(kw, any, lane, take, [&](uint32_t pos, uint32_t col, uint32_t key) {
                    view_store<K>(o, true, pos, col, bf16_val2(key) & 0xFFFFu);
                    amb |= K::ambiguous(key) ? 1u : 0u;
                });
            };
            if (cut == 0xFFFFFFFFu)
                direct([&](uint32_t key, uint32_t) { return key > T; });
            else
                direct([&](uint32_t key, uint32_t col) { return key > T || (key == T && col <= cut); });
        }
        // +-0 and NaN keys: the value bits come from the row (the rebuilt
        // bits of the same slot are overwritten)
        if (rv && __ballot(amb != 0u)) {
            const RowViews o = row_views<K>(a, row);
            auto fix = [&](auto take) {
                w16_write<LPL>(kw, any, lane, take, [&](uint32_t pos, uint32_t col, uint32_t key) {
                    if (!K::ambiguous(key)) return;
                    if (staged)
                        reinterpret_cast<uint16_t *>(stage + voff)[pos] = xr[col];
                    else
                        view_store_value<K>(o, true, pos, (uint32_t)xr[col]);
                });
            };
            if (cut == 0xFFFFFFFFu)
                fix([&](uint32_t key, uint32_t) { return key > T; });
            else
                fix([&](uint32_t key, uint32_t col) { return key > T || (key == T && col <= cut); });
        }
        if (staged) {
            wave_sync();
            if (!two)
                wave_copy_out(stage, reinterpret_cast<char *>(a.out_idx) + row * a.idx_stride * (int64_t)idx_bytes,
                              ibytes, lane);
            if (rv)
                wave_copy_out(stage + voff,
                              reinterpret_cast<char *>(a.out_val) + row * a.val_stride * 2,
                              (uint32_t)a.k * 2u, lane);
        }
        if (lane == 0 && a.nan_flag) a.nan_flag[row] = row_nan ? 1u : 0u;
        DSEL_STAMP((lane == 0), row, 4);
        if constexpr (GATHER) {
            if (lane == 0) {
                g_row[wid] = row;
                g_n[wid] = n;
                g_mode[wid] = staged ? 1 : 2;
            }
        }
      } while (false);
      if constexpr (GATHER) {
          // every wave's row selected and its index row written (and the
          // stores acknowledged, for the rows read back from memory): the
          // workgroup copies their keys, row by row
          drain_memory();
          __syncthreads();
#pragma unroll 1
          for (int w = 0; w < NW; ++w) {
              const int64_t grow = g_row[w];
              if (grow < 0) continue;  // uniform
              const int64_t gn = g_n[w];
              const int mode = g_mode[w];
              const int sh = a.idx64 ? 1 : 0;
              // the positions: a short row's, the wave's stage (low words of
              // int64 slots), or the index row in memory
              const int32_t *sp = reinterpret_cast<const int32_t *>(s_dyn + w * W16_WORDS);
              const uint32_t *ib = reinterpret_cast<const uint32_t *>(a.out_idx) +
                                   grow * a.idx_stride * (a.idx64 ? 2 : 1);
              uint32_t *s_off = s_dyn + NW * W16_WORDS;  // k words past the waves' regions
              if (mode == 0)
                  gather_tail<NW * 64>(a, grow, tid(), [&](uint32_t j) -> int64_t { return (int64_t)j < gn ? (int64_t)j : -1; }, s_off);
              else if (mode == 1)
                  gather_tail<NW * 64>(a, grow, tid(), [&](uint32_t j) -> int64_t { return sp[j << sh]; }, s_off);
              else
                  gather_tail<NW * 64>(a, grow, tid(), [&](uint32_t j) -> int64_t { return (int32_t)ld_agent(ib + (j << sh)); }, s_off);
          }
          __syncthreads();  // the stages are read: the next rows may reuse them
      }
    }
}

// ---------------------------------------------------------------------------
// Value order (sorted_index = 2): each row's selection, largest value first,
// equal values by ascending column.  One workgroup per row sorts the row's
// c = min(k, n) (key, column) pairs in LDS; the padding slots stay.  Runs
// after the top-k on the same stream, in place on its outputs.
//
// The select leaves every row in ascending column order, so a stable sort on
// the key alone orders equal keys by column.  The sort is least significant
// digit first over 9-bit digits of kmax - key, kmax the row's largest
// selected key, each pass stable; only the digits that span kmax - kmin
// needs get a pass (the selected keys all lie at or above the k-th largest,
// so the span is narrow: one pass for most bf16 rows, none for equal keys):
//   * pair j of a pass sits in batch (w*B + b) of 64, wave w's batch b,
//     lane j % 64, with B = ceil(c / 1024) batches per wave, so (w, b, lane)
//     runs in pair order;
//   * a wave ranks each batch's lanes among equal digits with nine ballots
//     and keeps per-(digit, wave) running counts in 16-bit LDS counters,
//     bit 15 marking a count of this pass (the scan rewrites every counter
//     as a prefix with the bit clear, so no pass clears them);
//   * one exclusive scan of the counts in digit-major order gives every
//     (digit, wave) its first slot; each pair goes to that slot plus its rank.
// Four workgroup barriers per pass; a bitonic network over 4096 pairs takes
// 78 steps, each a dependent LDS round trip.
// ---------------------------------------------------------------------------

// Order-preserving key of one value's bits (NaN on top, -0 with +0), the
// element form of the key words above.
template <class K>
__device__ __forceinline__ uint32_t key_of_bits(uint32_t bits) {
    if constexpr (K::PACK) {
        const uint32_t mag = bits & 0x7FFFu;
        if (mag > 0x7F80u) return 0xFFFFu;
        return (bits & 0x8000u) ? 0x8000u - mag : 0x8000u + mag;
    } else {
        const uint32_t mag = bits & 0x7FFFFFFFu;
        if (mag > 0x7F800000u) return 0xFFFFFFFFu;
        return (bits & 0x80000000u) ? 0x80000000u - mag : 0x80000000u + mag;
    }
}

constexpr int SORT_NT = 1024;               // threads of a value-order workgroup
constexpr int SORT_NW = SORT_NT / 64;       // its waves
constexpr int SORT_DB = 9;                  // digit bits
constexpr int SORT_CNT = (1 << SORT_DB) * SORT_NW;  // (digit, wave) counters, digit-major
constexpr int SORT_MAXB = 4;                // batches per wave: k <= 4096

template <class K>
__global__ __launch_bounds__(SORT_NT) void sort_rows_by_value(const TopkArgs a) {
    using raw_t = typename K::raw_t;
    // LDS: k pair words (key << 32 | ~column), the 16-bit counters, the wave
    // totals, the waves' smallest and largest keys
    extern __shared__ __attribute__((aligned(16))) uint64_t s_pair[];
    const int64_t row = a.row0 + blockIdx.x;
    if (row >= a.rows) return;
    const int t = (int)threadIdx.x;
    const int64_t n = valid_length(a, row);
    const uint32_t c = (uint32_t)(n < a.k ? n : a.k);
    if (c <= 1) return;
    // (the pair words rounded up to an even count: what follows is 16-byte aligned)
    uint16_t *cnt_base = reinterpret_cast<uint16_t *>(s_pair + ((a.k + 1) & ~(int64_t)1));
    uint16_t *cnt = cnt_base;
    uint32_t *wtot = reinterpret_cast<uint32_t *>(cnt_base + SORT_CNT);
    uint32_t *wmin = wtot + SORT_NW, *wmax = wmin + SORT_NW;
    const raw_t *xr = reinterpret_cast<const raw_t *>(a.x) + row * a.x_stride;
    const RowOut o = row_out<K>(a, row);
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0;
    for (uint32_t j = (uint32_t)t; j < c; j += SORT_NT) {
        const uint32_t col = o.idx64 ? (uint32_t)reinterpret_cast<const int64_t *>(o.idx)[j]
                                     : (uint32_t)reinterpret_cast<const int32_t *>(o.idx)[j];
        const uint32_t bits = o.val ? (uint32_t)reinterpret_cast<const raw_t *>(o.val)[j]
                                    : (uint32_t)xr[col];
        const uint32_t key = key_of_bits<K>(bits);
        kmin = min(kmin, key);
        kmax = max(kmax, key);
        s_pair[j] = ((uint64_t)key << 32) | (uint32_t)~col;
    }
    for (int i = t; i < SORT_CNT; i += SORT_NT) cnt_base[i] = 0;
    const uint32_t lane = (uint32_t)t & 63u, w = (uint32_t)t >> 6;
    kmin = ~wave_max_u32(~kmin);
    kmax = wave_max_u32(kmax);
    if (lane == 0) {
        wmin[w] = kmin;
        wmax[w] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < SORT_NW; ++v) {
        kmin = min(kmin, wmin[v]);
        kmax = max(kmax, wmax[v]);
    }
    const uint32_t span = kmax - kmin;
    const int passes = span == 0 ? 0 : (32 - __builtin_clz(span) + SORT_DB - 1) / SORT_DB;

    const uint32_t B = (c + SORT_NT - 1) / SORT_NT;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll 1
    for (int pass = 0; pass < passes; ++pass) {
        const int sh = SORT_DB * pass;
        uint64_t el[SORT_MAXB];
        uint32_t dg[SORT_MAXB], rk[SORT_MAXB];
#pragma unroll
        for (int b = 0; b < SORT_MAXB; ++b) {
            el[b] = 0;
            dg[b] = 0;
            rk[b] = 0;
            if ((uint32_t)b < B) {
                const uint32_t j = ((w * B + (uint32_t)b) << 6) + lane;
                const bool valid = j < c;
                const uint64_t e = valid ? s_pair[j] : 0ull;
                const uint32_t d = ((kmax - (uint32_t)(e >> 32)) >> sh) & ((1u << SORT_DB) - 1u);
                uint64_t peers = __ballot(valid);
#pragma unroll
                for (int bit = 0; bit < SORT_DB; ++bit) {
                    const uint64_t m = __ballot((d >> bit) & 1u);
                    peers &= ((d >> bit) & 1u) ? m : ~m;
                }
                uint32_t base = 0;
                if (valid) {
                    const uint32_t raw = cnt[d * SORT_NW + w];
                    base = (raw & 0x8000u) ? (raw & 0x7FFFu) : 0u;  // counted this pass, else 0
                }
                wave_sync();  // every lane has read the count before its leader adds
                if (valid && (uint32_t)__builtin_ctzll(peers) == lane)
                    cnt[d * SORT_NW + w] =
                        (uint16_t)(0x8000u | (base + (uint32_t)__builtin_popcountll(peers)));
                wave_sync();
                el[b] = e;
                dg[b] = d;
                rk[b] = base + (uint32_t)__builtin_popcountll(peers & below);
            }
        }
        __syncthreads();
        // exclusive scan of the counters, eight per thread
        static_assert(SORT_CNT == 8 * SORT_NT, "eight counters per thread");
        const uint4 q = reinterpret_cast<const uint4 *>(cnt)[t];
        uint32_t cv[8];
        {
            const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t raw = (wd[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                cv[i] = (raw & 0x8000u) ? (raw & 0x7FFFu) : 0u;
            }
        }
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) sum += cv[i];
        const uint32_t inc = wave_incl_scan(sum);
        if (lane == 63) wtot[w] = inc;
        __syncthreads();
        uint32_t pre = inc - sum;
#pragma unroll
        for (int v = 0; v < SORT_NW; v += 4) {
            const uint4 q4 = *reinterpret_cast<const uint4 *>(wtot + v);
            pre += ((uint32_t)v < w ? q4.x : 0u) + ((uint32_t)v + 1 < w ? q4.y : 0u) +
                   ((uint32_t)v + 2 < w ? q4.z : 0u) + ((uint32_t)v + 3 < w ? q4.w : 0u);
        }
        uint32_t pw[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const uint32_t lo = pre, hi = pre + cv[i];
            pw[i >> 1] = lo | (hi << 16);
            pre = hi + cv[i + 1];
        }
        reinterpret_cast<uint4 *>(cnt)[t] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        __syncthreads();
#pragma unroll
        for (int b = 0; b < SORT_MAXB; ++b) {
            if ((uint32_t)b < B && ((w * B + (uint32_t)b) << 6) + lane < c)
                s_pair[(uint32_t)cnt[dg[b] * SORT_NW + w] + rk[b]] = el[b];
        }
        __syncthreads();
    }
    for (uint32_t j = (uint32_t)t; j < c; j += SORT_NT) {
        const uint64_t e = s_pair[j];
        const uint32_t col = ~(uint32_t)e, key = (uint32_t)(e >> 32);
        store_index(o, j, col);
        if (o.val)
            store_value<K>(o, j, K::ambiguous(key) ? (uint32_t)xr[col] : K::value_bits(key));
    }
}

template <class K, int EPT, bool SPLIT, bool GATHER>
const void *kptr() {
    if constexpr (SPLIT)
        return reinterpret_cast<const void *>(&topk_rows_split<K, EPT>);
    else
        return reinterpret_cast<const void *>(&topk_rows_whole<K, EPT, GATHER>);
}

template <class K, bool SPLIT, bool GATHER = false>
const void *pick(int ept) {
    static_assert(!(SPLIT && GATHER), "split rows do not fuse the gather");
    switch (ept) {
        case 8: return kptr<K, 8, SPLIT, GATHER>();
        case 16: return kptr<K, 16, SPLIT, GATHER>();
        case 32: return kptr<K, 32, SPLIT, GATHER>();
        case 64: return kptr<K, 64, SPLIT, GATHER>();
        case 128:
            if constexpr (SPLIT) return kptr<K, 128, true, false>();
            return nullptr;
        default: return nullptr;
    }
}

}  // namespace

template <class K, bool RV, bool GATHER = false>
const void *pick_wave(int epl) {
    if constexpr (sizeof(typename K::raw_t) == 2) {
        switch (epl) {
            case 8: return reinterpret_cast<const void *>(&topk_rows_wave_bf16<1, RV, GATHER>);
            case 16: return reinterpret_cast<const void *>(&topk_rows_wave_bf16<2, RV, GATHER>);
            case 32: return reinterpret_cast<const void *>(&topk_rows_wave_bf16<4, RV, GATHER>);
            default: return nullptr;
        }
    } else if constexpr (GATHER) {
        return nullptr;  // fp32 one-wave rows do not fuse the gather
    } else {
        // (only fp32 rows instantiate the generic one-wave kernel)
        switch (epl) {
            case 8: return reinterpret_cast<const void *>(&topk_rows_wave<K, 8, RV>);
            case 16: return reinterpret_cast<const void *>(&topk_rows_wave<K, 16, RV>);
            case 32: return reinterpret_cast<const void *>(&topk_rows_wave<K, 32, RV>);
            default: return nullptr;
        }
    }
}

// ept = columns per thread of one workgroup's range (the whole row, or one
// split chunk), or per lane of a wave's row (kTopkWave).
const void *topk_kernel_ptr(int dtype, int ept, int kind, int ret_val, int gather) {
    if (gather) {
        if (ret_val) return nullptr;  // the fused gather returns no values
        if (kind == kTopkWave) return dtype == 0 ? pick_wave<Bf16Key, false, true>(ept) : nullptr;
        if (kind == kTopkWhole)
            return dtype == 0 ? pick<Bf16Key, false, true>(ept) : pick<F32Key, false, true>(ept);
        return nullptr;
    }
    if (kind == kTopkSplitWx) {
        if (dtype != 1) return nullptr;
        switch (ept) {
            case 8: return reinterpret_cast<const void *>(&topk_rows_wx<8>);
            case 16: return reinterpret_cast<const void *>(&topk_rows_wx<16>);
            case 32: return reinterpret_cast<const void *>(&topk_rows_wx<32>);
            case 64: return reinterpret_cast<const void *>(&topk_rows_wx<64>);
            case 128: return reinterpret_cast<const void *>(&topk_rows_wx<128>);
            default: return nullptr;
        }
    }
    if (kind == kTopkWave) {
        if (ret_val) return dtype == 0 ? pick_wave<Bf16Key, true>(ept) : pick_wave<F32Key, true>(ept);
        return dtype == 0 ? pick_wave<Bf16Key, false>(ept) : pick_wave<F32Key, false>(ept);
    }
    const bool split = kind == kTopkSplit;
    if (dtype == 0) return split ? pick<Bf16Key, true>(ept) : pick<Bf16Key, false>(ept);
    return split ? pick<F32Key, true>(ept) : pick<F32Key, false>(ept);
}

// The histogram, and the candidate list: cap entries plus one spare per
// lane (one word per bf16 entry, two per fp32 entry), from list_base.
int wave_kernel_waves(int kind, int gather) {
    return kind == kTopkWave && gather ? kGatherWaves : NWAVE;
}

size_t topk_dyn_lds(int dtype, int64_t cap, int ept, int kind, int64_t gather_k) {
    (void)ept;
    if (kind == kTopkWhole && gather_k > 0) {  // the fused gather stages k positions and k offsets
        const size_t sel = topk_dyn_lds(dtype, cap, ept, kind, 0);
        return sel > (size_t)gather_k * 8u ? sel : (size_t)gather_k * 8u;
    }
    if (kind == kTopkWave)  // (the fused gather: k offsets past the waves' regions)
        return ((size_t)(gather_k > 0 ? kGatherWaves : NWAVE) *
                    (dtype == 0 ? wave_lds_words<Bf16Key>() : wave_lds_words<F32Key>()) +
                (size_t)gather_k) * 4;
    const uint64_t hist = (uint64_t)(kBins + 64);
    if (kind == kTopkSplitWx)  // the histogram, the list with a spare entry per lane, group sums
        return (size_t)(kWxBins + 64 + 2 * ((uint64_t)cap + 64) + 256) * 4;
    const uint64_t base = kind == kTopkSplit ? split_list_base()
                          : dtype == 0      ? list_base<Bf16Key>()
                                            : list_base<F32Key>();
    const uint64_t words = base + (dtype == 0 ? 1u : 2u) * (uint64_t)(cap + 64);
    return (size_t)(words > hist ? words : hist) * 4;
}

uint32_t wave_hist_words(int dtype) {
    return dtype == 0 ? wave_lds_words<Bf16Key>() : wave_lds_words<F32Key>();
}

uint32_t wave_stage_words(int dtype, int64_t k, int idx_bytes, int ret_val, int per_cu) {
    constexpr uint64_t kLdsPerCu = 160u * 1024u, kLdsPerWg = 64u * 1024u;
    const uint32_t base = wave_hist_words(dtype);
    // bf16 rows stage indices and values one after the other in the
    // histogram's first W16_BINS words when each fits there
    if (dtype == 0 && (uint64_t)k * (uint64_t)idx_bytes <= (uint64_t)W16_BINS * 4u &&
        (!ret_val || (uint64_t)k * 2u <= (uint64_t)W16_BINS * 4u))
        return 0;
    const uint64_t stage = (((uint64_t)k * (uint64_t)idx_bytes + 15u) & ~(uint64_t)15u) +
                           (ret_val ? (uint64_t)k * (dtype == 0 ? 2u : 4u) : 0u);
    const uint64_t words = (stage + 15u) / 16u * 4u;  // whole 16-byte units: every stage stays aligned
    if (words <= base) return 0;  // fits the histogram's space
    const uint64_t wg = (uint64_t)NWAVE * (base + words) * 4u;
    if (wg > kLdsPerWg || (uint64_t)(per_cu > 0 ? per_cu : 1) * wg > kLdsPerCu) return 0;
    return (uint32_t)words;
}

hipError_t launch_topk(int dtype, int ept, int kind, const TopkArgs &a, unsigned grid,
                       hipStream_t stream) {
    const int gather = a.fg.n > 0 ? 1 : 0;
    const void *fn = topk_kernel_ptr(dtype, ept, kind, a.ret_val, gather);
    if (!fn) return hipErrorInvalidValue;
    TopkArgs copy = a;
    size_t lds = topk_dyn_lds(dtype, a.cap, ept, kind, gather ? a.k : 0);
    const int waves = wave_kernel_waves(kind, gather);
    if (kind == kTopkWave)
        lds = ((size_t)waves * (wave_hist_words(dtype) + copy.stage_words) + (gather ? (size_t)a.k : 0u)) * 4u;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(waves * 64), args, lds, stream);
}

// LDS bytes of a value-order launch: k pair words (rounded up to even), the
// 16-bit counters, the wave totals, minima and maxima.
static size_t value_sort_lds(int64_t k) {
    return (size_t)((k + 1) & ~(int64_t)1) * sizeof(uint64_t) + SORT_CNT * sizeof(uint16_t) +
           3 * SORT_NW * sizeof(uint32_t);
}

namespace {
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *p, int64_t words) {
    const int64_t step = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += step) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_words(uint32_t *p, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    const int64_t blocks = (words + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
    void *args[] = {&p, &words};
    return hipLaunchKernel(reinterpret_cast<const void *>(&zero_words_kernel), dim3(grid),
                           dim3(256), args, 0, stream);
}

hipError_t launch_value_sort(int dtype, const TopkArgs &a, unsigned grid, hipStream_t stream) {
    if (a.k < 1 || a.k > (int64_t)SORT_MAXB * SORT_NT) return hipErrorInvalidValue;
    const void *fn = dtype == 0 ? reinterpret_cast<const void *>(&sort_rows_by_value<Bf16Key>)
                                : reinterpret_cast<const void *>(&sort_rows_by_value<F32Key>);
    TopkArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(SORT_NT), args, value_sort_lds(a.k), stream);
}

}  // namespace dsel

#ifdef DSEL_PHASE_STAMPS
// The instrumented build's stamps: copy out (host buffer of
// kStampUnits * kStampsPerUnit words) and clear.
extern "C" int dsel_stamps_read(unsigned long long *host) {
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(dsel::g_stamps), sizeof(dsel::g_stamps));
}
extern "C" int dsel_stamps_clear() {
    static unsigned long long zero[dsel::kStampUnits * dsel::kStampsPerUnit];
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(dsel::g_stamps), zero, sizeof(zero));
}
#endif
