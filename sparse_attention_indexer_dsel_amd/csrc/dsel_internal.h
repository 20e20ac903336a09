// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsel {

// Workgroup shape of every top-k kernel: four wave64s.
constexpr int kTopkThreads = 256;
// Largest per-thread element count of a whole row (one workgroup per row)
// and of one split-row chunk; a workgroup holds kTopkThreads times that many
// columns in VGPRs.
constexpr int kMaxEpt = 64;
constexpr int kMaxSplitEpt = 128;
constexpr int64_t kBlockCapacity = (int64_t)kTopkThreads * kMaxEpt;
constexpr int64_t kChunkCapacity = (int64_t)kTopkThreads * kMaxSplitEpt;
// First-pass digit width: 2048 histogram bins in LDS.
constexpr int kBins = 2048;
// Workspace header (32-bit words) ahead of the per-row rendezvous slots;
// word 0 carries sticky error bits.
constexpr int kHeaderWords = 64;
constexpr int kSlotHeadWords = 16;
constexpr int kMaxPasses = 3;
// Most workgroups one row may be split over.
constexpr int kMaxSplit = 1024;

// Bins of the last radix pass: 5 bits for bf16 keys, 10 for fp32.
inline int last_pass_bins(int dtype) { return dtype == 0 ? 32 : 1024; }

// One-exchange split rows (bf16 keys, at most kOneMaxSplit workgroups per
// row): each workgroup publishes a header word and the suffix counts of its
// keys over the kOneKeys keys (16 first-digit bins of 32 keys) from the
// floor of its own top-k bin, in its own area of an exchange region that
// follows the workspace header.  The region has one area per workgroup the
// GPU can hold (kOneWgPerCu per compute unit), lies at the same place for
// every call and every slot layout, and is never cleared: a reader uses
// only words the header says were written by this call.  The row slots
// (counters, histograms) follow it.
// Area layout (words): the 16 counts at bin boundaries (the 128-byte line
// every reader fetches first), the header, then the 512 counts; padded to
// whole 128-byte lines.
constexpr int kOneKeys = 512;
constexpr int kOneHdr = 16;
constexpr int kOneFine = 32;
constexpr int kOneWords = kOneFine + kOneKeys;
constexpr int kOneMaxSplit = 64;
constexpr int kOneWgPerCu = 8;
inline int64_t one_region_words(int cus) { return (int64_t)kOneWgPerCu * cus * kOneWords; }
// ... and at most this many columns per thread (wider chunks would spill the
// exchange's registers).
constexpr int kOneMaxEpt = 64;

// Window exchange of split fp32 rows (at most kOneMaxSplit workgroups per
// row, one rendezvous): each workgroup's area in the same exchange region
// holds a header and the keys of a three-bin window of a 12-bit first digit
// around its estimate of the row's boundary bin, each bin at a fixed place
// (kWxBinCap keys a bin).  Like the
// bf16 areas it is never cleared: a reader uses only words the header says
// this call wrote.  A launch uses it only when its workgroups' areas fit the
// region.
constexpr int kWxBins = 4096;              // first digit: key >> 20
constexpr int kWxHdr = 16;                 // header words
constexpr int kWxKeys = 1024;              // window keys one workgroup may publish
constexpr int kWxBinCap = kWxKeys / 3;     // ... of each of the window's three bins
constexpr int kWxWords = kWxHdr + kWxKeys;
constexpr int kWxGather = 2048;            // boundary-bin keys of a row a workgroup may gather

// Per-row workspace slot (32-bit words): counters, one histogram per radix
// pass, per-workgroup counts, and each workgroup's suffix counts over the
// last pass's bins.
inline int64_t slot_words(int G, int dtype) {
    return kSlotHeadWords + (int64_t)kMaxPasses * kBins + 4 * (int64_t)G +
           (int64_t)G * (last_pass_bins(dtype) + 1);
}

// Gather of key rows fused into the top-k (dsel_topk_gather): after a row's
// select, the workers that selected it copy out_g[row, j, :] = key_g[b, p, :]
// for its k slots (b = row / rows_per_batch, p the slot's position).
constexpr int kMaxGatherKeys = 4;
// Waves per workgroup of the one-wave rows' kernel that fuses the gather.
constexpr int kGatherWaves = 8;
struct GatherKeyArgs {
    const char *key;
    char *out;                 // contiguous [rows, k, row bytes]
    int64_t batch_bytes;       // key strides in bytes
    int64_t row_bytes;
    int64_t len;               // key rows per batch
    int vecs;                  // 16-byte vectors per key row
    int vecs_log2;             // log2(vecs) when a power of two, else -1
};
struct FusedGather {
    int n;                     // keys (0: no gather)
    int pad_zero;              // positions outside [0, len): zero rows (else clamped)
    int64_t rows_per_batch;
    GatherKeyArgs k[kMaxGatherKeys];
};

struct TopkArgs {
    const void *x;
    int64_t rows;
    int64_t cols;
    int64_t x_stride;        // elements
    const int32_t *row_end;  // nullable
    void *out_idx;
    int64_t idx_stride;      // elements of the index type
    void *out_val;
    int64_t val_stride;      // elements of the value type
    uint8_t *nan_flag;       // nullable
    uint32_t *ws;            // workspace base (split rows only)
    int64_t row0;            // first row of this launch
    int64_t chunk;           // columns per workgroup (split rows only)
    int64_t slot_words;      // 32-bit words per row slot (split rows only)
    int64_t slot0;           // word offset of the first row slot (split rows only)
    int64_t cap;             // capacity of a workgroup's candidate list (entries)
    int k;
    int G;                   // workgroups per row
    int idx64;
    int ret_val;
    int one;                 // split bf16 rows: try the one-exchange select first
    int64_t idx_fill;        // index of the slots past a short row's length
    uint32_t val_fill;       // value bits of those slots
    uint32_t stage_words;    // one-wave rows: LDS words per wave for the staged output
                             // after the histograms (0: staged in the histogram's space)
    uint32_t spin_limit;     // split rows: polls of a rendezvous before it gives up
    int row_order;           // kRowsNatural or kRowsDualChunk (rows of one workgroup or wave)
    FusedGather fg;          // the fused gather's keys (instances that gather only)
};

// Order in which the workgroups (one-wave rows: the waves) of a launch take
// rows.  Dual chunk (PaddleFleet PR #1762, Description: the dual-chunk
// causal split): the t-th taker gets row t/2 for even t and row R-1-t/2 for
// odd t, so neighbouring takers pair a row from the front with its mirror
// from the back, and takers started early hold rows from both ends of a
// causal (or anti-causal) ramp of lengths.  A permutation of [0, R): the
// outputs are the same bytes in either order.
enum { kRowsNatural = 0, kRowsDualChunk = 1 };

__host__ __device__ inline int64_t taker_row(int order, int64_t t, int64_t R) {
    return order == kRowsDualChunk ? ((t & 1) ? R - 1 - (t >> 1) : (t >> 1)) : t;
}

// Polls of a split-row rendezvous before it gives up and records an error
// (about 0.1 s at the s_sleep granularity).
constexpr uint32_t kSpinLimit = 1u << 22;

// Sticky error bits in workspace word 0.
constexpr uint32_t kErrRendezvous = 1u;  // a split row's workgroups did not all meet

// Top-k kernel kinds: one workgroup per row, G workgroups per row, one wave
// per row, G workgroups per fp32 row through the window exchange.
enum { kTopkWhole = 0, kTopkSplit = 1, kTopkWave = 2, kTopkSplitWx = 3 };
// Rows of at most this many columns take one wave each.
constexpr int64_t kWaveCapacity = 64 * 32;

// Kernel instance for (dtype, elements per thread, kind, values returned,
// gather fused: one-wave bf16 rows and whole rows only); nullptr if none.  The two one-wave instances of a (dtype, ept) pair have
// the same occupancy.
const void *topk_kernel_ptr(int dtype, int ept, int kind, int ret_val = 0, int gather = 0);
// Elements per 16-byte vector for a dtype.
inline int topk_vec(int dtype) { return dtype == 0 ? 8 : 4; }
// Dynamic LDS bytes of a top-k launch with candidate capacity `cap` (for
// one-wave rows: with each wave's histogram only; gather_k > 0: whole rows
// that fuse the gather also stage that many positions).
size_t topk_dyn_lds(int dtype, int64_t cap, int ept, int kind, int64_t gather_k = 0);
// Waves per workgroup of a top-k launch (kTopkThreads / 64, or kGatherWaves
// for one-wave rows that fuse the gather).
int wave_kernel_waves(int kind, int gather);
// One-wave rows: LDS words of a wave's histogram, and the LDS words per wave
// of a separate stage for the row's output (k indices of idx_bytes each, and
// k values when ret_val) when it does not fit the histogram's space and
// `per_cu` workgroups with it still fit a compute unit; else 0.
uint32_t wave_hist_words(int dtype);
uint32_t wave_stage_words(int dtype, int64_t k, int idx_bytes, int ret_val, int per_cu);
hipError_t launch_topk(int dtype, int ept, int kind, const TopkArgs &a, unsigned grid,
                       hipStream_t stream);
// Value order of the top-k outputs of rows [a.row0, a.row0 + grid), in place.
hipError_t launch_value_sort(int dtype, const TopkArgs &a, unsigned grid, hipStream_t stream);

struct GatherArgs {
    const char *key;
    char *out;
    const void *pos;
    int64_t batch, len, R, P;
    int64_t key_batch_bytes, key_row_bytes;
    int64_t pos_row_stride;  // elements
    int row_vecs;            // 16-byte vectors per key row
    int row_vecs_log2;       // log2(row_vecs) when a power of two, else -1
    int pad_zero;            // positions outside [0, len): zero rows (else clamped)
};

hipError_t launch_gather(int pos64, const GatherArgs &a, hipStream_t stream);

// Zero `words` 32-bit words at `p` (a fill kernel: no memset node in a
// captured graph).
hipError_t launch_zero_words(uint32_t *p, int64_t words, hipStream_t stream);

}  // namespace dsel
