// C ABI of the selection library: argument checks, path planning, workspace
// sizing and launches on the caller's stream.  No allocation, no sync.
#include <atomic>
#include <cstdlib>
#include <mutex>

#include "../../include/dsel.h"
#include "dsel_internal.h"

namespace dsel {
namespace {

constexpr int64_t kAlign = 16;
constexpr int kMaxDevices = 64;

std::atomic<int> g_cu_count[kMaxDevices];

// Compute-unit count of the current device (cached per device), or -1.
int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    int cus = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cus > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return -1;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

bool aligned_ptr(const void *p) { return ((uintptr_t)p % kAlign) == 0; }

// Polls of a split-row rendezvous before it gives up.  DSEL_SPIN_LIMIT
// overrides it (tests force a rendezvous to give up from the host).
uint32_t spin_limit() {
    if (const char *env = std::getenv("DSEL_SPIN_LIMIT")) {
        const long v = std::strtol(env, nullptr, 10);
        if (v >= 1) return (uint32_t)(v < (long)kSpinLimit ? v : (long)kSpinLimit);
    }
    return kSpinLimit;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct TopkPlan {
    int kind = kTopkWhole;
    bool split = false;
    int G = 1;
    int ept = 0;
    int64_t chunk = 0;
    int64_t cap = 0;
    int64_t rows_per_launch = 0;
    int64_t grid = 0;  // workgroups per launch
    int64_t slot_words = 0;
    int64_t slot0 = 0;
    size_t ws_bytes = 0;
    bool one = false;  // split bf16 rows try the one-exchange select
    int per_cu = 0;    // one-wave rows: resident workgroups per CU the grid assumes
    bool fused = false;  // a gather was asked for and the plan's kernel fuses it
};

// Candidate-list capacity: k plus room for the boundary bin of the first
// digit (a quarter octave of values), at most 8192 entries and never more
// than the row; a row whose candidates exceed it takes the slower path that
// re-reads the row for each later radix pass.
int64_t candidate_cap(int64_t k, int64_t row_len) {
    int64_t cap = k + (k > 1536 ? k : 1536);
    if (cap > 8192) cap = 8192;
    if (row_len < cap) cap = row_len;
    return (cap + 255) / 256 * 256;
}

// A split row's workgroup lists only its own chunk's candidates: room for
// twice an even share of the row's, plus 512, and never more than the chunk
// or the whole-row capacity.  A workgroup holding more (ties, or values that
// crowd into one chunk) takes the slower path.
int64_t chunk_cap(int64_t k, int64_t cols, int64_t chunk, int G) {
    const int64_t row_cap = candidate_cap(k, cols);
    int64_t cap = 2 * row_cap / G + 512;
    if (cap > row_cap) cap = row_cap;
    if (cap > chunk) cap = chunk;
    return (cap + 255) / 256 * 256;
}

// Smallest instantiated per-thread element count covering `cols` columns
// with one workgroup (up to `max_ept`).
int pick_ept(int64_t cols, int max_ept) {
    for (int e = 8; e <= max_ept; e *= 2)
        if ((int64_t)kTopkThreads * e >= cols) return e;
    return 0;
}

// Workgroups per row: one when the row fits a workgroup (a split row pays a
// cross-workgroup rendezvous per radix pass, a few microseconds each, more
// than one workgroup takes over a row it can hold); otherwise enough to give
// the GPU about four workgroups per compute unit, but no fewer than 8192
// columns each (more workgroups per row contend on the row's histogram
// atomics), and at least enough to hold the row in VGPRs.
// DSEL_BLOCKS_PER_ROW overrides the choice (tuning and tests).
int choose_G(int64_t rows, int64_t cols, int cus) {
    const int64_t gmin = cdiv(cols, kChunkCapacity);
    int64_t G;
    if (cols <= kBlockCapacity) {
        G = 1;
    } else {
        const int64_t gpar = cdiv(4 * (int64_t)cus, rows > 0 ? rows : 1);
        const int64_t gchunk = cdiv(cols, 8192);
        G = gpar < gchunk ? gpar : gchunk;
        if (G < gmin) G = gmin;
        if (G < 1) G = 1;
    }
    if (const char *env = std::getenv("DSEL_BLOCKS_PER_ROW")) {
        const long v = std::strtol(env, nullptr, 10);
        if (v >= 1) G = v < gmin ? gmin : v;
    }
    if (G > kMaxSplit && gmin <= kMaxSplit) G = kMaxSplit;
    return (int)G;
}

// max_ws_words > 0 caps the split layout (rows per launch) to that many
// workspace words (the entry point that allocates nothing).
// gather: plan for the fused gather's kernel where the row kind has one
// (one-wave bf16 rows, whole rows); pl->fused says whether it does.
int plan_topk(int dtype, int64_t rows, int64_t cols, int64_t k, int ret_val, int64_t max_ws_words,
              TopkPlan *pl, bool gather = false) {
    const int cus = cu_count();
    if (cus <= 0) return DSEL_ERR_DEVICE;
    const int vec = topk_vec(dtype);
    int G = choose_G(rows, cols, cus);
    int64_t chunk = cols;
    if (G > 1) {
        chunk = cdiv(cdiv(cols, G), vec) * vec;
        G = (int)cdiv(cols, chunk);  // rounding may leave fewer workgroups
    }
    if (G > kMaxSplit) return DSEL_ERR_ARG;  // row longer than the split limit holds
    if (cols <= kWaveCapacity) {
        // one wave per row; workgroups of four waves walk the rows, as many
        // as the GPU holds at once
        pl->kind = kTopkWave;
        pl->split = false;
        pl->G = 1;
        pl->ept = 8;
        while ((int64_t)64 * pl->ept < cols) pl->ept *= 2;  // columns per lane
        pl->chunk = cols;
        pl->cap = 0;
        int per_cu = 0;
        pl->fused = gather && dtype == DSEL_BF16 && !ret_val;
        const int waves = wave_kernel_waves(kTopkWave, pl->fused ? 1 : 0);
        // (the instance the call launches: the values instance may differ)
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, topk_kernel_ptr(dtype, pl->ept, kTopkWave, ret_val, pl->fused ? 1 : 0),
                waves * 64, topk_dyn_lds(dtype, 0, pl->ept, kTopkWave, pl->fused ? k : 0)) != hipSuccess ||
            per_cu <= 0)
            return DSEL_ERR_DEVICE;
        pl->per_cu = per_cu;
        const int64_t slots = (int64_t)per_cu * cus;
        const int64_t wgs = cdiv(rows, waves);
        pl->rows_per_launch = rows;
        pl->grid = wgs < slots ? wgs : slots;
        pl->ws_bytes = 0;
        return DSEL_OK;
    }
    if (G <= 1 && cols <= kBlockCapacity) {
        // one workgroup per row: as many as the GPU holds at once, each
        // walking rows
        pl->kind = kTopkWhole;
        pl->split = false;
        pl->G = 1;
        pl->ept = pick_ept(cols, kMaxEpt);
        if (!pl->ept) return DSEL_ERR_ARG;
        pl->chunk = cols;
        pl->cap = candidate_cap(k, cols);
        pl->fused = gather && !ret_val;
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, topk_kernel_ptr(dtype, pl->ept, kTopkWhole, 0, pl->fused ? 1 : 0),
                kTopkThreads,
                topk_dyn_lds(dtype, pl->cap, pl->ept, kTopkWhole, pl->fused ? k : 0)) != hipSuccess ||
            per_cu <= 0)
            return DSEL_ERR_DEVICE;
        const int64_t slots = (int64_t)per_cu * cus;
        pl->rows_per_launch = rows;
        pl->grid = rows < slots ? rows : slots;
        pl->ws_bytes = 0;
        return DSEL_OK;
    }
    const int ept = pick_ept(chunk, kMaxSplitEpt);
    if (!ept) return DSEL_ERR_ARG;
    int64_t cap = chunk_cap(k, cols, chunk, G);
    // One exchange (bf16, at most kOneMaxSplit workgroups per row): a
    // workgroup lists every key from the floor of its own top-k bin, about k
    // plus one bin, so its list needs the whole-row capacity.
    // DSEL_SPLIT_ONE_EXCHANGE=0 turns it off (tests of the multi-pass path).
    // (fp32 rows: the window exchange, under the same switch)
    bool one = G <= kOneMaxSplit && (dtype != DSEL_BF16 || ept <= kOneMaxEpt);
    if (const char *env = std::getenv("DSEL_SPLIT_ONE_EXCHANGE"))
        if (std::strtol(env, nullptr, 10) == 0) one = false;
    if (one && dtype == DSEL_BF16) {
        const int64_t own = candidate_cap(k, chunk);
        if (own > cap) cap = own;
    }
    // every workgroup of a row must be resident at once: size launches by
    // the number of workgroups the GPU holds.  fp32 rows take the window
    // exchange's kernel when its areas fit the exchange region, else the
    // multi-pass kernel.
    const int64_t slot0 = kHeaderWords + one_region_words(cus);
    const int64_t sw = slot_words(G, dtype);
    int kind = (dtype == DSEL_F32 && one) ? kTopkSplitWx : kTopkSplit;
    int64_t rpl = 0;
    for (;;) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, topk_kernel_ptr(dtype, ept, kind),
                                                         kTopkThreads,
                                                         topk_dyn_lds(dtype, cap, ept, kind)) !=
                hipSuccess ||
            per_cu <= 0)
            return DSEL_ERR_DEVICE;
        const int64_t capacity = (int64_t)per_cu * cus;
        if (G > capacity) return DSEL_ERR_ARG;  // row longer than the GPU holds on chip
        rpl = capacity / G;
        if (rpl > rows) rpl = rows;
        if (max_ws_words > 0) {
            const int64_t fit = max_ws_words > slot0 ? (max_ws_words - slot0) / sw : 0;
            if (fit < 1) return DSEL_ERR_WORKSPACE;
            if (rpl > fit) rpl = fit;
        }
        if (kind == kTopkSplitWx && rpl * G * kWxWords > one_region_words(cus)) {
            kind = kTopkSplit;  // the areas do not fit: plan the multi-pass kernel
            one = false;
            continue;
        }
        break;
    }
    pl->kind = kind;
    pl->split = true;
    pl->G = G;
    pl->ept = ept;
    pl->chunk = chunk;
    pl->cap = cap;
    pl->rows_per_launch = rpl;
    pl->grid = rpl * G;
    // the exchange region is part of every split layout (so no slot of any
    // layout ever overlaps it) and holds one area per resident workgroup
    pl->one = one && rpl * G * (dtype == DSEL_BF16 ? kOneWords : kWxWords) <= one_region_words(cus);
    pl->slot_words = sw;
    pl->slot0 = slot0;
    pl->ws_bytes = (size_t)(pl->slot0 + rpl * pl->slot_words) * sizeof(uint32_t);
    return DSEL_OK;
}

}  // namespace
}  // namespace dsel

using namespace dsel;

extern "C" int dsel_stride_requirement(int64_t *in_align_bytes, int64_t *out_align_bytes) {
    if (!in_align_bytes || !out_align_bytes) return DSEL_ERR_ARG;
    *in_align_bytes = kAlign;
    *out_align_bytes = kAlign;
    return DSEL_OK;
}

extern "C" int dsel_topk(const void *x, int dtype, int64_t rows, int64_t cols,
                         int64_t x_row_stride, int64_t k, const int32_t *row_end,
                         int sorted_index, int indices_type, int return_value, void *out_idx,
                         int64_t idx_row_stride, void *out_val, int64_t val_row_stride,
                         uint8_t *nan_flag, void *workspace, size_t *workspace_bytes,
                         void *stream) {
    return dsel_topk_ex(x, dtype, rows, cols, x_row_stride, k, row_end, sorted_index,
                        indices_type, return_value, out_idx, idx_row_stride, out_val,
                        val_row_stride, nan_flag, workspace, workspace_bytes, stream, -1,
                        dtype == DSEL_BF16 ? 0xFF80u : 0xFF800000u, DSEL_ROWS_AUTO);
}

namespace {

// dsel_topk_ex, with the split layout capped at max_ws_words (0: no cap).
int topk_entry(const void *x, int dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
               int64_t k, const int32_t *row_end, int sorted_index, int indices_type,
               int return_value, void *out_idx, int64_t idx_row_stride, void *out_val,
               int64_t val_row_stride, uint8_t *nan_flag, void *workspace,
               size_t *workspace_bytes, void *stream, int64_t idx_fill, uint32_t val_fill_bits,
               int row_order, int64_t max_ws_words, const FusedGather *fg = nullptr) {
    // sorted_index 0 and 1: the output is ascending by construction; 2: a
    // value-order pass follows the select
    if (sorted_index < 0 || sorted_index > 2) return DSEL_ERR_ARG;
    if (dtype != DSEL_BF16 && dtype != DSEL_F32) return DSEL_ERR_ARG;
    if (indices_type != DSEL_I32 && indices_type != DSEL_I64) return DSEL_ERR_ARG;
    if (indices_type == DSEL_I32 && (idx_fill < INT32_MIN || idx_fill > INT32_MAX))
        return DSEL_ERR_ARG;
    if (dtype == DSEL_BF16 && val_fill_bits > 0xFFFFu) return DSEL_ERR_ARG;
    if (row_order < DSEL_ROWS_AUTO || row_order > DSEL_ROWS_DUAL_CHUNK) return DSEL_ERR_ARG;
    if (rows < 0 || cols < 1) return DSEL_ERR_ARG;
    if (k < 1 || k > 4096) return DSEL_ERR_K;
    if (!workspace_bytes) return DSEL_ERR_ARG;
    if (rows == 0) {
        if (!workspace) *workspace_bytes = 0;
        return DSEL_OK;
    }
    if (!x || !out_idx || (return_value && !out_val)) return DSEL_ERR_ARG;
    if (x_row_stride < cols || idx_row_stride < k || (return_value && val_row_stride < k))
        return DSEL_ERR_ARG;
    if (indices_type == DSEL_I32 && cols > INT32_MAX) return DSEL_ERR_ARG;
    const int64_t esz = dtype == DSEL_BF16 ? 2 : 4;
    const int64_t isz = indices_type == DSEL_I32 ? 4 : 8;
    if (!aligned_ptr(x) || (x_row_stride * esz) % kAlign || !aligned_ptr(out_idx) ||
        (idx_row_stride * isz) % kAlign)
        return DSEL_ERR_ALIGN;
    if (return_value && (!aligned_ptr(out_val) || (val_row_stride * esz) % kAlign))
        return DSEL_ERR_ALIGN;

    TopkPlan pl;
    // (value order sorts after the select: its gather runs after the sort;
    // the fused copy addresses a key's batch with 32-bit offsets)
    bool fuse = fg != nullptr && sorted_index != 2;
    for (int g = 0; fuse && g < fg->n; ++g) {
        const GatherKeyArgs &kg = fg->k[g];
        if ((kg.len - 1) * kg.row_bytes + (int64_t)kg.vecs * 16 >= ((int64_t)1 << 31) - 16) fuse = false;
    }
    const int st = plan_topk(dtype, rows, cols, k, return_value ? 1 : 0, max_ws_words, &pl, fuse);
    if (st != DSEL_OK) return st;
    if (!workspace) {
        *workspace_bytes = pl.ws_bytes;
        return DSEL_OK;
    }
    if (*workspace_bytes < pl.ws_bytes) return DSEL_ERR_WORKSPACE;
    if (pl.split && !aligned_ptr(workspace)) return DSEL_ERR_ALIGN;

    TopkArgs a{};
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.x_stride = x_row_stride;
    a.row_end = row_end;
    a.out_idx = out_idx;
    a.idx_stride = idx_row_stride;
    a.out_val = return_value ? out_val : nullptr;
    a.val_stride = val_row_stride;
    a.nan_flag = nan_flag;
    a.ws = reinterpret_cast<uint32_t *>(workspace);
    a.chunk = pl.chunk;
    a.slot_words = pl.slot_words;
    a.slot0 = pl.slot0;
    a.cap = pl.cap;
    a.k = (int)k;
    a.G = pl.G;
    a.idx64 = indices_type == DSEL_I64;
    a.ret_val = return_value ? 1 : 0;
    a.one = pl.one ? 1 : 0;
    a.idx_fill = idx_fill;
    a.val_fill = val_fill_bits;
    a.spin_limit = spin_limit();
    // rows of ragged length take the dual-chunk order unless told otherwise
    a.row_order = row_order == DSEL_ROWS_DUAL_CHUNK || (row_order == DSEL_ROWS_AUTO && row_end)
                      ? kRowsDualChunk
                      : kRowsNatural;
    // (only the values instance of the one-wave kernel reads a separate stage)
    a.stage_words = pl.kind == kTopkWave && a.ret_val
                        ? wave_stage_words(dtype, k, a.idx64 ? 8 : 4, a.ret_val, pl.per_cu)
                        : 0u;
    if (fg && pl.fused) a.fg = *fg;  // the select's kernel also gathers
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int64_t r0 = 0; r0 < rows; r0 += pl.rows_per_launch) {
        const int64_t nr = (rows - r0) < pl.rows_per_launch ? (rows - r0) : pl.rows_per_launch;
        a.row0 = r0;
        const int64_t grid = pl.split ? nr * pl.G : pl.grid;
        if (grid > INT32_MAX) return DSEL_ERR_ARG;
        if (launch_topk(dtype, pl.ept, pl.kind, a, (unsigned)grid, s) != hipSuccess)
            return DSEL_ERR_DEVICE;
    }
    if (sorted_index == 2) {
        // one workgroup per row, in launches of at most 2^30 rows
        constexpr int64_t kMaxGrid = (int64_t)1 << 30;
        for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid) {
            a.row0 = r0;
            const int64_t nr = (rows - r0) < kMaxGrid ? (rows - r0) : kMaxGrid;
            if (launch_value_sort(dtype, a, (unsigned)nr, s) != hipSuccess) return DSEL_ERR_DEVICE;
        }
    }
    if (fg && !pl.fused) {
        // rows whose kernel does not fuse the gather: the gather kernel on
        // the indices just written, one launch per key
        for (int g = 0; g < fg->n; ++g) {
            const GatherKeyArgs &kg = fg->k[g];
            GatherArgs ga{};
            ga.key = kg.key;
            ga.out = kg.out;
            ga.pos = out_idx;
            ga.batch = rows / fg->rows_per_batch;
            ga.len = kg.len;
            ga.R = fg->rows_per_batch;
            ga.P = k;
            ga.key_batch_bytes = kg.batch_bytes;
            ga.key_row_bytes = kg.row_bytes;
            ga.pos_row_stride = idx_row_stride;
            ga.row_vecs = kg.vecs;
            ga.row_vecs_log2 = kg.vecs_log2;
            ga.pad_zero = fg->pad_zero;
            if (launch_gather(indices_type == DSEL_I64, ga, s) != hipSuccess) return DSEL_ERR_DEVICE;
        }
    }
    return DSEL_OK;
}

// ---- the scratch of dsel_topk_noalloc ----------------------------------
// Split rows need device scratch (rendezvous counters, histograms, the
// exchange region).  dsel_topk_noalloc takes it from this array instead of
// a caller's workspace: each GPU the library runs on holds its own copy for
// the life of the process.  In host code `scratch` names a host-side stand-in
// only; the device address comes from hipGetSymbolAddress, once per device.
constexpr int64_t kScratchWords = (int64_t)8 << 20;  // 32 MiB
__device__ __align__(256) uint32_t scratch[kScratchWords];

std::mutex g_scratch_mu;
uint32_t *g_scratch[kMaxDevices];
std::atomic<bool> g_scratch_any{false};

// The current device's address of `scratch`, zero-filled on first use (on
// `s`, waited for unless `s` is being captured: then the fill is part of the
// graph), or nullptr on failure.
uint32_t *device_scratch(hipStream_t s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev]) return g_scratch[dev];
    uint32_t *ptr = nullptr;
    if (hipGetSymbolAddress(reinterpret_cast<void **>(&ptr), HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
        return nullptr;
    if (launch_zero_words(ptr, kScratchWords, s) != hipSuccess) return nullptr;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return nullptr;
    if (cap == hipStreamCaptureStatusNone && hipStreamSynchronize(s) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
    g_scratch_any.store(true);
    return ptr;
}

// The scratch of the current device if dsel_topk_noalloc has set it up there.
uint32_t *known_scratch() {
    if (!g_scratch_any.load()) return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch[dev];
}

}  // namespace

extern "C" int dsel_topk_noalloc(const void *x, int dtype, int64_t rows, int64_t cols,
                                 int64_t x_row_stride, int64_t k, const int32_t *row_end,
                                 int sorted_index, int indices_type, int return_value,
                                 void *out_idx, int64_t idx_row_stride, void *out_val,
                                 int64_t val_row_stride, uint8_t *nan_flag, void *stream,
                                 int64_t idx_fill, uint32_t val_fill_bits, int row_order) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    size_t bytes = (size_t)kScratchWords * sizeof(uint32_t);
    // argument checks and the plan first (nothing launched on an error)
    size_t need = 0;
    int st = topk_entry(x, dtype, rows, cols, x_row_stride, k, row_end, sorted_index,
                        indices_type, return_value, out_idx, idx_row_stride, out_val,
                        val_row_stride, nan_flag, nullptr, &need, stream, idx_fill,
                        val_fill_bits, row_order, kScratchWords);
    if (st != DSEL_OK || rows == 0) return st;
    uint32_t *ws = nullptr;
    if (need > 0) {  // split rows: the scratch
        ws = device_scratch(s);
        if (!ws) return DSEL_ERR_DEVICE;
    }
    // (a plan without split rows uses no workspace: any non-null pointer
    // with a size of 0 passes the workspace checks)
    return topk_entry(x, dtype, rows, cols, x_row_stride, k, row_end, sorted_index, indices_type,
                      return_value, out_idx, idx_row_stride, out_val, val_row_stride, nan_flag,
                      ws ? ws : reinterpret_cast<uint32_t *>(out_idx), ws ? &bytes : &need,
                      stream, idx_fill, val_fill_bits, row_order, kScratchWords);
}

extern "C" int dsel_topk_ex(const void *x, int dtype, int64_t rows, int64_t cols,
                            int64_t x_row_stride, int64_t k, const int32_t *row_end,
                            int sorted_index, int indices_type, int return_value, void *out_idx,
                            int64_t idx_row_stride, void *out_val, int64_t val_row_stride,
                            uint8_t *nan_flag, void *workspace, size_t *workspace_bytes,
                            void *stream, int64_t idx_fill, uint32_t val_fill_bits,
                            int row_order) {
    return topk_entry(x, dtype, rows, cols, x_row_stride, k, row_end, sorted_index, indices_type,
                      return_value, out_idx, idx_row_stride, out_val, val_row_stride, nan_flag,
                      workspace, workspace_bytes, stream, idx_fill, val_fill_bits, row_order, 0);
}

extern "C" int dsel_topk_gather(const void *x, int dtype, int64_t rows, int64_t cols,
                                int64_t x_row_stride, int64_t k, const int32_t *row_end,
                                int sorted_index, int indices_type, void *out_idx,
                                int64_t idx_row_stride, uint8_t *nan_flag, int64_t rows_per_batch,
                                const DselGatherKey *keys, int n_keys, int pad, void *workspace,
                                size_t *workspace_bytes, void *stream) {
    if (!keys || n_keys < 1 || n_keys > kMaxGatherKeys) return DSEL_ERR_ARG;
    if (pad != DSEL_PAD_CLAMP && pad != DSEL_PAD_ZERO) return DSEL_ERR_ARG;
    if (rows_per_batch < 1 || rows < 0 || rows % rows_per_batch != 0) return DSEL_ERR_ARG;
    FusedGather fg{};
    fg.n = n_keys;
    fg.pad_zero = pad == DSEL_PAD_ZERO ? 1 : 0;
    fg.rows_per_batch = rows_per_batch;
    for (int g = 0; g < n_keys; ++g) {
        const DselGatherKey &d = keys[g];
        if (d.dtype != DSEL_BF16 && d.dtype != DSEL_F32) return DSEL_ERR_ARG;
        if (d.len < 1 || d.dim < 1 || d.batch_stride < 0 || d.row_stride < 0) return DSEL_ERR_ARG;
        if (rows > 0 && (!d.key || !d.out)) return DSEL_ERR_ARG;
        const int64_t esz = d.dtype == DSEL_BF16 ? 2 : 4;
        if (!aligned_ptr(d.key) || !aligned_ptr(d.out) || (d.dim * esz) % kAlign ||
            (d.batch_stride * esz) % kAlign || (d.row_stride * esz) % kAlign)
            return DSEL_ERR_ALIGN;
        const int64_t rv = d.dim * esz / 16;
        if (rv > (1 << 20)) return DSEL_ERR_ARG;
        GatherKeyArgs &kg = fg.k[g];
        kg.key = reinterpret_cast<const char *>(d.key);
        kg.out = reinterpret_cast<char *>(d.out);
        kg.batch_bytes = d.batch_stride * esz;
        kg.row_bytes = d.row_stride * esz;
        kg.len = d.len;
        kg.vecs = (int)rv;
        kg.vecs_log2 = -1;
        if ((rv & (rv - 1)) == 0) {
            int l = 0;
            while ((1LL << l) < rv) ++l;
            kg.vecs_log2 = l;
        }
    }
    return topk_entry(x, dtype, rows, cols, x_row_stride, k, row_end, sorted_index, indices_type,
                      0, out_idx, idx_row_stride, nullptr, 0, nan_flag, workspace, workspace_bytes,
                      stream, -1, dtype == DSEL_BF16 ? 0xFF80u : 0xFF800000u, DSEL_ROWS_AUTO, 0,
                      &fg);
}

extern "C" int dsel_topk_check(void *workspace, size_t workspace_bytes, void *stream,
                               uint32_t *error_bits) {
    if (!error_bits) return DSEL_ERR_ARG;
    *error_bits = 0;
    if (!workspace) {
        // the scratch of dsel_topk_noalloc on the current device, if set up
        workspace = known_scratch();
        workspace_bytes = (size_t)kScratchWords * sizeof(uint32_t);
        if (!workspace) return DSEL_OK;
    }
    if (workspace_bytes < sizeof(uint32_t)) return DSEL_OK;  // nothing split ran on it
    if (!aligned_ptr(workspace)) return DSEL_ERR_ALIGN;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t bits = 0;
    if (hipMemcpyAsync(&bits, workspace, sizeof(bits), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return DSEL_ERR_DEVICE;
    if (!bits) return DSEL_OK;
    // a rendezvous gave up: the workgroups of a row did not all meet, so
    // counters and histograms may be left non-zero; zero the whole
    // workspace (the exchange region needs no clearing, but costs nothing)
    if (launch_zero_words(reinterpret_cast<uint32_t *>(workspace),
                          (int64_t)(workspace_bytes / sizeof(uint32_t)), s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return DSEL_ERR_DEVICE;
    *error_bits = bits;
    return DSEL_ERR_SPLIT;
}

extern "C" int dsel_gather_rows(const void *key, int dtype, int64_t batch, int64_t len,
                                int64_t dim, int64_t key_batch_stride, int64_t key_row_stride,
                                const void *pos, int pos_type, int64_t rows_per_batch,
                                int64_t per_row, int64_t pos_row_stride, void *out,
                                void *stream) {
    if (dtype != DSEL_BF16 && dtype != DSEL_F32) return DSEL_ERR_ARG;
    if (pos_type != DSEL_I32 && pos_type != DSEL_I64) return DSEL_ERR_ARG;
    if (batch < 0 || len < 1 || dim < 1 || rows_per_batch < 0 || per_row < 0)
        return DSEL_ERR_ARG;
    if (batch == 0 || rows_per_batch == 0 || per_row == 0) return DSEL_OK;
    if (!key || !pos || !out) return DSEL_ERR_ARG;
    if (pos_row_stride < per_row || key_batch_stride < 0 || key_row_stride < 0)
        return DSEL_ERR_ARG;
    const int64_t esz = dtype == DSEL_BF16 ? 2 : 4;
    const int64_t psz = pos_type == DSEL_I32 ? 4 : 8;
    if (!aligned_ptr(key) || !aligned_ptr(out) || (dim * esz) % kAlign ||
        (key_batch_stride * esz) % kAlign || (key_row_stride * esz) % kAlign ||
        ((uintptr_t)pos % psz) != 0)
        return DSEL_ERR_ALIGN;
    GatherArgs a{};
    a.key = reinterpret_cast<const char *>(key);
    a.out = reinterpret_cast<char *>(out);
    a.pos = pos;
    a.batch = batch;
    a.len = len;
    a.R = rows_per_batch;
    a.P = per_row;
    a.key_batch_bytes = key_batch_stride * esz;
    a.key_row_bytes = key_row_stride * esz;
    a.pos_row_stride = pos_row_stride;
    const int64_t rv = dim * esz / 16;
    if (rv > (1 << 20)) return DSEL_ERR_ARG;
    a.row_vecs = (int)rv;
    a.row_vecs_log2 = -1;
    if ((rv & (rv - 1)) == 0) {
        int l = 0;
        while ((1LL << l) < rv) ++l;
        a.row_vecs_log2 = l;
    }
    if (launch_gather(pos_type == DSEL_I64, a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return DSEL_ERR_DEVICE;
    return DSEL_OK;
}
