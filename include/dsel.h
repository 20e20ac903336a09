/*
 * dsel: row-wise top-k selection and compressed-key gather on MI355X (gfx950).
 *
 * C ABI.  Every pointer is a device pointer unless marked "host".  Every call
 * is asynchronous on the HIP stream passed as `stream` (a hipStream_t; NULL
 * means the legacy default stream); the library never allocates, frees or
 * synchronises, and keeps no state between calls apart from a per-device
 * cache of device attributes.
 *
 * Status codes: every entry point returns DSEL_OK (0) or a negative code.
 * Host-checkable faults return before anything is launched.  Data conditions
 * on the device never fault: NaN is reported through the per-row flag,
 * row ends are clamped to [0, cols] and gather positions to [0, len-1].
 */
#ifndef DSEL_H
#define DSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DSEL_OK = 0,
    DSEL_ERR_ARG = -1,        /* null required pointer, bad enum, negative size, short stride */
    DSEL_ERR_K = -2,          /* k outside [1, 4096] */
    DSEL_ERR_ALIGN = -3,      /* pointer or row stride not a multiple of the alignment */
    DSEL_ERR_WORKSPACE = -4,  /* workspace smaller than the size query returned */
    DSEL_ERR_DEVICE = -5,     /* no usable device, or a launch failed */
    DSEL_ERR_SPLIT = -6       /* dsel_topk_check: a split row's workgroups did not all meet */
};

enum { DSEL_BF16 = 0, DSEL_F32 = 1 };  /* value dtype (bf16 = upper half of binary32) */
enum { DSEL_I32 = 0, DSEL_I64 = 1 };   /* index dtype */

/*
 * Order in which a launch's workers take rows (dsel_topk_ex, dsel_topk_noalloc).
 * It changes timing only: every row's output is the same bytes in any order.
 *
 * PaddleFleet PR #1762, Description: under a causal mask the cost of a query
 * row grows with its position, and the dual-chunk split evens it out by
 * pairing chunk g with its mirror 2G-1-g.  Here the workers (one wave or one
 * workgroup per row) take rows 0, R-1, 1, R-2, 2, ... in launch order, so the
 * workers that start first hold rows from both ends of a ramp of row lengths
 * and the long rows no longer all start last.  Rows split over several
 * workgroups (over 16384 columns) always take the natural order.
 *   DSEL_ROWS_AUTO        dual chunk when row_end is given, else natural
 *   DSEL_ROWS_NATURAL     rows 0, 1, 2, ... in launch order
 *   DSEL_ROWS_DUAL_CHUNK  rows 0, R-1, 1, R-2, ...
 * Anything else: DSEL_ERR_ARG.
 */
enum { DSEL_ROWS_AUTO = 0, DSEL_ROWS_NATURAL = 1, DSEL_ROWS_DUAL_CHUNK = 2 };

/*
 * Byte alignment the library needs of row strides and base pointers.
 *
 * DeepSelect tutorial ("Sheshisa Imisebenzi ye-PyTorch TopK nge-DeepSelect"),
 * section "Ukuphatha Ukuqondaniswa Kwe-Stride": a query returns the input
 * and output row-stride alignments in bytes; an input whose row stride is
 * not a multiple must be padded, and outputs are laid out with row strides
 * aligned to the output figure.
 *
 * in_align_bytes, out_align_bytes: host pointers, both written (16 and 16:
 * one 16-byte vector load or store).  Returns DSEL_ERR_ARG if either is NULL.
 * Needs no device.
 */
int dsel_stride_requirement(int64_t *in_align_bytes, int64_t *out_align_bytes);

/*
 * Row-wise top-k.
 *
 * DeepSelect tutorial, sections "Ukusebenzisa i-TopK Okuyisisekelo" (call
 * shape and outputs), "Ukubuyisa ama-index kuphela" (values optional),
 * "Ukusebenzisa i-index buffer ekhona" (caller-owned index buffer),
 * "Ukusebenza Ngemigqa Enobude Obuhlukahlukene" (per-row exclusive end and
 * OOB fills), "Ukuphathwa kwe-NaN" (NaN check; rows of valid length <= k are
 * not checked) and "Ukusebenza namathiphu athuthukile" (k <= 4096).
 *
 * For row i with valid length n = clamp(row_end ? row_end[i] : cols, 0, cols)
 * and c = min(k, n), the selected set is the c largest entries of
 * x[i, 0:n) under: NaN above +inf (all NaNs equal), -0 == +0, and among equal
 * values the lower column first.  Then
 *     out_idx[i, 0:c) = the selected columns in ascending column order
 *                       (by value with sorted_index 2, below)
 *     out_idx[i, c:k) = -1 (dsel_topk_ex: the given fill index)
 *     out_val[i, 0:c) = bit copies of x at those columns (NaN payloads kept)
 *     out_val[i, c:k) = -inf (dsel_topk_ex: the given fill value bits)
 *     nan_flag[i]     = (n > k) && some x[i, 0:n) is NaN
 * The selected columns always come out ascending, so `sorted_index` 0 and 1
 * cost nothing and give the same bytes.  `sorted_index` 2 orders each row's
 * c selected entries by value instead: largest first, equal values by
 * ascending column, NaN above every value, -0 equal to +0 (the tutorial's
 * end-bound example and its tip on ordering "by index or by value"); a
 * radix sort in LDS runs after the select, so this order costs time.
 *
 * x             [rows, cols] bf16 or f32 (`dtype`), last dim contiguous,
 *               row stride `x_row_stride` elements (>= cols).
 * k             1..4096, else DSEL_ERR_K.
 * row_end       int32 [rows] or NULL (all rows full length).
 * sorted_index  0, 1 or 2 (see above), else DSEL_ERR_ARG.
 * indices_type  DSEL_I32 or DSEL_I64.
 * return_value  0/1; when 0, out_val is ignored and may be NULL.
 * out_idx       caller-owned [rows, >= k] of the index dtype, row stride
 *               `idx_row_stride` elements.
 * out_val       [rows, >= k] of the input dtype, row stride `val_row_stride`.
 * nan_flag      uint8 [rows] or NULL.
 * Alignment: x, out_idx, out_val and each row stride in bytes must be
 *               multiples of 16, else DSEL_ERR_ALIGN.
 * workspace     device scratch for rows split over several workgroups.
 *               Pass NULL to query: *workspace_bytes (host) receives the size
 *               and nothing is launched.  Otherwise *workspace_bytes is the
 *               size provided (DSEL_ERR_WORKSPACE if smaller than the query).
 *               The workspace must be zero-filled before its first use; every
 *               call leaves it zero-filled again, except (a) word 0, which
 *               holds sticky error bits (bit 0: a split-row rendezvous gave
 *               up; see dsel_topk_check, which reports and clears them), and
 *               (b) the exchange region that follows the 64-word header,
 *               8 * (compute units) * 544 words, which holds scratch that
 *               every call writes before it reads it.
 *               Calls that share one workspace must be stream-ordered.
 * rows == 0 launches nothing and returns DSEL_OK.
 */
int dsel_topk(const void *x, int dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
              int64_t k, const int32_t *row_end,
              int sorted_index, int indices_type, int return_value,
              void *out_idx, int64_t idx_row_stride,
              void *out_val, int64_t val_row_stride,
              uint8_t *nan_flag,
              void *workspace, size_t *workspace_bytes,
              void *stream);

/* dsel_topk with the out-of-range fills given (DeepSelect tutorial, section
 * "Ukusebenza Ngemigqa Enobude Obuhlukahlukene": slots past a row's valid
 * length hold `idx_oob_fill_value` and `value_oob_fill_value`) and the row
 * order chosen.  Same arguments, then:
 * idx_fill        index written to slots [c, k) of a row (c = min(k, n));
 *                 must fit the index dtype (int32 range for DSEL_I32), else
 *                 DSEL_ERR_ARG.
 * val_fill_bits   raw bits of the value written there (bf16: <= 0xFFFF, else
 *                 DSEL_ERR_ARG).
 * row_order       DSEL_ROWS_AUTO, DSEL_ROWS_NATURAL or DSEL_ROWS_DUAL_CHUNK.
 * dsel_topk is dsel_topk_ex with idx_fill -1, val_fill_bits of -inf and
 * DSEL_ROWS_AUTO. */
int dsel_topk_ex(const void *x, int dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
                 int64_t k, const int32_t *row_end,
                 int sorted_index, int indices_type, int return_value,
                 void *out_idx, int64_t idx_row_stride,
                 void *out_val, int64_t val_row_stride,
                 uint8_t *nan_flag,
                 void *workspace, size_t *workspace_bytes,
                 void *stream, int64_t idx_fill, uint32_t val_fill_bits, int row_order);

/*
 * Error state of split rows on a workspace, and its reset.
 *
 * A row longer than one workgroup holds (16384 columns) is split over
 * several workgroups that meet at rendezvous points in the workspace; the
 * launch never asks for more workgroups than the GPU holds at once, but
 * work from other streams or processes can keep some of them from starting.
 * Every wait is bounded (about 0.1 s): a workgroup that gives up sets bit 0
 * (1) of workspace word 0 and finishes, so the kernel always ends, but that
 * call's split rows hold undefined output and the workspace is left in an
 * undefined state.  dsel_topk_check reports and clears that state.
 *
 * workspace, workspace_bytes: the workspace and size given to dsel_topk;
 *            NULL: the scratch of dsel_topk_noalloc on the current device
 *            (DSEL_OK at once if that entry point never ran on it).
 * stream:     the stream of those calls; the call SYNCHRONISES it.
 * error_bits: host pointer; receives word 0 (0 when no error).
 * Returns DSEL_OK when no rendezvous gave up since the last check.  Else it
 * zero-fills the whole workspace (so it is ready for the next call), writes
 * the bits and returns DSEL_ERR_SPLIT.
 */
int dsel_topk_check(void *workspace, size_t workspace_bytes, void *stream, uint32_t *error_bits);

/*
 * dsel_topk_ex for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments as dsel_topk_ex without the workspace: split rows (rows
 * over 16384 columns) use a scratch array of the library instead, 32 MiB of
 * device memory that every GPU the library runs on holds from its first
 * call until the process ends.  The first call on a device looks the array
 * up and zero-fills it (on `stream`; waited for unless `stream` is being
 * captured); every call leaves it ready for the next.  The call allocates
 * and frees nothing.  A call whose rows need more scratch than the array
 * holds is split into several launches; a single row that needs more
 * returns DSEL_ERR_WORKSPACE before anything is launched.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (other streams, other threads) race and must not be made;
 * order them on one stream.  Split-row errors are read and cleared with
 * dsel_topk_check(NULL, 0, stream, &bits).
 */
int dsel_topk_noalloc(const void *x, int dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
                      int64_t k, const int32_t *row_end,
                      int sorted_index, int indices_type, int return_value,
                      void *out_idx, int64_t idx_row_stride,
                      void *out_val, int64_t val_row_stride,
                      uint8_t *nan_flag, void *stream, int64_t idx_fill, uint32_t val_fill_bits,
                      int row_order);

/*
 * Gather of key rows at selected positions, batch offset folded in.
 *
 * MindSpore hyper-parallel PR #1094 (gather compressed keys through one
 * index_select), English description and the Chinese section on the fix:
 * the batch offset b*len is folded into each position so the gather is a
 * single index_select of D-vectors over the flattened key; the result equals
 * key[batch_ids, positions] bit for bit, also for a non-contiguous key and
 * for repeated positions.
 *
 *   out[b, r, j, :] = key[b, clamp(pos[b, r, j], 0, len-1), :]
 *
 * key      [batch, len, dim] of element size 2 (DSEL_BF16) or 4 (DSEL_F32),
 *          last dim contiguous; element strides key_batch_stride (between
 *          batches) and key_row_stride (between rows).
 * pos      [batch, rows_per_batch, >= per_row] of DSEL_I32 or DSEL_I64
 *          (`pos_type`), row stride pos_row_stride elements, batch stride
 *          rows_per_batch * pos_row_stride (so a top-k index buffer
 *          [batch*rows_per_batch, idx_row_stride] feeds in directly).
 * out      contiguous [batch, rows_per_batch, per_row, dim], key dtype.
 * Alignment: key, out and dim*elt, key strides*elt must be multiples of 16;
 *          pos must be aligned to its element size.
 * Empty shapes (batch, rows_per_batch or per_row == 0) launch nothing.
 */
int dsel_gather_rows(const void *key, int dtype, int64_t batch, int64_t len, int64_t dim,
                     int64_t key_batch_stride, int64_t key_row_stride,
                     const void *pos, int pos_type, int64_t rows_per_batch, int64_t per_row,
                     int64_t pos_row_stride,
                     void *out, void *stream);

/*
 * Top-k with the gather of keys at the selected positions, in one call.
 *
 * MindSpore hyper-parallel PR #1094: its candidate chain selects each query
 * row's top positions, sorts them, masks the invalid ones and gathers the
 * compressed keys there (key[batch_ids, safe_positions]); the English
 * description and the section on the fix make the gather one index_select
 * over batch-offset positions.  This entry point runs the chain's tail for a
 * batch of rows: the top-k of dsel_topk (index fill -1, no values, row order
 * DSEL_ROWS_AUTO), then for each key g
 *     out_g[r, j, :] = key_g[r / rows_per_batch, p, :],  p = out_idx[r, j],
 * where a position outside [0, len_g) (the -1 of a short row's padding) is
 * clamped into it (DSEL_PAD_CLAMP: the "safe" positions, as dsel_gather_rows)
 * or gives a row of zeros (DSEL_PAD_ZERO: the masked fill).  For one-wave
 * bf16 rows (at most 2048 columns) and whole rows (at most 16384 columns)
 * the select's own workers copy each row's keys as soon as it is selected:
 * one launch, and the positions are never read back from HBM.  Other rows
 * (split rows, fp32 rows of at most 2048 columns, sorted_index 2) run the
 * select, then one gather launch per key.
 *
 * Top-k arguments as dsel_topk (return_value 0); sorted_index 0, 1 or 2 (the
 * slots are gathered in the order the indices come out).
 * rows_per_batch  query rows per batch: rows must be a multiple; row r
 *                 belongs to batch r / rows_per_batch.
 * keys, n_keys    host array of 1..4 key descriptors (DselGatherKey): key
 *                 [batch, len, dim] of DSEL_BF16 or DSEL_F32 elements, last
 *                 dim contiguous, element strides batch_stride and
 *                 row_stride; out contiguous [rows, k, dim].  key, out,
 *                 dim * elt and the strides * elt must be multiples of 16
 *                 (else DSEL_ERR_ALIGN).
 * pad             DSEL_PAD_CLAMP or DSEL_PAD_ZERO.
 * workspace       as dsel_topk (NULL: size query, nothing launched).
 * Returns DSEL_ERR_ARG for a bad key descriptor, n_keys, pad or
 * rows_per_batch, else what dsel_topk returns for the same top-k.
 */
enum { DSEL_PAD_CLAMP = 0, DSEL_PAD_ZERO = 1 };

typedef struct DselGatherKey {
    const void *key;
    int dtype;              /* DSEL_BF16 or DSEL_F32 */
    int64_t len, dim;       /* rows per batch, elements per row */
    int64_t batch_stride;   /* elements between batches */
    int64_t row_stride;     /* elements between rows */
    void *out;              /* contiguous [rows, k, dim] */
} DselGatherKey;

int dsel_topk_gather(const void *x, int dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
                     int64_t k, const int32_t *row_end, int sorted_index, int indices_type,
                     void *out_idx, int64_t idx_row_stride, uint8_t *nan_flag,
                     int64_t rows_per_batch, const DselGatherKey *keys, int n_keys, int pad,
                     void *workspace, size_t *workspace_bytes, void *stream);

/*
 * dsel_read_floor — a measurement helper, not part of the selection: the
 * streaming-read floor of the select's input.  One launch reads `bytes`
 * bytes at x once, with the load form of the whole-row and split top-k
 * kernels (16-byte loads with the non-temporal hint, sixteen in flight per
 * thread of 256-thread workgroups, each workgroup a 64 KiB block), and
 * writes the XOR of the 32-bit words of block b to out[b], so a caller can
 * check that every byte was read.  Timing it at a workload's input size
 * gives the read time no top-k kernel of that size can beat on the device.
 *
 * x      device memory, 16-byte aligned (else DSEL_ERR_ALIGN).
 * bytes  a positive multiple of 16 (else DSEL_ERR_ARG).
 * out    device memory for ceil(bytes / 65536) words (NULL: DSEL_ERR_ARG).
 * stream the HIP stream (NULL: the default stream).
 * Returns DSEL_ERR_DEVICE if the launch fails.
 */
int dsel_read_floor(const void *x, int64_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSEL_H */
