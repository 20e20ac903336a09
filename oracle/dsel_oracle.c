/*
 * CPU oracle for the selection step: row-wise top-k, then key gather.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is a plain, slow,
 * obviously correct statement of what the selection step computes.
 *
 * Top-k (DeepSelect tutorial, "Sheshisa Imisebenzi ye-PyTorch TopK nge-DeepSelect"):
 *   - section "Ukusebenzisa i-TopK Okuyisisekelo": input (rows, cols), last
 *     dim contiguous, row stride given; values keep the input dtype; indices
 *     are int32 or int64; with sorted_index each row's indices ascend.
 *   - section "Ukusebenzisa i-end" example and tip 3 of "Ukusebenza
 *     namathiphu athuthukile": a selection may also be ordered by value.
 *     sorted_index = 2 asks for that order: largest value first, equal
 *     values by ascending index, which is the ranking order itself.
 *   - section "Ukusebenza Ngemigqa Enobude Obuhlukahlukene": a per-row
 *     exclusive end; a row shorter than k is padded with the OOB fill values.
 *   - section "Ukuphathwa kwe-NaN": NaN checking is always on, and rows whose
 *     valid length is <= k are not checked.
 *   - section "Ukusebenza namathiphu athuthukile", tip 1: k <= 4096.
 * Readings where the pages are silent (stated once here, used below):
 *   - ranking is by value, larger first; equal values keep index order
 *     (the lower index wins);
 *   - every NaN ranks above +inf and all NaNs are equal to each other;
 *     -0 equals +0; denormals are ordinary values;
 *   - fills (section "Ukusebenza Ngemigqa Enobude Obuhlukahlukene" names
 *     them, gives no values) default to index -1 and value -inf; a call may
 *     give others;
 *   - a row's valid length is clamp(end, 0, cols); the NaN check is reported
 *     as a per-row flag instead of a device trap.
 *
 * Gather (MindSpore hyper-parallel PR #1094, English description and the
 * Chinese section on the fix): keys [B, L, D] are gathered at positions
 * [B, R, P]; the batch offset b*L is folded into the position so the gather
 * is one index_select over the flattened key.  Positions are clamped into
 * [0, L-1] (the "safe positions" the call sites pass); the copy is exact.
 *
 * Compile-time switch ORACLE_MUTANT=<n> plants one deliberate mistake; it is
 * used only by the tests that show the pins catch such mistakes.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { OR_BF16 = 0, OR_F32 = 1 };
enum { OR_I32 = 0, OR_I64 = 1 };

typedef struct {
    double v;      /* exact decoded value (not used when is_nan) */
    int is_nan;
    int64_t idx;
} or_entry;

/* bf16 is the upper half of an IEEE binary32: widen by a 16-bit shift. */
static double decode(const unsigned char *row, int dtype, int64_t j, int *is_nan) {
    float f;
    if (dtype == OR_BF16) {
        uint16_t h;
        memcpy(&h, row + 2 * j, 2);
        uint32_t w = ((uint32_t)h) << 16;
        memcpy(&f, &w, 4);
    } else {
        memcpy(&f, row + 4 * j, 4);
    }
    *is_nan = isnan(f) ? 1 : 0;
#if ORACLE_MUTANT == 3
    /* planted: -0 ranks below +0 */
    if (f == 0.0f && signbit(f)) return -1e-300;
#endif
    return (double)f;
}

/* Total order used to rank a row: a before b?  Returns <0 if a ranks first. */
static int cmp_entry(const void *pa, const void *pb) {
    const or_entry *a = (const or_entry *)pa, *b = (const or_entry *)pb;
#if ORACLE_MUTANT == 2
    /* planted: NaN ranks below everything */
    if (a->is_nan != b->is_nan) return a->is_nan ? 1 : -1;
#else
    if (a->is_nan != b->is_nan) return a->is_nan ? -1 : 1;
#endif
    if (!a->is_nan) {
#if ORACLE_MUTANT == 11
        /* planted: ascending instead of descending */
        if (a->v < b->v) return -1;
        if (a->v > b->v) return 1;
#else
        if (a->v > b->v) return -1;
        if (a->v < b->v) return 1;
#endif
    }
#if ORACLE_MUTANT == 1
    /* planted: ties broken towards the higher index */
    return (a->idx > b->idx) ? -1 : (a->idx < b->idx) ? 1 : 0;
#else
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx) ? 1 : 0;
#endif
}

static int cmp_idx(const void *pa, const void *pb) {
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    return (a < b) ? -1 : (a > b) ? 1 : 0;
}

typedef struct {
    const unsigned char *x;
    int dtype;
    int64_t rows, cols, x_row_stride, k;
    const int32_t *row_end;
    int sorted_index, indices_type, return_value;
    int64_t idx_fill;
    uint32_t val_fill;
    unsigned char *out_idx;
    int64_t idx_row_stride;
    unsigned char *out_val;
    int64_t val_row_stride;
    uint8_t *nan_flag;
    int64_t row_lo, row_hi;
    int status;
} topk_job;

static void put_index(unsigned char *row, int indices_type, int64_t slot, int64_t v) {
    if (indices_type == OR_I32) {
        int32_t t = (int32_t)v;
        memcpy(row + 4 * slot, &t, 4);
    } else {
        memcpy(row + 8 * slot, &v, 8);
    }
}

static void put_fill(unsigned char *row, int dtype, int64_t slot, uint32_t bits) {
    if (dtype == OR_BF16) {
        uint16_t h = (uint16_t)bits;
        memcpy(row + 2 * slot, &h, 2);
    } else {
        memcpy(row + 4 * slot, &bits, 4);
    }
}

static void *topk_rows(void *arg) {
    topk_job *J = (topk_job *)arg;
    const int esz = (J->dtype == OR_BF16) ? 2 : 4;
    or_entry *ent = (or_entry *)malloc(sizeof(or_entry) * (size_t)(J->cols > 0 ? J->cols : 1));
    int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)(J->k > 0 ? J->k : 1));
    if (!ent || !sel) { J->status = -1; free(ent); free(sel); return NULL; }
    for (int64_t i = J->row_lo; i < J->row_hi; ++i) {
        const unsigned char *row = J->x + (size_t)(i * J->x_row_stride) * esz;
        /* valid length: clamp(end, 0, cols) */
        int64_t n = J->row_end ? (int64_t)J->row_end[i] : J->cols;
#if ORACLE_MUTANT == 4
        n += 1; /* planted: end treated as inclusive */
#endif
        if (n < 0) n = 0;
        if (n > J->cols) n = J->cols;
        int64_t c = (J->k < n) ? J->k : n;

        int any_nan = 0;
        for (int64_t j = 0; j < n; ++j) {
            ent[j].v = decode(row, J->dtype, j, &ent[j].is_nan);
            ent[j].idx = j;
            any_nan |= ent[j].is_nan;
        }
        if (J->nan_flag) {
#if ORACLE_MUTANT == 5
            J->nan_flag[i] = (uint8_t)(any_nan ? 1 : 0); /* planted: short rows checked too */
#else
            J->nan_flag[i] = (uint8_t)((n > J->k && any_nan) ? 1 : 0);
#endif
        }
        /* rank the valid prefix; the comparator is a total order (value,
         * then index), so the result equals a stable sort by value */
        qsort(ent, (size_t)n, sizeof(or_entry), cmp_entry);
        for (int64_t s = 0; s < c; ++s) sel[s] = ent[s].idx;
#if ORACLE_MUTANT != 8
        if (J->sorted_index == 1) qsort(sel, (size_t)c, sizeof(int64_t), cmp_idx);
#endif
#if ORACLE_MUTANT == 13
        if (J->sorted_index == 2) /* planted: value order reversed */
            for (int64_t a = 0, b = c - 1; a < b; ++a, --b) { int64_t t = sel[a]; sel[a] = sel[b]; sel[b] = t; }
#endif
        unsigned char *orow = J->out_idx + (size_t)(i * J->idx_row_stride) * (J->indices_type == OR_I32 ? 4 : 8);
        for (int64_t s = 0; s < J->k; ++s) {
#if ORACLE_MUTANT == 6
            put_index(orow, J->indices_type, s, s < c ? sel[s] : 0); /* planted: pad with 0 */
#else
            put_index(orow, J->indices_type, s, s < c ? sel[s] : J->idx_fill);
#endif
        }
        if (J->return_value) {
            unsigned char *vrow = J->out_val + (size_t)(i * J->val_row_stride) * esz;
            for (int64_t s = 0; s < J->k; ++s) {
                if (s < c) {
                    int64_t src = sel[s];
#if ORACLE_MUTANT == 7
                    if (src + 1 < n) src += 1; /* planted: value read one column off */
#endif
                    memcpy(vrow + esz * s, row + esz * src, (size_t)esz); /* bit copy */
                } else {
                    put_fill(vrow, J->dtype, s, J->val_fill);
                }
            }
        }
    }
    free(ent);
    free(sel);
    return NULL;
}

/* Returns 0 on success, negative on bad arguments or allocation failure.
 * idx_fill / val_fill_bits: the index and value bits of slots past a short
 * row's length (the defaults are -1 and -inf). */
int oracle_topk(const void *x, int dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
                int64_t k, const int32_t *row_end, int sorted_index, int indices_type,
                int return_value, void *out_idx, int64_t idx_row_stride, void *out_val,
                int64_t val_row_stride, uint8_t *nan_flag, int nthreads, int64_t idx_fill,
                uint32_t val_fill_bits) {
    if (rows < 0 || cols < 0 || k < 1 || k > 4096) return -2;
    if (dtype != OR_BF16 && dtype != OR_F32) return -1;
    if (indices_type != OR_I32 && indices_type != OR_I64) return -1;
    if (sorted_index < 0 || sorted_index > 2) return -1;
    if (rows == 0) return 0;
    if (!x || !out_idx || (return_value && !out_val)) return -1;
    if (x_row_stride < cols || idx_row_stride < k || (return_value && val_row_stride < k)) return -1;
#if ORACLE_MUTANT == 12
    x_row_stride = cols; /* planted: row stride ignored */
#endif
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = (int)rows;
    topk_job *jobs = (topk_job *)calloc((size_t)nthreads, sizeof(topk_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -3; }
    int64_t per = (rows + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        topk_job *J = &jobs[t];
        J->x = (const unsigned char *)x; J->dtype = dtype; J->rows = rows; J->cols = cols;
        J->x_row_stride = x_row_stride; J->k = k; J->row_end = row_end;
        J->sorted_index = sorted_index; J->indices_type = indices_type; J->return_value = return_value;
        J->idx_fill = idx_fill; J->val_fill = val_fill_bits;
        J->out_idx = (unsigned char *)out_idx; J->idx_row_stride = idx_row_stride;
        J->out_val = (unsigned char *)out_val; J->val_row_stride = val_row_stride;
        J->nan_flag = nan_flag;
        J->row_lo = t * per;
        J->row_hi = (t + 1) * per < rows ? (t + 1) * per : rows;
        if (J->row_lo > J->row_hi) J->row_lo = J->row_hi;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, topk_rows, &jobs[t]);
    topk_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    int st = 0;
    for (int t = 0; t < nthreads; ++t) if (jobs[t].status) st = -3;
    free(jobs);
    free(th);
    return st;
}

/*
 * out[b, r, j, :] = key[b, clamp(pos[b, r, j], 0, len-1), :]
 * (MindSpore hyper-parallel PR #1094: key[batch_ids, safe_positions]); with
 * pad_zero, a position outside [0, len) gives a row of zeros instead (the
 * MaskedFill step of the same page's candidate chain).
 * key is addressed through element strides (batch, row); its last dim is
 * contiguous.  pos is [batch, rows_per_batch, per_row] with row stride
 * pos_row_stride (elements) and batch stride rows_per_batch*pos_row_stride.
 * out is contiguous [batch, rows_per_batch, per_row, dim].
 */
int oracle_gather(const void *key, int elt_size, int64_t batch, int64_t len, int64_t dim,
                  int64_t key_batch_stride, int64_t key_row_stride, const void *pos,
                  int pos_type, int64_t rows_per_batch, int64_t per_row,
                  int64_t pos_row_stride, void *out, int pad_zero) {
    if (batch < 0 || len < 1 || dim < 1 || rows_per_batch < 0 || per_row < 0) return -1;
    if (elt_size != 2 && elt_size != 4) return -1;
    if (pos_type != OR_I32 && pos_type != OR_I64) return -1;
    const unsigned char *K = (const unsigned char *)key;
    unsigned char *O = (unsigned char *)out;
    size_t row_bytes = (size_t)dim * (size_t)elt_size;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t r = 0; r < rows_per_batch; ++r) {
            int64_t prow = (b * rows_per_batch + r) * pos_row_stride;
            for (int64_t j = 0; j < per_row; ++j) {
                int64_t p;
                if (pos_type == OR_I32) {
                    int32_t t;
                    memcpy(&t, (const unsigned char *)pos + 4 * (size_t)(prow + j), 4);
                    p = t;
                } else {
                    memcpy(&p, (const unsigned char *)pos + 8 * (size_t)(prow + j), 8);
                }
#if ORACLE_MUTANT == 10
                p += 1; /* planted: position off by one */
#endif
                unsigned char *dst0 = O + (((size_t)(b * rows_per_batch + r) * (size_t)per_row + (size_t)j) * row_bytes);
#if ORACLE_MUTANT == 14
                int inside = p >= 0 && p <= len; /* planted: the masked fill lets position len through */
#else
                int inside = p >= 0 && p < len;
#endif
                if (pad_zero && !inside) {
                    /* the masked fill: a position outside the key gives a row of zeros */
                    memset(dst0, 0, row_bytes);
                    continue;
                }
                if (p < 0) p = 0;
                if (p > len - 1) p = len - 1;
#if ORACLE_MUTANT == 9
                int64_t src_b = 0; /* planted: batch offset dropped */
#else
                int64_t src_b = b;
#endif
                const unsigned char *src = K + (size_t)(src_b * key_batch_stride + p * key_row_stride) * elt_size;
                unsigned char *dst = O + (((size_t)(b * rows_per_batch + r) * (size_t)per_row + (size_t)j) * row_bytes);
                memcpy(dst, src, row_bytes);
            }
        }
    }
    return 0;
}
