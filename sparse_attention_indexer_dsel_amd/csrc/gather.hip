// Gather of key rows at selected positions with the batch offset folded in.
//
// MindSpore hyper-parallel PR #1094 (English description; Chinese section on
// the fix): the two-tensor form key[batch_ids, positions] becomes a single
// index_select of D-vectors over the flattened key at b*len + position; the
// result is the same bits.  Positions are clamped into [0, len-1], the
// "safe" positions its call sites pass; with pad_zero (the chain's masked
// fill, for the fused entry point's unfused rows) a position outside
// [0, len-1] gives a zero row instead.
//
// Layout here: one workgroup per (batch, query-row) pair walks that row's
// positions (staged in LDS); 16-byte vector copies, cached loads from the
// key (rows are revisited by neighbouring query rows) and non-temporal
// stores of the output, which is written once and never re-read.
#include "dsel_internal.h"

namespace dsel {
namespace {

constexpr int GT = 512;        // threads per workgroup (measured: 256 and 1024 were slower)
constexpr int UNROLL = 16;     // independent 16-byte copies in flight per thread
constexpr int POS_CHUNK = 1024;  // positions staged in LDS at a time

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (batch, query-row) pair: the row's positions are
// clamped and staged in LDS a chunk at a time (so no copy waits on a
// position load), then its D-vectors are copied with UNROLL 16-byte loads
// in flight per thread.
template <bool POS64, bool POW2>
__global__ __launch_bounds__(GT) void gather_rows_kernel(const GatherArgs a) {
    __shared__ int64_t s_off[POS_CHUNK];  // byte offset of each staged key row
    const int64_t pairs = a.batch * a.R;
    for (int64_t br = blockIdx.x; br < pairs; br += gridDim.x) {
        const int64_t b = br / a.R;
        const char *kb = a.key + b * a.key_batch_bytes;
        const int64_t prow = br * a.pos_row_stride;
        for (int64_t p0 = 0; p0 < a.P; p0 += POS_CHUNK) {
            const int cnt = (int)(a.P - p0 < POS_CHUNK ? a.P - p0 : POS_CHUNK);
            __syncthreads();  // the previous chunk's offsets are no longer read
            for (int j = threadIdx.x; j < cnt; j += GT) {
                int64_t p = POS64 ? reinterpret_cast<const int64_t *>(a.pos)[prow + p0 + j]
                                  : (int64_t)reinterpret_cast<const int32_t *>(a.pos)[prow + p0 + j];
                const bool in = p >= 0 && p < a.len;
                p = p < 0 ? 0 : (p >= a.len ? a.len - 1 : p);
                s_off[j] = (a.pad_zero && !in) ? -1 : p * a.key_row_bytes;  // -1: a zero row
            }
            __syncthreads();
            const int64_t total = (int64_t)cnt * a.row_vecs;
            u32x4 *ob = reinterpret_cast<u32x4 *>(a.out) + (br * a.P + p0) * a.row_vecs;
            for (int64_t i0 = threadIdx.x; i0 < total; i0 += (int64_t)GT * UNROLL) {
                u32x4 v[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {  // unconditional: clamped index
                    const int64_t i0u = i0 + (int64_t)u * GT;
                    const int64_t i = i0u < total ? i0u : total - 1;
                    const int64_t j = POW2 ? (i >> a.row_vecs_log2) : (i / a.row_vecs);
                    const int64_t vi = i - j * a.row_vecs;
                    const int64_t off = s_off[j];
                    v[u] = off < 0 ? u32x4{0u, 0u, 0u, 0u}
                                   : *reinterpret_cast<const u32x4 *>(kb + off + vi * 16);
                }
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    const int64_t i = i0 + (int64_t)u * GT;
                    if (i < total) __builtin_nontemporal_store(v[u], ob + i);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gather(int pos64, const GatherArgs &a, hipStream_t stream) {
    const int64_t pairs = a.batch * a.R;
    const unsigned grid = (unsigned)(pairs < (1 << 22) ? pairs : (1 << 22));
    const bool pow2 = a.row_vecs_log2 >= 0;
    GatherArgs copy = a;
    void *args[] = {&copy};
    const void *fn;
    if (pos64)
        fn = pow2 ? reinterpret_cast<const void *>(&gather_rows_kernel<true, true>)
                  : reinterpret_cast<const void *>(&gather_rows_kernel<true, false>);
    else
        fn = pow2 ? reinterpret_cast<const void *>(&gather_rows_kernel<false, true>)
                  : reinterpret_cast<const void *>(&gather_rows_kernel<false, false>);
    return hipLaunchKernel(fn, dim3(grid), dim3(GT), args, 0, stream);
}

}  // namespace dsel
