// The streaming-read floor: one launch that reads a buffer once with the
// select's load form, for the roofline of the select's input reads.
//
// Each 256-thread workgroup reads 64 KB: sixteen 16-byte loads per thread
// in coalesced order (load j of thread t at vector j * 256 + t of the
// workgroup's block), every one in flight at once, through a buffer view of
// the block (bytes past the end read as zero, so no load is guarded) and
// with the non-temporal hint, as the whole-row and split top-k kernels load
// their rows.  The loaded words are folded with XOR into one word per
// workgroup, so nothing is optimised away and a caller can check that every
// byte was read.
#include "dsel_internal.h"
#include "../../include/dsel.h"

namespace dsel {
namespace {

constexpr int FT = 256;                        // threads per workgroup
constexpr int FL = 16;                         // 16-byte loads per thread
constexpr int64_t kFloorBlock = (int64_t)FT * FL * 16;  // bytes per workgroup

__global__ __launch_bounds__(FT) void read_floor_kernel(const char *x, int64_t bytes, uint32_t *out) {
    const int64_t off = (int64_t)blockIdx.x * kFloorBlock;
    const int64_t left = bytes - off;
    const __amdgpu_buffer_rsrc_t view = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(x + off), (short)0, (int)(left < kFloorBlock ? left : kFloorBlock),
        0x00020000);
    constexpr int kNonTemporal = 2;  // the nt bit of a buffer load's cache policy
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v[FL];
#pragma unroll
    for (int j = 0; j < FL; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(view, (unsigned)((j * FT + (int)threadIdx.x) * 16),
                                                     0u, kNonTemporal);
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < FL; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
    __shared__ uint32_t s_w[FT / 64];
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < FT / 64; ++w) r ^= s_w[w];
        out[blockIdx.x] = r;
    }
}

}  // namespace
}  // namespace dsel

extern "C" int dsel_read_floor(const void *x, int64_t bytes, uint32_t *out, void *stream) {
    using namespace dsel;
    if (!x || !out || bytes <= 0 || bytes % 16 != 0) return DSEL_ERR_ARG;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return DSEL_ERR_ALIGN;
    const int64_t blocks = (bytes + kFloorBlock - 1) / kFloorBlock;
    if (blocks > INT32_MAX) return DSEL_ERR_ARG;
    const char *xc = reinterpret_cast<const char *>(x);
    void *args[] = {&xc, &bytes, &out};
    return hipLaunchKernel(reinterpret_cast<const void *>(&read_floor_kernel), dim3((unsigned)blocks),
                           dim3(FT), args, 0, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? DSEL_OK
               : DSEL_ERR_DEVICE;
}
