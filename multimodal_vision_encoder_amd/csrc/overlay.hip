// Overlay of visual rows onto the prompt embedding matrix ([Z] "Multimodal basics": vision
// vectors replace the image-placeholder rows; "Connect the complete image-to-text path":
// chunked prefill replaces only the rows inside its chunk, here expressed by negative
// destination rows that are skipped).  One block per visual row; fp32 -> bf16 (round to
// nearest even), 16-byte reads and 8-byte writes.  HBM-bound.
#include "kernels.h"

namespace {

__global__ __launch_bounds__(256) void overlay_kernel(uint16_t *__restrict__ embeds,
                                                      const float *__restrict__ src,
                                                      const int32_t *__restrict__ rows,
                                                      int hidden)
{
    const int64_t t = blockIdx.x;
    const int32_t r = rows[t];
    if (r < 0) return;
    const float *in = src + t * hidden;
    uint16_t *out = embeds + (int64_t)r * hidden;
    if ((hidden & 3) == 0) {
        for (int j = threadIdx.x * 4; j < hidden; j += 256 * 4) {
            const float4 v = *reinterpret_cast<const float4 *>(in + j);
            *reinterpret_cast<uint2 *>(out + j) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
        }
    } else {
        for (int j = threadIdx.x; j < hidden; j += 256) out[j] = f32_to_bf16(in[j]);
    }
}

// Embedding assembly of a prefill chunk ([Z] "Connect the complete image-to-text path": the
// aligner output replaces the IMAGE positions of each image span, learned vectors fill its
// START, NEWLINE and END positions, and a chunk replaces only the part of a span inside it).
// One block per span position inside the chunk: entry (row of the chunk, source), source >= 0
// a visual row (fp32 -> bf16, round to nearest even), source -1 - s the sentinel row s.
__global__ __launch_bounds__(256) void assemble_kernel(uint16_t *__restrict__ embeds,
                                                       const float *__restrict__ src,
                                                       const uint16_t *__restrict__ sentinels,
                                                       const int2 *__restrict__ entries, int hidden)
{
    const int2 e = entries[blockIdx.x];
    uint16_t *out = embeds + (int64_t)e.x * hidden;
    if (e.y >= 0) {
        const float *in = src + (int64_t)e.y * hidden;
        if ((hidden & 3) == 0) {
            for (int j = threadIdx.x * 4; j < hidden; j += 256 * 4) {
                const float4 v = *reinterpret_cast<const float4 *>(in + j);
                *reinterpret_cast<uint2 *>(out + j) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
            }
        } else {
            for (int j = threadIdx.x; j < hidden; j += 256) out[j] = f32_to_bf16(in[j]);
        }
    } else {
        const uint16_t *in = sentinels + (int64_t)(-1 - e.y) * hidden;
        if ((hidden & 7) == 0) {
            for (int j = threadIdx.x * 8; j < hidden; j += 256 * 8)
                *reinterpret_cast<uint4 *>(out + j) = *reinterpret_cast<const uint4 *>(in + j);
        } else {
            for (int j = threadIdx.x; j < hidden; j += 256) out[j] = in[j];
        }
    }
}

}  // namespace

hipError_t launch_assemble(uint16_t *embeds, const float *src, const uint16_t *sentinels,
                           const int32_t *entries, int64_t n_entries, int hidden, hipStream_t s)
{
    if (n_entries <= 0) return hipSuccess;
    hipLaunchKernelGGL(assemble_kernel, dim3((unsigned)n_entries), dim3(256), 0, s, embeds, src, sentinels,
                       reinterpret_cast<const int2 *>(entries), hidden);
    return hipGetLastError();
}

hipError_t launch_overlay(uint16_t *embeds, const float *src, const int32_t *rows, int64_t n_rows,
                          int hidden, hipStream_t s)
{
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(overlay_kernel, dim3((unsigned)n_rows), dim3(256), 0, s, embeds, src, rows,
                       hidden);
    return hipGetLastError();
}
