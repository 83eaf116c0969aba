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

}  // namespace

hipError_t launch_overlay(uint16_t *embeds, const float *src, const int32_t *rows, int64_t n_rows,
                          int hidden, hipStream_t s)
{
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(overlay_kernel, dim3((unsigned)n_rows), dim3(256), 0, s, embeds, src, rows,
                       hidden);
    return hipGetLastError();
}
