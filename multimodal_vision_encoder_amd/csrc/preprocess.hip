// Image preprocessing before the encoder: contain resize (bicubic) onto a gray canvas.
//
// [Z] "Step 1": the image is resized with contain semantics (bicubic) into a canvas whose
// sides are multiples of patch x merge pixels and centred on RGB 127 gray.  The resize is the
// Keys cubic convolution (a = -0.5) applied separably: output sample i of an axis sits at
// source coordinate (i + 0.5) * in/out; when shrinking, the kernel is stretched by in/out
// (support 2 * in/out) so that every source pixel contributes; taps outside the image are
// dropped and the remaining weights renormalised.  The horizontal pass keeps fp32 values in
// a scratch buffer [h][resized_w][3]; the vertical pass rounds half to even, clamps to
// 0..255, and writes the whole canvas (127 outside the resized image).  HBM-bound.
#include <math.h>

#include "kernels.h"

namespace {

__device__ __forceinline__ float keys_cubic(float x)
{
    constexpr float a = -0.5f;
    x = fabsf(x);
    if (x < 1.f) return ((a + 2.f) * x - (a + 3.f)) * x * x + 1.f;
    if (x < 2.f) return ((a * x - 5.f * a) * x + 8.f * a) * x - 4.f * a;
    return 0.f;
}

// Taps [lo, hi) and the centre / kernel stretch of output sample i of an axis n_in -> n_out.
struct Taps {
    int lo, hi;
    float c, inv_fs;   // centre, 1 / kernel stretch
};
__device__ __forceinline__ Taps taps_of(int i, int n_in, int n_out)
{
    const float scale = (float)n_in / (float)n_out, fs = fmaxf(scale, 1.f), support = 2.f * fs;
    const float c = ((float)i + 0.5f) * scale;
    Taps t;
    t.lo = max(0, (int)floorf(c - support));
    t.hi = min(n_in, (int)ceilf(c + support) + 1);
    t.c = c;
    t.inv_fs = 1.f / fs;
    return t;
}

// One thread per (source row, output column): three channels.
__global__ __launch_bounds__(256) void resize_h_kernel(const uint8_t *__restrict__ src, int h, int w,
                                                       float *__restrict__ tmp, int ow)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)h * ow) return;
    const int y = (int)(idx / ow), i = (int)(idx - (int64_t)y * ow);
    const Taps t = taps_of(i, w, ow);
    const uint8_t *row = src + (int64_t)y * w * 3;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, ks = 0.f;
    for (int j = t.lo; j < t.hi; ++j) {
        const float k = keys_cubic(((float)j + 0.5f - t.c) * t.inv_fs);
        a0 += k * (float)row[3 * j];
        a1 += k * (float)row[3 * j + 1];
        a2 += k * (float)row[3 * j + 2];
        ks += k;
    }
    float *o = tmp + idx * 3;
    const float inv = 1.f / ks;
    o[0] = a0 * inv;
    o[1] = a1 * inv;
    o[2] = a2 * inv;
}

// One thread per canvas pixel: three channels, 127 outside the resized image.
__global__ __launch_bounds__(256) void resize_v_kernel(const float *__restrict__ tmp, int h, int oh, int ow,
                                                       uint8_t *__restrict__ canvas, int ch, int cw, int oy, int ox)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)ch * cw) return;
    const int py = (int)(idx / cw), px = (int)(idx - (int64_t)py * cw);
    uint8_t *o = canvas + idx * 3;
    const int i = py - oy, x = px - ox;
    if (i < 0 || i >= oh || x < 0 || x >= ow) {
        o[0] = o[1] = o[2] = 127;
        return;
    }
    const Taps t = taps_of(i, h, oh);
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, ks = 0.f;
    for (int j = t.lo; j < t.hi; ++j) {
        const float k = keys_cubic(((float)j + 0.5f - t.c) * t.inv_fs);
        const float *v = tmp + ((int64_t)j * ow + x) * 3;
        a0 += k * v[0];
        a1 += k * v[1];
        a2 += k * v[2];
        ks += k;
    }
    const float inv = 1.f / ks;
    const float r[3] = {a0 * inv, a1 * inv, a2 * inv};
#pragma unroll
    for (int c = 0; c < 3; ++c) o[c] = (uint8_t)fminf(fmaxf(rintf(r[c]), 0.f), 255.f);
}

}  // namespace

hipError_t launch_preprocess(const uint8_t *src, int h, int w, float *tmp, int oh, int ow, uint8_t *canvas,
                             int ch, int cw, int oy, int ox, hipStream_t s)
{
    const int64_t n1 = (int64_t)h * ow, n2 = (int64_t)ch * cw;
    hipLaunchKernelGGL(resize_h_kernel, dim3((unsigned)ceil_div(n1, 256)), dim3(256), 0, s, src, h, w, tmp, ow);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(resize_v_kernel, dim3((unsigned)ceil_div(n2, 256)), dim3(256), 0, s, tmp, h, oh, ow, canvas,
                       ch, cw, oy, ox);
    return hipGetLastError();
}
