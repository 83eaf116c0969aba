// Shared device-side definitions of the gfx950 vision encoder kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 bit pattern

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kWave = 64;

// Per-image geometry of a packed batch (device copy built by the host planner).
struct ImgDesc {
    int32_t gh, gw;       // patch grid
    int32_t patch_off;    // first patch row of the image in the packed activations
    int32_t n;            // gh * gw
    int32_t tok_off;      // first merged-token row of the image in the output
    int32_t mh, mw;       // merged grid: ceil(gh/3), ceil(gw/3)
    int32_t vt_off;       // first column of the image in the transposed-V buffer (multiple of 64)
    int64_t pix_off;      // byte offset of the image in the pixel buffer
};

// One tile of rows of one image (attention query tiles, RoPE row tiles).
struct RowTile {
    int32_t img;
    int32_t r0;           // first row, local to the image
};

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 in one v_cvt_pk_bf16_f32 (round to nearest even); lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.f) & 0xFFFFu); }

// Index of the image containing `row` given ascending offsets off(0) = 0 <= ... (n entries).
template <class OffFn>
__device__ __forceinline__ int find_segment(int n, int64_t row, OffFn off)
{
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)off(mid) <= row) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ int image_of_patch(const ImgDesc *imgs, int n, int64_t row)
{
    return find_segment(n, row, [&](int i) { return imgs[i].patch_off; });
}

__device__ __forceinline__ int image_of_token(const ImgDesc *imgs, int n, int64_t row)
{
    return find_segment(n, row, [&](int i) { return imgs[i].tok_off; });
}

// Position (row, column) on its image's patch grid of packed patch `row`: patch p of an image
// sits at (p / gw, p % gw) ([G] V4 Flash vision row: RoPE uses the raw patch grid).
__device__ __forceinline__ int2 patch_grid_pos(const ImgDesc *imgs, int n, int64_t row)
{
    const ImgDesc &d = imgs[image_of_patch(imgs, n, row)];
    const int lr = (int)(row - d.patch_off), hp = lr / d.gw;
    return make_int2(hp, lr - hp * d.gw);
}

// cos and sin of the rotary angles i0 .. i0+7 (i0 % 8 == 0, i0 + 8 <= hd/2) of the patch at
// grid position hw ([Z] "Step 3": theta = [h f_0 .. h f_{Q-1}, w f_0 .. w f_{Q-1}], Q = hd/4),
// read from the host-built tables cos_t / sin_t [position][Q] (entry j of position p holds
// the angle p f_j).  Every RoPE rotation and the rotary-table dump read their angles here.
template <int HD>
__device__ __forceinline__ void rope_cos_sin8(const float *cos_t, const float *sin_t, int2 hw, int i0,
                                              float *cs, float *sn)
{
    constexpr int Q4 = HD / 4;
    if constexpr (Q4 % 8 == 0) {   // the 8 angles lie on one axis: two 16-byte loads each
        const int ax = i0 >= Q4, j0 = i0 - ax * Q4;
        const float4 *c4 = reinterpret_cast<const float4 *>(cos_t + (ax ? hw.y : hw.x) * Q4 + j0);
        const float4 *s4 = reinterpret_cast<const float4 *>(sin_t + (ax ? hw.y : hw.x) * Q4 + j0);
        const float4 c_a = c4[0], c_b = c4[1], s_a = s4[0], s_b = s4[1];
        cs[0] = c_a.x, cs[1] = c_a.y, cs[2] = c_a.z, cs[3] = c_a.w;
        cs[4] = c_b.x, cs[5] = c_b.y, cs[6] = c_b.z, cs[7] = c_b.w;
        sn[0] = s_a.x, sn[1] = s_a.y, sn[2] = s_a.z, sn[3] = s_a.w;
        sn[4] = s_b.x, sn[5] = s_b.y, sn[6] = s_b.z, sn[7] = s_b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = i0 + e, j = i < Q4 ? i : i - Q4, p = i < Q4 ? hw.x : hw.y;
            cs[e] = cos_t[p * Q4 + j];
            sn[e] = sin_t[p * Q4 + j];
        }
    }
}

// Source patch (local row inside the image) of position `pos` (dy*3 + dx) of merged token
// (my, mx), or -1 when it falls in the right/bottom zero padding.
__device__ __forceinline__ int merge_source(const ImgDesc &d, int my, int mx, int pos)
{
    int sy = 3 * my + pos / 3, sx = 3 * mx + pos % 3;
    return (sy < d.gh && sx < d.gw) ? sy * d.gw + sx : -1;
}

// MFMA 32x32x16 bf16 -> fp32 (gfx950).  A: lane l holds row l%32, k = 8*(l/32)..+7;
// B: lane l holds column l%32, same k; D: lane l holds column l%32, rows
// 8*(r/4) + 4*(l/32) + r%4 for register r.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// The same MFMA shape on IEEE binary16 operands (v_mfma_f32_32x32x16_f16).
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x16_t mfma32_f16(f16x8_t a, f16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8_t as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8_t, v); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
