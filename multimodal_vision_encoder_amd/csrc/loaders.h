// A-operand loaders of the bf16 GEMM.  Each returns 8 consecutive K elements (16 bytes) of
// one row of the virtual A matrix; rows at or beyond M read as zeros.  The same functions
// feed the debug dumps, so a dumped tensor is exactly what the GEMM consumed.
#pragma once

#include "common.h"

// Plain row-major bf16 activations [M][lda].
struct LoadPlain {
    const bf16_t *A;
    int64_t lda;
    int64_t M;
    __device__ __forceinline__ uint4 operator()(int64_t row, int k) const
    {
        if (row >= M) return make_uint4(0, 0, 0, 0);
        return *reinterpret_cast<const uint4 *>(A + row * lda + k);
    }
};

// Patchify fused into the patch projection ([Z] "Step 1": rows in (grid_y, grid_x) order,
// columns in (channel, y, x) order; pixels normalised as fmaf(u8, s_c, t_c), rounded to bf16;
// [Z] "Step 5": columns past 3*ps*ps read as zero, which leaves the product unchanged).
// Pixels are uint8 HWC per image, images packed back to back.
struct LoadPatch {
    const uint8_t *px;
    const ImgDesc *imgs;
    int n_img;
    int64_t M;
    int ps;              // patch side
    int cols;            // 3 * ps * ps
    float s0, s1, s2;    // 1 / (255 std_c)
    float t0, t1, t2;    // -mean_c / std_c

    __device__ __forceinline__ uint4 operator()(int64_t row, int k) const
    {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (row < M && k < cols) {
            const ImgDesc &d = imgs[image_of_patch(imgs, n_img, row)];
            const int local = (int)(row - d.patch_off);
            const int gy = local / d.gw, gx = local - gy * d.gw;
            const int64_t W = (int64_t)ps * d.gw;
            const uint8_t *base = px + d.pix_off + ((int64_t)gy * ps * W + (int64_t)gx * ps) * 3;
            const int pp = ps * ps;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk = k + j;
                float v = 0.f;
                if (kk < cols) {
                    const int c = kk / pp, r = kk - c * pp, y = r / ps, x = r - y * ps;
                    const float u = (float)base[((int64_t)y * W + x) * 3 + c];
                    const float s = c == 0 ? s0 : (c == 1 ? s1 : s2);
                    const float t = c == 0 ? t0 : (c == 1 ? t1 : t2);
                    v = __builtin_fmaf(u, s, t);
                }
                const uint32_t b = f32_to_bf16(v);
                w[j >> 1] |= (j & 1) ? (b << 16) : b;
            }
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};

// 3x3 merge gather fused into the projector ([Z] "Step 4").  The projector weight is stored
// position-major (column pos*D + c holds the original column c*9 + pos), so a K chunk is 8
// consecutive channels of one source patch row of the final-norm output `y` [N][D];
// positions in the right/bottom padding read as zero.
struct LoadMerge {
    const bf16_t *y;
    const ImgDesc *imgs;
    int n_img;
    int64_t M;           // merged tokens in the batch
    int D;

    __device__ __forceinline__ uint4 operator()(int64_t row, int k) const
    {
        if (row >= M) return make_uint4(0, 0, 0, 0);
        const ImgDesc &d = imgs[image_of_token(imgs, n_img, row)];
        const int local = (int)(row - d.tok_off);
        const int my = local / d.mw, mx = local - my * d.mw;
        const int pos = k / D, c = k - pos * D;
        const int src = merge_source(d, my, mx, pos);
        if (src < 0) return make_uint4(0, 0, 0, 0);
        return *reinterpret_cast<const uint4 *>(y + ((int64_t)d.patch_off + src) * D + c);
    }
};
