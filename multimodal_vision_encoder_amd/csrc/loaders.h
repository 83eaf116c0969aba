// A-operand sources of the bf16 GEMMs.  The same functions feed the debug dumps, so a dumped
// tensor is exactly what the GEMM consumed.
#pragma once

#include "common.h"

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

// ---------------------------------------------------------------------------------------
// Address sources for the direct-to-LDS GEMM: per row a small state, per K chunk the address
// of 16 bytes (8 bf16) to copy.  Rows past M are clamped to M-1 (their outputs are never
// stored).
// ---------------------------------------------------------------------------------------
// Plain activations [M][lda]: one base pointer per row.
struct SrcPlain {
    const bf16_t *A;
    int64_t lda, M;
    struct Row { const bf16_t *p; };
    __device__ __forceinline__ Row row(int64_t r) const { return Row{A + (r < M ? r : M - 1) * lda}; }
    __device__ __forceinline__ const bf16_t *addr(const Row &rw, int k) const { return rw.p + k; }
};

// 3x3 merge gather of the projector ([Z] "Step 4"): row = merged token (my, mx) of its image,
// K index = pos * D + c with pos = dy*3 + dx (position-major projector weight); positions in
// the right/bottom padding read 16 zero bytes from `zero`.
struct SrcMerge {
    const bf16_t *y;
    const ImgDesc *imgs;
    int n_img;
    int64_t M;
    int D;
    const bf16_t *zero;   // at least 16 zero bytes
    struct Row { const bf16_t *base; int gh, gw, y0, x0; };
    __device__ __forceinline__ Row row(int64_t r) const
    {
        if (r >= M) r = M - 1;
        const ImgDesc &d = imgs[image_of_token(imgs, n_img, r)];
        const int local = (int)(r - d.tok_off), my = local / d.mw, mx = local - my * d.mw;
        return Row{y + (int64_t)d.patch_off * D, d.gh, d.gw, 3 * my, 3 * mx};
    }
    __device__ __forceinline__ const bf16_t *addr(const Row &rw, int k) const
    {
        const int pos = k / D, c = k - pos * D;
        const int sy = rw.y0 + pos / 3, sx = rw.x0 + pos % 3;
        return (sy < rw.gh && sx < rw.gw) ? rw.base + ((int64_t)sy * rw.gw + sx) * D + c : zero;
    }
};

