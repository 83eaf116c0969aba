// 2D rotary position embedding on q and k, in place in the packed qkv rows, plus a
// transposed copy of v for the attention kernel.
//
// [Z] "Step 3": the angle vector of patch (h, w) is blocked by axis,
// theta = [h f_0 .. h f_{Q-1}, w f_0 .. w f_{Q-1}] with Q = hd/4 (not interleaved), and the
// half-vector rotation pairs element i with i + hd/2.  [G] V4 Flash vision row: positions
// are the raw patch grid.  cos/sin come from tables [position][j] built on the host.  The
// rotation is evaluated as two products and one sum, each rounded (no fused multiply-add).
//
// One block per (64-row tile of one image, head).  The v tile goes through LDS and is
// written as vt[head][d][column] so that the attention kernel can stage V^T with 16-byte
// loads; inside each group of 16 columns, column p holds key p with bits 2 and 3 swapped.
// Columns of the tile past the image's last patch are written as zeros, so every column
// the attention kernel reads is defined.  HBM-bound.
#include "kernels.h"

namespace {

// (a, b) turned by the angle with cosine c and sine s; products and sums rounded separately.
__device__ __forceinline__ void rotate(float a, float b, float c, float s, float &na, float &nb)
{
#pragma clang fp contract(off)
    na = a * c - b * s;
    nb = b * c + a * s;
}

template <int HD>
__global__ __launch_bounds__(256) void rope_kernel(bf16_t *__restrict__ qkv, bf16_t *__restrict__ vt,
                                                   int64_t ldv, const RowTile *__restrict__ tiles,
                                                   const ImgDesc *__restrict__ imgs, int D,
                                                   const float *__restrict__ cos_t,
                                                   const float *__restrict__ sin_t)
{
    constexpr int HALF = HD / 2, Q4 = HD / 4, T = kRopeTile;
    __shared__ bf16_t sv[HD][T + 2];

    const RowTile tile = tiles[blockIdx.x];
    const int head = blockIdx.y;
    const ImgDesc d = imgs[tile.img];
    const int64_t ld = 3 * (int64_t)D;
    bf16_t *base = qkv + (int64_t)d.patch_off * ld + head * HD;

    // q and k: one rotation pair (i, i + HALF) per work item
    for (int w = threadIdx.x; w < T * 2 * HALF; w += 256) {
        const int r = w / (2 * HALF), rem = w - r * (2 * HALF), part = rem / HALF,
                  i = rem - part * HALF;
        const int lr = tile.r0 + r;
        if (lr >= d.n) continue;
        const int hp = lr / d.gw, wp = lr - hp * d.gw;
        const int j = i < Q4 ? i : i - Q4;
        const int pos = i < Q4 ? hp : wp;
        const float c = cos_t[pos * Q4 + j], s = sin_t[pos * Q4 + j];
        bf16_t *v = base + (int64_t)lr * ld + part * D;
        float na, nb;
        rotate(bf16_to_f32(v[i]), bf16_to_f32(v[i + HALF]), c, s, na, nb);
        v[i] = f32_to_bf16(na);
        v[i + HALF] = f32_to_bf16(nb);
    }

    // v: tile -> LDS -> transposed store
    for (int w = threadIdx.x; w < T * HD; w += 256) {
        const int r = w / HD, dd = w - r * HD;
        const int lr = tile.r0 + r;
        sv[dd][r] = lr < d.n ? base[(int64_t)lr * ld + 2 * D + dd] : (bf16_t)0;
    }
    __syncthreads();
    // column p of each 16-column group holds key p with bits 2 and 3 swapped (an involution),
    // the order in which the attention kernel's P.V operand wants 8 keys per lane
    for (int w = threadIdx.x; w < HD * T; w += 256) {
        const int dd = w / T, p = w - dd * T;
        const int key = (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
        vt[((int64_t)head * HD + dd) * ldv + d.vt_off + tile.r0 + p] = sv[dd][key];
    }
}

template <int HD>
hipError_t run_rope(bf16_t *qkv, bf16_t *vt, int64_t ldv, const RowTile *tiles, int n_tiles,
                    const ImgDesc *imgs, int D, int H, const float *c, const float *s,
                    hipStream_t st)
{
    hipLaunchKernelGGL(rope_kernel<HD>, dim3(n_tiles, H), dim3(256), 0, st, qkv, vt, ldv, tiles,
                       imgs, D, c, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(bf16_t *qkv, bf16_t *vt, int64_t ldv, const RowTile *tiles, int n_tiles,
                       const ImgDesc *imgs, int D, int H, const float *cos_t, const float *sin_t,
                       hipStream_t s)
{
    if (n_tiles <= 0) return hipSuccess;
    switch (D / H) {
    case 16: return run_rope<16>(qkv, vt, ldv, tiles, n_tiles, imgs, D, H, cos_t, sin_t, s);
    case 32: return run_rope<32>(qkv, vt, ldv, tiles, n_tiles, imgs, D, H, cos_t, sin_t, s);
    case 64: return run_rope<64>(qkv, vt, ldv, tiles, n_tiles, imgs, D, H, cos_t, sin_t, s);
    case 128: return run_rope<128>(qkv, vt, ldv, tiles, n_tiles, imgs, D, H, cos_t, sin_t, s);
    default: return hipErrorInvalidValue;
    }
}
