// 2D rotary position embedding on q and k, in place in the packed qkv rows (k converted to
// binary16), plus a transposed binary16 copy of v for the attention kernel.
//
// [Z] "Step 3": the angle vector of patch (h, w) is blocked by axis,
// theta = [h f_0 .. h f_{Q-1}, w f_0 .. w f_{Q-1}] with Q = hd/4 (not interleaved), and the
// half-vector rotation pairs element i with i + hd/2.  [G] V4 Flash vision row: positions
// are the raw patch grid.  cos/sin come from tables [position][j] built on the host.  The
// rotation is evaluated as two products and one sum, each rounded (no fused multiply-add).
//
// One block per (64-row tile of one image, head).  q and k move as 16-byte chunks (8
// elements of the first half with the matching 8 of the second half).  The v tile goes
// through LDS and is written as vt[head][d][column] with 16-byte stores, so the attention
// kernel can stage V^T with 16-byte loads; inside each group of 16 columns, column p holds
// key p with bits 2 and 3 swapped.  Columns of the tile past the image's last patch are
// written as zeros, so every column the attention kernel reads is defined.  HBM-bound.
//
// The rotated q is stored as bf16.  The rotated k is rounded to bf16 like q and then stored
// as IEEE binary16, the operand type of the attention's score product; V^T is binary16 too
// (the operand type of P.V).  Every bf16 value of magnitude 2^-14 .. 65504 converts exactly
// (8 significant bits fit in 11), smaller ones keep an absolute error below 2^-25, larger
// ones saturate to +-65504 (NaN stays NaN).
#include "kernels.h"

namespace {

// (a, b) turned by the angle with cosine c and sine s; products and sums rounded separately.
__device__ __forceinline__ void rotate(float a, float b, float c, float s, float &na, float &nb)
{
#pragma clang fp contract(off)
    na = a * c - b * s;
    nb = b * c + a * s;
}

// Index with bits 2 and 3 exchanged (an involution on 0..15 within each 16-group).
__device__ __forceinline__ int swap23(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

__device__ __forceinline__ void unpack8(uint4 u, float *f)
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(w[j] << 16);
        f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
}

// bf16 bit pattern -> binary16 bit pattern (round to nearest even, saturating at 65504).
__device__ __forceinline__ uint16_t bf16_to_f16_sat(uint32_t b)
{
    float f = __uint_as_float(b << 16);
    if (__builtin_fabsf(f) > 65504.f) f = __builtin_copysignf(65504.f, f);
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ uint4 pack8(const float *f)
{
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
}

// Eight values rounded to bf16, then stored as binary16 bit patterns.
__device__ __forceinline__ uint4 pack8_f16_of_bf16(const float *f)
{
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t b = pack_bf16x2(f[2 * j], f[2 * j + 1]);
        w[j] = (uint32_t)bf16_to_f16_sat(b & 0xFFFFu) | ((uint32_t)bf16_to_f16_sat(b >> 16) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int HD>
__global__ __launch_bounds__(256) void rope_kernel(bf16_t *__restrict__ qkv, bf16_t *__restrict__ vt,
                                                   int64_t ldv, const RowTile *__restrict__ tiles,
                                                   const ImgDesc *__restrict__ imgs, int D,
                                                   const float *__restrict__ cos_t,
                                                   const float *__restrict__ sin_t)
{
    constexpr int HALF = HD / 2, T = kRopeTile, HC = HALF / 8;   // chunks per half
    constexpr int VLD = T + 8;                      // LDS row of the transposed v tile
    __shared__ __attribute__((aligned(16))) uint16_t sv[HD * VLD];   // binary16 bits

    const RowTile tile = tiles[blockIdx.x];
    const int head = blockIdx.y;
    const ImgDesc d = imgs[tile.img];
    const int64_t ld = 3 * (int64_t)D;
    bf16_t *base = qkv + (int64_t)d.patch_off * ld + head * HD;

    // q and k: one item = 8 elements of the first half and the 8 they pair with
    for (int w = threadIdx.x; w < T * 2 * HC; w += 256) {
        const int r = w / (2 * HC), rem = w - r * (2 * HC), part = rem / HC, ch = rem - part * HC;
        const int lr = tile.r0 + r;
        if (lr >= d.n) continue;
        const int hp = lr / d.gw;
        bf16_t *v = base + (int64_t)lr * ld + part * D + ch * 8;
        float a[8], b[8], cs[8], sn[8];
        unpack8(*reinterpret_cast<const uint4 *>(v), a);
        unpack8(*reinterpret_cast<const uint4 *>(v + HALF), b);
        rope_cos_sin8<HD>(cos_t, sin_t, make_int2(hp, lr - hp * d.gw), ch * 8, cs, sn);
        float na[8], nb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rotate(a[e], b[e], cs[e], sn[e], na[e], nb[e]);
        if (part == 0) {   // q
            *reinterpret_cast<uint4 *>(v) = pack8(na);
            *reinterpret_cast<uint4 *>(v + HALF) = pack8(nb);
        } else {           // k
            *reinterpret_cast<uint4 *>(v) = pack8_f16_of_bf16(na);
            *reinterpret_cast<uint4 *>(v + HALF) = pack8_f16_of_bf16(nb);
        }
    }

    // v: 16-byte row chunks -> binary16, LDS transposed (sv[d][key]) -> 16-byte stores of 8 columns
    constexpr int VC = HD / 8;                      // chunks per v row
    for (int w = threadIdx.x; w < T * VC; w += 256) {
        const int r = w / VC, ch = w - r * VC;
        const int lr = tile.r0 + r;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (lr < d.n) u = *reinterpret_cast<const uint4 *>(base + (int64_t)lr * ld + 2 * D + ch * 8);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sv[(ch * 8 + e) * VLD + r] = bf16_to_f16_sat((wd[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    }
    __syncthreads();
    // physical columns p..p+7 (p % 8 == 0) hold keys in two runs of 4: swap bits 2 and 3
    for (int w = threadIdx.x; w < HD * (T / 8); w += 256) {
        const int dd = w / (T / 8), p = (w - dd * (T / 8)) * 8;
        const int k0 = swap23(p), k1 = swap23(p + 4);   // keys at columns p and p + 4
        const uint2 lo = *reinterpret_cast<const uint2 *>(&sv[dd * VLD + k0]);
        const uint2 hi = *reinterpret_cast<const uint2 *>(&sv[dd * VLD + k1]);
        *reinterpret_cast<uint4 *>(vt + ((int64_t)head * HD + dd) * ldv + d.vt_off + tile.r0 + p) =
            make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
}

// Rotary table dump: row n of out (fp32 [M][hd]) = cos theta_0 .. theta_{hd/2-1} of packed
// patch n, then sin of the same angles; one thread per (patch, 8 angles).
template <int HD>
__global__ __launch_bounds__(256) void rope_dump_kernel(const ImgDesc *__restrict__ imgs, int n_img, int64_t M,
                                                        const float *__restrict__ cos_t,
                                                        const float *__restrict__ sin_t, float *__restrict__ out)
{
    constexpr int HALF = HD / 2, HC = HALF / 8;
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= M * HC) return;
    const int64_t row = w / HC;
    const int i0 = (int)(w - row * HC) * 8;
    float cs[8], sn[8];
    rope_cos_sin8<HD>(cos_t, sin_t, patch_grid_pos(imgs, n_img, row), i0, cs, sn);
    float4 *oc = reinterpret_cast<float4 *>(out + row * HD + i0);
    float4 *os = reinterpret_cast<float4 *>(out + row * HD + HALF + i0);
    oc[0] = make_float4(cs[0], cs[1], cs[2], cs[3]);
    oc[1] = make_float4(cs[4], cs[5], cs[6], cs[7]);
    os[0] = make_float4(sn[0], sn[1], sn[2], sn[3]);
    os[1] = make_float4(sn[4], sn[5], sn[6], sn[7]);
}

template <int HD>
hipError_t run_rope_dump(const ImgDesc *imgs, int n_img, int64_t M, const float *c, const float *s, float *out,
                         hipStream_t st)
{
    const int64_t threads = M * (HD / 16);
    hipLaunchKernelGGL(rope_dump_kernel<HD>, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, st, imgs, n_img,
                       M, c, s, out);
    return hipGetLastError();
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

hipError_t launch_dump_rope(const ImgDesc *imgs, int n_img, int64_t M, int hd, const float *cos_t,
                            const float *sin_t, float *out, hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    switch (hd) {
    case 16: return run_rope_dump<16>(imgs, n_img, M, cos_t, sin_t, out, s);
    case 32: return run_rope_dump<32>(imgs, n_img, M, cos_t, sin_t, out, s);
    case 64: return run_rope_dump<64>(imgs, n_img, M, cos_t, sin_t, out, s);
    case 128: return run_rope_dump<128>(imgs, n_img, M, cos_t, sin_t, out, s);
    default: return hipErrorInvalidValue;
    }
}
