// Patchify and the patch projection, plus the debug materialisation of fused-only tensors.
//
// The patch projection writes the normalised bf16 patch matrix once ([Z] "Step 1": rows in
// (grid_y, grid_x) order, columns (channel, y, x); columns past 3*ps*ps zero up to the padded
// K of the projection weight, [Z] "Step 5") and runs the large-tile GEMM of gemm_big.hip on
// it.  The matrix is ~12 MB at the 1024-token image; computing it inside the GEMM's A loader
// would cost the direct global -> LDS copies that the GEMM depends on.
#include "kernels.h"
#include "loaders.h"

namespace {

// One thread per 16-byte chunk (8 values) of the patch matrix [M][pitch].
__global__ __launch_bounds__(256) void patchify_kernel(LoadPatch al, bf16_t *out, int pitch)
{
    const int chunks = pitch / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= al.M * chunks) return;
    const int64_t row = idx / chunks;
    const int k = (int)(idx - row * chunks) * 8;
    *reinterpret_cast<uint4 *>(out + row * pitch + k) = al(row, k);
}

__global__ __launch_bounds__(256) void dump_patches_kernel(LoadPatch al, bf16_t *out)
{
    const int64_t row = blockIdx.x;
    for (int k = threadIdx.x * 8; k < al.cols; k += 256 * 8) {
        const uint4 v = al(row, k);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (k + j < al.cols)
                out[row * al.cols + k + j] = (bf16_t)((w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu);
    }
}

__global__ __launch_bounds__(256) void dump_merged_kernel(SrcMerge src, bf16_t *out)
{
    const int64_t row = blockIdx.x;
    const int D = src.D, K = 9 * D;
    const SrcMerge::Row rw = src.row(row);
    for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(src.addr(rw, k));
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        const int pos = k / D, c = k - pos * D;
#pragma unroll
        for (int j = 0; j < 8; ++j)   // channel-major column (c + j) * 9 + pos
            out[row * K + (int64_t)(c + j) * 9 + pos] =
                (bf16_t)((w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu);
    }
}

LoadPatch patch_loader(const uint8_t *px, const ImgDesc *imgs, int n_img, int64_t M,
                       const float *s3, const float *t3, int ps)
{
    return LoadPatch{px, imgs, n_img, M, ps, 3 * ps * ps, s3[0], s3[1], s3[2], t3[0], t3[1], t3[2]};
}

}  // namespace

hipError_t launch_patch_embed(const uint8_t *px, const ImgDesc *imgs, int n_img, int64_t M,
                              const float *s3, const float *t3, int ps, const bf16_t *Wpe,
                              int Kp, const bf16_t *bias, int D, bf16_t *patches, bf16_t *out,
                              const GemmWorkspace *ws, hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    if (Kp % 8 != 0 || Kp < 3 * ps * ps) return hipErrorInvalidValue;
    const LoadPatch al = patch_loader(px, imgs, n_img, M, s3, t3, ps);
    const int64_t threads = M * (Kp / 8);
    hipLaunchKernelGGL(patchify_kernel, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s, al,
                       patches, Kp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_linear(patches, M, Kp, Wpe, bias, D, ACT_NONE, false, out, ws, s);
}

hipError_t launch_dump_patches(const uint8_t *px, const ImgDesc *imgs, int n_img, int64_t M,
                               const float *s3, const float *t3, int ps, bf16_t *out,
                               hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    const LoadPatch al = patch_loader(px, imgs, n_img, M, s3, t3, ps);
    hipLaunchKernelGGL(dump_patches_kernel, dim3((unsigned)M), dim3(256), 0, s, al, out);
    return hipGetLastError();
}

hipError_t launch_dump_merged(const bf16_t *y, const ImgDesc *imgs, int n_img, int64_t Mtok,
                              int D, bf16_t *out, const bf16_t *zero, hipStream_t s)
{
    if (Mtok <= 0) return hipSuccess;
    SrcMerge src{y, imgs, n_img, Mtok, D, zero};
    hipLaunchKernelGGL(dump_merged_kernel, dim3((unsigned)Mtok), dim3(256), 0, s, src, out);
    return hipGetLastError();
}
