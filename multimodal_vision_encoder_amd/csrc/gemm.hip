// Debug materialisation of the tensors that exist only inside fused loaders: the patch
// matrix (patchify runs inside the patch projection's A loader, SrcPatch) and the merged
// projector input (the 3x3 gather inside the projector's A loader, SrcMerge).  Both go
// through the loaders' own device functions, so a dump is exactly what the GEMM consumed.
#include "kernels.h"
#include "loaders.h"

namespace {

// One thread per (patch, 8-column chunk of the loader's K order); the valid values are
// written at their (channel, y, x) column c ps^2 + y ps + x ([Z] "Step 1").
__global__ __launch_bounds__(256) void dump_patches_kernel(SrcPatch src, int kchunks, bf16_t *out)
{
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= src.M * kchunks) return;
    const int64_t row = w / kchunks;
    const int k = (int)(w - row * kchunks) * 8;
    const SrcPatch::Row rw = src.row(row);
    const SrcPatch::KChunk kc = src.chunk(k, src.consts());
    const uint4 v = src.convert(kc, src.load(rw, kc));
    const uint32_t h[4] = {v.x, v.y, v.z, v.w};
    const int ps = src.ps, pp = ps * ps;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (e >= kc.nv) break;
        const int b = kc.b0 + e, x = b / 3, c = b - 3 * x;
        out[(src.m_base + row) * 3 * pp + c * pp + kc.yc * ps + x] = (bf16_t)((h[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
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

}  // namespace

hipError_t launch_dump_patches(const uint8_t *lpx, int64_t pix_first, int64_t pix_bytes, const ImgDesc *imgs,
                               int n_img, int64_t m_first, int64_t M, const float *s3, const float *t3, int ps,
                               bf16_t *out, hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    if (ps > 64 || pix_bytes <= 0 || pix_bytes >= kPatchLaunchBytes) return hipErrorInvalidValue;
    const int kchunks = patch_gemm_k(ps) / 8;
    const int64_t threads = M * kchunks;
    hipLaunchKernelGGL(dump_patches_kernel, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s,
                       patch_source(lpx, pix_first, pix_bytes, imgs, n_img, m_first, M, s3, t3, ps), kchunks, out);
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
