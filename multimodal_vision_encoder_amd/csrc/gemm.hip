// bf16 "NT" GEMM on gfx950 MFMA with a computing A loader:  C[m][n] = sum_k A[m][k] W[n][k] + b.
// Used for the patch projection, whose A operand (patchify + normalisation) is computed
// rather than copied; the plain linear layers and the projector use gemm_big.hip.
//
// Block tile BM x BN x 64, 256 threads as 2 x 2 waves; each wave owns a (BM/2) x (BN/2)
// sub-tile built from v_mfma_f32_32x32x16_bf16 blocks.  A and W tiles are staged through
// LDS (rows padded to 72 elements) with register double buffering: the global loads of
// K-tile t+1 are in flight while the MFMAs of tile t run.  The MFMA is issued with the W
// fragment as its first operand so that each lane ends up holding 4 consecutive output
// columns of one row, which the epilogue stores as one 8- or 16-byte write.
// The A operand comes from a loader (here the patchify gather of loaders.h).
#include "kernels.h"
#include "loaders.h"

namespace {

constexpr int BK = 64;
constexpr int LDSW = BK + 8;   // padded LDS row (bf16 elements)

// Blocks are dispatched round-robin over the 8 XCDs; give each XCD a contiguous range of
// tiles (the host rounds the grid up to a multiple of 8) so neighbouring tiles share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nb)
{
    const int per = nb >> 3;
    return (bid & 7) * per + (bid >> 3);
}

// GELU, tanh form, evaluated term by term with each product and sum rounded (no fused
// multiply-add), as written: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).
__device__ __forceinline__ float gelu_tanh(float u)
{
#pragma clang fp contract(off)
    const float k0 = 0.7978845608028654f, k1 = 0.044715f;
    float inner = __fmul_rn(k0, __fadd_rn(u, __fmul_rn(__fmul_rn(__fmul_rn(k1, u), u), u)));
    return __fmul_rn(__fmul_rn(0.5f, u), __fadd_rn(1.0f, tanhf(inner)));
}

template <int ACT>
struct EpiBF16 {
    bf16_t *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ void operator()(int64_t m, int n, const float *v) const
    {
        if (m >= M) return;
        float r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float x = v[j];
            if (bias && n + j < N) x = __fadd_rn(x, bf16_to_f32(bias[n + j]));
            if (ACT == ACT_GELU_TANH) x = gelu_tanh(x);
            r[j] = x;
        }
        bf16_t *o = out + m * N + n;
        if ((N & 3) == 0 && n + 3 < N) {
            *reinterpret_cast<uint2 *>(o) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n + j < N) o[j] = f32_to_bf16(r[j]);
        }
    }
};

struct EpiF32 {
    float *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ void operator()(int64_t m, int n, const float *v) const
    {
        if (m >= M) return;
        float r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = (bias && n + j < N) ? __fadd_rn(v[j], bf16_to_f32(bias[n + j])) : v[j];
        float *o = out + m * N + n;
        if ((N & 3) == 0 && n + 3 < N) {
            *reinterpret_cast<float4 *>(o) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n + j < N) o[j] = r[j];
        }
    }
};

template <int BM, int BN, class AL, class EP>
__global__ __launch_bounds__(256) void gemm_nt_kernel(AL al, const bf16_t *__restrict__ W,
                                                      int N, int K, EP ep, int tiles_m,
                                                      int tiles_n)
{
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDSW];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDSW];

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    if (L >= tiles_m * tiles_n) return;
    const int tm = L / tiles_n, tn = L - (L / tiles_n) * tiles_n;
    const int64_t m0 = (int64_t)tm * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    constexpr int AC = BM * BK / 8 / 256;   // 16-byte chunks per thread
    constexpr int BC = BN * BK / 8 / 256;
    uint4 ra[AC], rb[BC];

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int c = tid + i * 256, row = c >> 3, kc = (c & 7) * 8;
            ra[i] = al(m0 + row, k0 + kc);
        }
#pragma unroll
        for (int i = 0; i < BC; ++i) {
            const int c = tid + i * 256, row = c >> 3, kc = (c & 7) * 8;
            const int n = n0 + row;
            rb[i] = n < N ? *reinterpret_cast<const uint4 *>(W + (int64_t)n * K + k0 + kc)
                          : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int c = tid + i * 256, row = c >> 3, kc = (c & 7) * 8;
            *reinterpret_cast<uint4 *>(&sA[buf][row * LDSW + kc]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BC; ++i) {
            const int c = tid + i * 256, row = c >> 3, kc = (c & 7) * 8;
            *reinterpret_cast<uint4 *>(&sB[buf][row * LDSW + kc]) = rb[i];
        }
    };

    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8_t af[TM], bw[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t *>(
                    &sA[cur][(wm * WM + i * 32 + l32) * LDSW + ks * 16 + g * 8]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bw[j] = *reinterpret_cast<const bf16x8_t *>(
                    &sB[cur][(wn * WN + j * 32 + l32) * LDSW + ks * 16 + g * 8]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(bw[j], af[i], acc[i][j]);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // acc[i][j][r]: output row m = l32 of the 32-block, column 8*(r/4) + 4*g + r%4.
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                ep(m0 + wm * WM + i * 32 + l32, n0 + wn * WN + j * 32 + 8 * q + 4 * g, v);
            }
}

template <int BM, int BN, class AL, class EP>
hipError_t run_gemm(AL al, const bf16_t *W, int64_t M, int N, int K, EP ep, hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    const int tiles_m = (int)ceil_div(M, BM), tiles_n = (int)ceil_div(N, BN);
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int grid = (int)(ceil_div(tiles, 8) * 8);
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, AL, EP>), dim3(grid), dim3(256), 0, s, al, W, N, K,
                       ep, tiles_m, tiles_n);
    return hipGetLastError();
}

template <class AL>
hipError_t dispatch_epilogue(AL al, const bf16_t *W, int64_t M, int N, int K, const bf16_t *bias,
                             int act, bool out_f32, void *out, hipStream_t s)
{
    if (out_f32) return run_gemm<128, 128>(al, W, M, N, K, EpiF32{(float *)out, bias, M, N}, s);
    if (act == ACT_GELU_TANH)
        return run_gemm<128, 128>(al, W, M, N, K,
                                  EpiBF16<ACT_GELU_TANH>{(bf16_t *)out, bias, M, N}, s);
    return run_gemm<128, 128>(al, W, M, N, K, EpiBF16<ACT_NONE>{(bf16_t *)out, bias, M, N}, s);
}

}  // namespace

hipError_t launch_patch_embed(const uint8_t *px, const ImgDesc *imgs, int n_img, int64_t M,
                              const float *s3, const float *t3, int ps, const bf16_t *Wpe,
                              int Kp, const bf16_t *bias, int D, bf16_t *out, hipStream_t s)
{
    LoadPatch al{px, imgs, n_img, M, ps, 3 * ps * ps, s3[0], s3[1], s3[2], t3[0], t3[1], t3[2]};
    return dispatch_epilogue(al, Wpe, M, D, Kp, bias, ACT_NONE, false, out, s);
}

// ---------------------------------------------------------------------------------------
// Debug dumps through the same loaders.
// ---------------------------------------------------------------------------------------
namespace {

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

}  // namespace

hipError_t launch_dump_patches(const uint8_t *px, const ImgDesc *imgs, int n_img, int64_t M,
                               const float *s3, const float *t3, int ps, bf16_t *out,
                               hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    LoadPatch al{px, imgs, n_img, M, ps, 3 * ps * ps, s3[0], s3[1], s3[2], t3[0], t3[1], t3[2]};
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
