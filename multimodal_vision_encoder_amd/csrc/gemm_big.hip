// Large-tile bf16 "NT" GEMM on gfx950 MFMA:  C[m][n] = epilogue(sum_k A[m][k] W[n][k]).
//
// Block tile BM x BN x 64 with 4 waves as 2 x 2; each wave owns a (BM/2) x (BN/2) tile of
// v_mfma_f32_32x32x16_bf16 blocks (128 x 128 at BM = BN = 256: 256 fp32 accumulators per
// lane, which the compiler keeps in the accumulation registers).  A and W tiles move global ->
// LDS with global_load_lds_dwordx4 (no register staging) into a 2-stage ring: the loads of
// k-tile t+1 are issued before the MFMAs of k-tile t and waited for after them, so one
// barrier per k-tile both publishes the next tile and frees the stage being refilled.  LDS
// rows are 64 bf16 (8 chunks of 16 bytes) with chunk j of row r stored at j ^ ((r / 2) % 8),
// so the operand reads of 16 consecutive rows hit distinct banks.  Each lane reads one 16-byte
// chunk per MFMA operand (ds_read_b128).  The MFMA is issued with the W fragment first so
// each lane holds 4 consecutive output columns of one row for the epilogue.
//
// The A rows come from an address source: plain row-major activations, or the 3x3 merge
// gather of the projector ([Z] "Step 4"), where positions in the right/bottom zero padding
// read from a zero page.  Rows past M are clamped to row M-1 and never stored.
#include "kernels.h"
#include "loaders.h"

namespace {

constexpr int BK = 64;

__device__ __forceinline__ int xcd_remap(int bid, int nb)
{
    const int per = nb >> 3;
    return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ void load_lds16(const void *g, void *lds_base)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS chunk swizzle of a 128-byte row: a ds_read_b128 is served 16 lanes at a time over 64
// four-byte banks (256 bytes), i.e. over two consecutive rows; XOR-ing the chunk index with
// (row / 2) % 8 gives 16 consecutive rows 16 distinct 16-byte slots of that window.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int ACT>
struct EpiBF16 {
    bf16_t *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ void operator()(int64_t m, int n, const float *v) const;
    __device__ __forceinline__ void full(int64_t m, int n, const float *v) const;
};

// GELU, tanh form: 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3), evaluated through
// the identity 0.5 (1 + tanh(z)) = 1 / (1 + e^(-2z)) with one v_exp_f32 (base 2) and one
// v_rcp_f32: gelu(u) = u / (1 + 2^(u (c1 + c2 u^2))), c1 = -2 sqrt(2/pi) log2(e),
// c2 = 0.044715 c1.  Large |u| saturate correctly (2^+inf -> u * 0, 2^-inf -> u).
__device__ __forceinline__ float gelu_tanh_big(float u)
{
    const float c1 = -2.3022082037717294f, c2 = -0.10294324161187608f;
    const float t = u * u;
    const float e = __builtin_amdgcn_exp2f(u * __builtin_fmaf(c2, t, c1));
    return u * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int ACT>
__device__ __forceinline__ void epi_bf16_full(bf16_t *out, const bf16_t *bias, int64_t m, int N, int n,
                                              const float *v)
{
    float r[4];
    if (bias) {
        const uint2 b = *reinterpret_cast<const uint2 *>(bias + n);
        r[0] = v[0] + __uint_as_float(b.x << 16);
        r[1] = v[1] + __uint_as_float(b.x & 0xFFFF0000u);
        r[2] = v[2] + __uint_as_float(b.y << 16);
        r[3] = v[3] + __uint_as_float(b.y & 0xFFFF0000u);
    } else {
        r[0] = v[0], r[1] = v[1], r[2] = v[2], r[3] = v[3];
    }
    if (ACT == ACT_GELU_TANH)
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = gelu_tanh_big(r[j]);
    *reinterpret_cast<uint2 *>(out + m * N + n) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
}

template <int ACT>
__device__ __forceinline__ void EpiBF16<ACT>::operator()(int64_t m, int n, const float *v) const
{
    if (m >= M) return;
    float r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float x = v[j];
        if (bias && n + j < N) x = x + bf16_to_f32(bias[n + j]);
        if (ACT == ACT_GELU_TANH) x = gelu_tanh_big(x);
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

template <int ACT>
__device__ __forceinline__ void EpiBF16<ACT>::full(int64_t m, int n, const float *v) const
{
    epi_bf16_full<ACT>(out, bias, m, N, n, v);
}

struct EpiF32 {
    float *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ void full(int64_t m, int n, const float *v) const
    {
        float4 r = make_float4(v[0], v[1], v[2], v[3]);
        if (bias) {
            const uint2 b = *reinterpret_cast<const uint2 *>(bias + n);
            r.x += __uint_as_float(b.x << 16);
            r.y += __uint_as_float(b.x & 0xFFFF0000u);
            r.z += __uint_as_float(b.y << 16);
            r.w += __uint_as_float(b.y & 0xFFFF0000u);
        }
        *reinterpret_cast<float4 *>(out + m * N + n) = r;
    }
    __device__ __forceinline__ void operator()(int64_t m, int n, const float *v) const
    {
        if (m >= M) return;
        float r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (bias && n + j < N) ? v[j] + bf16_to_f32(bias[n + j]) : v[j];
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

template <int BM, int BN, int NWM, int NWN, class SRC, class EP>
__global__ __launch_bounds__(64 * NWM * NWN, 1) void gemm_big_kernel(SRC src, const bf16_t *__restrict__ W,
                                                          int N, int K, EP ep, int tiles_m,
                                                          int tiles_n)
{
    constexpr int NT = 64 * NWM * NWN, NW = NWM * NWN;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
    constexpr int AL = BM * 8 / NT, BL = BN * 8 / NT;     // 16-byte loads per thread
    constexpr int WM = BM / NWM, WN = BN / NWN, TM = WM / 32, TN = WN / 32;
    static_assert(AL >= 1 && BL >= 1 && TM >= 1 && TN >= 1, "bad tile");
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    if (L >= tiles_m * tiles_n) return;
    const int tm = L / tiles_n, tn = L - tm * tiles_n;
    const int64_t m0 = (int64_t)tm * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    // rows this thread loads (fixed over the K loop); chunk c = (i*NW + wave)*64 + lane
    typename SRC::Row arow[AL];
    int aslot[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int c = (i * NW + wave) * 64 + lane, r = c >> 3;
        arow[i] = src.row(m0 + r);
        aslot[i] = ((c & 7) ^ swz(r)) * 8;
    }
    const bf16_t *wrow[BL];
    int wslot[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int c = (i * NW + wave) * 64 + lane, r = c >> 3;
        const int n = n0 + r < N ? n0 + r : N - 1;
        wrow[i] = W + (int64_t)n * K;
        wslot[i] = ((c & 7) ^ swz(r)) * 8;
    }
    auto issue = [&](int kt, int st) {
        char *sa = smem + st * STAGE, *sb = sa + A_BYTES;
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < AL; ++i) load_lds16(src.addr(arow[i], k0 + aslot[i]), sa + (i * NW + wave) * 1024);
#pragma unroll
        for (int i = 0; i < BL; ++i) load_lds16(wrow[i] + k0 + wslot[i], sb + (i * NW + wave) * 1024);
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int wm = wave / NWN, wn = wave % NWN;
    const int nk = K / BK;
    issue(0, 0);
    wait_vmem();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
        const char *sa = smem + cur * STAGE, *sb = sa + A_BYTES;
        // operand fragments double-buffered across the four 16-wide k-steps: the reads of
        // step ks+1 are in flight while the MFMAs of step ks run
        bf16x8_t af[2][TM], bw[2][TN];
        auto ldfrag = [&](int ks, int buf) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WM + i * 32 + l32;
                af[buf][i] = *reinterpret_cast<const bf16x8_t *>(sa + r * 128 + (((2 * ks + g) ^ swz(r)) * 16));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WN + j * 32 + l32;
                bw[buf][j] = *reinterpret_cast<const bf16x8_t *>(sb + r * 128 + (((2 * ks + g) ^ swz(r)) * 16));
            }
        };
        ldfrag(0, 0);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            if (ks + 1 < BK / 16) ldfrag(ks + 1, (ks + 1) & 1);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(bw[ks & 1][j], af[ks & 1][i], acc[i][j]);
        }
        wait_vmem();
        __syncthreads();
    }

    // acc[i][j][r]: output row l32 of the 32-block, column 8*(r/4) + 4*g + r%4.
    const bool full = m0 + BM <= ep.M && n0 + BN <= N && (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                const int64_t m = m0 + wm * WM + i * 32 + l32;
                const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * g;
                if (full) ep.full(m, n, v);
                else ep(m, n, v);
            }
}

#ifndef VIT_GEMM_NWM
#define VIT_GEMM_NWM 4
#endif

template <int BM, int BN, class SRC, class EP>
hipError_t run_big(SRC src, const bf16_t *W, int64_t M, int N, int K, EP ep, hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    constexpr int NWM = VIT_GEMM_NWM, NWN = 2;
    const int tiles_m = (int)ceil_div(M, BM), tiles_n = (int)ceil_div(N, BN);
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int grid = (int)(ceil_div(tiles, 8) * 8);
    hipLaunchKernelGGL((gemm_big_kernel<BM, BN, NWM, NWN, SRC, EP>), dim3(grid), dim3(64 * NWM * NWN),
                       0, s, src, W, N, K, ep, tiles_m, tiles_n);
    return hipGetLastError();
}

template <class SRC>
hipError_t dispatch(SRC src, const bf16_t *W, int64_t M, int N, int K, const bf16_t *bias, int act,
                    bool out_f32, void *out, hipStream_t s)
{
    // 256 x 256 tiles when they give at least one full wave of blocks, else 256 x 128
    const int64_t big_tiles = ceil_div(M, 256) * ceil_div(N, 256);
    const bool big = big_tiles >= 256;
    if (out_f32)
        return big ? run_big<256, 256>(src, W, M, N, K, EpiF32{(float *)out, bias, M, N}, s)
                   : run_big<256, 128>(src, W, M, N, K, EpiF32{(float *)out, bias, M, N}, s);
    if (act == ACT_GELU_TANH) {
        EpiBF16<ACT_GELU_TANH> ep{(bf16_t *)out, bias, M, N};
        return big ? run_big<256, 256>(src, W, M, N, K, ep, s) : run_big<256, 128>(src, W, M, N, K, ep, s);
    }
    EpiBF16<ACT_NONE> ep{(bf16_t *)out, bias, M, N};
    return big ? run_big<256, 256>(src, W, M, N, K, ep, s) : run_big<256, 128>(src, W, M, N, K, ep, s);
}

}  // namespace

hipError_t launch_linear(const bf16_t *A, int64_t M, int K, const bf16_t *W, const bf16_t *bias,
                         int N, int act, bool out_f32, void *out, hipStream_t s)
{
    return dispatch(SrcPlain{A, K, M}, W, M, N, K, bias, act, out_f32, out, s);
}

hipError_t launch_merge_project(const bf16_t *y, const ImgDesc *imgs, int n_img, int64_t Mtok,
                                int D, const bf16_t *Wp, const bf16_t *bias, int Dl, float *out,
                                const bf16_t *zero, hipStream_t s)
{
    return dispatch(SrcMerge{y, imgs, n_img, Mtok, D, zero}, Wp, Mtok, Dl, 9 * D, bias, ACT_NONE,
                    true, out, s);
}
