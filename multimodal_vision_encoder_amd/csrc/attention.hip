// Bidirectional flash attention over a packed multi-image batch (block-diagonal by image).
//
// Every patch attends to every patch of its own image and to nothing else ([Z] "Multimodal
// basics": attention gives each patch whole-image context; [L] DS4V: attention is
// bidirectional within each image's span).  Scale 1/sqrt(hd).
//
// One block = one (128-query tile of one image, head); 4 waves x 32 queries.  Per 64-key
// tile:
//   S^T = K Q^T           v_mfma_f32_32x32x16_bf16, K tile from LDS, Q^T kept in registers;
//                         computing the transpose puts one query per lane (column l%32), so
//                         the row max and row sum need only one cross-lane step (lane ^ 32).
//   online softmax        log2 domain (scale * log2 e folded into one multiply), running max
//                         and sum per query in fp32, P rounded to bf16 for the next MFMA.
//   O^T += V^T P^T        P^T is already in the B-operand layout of the S^T accumulator (the
//                         key order inside each 16-key chunk is permuted identically on both
//                         operands); V^T comes from LDS, staged from the transposed-V buffer.
// K and V^T tiles are double-buffered through LDS with the next tile's global loads in
// flight during the current tile's MFMAs.  Keys past the image end are masked to -inf;
// rows past the image end are loaded as zeros and never stored.
#include <math.h>

#include "kernels.h"

namespace {

__device__ __forceinline__ int xcd_remap(int bid, int nb)
{
    const int per = nb >> 3;
    return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int HD>
__global__ __launch_bounds__(256) void attention_kernel(
    const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ vt, int64_t ldv,
    bf16_t *__restrict__ o, const RowTile *__restrict__ work, int n_work,
    const ImgDesc *__restrict__ imgs, int D, int H, float scale_log2)
{
    constexpr int HDP = HD < 32 ? 32 : HD;   // MFMA-padded head dim
    constexpr int KS = HDP / 16;             // k-steps of S^T = K Q^T
    constexpr int DB = HDP / 32;             // 32-row blocks of O^T
    constexpr int KLD = HDP + 8;             // LDS row of K (bf16 elements)
    constexpr int VLD = 64 + 8;              // LDS row of V^T
    constexpr int KC = 64 * HDP / 8 / 256;   // 16-byte chunks per thread, K tile
    constexpr int VC = HDP * 64 / 8 / 256;   // same, V^T tile
    static_assert(KC >= 1 && VC >= 1, "tile too small for 256 threads");

    __shared__ __attribute__((aligned(16))) bf16_t Ks[2][64 * KLD];
    __shared__ __attribute__((aligned(16))) bf16_t Vs[2][HDP * VLD];

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    if (L >= n_work * H) return;
    const int head = L / n_work, wi = L - head * n_work;
    const RowTile wt = work[wi];
    const ImgDesc d = imgs[wt.img];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)D;
    const bf16_t *qbase = qkv + (int64_t)d.patch_off * ld + head * HD;
    const bf16_t *kbase = qbase + D;
    const bf16_t *vbase = vt + (int64_t)head * HD * ldv + d.vt_off;

    const int q = wt.r0 + wave * 32 + l32;   // this lane's query (local row)
    bf16x8_t qf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const int dd = 16 * kk + 8 * g;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (q < d.n && dd < HD) v = *reinterpret_cast<const uint4 *>(qbase + (int64_t)q * ld + dd);
        qf[kk] = as_bf16x8(v);
    }

    uint4 rk[KC], rv[VC];
    auto gload = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int c = tid + i * 256, key = c / (HDP / 8), dc = (c % (HDP / 8)) * 8;
            rk[i] = (kv0 + key < d.n && dc < HD)
                        ? *reinterpret_cast<const uint4 *>(kbase + (int64_t)(kv0 + key) * ld + dc)
                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VC; ++i) {
            const int c = tid + i * 256, dd = c >> 3, kc = (c & 7) * 8;
            rv[i] = dd < HD ? *reinterpret_cast<const uint4 *>(vbase + (int64_t)dd * ldv + kv0 + kc)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int c = tid + i * 256, key = c / (HDP / 8), dc = (c % (HDP / 8)) * 8;
            *reinterpret_cast<uint4 *>(&Ks[buf][key * KLD + dc]) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < VC; ++i) {
            const int c = tid + i * 256, dd = c >> 3, kc = (c & 7) * 8;
            *reinterpret_cast<uint4 *>(&Vs[buf][dd * VLD + kc]) = rv[i];
        }
    };

    f32x16_t oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int nkv = (d.n + 63) / 64;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int t = 0; t < nkv; ++t) {
        const int cur = t & 1, kv0 = t * 64;
        if (t + 1 < nkv) gload(kv0 + 64);

        // S^T[key][query] for 64 keys (two 32-key blocks)
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
                    &Ks[cur][(32 * kb + l32) * KLD + 16 * kk + 8 * g]);
                s[kb] = mfma32(a, qf[kk], s[kb]);
            }

        // online softmax for query l32 (lanes l and l^32 hold its two key halves)
        float mt = -INFINITY;
        const bool tail = kv0 + 64 > d.n;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[kb][r] * scale_log2;
                if (tail) {
                    const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= d.n) x = -INFINITY;
                }
                s[kb][r] = x;
                mt = fmaxf(mt, x);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(s[kb][r] - m_new);
                s[kb][r] = p;
                ls += p;
            }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;

        // P^T as B operand: chunk c covers keys 16c..16c+15; slot 8g+j <-> key
        // 16c + 8(j/4) + 4g + j%4, i.e. registers 8(c%2)+j of block c/2.
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int kb = c >> 1, r0 = 8 * (c & 1);
            uint4 pw;
            pw.x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
            pw.y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
            pw.z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
            pw.w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
            const bf16x8_t pf = as_bf16x8(pw);
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const bf16_t *vr = &Vs[cur][(32 * b + l32) * VLD + 16 * c + 4 * g];
                const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 8);
                oacc[b] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pf, oacc[b]);
            }
        }

        if (t + 1 < nkv) sstore(cur ^ 1);
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    if (q < d.n) {
        bf16_t *orow = o + ((int64_t)d.patch_off + q) * D + head * HD;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int dd = 32 * b + 8 * grp + 4 * g;
                if (dd < HD) {
                    const float a0 = oacc[b][4 * grp] * inv, a1 = oacc[b][4 * grp + 1] * inv,
                                a2 = oacc[b][4 * grp + 2] * inv, a3 = oacc[b][4 * grp + 3] * inv;
                    *reinterpret_cast<uint2 *>(orow + dd) =
                        make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
                }
            }
    }
}

template <int HD>
hipError_t run_attention(const bf16_t *qkv, const bf16_t *vt, int64_t ldv, bf16_t *o,
                         const RowTile *work, int n_work, const ImgDesc *imgs, int D, int H,
                         hipStream_t s)
{
    const int64_t total = (int64_t)n_work * H;
    const int grid = (int)(ceil_div(total, 8) * 8);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)HD));
    hipLaunchKernelGGL(attention_kernel<HD>, dim3(grid), dim3(256), 0, s, qkv, vt, ldv, o, work,
                       n_work, imgs, D, H, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const bf16_t *qkv, const bf16_t *vt, int64_t ldv, bf16_t *o,
                            const RowTile *work, int n_work, const ImgDesc *imgs, int D, int H,
                            hipStream_t s)
{
    if (n_work <= 0) return hipSuccess;
    switch (D / H) {
    case 16: return run_attention<16>(qkv, vt, ldv, o, work, n_work, imgs, D, H, s);
    case 32: return run_attention<32>(qkv, vt, ldv, o, work, n_work, imgs, D, H, s);
    case 64: return run_attention<64>(qkv, vt, ldv, o, work, n_work, imgs, D, H, s);
    case 128: return run_attention<128>(qkv, vt, ldv, o, work, n_work, imgs, D, H, s);
    default: return hipErrorInvalidValue;
    }
}
