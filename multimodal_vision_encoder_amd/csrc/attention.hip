// Bidirectional flash attention over a packed multi-image batch (block-diagonal by image).
//
// Every patch attends to every patch of its own image and to nothing else ([Z] "Multimodal
// basics": attention gives each patch whole-image context; [L] DS4V: attention is
// bidirectional within each image's span).  Scale 1/sqrt(hd).
//
// One block = 4 waves x 32 queries of one head of one image.  Keys come in tiles of 64.
//
// Data movement: K and V^T tiles go global -> LDS with global_load_lds_dwordx4 (no register
// staging) into a 3-stage ring; the loads of tile t+2 are issued at the start of iteration
// t and waited for at its end, so one barrier per tile both publishes tile t+1 and frees the
// stage being refilled.  LDS rows are stored as XOR-swizzled 16-byte chunks so that the MFMA
// operand reads (ds_read_b128, 16 lanes per LDS pass) are free of bank conflicts.
//
// Per tile and wave:
//   S^T = K Q^T           v_mfma_f32_32x32x16_bf16 with K from LDS and Q^T in registers;
//                         the transpose puts one query per lane (column l%32), so the row
//                         max and sum need one cross-lane step (v_permlane32_swap).  S^T of tile t+1
//                         is issued before the softmax of tile t so the MFMA pipe runs while
//                         the VALU works.
//   online softmax        p = exp2(s * c - m * c), c = log2(e)/sqrt(hd): one FMA and one
//                         v_exp_f32 per score.  The running max m is raised only when a score
//                         exceeds it by more than 8 (log2 units) somewhere in the wave
//                         (wave-uniform branch), so the O rescale is skipped on almost every
//                         tile and p stays below 2^8.  P is packed to bf16 with
//                         v_cvt_pk_bf16_f32; the row sum is taken on those bf16 values with
//                         v_dot2c_f32_bf16, so numerator and denominator use the same weights.
//   O^T += V^T P^T        P^T is already in the B-operand layout of the S^T accumulator (the
//                         key order inside each 16-key chunk is permuted identically on both
//                         operands).
// Keys past the image end (last tile only) are masked to -inf; their loads are clamped to
// the image's last row.  Query rows past the image end are zero and never stored.
#include <math.h>

#include <type_traits>

#include "kernels.h"

namespace {

__device__ __forceinline__ int xcd_remap(int bid, int nb)
{
    const int per = nb >> 3;
    return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float dot2_bf16(uint32_t p, float acc)
{
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p), one, acc, false);
}

// 16-byte global -> LDS copy; lane l writes lds_base + 16 l (lds_base is wave-uniform).
__device__ __forceinline__ void load_lds16(const void *g, void *lds_base)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(0): every global load of this wave, including the LDS-bound ones, done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Value of x held by lane l ^ 32 (v_permlane32_swap exchanges the two wave halves).
__device__ __forceinline__ float xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

constexpr float kLazyRescale = 8.0f;   // log2 units
constexpr int kStages = 3;

template <int HD>
struct AttnGeom {
    static constexpr int HDP = HD < 32 ? 32 : HD;   // MFMA-padded head dim
    static constexpr int KCH = HDP / 8;             // 16-byte chunks per K row (one key)
    static constexpr int K_BYTES = 64 * HDP * 2;    // one K tile
    static constexpr int V_BYTES = HDP * 64 * 2;    // one V^T tile (rows = head dims)
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int KLOADS = 64 * KCH / 256;   // 16-byte loads per thread per K tile
    static constexpr int VLOADS = HDP * 8 / 256;
    // A ds_read_b128 is served 16 lanes at a time over 64 four-byte banks (256 bytes); rows
    // of K hold HDP*2 bytes, so 256/(HDP*2) rows share that window.  Chunk j of row r is
    // stored at j ^ kswz(r), which gives 16 consecutive rows distinct 16-byte slots.
    static constexpr int KRPW = 128 / HDP;          // K rows per 256-byte window
    __device__ static int kswz(int r) { return (r / KRPW) % KCH; }
    __device__ static int vswz(int r) { return (r >> 1) & 7; }   // V^T rows are 128 bytes
};

template <int HD>
__global__ __launch_bounds__(256, 2) void attention_kernel(
    const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ vt, int64_t ldv,
    bf16_t *__restrict__ o, const RowTile *__restrict__ work, int n_work,
    const ImgDesc *__restrict__ imgs, int D, int H, float c_log2)
{
    using G = AttnGeom<HD>;
    constexpr int HDP = G::HDP, KCH = G::KCH, KS = HDP / 16, DB = HDP / 32;
    static_assert(G::KLOADS >= 1 && G::VLOADS >= 1, "tile too small for 256 threads");
    __shared__ __attribute__((aligned(1024))) char smem[kStages * G::STAGE];

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

    // Issue the loads of key tile t into stage st.  Chunk c of a stage (lane-contiguous per
    // instruction) holds logical chunk (c % KCH) ^ (row % KCH) of its row.
    auto issue = [&](int t, int st) {
        char *sk = smem + st * G::STAGE, *sv = sk + G::K_BYTES;
        const int kv0 = t * 64;
#pragma unroll
        for (int i = 0; i < G::KLOADS; ++i) {
            const int c = (i * 4 + wave) * 64 + lane, r = c / KCH, s = (c % KCH) ^ G::kswz(r);
            const int key = min(kv0 + r, d.n - 1);
            const int dd = (s * 8) % HD;            // pad chunks (HD < 32) re-read real data
            load_lds16(kbase + (int64_t)key * ld + dd, sk + (i * 4 + wave) * 1024);
        }
#pragma unroll
        for (int i = 0; i < G::VLOADS; ++i) {
            const int c = (i * 4 + wave) * 64 + lane, r = c >> 3, s = (c & 7) ^ G::vswz(r);
            const int dd = r % HD;
            load_lds16(vbase + (int64_t)dd * ldv + kv0 + s * 8, sv + (i * 4 + wave) * 1024);
        }
    };

    auto qk = [&](int st, f32x16_t *s) {
        const char *sk = smem + st * G::STAGE;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = 32 * kb + l32, ch = (2 * kk + g) ^ G::kswz(row);
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(sk + row * (HDP * 2) + ch * 16);
                s[kb] = mfma32(a, qf[kk], s[kb]);
            }
    };

    f32x16_t oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;   // running max (raw score units) and sum

    // softmax of one tile's scores into bf16 P (pk[chunk][pair]); MASK on the last tile
    auto softmax = [&](f32x16_t *s, int kv0, uint32_t (*pk)[4], auto mask_tag) {
        if constexpr (decltype(mask_tag)::value) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= d.n) s[kb][r] = -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, xor32(mx));
        if (__ballot((mx - m_run) * c_log2 > kLazyRescale)) {   // wave-uniform
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2((m_run - m_new) * c_log2);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        }
        const float mc = m_run * c_log2;
        float ls = l_run;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kb = c >> 1, r = 8 * (c & 1) + 2 * j;
                const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], c_log2, -mc));
                const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c_log2, -mc));
                pk[c][j] = pack_bf16x2(p0, p1);
                ls = dot2_bf16(pk[c][j], ls);
            }
        l_run = ls;
    };

    // O^T += V^T P^T.  Chunk c covers keys 16c..16c+15; B-operand slot 8g+j <-> key
    // 16c + 8(j/4) + 4g + j%4, i.e. registers 8(c%2)+j of S^T block c/2.  The transposed-V
    // buffer stores each 16-key group with key bits 2 and 3 swapped, so those 8 keys are the
    // 16-byte chunk 2c+g of the row: one ds_read_b128 per operand.
    auto pv = [&](int st, uint32_t (*pk)[4]) {
        const char *sv = smem + st * G::STAGE + G::K_BYTES;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8_t pf = as_bf16x8(make_uint4(pk[c][0], pk[c][1], pk[c][2], pk[c][3]));
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const int row = 32 * b + l32;
                const bf16x8_t va = *reinterpret_cast<const bf16x8_t *>(
                    sv + row * 128 + (((2 * c + g) ^ G::vswz(row)) * 16));
                oacc[b] = mfma32(va, pf, oacc[b]);
            }
        }
    };

    const int nkv = (d.n + 63) / 64;
    const bool ragged = (d.n & 63) != 0;
    issue(0, 0);
    if (nkv > 1) issue(1, 1);
    wait_vmem();
    __syncthreads();
    // one key tile: cur holds S^T of tile t, next receives S^T of tile t+1
    auto step = [&](int t, f32x16_t *cur, f32x16_t *next) {
        // tile t+1 is in LDS and stage (t+2)%3 is free (everyone finished iteration t-1)
        if (t + 2 < nkv) issue(t + 2, (t + 2) % kStages);
        if (t + 1 < nkv) qk((t + 1) % kStages, next);
        uint32_t pk[4][4];
        if (ragged && t == nkv - 1) softmax(cur, t * 64, pk, std::true_type{});
        else softmax(cur, t * 64, pk, std::false_type{});
        pv(t % kStages, pk);
        wait_vmem();
        __syncthreads();
    };
    f32x16_t sa[2], sb[2];
    qk(0, sa);
    for (int t = 0; t < nkv; t += 2) {      // unrolled by two so the S^T buffers swap roles
        step(t, sa, sb);
        if (t + 1 < nkv) step(t + 1, sb, sa);
    }

    const float l_tot = l_run + xor32(l_run);
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
    const float c_log2 = (float)(1.4426950408889634 / sqrt((double)HD));
    hipLaunchKernelGGL(attention_kernel<HD>, dim3(grid), dim3(256), 0, s, qkv, vt, ldv, o, work,
                       n_work, imgs, D, H, c_log2);
    return hipGetLastError();
}

}  // namespace

int attention_q_tile() { return 128; }

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
