// Bidirectional flash attention over a packed multi-image batch (block-diagonal by image).
//
// Every patch attends to every patch of its own image and to nothing else ([Z] "Multimodal
// basics": attention gives each patch whole-image context; [L] DS4V: attention is
// bidirectional within each image's span).  Scale 1/sqrt(hd).
//
// One block = 4 waves x 32 queries of one head of one image.  Keys come in tiles of 64.
//
// Data movement: K and V^T tiles go global -> LDS with global_load_lds_dwordx4 (no register
// staging) into two rings of 3 stages each (48 KB per block).  K of a tile is read one
// iteration before its V^T, so iteration t issues K of tile t+3 and V^T of tile t+2 and,
// before its closing barrier, waits only for the copies of the previous iteration: every copy
// has two iterations to land.  The copies are written as inline assembly (scalar base,
// 32-bit per-lane offset, fixed for all tiles) so the compiler neither inserts its
// conservative wait-for-all-copies before LDS reads nor recomputes addresses per tile; the
// barrier is a bare s_barrier for the same reason (the fence in __syncthreads waits for every
// copy).
// LDS rows are stored as XOR-swizzled 16-byte chunks so that the MFMA operand reads
// (ds_read_b128, 16 lanes per LDS pass) are free of bank conflicts.
//
// Per tile and wave:
//   S^T = K Q^T           v_mfma_f32_32x32x16_bf16 with K from LDS and Q^T in registers;
//                         the transpose puts one query per lane (column l%32), so the row
//                         max and sum need one cross-lane step (v_permlane32_swap).  S^T of
//                         tile t+1 and its row max are computed in iteration t, next to the
//                         softmax and P V of tile t, so the MFMA pipe runs while the VALU works.
//   online softmax        p = exp2(s * c - m * c), c = log2(e)/sqrt(hd): one FMA and one
//                         v_exp_f32 per score.  The running max m is raised only when a score
//                         exceeds it by more than 8 (log2 units) somewhere in the wave
//                         (wave-uniform branch at the top of the iteration), so the O rescale
//                         is skipped on almost every tile and p stays below 2^8.  P is packed
//                         to binary16 with v_cvt_pkrtz_f16_f32 (relative error below 2^-10,
//                         eight times finer than bf16: with near-uniform attention the output
//                         is a small average of large values, and bf16 weights alone would
//                         flip about a third of the bf16-rounded outputs); the row sum is
//                         taken on those same values with v_dot2c_f32_f16, so numerator and
//                         denominator use the same weights.
//   O^T += V^T P^T        v_mfma_f32_32x32x16_f16 on the binary16 V^T written by the RoPE
//                         kernel.  P^T is already in the B-operand layout of the S^T
//                         accumulator (the key order inside each 16-key chunk is permuted
//                         identically on both operands).
// Keys past the image end (last tile only) are masked to -inf; their loads are clamped to
// the image's last row.  Query rows past the image end are zero and never stored.  Past the
// last tile the ring is refilled with copies of the last tile, whose scores are computed and
// ignored, so the loop body has no tile-count branches.
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

// Two fp32 -> two binary16 in one v_cvt_pkrtz_f16_f32 (round toward zero); lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_f16x2_rtz(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// acc + (sum of the two binary16 halves of p), v_dot2c_f32_f16.
__device__ __forceinline__ float dot2_f16(uint32_t p, float acc)
{
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p), one, acc, false);
}

// 16-byte global -> LDS copy of base + off (base wave-uniform); lane l writes LDS byte address
// lds + 16 l (lds wave-uniform).  Inline assembly, so the compiler's wait-count insertion does
// not see an LDS write (it would wait for every outstanding copy before each LDS read); the
// kernel waits for its copies itself before each barrier.  m0 needs one wait state before the
// copy reads it.
__device__ __forceinline__ void load_lds16(const void *base, uint32_t off, uint32_t lds)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    // each half widened as unsigned: a signed low half would sign-extend into the high word
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
    __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     ::"v"(off), "s"(ub), "s"(lds) : "memory", "m0");
}

// s_waitcnt vmcnt(0): every global load of this wave, including the LDS-bound ones, done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N) lgkmcnt(0): all but this wave's newest N global loads done, LDS reads done.
template <int N>
__device__ __forceinline__ void wait_vmem_n()
{
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}
// Workgroup barrier without the memory-model fence of __syncthreads (whose release would wait
// for every outstanding global->LDS load); the callers wait for what they need first.
__device__ __forceinline__ void bare_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }

// Value of x held by lane l ^ 32 (v_permlane32_swap exchanges the two wave halves).
__device__ __forceinline__ float xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

constexpr float kLazyRescale = 8.0f;   // log2 units

template <int HD>
struct AttnGeom {
    static constexpr int HDP = HD < 32 ? 32 : HD;   // MFMA-padded head dim
    static constexpr int KCH = HDP / 8;             // 16-byte chunks per K row (one key)
    static constexpr int K_BYTES = 64 * HDP * 2;    // one K tile
    static constexpr int V_BYTES = HDP * 64 * 2;    // one V^T tile (rows = head dims)
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
    // separate rings for K (3 stages) and V^T (3 stages): K of tile t+1 is read one step
    // before V^T of tile t+1
    __shared__ __attribute__((aligned(1024))) char kst[3 * G::K_BYTES];
    __shared__ __attribute__((aligned(1024))) char vst[3 * G::V_BYTES];
    auto kstage = [&](auto st) -> char * { return kst + decltype(st)::value * G::K_BYTES; };
    auto vstage = [&](auto st) -> char * { return vst + decltype(st)::value * G::V_BYTES; };
    auto lds_addr = [&](const char *p) -> uint32_t {
        return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
    };

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    if (L >= n_work * H) return;
    const int head = L / n_work, wi = L - head * n_work;
    const RowTile wt = work[wi];
    const ImgDesc d = imgs[wt.img];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // Copies of key tile t into a stage.  Chunk c of a stage (lane-contiguous per instruction)
    // holds logical chunk (c % KCH) ^ kswz(row) of its row (V^T: ^ vswz(row)).  The per-lane
    // byte offsets are the same for every tile: a tile's copies are one scalar base plus these.
    uint32_t koff[G::KLOADS], voff[G::VLOADS];
    int krow[G::KLOADS], kdd[G::KLOADS];
#pragma unroll
    for (int i = 0; i < G::KLOADS; ++i) {
        const int c = (i * 4 + wave) * 64 + lane, r = c / KCH, s = (c % KCH) ^ G::kswz(r);
        krow[i] = r;
        kdd[i] = (s * 8) % HD;                      // pad chunks (HD < 32) re-read real data
        koff[i] = (uint32_t)(r * (int)ld + kdd[i]) * 2u;
    }
#pragma unroll
    for (int i = 0; i < G::VLOADS; ++i) {
        const int c = (i * 4 + wave) * 64 + lane, r = c >> 3, s = (c & 7) ^ G::vswz(r);
        voff[i] = (uint32_t)((int64_t)(r % HD) * ldv + s * 8) * 2u;
    }
    auto issue_k = [&](int t, auto st) {
        const uint32_t sk = lds_addr(kstage(st));
        const int kv0 = t * 64;
        const bf16_t *kb = kbase + (int64_t)kv0 * ld;
        if (kv0 + 64 <= d.n) {
#pragma unroll
            for (int i = 0; i < G::KLOADS; ++i) load_lds16(kb, koff[i], sk + (i * 4 + wave) * 1024);
        } else {   // last tile of a ragged image: rows past the end re-read its last row
#pragma unroll
            for (int i = 0; i < G::KLOADS; ++i) {
                const int r = min(krow[i], d.n - 1 - kv0);
                load_lds16(kb, (uint32_t)(r * (int)ld + kdd[i]) * 2u, sk + (i * 4 + wave) * 1024);
            }
        }
    };
    auto issue_v = [&](int t, auto st) {
        const uint32_t sv = lds_addr(vstage(st));
        const bf16_t *vb = vbase + t * 64;
#pragma unroll
        for (int i = 0; i < G::VLOADS; ++i) load_lds16(vb, voff[i], sv + (i * 4 + wave) * 1024);
    };

    // S^T of one tile: all K fragments are read from LDS first, then the MFMAs run
    auto qk = [&](auto st, f32x16_t *s) {
        const char *sk = kstage(st);
        bf16x8_t a[KS][2];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = 32 * kb + l32, ch = (2 * kk + g) ^ G::kswz(row);
                a[kk][kb] = *reinterpret_cast<const bf16x8_t *>(sk + row * (HDP * 2) + ch * 16);
            }
        const f32x16_t z = {};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(a[kk][kb], qf[kk], kk == 0 ? z : s[kb]);
    };

    f32x16_t oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;   // running max (raw score units) and sum

    auto mask_tile = [&](f32x16_t *s, int kv0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                if (key >= d.n) s[kb][r] = -INFINITY;
            }
    };
    auto tile_max = [&](const f32x16_t *s) {
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        return fmaxf(mx, xor32(mx));
    };

    // O^T += V^T P^T.  Chunk c covers keys 16c..16c+15; B-operand slot 8g+j <-> key
    // 16c + 8(j/4) + 4g + j%4, i.e. registers 8(c%2)+j of S^T block c/2.  The transposed-V
    // buffer stores each 16-key group with key bits 2 and 3 swapped, so those 8 keys are the
    // 16-byte chunk 2c+g of the row: one ds_read_b128 per operand.
    auto pv = [&](auto st, uint32_t (*pk)[4]) {
        const char *sv = vstage(st);
        f16x8_t va[4][DB];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const int row = 32 * b + l32;
                va[c][b] = *reinterpret_cast<const f16x8_t *>(sv + row * 128 + (((2 * c + g) ^ G::vswz(row)) * 16));
            }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f16x8_t pf = as_f16x8(make_uint4(pk[c][0], pk[c][1], pk[c][2], pk[c][3]));
#pragma unroll
            for (int b = 0; b < DB; ++b) oacc[b] = mfma32_f16(va[c][b], pf, oacc[b]);
        }
    };

    const int nkv = (d.n + 63) / 64;
    const bool ragged = (d.n & 63) != 0;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    // prologue: K of tiles 0..2, V^T of tiles 0..1; wait for K 0, V^T 0 and K 1
    issue_k(0, I0{});
    issue_v(0, I0{});
    issue_k(min(1, nkv - 1), I1{});
    issue_v(min(1, nkv - 1), I1{});
    issue_k(min(2, nkv - 1), I2{});
    wait_vmem_n<G::KLOADS + G::VLOADS>();
    bare_barrier();
    // One key tile: issue K of tile t+3 and V^T of tile t+2 (into the stages of K t and V^T t-1,
    // whose last readers were iterations t-1), S^T of tile t+1, softmax and P.V of tile t; then
    // wait for this wave's copies of the previous iteration (K t+2, V^T t+1) and publish them.
    // cur holds S^T of tile t and mx its row max; past the last tile the copies and S^T repeat
    // the last tile and are ignored.
    auto step = [&](int t, auto st, f32x16_t *cur, f32x16_t *next, float &mx) {
        constexpr int S = decltype(st)::value;
        using KQ = std::integral_constant<int, (S + 1) % 3>;   // K of tile t+1
        using KD = std::integral_constant<int, S % 3>;         // K of tile t+3
        using VP = std::integral_constant<int, S % 3>;         // V^T of tile t
        using VD = std::integral_constant<int, (S + 2) % 3>;   // V^T of tile t+2
        if (__ballot((mx - m_run) * c_log2 > kLazyRescale)) {   // wave-uniform, rare
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
        issue_k(min(t + 3, nkv - 1), KD{});
        issue_v(min(t + 2, nkv - 1), VD{});
        qk(KQ{}, next);
        uint32_t pk[4][4];
        float ls0 = l_run, ls1 = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kb = c >> 1, r = 8 * (c & 1) + 2 * j;
                const float p0 = fast_exp2(__builtin_fmaf(cur[kb][r], c_log2, -mc));
                const float p1 = fast_exp2(__builtin_fmaf(cur[kb][r + 1], c_log2, -mc));
                pk[c][j] = pack_f16x2_rtz(p0, p1);
                if (j & 1) ls1 = dot2_f16(pk[c][j], ls1);
                else ls0 = dot2_f16(pk[c][j], ls0);
            }
        l_run = ls0 + ls1;
        pv(VP{}, pk);
        if (ragged && t + 1 == nkv - 1) mask_tile(next, (t + 1) * 64);
        mx = tile_max(next);
        wait_vmem_n<G::KLOADS + G::VLOADS>();
        bare_barrier();
    };
    f32x16_t sa[2], sb[2];
    qk(I0{}, sa);
    if (ragged && nkv == 1) mask_tile(sa, 0);
    float mx = tile_max(sa);
    for (int t = 0; t < nkv; t += 6) {   // unrolled by six: rings of three, S^T buffers of two
        step(t, I0{}, sa, sb, mx);
        if (t + 1 < nkv) step(t + 1, I1{}, sb, sa, mx);
        if (t + 2 < nkv) step(t + 2, I2{}, sa, sb, mx);
        if (t + 3 < nkv) step(t + 3, I3{}, sb, sa, mx);
        if (t + 4 < nkv) step(t + 4, I4{}, sa, sb, mx);
        if (t + 5 < nkv) step(t + 5, I5{}, sb, sa, mx);
    }

    wait_vmem();
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
