// Bidirectional flash attention over a packed multi-image batch (block-diagonal by image).
//
// Every patch attends to every patch of its own image and to nothing else ([Z] "Multimodal
// basics": attention gives each patch whole-image context; [L] DS4V: attention is
// bidirectional within each image's span).  Scale 1/sqrt(hd).
//
// One block = 4 waves x 32 queries of one head of one image.  Keys come in tiles of 64.
//
// Data movement: K and V^T tiles go global -> LDS with global_load_lds_dwordx4 (no register
// staging) into two rings of 4 stages each (64 KB per block).  K of a tile is read one
// iteration before its V^T, so iteration t issues K of tile t+3 and V^T of tile t+2 and,
// before its closing barrier, waits only for its copies up to K of tile t+2: every copy has
// at least one whole iteration to land.  The copies are written as inline assembly (scalar base,
// 32-bit per-lane offset, fixed for all tiles) so the compiler neither inserts its
// conservative wait-for-all-copies before LDS reads nor recomputes addresses per tile; the
// barrier is a bare s_barrier for the same reason (the fence in __syncthreads waits for every
// copy).
// LDS rows are stored as XOR-swizzled 16-byte chunks so that the MFMA operand reads
// (ds_read_b128, 16 lanes per LDS pass) are free of bank conflicts.
//
// Scores in log2 units: each wave scales its q rows by log2(e)/sqrt(hd) once and rounds them
// to binary16; k is stored as binary16 by the RoPE kernel (exact for bf16 values of normal
// binary16 range).  Per tile and wave:
//   S^T = K Q^T - m       v_mfma_f32_32x32x16_f16 with K from LDS and Q^T in registers, the
//                         accumulator starting from -m (m = running row max, one value per
//                         lane: the transpose puts one query per lane, column l%32), so the
//                         scores come out already shifted.
//   online softmax        p = exp2(S) (one v_exp_f32 per score, no other arithmetic), packed
//                         to binary16 with v_cvt_pkrtz_f16_f32 (relative error below 2^-10,
//                         eight times finer than bf16: with near-uniform attention the output
//                         is a small average of large values, and bf16 weights alone would
//                         flip about a third of the bf16-rounded outputs); the row sum is
//                         taken on those same values with v_dot2c_f32_f16, so numerator and
//                         denominator use the same weights.  m only moves when a lane's tile
//                         sum exceeds 2^8 (wave-uniform branch, rare), which bounds every
//                         weight by 2^8 without a per-tile max.
//   O^T += V^T P^T        v_mfma_f32_32x32x16_f16 on the binary16 V^T written by the RoPE
//                         kernel.  P^T is already in the B-operand layout of the S^T
//                         accumulator (the key order inside each 16-key chunk is permuted
//                         identically on both operands).
// Each step reads all its MFMA operands from LDS first, runs the softmax of tile t while the
// reads land, then the MFMAs of S^T (tile t+1, into the registers the softmax freed) and of
// P.V (tile t); the other wave on the SIMD fills the gaps of either phase.
// Keys past the image end (last tile only) are masked to -inf; their loads are clamped to
// the image's last row.  Query rows past the image end are zero and never stored.  Past the
// last tile the ring is refilled with copies of the last tile, whose scores are computed and
// ignored, so the loop body has no tile-count branches.
#include <math.h>

#include <algorithm>
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
// The same barrier, issued only once x is available (so every LDS read that x depends on has
// completed in this wave).
__device__ __forceinline__ void barrier_after(float x) { __asm__ volatile("s_barrier" ::"v"(x) : "memory"); }

// Value of x held by lane l ^ 32 (v_permlane32_swap exchanges the two wave halves).
__device__ __forceinline__ float xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

constexpr float kLazySum = 256.f;   // largest weight (2^8) left unrescaled

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
    const ImgDesc *__restrict__ imgs, int D, int H, float c_log2, AttnSplit pl)
{
    using G = AttnGeom<HD>;
    constexpr int HDP = G::HDP, KCH = G::KCH, KS = HDP / 16, DB = HDP / 32;
    static_assert(G::KLOADS >= 1 && G::VLOADS >= 1, "tile too small for 256 threads");
    // K and V^T rings of four stages each; tile j sits in stage j % 4 of its ring
    __shared__ __attribute__((aligned(1024))) char kst[4 * G::K_BYTES];
    __shared__ __attribute__((aligned(1024))) char vst[4 * G::V_BYTES];
    auto kstage = [&](auto st) -> char * { return kst + decltype(st)::value * G::K_BYTES; };
    auto vstage = [&](auto st) -> char * { return vst + decltype(st)::value * G::V_BYTES; };
    auto lds_addr = [&](const char *p) -> uint32_t {
        return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
    };

    // block -> item (head, query tile) and key slice.  Blocks are dealt to the XCDs in turn, so
    // XCD x runs blocks x, x + 8, ... in that order: they take the x-th group of per_xcd
    // consecutive items (mostly one head: its K and V^T stay in that XCD's L2), first the
    // `full` whole items, then the key slices of the rest (neighbours for one item).
    const int xg = blockIdx.x & 7, jb = blockIdx.x >> 3;
    int L, split = 0, nsplit = 1, tix = 0;
    if (jb < pl.full) {
        L = xg * pl.per_xcd + jb;
    } else {
        const int u = jb - pl.full, tail = pl.per_xcd - pl.full;
        nsplit = pl.slices;
        split = u % nsplit;
        L = xg * pl.per_xcd + pl.full + u / nsplit;
        tix = xg * tail + u / nsplit;
    }
    if (L >= pl.items) return;
    const int head = L / n_work, wi = L - head * n_work;
    const RowTile wt = work[wi];
    const ImgDesc d = imgs[wt.img];
    // key tiles [t0, t0 + nkv) of the image's nkv_all
    const int nkv_all = (d.n + 63) / 64, per = (nkv_all + nsplit - 1) / nsplit;
    const int t0 = split * per, nkv = min(nkv_all, t0 + per) - t0;
    // this slice's rows of the partial buffers: [tail item][slice][query row of the tile]
    const int64_t prow0 = ((int64_t)tix * nsplit + split) * (4 * 32);

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)D;
    const bf16_t *qbase = qkv + (int64_t)d.patch_off * ld + head * HD;
    const bf16_t *kbase = qbase + D;
    const bf16_t *vbase = vt + (int64_t)head * HD * ldv + d.vt_off;

    const int q = wt.r0 + wave * 32 + l32;   // this lane's query (local row)
    if (nkv <= 0) {   // empty key slice (image shorter than the slices): weight zero in the merge
        if (q < d.n) {
            const int64_t pr = prow0 + wave * 32 + l32;
            uint16_t *prow = pl.part_o + pr * HD;
            for (int dd = 4 * g; dd < HD; dd += 8) *reinterpret_cast<uint2 *>(prow + dd) = make_uint2(0, 0);
            if (g == 0) reinterpret_cast<float2 *>(pl.part_ml)[pr] = make_float2(-INFINITY, 0.f);
        }
        return;
    }
    // q * log2(e)/sqrt(hd), rounded once to binary16: scores come out in log2 units
    f16x8_t qf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const int dd = 16 * kk + 8 * g;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (q < d.n && dd < HD) v = *reinterpret_cast<const uint4 *>(qbase + (int64_t)q * ld + dd);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = __uint_as_float(e & 1 ? w[e >> 1] & 0xFFFF0000u : w[e >> 1] << 16) * c_log2;
            qf[kk][e] = (_Float16)fminf(fmaxf(x, -65504.f), 65504.f);
        }
    }

    // Copies of key tile t into a stage.  Chunk c of a stage (lane-contiguous per instruction)
    // holds logical chunk (c % KCH) ^ kswz(row) of its row (V^T: ^ vswz(row)).  The per-lane
    // byte offsets are the same for every tile: a tile's copies are one scalar base plus these.
    uint32_t koff[G::KLOADS], voff[G::VLOADS];
#pragma unroll
    for (int i = 0; i < G::KLOADS; ++i) {
        const int c = (i * 4 + wave) * 64 + lane, r = c / KCH, sw = (c % KCH) ^ G::kswz(r);
        koff[i] = (uint32_t)(r * (int)ld + (sw * 8) % HD) * 2u;   // pad chunks (HD < 32) re-read real data
    }
#pragma unroll
    for (int i = 0; i < G::VLOADS; ++i) {
        const int c = (i * 4 + wave) * 64 + lane, r = c >> 3, sw = (c & 7) ^ G::vswz(r);
        voff[i] = (uint32_t)((int64_t)(r % HD) * ldv + sw * 8) * 2u;
    }
    auto issue_k = [&](int t, auto st) {   // t: tile index inside the slice
        const uint32_t sk = lds_addr(kstage(st));
        const int kv0 = (t0 + t) * 64;
        const bf16_t *kb = kbase + (int64_t)kv0 * ld;
        if (kv0 + 64 <= d.n) {
#pragma unroll
            for (int i = 0; i < G::KLOADS; ++i) load_lds16(kb, koff[i], sk + (i * 4 + wave) * 1024);
        } else {   // last tile of a ragged image: rows past the end re-read its last row
#pragma unroll
            for (int i = 0; i < G::KLOADS; ++i) {
                const int c = (i * 4 + wave) * 64 + lane, r = c / KCH, sw = (c % KCH) ^ G::kswz(r);
                const int rc = min(r, d.n - 1 - kv0);
                load_lds16(kb, (uint32_t)(rc * (int)ld + (sw * 8) % HD) * 2u, sk + (i * 4 + wave) * 1024);
            }
        }
    };
    auto issue_v = [&](int t, auto st) {
        const uint32_t sv = lds_addr(vstage(st));
        const bf16_t *vb = vbase + (t0 + t) * 64;
#pragma unroll
        for (int i = 0; i < G::VLOADS; ++i) load_lds16(vb, voff[i], sv + (i * 4 + wave) * 1024);
    };

    // MFMA operands of one step, read from LDS at its start (the copies were waited for before
    // the previous barrier).
    f16x8_t kf[KS][2];   // K of the next tile: A operands of S^T
    f16x8_t vf[4][DB];   // V^T of the previous tile: A operands of O^T
    auto read_k = [&](auto st) {
        const char *sk = kstage(st);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = 32 * kb + l32, ch = (2 * kk + g) ^ G::kswz(row);
                kf[kk][kb] = *reinterpret_cast<const f16x8_t *>(sk + row * (HDP * 2) + ch * 16);
            }
    };
    // V^T chunk c covers keys 16c..16c+15; B-operand slot 8g+j <-> key 16c + 8(j/4) + 4g + j%4,
    // i.e. registers 8(c%2)+j of S^T block c/2.  The transposed-V buffer stores each 16-key
    // group with key bits 2 and 3 swapped, so those 8 keys are the 16-byte chunk 2c+g of the
    // row: one ds_read_b128 per operand.
    auto read_v = [&](auto st) {
        const char *sv = vstage(st);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const int row = 32 * b + l32;
                vf[c][b] = *reinterpret_cast<const f16x8_t *>(sv + row * 128 + (((2 * c + g) ^ G::vswz(row)) * 16));
            }
    };

    f32x16_t oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
    float m_run = 0.f, l_run = 0.f;   // running max (log2 units) and this lane's part of the sum
    f32x16_t cm;                      // -m_run in every slot: the S^T accumulator's start

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
    auto set_max = [&](float m) {
        m_run = m;
#pragma unroll
        for (int r = 0; r < 16; ++r) cm[r] = -m;
    };
    auto shift = [&](f32x16_t *sc, float dl) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[kb][r] -= dl;
    };
    // exp2 of the shifted scores of one tile, packed to binary16 (round toward zero); returns
    // this lane's sum of the packed weights (v_dot2c on the same binary16 values, so the
    // numerator and the denominator use identical weights)
    auto softmax = [&](const f32x16_t *cur, uint32_t (*pk)[4]) {
        float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kb = c >> 1, r = 8 * (c & 1) + 2 * j;
                pk[c][j] = pack_f16x2_rtz(fast_exp2(cur[kb][r]), fast_exp2(cur[kb][r + 1]));
                if (j & 1) ls1 = dot2_f16(pk[c][j], ls1);
                else ls0 = dot2_f16(pk[c][j], ls0);
            }
        return ls0 + ls1;
    };
    // S^T of one tile (accumulator started from -m, so the scores come out shifted) and
    // O^T += V^T P^T of an earlier tile; P^T is already in the B-operand layout of the S^T
    // accumulator (the key order inside each 16-key chunk is permuted identically on both
    // operands).  The two products form four independent accumulation chains: S^T over the
    // KS 16-wide slices of the head dim, P.V over the 4 16-key slices of the tile.
    auto mfmas = [&](f32x16_t *sn, const uint32_t (*pk)[4], bool with_pv) {
        constexpr int NI = KS > 4 ? KS : 4;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (i < KS) sn[kb] = mfma32_f16(kf[i][kb], qf[i], i == 0 ? cm : sn[kb]);
            if (with_pv && i < 4) {
                const f16x8_t pf = as_f16x8(make_uint4(pk[i][0], pk[i][1], pk[i][2], pk[i][3]));
#pragma unroll
                for (int b = 0; b < DB; ++b) oacc[b] = mfma32_f16(vf[i][b], pf, oacc[b]);
            }
        }
    };

    // the image's ragged last tile, if it falls in this slice
    const bool ragged = (d.n & 63) != 0 && t0 + nkv == nkv_all;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using Yes = std::true_type;
    using No = std::false_type;
    // prologue: K of tiles 0..2, V^T of tiles 0..1; wait for K 0 and K 1
    issue_k(0, I0{});
    issue_k(min(1, nkv - 1), I1{});
    issue_v(0, I0{});
    issue_k(min(2, nkv - 1), I2{});
    issue_v(min(1, nkv - 1), I1{});
    wait_vmem_n<G::KLOADS + 2 * G::VLOADS>();
    bare_barrier();

    f32x16_t sc0[2], sc1[2];   // S^T of the current tile and of the next one (alternating)
    uint32_t pk0[4][4], pk1[4][4];   // binary16 weights of the current and previous tile
    {
        read_k(I0{});
        const f32x16_t z = {};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sc0[kb] = mfma32_f16(kf[kk][kb], qf[kk], kk == 0 ? z : sc0[kb]);
    }
    if (ragged && nkv == 1) mask_tile(sc0, t0 * 64);
    set_max(tile_max(sc0));   // finite: key 0 of the tile is always inside the image
    shift(sc0, m_run);

    // Step t: issue K of tile t+3 and V^T of tile t+2 (into the stages of K t-1 and V^T t-2,
    // last read in steps t-2 and t-1); read K of tile t+1 and V^T of tile t-1; then the MFMAs
    // of S^T(t+1) and of P.V(t-1) interleaved with the softmax of tile t; then wait for this
    // wave's copies up to K t+2 (V^T t too) and publish them.  Past the last tile the copies
    // and S^T repeat the last tile and are ignored.
    //
    // Lazy rescale: the running max only moves when a weight would exceed 2^8.  Every weight
    // is non-negative, so a lane's tile sum of at most 2^8 bounds each of its weights (an
    // overflow shows up as 65504 or inf in the sum).  Otherwise (wave-uniform, rare: the
    // first tiles of a row) the max moves up to the tile's row max, O (which already holds
    // P.V(t-1)) and the sum are scaled by 2^-delta, the scores of tiles t and t+1 are shifted
    // and the weights of tile t recomputed (all at most 1 now).
    auto step = [&](int t, auto st, f32x16_t *sc, f32x16_t *sn, uint32_t (*pk)[4],
                    uint32_t (*pkp)[4], auto pvt) {
        constexpr int S = decltype(st)::value;
        constexpr bool with_pv = decltype(pvt)::value;
        using KQ = std::integral_constant<int, (S + 1) % 4>;   // K of tile t+1
        using KD = std::integral_constant<int, (S + 3) % 4>;   // K of tile t+3
        using VP = std::integral_constant<int, (S + 3) % 4>;   // V^T of tile t-1
        using VD = std::integral_constant<int, (S + 2) % 4>;   // V^T of tile t+2
        issue_k(min(t + 3, nkv - 1), KD{});
        issue_v(min(t + 2, nkv - 1), VD{});
        read_k(KQ{});
        if (with_pv) read_v(VP{});
        // raised wave priority while this wave's MFMAs and softmax issue, so that of the two
        // waves on a SIMD the one in this phase goes first (measured: 0.6% per launch)
        __builtin_amdgcn_s_setprio(1);
        mfmas(sn, pkp, with_pv);
        float ts = softmax(sc, pk);
        // schedule: all LDS reads, a few VALU while they land, then 1 MFMA / 4 VALU pairs
        __builtin_amdgcn_sched_group_barrier(0x100, with_pv ? KS * 2 + 4 * DB : KS * 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        if (__ballot(!(ts <= kLazySum))) {
            const float dl = fmaxf(tile_max(sc), 0.f);
            set_max(m_run + dl);
            const float alpha = fast_exp2(-dl);
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
            shift(sc, dl);
            shift(sn, dl);
            ts = softmax(sc, pk);
        }
        l_run += ts;
        __builtin_amdgcn_s_setprio(0);
        if (ragged && t + 1 == nkv - 1) mask_tile(sn, (t0 + t + 1) * 64);
        wait_vmem_n<G::KLOADS + 2 * G::VLOADS>();
        bare_barrier();
    };
    // unrolled by four: rings of four, S^T and weight buffers of two
    step(0, I0{}, sc0, sc1, pk0, pk1, No{});
    for (int t = 1; t < nkv; t += 4) {
        step(t, I1{}, sc1, sc0, pk1, pk0, Yes{});
        if (t + 1 < nkv) step(t + 1, I2{}, sc0, sc1, pk0, pk1, Yes{});
        if (t + 2 < nkv) step(t + 2, I3{}, sc1, sc0, pk1, pk0, Yes{});
        if (t + 3 < nkv) step(t + 3, I0{}, sc0, sc1, pk0, pk1, Yes{});
    }
    // P.V of the last tile (its V^T was waited for at the end of the last step)
    {
        const int tl = nkv - 1;
        uint32_t(*pkl)[4] = (tl & 1) ? pk1 : pk0;
        switch (tl & 3) {
        case 0: read_v(I0{}); break;
        case 1: read_v(I1{}); break;
        case 2: read_v(I2{}); break;
        default: read_v(I3{}); break;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f16x8_t pf = as_f16x8(make_uint4(pkl[c][0], pkl[c][1], pkl[c][2], pkl[c][3]));
#pragma unroll
            for (int b = 0; b < DB; ++b) oacc[b] = mfma32_f16(vf[c][b], pf, oacc[b]);
        }
    }

    wait_vmem();
    const float l_tot = l_run + xor32(l_run);
    const float inv = 1.f / l_tot;
    if (q < d.n) {
        const int64_t row = (int64_t)d.patch_off + q;
        if (nsplit == 1) {
            bf16_t *orow = o + row * D + head * HD;
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
        } else {   // this slice's normalised output (binary16) and its (max, sum)
            const int64_t pr = prow0 + wave * 32 + l32;
            uint16_t *prow = pl.part_o + pr * HD;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    const int dd = 32 * b + 8 * grp + 4 * g;
                    if (dd < HD) {
                        uint32_t h[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const float a = fminf(fmaxf(oacc[b][4 * grp + 2 * e] * inv, -65504.f), 65504.f);
                            const float c = fminf(fmaxf(oacc[b][4 * grp + 2 * e + 1] * inv, -65504.f), 65504.f);
                            h[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)c) << 16);
                        }
                        *reinterpret_cast<uint2 *>(prow + dd) = make_uint2(h[0], h[1]);
                    }
                }
            if (g == 0) reinterpret_cast<float2 *>(pl.part_ml)[pr] = make_float2(m_run, l_tot);
        }
    }
}

// Merge of the key slices of the split items: with weights w_s = l_s 2^(m_s - M), M the
// largest slice max, out = sum_s w_s o_s / sum_s w_s, rounded once to bf16.  One thread per
// 8 consecutive columns of one query row of one split item (one head).  Empty slices carry
// l = 0, o = 0.
__global__ __launch_bounds__(256) void attention_merge_kernel(
    AttnSplit pl, const RowTile *__restrict__ work, int n_work, const ImgDesc *__restrict__ imgs,
    int D, int hd, bf16_t *__restrict__ o)
{
    constexpr int QT = 4 * 32;
    const int chunks = hd / 8, tail = pl.per_xcd - pl.full, ns = pl.slices;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)8 * tail * QT * chunks) return;
    const int tix = (int)(idx / (QT * chunks)), rem = (int)(idx - (int64_t)tix * QT * chunks);
    const int r = rem / chunks, col = (rem - r * chunks) * 8;
    // The partial rows of every thread of the grid lie inside the buffers (8 x tail x slices x
    // QT rows), so this thread's (max, sum) pairs and output chunks are loaded first, beside
    // the work-item and image lookups they do not depend on; rows past an image end are
    // dropped below without being stored.
    const float2 *ml = reinterpret_cast<const float2 *>(pl.part_ml);
    const int64_t pr0 = (int64_t)tix * ns * QT + r;   // slice sp at pr0 + sp * QT
    float2 m[4];
    uint4 u[4];
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
        if (sp < ns) {
            m[sp] = ml[pr0 + (int64_t)sp * QT];
            u[sp] = *reinterpret_cast<const uint4 *>(pl.part_o + (pr0 + (int64_t)sp * QT) * hd + col);
        }
    const int L = (tix / tail) * pl.per_xcd + pl.full + tix % tail;
    if (L >= pl.items) return;
    const int head = L / n_work, wi = L - head * n_work;
    const RowTile wt = work[wi];
    const ImgDesc d = imgs[wt.img];
    const int q = wt.r0 + r;
    if (q >= d.n) return;
    float mmax = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
        if (sp < ns) mmax = fmaxf(mmax, m[sp].x);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, wsum = 0.f;
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
        if (sp >= ns) break;
        const float w = m[sp].y == 0.f ? 0.f : m[sp].y * fast_exp2(m[sp].x - mmax);
        const uint32_t ww[4] = {u[sp].x, u[sp].y, u[sp].z, u[sp].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t hb = (uint16_t)((ww[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
            acc[e] += w * (float)__builtin_bit_cast(_Float16, hb);
        }
        wsum += w;
    }
    const float inv = 1.f / wsum;
    *reinterpret_cast<uint4 *>(o + ((int64_t)d.patch_off + q) * D + head * hd + col) =
        make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                   pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
}

template <int HD>
hipError_t run_attention(const bf16_t *qkv, const bf16_t *vt, int64_t ldv, bf16_t *o,
                         const RowTile *work, int n_work, const ImgDesc *imgs, int D, int H,
                         const AttnSplit &sp, hipStream_t s)
{
    const int tail = sp.per_xcd - sp.full;
    const int64_t grid = (int64_t)8 * (sp.full + (int64_t)tail * sp.slices);
    const float c_log2 = (float)(1.4426950408889634 / sqrt((double)HD));
    hipLaunchKernelGGL(attention_kernel<HD>, dim3((unsigned)grid), dim3(256), 0, s, qkv, vt, ldv, o, work,
                       n_work, imgs, D, H, c_log2, sp);
    return hipGetLastError();
}

template <int HD>
int blocks_per_cu()
{
    static int nb = 0;
    if (nb == 0) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, attention_kernel<HD>, 256, 0) != hipSuccess || v < 1) {
            (void)hipGetLastError();
            v = 1;
        }
        nb = v;
    }
    return nb;
}

}  // namespace

int attention_q_tile() { return 128; }

size_t attention_plan_bytes(const AttnSplit &sp, int D, int H)
{
    const int64_t tail = sp.per_xcd - sp.full;
    if (sp.slices <= 1 || tail <= 0) return 0;
    const int hd = D / H;
    return (size_t)8 * tail * sp.slices * attention_q_tile() * ((size_t)hd * sizeof(uint16_t) + sizeof(float2));
}

// Work split of a batch.  The blocks of one XCD fill its block slots (CUs x resident blocks)
// in rounds; when the last round is partial, its items are cut into key slices so that it
// occupies every slot for a fraction of a round.  A CU runs its attention blocks at about the
// same total rate with one or two resident, so the cut pays even when the slices only fill
// the CUs once.  At most 4 slices, each of at least two key tiles of the largest image.
AttnSplit attention_plan(const ImgDesc *imgs, int n_img, int n_work, int D, int H, int fixed)
{
    AttnSplit sp{0, 0, 1, 0, nullptr, nullptr};
    sp.items = n_work * H;
    sp.per_xcd = (int)ceil_div(sp.items, 8);
    sp.full = sp.per_xcd;
    if (n_work <= 0 || H <= 0 || n_img <= 0 || fixed == 1) return sp;
    if (fixed >= 2) {
        sp.full = 0;
        sp.slices = fixed;
        return sp;
    }
    int per_cu = 1;
    switch (D / H) {
    case 16: per_cu = blocks_per_cu<16>(); break;
    case 32: per_cu = blocks_per_cu<32>(); break;
    case 64: per_cu = blocks_per_cu<64>(); break;
    case 128: per_cu = blocks_per_cu<128>(); break;
    default: return sp;
    }
    const int slots = std::max(1, cu_count() / 8) * per_cu;   // block slots of one XCD
    const int full = sp.per_xcd / slots * slots, tail = sp.per_xcd - full;
    if (tail == 0) return sp;
    int max_nkv = 0;
    for (int i = 0; i < n_img; ++i) max_nkv = std::max(max_nkv, (int)ceil_div(imgs[i].n, 64));
    const int s = std::min({4, slots / tail, max_nkv / 2});
    if (s < 2) return sp;
    sp.full = full;
    sp.slices = s;
    return sp;
}

bool attention_needs_merge(const AttnSplit &sp) { return sp.per_xcd > sp.full && sp.slices > 1; }

hipError_t launch_attention_merge(bf16_t *o, const RowTile *work, int n_work, const ImgDesc *imgs, int D, int H,
                                  const AttnSplit &sp, hipStream_t s)
{
    if (n_work <= 0 || !attention_needs_merge(sp)) return hipSuccess;
    const int tail = sp.per_xcd - sp.full, hd = D / H;
    const int64_t threads = (int64_t)8 * tail * attention_q_tile() * (hd / 8);
    hipLaunchKernelGGL(attention_merge_kernel, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s, sp, work,
                       n_work, imgs, D, hd, o);
    return hipGetLastError();
}

hipError_t launch_attention(const bf16_t *qkv, const bf16_t *vt, int64_t ldv, bf16_t *o,
                            const RowTile *work, int n_work, const ImgDesc *imgs, int D, int H,
                            const AttnSplit &sp, hipStream_t s)
{
    if (n_work <= 0) return hipSuccess;
    const int tail = sp.per_xcd - sp.full;
    if (sp.items != n_work * H || sp.per_xcd != (int)ceil_div(sp.items, 8) || sp.full < 0 || tail < 0 ||
        sp.slices < 1 || sp.slices > 4 || (tail > 0 && sp.slices > 1 && (!sp.part_o || !sp.part_ml)))
        return hipErrorInvalidValue;
    switch (D / H) {
    case 16: return run_attention<16>(qkv, vt, ldv, o, work, n_work, imgs, D, H, sp, s);
    case 32: return run_attention<32>(qkv, vt, ldv, o, work, n_work, imgs, D, H, sp, s);
    case 64: return run_attention<64>(qkv, vt, ldv, o, work, n_work, imgs, D, H, sp, s);
    case 128: return run_attention<128>(qkv, vt, ldv, o, work, n_work, imgs, D, H, sp, s);
    default: return hipErrorInvalidValue;
    }
}
