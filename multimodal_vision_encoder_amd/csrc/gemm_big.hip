// Large-tile bf16 "NT" GEMM on gfx950 MFMA:  C[m][n] = epilogue(sum_k A[m][k] W[n][k]).
//
// Block tile BM x BN (256 x 256 or 256 x 128), k-tiles of 32, 8 waves.  Each wave owns a
// 64 x (BN/2) tile of v_mfma_f32_32x32x16_bf16 blocks, issued with the W fragment first so
// each lane holds 4 consecutive output columns of one row.
//
// Copies: A and W k-tiles move global -> LDS with global_load_lds_dwordx4 (no register
// staging) into a 4-stage ring.  They are inline assembly so that the compiler's wait-count
// insertion does not treat them as LDS writes that every LDS read must wait for; the kernel
// waits for its own copies with s_waitcnt vmcnt(N) before each barrier, and the barrier is a
// bare s_barrier (the fence of __syncthreads would wait for every outstanding copy).  LDS
// rows are 32 bf16 (4 chunks of 16 bytes); chunk j of row r sits at j ^ ((r / 4) % 4), so the
// operand reads (ds_read_b128, 16 lanes per LDS pass over 256 bytes) are conflict-free.
//
// Ping-pong: the 8 waves form two groups of 4 (one wave of each per SIMD).  Both run the same
// sequence [MFMAs of k-tile t | barrier | LDS reads of k-tile t+1 and copies of k-tile t+4 |
// barrier], group 1 one phase behind group 0, so in every phase one wave per SIMD keeps the
// matrix core busy while the other reads LDS and issues copies.  Group 0 copies the A tile,
// group 1 the W tile.
//
// Epilogue: bias and activation are applied in registers, the tile is staged in LDS (rows
// padded by 16 bytes) and written out as whole rows, 16 bytes per lane.
//
// Split-K tail: when the tile count leaves a last partial round of blocks, the leftover tiles
// can be split along K so that the last round fills the chip.  Each slice writes its fp32
// partial tile to a workspace; a second kernel sums the slices in slice order (so results do
// not depend on timing) and applies the epilogue.  The host enables it only where the time
// saved exceeds the cost of the partial traffic.
//
// The A rows come from an address source: plain row-major activations, or the 3x3 merge
// gather of the projector ([Z] "Step 4"), where positions in the right/bottom zero padding
// read from a zero page.  Rows past M are clamped to row M-1 and never stored.
#include <type_traits>

#include "kernels.h"
#include "loaders.h"

namespace {

constexpr int BK = 32;
constexpr int NS = 4;   // copy-ring stages

__device__ __forceinline__ int xcd_remap(int bid, int nb)
{
    const int per = nb >> 3;
    return (bid & 7) * per + (bid >> 3);
}

// 16-byte global -> LDS copy; lane l writes LDS byte address lds + 16 l (lds wave-uniform).
// m0 needs one wait state before the copy reads it.
__device__ __forceinline__ void copy16(const void *g, uint32_t lds)
{
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     ::"v"(g), "s"(lds) : "memory", "m0");
}

// s_waitcnt vmcnt(N) lgkmcnt(0): all but this wave's newest N global loads done, LDS reads done.
template <int N>
__device__ __forceinline__ void wait_vmem_n()
{
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void bare_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }

// LDS chunk swizzle of a 64-byte row (4 chunks of 16 bytes): a ds_read_b128 is served 16
// lanes at a time over 64 four-byte banks (256 bytes), i.e. over four consecutive rows;
// XOR-ing the chunk index with (row / 4) % 4 gives 16 consecutive rows 16 distinct 16-byte
// slots of that window.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

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

// bias (columns n..n+3; columns past N get none) and activation
template <int ACT>
__device__ __forceinline__ void bias_act(const bf16_t *bias, int N, int n, const float *v, float *r)
{
    if (bias && n + 3 < N) {
        const uint2 b = *reinterpret_cast<const uint2 *>(bias + n);
        r[0] = v[0] + __uint_as_float(b.x << 16);
        r[1] = v[1] + __uint_as_float(b.x & 0xFFFF0000u);
        r[2] = v[2] + __uint_as_float(b.y << 16);
        r[3] = v[3] + __uint_as_float(b.y & 0xFFFF0000u);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (bias && n + j < N) ? v[j] + bf16_to_f32(bias[n + j]) : v[j];
    }
    if (ACT == ACT_GELU_TANH)
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = gelu_tanh_big(r[j]);
}

// bf16 output.  put(): 4 results -> 8 bytes at dst (LDS staging).  store(): 4 results of row
// m, columns n..n+3, straight to global memory with row and column bounds.
template <int ACT>
struct EpiBF16 {
    static constexpr int OUT_BYTES = 2;
    bf16_t *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ void put(char *dst, int n, const float *v) const
    {
        float r[4];
        bias_act<ACT>(bias, N, n, v, r);
        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
    }
    __device__ __forceinline__ void store(int64_t m, int n, const float *v) const
    {
        if (m >= M) return;
        float r[4];
        bias_act<ACT>(bias, N, n, v, r);
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
    static constexpr int OUT_BYTES = 4;
    float *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ void put(char *dst, int n, const float *v) const
    {
        float r[4];
        bias_act<ACT_NONE>(bias, N, n, v, r);
        *reinterpret_cast<float4 *>(dst) = make_float4(r[0], r[1], r[2], r[3]);
    }
    __device__ __forceinline__ void store(int64_t m, int n, const float *v) const
    {
        if (m >= M) return;
        float r[4];
        bias_act<ACT_NONE>(bias, N, n, v, r);
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

// Raw fp32 partial tile of a K slice (no bias, no activation), [BM][BN] contiguous.
struct EpiPart {
    static constexpr int OUT_BYTES = 4;
    float *out;
    __device__ __forceinline__ void put(char *dst, int, const float *v) const
    {
        *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// Work split of one launch: tiles [0, full) are computed whole; when splits > 1 the remaining
// tiles are cut into `splits` K slices each (items = leftover tiles x splits, block count
// rounded up to items_pad, a multiple of 8) whose fp32 partials go to `part`.
struct SplitK {
    int full, splits, items, items_pad;
    float *part;
};

template <int BM, int BN, class SRC, class EP>
__global__ __launch_bounds__(512, 1) void gemm_big_kernel(SRC src, const bf16_t *__restrict__ W,
                                                          int N, int K, EP ep, int tiles_m,
                                                          int tiles_n, SplitK sk)
{
    constexpr int NT = 512, NWN = 2;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
    constexpr int CPR = BK / 8;                             // 16-byte chunks per LDS row
    constexpr int AL = BM * CPR / 256, BL = BN * CPR / 256;  // copies per thread of its group
    constexpr int WM = BM / 4, WN = BN / NWN, TM = WM / 32, TN = WN / 32;
    static_assert(AL >= 1 && BL >= 1 && TM >= 1 && TN >= 1, "bad tile");
    // the output tile is staged in LDS for the final writes when it fits (fp32 partial tiles
    // of split slices always use BN = 128); the staging area overlays the copy ring
    constexpr int OB = EP::OUT_BYTES, PITCH = BN * OB + 16, PPITCH = BN * 4 + 16;
    constexpr bool STAGED = BM * PITCH <= 160 * 1024;
    constexpr bool PSTAGED = BM * PPITCH <= 160 * 1024;
    constexpr int SMEM0 = (STAGED && BM * PITCH > NS * STAGE) ? BM * PITCH : NS * STAGE;
    constexpr int SMEM = (PSTAGED && BM * PPITCH > SMEM0) ? BM * PPITCH : SMEM0;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];
    auto stage = [&](auto st) -> char * { return smem + decltype(st)::value * STAGE; };
    auto stage_lds = [&](auto st) -> uint32_t {
        return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)stage(st);
    };

    // work item of this block
    int tile, item = -1;
    if (sk.splits <= 1) {
        tile = xcd_remap(blockIdx.x, gridDim.x);
        if (tile >= tiles_m * tiles_n) return;
    } else if ((int)blockIdx.x < sk.full) {
        tile = xcd_remap(blockIdx.x, sk.full);
    } else {
        item = xcd_remap(blockIdx.x - sk.full, sk.items_pad);
        if (item >= sk.items) return;
        tile = sk.full + item / sk.splits;
    }
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int64_t m0 = (int64_t)tm * BM;
    const int n0 = tn * BN;
    const int nk_all = K / BK;
    int kt0 = 0, nk = nk_all;
    if (item >= 0) {
        const int sl = item % sk.splits;
        kt0 = (int)((int64_t)nk_all * sl / sk.splits);
        nk = (int)((int64_t)nk_all * (sl + 1) / sk.splits) - kt0;
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int grp = wave >> 2, w4 = wave & 3;              // group 0: waves 0-3, group 1: 4-7
    const int wm = grp * 2 + (w4 >> 1), wn = w4 & 1;

    // group 0 copies the A tile, group 1 the W tile; chunk c = (i*4 + w4)*64 + lane of a tile
    // holds row c / CPR, logical chunk (c % CPR) ^ swz(row)
    typename SRC::Row arow[AL];
    int aslot[AL];
    const bf16_t *wptr[BL];
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int c = (i * 4 + w4) * 64 + lane, r = c / CPR;
            arow[i] = src.row(m0 + r);
            aslot[i] = ((c % CPR) ^ swz(r)) * 8;
        }
    } else {
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            const int c = (i * 4 + w4) * 64 + lane, r = c / CPR;
            const int n = n0 + r < N ? n0 + r : N - 1;
            wptr[i] = W + (int64_t)n * K + ((c % CPR) ^ swz(r)) * 8;
        }
    }
    auto issue = [&](int kt, auto st) {
        const int k0 = (kt0 + kt) * BK;
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < AL; ++i)
                copy16(src.addr(arow[i], k0 + aslot[i]), stage_lds(st) + (i * 4 + w4) * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < BL; ++i) copy16(wptr[i] + k0, stage_lds(st) + A_BYTES + (i * 4 + w4) * 1024);
        }
    };
    // this wave's copies of all but the newest NS-2 k-tiles landed, and its LDS reads done
    auto wait_ring = [&]() {
        if (grp == 0) wait_vmem_n<(NS - 2) * AL>();
        else wait_vmem_n<(NS - 2) * BL>();
    };
    // instructions stay on their side of a barrier (the MFMAs especially)
    auto sync = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        bare_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    bf16x8_t fa[BK / 16][TM], fb[BK / 16][TN];
    auto ldfrag = [&](auto st) {
        const char *sa = stage(st), *sb = sa + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WM + i * 32 + l32;
                fa[ks][i] = *reinterpret_cast<const bf16x8_t *>(sa + r * (BK * 2) + (((2 * ks + g) ^ swz(r)) * 16));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WN + j * 32 + l32;
                fb[ks][j] = *reinterpret_cast<const bf16x8_t *>(sb + r * (BK * 2) + (((2 * ks + g) ^ swz(r)) * 16));
            }
        }
    };
    auto mma = [&]() {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fb[ks][j], fa[ks][i], acc[i][j]);
        __builtin_amdgcn_s_setprio(0);
    };

    // K-tile t lives in stage t % 4: group 0 reads it in phase 2t-1, group 1 in phase 2t, and
    // both refill it (with k-tile t+4) in phases 2t+1 and 2t+2.  Past the last k-tile the
    // copies repeat the last one into the free stage, so every phase waits for the same count.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    issue(0, I0{});
    issue(min(1, nk - 1), I1{});
    issue(min(2, nk - 1), I2{});
    issue(min(3, nk - 1), I3{});
    if (grp == 0) wait_vmem_n<(NS - 1) * AL>();
    else wait_vmem_n<(NS - 1) * BL>();
    sync();
    ldfrag(I0{});
    if (grp == 1) {   // group 1 runs one phase behind
        wait_ring();
        sync();
    }
    auto step = [&](int t, auto st) {
        constexpr int S = decltype(st)::value;
        mma();
        wait_ring();
        sync();
        if (t + 1 < nk) ldfrag(std::integral_constant<int, (S + 1) % NS>{});
        issue(min(t + NS, nk - 1), std::integral_constant<int, S>{});
        wait_ring();
        sync();
    };
    for (int kt = 0; kt < nk; kt += NS) {
        step(kt, I0{});
        if (kt + 1 < nk) step(kt + 1, I1{});
        if (kt + 2 < nk) step(kt + 2, I2{});
        if (kt + 3 < nk) step(kt + 3, I3{});
    }
    if (grp == 0) sync();   // same barrier count as group 1
    wait_vmem_n<0>();       // the trailing copies of the last k-tile
    sync();

    // acc[i][j][r]: output row l32 of the 32-block, column 8*(r/4) + 4*g + r%4.
    // Stage rows of `pitch` bytes in LDS via put(), then write whole rows of the tile.
    auto staged = [&](const auto &e, int pitch, int ob, char *gout, int64_t gpitch, int rows,
                      int row_bytes) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                        acc[i][j][4 * q + 3]};
                    const int r = wm * WM + i * 32 + l32, c = wn * WN + j * 32 + 8 * q + 4 * g;
                    e.put(smem + r * pitch + c * ob, n0 + c, v);
                }
        __syncthreads();
        const int ch = BN * ob / 16;                        // 16-byte chunks per tile row
#pragma unroll 4
        for (int c = tid; c < BM * ch; c += NT) {
            const int r = c / ch, b = (c % ch) * 16;
            if (r >= rows) break;
            const uint4 val = *reinterpret_cast<const uint4 *>(smem + r * pitch + b);
            char *dst = gout + r * gpitch + b;
            if (b + 16 <= row_bytes) {
                *reinterpret_cast<uint4 *>(dst) = val;
            } else if (b < row_bytes) {                    // ragged right edge, 2-byte pieces
                const uint16_t *s16 = reinterpret_cast<const uint16_t *>(smem + r * pitch + b);
                for (int e2 = 0; e2 < (row_bytes - b) / 2; ++e2) reinterpret_cast<uint16_t *>(dst)[e2] = s16[e2];
            }
        }
    };
    if (item >= 0) {   // K slice: raw fp32 partial tile, every row and column (host: BN = 128)
        if constexpr (PSTAGED)
            staged(EpiPart{}, PPITCH, 4, reinterpret_cast<char *>(sk.part + (int64_t)item * BM * BN),
                   (int64_t)BN * 4, BM, BN * 4);
        return;
    }
    if (STAGED && ((int64_t)N * OB) % 16 == 0) {
        const int rows = (int)(ep.M - m0 < BM ? ep.M - m0 : BM);
        const int row_bytes = (N - n0 < BN ? N - n0 : BN) * OB;
        staged(ep, PITCH, OB, reinterpret_cast<char *>(ep.out) + (m0 * N + n0) * OB, (int64_t)N * OB,
               rows, row_bytes);
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                ep.store(m0 + wm * WM + i * 32 + l32, n0 + wn * WN + j * 32 + 8 * q + 4 * g, v);
            }
}

// Sum of the K slices of the leftover tiles, in slice order, then the epilogue.  One thread
// per 4 columns of a row; a wave covers 256 consecutive columns (whole rows).
template <int BM, int BN, class EP>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(EP ep, int tiles_n, SplitK sk)
{
    constexpr int Q = BN / 4;                              // column groups per row
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int left = sk.items / sk.splits;
    if (idx >= (int64_t)left * BM * Q) return;
    const int lt = (int)(idx / (BM * Q)), rem = (int)(idx - (int64_t)lt * BM * Q);
    const int r = rem / Q, cq = rem - r * Q;
    const int tile = sk.full + lt;
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const float *p = sk.part + (int64_t)lt * sk.splits * BM * BN + r * BN + cq * 4;
    float4 s = *reinterpret_cast<const float4 *>(p);
    for (int j = 1; j < sk.splits; ++j) {
        const float4 t = *reinterpret_cast<const float4 *>(p + (int64_t)j * BM * BN);
        s.x += t.x, s.y += t.y, s.z += t.z, s.w += t.w;
    }
    const float v[4] = {s.x, s.y, s.z, s.w};
    ep.store((int64_t)tm * BM + r, tn * BN + cq * 4, v);
}

// Split plan of a BM x BN launch (one block per CU).  With T tiles and P CUs, a last round of
// r = T mod P tiles leaves P - r CUs idle for a whole tile time; cutting those r tiles into s
// K slices shortens that round to about 1/s of a tile time, at the cost of writing and
// reading back r*s fp32 partial tiles.  Costs are modelled with the measured time of one
// 32-wide k-step of a 256 x 128 tile (about 0.5 us) and 4 TB/s for the partial traffic; the
// split is used when it saves at least 5 us.  Only 256 x 128 tiles with bf16 or fp32 output
// and N % 4 == 0 are split.
SplitK plan_split(int64_t M, int N, int K, int BM, int BN, bool allowed)
{
    SplitK sk{0, 1, 0, 0, nullptr};
    const int64_t tiles = ceil_div(M, BM) * ceil_div(N, BN);
    const int P = cu_count();
    if (!allowed || BN != 128 || (N & 3) != 0 || P % 8 != 0 || tiles < P) return sk;
    const int64_t full = tiles / P * P, left = tiles - full;
    if (left == 0) return sk;
    const int nk = K / BK;
    const double t_step = 0.5e-6 * ((double)BM * BN / (256.0 * 128.0));
    const double tile_bytes = (double)BM * BN * 4;
    double best_gain = 5e-6;
    int best_s = 1;
    for (int s = 2; s <= 8; s *= 2) {
        if (left * s > P || nk < 4 * s) break;
        const double gain = (1.0 - 1.0 / s) * nk * t_step - (double)left * s * tile_bytes * 2 / 4e12;
        if (gain > best_gain) best_gain = gain, best_s = s;
    }
    if (best_s == 1) return sk;
    sk.full = (int)full;
    sk.splits = best_s;
    sk.items = (int)(left * best_s);
    sk.items_pad = (int)(ceil_div(sk.items, 8) * 8);
    return sk;
}

template <int BM, int BN, class SRC, class EP>
hipError_t run_big(SRC src, const bf16_t *W, int64_t M, int N, int K, EP ep, const GemmWorkspace *ws,
                   hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    const int tiles_m = (int)ceil_div(M, BM), tiles_n = (int)ceil_div(N, BN);
    SplitK sk = plan_split(M, N, K, BM, BN, ws != nullptr);
    if (sk.splits > 1 && (size_t)sk.items * BM * BN * 4 > ws->bytes) sk = SplitK{0, 1, 0, 0, nullptr};
    if (sk.splits > 1) {
        sk.part = ws->part;
        hipLaunchKernelGGL((gemm_big_kernel<BM, BN, SRC, EP>), dim3(sk.full + sk.items_pad), dim3(512), 0, s,
                           src, W, N, K, ep, tiles_m, tiles_n, sk);
        const int64_t threads = (int64_t)(sk.items / sk.splits) * BM * (BN / 4);
        hipLaunchKernelGGL((gemm_split_reduce_kernel<BM, BN, EP>), dim3((unsigned)ceil_div(threads, 256)),
                           dim3(256), 0, s, ep, tiles_n, sk);
        return hipGetLastError();
    }
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int grid = (int)(ceil_div(tiles, 8) * 8);
    hipLaunchKernelGGL((gemm_big_kernel<BM, BN, SRC, EP>), dim3(grid), dim3(512), 0, s, src, W, N, K, ep,
                       tiles_m, tiles_n, sk);
    return hipGetLastError();
}

// 256 x 256 tiles when they give at least one full wave of blocks, else 256 x 128
bool use_big_tiles(int64_t M, int N) { return ceil_div(M, 256) * ceil_div(N, 256) >= cu_count(); }

template <class SRC>
hipError_t dispatch(SRC src, const bf16_t *W, int64_t M, int N, int K, const bf16_t *bias, int act,
                    bool out_f32, void *out, const GemmWorkspace *ws, hipStream_t s)
{
    const bool big = use_big_tiles(M, N);
    if (out_f32) {
        EpiF32 ep{(float *)out, bias, M, N};
        return big ? run_big<256, 256>(src, W, M, N, K, ep, ws, s) : run_big<256, 128>(src, W, M, N, K, ep, ws, s);
    }
    if (act == ACT_GELU_TANH) {
        EpiBF16<ACT_GELU_TANH> ep{(bf16_t *)out, bias, M, N};
        return big ? run_big<256, 256>(src, W, M, N, K, ep, ws, s) : run_big<256, 128>(src, W, M, N, K, ep, ws, s);
    }
    EpiBF16<ACT_NONE> ep{(bf16_t *)out, bias, M, N};
    return big ? run_big<256, 256>(src, W, M, N, K, ep, ws, s) : run_big<256, 128>(src, W, M, N, K, ep, ws, s);
}

}  // namespace

int cu_count()
{
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}


size_t gemm_workspace_max_bytes() { return (size_t)cu_count() * 256 * 128 * 4; }

size_t gemm_workspace_bytes(int64_t M, int N, int K)
{
    if (use_big_tiles(M, N)) return 0;
    const SplitK sk = plan_split(M, N, K, 256, 128, true);
    return sk.splits > 1 ? (size_t)sk.items * 256 * 128 * 4 : 0;
}

hipError_t launch_linear(const bf16_t *A, int64_t M, int K, const bf16_t *W, const bf16_t *bias,
                         int N, int act, bool out_f32, void *out, const GemmWorkspace *ws, hipStream_t s)
{
    return dispatch(SrcPlain{A, K, M}, W, M, N, K, bias, act, out_f32, out, ws, s);
}

hipError_t launch_merge_project(const bf16_t *y, const ImgDesc *imgs, int n_img, int64_t Mtok,
                                int D, const bf16_t *Wp, const bf16_t *bias, int Dl, float *out,
                                const bf16_t *zero, const GemmWorkspace *ws, hipStream_t s)
{
    return dispatch(SrcMerge{y, imgs, n_img, Mtok, D, zero}, Wp, Mtok, Dl, 9 * D, bias, ACT_NONE,
                    true, out, ws, s);
}
