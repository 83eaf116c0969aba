// Large-tile bf16 "NT" GEMM on gfx950 MFMA:  C[m][n] = epilogue(sum_k A[m][k] W[n][k]).
//
// Block tile BM x BN (256 x 256, 256 x 128 or 128 x 128, chosen from the launch's size).  256 x 256
// tiles of plain activations run on 4 waves, one per SIMD, each owning a 128 x 128 tile, with
// 64-wide k-tiles in two LDS stages (described at that branch of the kernel).  Every other launch
// runs the 8-wave form below: k-tiles of 32, each wave a (BM/4) x (BN/2) tile.  Both issue
// v_mfma_f32_32x32x16_bf16 with the W fragment first so each lane holds 4 consecutive output
// columns of one row, and share the epilogues.  Tiles are dealt to the 8 XCDs in contiguous
// ranges, in groups of 4 tile rows.
//
// The 8-wave form:
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
// Epilogue: each lane loads the bias of its columns once, bias and activation are applied in
// registers, the tile is staged in LDS (rows padded by 16 bytes) and written out as whole
// rows, 16 bytes per lane.  The SwiGLU epilogue pairs gate and up columns in registers.
//
// Split-K tail: when the tile count leaves a last partial round of blocks (or is below one
// round), the leftover tiles can be split along K so that the last round fills the chip.  Each slice writes its fp32
// partial tile to a workspace; a second kernel sums the slices in slice order (so results do
// not depend on timing) and applies the epilogue.  The host enables it only where the time
// saved exceeds the cost of the partial traffic.
//
// The A rows come from an address source: plain row-major activations, or the 3x3 merge
// gather of the projector ([Z] "Step 4"), where positions in the right/bottom zero padding
// read from a zero page.  Rows past M are clamped to row M-1 and never stored.  The patch
// projection's A comes from the pixels themselves (patchify fused into the loader): group 0
// copies the raw bytes of k-tile t+NS+2 global -> LDS in the step of k-tile t, and two steps
// later converts them to bf16 and writes them into their stage with ds_write (the bytes need
// arithmetic on the way, so the stage cannot be filled by the copies themselves).
#include <type_traits>

#include "kernels.h"
#include "loaders.h"

namespace {

constexpr int BK = 32;
constexpr int NS = 4;   // copy-ring stages (5 measured no faster)

// f(integral_constant<int, S>) for S = 0 .. NS-1 in order (compile-time ring stage indices)
template <class F, int... S>
__device__ __forceinline__ void each_stage(std::integer_sequence<int, S...>, F &&f)
{
    (f(std::integral_constant<int, S>{}), ...);
}

__device__ __forceinline__ int xcd_remap(int bid, int nb)
{
    const int per = nb >> 3;
    return (bid & 7) * per + (bid >> 3);
}

// Output tile (tm, tn) of tile index `tile`: tiles go in groups of 4 tile rows, and inside a
// group column by column, so the 32 tiles that run at the same time on one XCD (a contiguous
// range of indices) are 4 tile rows x 8 tile columns, which share more A and W rows in that
// XCD's L2 than two whole tile rows (measured: a few per cent on the projector and the SwiGLU
// step, neutral on the others).
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, int &tm, int &tn)
{
    constexpr int GM = 4;
    if (GM <= 1) {
        tm = tile / tiles_n;
        tn = tile - tm * tiles_n;
        return;
    }
    const int grp = tile / (GM * tiles_n), first = grp * GM;
    const int rows = tiles_m - first < GM ? tiles_m - first : GM;
    const int r = tile - grp * GM * tiles_n;
    tm = first + r % rows;
    tn = r / rows;
}

// 16-byte global -> LDS copy; lane l writes LDS byte address lds + 16 l (lds wave-uniform).
// m0 needs one wait state before the copy reads it.
__device__ __forceinline__ void copy16(const void *g, uint32_t lds)
{
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     ::"v"(g), "s"(lds) : "memory", "m0");
}

// 12-byte global -> LDS copy of base + off (base wave-uniform, off per lane, 4-byte aligned);
// lane l writes LDS bytes lds + 16 l .. lds + 16 l + 11 (the lanes keep a 16-byte pitch, as
// measured; the 4 bytes after each are left as they were).
__device__ __forceinline__ void copy12(const void *base, uint32_t off, uint32_t lds)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
    __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx3 %0, %1"
                     ::"v"(off), "s"(ub), "s"(lds) : "memory", "m0");
}

// 16-byte global -> LDS copy of base + off (base wave-uniform, off per lane); lane l writes LDS
// byte address lds + 16 l.
__device__ __forceinline__ void copy16_so(const void *base, uint32_t off, uint32_t lds)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
    __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     ::"v"(off), "s"(ub), "s"(lds) : "memory", "m0");
}

// s_waitcnt vmcnt(N) lgkmcnt(0): all but this wave's newest N global loads done, LDS reads done.
template <int N>
__device__ __forceinline__ void wait_vmem_n()
{
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N): all but this wave's newest N global loads done (LDS operations not waited for).
template <int N>
__device__ __forceinline__ void wait_vm_only()
{
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
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

// GELU, exact form: u Phi(u) = 0.5 u (1 + erf(u / sqrt 2)) (the official vision path, [Z]
// "End-to-end results and their limits": erf there, tanh in zLLM).
__device__ __forceinline__ float gelu_erf_big(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }

// SiLU: u sigmoid(u) = u / (1 + 2^(-u log2 e)); saturates to u and to -0 for large |u|.
__device__ __forceinline__ float silu_big(float u)
{
    return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u * -1.4426950408889634f));
}

// Bias of columns n..n+3 as four bf16 in a uint2 (zero without a bias and past N).  With
// N % 4 == 0, as in every encoder GEMM, it is one 8-byte load from a valid address (columns
// past N read the last four, and are never stored), with no branch on the column, so that
// an epilogue can issue the loads of all its columns before it waits for any of them.
__device__ __forceinline__ uint2 bias4(const bf16_t *bias, int N, int n)
{
    if (!bias) return make_uint2(0u, 0u);
    if ((N & 3) == 0) return *reinterpret_cast<const uint2 *>(bias + (n < N ? n : N - 4));
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = n + j < N ? (uint32_t)bias[n + j] : 0u;
    return make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
}

// r = v + bias (four bf16 in b), then the activation
template <int ACT>
__device__ __forceinline__ void add_act(uint2 b, const float *v, float *r)
{
    r[0] = v[0] + __uint_as_float(b.x << 16);
    r[1] = v[1] + __uint_as_float(b.x & 0xFFFF0000u);
    r[2] = v[2] + __uint_as_float(b.y << 16);
    r[3] = v[3] + __uint_as_float(b.y & 0xFFFF0000u);
    if (ACT == ACT_GELU_TANH)
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = gelu_tanh_big(r[j]);
    if (ACT == ACT_GELU_ERF)
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = gelu_erf_big(r[j]);
}

// bias (columns n..n+3; columns past N get none) and activation
template <int ACT>
__device__ __forceinline__ void bias_act(const bf16_t *bias, int N, int n, const float *v, float *r)
{
    add_act<ACT>(bias4(bias, N, n), v, r);
}

// bf16 output.  put(): 4 results -> 8 bytes at dst (LDS staging).  store(): 4 results of row
// m, columns n..n+3, straight to global memory with row and column bounds.
template <int ACT>
struct EpiBF16 {
    static constexpr int OUT_BYTES = 2;
    static constexpr bool CUSTOM = false, PAIRED = false, RESID = false;
    bf16_t *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ const bf16_t *bias_ptr() const { return bias; }
    __device__ __forceinline__ int ncols() const { return N; }
    __device__ __forceinline__ void put(char *dst, const float *v, uint2 b) const
    {
        float r[4];
        add_act<ACT>(b, v, r);
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

// 8 bf16 of x plus the 8 bf16 of d, each sum rounded to bf16 (round to nearest even).  The
// fp32 sum of two bf16 values is exact unless their exponents are far apart, and then the
// smaller one is far below half a bf16 unit of the larger: rounding via fp32 equals rounding
// the exact sum.
__device__ __forceinline__ uint4 add_bf16x8(uint4 x, uint4 d)
{
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ds[4] = {d.x, d.y, d.z, d.w};
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = pack_bf16x2(__uint_as_float(xs[i] << 16) + __uint_as_float(ds[i] << 16),
                           __uint_as_float(xs[i] & 0xFFFF0000u) + __uint_as_float(ds[i] & 0xFFFF0000u));
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// Residual update of the token stream by a block's projection ([Z] "Step 2" boundary table:
// the block output fixes the residual order; [Z] "Multimodal basics": pre-norm blocks):
//   x[m][n] = bf16(x[m][n] + bf16(acc + b[n]))
// the projection rounded to bf16 first, then the sum rounded again, as a separate residual
// add of the bf16 projection output would.  out is x itself, read and written in place:
// put() stages bf16(acc + b) and the row writer adds x on the way out.
struct EpiResid {
    static constexpr int OUT_BYTES = 2;
    static constexpr bool CUSTOM = false, PAIRED = false, RESID = true;
    bf16_t *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ const bf16_t *bias_ptr() const { return bias; }
    __device__ __forceinline__ int ncols() const { return N; }
    __device__ __forceinline__ void put(char *dst, const float *v, uint2 b) const
    {
        float r[4];
        add_act<ACT_NONE>(b, v, r);
        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
    }
    __device__ __forceinline__ void store(int64_t m, int n, const float *v) const
    {
        if (m >= M) return;
        float r[4];
        bias_act<ACT_NONE>(bias, N, n, v, r);
        bf16_t *o = out + m * N + n;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (n + j < N) o[j] = f32_to_bf16(bf16_to_f32(o[j]) + bf16_to_f32(f32_to_bf16(r[j])));
    }
};

struct EpiF32 {
    static constexpr int OUT_BYTES = 4;
    static constexpr bool CUSTOM = false, PAIRED = false, RESID = false;
    float *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ const bf16_t *bias_ptr() const { return bias; }
    __device__ __forceinline__ int ncols() const { return N; }
    __device__ __forceinline__ void put(char *dst, const float *v, uint2 b) const
    {
        float r[4];
        add_act<ACT_NONE>(b, v, r);
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
    static constexpr bool CUSTOM = false, PAIRED = false, RESID = false;
    float *out;
    __device__ __forceinline__ const bf16_t *bias_ptr() const { return nullptr; }
    __device__ __forceinline__ int ncols() const { return 4; }
    __device__ __forceinline__ void put(char *dst, const float *v, uint2) const
    {
        *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// SwiGLU gating of the official tower's MLP ([Z] "Comparing the DeepSeek V4.1 Flash and
// Qwen3-VL vision towers": RMSNorm and SwiGLU): h = bf16(silu(g) u), g and u the biased fp32
// results of the gate and up projections, rounded once.  The weight and bias hold the gate
// and up rows interleaved in groups of 8 (fused rows 16j .. 16j+7 = gate features 8j .. 8j+7,
// rows 16j+8 .. 16j+15 = up features 8j .. 8j+7).  A lane's accumulator block covers columns
// 8q + 4g .. 8q + 4g + 3 (q = 0..3) of a 32-column MFMA block, so blocks q = 0, 2 are gate
// values and q = 1, 3 the up values of the same 4 features: the gating needs no exchange.
// N is the fused width 2F; out is bf16 [M][N/2].
struct EpiSwiGLU {
    static constexpr int OUT_BYTES = 2;
    static constexpr bool CUSTOM = false, PAIRED = true, RESID = false;
    bf16_t *out;
    const bf16_t *bias;
    int64_t M;
    int N;
    __device__ __forceinline__ const bf16_t *bias_ptr() const { return bias; }
    __device__ __forceinline__ int ncols() const { return N; }
    // g, u: 4 gate and the matching 4 up results, bg, bu their biases -> 4 bf16 outputs at dst
    __device__ __forceinline__ void put2(char *dst, const float *g, const float *u, uint2 bg, uint2 bu) const
    {
        float rg[4], ru[4], h[4];
        add_act<ACT_NONE>(bg, g, rg);
        add_act<ACT_NONE>(bu, u, ru);
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = silu_big(rg[j]) * ru[j];
        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
    }
};

// (a, b) turned by the angle with cosine c and sine s; products and sums rounded separately.
__device__ __forceinline__ void rope_rotate(float a, float b, float c, float s, float &na, float &nb)
{
#pragma clang fp contract(off)
    na = a * c - b * s;
    nb = b * c + a * s;
}

// Index with bits 2 and 3 exchanged (an involution on 0..15 inside each group of 16).
__device__ __forceinline__ int swap23(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// bf16 bit pattern -> binary16 bit pattern (round to nearest even, saturating at 65504).
__device__ __forceinline__ uint32_t bf16_to_f16_sat(uint32_t b)
{
    float f = __uint_as_float(b << 16);
    if (__builtin_fabsf(f) > 65504.f) f = __builtin_copysignf(65504.f, f);
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// QKV projection with the 2D rotary embedding and the V^T relayout in the epilogue ([Z]
// "Step 3": angles blocked by axis, theta = [h f_0 .. h f_{Q-1}, w f_0 .. w f_{Q-1}] with
// Q = hd/4, rotation of element i with i + hd/2; [G] V4 Flash vision row: raw patch grid).
// The staged tile holds bf16(acc + bias), i.e. the bf16 qkv values; from there:
//   q columns: rotated, rounded to bf16, stored in place of q;
//   k columns: rotated, rounded to bf16, then stored as binary16 (the attention's score
//              operand type; exact for bf16 magnitudes 2^-14 .. 65504, larger saturate);
//   v columns: stored transposed as binary16, vt[head][d][col], where image i owns the
//              columns from its 64-aligned offset and inside each group of 16 columns, column
//              p holds key (p with bits 2 and 3 swapped); with store_v also kept as bf16 in
//              the qkv rows.  Columns past an image's last patch are not written here.
// Patch p of an image sits at (p / gw, p % gw) of its grid; cos/sin come from tables
// [position][hd/4] built on the host.
template <int HD>
struct EpiQKVRope {
    static constexpr int OUT_BYTES = 2;
    static constexpr bool CUSTOM = true, PAIRED = false, RESID = false;
    bf16_t *out;        // [M][3D]
    const bf16_t *bias;
    int64_t M;
    int N;              // 3D
    int D;
    uint16_t *vt;
    int64_t ldv;
    const ImgDesc *imgs;
    int n_img;
    const float *cos_t, *sin_t;
    int store_v;
    __device__ __forceinline__ const bf16_t *bias_ptr() const { return bias; }
    __device__ __forceinline__ int ncols() const { return N; }
    __device__ __forceinline__ void put(char *dst, const float *v, uint2 b) const
    {
        float r[4];
        add_act<ACT_NONE>(b, v, r);
        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
    }
    // Bytes of LDS past the staged tile that the epilogue uses: (row, column) on the image's
    // patch grid of every tile row.
    template <int BM>
    static constexpr int extra_lds() { return BM * 8; }
    // Before the staging barrier: grid position of each tile row into `pos`.
    template <int BM, int NT>
    __device__ __forceinline__ void prepare(char *pos, int64_t m0, int rows, int tid) const
    {
        for (int r = tid; r < rows; r += NT) reinterpret_cast<int2 *>(pos)[r] = patch_grid_pos(imgs, n_img, m0 + r);
    }
    template <int BM, int BN, int NT>
    __device__ __forceinline__ void write(const char *smem, int pitch, int64_t m0, int n0, int rows, int tid) const
    {
        constexpr int HALF = HD / 2, HC = HALF / 8, NHB = BN / HD;
        static_assert(HD >= 16 && BN % HD == 0, "head blocks must tile the column tile");
        const int2 *pos = reinterpret_cast<const int2 *>(smem + BM * pitch);
        // q and k (and v rows with store_v): item = (row, chunk of 8 elements of the first half
        // and the 8 they pair with); the chunk's 8 angles depend on the row alone, so they are
        // read once per item and serve every head block of the tile.  The items of one row are
        // consecutive lanes.
        for (int w = tid; w < BM * HC; w += NT) {
            const int r = w / HC, ch = w - r * HC;
            if (r >= rows) continue;
            const int64_t row = m0 + r;
            float cs[8], sn[8];
            if (n0 < 2 * D) rope_cos_sin8<HD>(cos_t, sin_t, pos[r], ch * 8, cs, sn);   // q or k columns
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
                const int c0 = n0 + hb * HD;
                if (c0 >= N) break;
                const int part = c0 / D;
                const char *src = smem + r * pitch + (hb * HD + ch * 8) * 2;
                bf16_t *dst = out + row * N + c0 + ch * 8;
                const uint4 ua = *reinterpret_cast<const uint4 *>(src);
                const uint4 ub = *reinterpret_cast<const uint4 *>(src + HALF * 2);
                if (part == 2) {
                    if (store_v) {
                        *reinterpret_cast<uint4 *>(dst) = ua;
                        *reinterpret_cast<uint4 *>(dst + HALF) = ub;
                    }
                    continue;
                }
                const uint32_t wa[4] = {ua.x, ua.y, ua.z, ua.w}, wb[4] = {ub.x, ub.y, ub.z, ub.w};
                float na[8], nb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = __uint_as_float(e & 1 ? wa[e >> 1] & 0xFFFF0000u : wa[e >> 1] << 16);
                    const float y = __uint_as_float(e & 1 ? wb[e >> 1] & 0xFFFF0000u : wb[e >> 1] << 16);
                    rope_rotate(x, y, cs[e], sn[e], na[e], nb[e]);
                }
                uint32_t pa[4], pb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pa[j] = pack_bf16x2(na[2 * j], na[2 * j + 1]);
                    pb[j] = pack_bf16x2(nb[2 * j], nb[2 * j + 1]);
                    if (part == 1) {
                        pa[j] = bf16_to_f16_sat(pa[j] & 0xFFFFu) | (bf16_to_f16_sat(pa[j] >> 16) << 16);
                        pb[j] = bf16_to_f16_sat(pb[j] & 0xFFFFu) | (bf16_to_f16_sat(pb[j] >> 16) << 16);
                    }
                }
                *reinterpret_cast<uint4 *>(dst) = make_uint4(pa[0], pa[1], pa[2], pa[3]);
                *reinterpret_cast<uint4 *>(dst + HALF) = make_uint4(pb[0], pb[1], pb[2], pb[3]);
            }
        }
        // V^T: per image in the tile, item = (run of 4 keys 4c..4c+3 of the image, 8 head dims).
        // The bit swap keeps each 4-aligned run on 4 consecutive columns, so a whole run is one
        // 8-byte store per dim; a run cut by the tile or the image end is stored per key.  The
        // lane reads the run's 4 tile rows as 16-byte pieces (dims o*8 .. o*8+7), so the LDS
        // reads of a wave spread over all banks.
        const int ilo = image_of_patch(imgs, n_img, m0), ihi = image_of_patch(imgs, n_img, m0 + rows - 1);
        constexpr int OCT = HD / 8;
        for (int hb = 0; hb < NHB; ++hb) {
            const int c0 = n0 + hb * HD;
            if (c0 >= N || c0 < 2 * D) continue;
            const int head = (c0 - 2 * D) / HD;
            for (int i = ilo; i <= ihi; ++i) {
                const int off = imgs[i].patch_off, n = imgs[i].n, voff = imgs[i].vt_off;
                const int klo = (int)max((int64_t)0, m0 - off);
                const int khi = (int)min((int64_t)n, m0 + rows - off);
                if (klo >= khi) continue;
                const int c_lo = klo >> 2, nruns = ((khi - 1) >> 2) - c_lo + 1;
                for (int w = tid; w < nruns * OCT; w += NT) {
                    const int o = w % OCT, k0 = 4 * (c_lo + w / OCT);
                    uint32_t h[4][4];   // [key e][dim pair]
                    bool whole = true;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int k = k0 + e;
                        if (k < klo || k >= khi) {
                            whole = false;
#pragma unroll
                            for (int j = 0; j < 4; ++j) h[e][j] = 0;
                            continue;
                        }
                        const int r = (int)(off + k - m0);
                        const uint4 u = *reinterpret_cast<const uint4 *>(smem + r * pitch + (hb * HD + o * 8) * 2);
                        h[e][0] = u.x, h[e][1] = u.y, h[e][2] = u.z, h[e][3] = u.w;
                    }
                    const int pc = swap23(k0);
                    uint16_t *vrow = vt + ((int64_t)head * HD + o * 8) * ldv + voff + pc;
#pragma unroll
                    for (int dd = 0; dd < 8; ++dd) {
                        uint32_t f[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[e] = bf16_to_f16_sat((h[e][dd >> 1] >> ((dd & 1) * 16)) & 0xFFFFu);
                        uint16_t *dst = vrow + (int64_t)dd * ldv;
                        if (whole) {
                            *reinterpret_cast<uint2 *>(dst) = make_uint2(f[0] | (f[1] << 16), f[2] | (f[3] << 16));
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (k0 + e >= klo && k0 + e < khi) dst[e] = (uint16_t)f[e];
                        }
                    }
                }
            }
        }
    }
};

// Zeros of the transposed-V columns past each image's last patch (up to its 64-aligned end),
// which the attention reads as masked keys.  One thread per (image, row of vt).
__global__ __launch_bounds__(256) void vt_tail_zero_kernel(uint16_t *__restrict__ vt, int64_t ldv,
                                                           const ImgDesc *__restrict__ imgs, int rows)
{
    const int r = blockIdx.y * 256 + threadIdx.x;
    if (r >= rows) return;
    const ImgDesc d = imgs[blockIdx.x];
    uint16_t *row = vt + (int64_t)r * ldv + d.vt_off;
    const int end = (d.n + 63) / 64 * 64;
    for (int k = d.n; k < end; ++k) row[swap23(k)] = 0;
}

// LDS a launch needs for its epilogue: the staged tile plus what a custom epilogue asks for.
template <class EP, bool C = EP::CUSTOM>
struct EpiExtra {
    template <int BM, int PITCH>
    static constexpr int bytes() { return 0; }
};
template <class EP>
struct EpiExtra<EP, true> {
    template <int BM, int PITCH>
    static constexpr int bytes() { return BM * PITCH + EP::template extra_lds<BM>(); }
};

// Work split of one launch: tiles [0, full) are computed whole; when splits > 1 the remaining
// tiles are cut into `splits` K slices each (items = leftover tiles x splits, block count
// rounded up to items_pad, a multiple of 8) whose fp32 partials go to `part`.
struct SplitK {
    int full, splits, items, items_pad;
    float *part;
};

template <int BM, int BN, class SRC, class EP, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gemm_big_kernel(SRC src, const bf16_t *__restrict__ W,
                                                              int N, int K, EP ep, int tiles_m,
                                                              int tiles_n, SplitK sk)
{
    static_assert(NW == 8 || (NW == 4 && std::is_same<SRC, SrcPlain>::value && BN == 256 && (BM == 256 || BM == 192)),
                  "8 waves, or 4 for 256 x 256 and 192 x 256 tiles of plain activations");
    static_assert(NW == 4 || BM != 192, "192-row tiles run on 4 waves");
    constexpr int NT = NW * 64, NWN = 2;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
    constexpr int CPR = BK / 8;                             // 16-byte chunks per LDS row
    constexpr int AL = BM * CPR / 256, BL = BN * CPR / 256;  // copies per thread of its group
    constexpr int WM = BM / (NW / 2), WN = BN / NWN, TM = WM / 32, TN = WN / 32;
    static_assert(AL >= 1 && BL >= 1 && TM >= 1 && TN >= 1, "bad tile");
    // the output tile is staged in LDS for the final writes when it fits (fp32 partial tiles
    // of split slices always use BN = 128); the staging area overlays the copy ring
    constexpr int OB = EP::OUT_BYTES, PITCH = BN * OB + 16, PPITCH = BN * 4 + 16;
    constexpr bool STAGED = BM * PITCH <= 160 * 1024;
    constexpr bool PSTAGED = BM * PPITCH <= 160 * 1024;
    constexpr int SMEM0 = (STAGED && BM * PITCH > NS * STAGE) ? BM * PITCH : NS * STAGE;
    constexpr int SMEM1 = (PSTAGED && BM * PPITCH > SMEM0) ? BM * PPITCH : SMEM0;
    constexpr int SMEM2 = EpiExtra<EP>::template bytes<BM, PITCH>() > SMEM1 ? EpiExtra<EP>::template bytes<BM, PITCH>() : SMEM1;
    // pixel A: two raw k-tiles (a 16-byte slot per chunk, BM * CPR chunks) after the ring, free
    // again before the epilogue stages its tile
    constexpr int RAWB = BM * CPR * 16;
    constexpr int SMEM = SRC::REG && NS * STAGE + 2 * RAWB > SMEM2 ? NS * STAGE + 2 * RAWB : SMEM2;
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
    int tm, tn;
    tile_coords(tile, tiles_m, tiles_n, tm, tn);
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
    // 8 waves: group 0 = waves 0-3, group 1 = waves 4-7; 4 waves: one group
    const int grp = NW == 8 ? wave >> 2 : 0, w4 = wave & 3;
    const int wm = NW == 8 ? grp * 2 + (w4 >> 1) : wave >> 1, wn = w4 & 1;

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

    if constexpr (NW == 4) {
        // One wave per SIMD with a (BM/2) x 128 output tile (128 x 128: half the LDS fragment
        // reads per MFMA of the 8-wave form), whole tiles only (no K slices).  K-tiles are 64 wide, so each
        // LDS row is one 128-byte line of A or W and every copy fetches whole lines; two LDS
        // stages of 64 KB.  Chunk c = (i * 4 + wave) * 64 + lane of a tile holds row c / 8,
        // logical chunk (c % 8) ^ ((row / 2) % 8): 16 consecutive rows of one ds_read_b128 pass
        // hit 16 distinct 16-byte bank groups.  The copies take a wave-uniform base (the
        // operand plus the k offset, in scalar registers) and a loop-invariant 32-bit offset per
        // lane, so the loop has no address arithmetic.  Step t (stage t % 2): sub-steps 0..2 of
        // k-tile t, each interleaved with the fragment reads of the next; wait for this wave's
        // copies of k-tile t+1 and its reads; barrier; sub-step 3, interleaved with the reads
        // of k-tile t+1's first sub-step and the copies of k-tile t+2 into stage t % 2.
        constexpr int KB = 64, CPR4 = KB / 8, A4 = BM * KB * 2, ST4 = (BM + BN) * KB * 2;
        constexpr int AL4 = BM * CPR4 / 256, BL4 = BN * CPR4 / 256, NC = AL4 + BL4, NF = TM + TN, NM = TM * TN;
        static_assert(2 * ST4 <= NS * STAGE, "two 64-wide stages fit the ring");
        auto swz8 = [](int r) { return (r >> 1) & 7; };
        // byte offsets of this lane's chunks from the operands' first rows (the host keeps both
        // operands under 2^31 bytes); rows past M (N) read row M-1 (N-1)
        uint32_t aoff[AL4], woff[BL4];
#pragma unroll
        for (int i = 0; i < AL4; ++i) {
            const int c = (i * 4 + wave) * 64 + lane, r = c / CPR4;
            const int64_t row = m0 + r < src.M ? m0 + r : src.M - 1;
            aoff[i] = (uint32_t)((row * src.lda + ((c % CPR4) ^ swz8(r)) * 8) * 2);
        }
#pragma unroll
        for (int i = 0; i < BL4; ++i) {
            const int c = (i * 4 + wave) * 64 + lane, r = c / CPR4;
            const int n = n0 + r < N ? n0 + r : N - 1;
            woff[i] = (uint32_t)(((int64_t)n * K + ((c % CPR4) ^ swz8(r)) * 8) * 2);
        }
        const int kb0 = kt0 * BK / KB, nkb = nk * BK / KB;
        auto slot_lds = [&](auto sl) -> uint32_t {
            return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)(smem + decltype(sl)::value * ST4);
        };
        auto cp = [&](int kt, auto sl, int x) __attribute__((always_inline)) {
            const int k0 = (kb0 + kt) * KB;
            if (x < AL4)
                copy16_so(src.A + k0, aoff[x], slot_lds(sl) + (x * 4 + wave) * 1024);
            else
                copy16_so(W + k0, woff[x - AL4], slot_lds(sl) + A4 + ((x - AL4) * 4 + wave) * 1024);
        };
        int lo[KB / 16];
#pragma unroll
        for (int ks = 0; ks < KB / 16; ++ks) lo[ks] = l32 * (KB * 2) + (((2 * ks + g) ^ ((l32 >> 1) & 7)) * 16);
        bf16x8_t fa[2][TM], fb[2][TN];
        auto rd = [&](auto sl, auto ksc, int x) __attribute__((always_inline)) {
            constexpr int KS = decltype(ksc)::value;
            const char *sa = smem + decltype(sl)::value * ST4;
            if (x < TM)
                fa[KS & 1][x] = *reinterpret_cast<const bf16x8_t *>(sa + (wm * WM + x * 32) * (KB * 2) + lo[KS]);
            else
                fb[KS & 1][x - TM] = *reinterpret_cast<const bf16x8_t *>(sa + A4 + (wn * WN + (x - TM) * 32) * (KB * 2) + lo[KS]);
        };
        using Z0 = std::integral_constant<int, 0>;
        using Z1 = std::integral_constant<int, 1>;
        auto step = [&](int t, auto sl) __attribute__((always_inline)) {
            constexpr int S = decltype(sl)::value;
            using SN = std::integral_constant<int, S ^ 1>;
            each_stage(std::make_integer_sequence<int, 3>{}, [&](auto ksc) {
                constexpr int KS = decltype(ksc)::value;
#pragma unroll
                for (int x = 0; x < (NM > NF ? NM : NF); ++x) {
                    if (x < NM) acc[x / TN][x % TN] = mfma32(fb[KS & 1][x % TN], fa[KS & 1][x / TN], acc[x / TN][x % TN]);
                    if (x < NF) rd(sl, std::integral_constant<int, KS + 1>{}, x);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
            wait_vmem_n<0>();
            sync();
            const int kc = min(t + 2, nkb - 1);
#pragma unroll
            for (int x = 0; x < (NM > NC ? NM : NC); ++x) {
                if (x < NM) acc[x / TN][x % TN] = mfma32(fb[1][x % TN], fa[1][x / TN], acc[x / TN][x % TN]);
                if (x < NF) rd(SN{}, Z0{}, x);
                if (x < NC) cp(kc, sl, x);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
#pragma unroll
        for (int x = 0; x < NC; ++x) cp(0, Z0{}, x);
#pragma unroll
        for (int x = 0; x < NC; ++x) cp(min(1, nkb - 1), Z1{}, x);
        wait_vmem_n<NC>();
        sync();
#pragma unroll
        for (int x = 0; x < NF; ++x) rd(Z0{}, Z0{}, x);
        int kt = 0;
        for (; kt + 1 < nkb; kt += 2) {
            step(kt, Z0{});
            step(kt + 1, Z1{});
        }
        if (kt < nkb) step(kt, Z0{});
        wait_vmem_n<0>();
        sync();
    } else {

    // group 0 copies the A tile, group 1 the W tile; chunk c = (i*4 + w4)*64 + lane of a tile
    // holds row c / CPR, logical chunk (c % CPR) ^ swz(row)
    // Register-staged A (pixel sources): both groups convert, group g the chunks
    // i = g AH .. g AH + AH - 1 (AH = AL / 2) of the same layout, and group 1 still copies W.
    constexpr int AH = SRC::REG ? AL / 2 : AL;
    static_assert(!SRC::REG || AL % 2 == 0, "the pixel chunks split evenly between the groups");
    typename SRC::Row arow[AL];
    int aslot[AL];
    const bf16_t *wptr[BL];
    if constexpr (SRC::REG) {
#pragma unroll
        for (int h = 0; h < AH; ++h) {
            const int i = grp * AH + h, c = (i * 4 + w4) * 64 + lane, r = c / CPR;
            arow[h] = src.row(m0 + r);
        }
    }
    if (grp == 0) {
        if constexpr (!SRC::REG) {
#pragma unroll
            for (int i = 0; i < AL; ++i) {
                const int c = (i * 4 + w4) * 64 + lane, r = c / CPR;
                arow[i] = src.row(m0 + r);
                aslot[i] = ((c % CPR) ^ swz(r)) * 8;
            }
        }
    }
    if (grp == 1) {
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            const int c = (i * 4 + w4) * 64 + lane, r = c / CPR;
            const int n = n0 + r < N ? n0 + r : N - 1;
            wptr[i] = W + (int64_t)n * K + ((c % CPR) ^ swz(r)) * 8;
        }
    }
    // The 12 raw bytes of each chunk of k-tile j go global -> LDS into raw slot j % 2 (each lane
    // reads back only what its own copy wrote, so no barrier), are converted two steps later
    // and written into their stage.  The thread's chunk of every row it fills is logical chunk alj; ash keeps
    // each chunk's first byte inside its dwords.
    uint32_t ash[2][SRC::REG ? AH : 1];
    constexpr int PL = AH;   // raw copies per k-tile of a thread (one 12-byte copy per chunk)
    const int alj = (lane & 3) ^ ((lane >> 4) & 3);
    typename SRC::Consts acs{};
    if constexpr (SRC::REG) acs = src.consts();
    // raw slot b: chunk i (0 .. AL-1) of wave w4 at (i * 4 + w4) * 1024 + 16 lane
    auto raw_at = [&](int b, int i) -> char * { return smem + NS * STAGE + b * RAWB + (i * 4 + w4) * 1024; };
    auto load_a = [&](int kt, auto buf) __attribute__((always_inline)) {
        if constexpr (SRC::REG) {
            constexpr int B = decltype(buf)::value;
            const auto kc = src.chunk((kt0 + kt) * BK + 8 * alj, acs);
#pragma unroll
            for (int h = 0; h < AH; ++h) {
                const auto a = src.addr(arow[h], kc);
                ash[B][h] = a.sh;
                copy12(src.px, a.o, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)raw_at(B, grp * AH + h));
            }
        }
    };
    auto put_a = [&](int kt, auto st, auto buf) __attribute__((always_inline)) {
        if constexpr (SRC::REG) {
            constexpr int B = decltype(buf)::value;
            const auto kc = src.chunk((kt0 + kt) * BK + 8 * alj, acs);
#pragma unroll
            for (int h = 0; h < AH; ++h) {
                const int i = grp * AH + h;
                const uint3 r3 = *reinterpret_cast<const uint3 *>(raw_at(B, i) + lane * 16);
                const RawChunk d{r3.x, r3.y, r3.z, ash[B][h]};
                *reinterpret_cast<uint4 *>(stage(st) + (i * 4 + w4) * 1024 + lane * 16) = src.convert(kc, d);
            }
        }
    };
    auto issue = [&](int kt, auto st) __attribute__((always_inline)) {
        const int k0 = (kt0 + kt) * BK;
        if (grp == 0) {
            if constexpr (!SRC::REG) {
#pragma unroll
                for (int i = 0; i < AL; ++i)
                    copy16(src.addr(arow[i], k0 + aslot[i]), stage_lds(st) + (i * 4 + w4) * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < BL; ++i) copy16(wptr[i] + k0, stage_lds(st) + A_BYTES + (i * 4 + w4) * 1024);
        }
    };
    // this wave's copies of all but the newest NS-2 k-tiles landed, and its LDS reads and writes
    // done.  Register-staged A: a step issues the raw copies of k-tile t+NS+2 and then (group 1)
    // the W copies of k-tile t+NS, so the newest two of each may stay in flight.
    static_assert(NS % 2 == 0 && NS - 2 == 2, "the raw A slots alternate with the stage parity");
    auto wait_ring = [&]() {
        if (grp == 0) {
            if constexpr (SRC::REG) wait_vmem_n<2 * PL>();
            else wait_vmem_n<(NS - 2) * AL>();
        } else {
            if constexpr (SRC::REG) wait_vmem_n<2 * PL + 2 * BL>();
            else wait_vmem_n<(NS - 2) * BL>();
        }
    };
    // before converting raw k-tile t+NS (copied two steps ago): only the raw copies of k-tile
    // t+NS+1 and (group 1) the W copies issued since may still be in flight.  Group 1 issues W
    // copies from step 0 on, after the raw copies of that step: before step 2 fewer of them
    // follow the raw k-tile being converted (none in step 0, one k-tile in step 1; the raw
    // copies of k-tiles NS and NS+1 came from the prologue), so the count is exact per step --
    // a larger one would let the conversion read a raw slot before its bytes land.
    auto wait_raw = [&](int t) {
        if (grp == 0) wait_vm_only<PL>();
        else if (t >= 2) wait_vm_only<PL + 2 * BL>();
        else if (t == 1) wait_vm_only<PL + BL>();
        else wait_vm_only<PL>();
        __asm__ volatile("" ::: "memory");   // the raw reads stay below the wait
    };
    bf16x8_t fa[BK / 16][TM], fb[BK / 16][TN];
    auto ldfrag = [&](auto st) __attribute__((always_inline)) {
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
    auto mma = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fb[ks][j], fa[ks][i], acc[i][j]);
        __builtin_amdgcn_s_setprio(0);
    };

    // K-tile t lives in stage t % NS: group 0 reads it in phase 2t-1, group 1 in phase 2t, and
    // both refill it (with k-tile t+NS) in phases 2t+1 and 2t+2.  Past the last k-tile the
    // copies repeat the last one into the free stage, so every phase waits for the same count.
    using I0 = std::integral_constant<int, 0>;
    constexpr auto stages = std::make_integer_sequence<int, NS>{};
    each_stage(stages, [&](auto st) { issue(min((int)decltype(st)::value, nk - 1), st); });
    if constexpr (SRC::REG) {
        // stages 0 .. NS-1 converted with two raw k-tiles in flight (each wait also covers the
        // W copies above); leaves raw k-tiles NS, NS+1 in flight
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        load_a(0, B0{});
        load_a(min(1, nk - 1), B1{});
        each_stage(stages, [&](auto st) {
            using B = std::integral_constant<int, decltype(st)::value % 2>;
            wait_vm_only<PL>();
            __asm__ volatile("" ::: "memory");   // the raw reads stay below the wait
            put_a(min((int)decltype(st)::value, nk - 1), st, B{});
            load_a(min((int)decltype(st)::value + 2, nk - 1), B{});
        });
        __asm__ volatile("" ::: "memory");   // the stage writes stay above the wait below
        wait_vmem_n<2 * PL>();
    } else {
        if (grp == 0) wait_vmem_n<(NS - 1) * AL>();
        else wait_vmem_n<(NS - 1) * BL>();
    }
    sync();
    ldfrag(I0{});
    if (grp == 1) {   // group 1 runs one phase behind
        wait_ring();
        sync();
    }
    auto step = [&](int t, auto st) __attribute__((always_inline)) {
        constexpr int S = decltype(st)::value;
        mma();
        wait_ring();
        sync();
        if (t + 1 < nk) ldfrag(std::integral_constant<int, (S + 1) % NS>{});
        if constexpr (SRC::REG) {   // raw k-tile t+NS (copied two steps ago) into stage S; copy t+NS+2
            using B = std::integral_constant<int, S % 2>;
            wait_raw(t);
            put_a(min(t + NS, nk - 1), std::integral_constant<int, S>{}, B{});
            load_a(min(t + NS + 2, nk - 1), B{});
        }
        issue(min(t + NS, nk - 1), std::integral_constant<int, S>{});
        if constexpr (SRC::REG) __asm__ volatile("" ::: "memory");   // the stage writes stay above wait_ring
        wait_ring();
        sync();
    };
    if constexpr (SRC::REG) {
        // whole groups of NS steps first: with no skipped step inside the loop body, the
        // compiler's count of the raw loads still in flight stays exact (its waits before the
        // conversions then leave the newest raw k-tile loading)
        int kt = 0;
        for (; kt + NS <= nk; kt += NS) each_stage(stages, [&](auto st) { step(kt + decltype(st)::value, st); });
        each_stage(stages, [&](auto st) {
            if (kt + decltype(st)::value < nk) step(kt + decltype(st)::value, st);
        });
    } else {
        for (int kt = 0; kt < nk; kt += NS)
            each_stage(stages, [&](auto st) {
                if (kt + decltype(st)::value < nk) step(kt + decltype(st)::value, st);
            });
    }
    if (grp == 0) sync();   // same barrier count as group 1
    wait_vmem_n<0>();       // the trailing copies of the last k-tile
    sync();
    }   // 8 waves

    // acc[i][j][r]: output row l32 of the 32-block, column 8*(r/4) + 4*g + r%4.
    // The bias of this lane's columns (the same for all its rows), loaded all at once: with a
    // bias and N % 4 == 0 (a uniform branch) as unconditional 8-byte loads with no wait between
    // them; otherwise column by column.
    auto bias_cols = [&](const auto &e, uint2 (*bpre)[4]) {
        const bf16_t *bp = e.bias_ptr();
        const int nc = e.ncols();
        if (bp && (nc & 3) == 0) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * g;
                    bpre[j][q] = *reinterpret_cast<const uint2 *>(bp + (n < nc ? n : nc - 4));
                }
        } else {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) bpre[j][q] = bias4(bp, nc, n0 + wn * WN + j * 32 + 8 * q + 4 * g);
        }
    };
    // Stage rows of `pitch` bytes in LDS via put(), then write whole rows of the tile.
    auto stage_tile = [&](const auto &e, int pitch, int ob) {
        uint2 bpre[TN][4];
        bias_cols(e, bpre);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                        acc[i][j][4 * q + 3]};
                    const int r = wm * WM + i * 32 + l32, c = wn * WN + j * 32 + 8 * q + 4 * g;
                    e.put(smem + r * pitch + c * ob, v, bpre[j][q]);
                    // accumulators are read as they are staged, not all at once up front
                    if (NW == 4) __builtin_amdgcn_sched_barrier(0);
                }
        __syncthreads();
    };
    // whole rows of a staged tile (tile_bytes per row) to global memory
    // A whole tile (every row, full width) reads all its chunks from LDS before it stores any,
    // so one wait covers the LDS latency of all of them; a partial tile goes chunk by chunk.
    // With a residual epilogue (bf16 tiles) each chunk is added to the bf16 values already at
    // its destination, whose loads are issued before the LDS reads.
    auto write_rows = [&](auto tbc, auto rsd, int pitch, char *gout, int64_t gpitch, int rows, int row_bytes) {
        constexpr int TB = decltype(tbc)::value, CH = TB / 16, IT = BM * CH / NT;
        constexpr bool RSD = decltype(rsd)::value;
        static_assert(BM * CH % NT == 0, "tile chunks must divide among the threads");
        if (rows == BM && row_bytes == TB) {
            uint4 val[IT], xv[IT];
            if constexpr (RSD) {
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int c = tid + it * NT, r = c / CH, b = (c % CH) * 16;
                    xv[it] = *reinterpret_cast<const uint4 *>(gout + r * gpitch + b);
                }
            }
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int c = tid + it * NT, r = c / CH, b = (c % CH) * 16;
                val[it] = *reinterpret_cast<const uint4 *>(smem + r * pitch + b);
            }
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int c = tid + it * NT, r = c / CH, b = (c % CH) * 16;
                if constexpr (RSD) val[it] = add_bf16x8(xv[it], val[it]);
                *reinterpret_cast<uint4 *>(gout + r * gpitch + b) = val[it];
            }
            return;
        }
        const int ch = CH;                                   // 16-byte chunks per tile row
#pragma unroll 4
        for (int c = tid; c < BM * ch; c += NT) {
            const int r = c / ch, b = (c % ch) * 16;
            if (r >= rows) break;
            uint4 val = *reinterpret_cast<const uint4 *>(smem + r * pitch + b);
            char *dst = gout + r * gpitch + b;
            if (b + 16 <= row_bytes) {
                if constexpr (RSD) val = add_bf16x8(*reinterpret_cast<const uint4 *>(dst), val);
                *reinterpret_cast<uint4 *>(dst) = val;
            } else if (b < row_bytes) {                    // ragged right edge, 2-byte pieces
                const uint16_t *s16 = reinterpret_cast<const uint16_t *>(smem + r * pitch + b);
                uint16_t *d16 = reinterpret_cast<uint16_t *>(dst);
                for (int e2 = 0; e2 < (row_bytes - b) / 2; ++e2) {
                    if constexpr (RSD)
                        d16[e2] = f32_to_bf16(bf16_to_f32(d16[e2]) + bf16_to_f32(s16[e2]));
                    else
                        d16[e2] = s16[e2];
                }
            }
        }
    };
    auto staged = [&](const auto &e, int pitch, int ob, char *gout, int64_t gpitch, int rows,
                      int row_bytes) {
        using E = std::decay_t<decltype(e)>;
        stage_tile(e, pitch, ob);
        write_rows(std::integral_constant<int, BN * E::OUT_BYTES>{}, std::integral_constant<bool, E::RESID>{}, pitch,
                   gout, gpitch, rows, row_bytes);
    };
    if (item >= 0) {   // K slice: raw fp32 partial tile, every row and column (host: BN = 128)
        if constexpr (PSTAGED)
            staged(EpiPart{}, PPITCH, 4, reinterpret_cast<char *>(sk.part + (int64_t)item * BM * BN),
                   (int64_t)BN * 4, BM, BN * 4);
        return;
    }
    if constexpr (EP::PAIRED) {
        // gating in registers: output column (wn WN + 32 j) / 2 + 8 p + 4 g of the tile takes
        // the gate block q = 2p and the up block q = 2p + 1; tile rows of BN/2 bf16
        constexpr int OPITCH = BN + 16;
        static_assert(BM * OPITCH <= SMEM, "paired staging exceeds the LDS of the kernel");
        uint2 bpre[TN][4];
        bias_cols(ep, bpre);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const float vg[4] = {acc[i][j][8 * p], acc[i][j][8 * p + 1], acc[i][j][8 * p + 2],
                                         acc[i][j][8 * p + 3]};
                    const float vu[4] = {acc[i][j][8 * p + 4], acc[i][j][8 * p + 5], acc[i][j][8 * p + 6],
                                         acc[i][j][8 * p + 7]};
                    const int r = wm * WM + i * 32 + l32, cb = wn * WN + j * 32;
                    ep.put2(smem + r * OPITCH + (cb / 2 + 8 * p + 4 * g) * 2, vg, vu, bpre[j][2 * p], bpre[j][2 * p + 1]);
                    if (NW == 4) __builtin_amdgcn_sched_barrier(0);
                }
        __syncthreads();
        const int rows = (int)(ep.M - m0 < BM ? ep.M - m0 : BM);
        const int row_bytes = N - n0 < BN ? N - n0 : BN;     // (fused columns / 2) x 2 bytes
        write_rows(std::integral_constant<int, BN>{}, std::false_type{}, OPITCH,
                   reinterpret_cast<char *>(ep.out) + (m0 * (N / 2) + n0 / 2) * 2,
                   (int64_t)N, rows, row_bytes);
    } else if constexpr (EP::CUSTOM) {
        static_assert(STAGED, "custom epilogues need the staged tile");
        const int rows_c = (int)(ep.M - m0 < BM ? ep.M - m0 : BM);
        ep.template prepare<BM, NT>(smem + BM * PITCH, m0, rows_c, tid);
        stage_tile(ep, PITCH, OB);
        ep.template write<BM, BN, NT>(smem, PITCH, m0, n0, (int)(ep.M - m0 < BM ? ep.M - m0 : BM), tid);
    } else {
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
}

// Sum of the K slices of the leftover tiles, in slice order, then the epilogue.  One thread
// per 4 columns of a row; a wave covers 256 consecutive columns (whole rows).
template <int BM, int BN, class EP>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(EP ep, int tiles_m, int tiles_n, SplitK sk)
{
    constexpr int Q = BN / 4;                              // column groups per row
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int left = sk.items / sk.splits;
    if (idx >= (int64_t)left * BM * Q) return;
    const int lt = (int)(idx / (BM * Q)), rem = (int)(idx - (int64_t)lt * BM * Q);
    const int r = rem / Q, cq = rem - r * Q;
    int tm, tn;
    tile_coords(sk.full + lt, tiles_m, tiles_n, tm, tn);
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
// r = T mod P tiles (all T tiles when T < P) leaves P - r CUs idle for a whole tile time;
// cutting those r tiles into s K slices shortens that round to about 1/s of a tile time, at
// the cost of writing and reading back r*s fp32 partial tiles.  Costs are modelled with the measured time of one
// 32-wide k-step of a 256 x 128 tile (about 0.5 us) and 4 TB/s for the partial traffic; the
// split is used when it saves at least 5 us.  Only 256 x 128 tiles with bf16 or fp32 output
// and N % 4 == 0 are split.
SplitK plan_split(int64_t M, int N, int K, int BM, int BN, bool allowed)
{
    SplitK sk{0, 1, 0, 0, nullptr};
    const int64_t tiles = ceil_div(M, BM) * ceil_div(N, BN);
    const int P = cu_count();
    if (!allowed || BN != 128 || (N & 3) != 0 || P % 8 != 0) return sk;
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

// Plain activations and a weight whose bytes stay under 2^31 (32-bit per-lane offsets).
template <class SRC>
bool plain_small(const SRC &src, int N, int K)
{
    if constexpr (std::is_same<SRC, SrcPlain>::value)
        return src.M * src.lda * 2 < ((int64_t)1 << 31) && (int64_t)N * K * 2 < ((int64_t)1 << 31);
    return false;
}

// 256 x 256 tiles of plain activations run on 4 waves (one per SIMD, 64-wide k-tiles; measured
// on the 9216-patch layer: QKV 78 -> 68 us, fc1 102 -> 94 us, SwiGLU step 172 -> 157 us, bitwise
// equal results); the other shapes and sources on 8.
template <int BM, int BN, class SRC, class EP>
hipError_t launch_big(dim3 grid, SRC src, const bf16_t *W, int N, int K, EP ep, int tiles_m, int tiles_n,
                      SplitK sk, hipStream_t s)
{
    if constexpr (BM == 192) {   // chosen only for plain activations under 2^31 bytes, whole tiles
        static_assert(BN == 256 && std::is_same<SRC, SrcPlain>::value, "192-row tiles: plain sources");
        if (sk.splits > 1 || !plain_small(src, N, K)) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_big_kernel<BM, BN, SRC, EP, 4>), grid, dim3(256), 0, s, src, W, N, K, ep, tiles_m,
                           tiles_n, sk);
        return hipGetLastError();
    } else {
    if constexpr (BM == 256 && BN == 256 && std::is_same<SRC, SrcPlain>::value) {
        if (sk.splits <= 1 && plain_small(src, N, K)) {
            hipLaunchKernelGGL((gemm_big_kernel<BM, BN, SRC, EP, 4>), grid, dim3(256), 0, s, src, W, N, K, ep,
                               tiles_m, tiles_n, sk);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_big_kernel<BM, BN, SRC, EP, 8>), grid, dim3(512), 0, s, src, W, N, K, ep, tiles_m,
                       tiles_n, sk);
    return hipGetLastError();
    }
}

template <int BM, int BN, class SRC, class EP>
hipError_t run_big(SRC src, const bf16_t *W, int64_t M, int N, int K, EP ep, const GemmWorkspace *ws,
                   hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    const int tiles_m = (int)ceil_div(M, BM), tiles_n = (int)ceil_div(N, BN);
    SplitK sk{0, 1, 0, 0, nullptr};
    if constexpr (!EP::CUSTOM && !EP::PAIRED) {   // custom and paired epilogues need whole tiles
        sk = plan_split(M, N, K, BM, BN, ws != nullptr);
        if (sk.splits > 1 && (size_t)sk.items * BM * BN * 4 > ws->bytes) sk = SplitK{0, 1, 0, 0, nullptr};
        if (sk.splits > 1) {
            sk.part = ws->part;
            const hipError_t e = launch_big<BM, BN>(dim3(sk.full + sk.items_pad), src, W, N, K, ep, tiles_m,
                                                   tiles_n, sk, s);
            if (e != hipSuccess) return e;
            const int64_t threads = (int64_t)(sk.items / sk.splits) * BM * (BN / 4);
            hipLaunchKernelGGL((gemm_split_reduce_kernel<BM, BN, EP>), dim3((unsigned)ceil_div(threads, 256)),
                               dim3(256), 0, s, ep, tiles_m, tiles_n, sk);
            return hipGetLastError();
        }
    }
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int grid = (int)(ceil_div(tiles, 8) * 8);
    return launch_big<BM, BN>(dim3(grid), src, W, N, K, ep, tiles_m, tiles_n, sk, s);
}

// 256 x 256 tiles when they give at least one full round of blocks, or, with K <= 2048, half
// a round: one partial round of the large tiles (their main loop runs about 1.4 times faster
// than that of 256 x 128 tiles) beats more rounds of smaller ones, measured on the out-projection
// of the 1024-token image (144 tiles, 40 -> 36 us) and the QKV and fc1 steps of the 384-token
// image (48 -> 44 and 49 -> 42 us); with long K the K-split tail of 256 x 128 tiles does better.
bool use_big_tiles(int64_t M, int N, int K)
{
    return ceil_div(M, 256) * ceil_div(N, 256) * (K <= 2048 ? 2 : 1) >= cu_count();
}

// The same operands and epilogue for rows m0.. of the output (A rows and output rows offset).
SrcPlain rows_from(const SrcPlain &s, int64_t m0) { return SrcPlain{s.A + m0 * s.lda, s.lda, s.M - m0}; }
template <int ACT>
EpiBF16<ACT> rows_from(const EpiBF16<ACT> &e, int64_t m0) { return EpiBF16<ACT>{e.out + m0 * e.N, e.bias, e.M - m0, e.N}; }
EpiF32 rows_from(const EpiF32 &e, int64_t m0) { return EpiF32{e.out + m0 * e.N, e.bias, e.M - m0, e.N}; }
EpiResid rows_from(const EpiResid &e, int64_t m0) { return EpiResid{e.out + m0 * e.N, e.bias, e.M - m0, e.N}; }
EpiSwiGLU rows_from(const EpiSwiGLU &e, int64_t m0) { return EpiSwiGLU{e.out + m0 * (e.N / 2), e.bias, e.M - m0, e.N}; }
SrcPatch rows_from(const SrcPatch &s, int64_t m0)
{
    SrcPatch r = s;
    r.m_base += m0;
    r.M -= m0;
    return r;
}

// Row tail of a multi-round launch (one block per CU): when the tiles of the last, partial
// round are whole rows of tiles, those rows run afterwards as 128 x 128 tiles, four times as
// many blocks of a quarter of the work, if they then fit in one round.  Returns the first
// row of that tail, or M when the launch is left as it is.
int64_t row_tail_start(int64_t M, int N, int BM, int BN)
{
    const int P = cu_count();
    const int64_t tiles_n = ceil_div(N, BN), tiles = ceil_div(M, BM) * tiles_n;
    if (tiles <= P || tiles % P == 0) return M;
    const int64_t main_tiles = tiles / P * P;
    if (main_tiles % tiles_n != 0) return M;
    const int64_t m_main = main_tiles / tiles_n * BM;
    if (ceil_div(M - m_main, 128) * ceil_div(N, 128) > P) return M;
    return m_main;
}

// A launch with BM x BN tiles, its partial last round of whole tile rows (if any) moved to a
// second launch of 128 x 128 tiles.  Launches that use the split-K tail keep it instead.
template <int BM, int BN, class SRC, class EP>
hipError_t run_rows(SRC src, const bf16_t *W, int64_t M, int N, int K, EP ep, const GemmWorkspace *ws,
                    hipStream_t s)
{
    const int64_t m_tail = plan_split(M, N, K, BM, BN, ws != nullptr).splits > 1 ? M : row_tail_start(M, N, BM, BN);
    if (m_tail == M) return run_big<BM, BN>(src, W, M, N, K, ep, ws, s);
    hipError_t e = run_big<BM, BN>(src, W, m_tail, N, K, ep, nullptr, s);
    if (e != hipSuccess) return e;
    return run_big<128, 128>(rows_from(src, m_tail), W, M - m_tail, N, K, rows_from(ep, m_tail), nullptr, s);
}

template <int BM, int BN, class EP>
hipError_t run_rows(SrcMerge src, const bf16_t *W, int64_t M, int N, int K, EP ep, const GemmWorkspace *ws,
                    hipStream_t s)
{
    return run_big<BM, BN>(src, W, M, N, K, ep, ws, s);
}

// Tile shape of a launch: 256 x 256 as use_big_tiles decides;
// 128 x 128 when 256 x 128 tiles would occupy at most half of the compute units and K is
// short (twice the blocks for the same work), or at any K when 128 x 128 tiles fill between
// three quarters and all of the compute units in one round (the 384-token image's fc2, K =
// 4096: 216 tiles in 40.5 us against 51.4 us for 112 tiles of 256 x 128 cut into two K slices
// plus their sum); 256 x 128 otherwise, with the K split of plan_split.
enum TileKind { TILES_256x256, TILES_128x128, TILES_256x128, TILES_192x256 };

// 192 x 256 tiles (4 waves, 96 x 128 per wave) for plain activations, when they leave less
// output area per compute unit over the launch's rounds than 256 x 256 tiles (rounds x tile
// rows, the 256 columns being common; the smaller tiles counted 1.1 times, their measured
// cost per output area), and they occupy at least half the compute units.  On the 9216-patch
// layer this takes the out-projection and fc2 (144 -> 192 tiles, 56 -> 75% of the compute
// units in their one round: 35.3 -> 32.3 and 104.6 -> 85.5 us), fc1 (576 tiles in 2.25
// rounds -> 768 in exactly 3: 92.5 -> 87.9 us) and the SwiGLU step (4.5 -> 6 rounds of
// smaller tiles); QKV keeps 256 x 256 (432 tiles: 2 rounds against 3), and so does fc1 of the
// 74,088-patch batch (19 rounds against 25 of 192 rows, 23.1 ms against 21.6 ms per pass).
bool use_192_tiles(int64_t M, int N, bool plain)
{
    if (!plain) return false;
    const int64_t P = cu_count();
    const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256), t192 = ceil_div(M, 192) * ceil_div(N, 256);
    if (t192 * 2 < P) return false;
    return ceil_div(t192, P) * 192 * 11 <= ceil_div(t256, P) * 256 * 10;
}

TileKind tile_kind(int64_t M, int N, int K, bool plain = false)
{
    if (use_big_tiles(M, N, K)) return use_192_tiles(M, N, plain) ? TILES_192x256 : TILES_256x256;
    if (use_192_tiles(M, N, plain)) return TILES_192x256;
    if (K <= 2048 && ceil_div(M, 256) * ceil_div(N, 128) * 2 <= cu_count()) return TILES_128x128;
    const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128);
    if (t128 <= cu_count() && t128 * 4 >= (int64_t)cu_count() * 3) return TILES_128x128;
    return TILES_256x128;
}

template <class SRC, class EP>
hipError_t run_shaped(SRC src, const bf16_t *W, int64_t M, int N, int K, EP ep, const GemmWorkspace *ws,
                      hipStream_t s)
{
    const bool plain = plain_small(src, N, K);
    switch (tile_kind(M, N, K, plain)) {
    case TILES_192x256:
        if constexpr (std::is_same<SRC, SrcPlain>::value) return run_rows<192, 256>(src, W, M, N, K, ep, ws, s);
        return hipErrorInvalidValue;
    case TILES_256x256: return run_rows<256, 256>(src, W, M, N, K, ep, ws, s);
    case TILES_128x128: return run_rows<128, 128>(src, W, M, N, K, ep, ws, s);
    default: return run_rows<256, 128>(src, W, M, N, K, ep, ws, s);
    }
}

template <class SRC>
hipError_t dispatch(SRC src, const bf16_t *W, int64_t M, int N, int K, const bf16_t *bias, int act,
                    bool out_f32, void *out, const GemmWorkspace *ws, hipStream_t s)
{
    if (out_f32) return run_shaped(src, W, M, N, K, EpiF32{(float *)out, bias, M, N}, ws, s);
    if (act == ACT_GELU_TANH) return run_shaped(src, W, M, N, K, EpiBF16<ACT_GELU_TANH>{(bf16_t *)out, bias, M, N}, ws, s);
    if (act == ACT_GELU_ERF) return run_shaped(src, W, M, N, K, EpiBF16<ACT_GELU_ERF>{(bf16_t *)out, bias, M, N}, ws, s);
    if (act == ACT_SWIGLU) return run_shaped(src, W, M, N, K, EpiSwiGLU{(bf16_t *)out, bias, M, N}, ws, s);
    return run_shaped(src, W, M, N, K, EpiBF16<ACT_NONE>{(bf16_t *)out, bias, M, N}, ws, s);
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

size_t linear_workspace_bytes(int64_t M, int K, int N, int act, bool out_f32)
{
    if (M <= 0 || (act == ACT_SWIGLU && !out_f32)) return 0;   // the paired epilogue never splits
    int BM = 256, BN = 128;
    switch (tile_kind(M, N, K, (int64_t)M * K * 2 < ((int64_t)1 << 31) && (int64_t)N * K * 2 < ((int64_t)1 << 31))) {
    case TILES_192x256:
    case TILES_256x256: return 0;                              // only BN = 128 tiles split
    case TILES_128x128: BM = 128; break;
    default: break;
    }
    const SplitK sk = plan_split(M, N, K, BM, BN, true);
    return sk.splits > 1 ? (size_t)sk.items * BM * BN * 4 : 0;
}


hipError_t launch_linear(const bf16_t *A, int64_t M, int K, const bf16_t *W, const bf16_t *bias,
                         int N, int act, bool out_f32, void *out, const GemmWorkspace *ws, hipStream_t s)
{
    return dispatch(SrcPlain{A, K, M}, W, M, N, K, bias, act, out_f32, out, ws, s);
}

hipError_t launch_linear_residual(const bf16_t *A, int64_t M, int K, const bf16_t *W, const bf16_t *bias, int N,
                                  bf16_t *x, const GemmWorkspace *ws, hipStream_t s)
{
    return run_shaped(SrcPlain{A, K, M}, W, M, N, K, EpiResid{x, bias, M, N}, ws, s);
}

hipError_t launch_patch_embed(const uint8_t *lpx, int64_t pix_first, int64_t pix_bytes, const ImgDesc *imgs,
                              int n_img, int64_t m_first, int64_t M, const float *s3, const float *t3, int ps,
                              const bf16_t *Wpe, int Kp, const bf16_t *bias, int D, bf16_t *out,
                              const GemmWorkspace *ws, hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    if (Kp != patch_gemm_k(ps) || ps > 64 || pix_bytes <= 0 || pix_bytes >= kPatchLaunchBytes)
        return hipErrorInvalidValue;
    const SrcPatch src = patch_source(lpx, pix_first, pix_bytes, imgs, n_img, m_first, M, s3, t3, ps);
    const EpiBF16<ACT_NONE> ep{out + m_first * D, bias, M, D};
    // The pixel conversion costs VALU work per A element, the MFMA work per A element grows
    // with BN: 256 x 256 tiles whenever they give a quarter of a round of blocks.
    if (ceil_div(M, 256) * ceil_div(D, 256) * 4 >= cu_count()) return run_rows<256, 256>(src, Wpe, M, D, Kp, ep, ws, s);
    return run_rows<128, 128>(src, Wpe, M, D, Kp, ep, ws, s);
}

template <int HD>
hipError_t run_qkv_rope(const bf16_t *A, int64_t M, int D, const bf16_t *W, const bf16_t *bias,
                        bf16_t *qkv, uint16_t *vt, int64_t ldv, const ImgDesc *imgs, int n_img,
                        const float *cos_t, const float *sin_t, bool store_v, hipStream_t s)
{
    const int N = 3 * D;
    EpiQKVRope<HD> ep{qkv, bias, M, N, D, vt, ldv, imgs, n_img, cos_t, sin_t, store_v ? 1 : 0};
    const SrcPlain src{A, D, M};
    if (use_192_tiles(M, N, plain_small(src, N, D))) return run_big<192, 256>(src, W, M, N, D, ep, nullptr, s);
    return use_big_tiles(M, N, D) ? run_big<256, 256>(src, W, M, N, D, ep, nullptr, s)
                                  : run_big<256, 128>(src, W, M, N, D, ep, nullptr, s);
}

hipError_t launch_qkv_rope(const bf16_t *A, int64_t M, int D, int H, const bf16_t *W, const bf16_t *bias,
                           bf16_t *qkv, uint16_t *vt, int64_t ldv, const ImgDesc *imgs, int n_img,
                           const float *cos_t, const float *sin_t, bool store_v, hipStream_t s)
{
    switch (D / H) {
    case 16: return run_qkv_rope<16>(A, M, D, W, bias, qkv, vt, ldv, imgs, n_img, cos_t, sin_t, store_v, s);
    case 32: return run_qkv_rope<32>(A, M, D, W, bias, qkv, vt, ldv, imgs, n_img, cos_t, sin_t, store_v, s);
    case 64: return run_qkv_rope<64>(A, M, D, W, bias, qkv, vt, ldv, imgs, n_img, cos_t, sin_t, store_v, s);
    case 128: return run_qkv_rope<128>(A, M, D, W, bias, qkv, vt, ldv, imgs, n_img, cos_t, sin_t, store_v, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_vt_tail_zero(uint16_t *vt, int64_t ldv, const ImgDesc *imgs, int n_img, int rows,
                               hipStream_t s)
{
    if (n_img <= 0 || rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(vt_tail_zero_kernel, dim3(n_img, (unsigned)ceil_div(rows, 256)), dim3(256), 0, s, vt,
                       ldv, imgs, rows);
    return hipGetLastError();
}

hipError_t launch_merge_project(const bf16_t *y, const ImgDesc *imgs, int n_img, int64_t Mtok,
                                int D, const bf16_t *Wp, const bf16_t *bias, int Dl, int act, bool out_f32,
                                void *out, const bf16_t *zero, const GemmWorkspace *ws, hipStream_t s)
{
    return dispatch(SrcMerge{y, imgs, n_img, Mtok, D, zero}, Wp, Mtok, Dl, 9 * D, bias, act, out_f32, out, ws,
                    s);
}
