// Residual add + LayerNorm or RMSNorm, one wave (64 lanes) per row of width D, two rows per
// wave.
//
//   x   = bf16(x + delta)          (when delta is given; written back to xout)
//   out = bf16((x - mean) * r * g + b),  r = 1 / sqrt(var + eps) rounded once per row,
//         mean and biased variance over the row
//   or, RMSNorm (the official tower: [Z] "Comparing the DeepSeek V4.1 Flash and Qwen3-VL
//   vision towers"; "Step 2" boundary table, RMSNorm semantics at the final norm):
//   out = bf16(x * r * g),  r = 1 / sqrt(mean(x^2) + eps)
//
// Pre-norm blocks and the final norm ([Z] "Step 2" boundary table); the encoder's residual
// adds run in the epilogues of the out-projection and fc2, so there it takes no delta (the
// delta form serves vit_op_layernorm / vit_op_rmsnorm).  The rows stay in registers: each
// lane holds D/64 elements of each row (16 at D = 1024, loaded as two 16-byte chunks so that
// a wave reads 1 KB contiguous per instruction); statistics are two-pass (mean, then squared
// deviations) with DPP reductions inside each 16-lane row and the four row sums read as
// scalars.  Scaling by the per-row reciprocal instead of dividing every element moves a
// normalised value by at most one fp32 ulp before the bf16 rounding.  HBM-bound: it reads
// x (+ delta) and writes out (+ x) once.
#include "kernels.h"

namespace {

// Sum over the wave, the same value in every lane: within each row of 16 lanes by DPP moves
// (lane ^ 1, lane ^ 2, then rotations by 4 and 8 add the other quads), then the four row
// sums read as scalars.  No LDS round trips.
__device__ __forceinline__ float wave_sum(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    const int iv = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
    return (r0 + r1) + (r2 + r3);
}

template <int EPL>
__device__ __forceinline__ void load_row(const bf16_t *p, int lane, float *v)
{
    if constexpr (EPL >= 8) {
#pragma unroll
        for (int q = 0; q < EPL / 8; ++q) {
            const uint4 u = *reinterpret_cast<const uint4 *>(p + q * 512 + lane * 8);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[q * 8 + j] = bf16_to_f32((bf16_t)((w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu));
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[e] = bf16_to_f32(p[lane * EPL + e]);
    }
}

template <int EPL>
__device__ __forceinline__ void store_row(bf16_t *p, int lane, const float *v)
{
    if constexpr (EPL >= 8) {
#pragma unroll
        for (int q = 0; q < EPL / 8; ++q) {
            uint4 u;
            u.x = pack_bf16x2(v[q * 8 + 0], v[q * 8 + 1]);
            u.y = pack_bf16x2(v[q * 8 + 2], v[q * 8 + 3]);
            u.z = pack_bf16x2(v[q * 8 + 4], v[q * 8 + 5]);
            u.w = pack_bf16x2(v[q * 8 + 6], v[q * 8 + 7]);
            *reinterpret_cast<uint4 *>(p + q * 512 + lane * 8) = u;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) p[lane * EPL + e] = f32_to_bf16(v[e]);
    }
}

// Each wave normalises RPW rows: it issues the loads of all its rows first, unpacks gamma and
// beta once for them, and scales each row by one reciprocal of its deviation (a single
// division per row instead of one per element).
template <int EPL, bool RMS, int RPW>
__global__ __launch_bounds__(256) void layernorm_kernel(const bf16_t *__restrict__ x,
                                                        const bf16_t *__restrict__ delta,
                                                        bf16_t *xout, int64_t M,
                                                        const bf16_t *__restrict__ g,
                                                        const bf16_t *__restrict__ b, float eps,
                                                        bf16_t *__restrict__ out)
{
    constexpr int D = EPL * 64;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
    const int lane = threadIdx.x & 63;
    if (row0 >= M) return;

    float v[RPW][EPL];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
        if (row0 + rr < M) load_row<EPL>(x + (row0 + rr) * D, lane, v[rr]);
    if (delta) {
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            if (row0 + rr >= M) continue;
            float d[EPL];
            load_row<EPL>(delta + (row0 + rr) * D, lane, d);
#pragma unroll
            for (int e = 0; e < EPL; ++e) v[rr][e] = bf16_to_f32(f32_to_bf16(__fadd_rn(v[rr][e], d[e])));
            store_row<EPL>(xout + (row0 + rr) * D, lane, v[rr]);
        }
    }
    // gamma and beta in the same lane layout as the rows (16-byte loads), once for all rows
    float gv[EPL], bv[EPL];
    load_row<EPL>(g, lane, gv);
    if constexpr (!RMS) load_row<EPL>(b, lane, bv);
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        if (row0 + rr >= M) continue;
        float mu = 0.f;
        if constexpr (!RMS) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) s += v[rr][e];
            mu = wave_sum(s) / (float)D;
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float dv = v[rr][e] - mu;
            ss = __builtin_fmaf(dv, dv, ss);
        }
        const float var = wave_sum(ss) / (float)D;
        const float inv = __fdiv_rn(1.f, sqrtf(var + eps));
        float y[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
#pragma clang fp contract(off)
            if constexpr (RMS) y[e] = __fmul_rn(__fmul_rn(v[rr][e], inv), gv[e]);
            else y[e] = __fadd_rn(__fmul_rn(__fmul_rn(v[rr][e] - mu, inv), gv[e]), bv[e]);
        }
        store_row<EPL>(out + (row0 + rr) * D, lane, y);
    }
}

template <int EPL>
hipError_t run_ln(const bf16_t *x, const bf16_t *delta, bf16_t *xout, int64_t M, const bf16_t *g,
                  const bf16_t *b, float eps, bool rms, bf16_t *out, hipStream_t s)
{
    constexpr int RPW = 2;
    const dim3 grid((unsigned)ceil_div(M, 4 * RPW));
    if (rms)
        hipLaunchKernelGGL((layernorm_kernel<EPL, true, RPW>), grid, dim3(256), 0, s, x, delta, xout, M, g, b,
                           eps, out);
    else
        hipLaunchKernelGGL((layernorm_kernel<EPL, false, RPW>), grid, dim3(256), 0, s, x, delta, xout, M, g, b,
                           eps, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layernorm(const bf16_t *x, const bf16_t *delta, bf16_t *xout, int64_t M, int D,
                            const bf16_t *g, const bf16_t *b, float eps, bool rms, bf16_t *out,
                            hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    switch (D) {
    case 64: return run_ln<1>(x, delta, xout, M, g, b, eps, rms, out, s);
    case 128: return run_ln<2>(x, delta, xout, M, g, b, eps, rms, out, s);
    case 256: return run_ln<4>(x, delta, xout, M, g, b, eps, rms, out, s);
    case 512: return run_ln<8>(x, delta, xout, M, g, b, eps, rms, out, s);
    case 1024: return run_ln<16>(x, delta, xout, M, g, b, eps, rms, out, s);
    case 1536: return run_ln<24>(x, delta, xout, M, g, b, eps, rms, out, s);
    case 2048: return run_ln<32>(x, delta, xout, M, g, b, eps, rms, out, s);
    default: return hipErrorInvalidValue;
    }
}
