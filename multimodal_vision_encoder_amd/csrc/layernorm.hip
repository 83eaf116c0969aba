// Residual add + LayerNorm or RMSNorm, one wave (64 lanes) per row of width D.
//
//   x   = bf16(x + delta)          (when delta is given; written back to xout)
//   out = bf16((x - mean) / sqrt(var + eps) * g + b),  mean and biased variance over the row
//   or, RMSNorm (the official tower: [Z] "Comparing the DeepSeek V4.1 Flash and Qwen3-VL
//   vision towers"; "Step 2" boundary table, RMSNorm semantics at the final norm):
//   out = bf16(x / sqrt(mean(x^2) + eps) * g)
//
// Pre-norm blocks and the final norm ([Z] "Step 2" boundary table); the encoder's residual
// adds run in the epilogues of the out-projection and fc2, so there it takes no delta (the
// delta form serves vit_op_layernorm / vit_op_rmsnorm).  The row stays in
// registers: each lane holds D/64 elements (16 at D = 1024, loaded as two 16-byte chunks
// so that a wave reads 1 KB contiguous per instruction); statistics are two-pass (mean,
// then squared deviations) with butterfly reductions across the wave.  HBM-bound: it reads
// x (+ delta) and writes out (+ x) once.
#include "kernels.h"

namespace {

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
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

template <int EPL, bool RMS>
__global__ __launch_bounds__(256) void layernorm_kernel(const bf16_t *__restrict__ x,
                                                        const bf16_t *__restrict__ delta,
                                                        bf16_t *xout, int64_t M,
                                                        const bf16_t *__restrict__ g,
                                                        const bf16_t *__restrict__ b, float eps,
                                                        bf16_t *__restrict__ out)
{
    constexpr int D = EPL * 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;

    float v[EPL];
    load_row<EPL>(x + row * D, lane, v);
    if (delta) {
        float d[EPL];
        load_row<EPL>(delta + row * D, lane, d);
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[e] = bf16_to_f32(f32_to_bf16(__fadd_rn(v[e], d[e])));
        store_row<EPL>(xout + row * D, lane, v);
    }
    float mu = 0.f;
    if constexpr (!RMS) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s += v[e];
        mu = wave_sum(s) / (float)D;
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const float dv = v[e] - mu;
        ss = __builtin_fmaf(dv, dv, ss);
    }
    const float var = wave_sum(ss) / (float)D;
    const float den = sqrtf(var + eps);
    // gamma and beta in the same lane layout as the row (16-byte loads)
    float gv[EPL], y[EPL];
    load_row<EPL>(g, lane, gv);
    if constexpr (RMS) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) y[e] = __fmul_rn(__fdiv_rn(v[e], den), gv[e]);
    } else {
        float bv[EPL];
        load_row<EPL>(b, lane, bv);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
#pragma clang fp contract(off)
            y[e] = __fadd_rn(__fmul_rn(__fdiv_rn(v[e] - mu, den), gv[e]), bv[e]);
        }
    }
    store_row<EPL>(out + row * D, lane, y);
}

template <int EPL>
hipError_t run_ln(const bf16_t *x, const bf16_t *delta, bf16_t *xout, int64_t M, const bf16_t *g,
                  const bf16_t *b, float eps, bool rms, bf16_t *out, hipStream_t s)
{
    if (rms)
        hipLaunchKernelGGL((layernorm_kernel<EPL, true>), dim3((unsigned)ceil_div(M, 4)), dim3(256), 0, s, x,
                           delta, xout, M, g, b, eps, out);
    else
        hipLaunchKernelGGL((layernorm_kernel<EPL, false>), dim3((unsigned)ceil_div(M, 4)), dim3(256), 0, s, x,
                           delta, xout, M, g, b, eps, out);
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
