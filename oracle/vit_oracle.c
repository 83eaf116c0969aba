/*
 * CPU oracle for the DeepSeek V4 / V4.1 Flash vision encoder forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no source with the HIP library.
 *
 * Plain, single-threaded, slow and obvious.  Every function below is the textbook
 * definition of one step, with the bf16 rounding points of the encoder made explicit.
 * Arithmetic is in `real` (float by default; the same file compiled with
 * -DORC_REAL=double gives the fp64 twin used to bound the fp32 oracle's own error).
 * Build: -O3 -ffp-contract=off, no fast-math: every sum runs in index order, one
 * multiply and one add per term, and fmaf is called only where the method says fma.
 *
 * Sources (web pages; cited by title and section):
 *  [Z]  "DeepSeek V4.1 Flash Engineering, Part 3: Integrating Vision" (zhuai.tech)
 *  [G]  ds4-learning "glossary/vision" (the V4 Flash and V4.1 Flash vision sections)
 * Readings taken where the pages are silent are listed next to the function they affect.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORC_REAL
#define ORC_REAL float
#endif
typedef ORC_REAL real;

#define ORC_IS_DOUBLE (sizeof(real) == sizeof(double))

/* ---------------------------------------------------------------------------------------
 * bf16 rounding.  [G] V4 Flash vision row: intermediates are rounded to BF16.
 * Round to nearest, ties to even, to 8 significant bits, directly from `real`.
 * ------------------------------------------------------------------------------------- */
static float bf16_from_float(float f)
{
    union { float f; uint32_t u; } v = { f };
    v.u += 0x7FFFu + ((v.u >> 16) & 1u);
    v.u &= 0xFFFF0000u;
    return v.f;
}

static double bf16_from_double(double d)
{
    if (d == 0.0 || !isfinite(d)) return d;
    int e;
    frexp(d, &e);                            /* d = m * 2^e, 0.5 <= |m| < 1 */
    int q = e - 8;                           /* quantum: 8 significant bits ... */
    if (q < -133) q = -133;                  /* ... but no finer than the smallest bf16 subnormal */
    return ldexp(nearbyint(ldexp(d, -q)), q);    /* ties to even (default rounding mode) */
}

static real R(real x)
{
    return ORC_IS_DOUBLE ? (real)bf16_from_double((double)x) : (real)bf16_from_float((float)x);
}

real orc_round_bf16(real x) { return R(x); }

void orc_round_bf16_array(real *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) x[i] = R(x[i]);
}

int orc_real_size(void) { return (int)sizeof(real); }

/* ---------------------------------------------------------------------------------------
 * Patchify + normalisation.  [Z] "Multimodal basics" (14x14 RGB patches, one row per patch,
 * grid coordinates kept); "Step 1" items 5-6 (flatten order (grid_y, grid_x, channel, y, x);
 * pixels mapped from [0,255] to the normalised range); "Step 5" (3*14*14 = 588 columns).
 *
 * img: uint8 HWC [ps*gh][ps*gw][3].  P: [gh*gw][3*ps*ps], row n = gy*gw + gx,
 * column c*ps*ps + y*ps + x.  Value = bf16(fmaf(u8, s_c, t_c)) with s_c = 1/(255 std_c),
 * t_c = -mean_c/std_c given in fp32 (reading: the per-channel affine map written as one fma).
 * ------------------------------------------------------------------------------------- */
void orc_patchify(const uint8_t *img, int gh, int gw, int ps, const float *s, const float *t,
                  real *P)
{
    const int64_t W = (int64_t)ps * gw;               /* image width in pixels */
    const int cols = 3 * ps * ps;
    for (int gy = 0; gy < gh; ++gy)
        for (int gx = 0; gx < gw; ++gx) {
            real *row = P + ((int64_t)gy * gw + gx) * cols;
            for (int c = 0; c < 3; ++c)
                for (int y = 0; y < ps; ++y)
                    for (int x = 0; x < ps; ++x) {
                        int64_t py = (int64_t)gy * ps + y, px = (int64_t)gx * ps + x;
                        float u = (float)img[(py * W + px) * 3 + c];
                        row[c * ps * ps + y * ps + x] = R((real)fmaf(u, s[c], t[c]));
                    }
        }
}

/* ---------------------------------------------------------------------------------------
 * Linear layer  out[i][j] = act(sum_k A[i][k] W[j][k] + b[j]),  optionally rounded to bf16.
 * [Z] "Multimodal basics" (patch projection), "Step 2" boundary table (QKV bias, the
 * aligner's linear projection).  W is passed transposed, Wt[k][j] = W[j][k], so that the
 * k-sum for every output runs in index order while the inner loop walks j contiguously.
 * act: 0 none, 1 GELU with the tanh approximation ([Z] "End-to-end results": tanh GELU),
 * 2 GELU in the exact erf form (the official path, same section).
 * Rows [r0, r1) of the output are computed.
 * ------------------------------------------------------------------------------------- */
static real gelu_tanh(real u)
{
    const real k0 = (real)0.7978845608028654;   /* sqrt(2/pi) */
    const real k1 = (real)0.044715;
    real inner = k0 * (u + k1 * u * u * u);
    return (real)0.5 * u * ((real)1 + (ORC_IS_DOUBLE ? (real)tanh((double)inner)
                                                     : (real)tanhf((float)inner)));
}

real orc_gelu_tanh(real u) { return gelu_tanh(u); }

/* GELU in its exact form u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), the form of the official
 * vision path ([Z] "End-to-end results": the official path uses erf, zLLM the tanh form). */
static real gelu_erf(real u)
{
    const real r2 = (real)1.4142135623730951;   /* sqrt(2) */
    return (real)0.5 * u * ((real)1 + (ORC_IS_DOUBLE ? (real)erf((double)(u / r2))
                                                     : (real)erff((float)(u / r2))));
}

real orc_gelu_erf(real u) { return gelu_erf(u); }

/* SiLU (swish) u * sigmoid(u) = u / (1 + e^-u), the gate activation of SwiGLU. */
static real silu(real u)
{
    return u / ((real)1 + (ORC_IS_DOUBLE ? (real)exp(-(double)u) : (real)expf(-(float)u)));
}

real orc_silu(real u) { return silu(u); }

/* SwiGLU gating of the official tower's MLP ([Z] "Comparing the DeepSeek V4.1 Flash and
 * Qwen3-VL vision towers": the official tower uses RMSNorm and SwiGLU): h = bf16(silu(g) * u) elementwise, where g and u
 * are the unrounded outputs (bias included) of the gate and up projections of the same
 * input.  Reading: like the GELU MLP's first linear, projection, activation and gating form
 * one step with one bf16 rounding at its end. */
void orc_swiglu(const real *g, const real *u, int64_t n, real *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = R(silu(g[i]) * u[i]);
}

void orc_transpose(const real *W, int64_t rows, int64_t cols, real *Wt)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            Wt[c * rows + r] = W[r * cols + c];
}

int orc_linear(const real *A, int64_t lda, int64_t r0, int64_t r1, int K, const real *Wt,
               const real *bias, int N, int act, int round_out, real *out, int64_t ldo)
{
    real *acc = (real *)malloc(sizeof(real) * (size_t)N);
    if (!acc) return -1;
    for (int64_t i = r0; i < r1; ++i) {
        const real *a = A + i * lda;
        for (int j = 0; j < N; ++j) acc[j] = 0;
        for (int k = 0; k < K; ++k) {
            const real ak = a[k];
            const real *w = Wt + (int64_t)k * N;
            for (int j = 0; j < N; ++j) acc[j] += ak * w[j];
        }
        real *o = out + i * ldo;
        for (int j = 0; j < N; ++j) {
            real v = acc[j] + (bias ? bias[j] : 0);
            if (act == 1) v = gelu_tanh(v);
            else if (act == 2) v = gelu_erf(v);
            o[j] = round_out ? R(v) : v;
        }
    }
    free(acc);
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * LayerNorm, rows [r0, r1):  mu = sum x / D,  var = sum (x - mu)^2 / D  (biased),
 * y = bf16((x - mu) / sqrt(var + eps) * g + b).  Pre-norm blocks and the final norm:
 * [Z] "Step 2" boundary table (final norm output after the 32 blocks).  The pages name
 * RMSNorm for the official tower; the workload specification fixes pre-LayerNorm with
 * eps 1e-6, which is the reading taken here.
 * ------------------------------------------------------------------------------------- */
void orc_layernorm(const real *x, int64_t ld, int64_t r0, int64_t r1, int D, const real *g,
                   const real *b, real eps, real *out, int64_t ldo)
{
    for (int64_t i = r0; i < r1; ++i) {
        const real *xr = x + i * ld;
        real sum = 0;
        for (int k = 0; k < D; ++k) sum += xr[k];
        real mu = sum / (real)D;
        real ss = 0;
        for (int k = 0; k < D; ++k) { real d = xr[k] - mu; ss += d * d; }
        real var = ss / (real)D;
        real den = ORC_IS_DOUBLE ? (real)sqrt((double)(var + eps)) : (real)sqrtf((float)(var + eps));
        real *o = out + i * ldo;
        for (int k = 0; k < D; ++k) o[k] = R((xr[k] - mu) / den * g[k] + b[k]);
    }
}

/* ---------------------------------------------------------------------------------------
 * RMSNorm, rows [r0, r1):  ms = sum x^2 / D,  y = bf16(x / sqrt(ms + eps) * g).  The block
 * norms and the final norm of the official tower ([Z] "Comparing the DeepSeek V4.1 Flash
 * and Qwen3-VL vision towers": RMSNorm and SwiGLU; "Step 2" boundary table: RMSNorm semantics at the final-norm
 * boundary).  No mean is subtracted and there is no additive term.  Reading: the same eps
 * as the LayerNorm form (1e-6), added to the mean square inside the square root.
 * ------------------------------------------------------------------------------------- */
void orc_rmsnorm(const real *x, int64_t ld, int64_t r0, int64_t r1, int D, const real *g,
                 real eps, real *out, int64_t ldo)
{
    for (int64_t i = r0; i < r1; ++i) {
        const real *xr = x + i * ld;
        real ss = 0;
        for (int k = 0; k < D; ++k) ss += xr[k] * xr[k];
        real ms = ss / (real)D;
        real den = ORC_IS_DOUBLE ? (real)sqrt((double)(ms + eps)) : (real)sqrtf((float)(ms + eps));
        real *o = out + i * ldo;
        for (int k = 0; k < D; ++k) o[k] = R(xr[k] / den * g[k]);
    }
}

/* Residual: out = bf16(a + b), one rounding of the fp sum. */
void orc_add_round(const real *a, const real *b, int64_t n, real *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = R(a[i] + b[i]);
}

/* ---------------------------------------------------------------------------------------
 * 2D rotary position embedding.  [Z] "Step 3": the angle vector is blocked by axis,
 * [h f_0 .. h f_n, w f_0 .. w f_n] (not interleaved), with the half-vector rotation
 * convention.  [G] V4 Flash row: positions are the raw (unmerged) patch grid.
 * Reading: for head dim hd, half = hd/2 angles, the first hd/4 use the row index h and the
 * next hd/4 the column index w, f_j = base^(-2j/half); pairs (i, i + half) rotate by theta_i.
 *
 * orc_rope_angle gives (cos, sin) of theta_i at patch (h, w): computed in double, rounded.
 * ------------------------------------------------------------------------------------- */
void orc_rope_angle(int h, int w, int i, int hd, double base, real *c, real *s)
{
    int half = hd / 2, quarter = hd / 4;
    int j = i < quarter ? i : i - quarter;
    double pos = i < quarter ? (double)h : (double)w;
    double f = pow(base, -2.0 * (double)j / (double)half);
    double ang = pos * f;
    *c = (real)cos(ang);
    *s = (real)sin(ang);
}

/* In place on q and k inside packed qkv rows [q(D) | k(D) | v(D)] (head-major inside each),
 * rows [r0, r1) of one image whose patch n sits at (n / gw, n % gw). */
void orc_rope_qk(real *qkv, int64_t ld, int64_t r0, int64_t r1, int gw, int D, int H,
                 double base)
{
    const int hd = D / H, half = hd / 2;
    for (int64_t n = r0; n < r1; ++n) {
        int h = (int)(n / gw), w = (int)(n % gw);
        for (int part = 0; part < 2; ++part)              /* q, then k */
            for (int head = 0; head < H; ++head) {
                real *v = qkv + n * ld + (int64_t)part * D + (int64_t)head * hd;
                for (int i = 0; i < half; ++i) {
                    real c, s;
                    orc_rope_angle(h, w, i, hd, base, &c, &s);
                    real a = v[i], b = v[i + half];
                    real na = a * c - b * s;
                    real nb = b * c + a * s;
                    v[i] = R(na);
                    v[i + half] = R(nb);
                }
            }
    }
}

/* ---------------------------------------------------------------------------------------
 * Bidirectional (non-causal) multi-head attention within one image.  [Z] "Multimodal basics"
 * (ViT attention gives each patch whole-image context).  Scale 1/sqrt(hd) (reading: the
 * usual dot-product scale).  Per head and query i: s_j = (q_i . k_j) * scale, p = softmax(s)
 * with the row max subtracted, o_i = sum_j p_j v_j, then bf16.
 * qkv rows [q | k | v] of the n patches of this image; queries [q0, q1); o: [n][D].
 * ------------------------------------------------------------------------------------- */
int orc_attention(const real *qkv, int64_t ld, int64_t n, int D, int H, int64_t q0, int64_t q1,
                  real *o, int64_t ldo)
{
    const int hd = D / H;
    const real scale = (real)(1.0 / sqrt((double)hd));
    real *kt = (real *)malloc(sizeof(real) * (size_t)(hd * n));   /* kt[d][j] */
    real *s = (real *)malloc(sizeof(real) * (size_t)n);
    real *acc = (real *)malloc(sizeof(real) * (size_t)hd);
    if (!kt || !s || !acc) { free(kt); free(s); free(acc); return -1; }
    for (int head = 0; head < H; ++head) {
        const int64_t qo = (int64_t)head * hd, ko = D + qo, vo = 2 * (int64_t)D + qo;
        for (int64_t j = 0; j < n; ++j)
            for (int d = 0; d < hd; ++d) kt[(int64_t)d * n + j] = qkv[j * ld + ko + d];
        for (int64_t i = q0; i < q1; ++i) {
            const real *q = qkv + i * ld + qo;
            for (int64_t j = 0; j < n; ++j) s[j] = 0;
            for (int d = 0; d < hd; ++d) {                 /* s_j = sum_d q_d k_jd, d in order */
                const real qd = q[d];
                const real *kd = kt + (int64_t)d * n;
                for (int64_t j = 0; j < n; ++j) s[j] += qd * kd[j];
            }
            real m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) { s[j] *= scale; if (s[j] > m) m = s[j]; }
            real sum = 0;
            for (int64_t j = 0; j < n; ++j) {
                s[j] = ORC_IS_DOUBLE ? (real)exp((double)(s[j] - m)) : (real)expf((float)(s[j] - m));
                sum += s[j];
            }
            for (int64_t j = 0; j < n; ++j) s[j] = s[j] / sum;  /* p */
            for (int d = 0; d < hd; ++d) acc[d] = 0;
            for (int64_t j = 0; j < n; ++j) {
                const real pj = s[j];
                const real *v = qkv + j * ld + vo;
                for (int d = 0; d < hd; ++d) acc[d] += pj * v[d];
            }
            real *out = o + i * ldo + qo;
            for (int d = 0; d < hd; ++d) out[d] = R(acc[d]);
        }
    }
    free(kt); free(s); free(acc);
    return 0;
}

/* Softmax row of the scaled scores of one query (pins: rows sum to 1). */
void orc_softmax_row(const real *qkv, int64_t ld, int64_t n, int D, int H, int head, int64_t i,
                     real *p)
{
    const int hd = D / H;
    const real scale = (real)(1.0 / sqrt((double)hd));
    const real *q = qkv + i * ld + (int64_t)head * hd;
    real m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        const real *k = qkv + j * ld + D + (int64_t)head * hd;
        real acc = 0;
        for (int d = 0; d < hd; ++d) acc += q[d] * k[d];
        p[j] = acc * scale;
        if (p[j] > m) m = p[j];
    }
    real sum = 0;
    for (int64_t j = 0; j < n; ++j) {
        p[j] = ORC_IS_DOUBLE ? (real)exp((double)(p[j] - m)) : (real)expf((float)(p[j] - m));
        sum += p[j];
    }
    for (int64_t j = 0; j < n; ++j) p[j] = p[j] / sum;
}

/* ---------------------------------------------------------------------------------------
 * 3x3 spatial merge.  [Z] "Step 4": pad right and bottom with zeros to multiples of 3 on the
 * 2D grid (not on the flattened rows), map each (source_y, source_x) to its window and the
 * offset inside it, and unfold channel-major: [9 positions of channel 0, 9 of channel 1, ...].
 * Reading: inside a window the 9 positions are row-major, k = dy*3 + dx; windows row-major.
 * y: [gh*gw][D] (row = gy*gw + gx).  A: [mh*mw][9D], A[t][c*9 + k].
 * ------------------------------------------------------------------------------------- */
void orc_merge(const real *y, int gh, int gw, int D, int m, real *A)
{
    const int mh = (gh + m - 1) / m, mw = (gw + m - 1) / m, mm = m * m;
    memset(A, 0, sizeof(real) * (size_t)mh * mw * mm * D);
    for (int sy = 0; sy < gh; ++sy)
        for (int sx = 0; sx < gw; ++sx) {
            int t = (sy / m) * mw + (sx / m);
            int k = (sy % m) * m + (sx % m);
            const real *src = y + ((int64_t)sy * gw + sx) * D;
            real *dst = A + (int64_t)t * mm * D;
            for (int c = 0; c < D; ++c) dst[(int64_t)c * mm + k] = src[c];
        }
}
