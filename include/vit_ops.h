/*
 * vit_ops.h -- single-step entry points of the MI355X vision encoder.
 *
 * Each call launches exactly the kernel(s) that vit_encode uses for that step, with the same
 * launch configuration, on caller-provided device buffers (vit_op_rope is the exception: a
 * standalone form of the rotation that vit_encode runs inside vit_op_qkv_rope's kernel).  They exist so that every step can
 * be checked and timed in isolation at the encoder's real shapes.  Conventions are those of
 * vit.h (bf16 as uint16_t, d_* device pointers, asynchronous on `stream`, validation before
 * any launch, VIT_E_* codes, text in vit_last_error(ctx)).  `ctx` must be non-NULL; only
 * vit_op_rope, vit_op_attention and vit_op_merge_project read its configuration and tables.
 */
#ifndef VIT_OPS_H
#define VIT_OPS_H

#include "vit.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { VIT_ACT_NONE = 0, VIT_ACT_GELU_TANH = 1, VIT_ACT_GELU_ERF = 2, VIT_ACT_SWIGLU = 3 };

/* Linear layer on bf16 MFMA with fp32 accumulation ([Z] "Multimodal basics": patch
 * projection and the block's linear layers; "End-to-end results and their limits": tanh GELU
 * in zLLM, erf GELU in the official path):
 *   out[i][j] = act(sum_k A[i][k] W[j][k] + b[j])
 * A bf16 [M][K] (row stride K), W bf16 [N][K], b bf16 [N] or NULL.  out is bf16 [M][N]
 * rounded once after the activation (out_f32 == 0) or fp32 [M][N] (out_f32 != 0, act must be
 * VIT_ACT_NONE).
 * VIT_ACT_SWIGLU is the first step of the official tower's MLP ([Z] "Comparing the DeepSeek
 * V4.1 Flash and Qwen3-VL vision towers"): W and b hold N = 2F rows, the gate and up
 * projections interleaved in groups of 8 (rows 16j .. 16j+7 = gate rows 8j .. 8j+7, rows
 * 16j+8 .. 16j+15 = up rows 8j .. 8j+7), and out is bf16 [M][N/2] with
 * out[i][f] = bf16(silu(g) * u), g and u the biased fp32 gate and up results of feature f.
 * vit_create builds this interleaved weight from the blob's W_gate and W_up.  N % 16 == 0.
 * Requires M >= 0, N >= 1, K >= 64 and K % 64 == 0. */
vit_status vit_op_linear(vit_ctx *ctx, const uint16_t *d_A, int64_t M, int32_t K,
                         const uint16_t *d_W, const uint16_t *d_b, int32_t N, int32_t act,
                         int32_t out_f32, void *d_out, void *stream);

/* vit_op_linear for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments, kernels and
 * results (bitwise) as vit_op_linear, but the fp32 split-K partial tiles live in a fixed
 * device scratch of 32 MiB that the library holds on every GPU it runs on until the process
 * ends, instead of the context's workspace; the call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).  All calls on one GPU share that scratch: calls
 * that overlap in time on one GPU (different streams or threads) race and must be
 * serialised by the caller.  Nothing in the scratch needs to start at zero (each launch
 * writes every partial it reads).  VIT_E_ARG as vit_op_linear, and also when the K split
 * chosen for these sizes would need more than the 32 MiB (not on a 256-CU MI355X, where one
 * split round holds at most one 256 x 128 fp32 tile per compute unit). */
vit_status vit_op_linear_noalloc(vit_ctx *ctx, const uint16_t *d_A, int64_t M, int32_t K,
                                 const uint16_t *d_W, const uint16_t *d_b, int32_t N, int32_t act,
                                 int32_t out_f32, void *d_out, void *stream);

/* Linear layer with the block's residual add, as vit_encode runs the out-projection and fc2
 * ([Z] "Step 2" boundary table: the block output fixes the residual order; [Z] "Multimodal
 * basics": pre-norm transformer blocks):
 *   x[i][j] = bf16(x[i][j] + bf16(sum_k A[i][k] W[j][k] + b[j]))
 * i.e. vit_op_linear (VIT_ACT_NONE, bf16 output) followed by the residual add of
 * vit_op_layernorm, bitwise, in one pass: the sum is formed as the product tile is written.
 * A bf16 [M][K], W bf16 [N][K], b bf16 [N] or NULL, x bf16 [M][N] read and updated in place.
 * VIT_E_ARG when A and x overlap, or as vit_op_linear for the sizes. */
vit_status vit_op_linear_residual(vit_ctx *ctx, const uint16_t *d_A, int64_t M, int32_t K,
                                  const uint16_t *d_W, const uint16_t *d_b, int32_t N, uint16_t *d_x,
                                  void *stream);

/* Residual add + LayerNorm over rows of width D (D in {64, 128, 256, 512, 1024, 1536, 2048}):
 *   if d_delta != NULL:  x = bf16(x + delta), written to d_xout (may alias d_x);
 *   out = bf16((x - mean) * r * g + b), mean/var over the row (biased), r = 1/sqrt(var + eps)
 *   rounded once per row (within one fp32 ulp of dividing by the root; compared with the
 *   division form within one bf16 ulp).
 * x, delta, xout, out are bf16 [M][D]; g, b bf16 [D]. */
vit_status vit_op_layernorm(vit_ctx *ctx, const uint16_t *d_x, const uint16_t *d_delta,
                            uint16_t *d_xout, int64_t M, int32_t D, const uint16_t *d_g,
                            const uint16_t *d_b, float eps, uint16_t *d_out, void *stream);

/* Residual add + RMSNorm, the official tower's norm ([Z] "Comparing the DeepSeek V4.1 Flash
 * and Qwen3-VL vision towers"; "Step 2" boundary table: RMSNorm semantics at the final norm),
 * same kernel and conventions as vit_op_layernorm with:
 *   out = bf16(x * r * g), r = 1/sqrt(mean(x^2) + eps) rounded once per row   (no mean
 *   subtracted, no beta). */
vit_status vit_op_rmsnorm(vit_ctx *ctx, const uint16_t *d_x, const uint16_t *d_delta,
                          uint16_t *d_xout, int64_t M, int32_t D, const uint16_t *d_g,
                          float eps, uint16_t *d_out, void *stream);

/* Row stride (in elements) of the transposed-V buffer for a batch: the buffer is
 * binary16 [heads][head_dim][stride] and image i owns columns starting at a multiple of 64,
 * stride = sum over images of ceil(gh*gw / 64) * 64.  -1 if an argument is invalid. */
int64_t vit_vt_stride(const vit_grid *h_grids, int32_t n_images);

/* QKV projection of one layer with the 2D rotary embedding and the transposed-V copy in its
 * epilogue, as vit_encode runs it ([Z] "Step 2" table: QKV with bias; "Step 3": RoPE on q
 * and k; [G] V4: raw patch grid):
 *   qkv = bf16(x W^T + b), x = bf16 [N][D] (N patches of the batch), W = bf16 [3D][D],
 *   b = bf16 [3D] or NULL; then q and k rotated and stored in d_qkv = [N][3D] exactly as
 *   vit_op_rope stores them (q bf16, k binary16 bit patterns), and v written to d_vt in
 *   vit_op_rope's transposed layout (including the zero columns past each image's end).
 *   The v columns of d_qkv are written (bf16) only when store_v != 0; vit_encode skips them.
 * The rotation acts on the bf16-rounded projection, so for the same qkv values the results
 * are bitwise those of vit_op_linear followed by vit_op_rope. */
vit_status vit_op_qkv_rope(vit_ctx *ctx, const uint16_t *d_x, const uint16_t *d_W, const uint16_t *d_b,
                           const vit_grid *h_grids, int32_t n_images, uint16_t *d_qkv, uint16_t *d_vt,
                           int32_t store_v, void *stream);

/* 2D RoPE on q and k as a separate pass over a qkv buffer (vit_encode fuses this step into the
 * QKV projection, vit_op_qkv_rope; this entry point prepares attention inputs from any qkv)
 * ([Z] "Step 3": height/width-blocked angles, half-vector rotation;
 * [G] V4: raw patch grid) in place inside d_qkv = bf16 [N][3D] (q | k | v, head-major).
 * Rotated q is stored as bf16; rotated k is rounded to bf16 and then stored as IEEE binary16
 * bit patterns (the attention's score operand type), so after this call columns D..2D-1 of
 * d_qkv hold binary16.  v is copied transposed to d_vt = IEEE binary16 [H][hd][vit_vt_stride(grids)] (the operand
 * type of the attention's P.V product) for the attention: image i owns the columns from its
 * 64-aligned offset; inside every group of 16 columns, column p holds key (p with bits 2 and
 * 3 swapped); columns past the image's last patch are written as zeros.  Both conversions
 * from bf16 round to nearest even, which is exact for magnitudes 2^-14 .. 65504; larger
 * values saturate to +-65504.
 * Patch n of an image sits at (n / gw, n % gw) of that image's grid. */
vit_status vit_op_rope(vit_ctx *ctx, uint16_t *d_qkv, uint16_t *d_vt, const vit_grid *h_grids,
                       int32_t n_images, void *stream);

/* Bidirectional softmax attention inside each image of a packed batch (block-diagonal),
 * scale 1/sqrt(head_dim): d_o = bf16 [N][D], head h in columns h*hd .. h*hd+hd-1.
 * Inputs as produced by vit_op_rope (bf16 q, binary16 k in d_qkv; binary16 V^T).  Scores are
 * formed from q * log2(e)/sqrt(head_dim) rounded to binary16; softmax weights enter the
 * value product as binary16. */
vit_status vit_op_attention(vit_ctx *ctx, const uint16_t *d_qkv, const uint16_t *d_vt,
                            const vit_grid *h_grids, int32_t n_images, uint16_t *d_o,
                            void *stream);

/* Key slices of the attention (vit_encode and vit_op_attention).  With n slices the keys of
 * a (query tile, head) are cut into n contiguous ranges processed by separate blocks; each
 * range's output, normalised by its own softmax sum, is kept as binary16 with its (max, sum),
 * and a merge weights the ranges by sum * 2^(max - overall max) and rounds once to bf16.  The
 * results agree with the unsliced attention within the same error bounds (not bitwise).
 * n = 0 (the default) cuts only the (query tile, head) items that would form a last, partial
 * round of blocks on the GPU, into up to 4 slices each, so that round occupies every block
 * slot for a fraction of its length; the other items run whole.  n = 1 never cuts; n = 2..4
 * cuts every item into n slices.  VIT_E_ARG for other values. */
vit_status vit_set_attention_split(vit_ctx *ctx, int32_t n);

/* 3x3 merge + aligner ([Z] "Step 4": right/bottom zero padding on the 2D grid,
 * channel-major unfold; then the aligner projection, or with aligner_hidden > 0 the two
 * projections with the configured GELU between them, the inner result rounded to bf16 in a
 * context buffer grown on demand): d_y = bf16 [N][D] final-norm rows, d_out = fp32
 * [M][out_hidden] using the context's aligner weights. */
vit_status vit_op_merge_project(vit_ctx *ctx, const uint16_t *d_y, const vit_grid *h_grids,
                                int32_t n_images, float *d_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VIT_OPS_H */
