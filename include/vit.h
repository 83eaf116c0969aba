/*
 * vit.h -- C ABI of the MI355X (gfx950) vision encoder for DeepSeek V4 / V4.1 Flash.
 *
 * The encoder turns images into visual rows for the language model in five stages:
 * 14x14 RGB patchify, patch projection, a stack of pre-norm ViT blocks with 2D RoPE
 * (LayerNorm + GELU MLP, or the official RMSNorm + SwiGLU layers, see vit_config), a 3x3
 * spatial merge, and the aligner projection(s) to the language hidden width.
 * Sources (web pages, cited by title and section):
 *   [Z] "DeepSeek V4.1 Flash Engineering, Part 3: Integrating Vision" (zhuai.tech)
 *   [G] ds4-learning "glossary/vision": V4 Flash Vision-Exp and V4.1 Flash vision rows
 *   [L] lucebox "docs/image-input.md": DS4V section
 *
 * Conventions
 *  - bf16 values travel as uint16_t bit patterns.
 *  - Pointers named d_* are device pointers (HIP, current device); h_* are host pointers.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call that
 *    takes a stream only enqueues work on it and returns without synchronising; results are
 *    valid once that stream has synchronised.  A context is not thread-safe: use one per
 *    stream.
 *  - All arguments of a call are validated before anything is enqueued, so a rejected call
 *    publishes no partial output ([L] DS4V: failed multi-image encoding publishes no partial
 *    embedding matrices).
 *  - The caller owns every buffer it passes; the library keeps no pointer after a call
 *    returns.  The context owns its device copy of the weights, tables and workspace.
 */
#ifndef VIT_H
#define VIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VIT_OK = 0,
    VIT_E_ARG = 1,      /* invalid argument (null pointer, bad size, bad grid, bad row index) */
    VIT_E_BUDGET = 2,   /* an image exceeds max_tokens_per_image merged tokens */
    VIT_E_NOMEM = 3,    /* device or pinned-host allocation failed, or over the reserve cap */
    VIT_E_DEVICE = 4    /* a HIP call or kernel launch failed; see vit_last_error */
} vit_status;

typedef struct vit_ctx vit_ctx;

/* Patch grid of one image: the image is (patch*gh) x (patch*gw) pixels. */
typedef struct { int32_t gh, gw; } vit_grid;

/* Encoder dimensions.  [Z] "Step 1": 14x14 patches, hidden 1024, 16 heads, 32 layers, 3x3
 * merge, 5120-wide projection (4096 for V4, [G]); token cap 1024 for V4.1, 384 for V4 ([G]).
 * Supported by this build: hidden in {64, 128, 256, 512, 1024, 1536, 2048}, head_dim =
 * hidden/heads in {16, 32, 64, 128}, mlp % 64 == 0, patch in [1, 64] (14 for the V4 / V4.1
 * towers), merge 3, out_hidden >= 1.
 *
 * Layer kinds.  All zero gives the pre-LayerNorm tower with a GELU (tanh form) MLP and one
 * aligner projection.  The official tower's layers ([Z] "Comparing the DeepSeek V4.1 Flash and
 * Qwen3-VL vision towers": RMSNorm and SwiGLU; "Step 2" boundary table: RMSNorm semantics at
 * the final norm, two linear projections in the aligner; "End-to-end results and their
 * limits": erf GELU in the official path) are selected by:
 *   norm_kind       0 LayerNorm (gamma, beta), 1 RMSNorm bf16(x / sqrt(mean(x^2) + eps) * g);
 *   mlp_kind        0 fc2(GELU(fc1 x)), 1 SwiGLU down(bf16(silu(gate x) * up x)), where the
 *                   gate and up projections, SiLU and the product form one step rounded once;
 *   gelu_kind       0 tanh form, 1 erf form, wherever a GELU appears (the GELU MLP and the
 *                   aligner between its projections);
 *   aligner_hidden  0 one projection 9D -> out_hidden (fp32 out); > 0 (a multiple of 64) two:
 *                   bf16(GELU(9D -> aligner_hidden)), then aligner_hidden -> out_hidden (fp32).
 * Readings where the pages name only the layer kind: RMSNorm uses ln_eps; SwiGLU and the
 * aligner keep biases (a zero bias gives the bias-free form). */
typedef struct {
    int32_t layers, hidden, heads, mlp, patch, merge, out_hidden, max_tokens_per_image;
    float ln_eps;        /* LayerNorm / RMSNorm epsilon (1e-6) */
    float rope_base;     /* 2D RoPE frequency base (10000) */
    float pix_mean[3];   /* per-channel pixel normalisation: v = (u8/255 - mean) / std, */
    float pix_std[3];    /* evaluated as fmaf(u8, 1/(255 std), -mean/std) in fp32 */
    int32_t norm_kind, mlp_kind, gelu_kind, aligner_hidden;   /* layer kinds, see above */
} vit_config;

/* Weights: one host bf16 blob, tensors back to back, every matrix [out][in] row-major:
 *   W_pe [D][3*patch^2], b_pe [D];
 *   per layer: ln1.g [D], ln1.b [D], W_qkv [3D][D] (rows: q | k | v, head-major inside
 *   each), b_qkv [3D], W_o [D][D], b_o [D], ln2.g [D], ln2.b [D], W_1 [F][D], b_1 [F],
 *   W_2 [D][F], b_2 [D];
 *   lnf.g [D], lnf.b [D], W_proj [out_hidden][9D] (input column c*9 + k: channel-major 3x3
 *   unfold, [Z] "Step 4"), b_proj [out_hidden].
 * With norm_kind = 1 every ".b" of a norm (ln1.b, ln2.b, lnf.b) is absent.  With mlp_kind = 1
 * the per-layer W_1, b_1, W_2, b_2 are replaced by W_gate [F][D], b_gate [F], W_up [F][D],
 * b_up [F], W_down [D][F], b_down [D].  With aligner_hidden = A > 0 the projector is W_proj
 * [A][9D], b_proj [A], W_proj2 [out_hidden][A], b_proj2 [out_hidden].
 * blob_elems must equal that total. */
typedef struct {
    vit_config cfg;
    const uint16_t *blob;
    size_t blob_elems;
} vit_weights;

/* Number of bf16 elements vit_create expects in the blob for `cfg` (0 if cfg is invalid). */
size_t vit_blob_elems(const vit_config *cfg);

/* Create a context on the current HIP device: validates cfg, copies the weights to the
 * device (the host blob may be freed afterwards) and prepares the derived tables.
 * Synchronous.  On failure *out is NULL and vit_last_error(NULL) describes why. */
vit_status vit_create(const vit_weights *w, vit_ctx **out);

/* Release everything the context owns.  Waits for the device first.  NULL is a no-op. */
void vit_destroy(vit_ctx *ctx);

/* Optional: pre-size the workspace for up to max_patches patches in one call (including the
 * aligner's inner rows when aligner_hidden > 0), and cap it there (a later vit_encode needing
 * more returns VIT_E_NOMEM).  max_patches <= 0 removes the cap.  Synchronous. */
vit_status vit_reserve(vit_ctx *ctx, int64_t max_patches);

/* Merged visual tokens of a batch: sum over images of ceil(gh/3) * ceil(gw/3)
 * ([Z] "Step 4": right/bottom padding to multiples of 3).  -1 if an argument is invalid. */
int64_t vit_num_tokens(const vit_ctx *ctx, const vit_grid *h_grids, int32_t n_images);

/* Patches of a batch: sum of gh * gw.  -1 if an argument is invalid. */
int64_t vit_num_patches(const vit_ctx *ctx, const vit_grid *h_grids, int32_t n_images);

/* Encode a packed batch of images into visual rows.
 *   d_pixels:  uint8 RGB, each image HWC [patch*gh][patch*gw][3], images back to back.
 *   h_grids:   n_images patch grids (host), 0 <= n_images <= 4096.  Each side in [1, 4096]
 *              (else VIT_E_ARG: the rotary tables cover 4096 positions per axis) and each
 *              image's merged token count <= max_tokens_per_image (else VIT_E_BUDGET).
 *   d_out_rows: fp32 [vit_num_tokens][out_hidden], image-major, merged tokens row-major
 *              inside each image ([G] V4.1: plain row-major stream).
 * Attention is bidirectional inside each image and never crosses images ([L] DS4V).
 * Operand precision inside attention: the tensors between steps are bf16 ([G] V4 Flash row:
 * intermediates rounded to BF16), but the attention contraction runs on IEEE binary16 MFMA
 * operands.  Rotated k and v are converted from bf16 to binary16 (round to nearest even:
 * exact for magnitudes 2^-14 .. 65504, subnormal below, saturating to +-65504 above);
 * q is scaled by log2(e)/sqrt(head_dim) and rounded once to binary16 (relative error
 * <= 2^-11, same saturation); the softmax weights enter the value product as binary16
 * (relative error < 2^-10).  With the encoder's LayerNorm inputs these values stay far
 * inside the range; k or v entries beyond 65504 in magnitude would be clamped.
 * Results are bitwise reproducible for the same batch.  The work split (K slices of the
 * GEMMs, key slices of the attention) is chosen from the size of the whole batch, so the
 * rows of one image encoded in different batches can differ in summation order, within the
 * same error bounds.
 * Returns without synchronising the stream. */
vit_status vit_encode(vit_ctx *ctx, const uint8_t *d_pixels, const vit_grid *h_grids,
                      int32_t n_images, float *d_out_rows, void *stream);

/* Token types of the image span layout (PAD only in the V4 Flash layout). */
enum { VIT_TOK_START = 1, VIT_TOK_IMAGE = 2, VIT_TOK_NEWLINE = 3, VIT_TOK_END = 4, VIT_TOK_PAD = 5 };

/* Span layouts: the V4.1 stream (vit_layout) and the V4 Flash stream (vit_layout_v4). */
enum { VIT_SPAN_V41 = 0, VIT_SPAN_V4 = 1 };

/* Span layout of a batch ([Z] "Connect the complete image-to-text path"; [G] V4.1: START,
 * then per merged row width x IMAGE and one NEWLINE, then END; identity order).  Writes
 * *n_positions = sum of 2 + mh*(mw+1); if h_types / h_src are non-NULL they must hold that
 * many entries: h_types[p] is a VIT_TOK_* value and h_src[p] the visual row (image-major
 * numbering, as in vit_encode's output) of an IMAGE position, -1 elsewhere.  Host only. */
vit_status vit_layout(const vit_grid *h_grids, int32_t n_images, int32_t merge,
                      int32_t *h_types, int32_t *h_src, int64_t *n_positions);

/* V4 Flash span layout, same conventions as vit_layout.  The pages name its parts without a
 * formula ([G] V4 Flash Vision-Exp column: synthetic sentinel tokens, row-pair interleave,
 * pos % 4 alignment; V4.1 Flash row: V4.1 drops the row-pair interleave and compress_pad;
 * [L] DS4V: the projector's tile permutation is applied once when rows are assembled with the
 * named sentinel embeddings).  Reading implemented here, not checked against the official
 * model: START; then for each pair of merged rows (2p, 2p+1) -- a last lone row when mh is
 * odd -- the pair's IMAGE positions column by column, (2p, c) then (2p+1, c), and one
 * NEWLINE; then END; then VIT_TOK_PAD positions up to a multiple of 4 (compress_pad), so a
 * span that starts at a multiple of 4 also ends on one.  h_src still numbers visual rows as
 * vit_encode emits them (row-major in each image): the interleave is a permutation of the
 * IMAGE positions.  Per image 4 * ceil((2 + ceil(mh/2) + mh*mw) / 4) positions.  Host only. */
vit_status vit_layout_v4(const vit_grid *h_grids, int32_t n_images, int32_t merge, int32_t *h_types,
                         int32_t *h_src, int64_t *n_positions);

/* Span layout vit_assemble writes: VIT_SPAN_V41 (default) or VIT_SPAN_V4 (vit_layout_v4's
 * positions; span starts must then be multiples of 4, else vit_assemble returns VIT_E_ARG, and
 * PAD positions are left as they are).  VIT_E_ARG for other values. */
vit_status vit_set_span_layout(vit_ctx *ctx, int32_t layout);

/* Overlay visual rows onto prompt embeddings ([Z] "Multimodal basics": vision vectors
 * replace the image-placeholder rows):  d_embeds[h_rows[t]][:] = bf16_rne(d_rows[t][:]) for
 * t < n_rows.  d_embeds is bf16 [n_embed_rows][hidden], d_rows fp32 [n_rows][hidden].
 * h_rows[t] < 0 skips row t (chunked prefill writes only the rows inside its chunk,
 * [Z] "Connect the complete image-to-text path").  VIT_E_ARG if ctx is NULL, hidden !=
 * out_hidden, a row index >= n_embed_rows, or two rows name the same destination. */
vit_status vit_overlay(vit_ctx *ctx, uint16_t *d_embeds, int64_t n_embed_rows,
                       const int32_t *h_rows, const float *d_rows, int64_t n_rows,
                       int32_t hidden, void *stream);

/* Preprocessing plan of one image ([Z] "Step 1": the largest grid that fits the aspect ratio
 * and the token budget, sides constrained to the patch x merge grid, contain resize, the result
 * centred on RGB 127 gray; images below the minimum pixel count are enlarged proportionally
 * first; [G] V4.1 row: 1024 tokens, minimum 295,936 pixels, no aspect clamp; V4 Flash row:
 * 384 tokens, minimum 147,456 pixels, aspect clamped to 8:1).  Readings where the pages are
 * silent: enlargement by sqrt(min_pixels / (height * width)) without rounding; the aspect clamp
 * lengthens the short side of the planning size; with a = H/(patch*merge), b = W/(patch*merge)
 * the grid is (round(a), round(b)) (ties to even, at least 1) when a*b fits the budget, else
 * floor(a r) x floor(b r) with r = sqrt(budget / (a b)) grown one row or column at a time while
 * the budget allows, each step keeping log(columns / rows) closest to log(b / a) (rows first
 * on a tie); contain: the limiting side fills the canvas, the other is
 * round(other * canvas side / limiting side), ties to even, at least 1; offsets are
 * floor((canvas - resized) / 2).  Host only.  VIT_E_ARG for sizes outside 1..65536 or negative
 * parameters (max_aspect 0 = no clamp). */
typedef struct {
    int32_t gh, gw;                /* patch grid of the canvas (multiples of merge) */
    int32_t canvas_h, canvas_w;    /* canvas pixels: patch * gh x patch * gw */
    int32_t resized_h, resized_w;  /* the contained image inside the canvas */
    int32_t off_y, off_x;          /* its top-left corner in the canvas */
} vit_image_plan;
vit_status vit_plan_image(int32_t height, int32_t width, int32_t patch, int32_t merge, int32_t max_tokens,
                          int64_t min_pixels, int32_t max_aspect, vit_image_plan *out);

/* The canvas of a plan ([Z] "Step 1" items 3-4): d_src = uint8 RGB HWC [height][width][3],
 * d_canvas = uint8 RGB HWC [canvas_h][canvas_w][3] (device, caller-owned), the image resized to
 * resized_h x resized_w at (off_y, off_x) and 127 elsewhere; ready for vit_encode with grid
 * (gh, gw).  Resize: the Keys cubic convolution (a = -0.5), separable, sample i of an axis at
 * source coordinate (i + 0.5) * in/out, the kernel stretched by in/out when shrinking, taps
 * outside the image dropped and the weights renormalised, horizontal pass first in fp32,
 * rounded half to even and clamped to 0..255 at the end.  A context scratch of
 * height * resized_w * 12 bytes is grown on demand.  VIT_E_ARG if a pointer is NULL or the
 * plan does not fit the canvas or the context's patch size; VIT_E_NOMEM if the scratch cannot
 * be allocated.  Asynchronous on `stream`. */
vit_status vit_preprocess(vit_ctx *ctx, const uint8_t *d_src, int32_t height, int32_t width,
                          const vit_image_plan *plan, uint8_t *d_canvas, void *stream);

/* Learned embedding rows of an image span's non-IMAGE positions ([Z] "Connect the complete
 * image-to-text path": the aligner output replaces the IMAGE positions and learned vectors
 * fill the boundary and newline positions).  h_sentinels: host bf16 [3][hidden], rows START,
 * NEWLINE, END, copied to the device before the call returns (replacing any earlier set).
 * VIT_E_ARG if ctx or h_sentinels is NULL or hidden != out_hidden; VIT_E_NOMEM if the
 * device copy cannot be allocated. */
vit_status vit_set_sentinels(vit_ctx *ctx, const uint16_t *h_sentinels, int32_t hidden);

/* Embedding assembly of one prefill chunk ([Z] "Connect the complete image-to-text path": an
 * image span may cross a chunk boundary, so each image keeps its token range and a chunk
 * replaces only the part of each span that lies inside it).
 *   Image i's span, in vit_layout's order (START, per merged row mw IMAGE and one NEWLINE,
 *   END: 2 + mh*(mw+1) positions), starts at prompt position h_span_start[i] (host).
 *   d_embeds: bf16 [chunk_hi - chunk_lo][hidden]; row j is prompt position chunk_lo + j.
 *   d_rows:   fp32 visual rows [vit_num_tokens(h_grids)][hidden] as vit_encode writes them.
 * Every span position p in [chunk_lo, chunk_hi) is written: an IMAGE position takes the next
 * visual row of its image (row-major merged order) rounded to bf16 (nearest even); START,
 * NEWLINE and END take the rows set by vit_set_sentinels.  All other rows are left as they
 * are; a chunk that meets no span launches nothing.  VIT_E_ARG if ctx is NULL, hidden !=
 * out_hidden, chunk_lo < 0 or chunk_hi < chunk_lo, a grid is invalid (VIT_E_BUDGET over the
 * token budget), a span start is negative, two spans overlap, no sentinels were set, or a
 * pointer needed for the chunk is NULL.  Asynchronous on `stream`. */
vit_status vit_assemble(vit_ctx *ctx, uint16_t *d_embeds, int64_t chunk_lo, int64_t chunk_hi,
                        int32_t hidden, const vit_grid *h_grids, int32_t n_images,
                        const int64_t *h_span_start, const float *d_rows, void *stream);

/* Debug boundaries ([Z] "Step 2": compare patches, block outputs, final norm and aligner
 * input to find the earliest divergence).  vit_dump runs the encoder up to the boundary on
 * the given batch and copies that tensor into d_dst (dst_bytes must equal its size):
 *   VIT_DUMP_PATCHES     bf16 [N][3*patch^2]   patchify output (same loader as the GEMM)
 *   VIT_DUMP_EMBED       bf16 [N][D]           patch projection output
 *   VIT_DUMP_QKV         bf16 [N][3D]          q,k after RoPE and v of layer `arg`; the k
 *                                              columns hold binary16 (as vit_op_rope)
 *   VIT_DUMP_ATTN        bf16 [N][D]           attention output of layer `arg`
 *   VIT_DUMP_LAYER       bf16 [N][D]           residual stream after layer `arg`
 *   VIT_DUMP_FINAL_NORM  bf16 [N][D]           final norm output (LayerNorm or RMSNorm)
 *   VIT_DUMP_MERGED      bf16 [M][9D]          merged projector input, channel-major
 *                                              (same gather as the projector GEMM)
 *   VIT_DUMP_ROPE        fp32 [N][hd]          2D RoPE cos/sin ([Z] "Step 2" table, the
 *                                              "2D RoPE cos/sin" boundary): row n holds
 *                                              cos theta_0 .. theta_{hd/2-1} of patch n, then
 *                                              sin of the same angles, read through the same
 *                                              device lookup as the QKV epilogue's rotation;
 *                                              theta = [h f_0 .. h f_{hd/4-1}, w f_0 ..], f_j =
 *                                              base^(-4j/hd) ([Z] "Step 3"); d_pixels is not
 *                                              read (may be NULL); d_dst 16-byte aligned
 * N = patches, M = merged tokens of the batch. */
enum {
    VIT_DUMP_PATCHES = 0, VIT_DUMP_EMBED = 1, VIT_DUMP_QKV = 2, VIT_DUMP_ATTN = 3,
    VIT_DUMP_LAYER = 4, VIT_DUMP_FINAL_NORM = 5, VIT_DUMP_MERGED = 6, VIT_DUMP_ROPE = 7
};
vit_status vit_dump(vit_ctx *ctx, int32_t boundary, int32_t arg, const uint8_t *d_pixels,
                    const vit_grid *h_grids, int32_t n_images, void *d_dst, size_t dst_bytes,
                    void *stream);

/* Per-step kernel timing, for profiling.  While enabled, vit_encode and vit_overlay record a
 * HIP event pair around every kernel launch on the caller's stream (no synchronisation);
 * vit_timing_read waits for the last recorded event, writes the summed milliseconds and the
 * launch count of each step kind into ms[VIT_STEP_COUNT] / launches[VIT_STEP_COUNT] (either
 * may be NULL) and starts a new accumulation.  Disabled by default.  VIT_STEP_LAYERNORM also
 * counts the RMSNorm of the official layers, VIT_STEP_FC1 their SwiGLU step (gate and up
 * projections in one launch), VIT_STEP_FC2 the down projection, and VIT_STEP_PROJECTOR the
 * whole aligner (both projections when there are two).  VIT_STEP_ATTENTION is the attention
 * kernel alone; VIT_STEP_ATTN_MERGE the merge of its key-sliced items, when a batch has any. */
enum {
    VIT_STEP_PATCH_EMBED = 0, VIT_STEP_LAYERNORM = 1, VIT_STEP_QKV = 2, VIT_STEP_ROPE = 3,
    VIT_STEP_ATTENTION = 4, VIT_STEP_OUT_PROJ = 5, VIT_STEP_FC1 = 6, VIT_STEP_FC2 = 7,
    VIT_STEP_PROJECTOR = 8, VIT_STEP_OVERLAY = 9, VIT_STEP_ATTN_MERGE = 10, VIT_STEP_COUNT = 11
};
vit_status vit_timing_enable(vit_ctx *ctx, int32_t enable);
vit_status vit_timing_read(vit_ctx *ctx, float *ms, int64_t *launches);

/* Text of the last error on ctx (or of the last failed vit_create on this thread when ctx
 * is NULL).  Never NULL; valid until the next call on the same ctx / thread. */
const char *vit_last_error(const vit_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* VIT_H */
