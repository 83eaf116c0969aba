// Host-side launchers of the gfx950 encoder kernels (one per hot-path step).
#pragma once

#include "common.h"

// Device scratch for the split-K tail of the GEMMs (fp32 partial tiles); NULL or too small
// disables the split.
struct GemmWorkspace {
    float *part;
    size_t bytes;
};

// Bytes of GemmWorkspace the largest split of any shape uses on this device (at most one
// fp32 256 x 128 partial tile per compute unit).
size_t gemm_workspace_max_bytes();

// Bytes of GemmWorkspace that launch_linear with these arguments uses (0: no K split), given
// a workspace of gemm_workspace_max_bytes().
size_t linear_workspace_bytes(int64_t M, int K, int N, int act, bool out_f32);

// Activation of the linear epilogue.  ACT_SWIGLU: W and b hold the gate and up rows
// interleaved in groups of 8 (N = 2F fused rows), out = bf16 [M][N/2] = bf16(silu(g) u).
enum { ACT_NONE = 0, ACT_GELU_TANH = 1, ACT_GELU_ERF = 2, ACT_SWIGLU = 3 };

// out = act(A W^T + b) on bf16 MFMA, fp32 accumulation; out bf16 (rounded once) or fp32
// (ACT_NONE only).  A bf16 [M][K], W bf16 [N][K]; K % 64 == 0.
hipError_t launch_linear(const bf16_t *A, int64_t M, int K, const bf16_t *W, const bf16_t *bias,
                         int N, int act, bool out_f32, void *out, const GemmWorkspace *ws,
                         hipStream_t s);

// Linear layer with the block's residual add: x = bf16(x + bf16(A W^T + b)), x bf16 [M][N]
// read and written in place (A must not overlap it); tiles, K split and workspace as
// launch_linear with ACT_NONE and bf16 output.
hipError_t launch_linear_residual(const bf16_t *A, int64_t M, int K, const bf16_t *W, const bf16_t *bias, int N,
                                  bf16_t *x, const GemmWorkspace *ws, hipStream_t s);

// Patchify fused into the patch projection: x0 = bf16(P W_pe^T + b) for patch rows
// [m_first, m_first + M) (out is the whole [N][D] output), the patch matrix P computed from
// the pixels inside the GEMM's A loader.  Those rows' images hold the pix_bytes (< 2^31) bytes
// at lpx, the first at offset pix_first of the batch's pixels (fewer than 12 bytes plus the
// misalignment of lpx: lpx must have 16 readable bytes); Wpe holds the projection weight in
// the loader's K order (SrcPatch in loaders.h), Kp = patch_gemm_k(ps).
hipError_t launch_patch_embed(const uint8_t *lpx, int64_t pix_first, int64_t pix_bytes, const ImgDesc *imgs,
                              int n_img, int64_t m_first, int64_t M, const float *s3, const float *t3, int ps,
                              const bf16_t *Wpe, int Kp, const bf16_t *bias, int D, bf16_t *out,
                              const GemmWorkspace *ws, hipStream_t s);

// 3x3 merge gather + projector: out [Mtok][Dl], fp32 or bf16 after `act`; Wp position-major
// [Dl][9D]; `zero` points at >= 16 zero bytes (read for positions in the right/bottom padding).
hipError_t launch_merge_project(const bf16_t *y, const ImgDesc *imgs, int n_img, int64_t Mtok,
                                int D, const bf16_t *Wp, const bf16_t *bias, int Dl, int act, bool out_f32,
                                void *out, const bf16_t *zero, const GemmWorkspace *ws, hipStream_t s);

// Optional residual add + LayerNorm, or RMSNorm with `rms` (b unused), rows of width D.
hipError_t launch_layernorm(const bf16_t *x, const bf16_t *delta, bf16_t *xout, int64_t M, int D,
                            const bf16_t *g, const bf16_t *b, float eps, bool rms, bf16_t *out,
                            hipStream_t s);

// 2D RoPE on q,k in place + transposed copy of v; one block per (64-row tile, head).
hipError_t launch_rope(bf16_t *qkv, bf16_t *vt, int64_t ldv, const RowTile *tiles, int n_tiles,
                       const ImgDesc *imgs, int D, int H, const float *cos_t,
                       const float *sin_t, hipStream_t s);

// QKV projection (N = 3D, K = D) with 2D RoPE on q and k and the transposed binary16 copy of
// v in the GEMM epilogue: qkv = [bf16 q | binary16 k | v (only with store_v)], vt as
// launch_rope writes it, except the columns past each image's end (launch_vt_tail_zero).
hipError_t launch_qkv_rope(const bf16_t *A, int64_t M, int D, int H, const bf16_t *W, const bf16_t *bias,
                           bf16_t *qkv, uint16_t *vt, int64_t ldv, const ImgDesc *imgs, int n_img,
                           const float *cos_t, const float *sin_t, bool store_v, hipStream_t s);
// Zeros in vt's columns past each image's last patch (up to its 64-aligned end); `rows` =
// heads x head_dim.
hipError_t launch_vt_tail_zero(uint16_t *vt, int64_t ldv, const ImgDesc *imgs, int n_img, int rows,
                               hipStream_t s);

// Block-diagonal flash attention over work items (query tile of attention_q_tile() rows,
// head), item L = head * n_work + tile.  The items are dealt to 8 groups of per_xcd
// consecutive items (one group per XCD of the GPU); in each group the first `full` items run
// whole, and each of the others is cut into `slices` key ranges run by separate blocks.  Each
// range writes its output normalised by its own softmax sum (binary16) to part_o and its
// (max, sum) to part_ml, in tail-item-major order, and a merge kernel writes o for those items.
// attention_plan() picks the split for a batch; attention_plan_bytes() sizes the scratch.
struct AttnSplit {
    int per_xcd, full, slices, items;
    uint16_t *part_o;
    float *part_ml;
};
// fixed: 0 = chosen from the batch (split only the items of a last, partial round of blocks),
// 1 = never split, 2..4 = every item cut into that many key ranges.
AttnSplit attention_plan(const ImgDesc *h_imgs, int n_img, int n_work, int D, int H, int fixed);
size_t attention_plan_bytes(const AttnSplit &sp, int D, int H);
// launch_attention runs the attention kernel; when the split has key-sliced items
// (attention_needs_merge), launch_attention_merge must follow it on the same stream to write
// their rows of o.
hipError_t launch_attention(const bf16_t *qkv, const bf16_t *vt, int64_t ldv, bf16_t *o,
                            const RowTile *work, int n_work, const ImgDesc *imgs, int D, int H,
                            const AttnSplit &sp, hipStream_t s);
bool attention_needs_merge(const AttnSplit &sp);
hipError_t launch_attention_merge(bf16_t *o, const RowTile *work, int n_work, const ImgDesc *imgs, int D, int H,
                                  const AttnSplit &sp, hipStream_t s);

// Compute units of the current device.
int cu_count();

// Contain resize (bicubic) of a uint8 HWC image h x w into the oh x ow region at (oy, ox) of a
// ch x cw canvas, 127 elsewhere; tmp is fp32 scratch of h * ow * 3 floats.
hipError_t launch_preprocess(const uint8_t *src, int h, int w, float *tmp, int oh, int ow, uint8_t *canvas,
                             int ch, int cw, int oy, int ox, hipStream_t s);

// Chunk assembly: for each entry (row r, source v) of `entries` (int32 pairs), embeds[r] =
// bf16(src[v]) when v >= 0, else the bf16 sentinel row -1 - v.
hipError_t launch_assemble(uint16_t *embeds, const float *src, const uint16_t *sentinels,
                           const int32_t *entries, int64_t n_entries, int hidden, hipStream_t s);

// embeds[rows[t]] = bf16(src[t]) for rows[t] >= 0.
hipError_t launch_overlay(uint16_t *embeds, const float *src, const int32_t *rows, int64_t n_rows,
                          int hidden, hipStream_t s);

// Debug materialisation of fused-only tensors through the GEMM loaders.
// Patch matrix rows [m_first, m_first + M) in the pages' (channel, y, x) column order, through
// the patch projection's own loader (arguments as launch_patch_embed; out is [N][3 ps^2]).
hipError_t launch_dump_patches(const uint8_t *lpx, int64_t pix_first, int64_t pix_bytes, const ImgDesc *imgs,
                               int n_img, int64_t m_first, int64_t M, const float *s3, const float *t3, int ps,
                               bf16_t *out, hipStream_t s);
hipError_t launch_dump_merged(const bf16_t *y, const ImgDesc *imgs, int n_img, int64_t Mtok,
                              int D, bf16_t *out, const bf16_t *zero, hipStream_t s);
// Rotary angles of every packed patch as the RoPE rotations read them: out fp32 [M][hd] =
// [cos theta_0 .. theta_{hd/2-1} | sin of the same].
hipError_t launch_dump_rope(const ImgDesc *imgs, int n_img, int64_t M, int hd, const float *cos_t,
                            const float *sin_t, float *out, hipStream_t s);

// Rows of an attention query tile (one block) and of a RoPE tile.
int attention_q_tile();
constexpr int kRopeTile = 64;
