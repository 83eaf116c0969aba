// A-operand sources of the bf16 GEMMs.  The same functions feed the debug dumps, so a dumped
// tensor is exactly what the GEMM consumed.
#pragma once

#include "common.h"

// Patchify fused into the patch projection's A operand ([Z] "Step 1": rows are patches in
// (grid_y, grid_x) order, pixels normalised as fmaf(u8, s_c, t_c) and rounded to bf16; [Z]
// "Step 5": the padded K columns hold zeros).  Pixels are uint8 HWC per image, images packed
// back to back.
//
// K order of the GEMM.  The pages order a patch's 3*ps*ps values as (channel, y, x); the GEMM
// instead walks them as the image stores them: row segment y of the patch (its 3*ps bytes
// x0 c0 x0 c1 x0 c2 x1 c0 ...), each segment padded with zeros to RP = ceil(3 ps / 8) * 8
// columns, K = ps * RP rounded up to a multiple of 32.  vit_create permutes the projection
// weight into this order (its other columns zero), so the product is the same sum.  Every
// 8-column chunk of a row is then 8 consecutive pixel bytes, fetched as one aligned 12-byte
// load and converted in registers: chunk (y, b0) covers bytes b0 .. b0+7 of segment y, byte
// b of a segment is pixel x = b / 3, channel c = b % 3.
struct RawChunk {
    uint32_t d0, d1, d2;   // 12 bytes from a 4-byte-aligned offset at or below the chunk
    uint32_t sh;           // the chunk's first byte inside them (0 .. 11)
};

// Pixel bytes of a launch are addressed as 32-bit offsets from one 4-byte-aligned base (the
// loads take the base in scalar registers and the offset per lane), so one launch covers less
// than 2^31 bytes of pixels; larger batches are projected in groups of whole images.  The 12
// bytes read for a chunk start at most at last12, so that they end with the last dword that
// holds a pixel byte (launches of fewer than 12 pixel bytes read a 16-byte padded copy).
struct SrcPatch {
    static constexpr bool REG = true;   // A converted on the way into LDS
    const uint8_t *px;   // 4-byte-aligned base of this launch's pixel bytes
    int64_t pix_sub;     // an image's offset from px is its pix_off - pix_sub
    uint32_t last12;     // largest offset of a chunk's 12-byte read
    const ImgDesc *imgs;
    int n_img;
    int64_t m_base;      // first patch row of this launch
    int64_t M;           // rows of this launch
    int ps, sb, rp;      // patch side, segment bytes 3 ps, padded segment columns
    float inv_rp;        // 1 / rp
    float s0, s1, s2;    // 1 / (255 std_c)
    float t0, t1, t2;    // -mean_c / std_c

    struct Row {
        uint32_t off;    // offset of the patch's top-left pixel byte
        int rs;          // bytes per image row
    };
    // The chunk at column k of every row: segment y (clamped into the patch for the K
    // padding), first byte b0, valid columns nv (0 past the patch), and the scale and offset
    // of byte e (channel (b0 + e) % 3): (s_a, t_a) for e % 3 == 0, then (s_b, t_b), (s_c, t_c).
    struct KChunk {
        int yc, b0, nv;
        float sa, sb, sc, ta, tb, tc;
    };
    // The six channel constants as opaque wave-uniform values, read once per thread: chunk()
    // selects among values, never among their kernel-argument addresses.
    struct Consts {
        float s0, s1, s2, t0, t1, t2;
    };
    __device__ __forceinline__ Consts consts() const
    {
        auto u = [](float f) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(f))); };
        return Consts{u(s0), u(s1), u(s2), u(t0), u(t1), u(t2)};
    }

    __device__ __forceinline__ Row row(int64_t r) const
    {
        r += m_base;
        const int64_t last = m_base + M - 1;
        if (r > last) r = last;
        const ImgDesc &d = imgs[image_of_patch(imgs, n_img, r)];
        const int local = (int)(r - d.patch_off), gy = local / d.gw, gx = local - gy * d.gw;
        const int rs = ps * d.gw * 3;
        return Row{(uint32_t)(d.pix_off - pix_sub + (int64_t)gy * ps * rs + (int64_t)gx * ps * 3), rs};
    }
    // k % 8 == 0, k < 2^14 (ps <= 64).  y = floor(k / rp) from the rounded product
    // (k + 1/2) / rp: its fraction stays at least 1/(2 rp) away from an integer, far above
    // the float error.
    __device__ __forceinline__ KChunk chunk(int k, Consts cs) const
    {
        const int y = (int)(((float)k + 0.5f) * inv_rp);
        const int b0 = k - y * rp;
        const int cph = b0 - 3 * ((b0 * 171) >> 9);   // b0 % 3 (floor(b0 / 3) exact for b0 < 256)
        const bool c0 = cph == 0, c1 = cph == 1;
        KChunk kc;
        kc.yc = y < ps ? y : ps - 1;
        kc.b0 = b0;
        kc.nv = y < ps ? min(sb - b0, 8) : 0;
        kc.sa = c0 ? cs.s0 : (c1 ? cs.s1 : cs.s2);
        kc.sb = c0 ? cs.s1 : (c1 ? cs.s2 : cs.s0);
        kc.sc = c0 ? cs.s2 : (c1 ? cs.s0 : cs.s1);
        kc.ta = c0 ? cs.t0 : (c1 ? cs.t1 : cs.t2);
        kc.tb = c0 ? cs.t1 : (c1 ? cs.t2 : cs.t0);
        kc.tc = c0 ? cs.t2 : (c1 ? cs.t0 : cs.t1);
        return kc;
    }
    // Offset of the chunk's 12-byte read: the aligned offset at or below its first byte,
    // lowered for the chunks that end the buffer so the read stays on dwords that hold pixel
    // bytes (a dword with a valid byte never crosses a page); sh: the chunk's first byte inside
    // the 12.  The bytes a chunk needs (its valid columns) are always inside the read.
    struct ChunkAddr {
        uint32_t o, sh;
    };
    __device__ __forceinline__ ChunkAddr addr(const Row &rw, const KChunk &kc) const
    {
        const uint32_t o = rw.off + (uint32_t)(kc.yc * rw.rs + kc.b0), o0 = min(o & ~3u, last12);
        return ChunkAddr{o0, o - o0};
    }
    // The 12 bytes read directly (global loads; the debug dump uses this).
    __device__ __forceinline__ RawChunk load(const Row &rw, const KChunk &kc) const
    {
        typedef __attribute__((address_space(1))) const uint32_t g_u32;
        const ChunkAddr a = addr(rw, kc);
        const g_u32 *p = (g_u32 *)(px + a.o);
        return RawChunk{p[0], p[1], p[2], a.sh};
    }
    // The 8 bf16 values of a loaded chunk: byte e is channel (cph + e) % 3; columns past nv
    // are zero.
    __device__ __forceinline__ uint4 convert(const KChunk &kc, const RawChunk &d) const
    {
        uint32_t x0 = d.d0, x1 = d.d1, x2 = d.d2;
        if (d.sh > 3) {   // a read lowered at the end of the buffer: drop its leading dwords
            x0 = d.sh > 7 ? d.d2 : d.d1;
            x1 = d.sh > 7 ? 0u : d.d2;
            x2 = 0u;
        }
        const uint32_t lo = __builtin_amdgcn_alignbyte(x1, x0, d.sh & 3u);
        const uint32_t hi = __builtin_amdgcn_alignbyte(x2, x1, d.sh & 3u);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = e < 4 ? lo : hi;
            const float sc = e % 3 == 0 ? kc.sa : (e % 3 == 1 ? kc.sb : kc.sc);
            const float tc = e % 3 == 0 ? kc.ta : (e % 3 == 1 ? kc.tb : kc.tc);
            v[e] = __builtin_fmaf((float)((w >> (8 * (e & 3))) & 0xFFu), sc, tc);
        }
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t m = (2 * j < kc.nv ? 0x0000FFFFu : 0u) | (2 * j + 1 < kc.nv ? 0xFFFF0000u : 0u);
            o[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]) & m;
        }
        return make_uint4(o[0], o[1], o[2], o[3]);
    }
};

// Columns of a patch row segment (3 ps bytes) padded to whole 8-column chunks, and the K of
// the patch projection in the loader's order (ps segments, rounded up to a multiple of 32).
inline int patch_segment_cols(int ps) { return (3 * ps + 7) / 8 * 8; }
inline int patch_gemm_k(int ps) { return (ps * patch_segment_cols(ps) + 31) / 32 * 32; }

// Most pixel bytes one SrcPatch launch may cover.
constexpr int64_t kPatchLaunchBytes = (int64_t)1 << 31;

// The pixel source of patch rows [m_first, m_first + M), whose images hold the pix_bytes
// bytes (< kPatchLaunchBytes) at lpx, the first of them at offset pix_first of the batch (the
// images' pix_off count from there).  When the launch's bytes and the misalignment of lpx
// add up to fewer than 12, lpx must point at a copy with at least 16 readable bytes.
inline SrcPatch patch_source(const uint8_t *lpx, int64_t pix_first, int64_t pix_bytes, const ImgDesc *imgs,
                             int n_img, int64_t m_first, int64_t M, const float *s3, const float *t3, int ps)
{
    const uintptr_t abs = (uintptr_t)lpx, mis = abs & 3;
    const int64_t lastd = (pix_bytes + (int64_t)mis - 1) & ~(int64_t)3;
    const int rp = patch_segment_cols(ps);
    return SrcPatch{(const uint8_t *)(abs - mis), pix_first - (int64_t)mis, (uint32_t)(lastd >= 8 ? lastd - 8 : 0),
                    imgs, n_img, m_first, M, ps, 3 * ps, rp, 1.0f / (float)rp, s3[0], s3[1], s3[2], t3[0], t3[1],
                    t3[2]};
}

// ---------------------------------------------------------------------------------------
// Address sources for the direct-to-LDS GEMM: per row a small state, per K chunk the address
// of 16 bytes (8 bf16) to copy.  Rows past M are clamped to M-1 (their outputs are never
// stored).
// ---------------------------------------------------------------------------------------
// Plain activations [M][lda]: one base pointer per row.
struct SrcPlain {
    static constexpr bool REG = false;
    struct Consts {};
    const bf16_t *A;
    int64_t lda, M;
    struct Row { const bf16_t *p; };
    __device__ __forceinline__ Row row(int64_t r) const { return Row{A + (r < M ? r : M - 1) * lda}; }
    __device__ __forceinline__ const bf16_t *addr(const Row &rw, int k) const { return rw.p + k; }
};

// 3x3 merge gather of the projector ([Z] "Step 4"): row = merged token (my, mx) of its image,
// K index = pos * D + c with pos = dy*3 + dx (position-major projector weight); positions in
// the right/bottom padding read 16 zero bytes from `zero`.
struct SrcMerge {
    static constexpr bool REG = false;
    struct Consts {};
    const bf16_t *y;
    const ImgDesc *imgs;
    int n_img;
    int64_t M;
    int D;
    const bf16_t *zero;   // at least 16 zero bytes
    struct Row { const bf16_t *base; int gh, gw, y0, x0; };
    __device__ __forceinline__ Row row(int64_t r) const
    {
        if (r >= M) r = M - 1;
        const ImgDesc &d = imgs[image_of_token(imgs, n_img, r)];
        const int local = (int)(r - d.tok_off), my = local / d.mw, mx = local - my * d.mw;
        return Row{y + (int64_t)d.patch_off * D, d.gh, d.gw, 3 * my, 3 * mx};
    }
    __device__ __forceinline__ const bf16_t *addr(const Row &rw, int k) const
    {
        const int pos = k / D, c = k - pos * D;
        const int sy = rw.y0 + pos / 3, sx = rw.x0 + pos % 3;
        return (sy < rw.gh && sx < rw.gw) ? rw.base + ((int64_t)sy * rw.gw + sx) * D + c : zero;
    }
};

