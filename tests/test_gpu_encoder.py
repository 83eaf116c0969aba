"""End-to-end parity of vit_encode / vit_dump / vit_overlay against the CPU oracle, plus the
boundary's error behaviour, determinism and image isolation."""
from dataclasses import replace

import numpy as np
import pytest

import multimodal_vision_encoder_amd as vit
import oracle
import synth
from tests.gpu_util import (assert_bf16_close, assert_projector_gate, from_dev_bf16, raw_encode,
                            qkv_after_rope, rel_l2, require_gpu)

pytestmark = pytest.mark.gpu


def run(cfg, blob, grids, pixels=None):
    torch = require_gpu()
    px = synth.make_pixels(cfg, grids) if pixels is None else pixels
    enc = vit.Encoder(cfg, blob)
    out = enc.encode(torch.from_numpy(px).cuda(), grids)
    torch.cuda.synchronize()
    return enc, px, out.cpu().numpy()


# ------------------------------------------------------------------------------------------
# bit-exact parts: patchify, the K padding of the patch projection, merge gather, overlay
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,grids", [(synth.TINY, [(6, 6)]), (synth.V41, [(5, 7), (2, 9), (1, 1)]),
                                       (synth.V41, [(24, 24)]),
                                       (replace(synth.TINY, patch=16), [(5, 7), (1, 1), (3, 6)]),
                                       (replace(synth.TINY, patch=8), [(6, 5), (2, 2)]),
                                       (replace(synth.TINY, patch=1), [(9, 7)]),
                                       (replace(synth.TINY, patch=32), [(3, 4)]),
                                       (replace(synth.TINY, patch=7), [(5, 3), (1, 1), (2, 7)]),
                                       (replace(synth.TINY, patch=3), [(1, 1)]),
                                       (replace(synth.TINY, patch=1), [(1, 1)]),
                                       (replace(synth.TINY, patch=64), [(2, 3)]),
                                       (replace(synth.TINY, patch=1), [(1, 1), (1, 1), (1, 1)]),
                                       (replace(synth.TINY, patch=2), [(1, 1)])],
                         ids=["tiny", "ragged", "one_layer", "patch16", "patch8", "patch1", "patch32", "patch7",
                              "patch3_one_patch", "patch1_three_bytes", "patch64", "patch1_nine_bytes",
                              "patch2_twelve_bytes"])
@pytest.mark.parametrize("misalign", [0, 1, 3], ids=["aligned", "px+1", "px+3"])
def test_patchify_bit_exact(cfg, grids, misalign):
    """The patch matrix the fused loader feeds the patch projection (dumped through the same
    device functions), bit-exact against the oracle's patchify: patch sides 1 to 64 (segments
    of 3 to 192 bytes, odd sides misaligning every other segment), packed ragged batches,
    batches of 3, 9 and 12 bytes (under 12, the loader reads a padded copy), and pixel buffers
    that start 1 or 3 bytes past an aligned address (the loader reads 12 aligned bytes around
    each chunk, lowered at the end of the buffer so that it never passes the last dword)."""
    torch = require_gpu()
    c1 = replace(cfg, layers=0, out_hidden=16)
    enc = vit.Encoder(c1, synth.make_weights(c1))
    px = synth.make_pixels(c1, grids)
    store = torch.zeros(px.size + 8, dtype=torch.uint8, device="cuda")
    store[misalign:misalign + px.size] = torch.from_numpy(px).cuda()
    d_px = store[misalign:misalign + px.size]
    assert d_px.data_ptr() % 4 == misalign
    got = from_dev_bf16(enc.dump(vit.DUMP_PATCHES, d_px, grids))
    torch.cuda.synchronize()
    off, pix = 0, 0
    for gh, gw in grids:
        n, npx = gh * gw, c1.patch * gh * c1.patch * gw * 3
        assert np.array_equal(got[off:off + n], oracle.patchify(px[pix:pix + npx], gh, gw, c1))
        off += n
        pix += npx


@pytest.mark.parametrize("grids", [[(7, 5), (3, 3)], [(96, 96), (7, 5), (3, 3)]], ids=["small", "96x96_packed"])
def test_identity_patch_projection_bit_exact(grids):
    """W_pe = identity (D = 1024 >= 588 columns), b = 0: x0[:, :588] = patches and 0 after;
    exact because each output has one non-zero product, so the patchify inside the projection's
    A loader, the permutation of W_pe into the loader's K order (588 columns spread over 672)
    and its zero columns are checked together, on every row (9,260 rows: 148 tiles of 256 x 256,
    a ragged last tile row)."""
    torch = require_gpu()
    cfg = replace(synth.V41, layers=0, out_hidden=16)
    blob = synth.make_weights(cfg)
    W = synth.split_weights(cfg, blob)
    W["pe.w"][:] = 0
    W["pe.w"][np.arange(588), np.arange(588)] = 0x3F80
    enc = vit.Encoder(cfg, blob)
    px = synth.make_pixels(cfg, grids)
    x0 = from_dev_bf16(enc.dump(vit.DUMP_EMBED, torch.from_numpy(px).cuda(), grids))
    torch.cuda.synchronize()
    parts, off = [], 0
    for gh, gw in grids:
        n = 14 * gh * 14 * gw * 3
        parts.append(oracle.patchify(px[off:off + n], gh, gw, cfg))
        off += n
    assert np.array_equal(x0[:, :588], np.concatenate(parts))
    assert not x0[:, 588:].any()


def test_patch_projection_over_2gib_of_pixels():
    """A batch of 400 images of 96 x 96 patches holds 2.17 GB of pixels, more than one launch of
    the fused patch loader addresses (under 2^31 bytes): the projection runs in groups of whole
    images (here 396 and 4).  The patch matrix and the projection of the first image, the two
    images at the group boundary and the last image match the oracle (patches bit-exact).
    Pixels drawn on the GPU from a seeded generator (2 GB would take minutes on the host)."""
    torch = require_gpu()
    cfg = replace(synth.TINY, layers=0, out_hidden=16)
    blob = synth.make_weights(cfg)
    W = oracle.Weights(cfg, blob)
    enc = vit.Encoder(cfg, blob)
    grids = [(96, 96)] * 400
    per = 14 * 96 * 14 * 96 * 3
    assert 396 * per < 2 ** 31 < 397 * per
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20251202)
    d_px = torch.randint(0, 256, (400 * per,), dtype=torch.uint8, device="cuda", generator=gen)
    P = enc.dump(vit.DUMP_PATCHES, d_px, grids)
    X = enc.dump(vit.DUMP_EMBED, d_px, grids)
    torch.cuda.synchronize()
    for i in (0, 395, 396, 399):
        img = d_px[i * per:(i + 1) * per].cpu().numpy()
        want = oracle.patchify(img, 96, 96, cfg)
        got = from_dev_bf16(P[i * 9216:(i + 1) * 9216])
        assert np.array_equal(got, want), i
        x_want = oracle.linear(want, None, W["pe.b"], Wt=W.T("pe.w"))
        # slack for an fp32 sum taken in another order: 2^-18 sum_k |p_k w_k| per output
        slack = 2.0 ** -18 * (np.abs(want).astype(np.float64) @ np.abs(W.T("pe.w")).astype(np.float64))
        assert_bf16_close(from_dev_bf16(X[i * 9216:(i + 1) * 9216]), x_want, atol=slack,
                          what=f"embed of image {i}")


@pytest.mark.parametrize("cfg,grids", [(synth.V41, [(5, 7), (96, 96), (1, 1), (3, 11)]),
                                       (synth.TINY, [(6, 6), (2, 9)]),
                                       (replace(synth.V41, heads=8, rope_base=500.0), [(9, 4), (13, 2)])],
                         ids=["hd64_packed", "hd16", "hd128_base500"])
def test_rope_dump_matches_oracle_angles(cfg, grids):
    """[Z] "Step 2" table, the "2D RoPE cos/sin" boundary: the cos and sin of every rotary
    angle of every patch of a packed batch, read through the device lookup the QKV epilogue
    rotates with, equal the oracle's angle function bit for bit (both evaluate the angle in
    double and round once).  The 96x96 image is checked on every row of its first and last
    grid rows and on 64 sampled rows in between."""
    torch = require_gpu()
    c0 = replace(cfg, layers=0, out_hidden=16)
    enc = vit.Encoder(c0, synth.make_weights(c0))
    px = synth.make_pixels(c0, grids)
    got = enc.dump(vit.DUMP_ROPE, torch.from_numpy(px).cuda(), grids).cpu().numpy()
    torch.cuda.synchronize()
    hd, half = c0.hidden // c0.heads, c0.hidden // c0.heads // 2
    assert got.shape == (sum(gh * gw for gh, gw in grids), hd) and got.dtype == np.float32
    rng = np.random.default_rng(7)
    off = 0
    for gh, gw in grids:
        n = gh * gw
        rows = np.arange(n)
        if n > 512:
            rows = np.unique(np.concatenate([np.arange(gw), np.arange(n - gw, n), rng.integers(0, n, 64)]))
        for p in rows:
            h, w = divmod(int(p), gw)
            want = np.array([oracle.rope_angle(h, w, i, hd, c0.rope_base) for i in range(half)], np.float32)
            assert np.array_equal(got[off + p, :half], want[:, 0]), (gh, gw, p)
            assert np.array_equal(got[off + p, half:], want[:, 1]), (gh, gw, p)
        off += n


def test_rope_dump_contract():
    """The RoPE boundary reads no pixels (NULL accepted), and refuses a destination of the
    wrong size or one not 16-byte aligned, writing nothing."""
    import ctypes
    torch = require_gpu()
    c0 = replace(synth.V41, layers=0, out_hidden=16)
    enc = vit.Encoder(c0, synth.make_weights(c0))
    grids = [(4, 5), (2, 3)]
    buf = torch.full((26 * 64 + 4,), 7.0, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(dst, nbytes):
        return vit.lib().vit_dump(enc._ctx, vit.DUMP_ROPE, 0, None, vit.grid_array(grids), len(grids),
                                  ctypes.c_void_p(dst), nbytes, stream)
    assert call(buf.data_ptr(), 26 * 64 * 4) == vit.VIT_OK
    torch.cuda.synchronize()
    ref = buf[:26 * 64].clone()
    assert not torch.equal(ref, torch.full_like(ref, 7.0))
    buf.fill_(7.0)
    torch.cuda.synchronize()
    assert call(buf.data_ptr() + 4, 26 * 64 * 4) == vit.VIT_E_ARG          # misaligned
    assert call(buf.data_ptr(), 26 * 64 * 4 - 4) == vit.VIT_E_ARG          # wrong size
    torch.cuda.synchronize()
    assert torch.equal(buf, torch.full_like(buf, 7.0))


@pytest.mark.parametrize("base,grids", [(synth.TINY, [(5, 7), (6, 6), (1, 2)]),
                                        (synth.V41, [(5, 7), (96, 96), (4, 9), (1, 2)])],
                         ids=["d64", "d1024_96x96"])
def test_merge_gather_one_hot_projector_bit_exact(base, grids):
    """W_proj row j = e_sigma(j) over all 9D columns (out_hidden = 9D: 9,216 columns at full
    width), b = 0: the projector output is the merged input permuted by sigma, exactly; the
    merged input comes from the oracle's merge of the same seeded rows ([Z] "Step 4": channel-
    major 3x3 unfold with right/bottom padding, which the 5x7 and 4x9 grids exercise)."""
    torch = require_gpu()
    cfg = replace(base, layers=0, out_hidden=9 * base.hidden)
    blob = synth.make_weights(cfg)
    W = synth.split_weights(cfg, blob)
    sigma = np.random.default_rng(7).permutation(9 * cfg.hidden)
    W["proj.w"][:] = 0
    W["proj.w"][np.arange(9 * cfg.hidden), sigma] = 0x3F80
    enc = vit.Encoder(cfg, blob)
    N = sum(a * b for a, b in grids)
    y = synth.normal_bf16(201, 0, N * cfg.hidden).reshape(N, cfg.hidden)
    from tests.gpu_util import to_dev_bf16
    got = enc.op_merge_project(to_dev_bf16(y), grids).cpu().numpy()
    torch.cuda.synchronize()
    yf = synth.bf16_bits_to_f32(y)
    off, want = 0, []
    for gh, gw in grids:
        want.append(oracle.merge(yf[off:off + gh * gw], gh, gw)[:, sigma])
        off += gh * gw
    assert np.array_equal(got, np.concatenate(want))


@pytest.mark.parametrize("cfg,grids", [(synth.TINY, [(5, 7), (6, 9)]),
                                       (replace(synth.V41, layers=0), [(5, 7), (96, 96), (4, 9)])],
                         ids=["d64", "d1024_96x96"])
def test_merged_dump_is_the_channel_major_unfold_of_the_final_norm(cfg, grids):
    """vit_dump(MERGED) (the projector's own gather) equals the unfold of vit_dump(FINAL_NORM)
    with right/bottom zero padding, element for element, at width 64 and at full width."""
    torch = require_gpu()
    enc = vit.Encoder(cfg, synth.make_weights(cfg))
    px = torch.from_numpy(synth.make_pixels(cfg, grids)).cuda()
    y = enc.dump(vit.DUMP_FINAL_NORM, px, grids).float()
    A = from_dev_bf16(enc.dump(vit.DUMP_MERGED, px, grids))
    torch.cuda.synchronize()
    off, t0 = 0, 0
    for gh, gw in grids:
        img = y[off:off + gh * gw].reshape(gh, gw, -1).permute(2, 0, 1)[None].cpu()
        img = torch.nn.functional.pad(img, (0, (-gw) % 3, 0, (-gh) % 3))
        want = torch.nn.functional.unfold(img, 3, stride=3)[0].T.numpy()
        assert np.array_equal(A[t0:t0 + want.shape[0]], want)
        off += gh * gw
        t0 += want.shape[0]


# ------------------------------------------------------------------------------------------
# end to end
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("perturbed", [False, True])
def test_tiny_end_to_end(perturbed):
    wl = synth.workload("tiny")
    blob = synth.make_weights(wl.cfg, perturbed=perturbed)
    enc, px, got = run(wl.cfg, blob, wl.grids)
    want = oracle.encode(wl.cfg, blob, px, wl.grids)
    assert got.shape == (4, 128)
    assert_projector_gate(got, want, "tiny")


@pytest.mark.parametrize("patch", [16, 8])
def test_other_patch_sizes_end_to_end(patch):
    """Patch sides other than 14 (K = 3 p^2 = 768 and 192, zero-padded to multiples of 64)."""
    cfg = replace(synth.TINY, patch=patch)
    grids = [(6, 6), (5, 7), (1, 1)]
    blob = synth.make_weights(cfg, perturbed=True)
    enc, px, got = run(cfg, blob, grids)
    want = oracle.encode(cfg, blob, px, grids)
    assert_projector_gate(got, want, f"patch {patch}")


def test_tiny_ragged_multi_image():
    cfg = synth.TINY
    grids = [(5, 7), (6, 6), (1, 1), (10, 4)]
    blob = synth.make_weights(cfg, perturbed=True)
    enc, px, got = run(cfg, blob, grids)
    want = oracle.encode(cfg, blob, px, grids)
    assert got.shape[0] == 6 + 4 + 1 + 8
    assert_projector_gate(got, want, "tiny ragged")


@pytest.mark.parametrize("perturbed", [False, True])
def test_one_layer_end_to_end(perturbed):
    """One full-width layer (336x336 image, 576 patches, 9216 -> 5120 projector), with the
    boundary tensors compared on the way to locate the first divergence."""
    torch = require_gpu()
    wl = synth.workload("one_layer")
    blob = synth.make_weights(wl.cfg, perturbed=perturbed)
    enc, px, got = run(wl.cfg, blob, wl.grids)
    W = oracle.Weights(wl.cfg, blob)
    dumps = {}
    want = oracle.encode_image(wl.cfg, W, px, 24, 24, workers=8, dumps=dumps)
    d_px = torch.from_numpy(px).cuda()
    assert np.array_equal(from_dev_bf16(enc.dump(vit.DUMP_PATCHES, d_px, wl.grids)), dumps["patches"])
    assert_bf16_close(from_dev_bf16(enc.dump(vit.DUMP_EMBED, d_px, wl.grids)), dumps["embed"],
                      atol=1e-6, what="embed")
    for name, b, arg in (("qkv0", vit.DUMP_QKV, 0), ("attn0", vit.DUMP_ATTN, 0),
                         ("layer0", vit.DUMP_LAYER, 0), ("final_norm", vit.DUMP_FINAL_NORM, 0)):
        t = enc.dump(b, d_px, wl.grids, arg=arg)
        g = qkv_after_rope(t, wl.cfg.hidden) if b == vit.DUMP_QKV else from_dev_bf16(t)
        assert rel_l2(g, dumps[name]) < 1e-2, name
    assert_projector_gate(got, want, "one layer")


@pytest.mark.parametrize("perturbed", [False, True])
def test_official_variant_tiny_end_to_end(perturbed):
    """RMSNorm blocks and final norm, SwiGLU MLP, erf GELU, two-linear aligner; ragged images."""
    cfg = synth.TINY_OFFICIAL
    grids = [(6, 6), (5, 7), (1, 1)]
    blob = synth.make_weights(cfg, perturbed=perturbed)
    enc, px, got = run(cfg, blob, grids)
    want = oracle.encode(cfg, blob, px, grids)
    assert got.shape == (4 + 6 + 1, cfg.out_hidden)
    assert_projector_gate(got, want, "official tiny")


def test_official_variant_one_layer_end_to_end():
    """One full-width official-variant layer (336x336 image, F = 4096 SwiGLU, 9216 -> 5120 ->
    5120 aligner) with the boundary tensors compared on the way."""
    torch = require_gpu()
    cfg = replace(synth.V41_OFFICIAL, layers=1)
    grids = [(24, 24)]
    blob = synth.make_weights(cfg, perturbed=True)
    enc, px, got = run(cfg, blob, grids)
    W = oracle.Weights(cfg, blob)
    dumps = {}
    want = oracle.encode_image(cfg, W, px, 24, 24, workers=8, dumps=dumps)
    d_px = torch.from_numpy(px).cuda()
    for name, b, arg in (("layer0", vit.DUMP_LAYER, 0), ("final_norm", vit.DUMP_FINAL_NORM, 0)):
        g = from_dev_bf16(enc.dump(b, d_px, grids, arg=arg))
        assert rel_l2(g, dumps[name]) < 1e-2, name
    assert_projector_gate(got, want, "official one layer")


@pytest.mark.parametrize("hidden,heads,official", [(128, 4, False), (256, 2, False), (512, 16, True),
                                                    (1536, 12, False), (2048, 16, True), (128, 8, True)],
                         ids=["d128_hd32", "d256_hd128", "d512_hd32_official", "d1536_hd128",
                              "d2048_hd128_official", "d128_hd16_official"])
def test_widths_and_head_dims_end_to_end(hidden, heads, official):
    """The other widths (128 .. 2048) and head dims (16, 32, 128) the build supports, both
    layer kinds, two layers, on a ragged batch (6x6, 5x7, 1x1, 9x12) against the oracle.
    Gate: rel-L2 <= 1e-2, and max-abs within 5e-2 or, for the wide aligners whose outputs sum
    up to 9 x 2048 products, within 1.5 x the gap between the fp32 oracle and its fp64 twin on
    the same rows (an exact implementation can be no closer to the fp32 oracle)."""
    cfg = replace(synth.TINY, hidden=hidden, heads=heads, mlp=4 * hidden, layers=2, out_hidden=192,
                  pix_mean=synth.V41.pix_mean, pix_std=synth.V41.pix_std)
    if official:
        cfg = replace(cfg, norm_kind=1, mlp_kind=1, gelu_kind=1, aligner_hidden=256)
    grids = [(6, 6), (5, 7), (1, 1), (9, 12)]
    blob = synth.make_weights(cfg, perturbed=True)
    enc, px, got = run(cfg, blob, grids)
    want = oracle.encode(cfg, blob, px, grids, workers=8)
    assert got.shape == (4 + 6 + 1 + 12, cfg.out_hidden)
    r, m = rel_l2(got, want), float(np.abs(got - want).max())
    bound = 5e-2
    if m > bound:
        w64 = oracle.encode(cfg, blob, px, grids, prec="f64", workers=8)
        bound = max(bound, 1.5 * float(np.abs(w64 - want).max()))
    assert r <= 1e-2 and m <= bound, (hidden, heads, r, m, bound)
    enc.close()


def test_many_small_images():
    """300 seeded grids from 1x1 to 12x12 in one call (13,557 patches, 1,992 tokens): the
    per-image metadata, the 64-aligned transposed-V columns of each image, the attention work
    list and the merge gather all at many images, against the oracle image by image."""
    cfg = synth.TINY
    rng = np.random.default_rng(31)
    grids = [(int(a), int(b)) for a, b in rng.integers(1, 13, size=(300, 2))]
    blob = synth.make_weights(cfg, perturbed=True)
    enc, px, got = run(cfg, blob, grids)
    want = oracle.encode(cfg, blob, px, grids)
    assert got.shape == want.shape
    assert_projector_gate(got, want, "300 small images")


def test_official_variant_reserve():
    """After vit_reserve the two-projection aligner's inner rows are sized for the reserved
    patches: a batch of 1x1 images (one merged token per patch, the most tokens a batch can
    have) encodes within the cap, bitwise as an unreserved context does; a batch larger than
    the reserved workspace (at least 64 patches) is refused with VIT_E_NOMEM and writes
    nothing."""
    torch = require_gpu()
    cfg = synth.TINY_OFFICIAL
    blob = synth.make_weights(cfg, perturbed=True)
    grids = [(1, 1)] * 12 + [(6, 6)]
    n = 12 + 36
    px = torch.from_numpy(synth.make_pixels(cfg, grids)).cuda()
    free = vit.Encoder(cfg, blob)
    want = free.encode(px, grids).cpu().numpy()
    enc = vit.Encoder(cfg, blob)
    enc.reserve(n)
    got = enc.encode(px, grids).cpu().numpy()
    assert got.shape == (16, cfg.out_hidden) and np.array_equal(got, want)
    big = grids + [(6, 6)]          # 84 patches: beyond the workspace the reserve allocated
    px2 = torch.from_numpy(synth.make_pixels(cfg, big)).cuda()
    out = torch.full((20, cfg.out_hidden), 7.0, device="cuda")
    with pytest.raises(vit.VitError) as e:
        enc.encode(px2, big, out=out)
    assert e.value.status == vit.VIT_E_NOMEM
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    free.close()
    enc.close()


def test_uniform_gray_image_rows_agree():
    """A flat RGB-127 canvas: all patches equal, v equal at every position, so every visual
    row is the same vector up to rounding (positions enter only through q and k)."""
    cfg = synth.V41_ONE_LAYER
    grids = [(12, 12)]
    px = np.full(14 * 12 * 14 * 12 * 3, 127, np.uint8)
    blob = synth.make_weights(cfg)
    enc, _, got = run(cfg, blob, grids, pixels=px)
    want = oracle.encode(cfg, blob, px, grids, workers=8)
    assert_projector_gate(got, want, "uniform")
    assert rel_l2(got, np.repeat(got[:1], got.shape[0], 0)) < 1e-2


# ------------------------------------------------------------------------------------------
# boundary behaviour
# ------------------------------------------------------------------------------------------
def test_errors_publish_nothing():
    torch = require_gpu()
    cfg = synth.TINY
    enc = vit.Encoder(cfg, synth.make_weights(cfg))
    grids_ok = [(6, 6)]
    px = torch.from_numpy(synth.make_pixels(cfg, grids_ok)).cuda()
    out = torch.full((4, cfg.out_hidden), 7.0, device="cuda")
    over = replace(cfg, max_tokens_per_image=3)
    enc_small = vit.Encoder(over, synth.make_weights(over))
    with pytest.raises(vit.VitError) as e:
        enc_small.encode(px, grids_ok, out=out)
    assert e.value.status == vit.VIT_E_BUDGET
    # the library's own checks, through the C ABI (the binding refuses these grids itself)
    assert raw_encode(enc, px, [(6, 6), (0, 3)], out) == vit.VIT_E_ARG
    assert raw_encode(enc, px, [(6, 6), (6000, 1)], out) == vit.VIT_E_ARG
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call must not write any output"
    # an empty batch is valid and writes nothing
    assert raw_encode(enc, px, [], out) == vit.VIT_OK
    assert enc.encode(px[:0], []).shape == (0, cfg.out_hidden)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # the binding refuses tensors the kernels would overrun
    with pytest.raises(ValueError):
        enc.encode(px[:-1], grids_ok, out=out)
    with pytest.raises(ValueError):
        enc.encode(px, [(6, 6), (0, 3)], out=out)
    with pytest.raises(ValueError):
        enc.encode(px, grids_ok, out=out[:3])
    with pytest.raises(ValueError):
        enc.encode(px, grids_ok, out=out.to(torch.bfloat16))
    with pytest.raises(vit.VitError):
        enc.overlay(torch.zeros((8, cfg.out_hidden), dtype=torch.bfloat16, device="cuda"),
                    [1, 1], torch.zeros((2, cfg.out_hidden), device="cuda"))
    with pytest.raises(vit.VitError):
        enc.overlay(torch.zeros((8, cfg.out_hidden), dtype=torch.bfloat16, device="cuda"),
                    [8], torch.zeros((1, cfg.out_hidden), device="cuda"))
    enc.close()
    enc_small.close()


def test_deterministic_and_isolated():
    """Two runs of a batch are bitwise identical.  An image's rows do not depend on the other
    images of the packed batch beyond summation order (the GEMM K split is chosen from the
    batch size: here the lone image's patch projection is cut into K slices, the pair's is
    not): encoded alone or next to another image, they meet the parity gate against the
    oracle and against each other."""
    torch = require_gpu()
    cfg = synth.V41_ONE_LAYER
    blob = synth.make_weights(cfg, perturbed=True)
    grids = [(12, 15), (9, 9)]
    px = synth.make_pixels(cfg, grids)
    enc = vit.Encoder(cfg, blob)
    d = torch.from_numpy(px).cuda()
    a = enc.encode(d, grids).cpu().numpy()
    b = enc.encode(d, grids).cpu().numpy()
    n0 = 14 * 12 * 14 * 15 * 3
    alone = enc.encode(torch.from_numpy(px[n0:]).cuda(), grids[1:]).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(a, b)
    want = oracle.encode(cfg, blob, px[n0:], grids[1:], workers=8)
    assert_projector_gate(a[4 * 5:], want, "in the batch")
    assert_projector_gate(alone, want, "alone")
    assert_projector_gate(a[4 * 5:], alone, "in the batch against alone")


# ------------------------------------------------------------------------------------------
# preprocessing: contain resize onto the gray canvas
# ------------------------------------------------------------------------------------------
_V41P = dict(max_tokens=1024, min_pixels=295936, max_aspect=0)
_V4P = dict(max_tokens=384, min_pixels=147456, max_aspect=8)


@pytest.mark.parametrize("h,w,prof", [(1344, 1344, _V41P), (1000, 700, _V41P), (2900, 1900, _V41P),
                                      (200, 150, _V41P), (300, 2900, _V4P), (9, 400, _V4P), (1, 1, _V4P)],
                         ids=["same-size", "enlarge-to-grid", "shrink", "min-pixels", "aspect-clamp",
                              "thin", "single-pixel"])
def test_preprocess_canvas_matches_oracle(h, w, prof):
    """The GPU canvas against the oracle's (fp64 weights and sums): the gray padding and the
    placement exact, every resized pixel within one level.  Off-by-one levels come from the
    fp32 sums (two passes of up to ~16 taps of values <= 255: absolute error about 2e-3) landing
    on the other side of a .5 than the fp64 ones; with fractional parts spread uniformly that is
    about 0.4% of the pixels, so at most 0.5% may differ."""
    from oracle import preprocess as pp
    torch = require_gpu()
    enc = vit.Encoder(synth.TINY, synth.make_weights(synth.TINY))
    img = synth.uniform_bytes(31, h, h * w * 3).reshape(h, w, 3)
    plan = vit.plan_image(h, w, **prof)
    got = enc.preprocess(torch.from_numpy(img).cuda(), h, w, plan)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = pp.preprocess(img, plan)
    assert got.shape == want.shape
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    y0, x0, rh, rw = plan["off_y"], plan["off_x"], plan["resized_h"], plan["resized_w"]
    pad = np.ones(got.shape[:2], bool)
    pad[y0:y0 + rh, x0:x0 + rw] = False
    assert (got[pad] == 127).all()
    assert diff.max() <= 1
    assert (diff > 0).mean() <= 5e-3
    enc.close()


def test_preprocess_then_encode():
    """A 100 x 160 image through the whole chain on the GPU (plan, canvas, encode) against the
    oracle's canvas encoded by the oracle: the projector gate."""
    from oracle import preprocess as pp
    torch = require_gpu()
    cfg = synth.TINY
    blob = synth.make_weights(cfg)
    enc = vit.Encoder(cfg, blob)
    h, w = 100, 160
    img = synth.uniform_bytes(32, 0, h * w * 3).reshape(h, w, 3)
    plan = vit.plan_image(h, w, patch=cfg.patch, merge=3, max_tokens=cfg.max_tokens_per_image,
                          min_pixels=295936, max_aspect=0)
    grids = [(plan["gh"], plan["gw"])]
    canvas = enc.preprocess(torch.from_numpy(img).cuda(), h, w, plan)
    got = enc.encode(canvas.reshape(-1), grids)
    torch.cuda.synchronize()
    want = oracle.encode(cfg, blob, pp.preprocess(img, plan).reshape(-1), grids, workers=8)
    assert_projector_gate(got.cpu().numpy(), want, "preprocess + encode")
    enc.close()
