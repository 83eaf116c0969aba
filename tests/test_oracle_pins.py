"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values the pages state, closed forms, invariants, library routines (torch / numpy in fp64)
and brute force on tiny inputs.  Each test names the mistake it is there to catch.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def page_facts():
    out = {}
    with open(os.path.join(HERE, "golden", "page_facts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = float(v)
    return out


def bf16_torch(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


# ------------------------------------------------------------------------------------------
# bf16 rounding (every rounding point of the encoder)
# ------------------------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 20000),
                        # exact ties: bf16 value + half ulp, both parities
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),  # subnormal
                        ((np.arange(1, 4000, dtype=np.uint32) << 16) + (100 << 23) | 0x8000).view(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-30], np.float32)])
    assert np.array_equal(oracle.round_bf16(x), bf16_torch(x))
    # the fp64 twin rounds the same values the same way
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64), "f64").astype(np.float32), bf16_torch(x))


# ------------------------------------------------------------------------------------------
# patchify: order (grid_y, grid_x, channel, y, x) and the pixel map
# ------------------------------------------------------------------------------------------
def _closed_form_image(gh, gw, ps=14):
    y, x, c = np.meshgrid(np.arange(ps * gh), np.arange(ps * gw), np.arange(3), indexing="ij")
    return ((7 * y + 3 * x + 11 * c) % 256).astype(np.uint8)


@pytest.mark.parametrize("cfg", [synth.TINY, synth.V41], ids=["clip", "unit"])
def test_patchify_closed_form(cfg):
    """Catches a wrong flatten order (e.g. HWC inside the row, or x/y swapped) and a wrong
    normalisation constant: each element is checked against its closed form."""
    gh, gw = 4, 5
    img = _closed_form_image(gh, gw)
    P = oracle.patchify(img.reshape(-1), gh, gw, cfg)
    # the constants from their definition (fp32 of 1/(255 std_c) and -mean_c/std_c), not from
    # the oracle's own helper
    mean = np.float32(cfg.pix_mean).astype(np.float64)
    std = np.float32(cfg.pix_std).astype(np.float64)
    s = (1.0 / (255.0 * std)).astype(np.float32)
    t = (-mean / std).astype(np.float32)
    # reference order by reshaping the image: (gy, y, gx, x, c) -> (gy, gx, c, y, x)
    blocks = img.reshape(gh, 14, gw, 14, 3).transpose(0, 2, 4, 1, 3).reshape(gh * gw, 588)
    chan = np.repeat(np.arange(3), 196)
    # u*s + t in double is exact (8-bit times 24-bit), so one rounding to fp32 equals fmaf
    want = bf16_torch((blocks.astype(np.float64) * s[chan].astype(np.float64)
                       + t[chan].astype(np.float64)).astype(np.float32))
    assert np.array_equal(P, want)
    # element-by-element closed form for a few entries
    for gy, gx, c, yy, xx in [(0, 0, 0, 0, 0), (3, 4, 2, 13, 13), (1, 2, 1, 5, 9)]:
        u = (7 * (gy * 14 + yy) + 3 * (gx * 14 + xx) + 11 * c) % 256
        assert P[gy * gw + gx, c * 196 + yy * 14 + xx] == want[gy * gw + gx, c * 196 + yy * 14 + xx]
        assert blocks[gy * gw + gx, c * 196 + yy * 14 + xx] == u


def test_pixel_map_endpoints():
    """[0, 255] maps onto [-1, 1] with mean = std = 0.5."""
    img = np.zeros((14, 14, 3), np.uint8)
    img[0, 0] = 255
    P = oracle.patchify(img.reshape(-1), 1, 1, synth.V41)
    assert P[0, 1] == -1.0
    assert P[0, 0] == 1.0 and P[0, 196] == 1.0 and P[0, 392] == 1.0


# ------------------------------------------------------------------------------------------
# facts stated by the pages
# ------------------------------------------------------------------------------------------
def test_page_dimensions():
    f = page_facts()
    cfg = synth.V41
    assert cfg.patch == f["patch_side"] and cfg.patch_dim == f["patch_columns"]
    assert cfg.hidden == f["vision_hidden"] and cfg.heads == f["vision_heads"]
    assert cfg.layers == f["vision_layers"] and cfg.merge == f["merge_window"]
    assert cfg.out_hidden == f["lm_hidden_v41"] and cfg.max_tokens_per_image == f["max_tokens_v41"]
    assert synth.V4.out_hidden == f["lm_hidden_v4"] and synth.V4.max_tokens_per_image == f["max_tokens_v4"]


@pytest.mark.parametrize("px,grid,tokens", [((84, 84), (6, 6), 4), ((336, 336), (24, 24), 64),
                                            ((756, 882), (54, 63), 378),
                                            ((1344, 1344), (96, 96), 1024)])
def test_token_counts(px, grid, tokens):
    """Token counts are grid/3 per axis; the 1344x1344 image sits exactly at the V4.1 cap and
    the 756x882 one under the V4 cap."""
    f = page_facts()
    gh, gw = px[0] // int(f["patch_side"]), px[1] // int(f["patch_side"])
    assert (gh, gw) == grid
    assert synth.V41.tokens(gh, gw) == tokens
    A = oracle.merge(np.zeros((gh * gw, 1), np.float32), gh, gw)
    assert A.shape[0] == tokens
    if tokens == 1024:
        assert tokens == f["max_tokens_v41"]
    if tokens == 378:
        assert tokens <= f["max_tokens_v4"]


def test_parameter_count_matches_published_size():
    """LayerNorm blocks + GELU MLP + one projector: 450.87 M bf16 parameters = 0.90 GB, the
    size of the published V4.1 vision download (a sanity check on the architecture reading)."""
    n = synth.V41.blob_elems()
    assert n == 450_875_392
    assert abs(2 * n / 1e9 - page_facts()["v41_weight_gb"]) < 0.01


# ------------------------------------------------------------------------------------------
# linear layers, GELU, LayerNorm
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("prec", ["f32", "f64"])
def test_linear_vs_numpy_fp64(prec):
    """Catches a transposed weight, a dropped bias or an off-by-one in K."""
    rng = np.random.default_rng(2)
    A = rng.standard_normal((7, 13))
    W = rng.standard_normal((5, 13))
    b = rng.standard_normal(5)
    got = oracle.linear(A, W, b, round_out=False, prec=prec)
    want = A @ W.T + b
    tol = 1e-5 if prec == "f32" else 1e-12
    np.testing.assert_allclose(got, want, rtol=tol, atol=tol)
    # rows split over workers give identical results
    got2 = oracle.linear(A, W, b, round_out=False, prec=prec, workers=3)
    assert np.array_equal(got, got2)


def test_linear_one_hot_is_exact_copy():
    rng = np.random.default_rng(3)
    A = bf16_torch(rng.standard_normal((9, 40)))
    sel = rng.permutation(40)[:11]
    W = np.zeros((11, 40), np.float32)
    W[np.arange(11), sel] = 1.0
    got = oracle.linear(A, W, None)
    assert np.array_equal(got, A[:, sel])


def test_gelu_tanh_vs_torch_and_identities():
    import torch
    u = np.linspace(-8, 8, 2001)
    got = np.array([oracle.gelu_tanh(v, "f64") for v in u])
    want = torch.nn.functional.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)
    got32 = np.array([oracle.gelu_tanh(v) for v in u])
    np.testing.assert_allclose(got32, want, rtol=0, atol=2e-6)
    assert oracle.gelu_tanh(0.0) == 0.0
    np.testing.assert_allclose(got - got[::-1], u, atol=1e-12)       # gelu(u) - gelu(-u) = u
    # the tanh form stays within ~1e-3 of the erf form, as the first page reports
    erf = torch.nn.functional.gelu(torch.from_numpy(u)).numpy()
    assert np.abs(got - erf).max() < 1e-3


def test_linear_gelu_epilogue_single_rounding():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((6, 8))
    W = rng.standard_normal((5, 8))
    b = rng.standard_normal(5)
    got = oracle.linear(A, W, b, act=1, prec="f64")
    import torch
    pre = torch.from_numpy(A @ W.T + b)
    want = torch.nn.functional.gelu(pre, approximate="tanh").to(torch.bfloat16).to(torch.float64).numpy()
    assert np.abs(got - want).max() <= 2 ** -7 * np.abs(want).max()


@pytest.mark.parametrize("prec", ["f32", "f64"])
def test_layernorm_vs_torch(prec):
    import torch
    rng = np.random.default_rng(5)
    x = rng.standard_normal((10, 64)) * 3 + 1
    x[3] = 0.5 + 1e-4 * rng.standard_normal(64)      # variance far below eps: eps placement shows
    g = 1 + 0.1 * rng.standard_normal(64)
    b = 0.1 * rng.standard_normal(64)
    # inputs exactly representable in the oracle's precision
    dt = np.float32 if prec == "f32" else np.float64
    x, g, b = (v.astype(dt).astype(np.float64) for v in (x, g, b))
    got = oracle.layernorm(x, g, b, 1e-6, prec)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (64,), torch.from_numpy(g),
                                          torch.from_numpy(b), eps=1e-6).numpy()
    # outputs are bf16-rounded: allow one bf16 ulp (plus fp32 cancellation in x - mu on the
    # near-constant row for the fp32 oracle)
    atol = 2e-3 if prec == "f32" else 1e-6
    assert np.all(np.abs(got - want) <= 2 ** -8 * np.abs(want) + atol)


def test_layernorm_constant_row_gives_beta_and_is_shift_invariant():
    g = np.linspace(0.5, 1.5, 64)
    b = bf16_torch(np.linspace(-1, 1, 64))
    x = np.full((1, 64), 3.25)
    assert np.array_equal(oracle.layernorm(x, g, b, 1e-6), b[None, :])
    rng = np.random.default_rng(6)
    x = bf16_torch(rng.standard_normal((4, 64)))
    y1 = oracle.layernorm(x, np.ones(64), np.zeros(64), 1e-6, "f64")
    y2 = oracle.layernorm(x * 4.0 + 8.0, np.ones(64), np.zeros(64), 1e-6, "f64")
    assert np.abs(y1 - y2).max() <= 2 ** -7 * np.abs(y1).max()
    np.testing.assert_allclose(y1.mean(1), 0, atol=2e-2)
    np.testing.assert_allclose(y1.var(1), 1, atol=2e-2)


# ------------------------------------------------------------------------------------------
# 2D RoPE
# ------------------------------------------------------------------------------------------
def _qkv_rows(n, D, seed):
    rng = np.random.default_rng(seed)
    return bf16_torch(rng.standard_normal((n, 3 * D)))


def test_rope_origin_is_identity():
    qkv = _qkv_rows(1, 1024, 7)
    assert np.array_equal(oracle.rope_qk(qkv, 5, 1024, 16, 1e4), qkv)


def test_rope_vs_complex_rotation_fp64():
    """z_i = q_i + i q_{i+32} turns by exp(i theta_i) with theta = [h f_0..h f_15, w f_0..w f_15],
    f_j = base^(-j/16): catches interleaved angle layouts, a sign error or wrong frequencies."""
    D, H, gw, n = 128, 2, 7, 21
    qkv = _qkv_rows(n, D, 8)
    got = oracle.rope_qk(qkv, gw, D, H, 1e4, prec="f64")
    f = 1e4 ** (-np.arange(16) / 16.0)
    for r in range(n):
        h, w = divmod(r, gw)
        theta = np.concatenate([h * f, w * f])
        for part in (0, 1):
            for head in range(H):
                v = qkv[r, part * D + head * 64: part * D + head * 64 + 64].astype(np.float64)
                z = (v[:32] + 1j * v[32:]) * np.exp(1j * theta)
                want = np.concatenate([z.real, z.imag])
                g = got[r, part * D + head * 64: part * D + head * 64 + 64]
                assert np.abs(g - want).max() <= 2 ** -8 * np.abs(want).max() + 1e-12
        assert np.array_equal(got[r, 2 * D:], qkv[r, 2 * D:])          # v untouched


def test_rope_axis_blocks():
    """A row shift changes only the height block {0..15, 32..47}; a column shift only the
    width block {16..31, 48..63} (separates blocked from interleaved layouts)."""
    D, H = 64, 1
    q = _qkv_rows(1, D, 9)
    gw = 10
    rows = np.repeat(q, 3 * gw, axis=0)          # same vector at every position of a 3 x 10 grid
    out = oracle.rope_qk(rows, gw, D, H, 1e4)
    hblock = np.r_[0:16, 32:48]
    wblock = np.r_[16:32, 48:64]
    a, b, c = out[0 * gw + 2], out[1 * gw + 2], out[0 * gw + 5]   # (0,2), (1,2), (0,5)
    for part in (0, 1):
        o = part * D
        assert np.array_equal(a[o + wblock], b[o + wblock]) and not np.array_equal(a[o + hblock], b[o + hblock])
        assert np.array_equal(a[o + hblock], c[o + hblock]) and not np.array_equal(a[o + wblock], c[o + wblock])


def test_rope_relative_position_invariance():
    """With the same q and k vector at every patch, the score between (h,w) and (h',w')
    depends only on (h-h', w-w'): shifting both positions leaves it unchanged."""
    D, H, gh, gw = 64, 1, 9, 11
    rng = np.random.default_rng(10)
    qk = rng.standard_normal(2 * D)
    rows = np.zeros((gh * gw, 3 * D))
    rows[:, :2 * D] = qk
    out = oracle.rope_qk(rows, gw, D, H, 1e4, prec="f64")

    def score(p, q):
        return out[p[0] * gw + p[1], :D] @ out[q[0] * gw + q[1], D:2 * D]
    # outputs are bf16-rounded, so the invariance holds to bf16 precision
    tol = 2 * 2 ** -8 * (np.abs(qk[:D]) @ np.abs(qk[D:]))
    for (p, q, s) in [((1, 2), (4, 7), (2, 1)), ((0, 0), (3, 3), (5, 6)), ((8, 10), (2, 4), (-2, -4))]:
        p2 = (p[0] + s[0], p[1] + s[1])
        q2 = (q[0] + s[0], q[1] + s[1])
        assert all(0 <= a < gh and 0 <= b < gw for a, b in (p, q, p2, q2))
        assert abs(score(p, q) - score(p2, q2)) < tol
    # while a change of the relative offset does change the score
    assert abs(score((1, 2), (4, 7)) - score((1, 2), (4, 8))) > tol


def test_rope_angles_blocked():
    c, s = oracle.rope_angle(3, 5, 0, 64, 1e4, "f64")
    assert (c, s) == (math.cos(3.0), math.sin(3.0))
    c, s = oracle.rope_angle(3, 5, 16, 64, 1e4, "f64")
    assert (c, s) == (math.cos(5.0), math.sin(5.0))
    c, s = oracle.rope_angle(3, 5, 17, 64, 1e4, "f64")
    assert abs(c - math.cos(5 * 1e4 ** (-1 / 16))) < 1e-15


# ------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------
def test_softmax_rows_sum_to_one():
    import torch
    qkv = _qkv_rows(50, 64, 11) * 4
    for i in (0, 17, 49):
        p = oracle.softmax_row(qkv, 64, 4, 2, i)
        assert abs(p.sum() - 1) < 1e-5 and (p >= 0).all()
        # and it is the softmax of the scaled scores (head 2 = columns 32..47, scale 1/4)
        q = torch.from_numpy(qkv[i, 32:48].astype(np.float64))
        k = torch.from_numpy(qkv[:, 64 + 32:64 + 48].astype(np.float64))
        want = torch.softmax(k @ q / 4.0, 0).numpy()
        np.testing.assert_allclose(p, want, rtol=1e-4, atol=1e-7)


def test_attention_vs_torch_sdpa_fp64():
    """Catches a missing scale, a transposed score matrix or mixing heads."""
    import torch
    n, D, H = 37, 64, 4
    qkv = _qkv_rows(n, D, 12) * 2
    got = oracle.attention(qkv, D, H, prec="f64")
    t = torch.from_numpy(qkv.astype(np.float64)).reshape(n, 3, H, D // H).permute(1, 2, 0, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2])
    want = ref.permute(1, 0, 2).reshape(n, D).numpy()
    assert np.abs(got - want).max() <= 2 ** -8 * np.abs(want).max()
    got32 = oracle.attention(qkv, D, H, workers=4)
    assert np.abs(got32 - want).max() <= 2 ** -7 * np.abs(want).max()


def test_attention_special_cases():
    n, D, H = 30, 64, 4
    qkv = _qkv_rows(n, D, 13)
    v = qkv[:, 2 * D:]
    # constant V -> constant output
    c = qkv.copy()
    c[:, 2 * D:] = v[0]
    assert np.array_equal(oracle.attention(c, D, H), np.repeat(v[:1], n, 0))
    # Q = 0 -> mean of V over the image
    z = qkv.copy()
    z[:, :D] = 0
    want = bf16_torch(v.astype(np.float64).mean(0))
    got = oracle.attention(z, D, H, prec="f64")
    assert np.abs(got - want).max() <= 2 ** -8 * np.abs(want).max()
    # one patch -> output equals V exactly
    assert np.array_equal(oracle.attention(qkv[:1], D, H), qkv[:1, 2 * D:])
    # permuting keys with their values leaves every output unchanged (no position leak)
    perm = np.random.default_rng(14).permutation(n)
    kp = qkv.copy()
    kp[:, D:] = qkv[perm, D:]
    a = oracle.attention(qkv, D, H, prec="f64")
    b = oracle.attention(kp, D, H, prec="f64")
    assert np.abs(a - b).max() <= 2 ** -8 * np.abs(a).max()


# ------------------------------------------------------------------------------------------
# 3x3 merge
# ------------------------------------------------------------------------------------------
def _tagged(gh, gw, D):
    """y[n][c] = n * D + c + 1: every (patch, channel) gets a distinct positive value."""
    return (np.arange(gh * gw * D, dtype=np.float64) + 1).reshape(gh * gw, D)


def test_merge_is_a_permutation():
    gh, gw, D = 6, 9, 5
    y = _tagged(gh, gw, D)
    A = oracle.merge(y, gh, gw, prec="f64")
    assert A.shape == (6, 45)
    assert np.array_equal(np.sort(A.reshape(-1)), np.sort(y.reshape(-1)))


def test_merge_matches_torch_unfold_with_padding():
    """Right/bottom zero padding on the 2D grid plus the channel-major unfold, against
    torch.nn.functional.unfold; a 5x7 grid exercises both padded edges."""
    import torch
    for gh, gw in [(5, 7), (6, 6), (1, 1), (4, 3)]:
        D = 4
        y = _tagged(gh, gw, D)
        A = oracle.merge(y, gh, gw, prec="f64")
        img = torch.from_numpy(y).reshape(gh, gw, D).permute(2, 0, 1)[None]
        img = torch.nn.functional.pad(img, (0, (-gw) % 3, 0, (-gh) % 3))
        want = torch.nn.functional.unfold(img, 3, stride=3)[0].T.numpy()
        assert np.array_equal(A, want)
        zeros = (A == 0).sum()
        mh, mw = -(-gh // 3), -(-gw // 3)
        assert zeros == (mh * mw * 9 - gh * gw) * D


# ------------------------------------------------------------------------------------------
# layout and overlay
# ------------------------------------------------------------------------------------------
def test_layout_closed_form():
    types, src = oracle.layout([(96, 96)])
    assert len(types) == 2 + 32 * 33 == 1058
    assert types[0] == oracle.TOK_START and types[-1] == oracle.TOK_END
    for r in range(32):
        for c in range(32):
            pos = 1 + r * 33 + c
            assert types[pos] == oracle.TOK_IMAGE and src[pos] == r * 32 + c
        assert types[1 + r * 33 + 32] == oracle.TOK_NEWLINE
    assert (src[types == oracle.TOK_IMAGE] == np.arange(1024)).all()  # identity order
    types, src = oracle.layout([(6, 6), (5, 7)])
    assert len(types) == (2 + 2 * 3) + (2 + 2 * 4)
    assert list(src[types == oracle.TOK_IMAGE]) == list(range(4 + 6))


def test_overlay_rows():
    emb = np.arange(40, dtype=np.uint16).reshape(10, 4)
    rows = np.array([[1.0, 2.0, 3.0, 1.00390625], [-1.0, 0.5, 0.0, 7.0]], np.float32)
    out = oracle.overlay(emb, [7, -1], rows)
    assert np.array_equal(out[[0, 1, 2, 3, 4, 5, 6, 8, 9]], emb[[0, 1, 2, 3, 4, 5, 6, 8, 9]])
    want = bf16_torch(rows[0])
    assert np.array_equal(oracle.bf16_to_float(out[7]), want)


def _sentinels(hidden):
    return synth.make_sentinels(hidden)


def test_assemble_span_sequence():
    """A 6x9 patch grid merges to 2x3 tokens: its span is S I0 I1 I2 N I3 I4 I5 N E (10
    positions), placed here at prompt position 3 of a 16-row prompt; text rows stay as
    they were."""
    hidden = 8
    sent = _sentinels(hidden)
    rows = (np.arange(6 * hidden, dtype=np.float32).reshape(6, hidden) + 0.25) * 1.5
    emb = (np.arange(16 * hidden) % 65000).astype(np.uint16).reshape(16, hidden)
    out = oracle.assemble(emb, 0, 16, [(6, 9)], [3], rows, sent)
    seq = ["S", 0, 1, 2, "N", 3, 4, 5, "N", "E"]
    for k, tok in enumerate(seq):
        got = out[3 + k]
        if tok == "S":
            assert np.array_equal(got, sent[0])
        elif tok == "N":
            assert np.array_equal(got, sent[1])
        elif tok == "E":
            assert np.array_equal(got, sent[2])
        else:
            assert np.array_equal(oracle.bf16_to_float(got), bf16_torch(rows[tok]))
    keep = [0, 1, 2, 13, 14, 15]
    assert np.array_equal(out[keep], emb[keep])


def test_assemble_chunks_agree_with_one_pass():
    """Chunked prefill: assembling the prompt in chunks of any size (a span crossing chunk
    boundaries, a chunk inside one span, empty chunks) equals assembling it at once."""
    hidden = 6
    sent = _sentinels(hidden)
    grids = [(6, 6), (5, 7), (3, 3)]
    starts = [2, 16, 33]             # spans of 8, 10 and 4 positions, text in between
    R = 40
    n_vis = 4 + 6 + 1
    rows = synth.normal_f32(7, 0, n_vis * hidden, 0.0, 1.0).reshape(n_vis, hidden)
    emb = synth.normal_bf16(7, 1, R * hidden).reshape(R, hidden)
    whole = oracle.assemble(emb, 0, R, grids, starts, rows, sent)
    for cuts in ([0, 5, 11, 20, 21, 40], [0, 17, 17, 40], [0, 40], list(range(0, 41, 3)) + [40]):
        parts = [oracle.assemble(emb[a:b], a, b, grids, starts, rows, sent)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        assert np.array_equal(np.concatenate(parts), whole)


def test_assemble_image_rows_match_overlay():
    """The IMAGE positions of an assembled prompt are the overlay of the visual rows onto
    those positions; the START/NEWLINE/END positions are the only other rows changed."""
    hidden = 4
    sent = _sentinels(hidden)
    grids = [(7, 4), (3, 9)]
    starts = [1, 20]
    R = 36
    rows = synth.normal_f32(8, 0, (6 + 3) * hidden).reshape(9, hidden)
    emb = synth.normal_bf16(8, 1, R * hidden).reshape(R, hidden)
    got = oracle.assemble(emb, 0, R, grids, starts, rows, sent)
    place = []
    for (gh, gw), s0 in zip(grids, starts):
        types, src = oracle.layout([(gh, gw)])
        place += [s0 + k for k in np.nonzero(types == oracle.TOK_IMAGE)[0]]
    ov = oracle.overlay(emb, place, rows)
    img = np.array(place)
    assert np.array_equal(got[img], ov[img])
    changed = np.nonzero((got != emb).any(axis=1))[0]
    spans = set()
    for (gh, gw), s0 in zip(grids, starts):
        spans |= set(range(s0, s0 + 2 + -(-gh // 3) * (-(-gw // 3) + 1)))
    assert set(changed) <= spans


# ------------------------------------------------------------------------------------------
# whole encoder
# ------------------------------------------------------------------------------------------
def test_encoder_fp32_vs_fp64_twin():
    """Same rounding points, different arithmetic precision: the gap bounds the fp32
    oracle's own error on the tiny workload."""
    wl = synth.workload("tiny")
    blob = synth.make_weights(wl.cfg, perturbed=True)
    px = synth.make_pixels(wl.cfg, wl.grids)
    a = oracle.encode(wl.cfg, blob, px, wl.grids)
    b = oracle.encode(wl.cfg, blob, px, wl.grids, prec="f64")
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel < 1e-2, rel


def test_uniform_image_gives_identical_rows():
    """A flat RGB-127 image gives identical patches; identical rows stay identical through
    attention (every row attends to the same values), RoPE acts per position, so rows may
    differ after RoPE only through positions -- hence check the patch-embed output and that
    a 1x1 grid (no positional variety) equals a direct computation."""
    cfg = synth.TINY
    gh, gw = 3, 3
    img = np.full((14 * gh, 14 * gw, 3), 127, np.uint8).reshape(-1)
    d = {}
    blob = synth.make_weights(cfg)
    W = oracle.Weights(cfg, blob)
    out = oracle.encode_image(cfg, W, img, gh, gw, dumps=d)
    assert (d["patches"] == d["patches"][0]).all()
    assert (d["embed"] == d["embed"][0]).all()
    assert out.shape == (1, cfg.out_hidden)


def test_packed_batch_is_per_image():
    """A packed batch is the concatenation of per-image results (attention never crosses
    images), so image order only permutes rows."""
    cfg = synth.TINY
    grids = [(6, 6), (3, 9)]
    blob = synth.make_weights(cfg)
    px = synth.make_pixels(cfg, grids)
    out = oracle.encode(cfg, blob, px, grids)
    n0 = 14 * 6 * 14 * 6 * 3
    px_rev = np.concatenate([px[n0:], px[:n0]])
    out_rev = oracle.encode(cfg, blob, px_rev, grids[::-1])
    assert np.array_equal(out, np.concatenate([out_rev[3:], out_rev[:3]]))


# ------------------------------------------------------------------------------------------
# official-layer variant: RMSNorm, SiLU / SwiGLU, erf GELU, two-linear aligner
# ------------------------------------------------------------------------------------------
def test_gelu_erf_vs_torch_and_closed_form():
    """Exact GELU: torch's erf form to fp64 rounding; u Phi(u) at u = +-1 from the standard
    normal table (Phi(1) = 0.8413447460685429); the odd identity gelu(u) - gelu(-u) = u; and
    the tanh form stays within the ~1e-3 the first page reports for the two forms."""
    import torch
    u = np.linspace(-8, 8, 2001)
    got = np.array([oracle.gelu_erf(v, "f64") for v in u])
    want = torch.nn.functional.gelu(torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)
    got32 = np.array([oracle.gelu_erf(v) for v in u])
    np.testing.assert_allclose(got32, want, rtol=0, atol=2e-6)
    assert abs(oracle.gelu_erf(1.0, "f64") - 0.8413447460685429) < 1e-15
    assert abs(oracle.gelu_erf(-1.0, "f64") + 0.15865525393145707) < 1e-15
    np.testing.assert_allclose(got - got[::-1], u, atol=1e-12)
    tanh = np.array([oracle.gelu_tanh(v, "f64") for v in u])
    assert 1e-4 < np.abs(got - tanh).max() < 1e-3


def test_silu_closed_forms():
    """silu(u) = u sigmoid(u): sigmoid(ln 3) = 3/4 gives silu(+-ln 3) = 0.75 ln 3 and
    -0.25 ln 3; silu(0) = 0; torch's silu to fp64 rounding on a sweep."""
    import torch
    l3 = math.log(3.0)
    assert abs(oracle.silu(l3, "f64") - 0.75 * l3) < 1e-15
    assert abs(oracle.silu(-l3, "f64") + 0.25 * l3) < 1e-15
    assert oracle.silu(0.0, "f64") == 0.0
    u = np.linspace(-30, 30, 1201)
    got = np.array([oracle.silu(v, "f64") for v in u])
    want = torch.nn.functional.silu(torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=1e-300)


def test_swiglu_gate_and_up_roles():
    """h = bf16(silu(g) u): the activation acts on the gate operand only.  With u = 1 the
    result is bf16(silu(g)); with g = 0 it is 0 whatever u is; torch's silu product rounded
    once to bf16 elsewhere."""
    import torch
    rng = np.random.default_rng(21)
    g = rng.standard_normal(4096) * 3
    u = rng.standard_normal(4096) * 2
    got = oracle.swiglu(g, u, "f64")
    want = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).to(torch.bfloat16)
    assert np.array_equal(got, want.to(torch.float64).numpy())
    ones = oracle.swiglu(g, np.ones_like(g), "f64")
    assert np.array_equal(ones, torch.nn.functional.silu(torch.from_numpy(g)).to(torch.bfloat16)
                          .to(torch.float64).numpy())
    assert not np.array_equal(ones, oracle.swiglu(np.ones_like(g), g, "f64"))
    assert (oracle.swiglu(np.zeros_like(g), u, "f64") == 0).all()


@pytest.mark.parametrize("prec", ["f32", "f64"])
def test_rmsnorm_vs_torch(prec):
    """torch's rms_norm (mean square over the row, eps inside the square root, weight only),
    with a row whose mean square is far below eps so that eps placement shows."""
    import torch
    rng = np.random.default_rng(22)
    x = rng.standard_normal((10, 64)) * 3 + 1
    x[3] = 1e-4 * rng.standard_normal(64)
    g = 1 + 0.1 * rng.standard_normal(64)
    dt = np.float32 if prec == "f32" else np.float64
    x, g = (v.astype(dt).astype(np.float64) for v in (x, g))
    got = oracle.rmsnorm(x, g, 1e-6, prec)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    atol = 1e-6 if prec == "f32" else 1e-9
    assert np.all(np.abs(got - want) <= 2 ** -8 * np.abs(want) + atol)


def test_rmsnorm_closed_forms():
    """A constant row c gives c / sqrt(c^2 + eps) g (no mean is subtracted: a LayerNorm would
    give its beta); x = (3, 4) gives x / sqrt(12.5 + eps); rows made of (v, -v) pairs have a
    mean of exactly 0 in any summation order, where RMSNorm equals LayerNorm with beta = 0
    bit for bit."""
    g = np.linspace(0.5, 1.5, 64)
    x = np.full((1, 64), -2.5)
    want = oracle.round_bf16(-2.5 / math.sqrt(6.25 + 1e-6) * g, "f64")
    assert np.array_equal(oracle.rmsnorm(x, g, 1e-6, "f64"), want[None, :])
    got = oracle.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.5, "f64")
    assert np.array_equal(got[0], oracle.round_bf16(np.array([3.0, 4.0]) / math.sqrt(13.0), "f64"))
    rng = np.random.default_rng(23)
    v = bf16_torch(rng.standard_normal((5, 32)))
    xz = np.stack([v, -v], axis=2).reshape(5, 64)
    gz = 1 + 0.1 * rng.standard_normal(64)
    for prec in ("f32", "f64"):
        assert np.array_equal(oracle.rmsnorm(xz, gz, 1e-6, prec),
                              oracle.layernorm(xz, gz, np.zeros(64), 1e-6, prec))


def test_linear_gelu_erf_unrounded_and_rounded():
    """act = 2 is the erf GELU of the biased product: unrounded it matches torch's gelu of
    A W^T + b to fp64 rounding; rounded, every element is that value rounded once to bf16."""
    import torch
    rng = np.random.default_rng(24)
    A = rng.standard_normal((6, 8))
    W = rng.standard_normal((5, 8))
    b = rng.standard_normal(5)
    pre = torch.from_numpy(A @ W.T + b)
    want = torch.nn.functional.gelu(pre).numpy()
    got = oracle.linear(A, W, b, act=2, round_out=False, prec="f64")
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    got_r = oracle.linear(A, W, b, act=2, prec="f64")
    assert np.array_equal(got_r, oracle.round_bf16(got, "f64"))


def _variant_weights(cfg, **over):
    """Weights of `cfg` by name as fp64 arrays, with some tensors replaced."""
    blob = synth.make_weights(cfg, perturbed=True)
    W = oracle.Weights(cfg, blob, "f64")
    for k, v in over.items():
        W.t[k] = np.asarray(v, np.float64)
        W.tt[k] = np.ascontiguousarray(np.asarray(v, np.float64).T)
    return W


def test_swiglu_mlp_special_case():
    """With up = 0 weights and bias 1, and down = identity with bias 0 (F = D), the SwiGLU MLP
    reduces to bf16(silu(x W_gate^T + b_gate)): torch's silu on the gate projection, rounded
    once.  Swapping gate and up, or applying the activation after the product, breaks it."""
    import torch
    from dataclasses import replace
    cfg = replace(synth.TINY_OFFICIAL, mlp=64, layers=1)
    D = cfg.hidden
    W = _variant_weights(cfg, **{"l0.up.w": np.zeros((D, D)), "l0.up.b": np.ones(D),
                                 "l0.down.w": np.eye(D), "l0.down.b": np.zeros(D)})
    rng = np.random.default_rng(25)
    x = bf16_torch(rng.standard_normal((7, D)))
    got = oracle.mlp(cfg, x, W, 0, prec="f64")
    pre = torch.from_numpy(x @ W["l0.gate.w"].T + W["l0.gate.b"])
    want = torch.nn.functional.silu(pre).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)


def test_two_linear_aligner_special_case():
    """With the second projection 2 I (inner width = out width) and bias 0, the aligner gives
    2 bf16(gelu_erf(A W_1^T + b_1)) exactly: the GELU sits between the two projections and the
    first is rounded after it."""
    import torch
    from dataclasses import replace
    cfg = replace(synth.TINY_OFFICIAL, aligner_hidden=synth.TINY_OFFICIAL.out_hidden, layers=1)
    Dl = cfg.out_hidden
    W = _variant_weights(cfg, **{"proj2.w": 2 * np.eye(Dl), "proj2.b": np.zeros(Dl)})
    rng = np.random.default_rng(26)
    A = bf16_torch(rng.standard_normal((5, 9 * cfg.hidden)))
    got = oracle.aligner(cfg, A, W, prec="f64")
    pre = torch.from_numpy(A @ W["proj.w"].T + W["proj.b"])
    want = 2 * torch.nn.functional.gelu(pre).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.abs(got - want).max() == 0


def test_official_variant_blob_and_twin():
    """The variant's tensor list (no beta for RMSNorm, gate/up/down, two projections) and its
    encoder's fp32 oracle against the fp64 twin on the tiny workload."""
    cfg = synth.TINY_OFFICIAL
    names = [n for n, _ in cfg.tensor_shapes()]
    assert not any(n.endswith(".b") and (".ln" in n or n.startswith("lnf")) for n in names)
    assert {"l0.gate.w", "l0.up.w", "l0.down.w", "proj2.w"} <= set(names)
    D, F, Da, Dl = cfg.hidden, cfg.mlp, cfg.aligner_hidden, cfg.out_hidden
    per_layer = D + 3 * D * D + 3 * D + D * D + D + D + 3 * F * D + 2 * F + D
    assert cfg.blob_elems() == (D * cfg.patch_dim + D + cfg.layers * per_layer + D
                                + Da * 9 * D + Da + Dl * Da + Dl)
    grids = [(6, 6), (4, 5)]
    blob = synth.make_weights(cfg, perturbed=True)
    px = synth.make_pixels(cfg, grids)
    a = oracle.encode(cfg, blob, px, grids)
    b = oracle.encode(cfg, blob, px, grids, prec="f64")
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel < 1e-2, rel


def test_official_variant_final_norm_is_rms():
    """At the final-norm boundary the variant's rows are RMSNorm outputs of the last block:
    with gamma = 1 each row's mean square is 1 up to bf16 rounding, while its mean is not 0."""
    from dataclasses import replace
    cfg = replace(synth.TINY_OFFICIAL, layers=1)
    blob = synth.make_weights(cfg)
    W = oracle.Weights(cfg, blob, "f64")
    gh, gw = 6, 6
    px = synth.make_pixels(cfg, [(gh, gw)])
    d = {}
    oracle.encode_image(cfg, W, px, gh, gw, prec="f64", dumps=d)
    y = d["final_norm"]
    np.testing.assert_allclose((y * y).mean(1), 1.0, atol=1e-2)
    assert np.array_equal(y, oracle.rmsnorm(d["layer0"], np.ones(cfg.hidden), cfg.ln_eps, "f64"))
    assert np.abs(y.mean(1)).max() > 1e-3
