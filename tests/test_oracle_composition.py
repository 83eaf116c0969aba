"""Pins of the oracle's composition: where each norm sits, where the residual stream is rounded,
which columns feed attention, that RoPE takes each patch's (row, column) on the grid, the final
norm, the merge and the aligner -- and the pixel map's mean/std roles.

The per-step functions are pinned one by one in ``test_oracle_pins.py``.  Here the whole
encoder is checked against
  * closed forms of special weights and images, where a block reduces to something written out
    by hand ([Z] "DeepSeek V4.1 Flash Engineering, Part 3: Integrating Vision", "Step 2"
    boundary table: block 0's output isolates the patch projection, the QKV bias, attention
    and the residual order), and
  * an independent fp64 composition of library routines (torch's layer_norm / rms_norm,
    linear, a complex-number rotation, scaled_dot_product_attention, gelu / silu, unfold) on
    tiny grids, brute force that shares no arithmetic with the oracle: its own bf16 rounding
    (round-to-odd to fp32, then torch's fp32 -> bf16), its own patch extraction.
Every rounding point R1..R13 of the method appears in both, so the fp64 oracle must agree with
the brute force bit for bit on every bf16 tensor and to fp64 rounding on the fp32 output.
"""
import math
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth


# ------------------------------------------------------------------------------------------
# brute-force helpers (no oracle code)
# ------------------------------------------------------------------------------------------
def bf16(x):
    """fp64 -> bf16 value (as fp64), nearest even, computed as round-to-odd into fp32 followed
    by torch's fp32 -> bf16 rounding (round-to-odd into a format with >= 2 extra bits makes the
    second rounding correct)."""
    import torch
    x = np.asarray(x, np.float64)
    f = x.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(x)
    f = np.where(over, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    inexact = (f.astype(np.float64) != x).astype(np.uint32)
    f = (f.view(np.uint32) | inexact).view(np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()


def patches_bruteforce(img, gh, gw, cfg):
    """[Z] "Step 1" items 5-6: one row per patch in (grid_y, grid_x) order, (c, y, x) inside
    the row; v = u8 * s_c + t_c with s_c = 1/(255 std_c), t_c = -mean_c/std_c (fp32 constants)
    evaluated exactly in double and rounded once to fp32 (that is the fma), then to bf16."""
    ps = cfg.patch
    img = np.asarray(img, np.uint8).reshape(ps * gh, ps * gw, 3)
    blocks = img.reshape(gh, ps, gw, ps, 3).transpose(0, 2, 4, 1, 3).reshape(gh * gw, 3 * ps * ps)
    mean = np.float32(cfg.pix_mean).astype(np.float64)
    std = np.float32(cfg.pix_std).astype(np.float64)
    s = (1.0 / (255.0 * std)).astype(np.float32).astype(np.float64)
    t = (-mean / std).astype(np.float32).astype(np.float64)
    chan = np.repeat(np.arange(3), ps * ps)
    v = (blocks.astype(np.float64) * s[chan] + t[chan]).astype(np.float32)
    return bf16(v)


def rope_bruteforce(x, gh, gw, H, base):
    """Rotate each head's pairs (i, i + hd/2) as the complex number x_i + i x_{i+hd/2} times
    e^{i theta_i}; theta_i = row * f_i for i < hd/4, col * f_{i - hd/4} after, f_j =
    base^(-2j/(hd/2)); cos and sin in fp64, rounded to fp32 ([Z] "Step 3"; patch n sits at
    (n // gw, n % gw))."""
    import torch
    n, D = x.shape
    hd = D // H
    half, quarter = hd // 2, hd // 4
    f = base ** (-2.0 * np.arange(quarter) / half)
    row, col = np.divmod(np.arange(n), gw)
    theta = np.concatenate([row[:, None] * f[None], col[:, None] * f[None]], axis=1)   # [n][half]
    c = np.cos(theta).astype(np.float32).astype(np.float64)
    s = np.sin(theta).astype(np.float32).astype(np.float64)
    rot = torch.complex(torch.from_numpy(c), torch.from_numpy(s))
    xh = torch.from_numpy(x.reshape(n, H, hd))
    z = torch.complex(xh[..., :half], xh[..., half:]) * rot[:, None, :]
    out = torch.cat([z.real, z.imag], dim=-1)
    return out.reshape(n, D).numpy()


def encode_bruteforce(cfg, W, img, gh, gw):
    """The whole encoder on one image, from torch library routines in fp64, bf16 after every
    step the method rounds.  Returns (layer outputs, final norm, merged rows, aligner out)."""
    import torch
    import torch.nn.functional as F
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    D, H = cfg.hidden, cfg.heads
    hd = D // H
    rms = cfg.norm_kind == 1

    def norm(x, name):
        if rms:
            return F.rms_norm(T(x), (D,), T(W[name + ".g"]), cfg.ln_eps).numpy()
        return F.layer_norm(T(x), (D,), T(W[name + ".g"]), T(W[name + ".b"]), cfg.ln_eps).numpy()

    def lin(x, name, act=None):
        y = F.linear(T(x), T(W[name + ".w"]), T(W[name + ".b"]))
        if act == "gelu":
            y = F.gelu(y, approximate="none" if cfg.gelu_kind == 1 else "tanh")
        return y.numpy()

    x = bf16(lin(patches_bruteforce(img, gh, gw, cfg), "pe"))
    layers = []
    for l in range(cfg.layers):
        h = bf16(norm(x, f"l{l}.ln1"))
        qkv = bf16(lin(h, f"l{l}.qkv"))
        q = bf16(rope_bruteforce(qkv[:, :D], gh, gw, H, cfg.rope_base))
        k = bf16(rope_bruteforce(qkv[:, D:2 * D], gh, gw, H, cfg.rope_base))
        v = qkv[:, 2 * D:]
        heads = lambda a: T(a).reshape(-1, H, hd).transpose(0, 1).contiguous()
        o = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), scale=1.0 / math.sqrt(hd))
        o = bf16(o.transpose(0, 1).reshape(-1, D).numpy())
        x = bf16(x + bf16(lin(o, f"l{l}.o")))
        h2 = bf16(norm(x, f"l{l}.ln2"))
        if cfg.mlp_kind == 1:
            g, u = lin(h2, f"l{l}.gate"), lin(h2, f"l{l}.up")
            m = bf16(lin(bf16(F.silu(T(g)).numpy() * u), f"l{l}.down"))
        else:
            m = bf16(lin(bf16(lin(h2, f"l{l}.fc1", act="gelu")), f"l{l}.fc2"))
        x = bf16(x + m)
        layers.append(x)
    y = bf16(norm(x, "lnf"))
    mh, mw = -(-gh // cfg.merge), -(-gw // cfg.merge)
    grid = torch.zeros(1, D, mh * cfg.merge, mw * cfg.merge, dtype=torch.float64)
    grid[0, :, :gh, :gw] = T(y).T.reshape(D, gh, gw)
    A = F.unfold(grid, cfg.merge, stride=cfg.merge)[0].T.numpy()      # [mh*mw][D*9], c*9 + k
    if cfg.aligner_hidden > 0:
        out = lin(bf16(lin(A, "proj", act="gelu")), "proj2")
    else:
        out = lin(A, "proj")
    return layers, y, A, out


def weights64(cfg, perturbed=True, **over):
    W = oracle.Weights(cfg, synth.make_weights(cfg, perturbed=perturbed), "f64")
    for k, v in over.items():
        W.t[k] = np.asarray(v, np.float64)
        W.tt[k] = np.ascontiguousarray(np.asarray(v, np.float64).T)
    return W


def run_oracle(cfg, W, img, gh, gw):
    d = {}
    out = oracle.encode_image(cfg, W, img, gh, gw, prec="f64", dumps=d)
    return d, out


TINY3 = replace(synth.TINY, layers=3)
CASES = [(TINY3, (4, 5)), (TINY3, (5, 7)), (replace(synth.TINY_OFFICIAL, layers=2), (4, 7)),
         (replace(synth.TINY, layers=2, gelu_kind=1, aligner_hidden=64), (3, 2))]


@pytest.mark.parametrize("cfg,grid", CASES, ids=["ln_4x5", "ln_5x7_padded", "official_4x7",
                                                 "erf_two_linear_3x2"])
def test_encoder_equals_bruteforce_composition(cfg, grid):
    """Catches a norm in the wrong place (post-norm, a missing LN1 / LN2 / final norm), a
    residual stream kept unrounded, RoPE skipped or fed the wrong grid side, q/k/v blocks
    exchanged, a transposed merge, and an aligner GELU in the wrong place: every layer's
    residual stream, the final norm and the merged rows are compared bit for bit, the fp32
    aligner output to fp64 rounding."""
    gh, gw = grid
    W = weights64(cfg)
    img = synth.make_pixels(cfg, [grid], seed=0x5EED00F0)
    d, out = run_oracle(cfg, W, img, gh, gw)
    layers, y, A, want = encode_bruteforce(cfg, W, img, gh, gw)
    assert np.array_equal(d["patches"], patches_bruteforce(img, gh, gw, cfg))
    for l, xl in enumerate(layers):
        assert np.array_equal(d[f"layer{l}"], xl), f"residual stream after layer {l}"
    assert np.array_equal(d["final_norm"], y)
    assert np.array_equal(d["merged"], A)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


def test_zero_output_projections_keep_the_patch_embedding():
    """With W_o = b_o = W_2 = b_2 = 0 every sublayer adds exact zeros, so the residual stream
    after every layer is the patch projection x0 bit for bit, and the output is the aligner
    applied to merge(final_norm(x0)).  Catches a block that replaces x instead of adding to it,
    and a final norm applied to anything but the last residual stream."""
    import torch
    import torch.nn.functional as F
    cfg = TINY3
    D, F_ = cfg.hidden, cfg.mlp
    zeros = {}
    for l in range(cfg.layers):
        zeros.update({f"l{l}.o.w": np.zeros((D, D)), f"l{l}.o.b": np.zeros(D),
                      f"l{l}.fc2.w": np.zeros((D, F_)), f"l{l}.fc2.b": np.zeros(D)})
    W = weights64(cfg, **zeros)
    gh, gw = 6, 6
    img = synth.make_pixels(cfg, [(gh, gw)], seed=0x5EED00F1)
    d, out = run_oracle(cfg, W, img, gh, gw)
    x0 = d["embed"]
    for l in range(cfg.layers):
        assert np.array_equal(d[f"layer{l}"], x0)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    y = bf16(F.layer_norm(T(x0), (D,), T(W["lnf.g"]), T(W["lnf.b"]), cfg.ln_eps).numpy())
    assert np.array_equal(d["final_norm"], y)
    g = T(y).T.reshape(1, D, gh, gw)
    A = F.unfold(g, 3, stride=3)[0].T
    want = F.linear(A, T(W["proj.w"]), T(W["proj.b"])).numpy()
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


def test_constant_values_block_closed_form():
    """W_qkv = 0 with a value bias b_v: every v row is b_v, so attention returns b_v exactly
    whatever the scores (softmax weights sum to one), and block 0 is written out by hand:
        x' = bf16(x0 + bf16(b_v W_o^T + b_o)),
        x1 = bf16(x' + bf16(bf16(gelu(bf16(LN2(x'))) W_1^T + b_1)) W_2^T + b_2)).
    Catches a residual stream not rounded at the two adds, LN2 missing or moved, and the v
    block read from the q or k columns."""
    import torch
    import torch.nn.functional as F
    cfg = replace(synth.TINY, layers=1)
    D = cfg.hidden
    rng = np.random.default_rng(77)
    bqkv = bf16(rng.standard_normal(3 * D) * 0.5)
    W = weights64(cfg, **{"l0.qkv.w": np.zeros((3 * D, D)), "l0.qkv.b": bqkv})
    gh, gw = 6, 6
    img = synth.make_pixels(cfg, [(gh, gw)], seed=0x5EED00F2)
    d, _ = run_oracle(cfg, W, img, gh, gw)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    bv = bqkv[2 * D:]
    assert np.array_equal(d["attn0"], np.broadcast_to(bv, (gh * gw, D)))
    a = bf16(F.linear(T(bv), T(W["l0.o.w"]), T(W["l0.o.b"])).numpy())
    xp = bf16(d["embed"] + a[None, :])
    h = bf16(F.layer_norm(T(xp), (D,), T(W["l0.ln2.g"]), T(W["l0.ln2.b"]), cfg.ln_eps).numpy())
    u = bf16(F.gelu(F.linear(T(h), T(W["l0.fc1.w"]), T(W["l0.fc1.b"])), approximate="tanh").numpy())
    f = bf16(F.linear(T(u), T(W["l0.fc2.w"]), T(W["l0.fc2.b"])).numpy())
    assert np.array_equal(d["layer0"], bf16(xp + f))


def test_uniform_image_block_closed_form():
    """A flat image gives identical patches, hence identical rows in every layer: identical v
    rows make attention return v whatever RoPE does to q and k ([Z] "Step 1": images are
    centred on an RGB 127 canvas).  Each layer is then a per-row map written out by hand with
    random weights:
        v = bf16(bf16(LN1(x)) W_v^T + b_v),  x' = bf16(x + bf16(v W_o^T + b_o)),
        x'' = bf16(x' + MLP(bf16(LN2(x')))).
    Catches LN1 missing or moved (W_qkv is random here) and v taken from the wrong block."""
    import torch
    import torch.nn.functional as F
    cfg = TINY3
    D = cfg.hidden
    W = weights64(cfg)
    gh, gw = 3, 6
    img = np.full((14 * gh, 14 * gw, 3), 127, np.uint8).reshape(-1)
    d, out = run_oracle(cfg, W, img, gh, gw)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    LN = lambda x, n: bf16(F.layer_norm(T(x), (D,), T(W[n + ".g"]), T(W[n + ".b"]), cfg.ln_eps).numpy())
    lin = lambda x, w, b: F.linear(T(x), T(w), T(b))
    x = d["embed"][:1]
    assert (d["embed"] == x).all()
    for l in range(cfg.layers):
        qkv_w, qkv_b = W[f"l{l}.qkv.w"], W[f"l{l}.qkv.b"]
        v = bf16(lin(LN(x, f"l{l}.ln1"), qkv_w[2 * D:], qkv_b[2 * D:]).numpy())
        x = bf16(x + bf16(lin(v, W[f"l{l}.o.w"], W[f"l{l}.o.b"]).numpy()))
        u = bf16(F.gelu(lin(LN(x, f"l{l}.ln2"), W[f"l{l}.fc1.w"], W[f"l{l}.fc1.b"]),
                        approximate="tanh").numpy())
        x = bf16(x + bf16(lin(u, W[f"l{l}.fc2.w"], W[f"l{l}.fc2.b"]).numpy()))
        assert np.array_equal(d[f"layer{l}"], np.broadcast_to(x, (gh * gw, D))), f"layer {l}"
    assert (out == out[0]).all()


# ------------------------------------------------------------------------------------------
# pixel map: mean and std roles, by hand-written values
# ------------------------------------------------------------------------------------------
# The CLIP constants (mean 0.48145466, 0.4578275, 0.40821073; std 0.26862954, 0.26130258,
# 0.27577711).  u = 0 maps to -mean_c/std_c and u = 255 to (1 - mean_c)/std_c, worked out by
# hand to 6 digits:
CLIP_AT_0 = (-1.792263, -1.752097, -1.480220)
CLIP_AT_255 = (1.930336, 2.074884, 2.145897)
# Their bf16 values (spacing 2^-7 in [1, 2), 2^-6 in [2, 4)); none lies within 1e-4 of a
# rounding midpoint, so 6 digits decide them:
CLIP_AT_0_BF16 = (-1.7890625, -1.75, -1.4765625)
CLIP_AT_255_BF16 = (1.9296875, 2.078125, 2.140625)


def test_clip_pixel_map_endpoints_by_hand():
    """Catches mean and std exchanged (or std applied before the mean) in the pixel map:
    u = 0 and u = 255 in each channel of the CLIP-normalised tiny workload give the
    hand-written values above (R3: v = (u/255 - mean_c)/std_c)."""
    cfg = synth.TINY
    for c in range(3):
        assert abs(-cfg.pix_mean[c] / cfg.pix_std[c] - CLIP_AT_0[c]) < 1e-6
        assert abs((1 - cfg.pix_mean[c]) / cfg.pix_std[c] - CLIP_AT_255[c]) < 1e-6
        for v, b in ((CLIP_AT_0[c], CLIP_AT_0_BF16[c]), (CLIP_AT_255[c], CLIP_AT_255_BF16[c])):
            step = 2.0 ** (math.floor(math.log2(abs(v))) - 7)
            assert abs(abs(v - b) - step / 2) > 1e-4     # far from a midpoint
            assert abs(v - b) < step / 2
    img = np.zeros((14, 14, 3), np.uint8)
    img[7, :, :] = 255
    P = oracle.patchify(img.reshape(-1), 1, 1, cfg)
    for c in range(3):
        assert P[0, c * 196 + 0] == CLIP_AT_0_BF16[c]
        assert P[0, c * 196 + 7 * 14 + 3] == CLIP_AT_255_BF16[c]
    s, t = oracle.pixel_affine(cfg.pix_mean, cfg.pix_std)
    np.testing.assert_allclose(t, CLIP_AT_0, atol=2e-6)
    np.testing.assert_allclose(255 * s.astype(np.float64) + t, CLIP_AT_255, atol=2e-6)
