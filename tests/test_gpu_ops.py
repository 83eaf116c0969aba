"""Per-step parity of the HIP kernels against the CPU oracle, on seeded inputs that come
from the generator (never from the GPU), at small ragged sizes and at the encoder's real
shapes (sampled rows where the oracle would be too slow for all of them)."""
import numpy as np
import pytest

import multimodal_vision_encoder_amd as vit
import oracle
import synth
from tests.gpu_util import (assert_bf16_close, bf16_bits_of, f16_of, from_dev_bf16,
                            qkv_after_rope, require_gpu, seeded_bf16, to_dev_bf16, rel_l2)

pytestmark = pytest.mark.gpu

_encs = {}


def encoder(name="tiny", perturbed=False):
    """Encoder contexts are cached per (config, weights) for the session."""
    key = (name, perturbed)
    if key not in _encs:
        require_gpu()
        cfg = {"tiny": synth.TINY, "v41_1layer": synth.V41_ONE_LAYER}[name]
        blob = synth.make_weights(cfg, perturbed=perturbed)
        _encs[key] = (vit.Encoder(cfg, blob), cfg, blob)
    return _encs[key]


def f32(bits):
    return synth.bf16_bits_to_f32(bits)


def sum_bound(A, W):
    """Absolute slack for fp32 sums taken in another order: 2^-18 * sum_k |a_k w_k| per
    output (about sqrt(K) ulps of the largest partial sum, far below one bf16 ulp of a
    typical output, but it covers outputs that cancel to near zero)."""
    return 2.0 ** -18 * (np.abs(f32(A)).astype(np.float64) @ np.abs(f32(W)).astype(np.float64).T)


# ------------------------------------------------------------------------------------------
# linear layers (QKV, out-proj, fc1 + GELU, fc2, projector epilogue)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N,act,out_f32", [
    (300, 128, 200, vit.ACT_NONE, False),       # ragged M and N, several tiles
    (1, 64, 5, vit.ACT_NONE, True),             # degenerate single row, tiny N
    (257, 192, 130, vit.ACT_GELU_TANH, False),
    (129, 256, 64, vit.ACT_NONE, True),
])
def test_linear_small(M, K, N, act, out_f32):
    torch = require_gpu()
    enc, _, _ = encoder()
    A = seeded_bf16((M, K), 101, 0)
    W = seeded_bf16((N, K), 101, 1, std=0.05)
    b = seeded_bf16((N,), 101, 2, std=0.1)
    got = enc.op_linear(to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b), act, out_f32)
    torch.cuda.synchronize()
    want = oracle.linear(f32(A), f32(W), f32(b), act=act, round_out=not out_f32)
    if out_f32:
        np.testing.assert_allclose(got.cpu().numpy(), want, rtol=1e-5, atol=1e-5)
    else:
        assert_bf16_close(from_dev_bf16(got), want, atol=sum_bound(A, W), what="linear")


def test_linear_one_hot_is_exact():
    """One-hot weight rows copy input columns: exact, whatever the accumulation order."""
    torch = require_gpu()
    enc, _, _ = encoder()
    M, K, N = 200, 256, 96
    A = seeded_bf16((M, K), 102)
    sel = np.random.default_rng(0).permutation(K)[:N]
    W = np.zeros((N, K), np.uint16)
    W[np.arange(N), sel] = 0x3F80
    got = from_dev_bf16(enc.op_linear(to_dev_bf16(A), to_dev_bf16(W), None))
    torch.cuda.synchronize()
    assert np.array_equal(got, f32(A)[:, sel])


@pytest.mark.parametrize("N,K,act", [(3072, 1024, vit.ACT_NONE), (1024, 1024, vit.ACT_NONE),
                                     (4096, 1024, vit.ACT_GELU_TANH), (1024, 4096, vit.ACT_NONE)],
                         ids=["qkv", "out_proj", "fc1_gelu", "fc2"])
def test_linear_full_size_sampled(N, K, act):
    """The block's GEMMs at the 1024-token image's shape (M = 9216 patches), checked on
    sampled rows including the last tile."""
    torch = require_gpu()
    enc, _, _ = encoder()
    M = 9216
    A = seeded_bf16((M, K), 103, 0)
    W = seeded_bf16((N, K), 103, 1, std=0.02)
    b = seeded_bf16((N,), 103, 2, std=0.02)
    got = from_dev_bf16(enc.op_linear(to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b), act))
    torch.cuda.synchronize()
    # rows in the first tile row, the middle and the last tile rows (8192..9215)
    rows = np.r_[0:3, 127:130, 4000:4003, 8192:8196, 8700:8703, M - 5:M]
    want = oracle.linear(f32(A[rows]), f32(W), f32(b), act=act)
    assert_bf16_close(got[rows], want, atol=sum_bound(A[rows], W), what="linear full size")


@pytest.mark.parametrize("K", [64, 192, 320], ids=["one_ktile", "three_ktiles", "five_ktiles"])
@pytest.mark.parametrize("act", [vit.ACT_NONE, vit.ACT_GELU_TANH], ids=["plain", "gelu"])
@pytest.mark.parametrize("M,N", [(3900, 4056), (4000, 2000)], ids=["tiles256", "tiles192"])
def test_linear_big_tiles_every_row(M, N, K, act):
    """One round of 4-wave tiles of plain activations (64-wide k-tiles, two LDS stages):
    3900 x 4056 runs as 256 x 256 tiles (a ragged last tile row of 60 rows and column of 216),
    4000 x 2000 as 192 x 256 tiles (168 of them; last tile row 160 rows, last column 208).
    K = 64, 192, 320 give 1, 3 and 5 k-tiles (fewer than the two stages, and an odd count that
    ends on the peeled step).  Every output is compared with the oracle; the residual form of
    the same launch is checked bitwise against linear + add."""
    torch = require_gpu()
    enc, _, _ = encoder()
    A = seeded_bf16((M, K), 131, 0)
    W = seeded_bf16((N, K), 131, 1, std=0.05)
    b = seeded_bf16((N,), 131, 2, std=0.1)
    dA, dW, db = to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b)
    got = from_dev_bf16(enc.op_linear(dA, dW, db, act))
    torch.cuda.synchronize()
    want = oracle.linear(f32(A), f32(W), f32(b), act=act, workers=8)
    assert_bf16_close(got, want, atol=sum_bound(A, W), what="256 x 256 tiles, every row")
    if act == vit.ACT_NONE:
        x = seeded_bf16((M, N), 131, 3, std=2.0)
        dx = to_dev_bf16(x)
        enc.op_linear_residual(dA, dW, db, dx)
        torch.cuda.synchronize()
        want_x = oracle.add_round(f32(x), got)
        assert np.array_equal(bf16_bits_of(from_dev_bf16(dx)), bf16_bits_of(want_x)), "residual form differs"


@pytest.mark.parametrize("act,out_f32", [(vit.ACT_GELU_TANH, False), (vit.ACT_NONE, True)])
def test_linear_row_tail(act, out_f32):
    """776 tiles of 256 x 256 on 256 compute units (192-row tiles would need a fifth round): the
    last round's 8 tiles are one whole tile row (rows 24576..24699, ragged), which runs as a
    second launch of 128 x 128 tiles (ragged in M and N); every row of that tail and rows on
    both sides of the seam are checked."""
    torch = require_gpu()
    enc, _, _ = encoder()
    M, K, N = 24700, 1024, 2000
    A = seeded_bf16((M, K), 108, 0)
    W = seeded_bf16((N, K), 108, 1, std=0.02)
    b = seeded_bf16((N,), 108, 2, std=0.02)
    got = enc.op_linear(to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b), act, out_f32)
    torch.cuda.synchronize()
    rows = np.r_[0:2, 12000:12002, 24572:M]
    want = oracle.linear(f32(A[rows]), f32(W), f32(b), act=act, round_out=not out_f32, workers=8)
    if out_f32:
        g = got.cpu().numpy()[rows]
        assert np.all(np.abs(g - want) <= sum_bound(A[rows], W) + 1e-6 * np.abs(want))
    else:
        assert_bf16_close(from_dev_bf16(got)[rows], want, atol=sum_bound(A[rows], W), what="row tail")


@pytest.mark.parametrize("act,out_f32", [(vit.ACT_GELU_TANH, False), (vit.ACT_NONE, True)])
def test_linear_split_k_tail(act, out_f32):
    """K = 4096 with ragged M and N (rows 8192..8399 and columns 1016..1019 in partial tiles).
    Plain activations of this size run as one round of 192 x 256 tiles; the K split of a
    leftover round is reached by the gathered projector source (test_merge_project_split_k_tail)."""
    torch = require_gpu()
    enc, _, _ = encoder()
    M, K, N = 8400, 4096, 1020
    A = seeded_bf16((M, K), 107, 0)
    W = seeded_bf16((N, K), 107, 1, std=0.02)
    b = seeded_bf16((N,), 107, 2, std=0.02)
    got = enc.op_linear(to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b), act, out_f32)
    torch.cuda.synchronize()
    rows = np.r_[0:2, 4000:4002, 8190:8196, 8300:8302, M - 4:M]
    want = oracle.linear(f32(A[rows]), f32(W), f32(b), act=act, round_out=not out_f32)
    if out_f32:
        g = got.cpu().numpy()[rows]
        assert np.all(np.abs(g - want) <= sum_bound(A[rows], W) + 1e-6 * np.abs(want))
    else:
        assert_bf16_close(from_dev_bf16(got)[rows], want, atol=sum_bound(A[rows], W), what="split-K tail")


@pytest.mark.parametrize("M,K,N,out_f32", [(378, 9216, 4096, True), (3402, 4096, 1024, False)],
                         ids=["projector_v4", "fc2_v4"])
def test_linear_split_k_under_one_round(M, K, N, out_f32):
    """Launches with fewer tiles than compute units.  The 384-token image's projector (64
    tiles of 256 x 128): every tile is cut into K slices whose fp32 partials a second kernel
    sums in slice order.  Its fc2 (K = 4096) runs as 216 unsplit tiles of 128 x 128, which fill
    84% of the compute units.  Rows in every tile row are checked."""
    torch = require_gpu()
    enc, _, _ = encoder()
    A = seeded_bf16((M, K), 128, 0)
    W = seeded_bf16((N, K), 128, 1, std=0.02)
    b = seeded_bf16((N,), 128, 2, std=0.02)
    got = enc.op_linear(to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b), vit.ACT_NONE, out_f32)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0:2, 255:258, np.arange(0, M, 211), M - 3:M])
    want = oracle.linear(f32(A[rows]), f32(W), f32(b), round_out=not out_f32, workers=8)
    if out_f32:
        g = got.cpu().numpy()[rows]
        assert np.all(np.abs(g - want) <= sum_bound(A[rows], W) + 1e-6 * np.abs(want))
    else:
        assert_bf16_close(from_dev_bf16(got)[rows], want, atol=sum_bound(A[rows], W), what="split-K under one round")


# ------------------------------------------------------------------------------------------
# LayerNorm (+ residual)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [
    (300, 128, 200),     # ragged M, several tiles, rows of 400 bytes (staged writer)
    (257, 192, 130),     # rows of 260 bytes: per-element stores
    (1, 64, 5),          # degenerate single row, tiny N
    (9216, 1024, 1024),  # out-projection of the 1024-token image (192 x 256 tiles)
    (9216, 4096, 1024),  # fc2 of that image (192 x 256 tiles, one round)
    (24700, 1024, 2000),  # 256 x 256 tiles, rows 24576.. as the 128 x 128 row tail
    (3402, 4096, 1024),  # fc2 of the 384-token image (216 tiles of 128 x 128, one round)
], ids=["small", "unstaged", "one_row", "out_proj_1024", "fc2_1024", "row_tail", "fc2_384"])
def test_linear_residual(M, K, N):
    """x = bf16(x + bf16(A W^T + b)) in place: bitwise the residual add ([Z] "Step 2" table,
    residual order of the block output; the oracle's add_round) of vit_op_linear's own output,
    which the linear tests pin to the oracle; sampled rows also against the oracle directly."""
    torch = require_gpu()
    enc, _, _ = encoder()
    A = seeded_bf16((M, K), 109, 0)
    W = seeded_bf16((N, K), 109, 1, std=0.03)
    b = seeded_bf16((N,), 109, 2, std=0.1)
    x = seeded_bf16((M, N), 109, 3, std=2.0)
    dA, dW, db = to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b)
    dx = to_dev_bf16(x)
    d = enc.op_linear(dA, dW, db, vit.ACT_NONE, False)
    got = enc.op_linear_residual(dA, dW, db, dx)
    torch.cuda.synchronize()
    assert got.data_ptr() == dx.data_ptr()
    g = from_dev_bf16(got)
    want = oracle.add_round(f32(x), from_dev_bf16(d))
    assert np.array_equal(bf16_bits_of(g), bf16_bits_of(want)), "fused residual differs from linear + add"
    rows = np.unique(np.r_[0, M // 2, M - 1, max(0, M - 300):M:37])
    d_o = oracle.linear(f32(A[rows]), f32(W), f32(b), act=vit.ACT_NONE, round_out=True, workers=8)
    w_o = oracle.add_round(f32(x[rows]), d_o)
    tol = 2.0 ** -7 * (np.abs(w_o) + np.abs(d_o)) + sum_bound(A[rows], W)
    assert np.all(np.abs(g[rows] - w_o) <= tol), "fused residual off the oracle"


def test_linear_residual_rejects_overlap():
    torch = require_gpu()
    enc, _, _ = encoder()
    buf = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vit.VitError):
        enc.op_linear_residual(buf, W, None, buf.view(-1)[:64 * 64].view(64, 64))


@pytest.mark.parametrize("M,D,residual", [(37, 64, False), (1000, 1024, True), (9216, 1024, True),
                                          (5, 256, True)])
def test_layernorm(M, D, residual):
    torch = require_gpu()
    enc, _, _ = encoder()
    x = seeded_bf16((M, D), 104, 0, std=2.0, mean=0.5)
    dl = seeded_bf16((M, D), 104, 1, std=1.0)
    g = seeded_bf16((D,), 104, 2, std=0.1, mean=1.0)
    b = seeded_bf16((D,), 104, 3, std=0.1)
    dx = to_dev_bf16(x)
    out = enc.op_layernorm(dx, to_dev_bf16(g), to_dev_bf16(b), 1e-6,
                           delta=to_dev_bf16(dl) if residual else None, xout=dx if residual else None)
    torch.cuda.synchronize()
    xr = oracle.add_round(f32(x), f32(dl)) if residual else f32(x)
    if residual:
        assert np.array_equal(from_dev_bf16(dx), xr), "residual add must be exact"
    want = oracle.layernorm(xr, f32(g), f32(b), 1e-6)
    assert_bf16_close(from_dev_bf16(out), want, atol=1e-6, what="layernorm")


# ------------------------------------------------------------------------------------------
# official-layer variant: RMSNorm, erf GELU, SwiGLU, two-linear aligner
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,D,residual", [(37, 64, False), (1000, 1024, True), (9216, 1024, True),
                                          (5, 256, True), (3, 2048, False)])
def test_rmsnorm(M, D, residual):
    torch = require_gpu()
    enc, _, _ = encoder()
    x = seeded_bf16((M, D), 120, 0, std=2.0, mean=0.5)
    x[0, :] = 0                                   # an all-zero row: eps alone in the root
    dl = seeded_bf16((M, D), 120, 1, std=1.0)
    g = seeded_bf16((D,), 120, 2, std=0.1, mean=1.0)
    dx = to_dev_bf16(x)
    out = enc.op_rmsnorm(dx, to_dev_bf16(g), 1e-6, delta=to_dev_bf16(dl) if residual else None,
                         xout=dx if residual else None)
    torch.cuda.synchronize()
    xr = oracle.add_round(f32(x), f32(dl)) if residual else f32(x)
    if residual:
        assert np.array_equal(from_dev_bf16(dx), xr), "residual add must be exact"
    want = oracle.rmsnorm(xr, f32(g), 1e-6)
    assert_bf16_close(from_dev_bf16(out), want, atol=1e-6, what="rmsnorm")


def _swiglu_want(A, Wg, bg, Wu, bu, workers=1):
    """Oracle SwiGLU step and its slack: the gate and up sums (fp32, another order) move h by
    at most |silu'(g)| |u| dg + |silu(g)| du, with |silu'| <= 1.1 and |silu(g)| <= |g|."""
    g = oracle.linear(f32(A), f32(Wg), f32(bg), round_out=False, workers=workers)
    u = oracle.linear(f32(A), f32(Wu), f32(bu), round_out=False, workers=workers)
    h = oracle.swiglu(g, u)
    slack = 1.1 * np.abs(u) * sum_bound(A, Wg) + np.abs(g) * sum_bound(A, Wu) + 1e-6 * np.abs(h)
    return h, slack


@pytest.mark.parametrize("M,K,F", [(300, 128, 200), (1, 64, 8), (257, 192, 64), (129, 256, 520)])
def test_linear_swiglu_small(M, K, F):
    """Gate and up projections with silu(g) u in the epilogue, weights interleaved in groups
    of 8 rows; ragged M and F (F = 200, 520: the last 256-wide fused tile is partial)."""
    torch = require_gpu()
    enc, _, _ = encoder()
    A = seeded_bf16((M, K), 121, 0)
    Wg = seeded_bf16((F, K), 121, 1, std=0.05)
    Wu = seeded_bf16((F, K), 121, 2, std=0.05)
    bg = seeded_bf16((F,), 121, 3, std=0.1)
    bu = seeded_bf16((F,), 121, 4, std=0.1)
    W = vit.swiglu_interleave(Wg, Wu)
    b = vit.swiglu_interleave(bg, bu)
    got = enc.op_linear(to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b), vit.ACT_SWIGLU)
    torch.cuda.synchronize()
    assert tuple(got.shape) == (M, F)
    want, slack = _swiglu_want(A, Wg, bg, Wu, bu)
    assert_bf16_close(from_dev_bf16(got), want, atol=slack, what="swiglu")


def test_linear_swiglu_gate_up_roles_exact():
    """Gate weights 0 with bias b_g and up weights one-hot: h = bf16(silu(b_g) a_sel), a single
    product per output, so the only rounding is the final one -- checked bit for bit against
    the oracle with the same operands (silu on the GPU uses exp2 and a reciprocal: values
    within 2 ulps of fp32, compared at bf16 with one-ulp slack)."""
    torch = require_gpu()
    enc, _, _ = encoder()
    M, K, F = 200, 128, 96
    A = seeded_bf16((M, K), 122)
    sel = np.random.default_rng(1).permutation(K)[:F]
    Wu = np.zeros((F, K), np.uint16)
    Wu[np.arange(F), sel] = 0x3F80
    Wg = np.zeros((F, K), np.uint16)
    bg = seeded_bf16((F,), 122, 1, std=2.0)
    bu = np.zeros(F, np.uint16)
    got = from_dev_bf16(enc.op_linear(to_dev_bf16(A), to_dev_bf16(vit.swiglu_interleave(Wg, Wu)),
                                      to_dev_bf16(vit.swiglu_interleave(bg, bu)), vit.ACT_SWIGLU))
    torch.cuda.synchronize()
    want = oracle.swiglu(np.broadcast_to(f32(bg), (M, F)), f32(A)[:, sel])
    assert_bf16_close(got, want, what="swiglu roles")
    # swapped roles would give bf16(silu(a_sel) b_g): make sure that differs on this input
    assert not np.array_equal(want, oracle.swiglu(f32(A)[:, sel], np.broadcast_to(f32(bg), (M, F))))


@pytest.mark.parametrize("M", [9216, 6200], ids=["one_image", "row_tail"])
def test_linear_swiglu_full_size_sampled(M):
    """The official MLP's first step at the 1024-token image's shape (K = 1024, F = 4096, 8192
    fused rows), and at a row count whose last round runs as the 128 x 128 row tail (800 tiles
    of 256 x 256: rows 6144..6199 after the first 768)."""
    torch = require_gpu()
    enc, _, _ = encoder()
    K, F = 1024, 4096
    A = seeded_bf16((M, K), 123, 0)
    Wg = seeded_bf16((F, K), 123, 1, std=0.02)
    Wu = seeded_bf16((F, K), 123, 2, std=0.02)
    bg = seeded_bf16((F,), 123, 3, std=0.02)
    bu = seeded_bf16((F,), 123, 4, std=0.02)
    got = from_dev_bf16(enc.op_linear(to_dev_bf16(A), to_dev_bf16(vit.swiglu_interleave(Wg, Wu)),
                                      to_dev_bf16(vit.swiglu_interleave(bg, bu)), vit.ACT_SWIGLU))
    torch.cuda.synchronize()
    seam = 8192 if M == 9216 else 6144
    rows = np.unique(np.r_[0:3, 127:130, 4000:4003, seam - 4:seam + 4, M - 5:M])
    want, slack = _swiglu_want(A[rows], Wg, bg, Wu, bu, workers=8)
    assert_bf16_close(got[rows], want, atol=slack, what="swiglu full size")


@pytest.mark.parametrize("M,K,N", [(257, 192, 130), (1024, 9216, 5120)], ids=["small", "aligner"])
def test_linear_gelu_erf(M, K, N):
    torch = require_gpu()
    enc, _, _ = encoder()
    A = seeded_bf16((M, K), 124, 0)
    W = seeded_bf16((N, K), 124, 1, std=0.02)
    b = seeded_bf16((N,), 124, 2, std=0.1)
    got = from_dev_bf16(enc.op_linear(to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(b), vit.ACT_GELU_ERF))
    torch.cuda.synchronize()
    rows = np.arange(M) if M < 1000 else np.r_[0:3, 500:503, M - 4:M]
    want = oracle.linear(f32(A[rows]), f32(W), f32(b), act=2)
    assert_bf16_close(got[rows], want, atol=1.2 * sum_bound(A[rows], W) + 1e-6, what="gelu erf")


def test_linear_rejects_activation_with_fp32_output():
    require_gpu()
    enc, _, _ = encoder()
    A = to_dev_bf16(seeded_bf16((8, 64), 125))
    W = to_dev_bf16(seeded_bf16((16, 64), 125, 1))
    with pytest.raises(vit.VitError):
        enc.op_linear(A, W, None, vit.ACT_GELU_ERF, out_f32=True)
    with pytest.raises(vit.VitError):
        enc.op_linear(A, to_dev_bf16(seeded_bf16((24, 64), 125, 2)), None, vit.ACT_SWIGLU)


_official = {}


def official_encoder():
    if "tiny" not in _official:
        require_gpu()
        cfg = synth.TINY_OFFICIAL
        blob = synth.make_weights(cfg, perturbed=True)
        _official["tiny"] = (vit.Encoder(cfg, blob), cfg, blob)
    return _official["tiny"]


@pytest.mark.parametrize("grids", [[(6, 6)], [(5, 7), (3, 9), (1, 1), (4, 8)]])
def test_two_linear_aligner(grids):
    """Merge gather + first projection + erf GELU (bf16), then the second projection (fp32)."""
    torch = require_gpu()
    enc, cfg, blob = official_encoder()
    N = sum(a * b for a, b in grids)
    y = seeded_bf16((N, cfg.hidden), 126)
    got = enc.op_merge_project(to_dev_bf16(y), grids).cpu().numpy()
    torch.cuda.synchronize()
    W = oracle.Weights(cfg, blob)
    off, want = 0, []
    for gh, gw in grids:
        A = oracle.merge(f32(y[off:off + gh * gw]), gh, gw)
        want.append(oracle.aligner(cfg, A, W))
        off += gh * gw
    want = np.concatenate(want)
    assert got.shape == want.shape
    assert rel_l2(got, want) < 1e-3 and np.abs(got - want).max() <= 1e-2 * np.abs(want).max()


# ------------------------------------------------------------------------------------------
# RoPE + attention
# ------------------------------------------------------------------------------------------
def _qkv_for(grids, D, seed, std=1.0):
    N = sum(gh * gw for gh, gw in grids)
    return seeded_bf16((N, 3 * D), seed, 0, std=std)


def _oracle_rope(qkv_f, grids, cfg):
    out, off = [], 0
    for gh, gw in grids:
        n = gh * gw
        out.append(oracle.rope_qk(qkv_f[off:off + n], gw, cfg.hidden, cfg.heads, cfg.rope_base))
        off += n
    return np.concatenate(out)


@pytest.mark.parametrize("name,grids", [("tiny", [(6, 6)]), ("tiny", [(5, 7), (1, 1), (9, 12)]),
                                        ("v41_1layer", [(24, 24)]), ("v41_1layer", [(7, 11), (30, 3)])])
def test_rope_exact(name, grids):
    """RoPE multiplies by the same fp32 cos/sin and rounds once per element on both sides."""
    torch = require_gpu()
    enc, cfg, _ = encoder(name)
    qkv = _qkv_for(grids, cfg.hidden, 105)
    d = to_dev_bf16(qkv)
    vt = enc.op_rope(d, grids)
    torch.cuda.synchronize()
    want = _oracle_rope(f32(qkv), grids, cfg)
    D = cfg.hidden
    got = qkv_after_rope(d, D)
    # q and v bf16 as the oracle rounds them; k is the oracle's bf16 value stored as binary16
    assert np.array_equal(got[:, :D], want[:, :D])
    assert np.array_equal(got[:, 2 * D:], want[:, 2 * D:])
    assert np.array_equal(got[:, D:2 * D], f16_of(want[:, D:2 * D]))
    _check_vt(vt, f32(qkv[:, 2 * D:]), grids, cfg)


def _check_vt(vt, v_bf16, grids, cfg):
    """v transposed per head as binary16 (round to nearest even, saturating at 65504: exact
    except below 2^-14, where binary16 is subnormal), each image at its own 64-aligned column
    block, zero padding; inside each 16-column group, column p holds key p with bits 2 and 3
    swapped."""
    import torch
    assert vt.dtype == torch.float16
    vtn = vt.float().cpu().numpy()
    H, hd = cfg.heads, cfg.head_dim
    off = col = 0
    for gh, gw in grids:
        n = gh * gw
        pad = -(-n // 64) * 64
        v = np.zeros((H, hd, pad), np.float32)
        vv = np.clip(v_bf16[off:off + n], -65504, 65504)
        v[:, :, :n] = vv.astype(np.float16).astype(np.float32).reshape(n, H, hd).transpose(1, 2, 0)
        p = np.arange(pad)
        key = (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1)
        assert np.array_equal(vtn[:, :, col:col + pad], v[:, :, key])
        off += n
        col += pad


@pytest.mark.parametrize("name,grids", [("tiny", [(6, 6)]), ("tiny", [(5, 7), (1, 1), (9, 12), (2, 3)]),
                                        ("v41_1layer", [(24, 24)]),
                                        ("v41_1layer", [(7, 11), (30, 3), (13, 21)])])
def test_qkv_rope_fused_one_hot(name, grids):
    """The QKV projection with RoPE and the transposed-V copy in its epilogue (the encoder's
    path).  One-hot weight rows copy input columns exactly, plus a bias with one rounding, so
    q, k, v and V^T must equal bitwise the oracle's RoPE of those values.  The ragged grids put
    images at offsets that are not multiples of 4 and across a 256-row tile boundary."""
    torch = require_gpu()
    enc, cfg, _ = encoder(name)
    D = cfg.hidden
    N = sum(gh * gw for gh, gw in grids)
    x = seeded_bf16((N, D), 120, 0)
    sigma = np.random.default_rng(120).integers(0, D, 3 * D)
    W = np.zeros((3 * D, D), np.uint16)
    W[np.arange(3 * D), sigma] = 0x3F80          # bf16 1.0
    b = seeded_bf16((3 * D,), 120, 1, std=0.1)
    qkv, vt = enc.op_qkv_rope(to_dev_bf16(x), to_dev_bf16(W), to_dev_bf16(b), grids, store_v=True)
    torch.cuda.synchronize()
    proj = oracle.linear(f32(x), f32(W), f32(b), round_out=True)
    want = _oracle_rope(proj, grids, cfg)
    got = qkv_after_rope(qkv, D)
    assert np.array_equal(got[:, :D], want[:, :D])
    assert np.array_equal(got[:, D:2 * D], f16_of(want[:, D:2 * D]))
    assert np.array_equal(got[:, 2 * D:], want[:, 2 * D:])
    _check_vt(vt, proj[:, 2 * D:], grids, cfg)


@pytest.mark.parametrize("grids", [[(96, 96)], [(54, 63), (13, 21)]], ids=["v41_1024", "packed"])
def test_qkv_rope_fused_equals_separate_steps(grids):
    """At full width with random weights the fused kernel equals the linear layer followed by
    the separate RoPE pass, bitwise (same tiles, same accumulation order, same rotation)."""
    torch = require_gpu()
    enc, cfg, _ = encoder("v41_1layer")
    D = cfg.hidden
    N = sum(gh * gw for gh, gw in grids)
    x = to_dev_bf16(seeded_bf16((N, D), 121, 0))
    W = to_dev_bf16(seeded_bf16((3 * D, D), 121, 1, std=0.02))
    b = to_dev_bf16(seeded_bf16((3 * D,), 121, 2, std=0.02))
    qkv, vt = enc.op_qkv_rope(x, W, b, grids)
    lin = enc.op_linear(x, W, b)
    vt2 = enc.op_rope(lin, grids)
    torch.cuda.synchronize()
    a = qkv.view(torch.int16)[:, :2 * D].cpu().numpy()
    c = lin.view(torch.int16)[:, :2 * D].cpu().numpy()
    assert np.array_equal(a, c)
    assert torch.equal(vt.view(torch.int16), vt2.view(torch.int16))


def _attention_check(got, qkv_rot, grids, cfg, rows_per_image=None):
    off = 0
    for gh, gw in grids:
        n = gh * gw
        sl = qkv_rot[off:off + n]
        rows = range(n) if rows_per_image is None else sorted(set(r for r in rows_per_image(n)))
        for r in rows:
            want = oracle.attention(sl, cfg.hidden, cfg.heads, rows=(r, r + 1))[r]
            g = got[off + r]
            vmax = np.abs(sl[:, 2 * cfg.hidden:]).max()
            # the scores use q * log2(e)/sqrt(hd) rounded to binary16 (2^-11 relative per
            # element); P enters P.V as binary16 rounded toward zero (below 2^-10 relative per
            # weight, plus 2^-24 absolute for subnormal weights); plus the output rounding on
            # both sides
            tol = 2.0 ** -8 * vmax + 2.0 ** -7 * np.abs(want)
            assert np.all(np.abs(g - want) <= tol), (gh, gw, r, np.abs(g - want).max())
        off += n


@pytest.mark.parametrize("name,grids", [("tiny", [(6, 6)]), ("tiny", [(5, 7), (1, 1), (12, 15)]),
                                        ("v41_1layer", [(24, 24)]),
                                        ("v41_1layer", [(13, 21), (1, 2), (3, 3)])])
def test_attention_small(name, grids):
    torch = require_gpu()
    enc, cfg, _ = encoder(name)
    qkv = _qkv_for(grids, cfg.hidden, 106)
    d = to_dev_bf16(qkv)
    vt = enc.op_rope(d, grids)
    o = enc.op_attention(d, vt, grids)
    torch.cuda.synchronize()
    rot = _oracle_rope(f32(qkv), grids, cfg)
    _attention_check(from_dev_bf16(o), rot, grids, cfg,
                     rows_per_image=lambda n: list(range(min(n, 20))) + [n - 1, n // 2])


@pytest.mark.parametrize("hidden,heads", [(128, 8), (128, 4), (1024, 16), (256, 2), (1024, 8)],
                         ids=["hd16", "hd32", "hd64", "hd128_h2", "hd128_h8"])
def test_attention_head_dims(hidden, heads):
    """Every supported head dim with unit-variance q and k, so the softmax is far from
    uniform and every head dimension moves the scores; ragged images and one spanning several
    query tiles and key slices."""
    from dataclasses import replace
    torch = require_gpu()
    cfg = replace(synth.TINY, hidden=hidden, heads=heads, mlp=256, layers=0, out_hidden=16)
    key = ("hd", hidden, heads)
    if key not in _encs:
        _encs[key] = (vit.Encoder(cfg, synth.make_weights(cfg)), cfg, None)
    enc = _encs[key][0]
    grids = [(5, 7), (1, 1), (20, 21), (2, 3)]
    qkv = _qkv_for(grids, hidden, 127)
    d = to_dev_bf16(qkv)
    vt = enc.op_rope(d, grids)
    for split in (0, 3):
        enc.set_attention_split(split)
        o = enc.op_attention(d, vt, grids)
        torch.cuda.synchronize()
        rot = _oracle_rope(f32(qkv), grids, cfg)
        _attention_check(from_dev_bf16(o), rot, grids, cfg,
                         rows_per_image=lambda n: list(range(min(n, 12))) + [n - 1, n // 2, 200 % n])
    enc.set_attention_split(0)


def _bf16_bits_rne(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("big", ["q", "k", "v"])
def test_attention_binary16_operand_range(big):
    """The attention's binary16 operands near the top of their range: one of q, k, v drawn with
    standard deviation 2^11 .. 2^13 and entries of magnitude 2^15 planted in every head (after
    the rotation up to 2^15 * sqrt(2) = 46,341 < 65,504), the others scaled so that the scores
    stay those of an ordinary softmax.  Checked against the oracle at the attention bound on
    every query row."""
    torch = require_gpu()
    enc, cfg, _ = encoder("v41_1layer")
    D, H = cfg.hidden, cfg.heads
    grids = [(5, 7), (12, 11)]
    N = sum(a * b for a, b in grids)
    scale = {"q": (2.0 ** 11, 2.0 ** -9, 1.0), "k": (2.0 ** -9, 2.0 ** 11, 1.0),
             "v": (1.0, 1.0, 2.0 ** 13)}[big]
    x = synth.normal_f32(131, "qkv".index(big), N * 3 * D).reshape(N, 3, D)
    x = x * np.array(scale, np.float32)[None, :, None]
    j = "qkv".index(big)
    rng = np.random.default_rng(131)
    for h in range(H):
        rows = rng.choice(N, 3, replace=False)
        cols = h * (D // H) + rng.choice(D // H, 3, replace=False)
        x[rows, j, cols] = np.float32(2.0 ** 15) * np.sign(rng.standard_normal(3)).astype(np.float32)
    x = np.clip(x, -2.0 ** 15, 2.0 ** 15).reshape(N, 3 * D)
    qkv = _bf16_bits_rne(x)
    assert np.abs(f32(qkv)).max() == 2.0 ** 15
    d = to_dev_bf16(qkv)
    vt = enc.op_rope(d, grids)
    o = enc.op_attention(d, vt, grids)
    torch.cuda.synchronize()
    got = from_dev_bf16(o)
    assert np.isfinite(got).all()
    rot = _oracle_rope(f32(qkv), grids, cfg)
    assert np.abs(rot[:, :2 * D]).max() < 65504
    _attention_check(got, rot, grids, cfg)


def test_attention_single_patch_image_is_v():
    """A 1-patch image attends only to itself: output = v exactly."""
    torch = require_gpu()
    enc, cfg, _ = encoder("v41_1layer")
    grids = [(1, 1), (2, 3), (1, 1)]
    qkv = _qkv_for(grids, cfg.hidden, 107)
    d = to_dev_bf16(qkv)
    vt = enc.op_rope(d, grids)
    o = from_dev_bf16(enc.op_attention(d, vt, grids))
    torch.cuda.synchronize()
    D = cfg.hidden
    assert np.array_equal(o[0], f32(qkv[0, 2 * D:]))
    assert np.array_equal(o[7], f32(qkv[7, 2 * D:]))


def test_attention_images_are_isolated():
    """Changing one image of a packed batch leaves the other images bitwise unchanged."""
    torch = require_gpu()
    enc, cfg, _ = encoder("v41_1layer")
    grids = [(9, 12), (15, 6), (4, 4)]
    qkv = _qkv_for(grids, cfg.hidden, 108)
    qkv2 = qkv.copy()
    n0 = 9 * 12
    qkv2[n0:n0 + 90] = _qkv_for([(9, 10)], cfg.hidden, 109)
    outs = []
    for q in (qkv, qkv2):
        d = to_dev_bf16(q)
        vt = enc.op_rope(d, grids)
        outs.append(from_dev_bf16(enc.op_attention(d, vt, grids)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0][:n0], outs[1][:n0])
    assert np.array_equal(outs[0][n0 + 90:], outs[1][n0 + 90:])
    assert not np.array_equal(outs[0][n0:n0 + 90], outs[1][n0:n0 + 90])


@pytest.mark.parametrize("grids", [[(96, 96)], [(54, 63)]], ids=["v41_1024", "v4_384"])
def test_attention_full_size_sampled(grids):
    """Attention over one 9216-patch (or 3402-patch) image, sampled query rows."""
    torch = require_gpu()
    enc, cfg, _ = encoder("v41_1layer")
    qkv = _qkv_for(grids, cfg.hidden, 110)
    d = to_dev_bf16(qkv)
    vt = enc.op_rope(d, grids)
    o = from_dev_bf16(enc.op_attention(d, vt, grids))
    torch.cuda.synchronize()
    rot = _oracle_rope(f32(qkv), grids, cfg)
    _attention_check(o, rot, grids, cfg, rows_per_image=lambda n: [0, 1, 127, 128, n // 3, n - 1])


@pytest.mark.parametrize("grids", [[(96, 96)], [(54, 63)], [(13, 21), (1, 2), (3, 3)]],
                         ids=["v41_1024", "v4_384", "ragged_small"])
def test_attention_key_slices(grids):
    """Every fixed number of key slices (1..4; short images leave some slices empty) meets the
    oracle bound on sampled rows.  The automatic plan runs each (query tile, head) either whole
    or cut into a fixed number of slices, so each of its outputs equals bitwise the same
    output of one of the fixed runs."""
    torch = require_gpu()
    enc, cfg, _ = encoder("v41_1layer")
    qkv = _qkv_for(grids, cfg.hidden, 112)
    outs = {}
    try:
        for n in (1, 2, 3, 4, 0):
            enc.set_attention_split(n)
            d = to_dev_bf16(qkv)
            vt = enc.op_rope(d, grids)
            outs[n] = from_dev_bf16(enc.op_attention(d, vt, grids))
        torch.cuda.synchronize()
        with pytest.raises(vit.VitError):
            enc.set_attention_split(5)
    finally:
        enc.set_attention_split(0)
    rot = _oracle_rope(f32(qkv), grids, cfg)
    for n in (1, 2, 3, 4):
        _attention_check(outs[n], rot, grids, cfg, rows_per_image=lambda m: [r for r in (0, 1, 63, 64, m // 2, m - 1) if r < m])
    same = np.zeros(outs[0].shape, bool)
    for n in (1, 2, 3, 4):
        same |= outs[0] == outs[n]
    assert same.all()


def test_attention_packed16_sampled():
    """The packed 16-image batch (varlen, block-diagonal), sampled rows of every image."""
    torch = require_gpu()
    enc, cfg, _ = encoder("v41_1layer")
    grids = synth.workload("packed16").grids
    qkv = _qkv_for(grids, cfg.hidden, 111)
    d = to_dev_bf16(qkv)
    vt = enc.op_rope(d, grids)
    o = from_dev_bf16(enc.op_attention(d, vt, grids))
    torch.cuda.synchronize()
    off = 0
    for gh, gw in grids:
        n = gh * gw
        sl = oracle.rope_qk(f32(qkv[off:off + n]), gw, cfg.hidden, cfg.heads, cfg.rope_base)
        for r in (0, n - 1):
            want = oracle.attention(sl, cfg.hidden, cfg.heads, rows=(r, r + 1))[r]
            tol = 2.0 ** -8 * np.abs(sl[:, 2 * cfg.hidden:]).max() + 2.0 ** -7 * np.abs(want)
            assert np.all(np.abs(o[off + r] - want) <= tol), (gh, gw, r)
        off += n


# ------------------------------------------------------------------------------------------
# merge + projector, overlay
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("grids", [[(6, 6)], [(5, 7)], [(5, 7), (3, 9), (1, 1), (4, 8)]])
def test_merge_project(grids):
    torch = require_gpu()
    enc, cfg, blob = encoder("tiny", perturbed=True)
    N = sum(a * b for a, b in grids)
    y = seeded_bf16((N, cfg.hidden), 112)
    got = enc.op_merge_project(to_dev_bf16(y), grids).cpu().numpy()
    torch.cuda.synchronize()
    W = oracle.Weights(cfg, blob)
    off, want = 0, []
    for gh, gw in grids:
        A = oracle.merge(f32(y[off:off + gh * gw]), gh, gw)
        want.append(oracle.linear(A, W["proj.w"], W["proj.b"], round_out=False))
        off += gh * gw
    want = np.concatenate(want)
    np.testing.assert_allclose(got, want, rtol=1e-4, atol=1e-4)


def test_merge_project_split_k_tail():
    """The merge gather into the projector at full width for two 1024-token images: 320 tiles
    of 256 x 128 (2048 rows x 40 column tiles, K = 9216) leave a round of 64 tiles, which are
    cut into K slices whose fp32 partials a second kernel sums.  Rows in every tile row, the
    leftover ones included, against the oracle's merge and linear."""
    torch = require_gpu()
    enc, cfg, blob = encoder("v41_1layer")
    grids = [(96, 96), (96, 96)]
    N = sum(a * b for a, b in grids)
    y = seeded_bf16((N, cfg.hidden), 131)
    got = enc.op_merge_project(to_dev_bf16(y), grids).cpu().numpy()
    torch.cuda.synchronize()
    W = oracle.Weights(cfg, blob)
    rows = np.unique(np.r_[0:2, 255:258, np.arange(0, 2048, 233), 1790:1794, 2044:2048])
    A = np.concatenate([oracle.merge(f32(y[:9216]), 96, 96), oracle.merge(f32(y[9216:]), 96, 96)])[rows]
    Wp = W["proj.w"]
    want = oracle.linear(A, Wp, W["proj.b"], round_out=False, workers=8)
    g = got[rows]
    assert g.shape == want.shape
    # sum_bound's slack, from fp32 operands: 2^-18 * sum_k |a_k w_k| per output
    slack = 2.0 ** -18 * (np.abs(A).astype(np.float64) @ np.abs(Wp).astype(np.float64).T)
    assert np.all(np.abs(g - want) <= slack + 1e-6 * np.abs(want))


def test_overlay_exact():
    torch = require_gpu()
    enc, cfg, _ = encoder("tiny")
    R, Dl, T = 50, cfg.out_hidden, 12
    emb = seeded_bf16((R, Dl), 113)
    rows = synth.normal_f32(113, 1, T * Dl, 0.0, 3.0).reshape(T, Dl)
    dst = list(synth.seeded_distinct_rows(T, R))
    dst[3] = -1
    d_emb = to_dev_bf16(emb)
    enc.overlay(d_emb, dst, torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    want = oracle.overlay(emb, dst, rows)
    got = d_emb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


def _prompt(grids, gaps, seed):
    """Span starts for images separated by text runs of the given lengths, and the prompt
    length (a last text run of gaps[-1] rows)."""
    starts, pos = [], 0
    for (gh, gw), g in zip(grids, gaps):
        pos += g
        starts.append(pos)
        pos += 2 + -(-gh // 3) * (-(-gw // 3) + 1)
    return starts, pos + gaps[-1]


def test_assemble_v4_span_layout_chunks_exact():
    """The V4 Flash span reading (row-pair interleave, spans at multiples of 4, PAD positions
    left as they are) written whole and chunk by chunk: bitwise the oracle's assembly."""
    torch = require_gpu()
    cfg = synth.TINY
    enc = vit.Encoder(cfg, synth.make_weights(cfg))
    enc.set_span_layout(vit.SPAN_V4)
    Dl = cfg.out_hidden
    sent = synth.make_sentinels(Dl)
    enc.set_sentinels(sent)
    grids = [(6, 9), (5, 7), (3, 3), (12, 3)]
    starts, pos = [], 8
    for g in grids:
        starts.append(pos)
        t, _ = oracle.layout_v4([g])
        pos += len(t) + 4
    R = pos + 4
    n_vis = sum(cfg.tokens(*g) for g in grids)
    rows = synth.normal_f32(115, 0, n_vis * Dl, 0.0, 3.0).reshape(n_vis, Dl)
    emb = seeded_bf16((R, Dl), 115, 1)
    d_rows = torch.from_numpy(rows).cuda()
    want = oracle.assemble(emb, 0, R, grids, starts, rows, sent, v4=True)
    for cuts in ([0, R], [0, 9, 13, 30, R], list(range(0, R, 7)) + [R]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            d = to_dev_bf16(emb[a:b])
            enc.assemble(d, a, grids, starts, d_rows)
            torch.cuda.synchronize()
            parts.append(d.view(torch.int16).cpu().numpy().view(np.uint16).reshape(b - a, Dl))
        assert np.array_equal(np.concatenate(parts), want)
    with pytest.raises(vit.VitError):   # a V4 span must start at a multiple of 4
        enc.assemble(to_dev_bf16(emb), 0, grids[:1], [2], d_rows[:cfg.tokens(*grids[0])])
    enc.close()


def test_assemble_chunks_exact():
    """Learned START/NEWLINE/END rows and the visual rows of four images, written into a
    prompt whole and chunk by chunk (a chunk inside one span, cuts through spans, an empty
    chunk): bitwise the oracle's assembly, other rows untouched."""
    torch = require_gpu()
    cfg = synth.TINY
    enc = vit.Encoder(cfg, synth.make_weights(cfg))
    Dl = cfg.out_hidden
    sent = synth.make_sentinels(Dl)
    grids = [(6, 6), (5, 7), (3, 3), (1, 1)]
    starts, R = _prompt(grids, [3, 0, 5, 1, 4], 0)
    n_vis = sum(-(-gh // 3) * -(-gw // 3) for gh, gw in grids)
    rows = synth.normal_f32(114, 0, n_vis * Dl, 0.0, 3.0).reshape(n_vis, Dl)
    emb = seeded_bf16((R, Dl), 114, 1)
    d_rows = torch.from_numpy(rows).cuda()
    with pytest.raises(vit.VitError):   # no sentinel rows yet
        enc.assemble(to_dev_bf16(emb), 0, grids, starts, d_rows)
    enc.set_sentinels(sent)
    want = oracle.assemble(emb, 0, R, grids, starts, rows, sent)
    d = to_dev_bf16(emb)
    enc.assemble(d, 0, grids, starts, d_rows)
    torch.cuda.synchronize()
    assert np.array_equal(d.view(torch.int16).cpu().numpy().view(np.uint16), want)
    for cuts in ([0, 7, 8, 8, 20, R], [0, 4, 12, R], list(range(0, R, 5)) + [R]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            d = to_dev_bf16(emb[a:b]) if b > a else torch.empty((0, Dl), dtype=torch.bfloat16, device="cuda")
            enc.assemble(d, a, grids, starts, d_rows)
            torch.cuda.synchronize()
            parts.append(d.view(torch.int16).cpu().numpy().view(np.uint16).reshape(b - a, Dl))
        assert np.array_equal(np.concatenate(parts), want)
    m1 = cfg.tokens(*grids[0])
    m2 = m1 + cfg.tokens(*grids[1])
    with pytest.raises(vit.VitError):   # overlapping spans
        enc.assemble(to_dev_bf16(emb), 0, grids[:2], [starts[0], starts[0] + 3], d_rows[:m2])
    with pytest.raises(vit.VitError):   # negative span start
        enc.assemble(to_dev_bf16(emb), 0, grids[:1], [-1], d_rows[:m1])
    with pytest.raises(ValueError):     # visual rows of another batch
        enc.assemble(to_dev_bf16(emb), 0, grids[:1], [0], d_rows)
    enc.close()

