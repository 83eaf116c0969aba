"""CPU oracle of the vision-encoder forward pass.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product (the HIP library and its binding)
never does, and this package never imports the product.

The arithmetic lives in ``vit_oracle.c`` (plain, single-threaded C, fp32 by default, with an
fp64 twin).  This file only marshals numpy arrays and sequences the steps in the order the
pages give them:
  [Z] "DeepSeek V4.1 Flash Engineering, Part 3: Integrating Vision" (zhuai.tech):
      "Multimodal basics", "Connect the complete image-to-text path", "Step 1" .. "Step 5";
  [G] ds4-learning "glossary/vision": V4 Flash and V4.1 Flash vision rows.

``workers`` > 1 splits the rows of a step over threads (each row is still computed by the
same single-threaded loop; results do not depend on the split).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vit_oracle.c")
_LIBS = {"f32": os.path.join(_HERE, "liboracle_f32.so"),
         "f64": os.path.join(_HERE, "liboracle_f64.so")}
_FLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]

# Span token types (row-major layout: START, (IMAGE x mw, NEWLINE) x mh, END; the V4 Flash
# reading adds PAD positions at the end of a span).
TOK_TEXT, TOK_START, TOK_IMAGE, TOK_NEWLINE, TOK_END, TOK_PAD = 0, 1, 2, 3, 4, 5


def build(force: bool = True):
    """Compile the fp32 and fp64 oracle libraries with gcc."""
    for prec, path in _LIBS.items():
        if force or not os.path.exists(path):
            real = "float" if prec == "f32" else "double"
            tmp = path + ".tmp"
            subprocess.check_call(["gcc", *_FLAGS, f"-DORC_REAL={real}", "-o", tmp, _SRC, "-lm"])
            os.replace(tmp, path)
    return list(_LIBS.values())


_libs: dict = {}


class _Lib:
    def __init__(self, prec: str):
        if not os.path.exists(_LIBS[prec]):
            build(force=False)
        L = ctypes.CDLL(_LIBS[prec])
        self.prec = prec
        self.dtype = np.float32 if prec == "f32" else np.float64
        r = ctypes.c_float if prec == "f32" else ctypes.c_double
        i32, i64, vp, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.orc_real_size.restype = i32
        assert L.orc_real_size() == np.dtype(self.dtype).itemsize
        L.orc_round_bf16.restype = r
        L.orc_round_bf16.argtypes = [r]
        L.orc_round_bf16_array.argtypes = [vp, i64]
        L.orc_gelu_tanh.restype = r
        L.orc_gelu_tanh.argtypes = [r]
        L.orc_gelu_erf.restype = r
        L.orc_gelu_erf.argtypes = [r]
        L.orc_silu.restype = r
        L.orc_silu.argtypes = [r]
        L.orc_swiglu.argtypes = [vp, vp, i64, vp]
        L.orc_rmsnorm.argtypes = [vp, i64, i64, i64, i32, vp, r, vp, i64]
        L.orc_patchify.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.orc_linear.restype = i32
        L.orc_linear.argtypes = [vp, i64, i64, i64, i32, vp, vp, i32, i32, i32, vp, i64]
        L.orc_layernorm.argtypes = [vp, i64, i64, i64, i32, vp, vp, r, vp, i64]
        L.orc_add_round.argtypes = [vp, vp, i64, vp]
        L.orc_rope_angle.argtypes = [i32, i32, i32, i32, dbl, vp, vp]
        L.orc_rope_qk.argtypes = [vp, i64, i64, i64, i32, i32, i32, dbl]
        L.orc_attention.restype = i32
        L.orc_attention.argtypes = [vp, i64, i64, i32, i32, i64, i64, vp, i64]
        L.orc_softmax_row.argtypes = [vp, i64, i64, i32, i32, i32, i64, vp]
        L.orc_merge.argtypes = [vp, i32, i32, i32, i32, vp]
        self.L = L


def lib(prec: str = "f32") -> _Lib:
    if prec not in _libs:
        _libs[prec] = _Lib(prec)
    return _libs[prec]


def _p(a: np.ndarray):
    return a.ctypes.data


def _split(n: int, workers: int):
    workers = max(1, min(workers, n))
    step = (n + workers - 1) // workers
    return [(s, min(n, s + step)) for s in range(0, n, step)]


def _run(fn, n: int, workers: int):
    parts = _split(n, workers)
    if len(parts) <= 1:
        for a, b in parts:
            fn(a, b)
        return
    with ThreadPoolExecutor(max_workers=len(parts)) as ex:
        list(ex.map(lambda ab: fn(*ab), parts))


# ------------------------------------------------------------------------------------------
# host format helpers (bit reinterpretation only)
# ------------------------------------------------------------------------------------------
def bf16_to_float(bits: np.ndarray, dtype=np.float32) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(dtype)


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (values already bf16 stay exact)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def pixel_affine(mean, std):
    """Per-channel (s_c, t_c) in fp32: s_c = 1/(255 std_c), t_c = -mean_c/std_c, evaluated in
    double from the fp32 values of mean and std (the configuration carries them in fp32)."""
    m32 = [float(np.float32(m)) for m in mean]
    s32 = [float(np.float32(sd)) for sd in std]
    s = np.array([1.0 / (255.0 * sd) for sd in s32], dtype=np.float32)
    t = np.array([-m / sd for m, sd in zip(m32, s32)], dtype=np.float32)
    return s, t


# ------------------------------------------------------------------------------------------
# steps
# ------------------------------------------------------------------------------------------
def round_bf16(x: np.ndarray, prec: str = "f32") -> np.ndarray:
    L = lib(prec)
    y = np.ascontiguousarray(x, dtype=L.dtype).copy()
    L.L.orc_round_bf16_array(_p(y), y.size)
    return y


def gelu_tanh(u: float, prec: str = "f32") -> float:
    return lib(prec).L.orc_gelu_tanh(u)


def gelu_erf(u: float, prec: str = "f32") -> float:
    return lib(prec).L.orc_gelu_erf(u)


def silu(u: float, prec: str = "f32") -> float:
    return lib(prec).L.orc_silu(u)


def patchify(img: np.ndarray, gh: int, gw: int, cfg, prec: str = "f32") -> np.ndarray:
    """[Z] "Step 1" items 5-6: one bf16 row per 14x14 patch, (c, y, x) inside the row."""
    L = lib(prec)
    img = np.ascontiguousarray(img, dtype=np.uint8)
    assert img.size == (cfg.patch * gh) * (cfg.patch * gw) * 3
    s, t = pixel_affine(cfg.pix_mean, cfg.pix_std)
    P = np.empty((gh * gw, cfg.patch_dim), dtype=L.dtype)
    L.L.orc_patchify(_p(img), gh, gw, cfg.patch, _p(s), _p(t), _p(P))
    return P


def linear(A: np.ndarray, W: np.ndarray | None, b: np.ndarray | None, act: int = 0,
           round_out: bool = True, prec: str = "f32", workers: int = 1,
           Wt: np.ndarray | None = None) -> np.ndarray:
    """out = act(A W^T + b), W given [out][in] (or already transposed as ``Wt`` [in][out]);
    bf16-rounded unless round_out is False."""
    L = lib(prec)
    A = np.ascontiguousarray(A, dtype=L.dtype)
    if Wt is None:
        Wt = np.asarray(W, dtype=L.dtype).T
    Wt = np.ascontiguousarray(Wt, dtype=L.dtype)
    M, K = A.shape
    N = Wt.shape[1]
    assert Wt.shape[0] == K
    bb = None if b is None else np.ascontiguousarray(b, dtype=L.dtype)
    out = np.empty((M, N), dtype=L.dtype)

    def f(r0, r1):
        rc = L.L.orc_linear(_p(A), K, r0, r1, K, _p(Wt), None if bb is None else _p(bb), N,
                            act, 1 if round_out else 0, _p(out), N)
        assert rc == 0
    _run(f, M, workers)
    return out


def layernorm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float, prec: str = "f32",
              workers: int = 1) -> np.ndarray:
    L = lib(prec)
    x = np.ascontiguousarray(x, dtype=L.dtype)
    g = np.ascontiguousarray(g, dtype=L.dtype)
    b = np.ascontiguousarray(b, dtype=L.dtype)
    M, D = x.shape
    out = np.empty_like(x)
    _run(lambda r0, r1: L.L.orc_layernorm(_p(x), D, r0, r1, D, _p(g), _p(b), eps, _p(out), D),
         M, workers)
    return out


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float, prec: str = "f32",
            workers: int = 1) -> np.ndarray:
    """Official tower norm: bf16(x / sqrt(mean(x^2) + eps) * g) per row."""
    L = lib(prec)
    x = np.ascontiguousarray(x, dtype=L.dtype)
    g = np.ascontiguousarray(g, dtype=L.dtype)
    M, D = x.shape
    out = np.empty_like(x)
    _run(lambda r0, r1: L.L.orc_rmsnorm(_p(x), D, r0, r1, D, _p(g), eps, _p(out), D), M, workers)
    return out


def swiglu(g: np.ndarray, u: np.ndarray, prec: str = "f32") -> np.ndarray:
    """bf16(silu(g) * u) elementwise on the unrounded gate and up projections."""
    L = lib(prec)
    g = np.ascontiguousarray(g, dtype=L.dtype)
    u = np.ascontiguousarray(u, dtype=L.dtype)
    assert g.shape == u.shape
    out = np.empty_like(g)
    L.L.orc_swiglu(_p(g), _p(u), g.size, _p(out))
    return out


def norm(cfg, x: np.ndarray, W, name: str, **kw) -> np.ndarray:
    """The configured norm of a block or the final norm: LayerNorm (gamma, beta) or, in the
    official-layer variant, RMSNorm (gamma only)."""
    if cfg.norm_kind == 1:
        return rmsnorm(x, W[name + ".g"], cfg.ln_eps, **kw)
    return layernorm(x, W[name + ".g"], W[name + ".b"], cfg.ln_eps, **kw)


def mlp(cfg, x: np.ndarray, W, l: int, **kw) -> np.ndarray:
    """The block's MLP: fc2(GELU(fc1 x)) with the configured GELU form, or, in the
    official-layer variant, down(silu(gate x) * up x) (SwiGLU)."""
    if cfg.mlp_kind == 1:
        g = linear(x, None, W[f"l{l}.gate.b"], round_out=False, Wt=W.T(f"l{l}.gate.w"), **kw)
        u = linear(x, None, W[f"l{l}.up.b"], round_out=False, Wt=W.T(f"l{l}.up.w"), **kw)
        h = swiglu(g, u, kw.get("prec", "f32"))
        return linear(h, None, W[f"l{l}.down.b"], Wt=W.T(f"l{l}.down.w"), **kw)
    act = 2 if cfg.gelu_kind == 1 else 1
    h = linear(x, None, W[f"l{l}.fc1.b"], act=act, Wt=W.T(f"l{l}.fc1.w"), **kw)
    return linear(h, None, W[f"l{l}.fc2.b"], Wt=W.T(f"l{l}.fc2.w"), **kw)


def aligner(cfg, A: np.ndarray, W, **kw) -> np.ndarray:
    """Projection of the merged rows (fp32 out).  One linear, or with ``aligner_hidden`` > 0
    two linears with the configured GELU between them ([Z] "Step 2" boundary table: the
    aligner output covers two linear projections): the first rounded to bf16 after its GELU,
    the second kept in fp32."""
    if cfg.aligner_hidden > 0:
        act = 2 if cfg.gelu_kind == 1 else 1
        a1 = linear(A, None, W["proj.b"], act=act, Wt=W.T("proj.w"), **kw)
        return linear(a1, None, W["proj2.b"], round_out=False, Wt=W.T("proj2.w"), **kw)
    return linear(A, None, W["proj.b"], round_out=False, Wt=W.T("proj.w"), **kw)


def add_round(a: np.ndarray, b: np.ndarray, prec: str = "f32") -> np.ndarray:
    L = lib(prec)
    a = np.ascontiguousarray(a, dtype=L.dtype)
    b = np.ascontiguousarray(b, dtype=L.dtype)
    out = np.empty_like(a)
    L.L.orc_add_round(_p(a), _p(b), a.size, _p(out))
    return out


def rope_angle(h: int, w: int, i: int, hd: int, base: float, prec: str = "f32"):
    L = lib(prec)
    c = np.zeros(1, L.dtype)
    s = np.zeros(1, L.dtype)
    L.L.orc_rope_angle(h, w, i, hd, base, _p(c), _p(s))
    return float(c[0]), float(s[0])


def rope_qk(qkv: np.ndarray, gw: int, D: int, H: int, base: float, prec: str = "f32",
            workers: int = 1) -> np.ndarray:
    """[Z] "Step 3": blocked height/width angles, rotate-half; returns a rotated copy."""
    L = lib(prec)
    out = np.ascontiguousarray(qkv, dtype=L.dtype).copy()
    n, ld = out.shape
    _run(lambda r0, r1: L.L.orc_rope_qk(_p(out), ld, r0, r1, gw, D, H, base), n, workers)
    return out


def attention(qkv: np.ndarray, D: int, H: int, prec: str = "f32", workers: int = 1,
              rows: tuple | None = None) -> np.ndarray:
    """Non-causal softmax attention over all patches of ONE image; bf16 output [n][D].
    ``rows=(q0, q1)`` computes only those query rows (the rest stay zero)."""
    L = lib(prec)
    qkv = np.ascontiguousarray(qkv, dtype=L.dtype)
    n, ld = qkv.shape
    o = np.zeros((n, D), dtype=L.dtype)
    q0, q1 = rows if rows is not None else (0, n)

    def f(a, b):
        rc = L.L.orc_attention(_p(qkv), ld, n, D, H, q0 + a, q0 + b, _p(o), D)
        assert rc == 0
    _run(f, q1 - q0, workers)
    return o


def softmax_row(qkv: np.ndarray, D: int, H: int, head: int, i: int, prec: str = "f32"):
    L = lib(prec)
    qkv = np.ascontiguousarray(qkv, dtype=L.dtype)
    n, ld = qkv.shape
    p = np.empty(n, dtype=L.dtype)
    L.L.orc_softmax_row(_p(qkv), ld, n, D, H, head, i, _p(p))
    return p


def merge(y: np.ndarray, gh: int, gw: int, m: int = 3, prec: str = "f32") -> np.ndarray:
    """[Z] "Step 4": right/bottom zero padding on the 2D grid, channel-major 3x3 unfold."""
    L = lib(prec)
    y = np.ascontiguousarray(y, dtype=L.dtype)
    D = y.shape[1]
    mh, mw = -(-gh // m), -(-gw // m)
    A = np.empty((mh * mw, m * m * D), dtype=L.dtype)
    L.L.orc_merge(_p(y), gh, gw, D, m, _p(A))
    return A


# ------------------------------------------------------------------------------------------
# the whole encoder, one image at a time (attention never crosses images)
# ------------------------------------------------------------------------------------------
class Weights:
    """The weight blob as `real` arrays by name (bf16 values widened exactly), converted on
    first use; ``T(name)`` caches the transposed [in][out] copy of a matrix."""

    def __init__(self, cfg, blob: np.ndarray, prec: str = "f32"):
        from synth import split_weights
        self.dt = lib(prec).dtype
        self.raw = split_weights(cfg, blob)
        self.t, self.tt = {}, {}

    def __getitem__(self, k):
        if k not in self.t:
            self.t[k] = bf16_to_float(self.raw[k], self.dt)
        return self.t[k]

    def T(self, k):
        if k not in self.tt:
            self.tt[k] = np.ascontiguousarray(bf16_to_float(self.raw[k].T, self.dt))
        return self.tt[k]


def block(cfg, W: Weights, x: np.ndarray, gh: int, gw: int, l: int, prec: str = "f32",
          workers: int = 1, dumps: dict | None = None) -> np.ndarray:
    """Pre-norm block l on the residual stream x (bf16 values, [gh*gw][D]) of one image:
    LN -> QKV (bias) -> 2D RoPE on q, k -> attention -> out-proj -> residual (bf16) ->
    LN -> MLP -> residual (bf16).  ``dumps`` receives the rotated qkv and the attention
    output ([Z] "Step 2" boundary table)."""
    D, H = cfg.hidden, cfg.heads
    kw = dict(prec=prec, workers=workers)
    ln = norm(cfg, x, W, f"l{l}.ln1", **kw)
    qkv = linear(ln, None, W[f"l{l}.qkv.b"], Wt=W.T(f"l{l}.qkv.w"), **kw)
    qkv = rope_qk(qkv, gw, D, H, cfg.rope_base, **kw)
    o = attention(qkv, D, H, **kw)
    a = linear(o, None, W[f"l{l}.o.b"], Wt=W.T(f"l{l}.o.w"), **kw)
    x = add_round(x, a, prec)
    ln2 = norm(cfg, x, W, f"l{l}.ln2", **kw)
    f = mlp(cfg, ln2, W, l, **kw)
    x = add_round(x, f, prec)
    if dumps is not None:
        dumps["qkv"] = qkv
        dumps["attn"] = o
    return x


def encode_image(cfg, W: Weights, img: np.ndarray, gh: int, gw: int, prec: str = "f32",
                 workers: int = 1, dumps: dict | None = None, layers: int | None = None):
    """Visual rows (fp32, [mh*mw][out_hidden]) of one image.

    Steps ([Z] "Connect the complete image-to-text path" and "Step 1".."Step 5"):
      patchify+normalise (bf16) -> patch projection (bf16) -> `layers` pre-norm blocks
      [LN -> QKV (bias) -> 2D RoPE on q,k -> attention -> out-proj -> residual ->
       LN -> fc1 + GELU-tanh -> fc2 -> residual], each output rounded to bf16
      -> final LN (bf16) -> 3x3 merge -> projection (kept in fp32).
    The official-layer variant (``cfg.norm_kind``, ``cfg.mlp_kind``, ``cfg.gelu_kind``,
    ``cfg.aligner_hidden``) swaps in RMSNorm, the SwiGLU MLP, erf GELU and the two-linear
    aligner at the same places (see ``norm``, ``mlp`` and ``aligner``).
    ``dumps``, if given, receives the boundary tensors of [Z] "Step 2".
    """
    nl = cfg.layers if layers is None else layers
    kw = dict(prec=prec, workers=workers)
    P = patchify(img, gh, gw, cfg, prec)
    x = linear(P, None, W["pe.b"], Wt=W.T("pe.w"), **kw)
    if dumps is not None:
        dumps["patches"] = P
        dumps["embed"] = x
    for l in range(nl):
        inner = {} if dumps is not None and l == 0 else None
        x = block(cfg, W, x, gh, gw, l, dumps=inner, **kw)
        if dumps is not None:
            dumps[f"layer{l}"] = x
            if l == 0:
                dumps["qkv0"] = inner["qkv"]
                dumps["attn0"] = inner["attn"]
    y = norm(cfg, x, W, "lnf", **kw)
    A = merge(y, gh, gw, cfg.merge, prec)
    out = aligner(cfg, A, W, **kw)
    if dumps is not None:
        dumps["final_norm"] = y
        dumps["merged"] = A
    return out


def encode(cfg, blob: np.ndarray, pixels: np.ndarray, grids, prec: str = "f32",
           workers: int = 1, images=None):
    """Visual rows of a packed batch, image-major (fp32).  ``images`` selects a subset
    (returns a dict image -> rows)."""
    W = Weights(cfg, blob, prec)
    offs = [0]
    for gh, gw in grids:
        offs.append(offs[-1] + (cfg.patch * gh) * (cfg.patch * gw) * 3)
    sel = range(len(grids)) if images is None else images
    res = {}
    for i in sel:
        gh, gw = grids[i]
        res[i] = encode_image(cfg, W, pixels[offs[i]:offs[i + 1]], gh, gw, prec, workers)
    if images is not None:
        return res
    return np.concatenate([res[i] for i in range(len(grids))]) if grids else \
        np.zeros((0, cfg.out_hidden), np.float32)


# ------------------------------------------------------------------------------------------
# image span layout and overlay ([Z] "Connect the complete image-to-text path";
# [G] V4.1 Flash vision: plain row-major stream, identity permutation)
# ------------------------------------------------------------------------------------------
def layout(grids, merge: int = 3):
    """Per image: START, then per merged row (IMAGE x mw, NEWLINE), then END.
    Returns (types[int32], src[int32]): src is the visual row (image-major numbering) of an
    IMAGE position and -1 elsewhere."""
    types, src, row = [], [], 0
    for gh, gw in grids:
        mh, mw = -(-gh // merge), -(-gw // merge)
        types.append(TOK_START)
        src.append(-1)
        for r in range(mh):
            for c in range(mw):
                types.append(TOK_IMAGE)
                src.append(row)
                row += 1
            types.append(TOK_NEWLINE)
            src.append(-1)
        types.append(TOK_END)
        src.append(-1)
    return np.array(types, np.int32), np.array(src, np.int32)


def layout_v4(grids, merge: int = 3, align: int = 4):
    """The V4 Flash span layout, as read from [G] (V4 Flash Vision-Exp column: synthetic
    sentinel tokens, row-pair interleave, pos % 4 alignment; V4.1 row: V4.1 drops the
    row-pair interleave and compress_pad) and [L] DS4V (the projector's tile permutation is
    applied once when rows are assembled with the named sentinel embeddings).  Reading (parity
    unpinned: the pages give no formula):
      START; then for each pair of merged rows (2p, 2p+1) -- the last row alone when mh is
      odd -- the pair's IMAGE positions column by column, (2p, c) then (2p+1, c), followed by
      one NEWLINE; then END; then PAD positions up to a multiple of `align` (compress_pad),
      so that a span placed at a multiple of `align` ends on one too.
    Returns (types, src) like ``layout``: src is the visual row (image-major, row-major inside
    the image as the encoder emits them) of an IMAGE position and -1 elsewhere."""
    types, src, first = [], [], 0
    for gh, gw in grids:
        mh, mw = -(-gh // merge), -(-gw // merge)
        span_t, span_s = [TOK_START], [-1]
        for p in range(0, mh, 2):
            rows_of_pair = [r for r in (p, p + 1) if r < mh]
            for c in range(mw):
                for r in rows_of_pair:
                    span_t.append(TOK_IMAGE)
                    span_s.append(first + r * mw + c)
            span_t.append(TOK_NEWLINE)
            span_s.append(-1)
        span_t.append(TOK_END)
        span_s.append(-1)
        while len(span_t) % align:
            span_t.append(TOK_PAD)
            span_s.append(-1)
        types += span_t
        src += span_s
        first += mh * mw
    return np.array(types, np.int32), np.array(src, np.int32)


def overlay(embeds_bits: np.ndarray, placeholder_rows, rows: np.ndarray) -> np.ndarray:
    """embeds[placeholder_rows[t]] = bf16(rows[t]); rows with a negative index are skipped.
    [Z] "Multimodal basics": vision vectors replace the image-placeholder rows."""
    out = embeds_bits.copy()
    for t, r in enumerate(placeholder_rows):
        if r >= 0:
            out[r] = float_to_bf16_bits(rows[t])
    return out


def assemble(embeds_bits: np.ndarray, chunk_lo: int, chunk_hi: int, grids, span_start,
             rows: np.ndarray, sentinels_bits: np.ndarray, merge: int = 3, v4: bool = False) -> np.ndarray:
    """Embedding rows of one prefill chunk.  [Z] "Connect the complete image-to-text path":
    each image placeholder becomes the span START, (IMAGE x mw, NEWLINE) x mh, END; the
    aligner output replaces the IMAGE positions and learned vectors fill START, NEWLINE and
    END; with chunked prefill an image span may cross a chunk boundary, and a chunk replaces
    only the part of each span that lies inside it.

    ``embeds_bits`` (bf16 bits, one row per prompt position chunk_lo .. chunk_hi-1) is copied;
    image i's span starts at prompt position span_start[i]; IMAGE positions take the image's
    visual rows (image-major, as the encoder emits them) rounded to bf16; the other span
    positions take sentinels_bits[0 / 1 / 2] for START / NEWLINE / END.  With ``v4`` the spans
    follow ``layout_v4`` and its PAD positions are left as they are."""
    out = embeds_bits.copy()
    which = {TOK_START: 0, TOK_NEWLINE: 1, TOK_END: 2}
    first = 0   # first visual row of the current image
    for (gh, gw), s0 in zip(grids, span_start):
        types, src = (layout_v4 if v4 else layout)([(gh, gw)], merge)
        for k in range(len(types)):
            p = s0 + k
            if not chunk_lo <= p < chunk_hi or types[k] == TOK_PAD:
                continue
            if types[k] == TOK_IMAGE:
                out[p - chunk_lo] = float_to_bf16_bits(rows[first + src[k]])
            else:
                out[p - chunk_lo] = sentinels_bits[which[int(types[k])]]
        first += (-(-gh // merge)) * (-(-gw // merge))
    return out

