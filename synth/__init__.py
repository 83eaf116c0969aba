"""Seeded synthetic inputs for the vision encoder: weights, images, grids, offsets.

This module only draws random numbers and lays them out in the agreed host
formats; it contains none of the encoder's arithmetic.  Both the CPU oracle and
the HIP library receive exactly these arrays.

Generator: SplitMix64 used counter-style (see ``synth.c``), so every tensor,
image and grid is a pure function of its seed, stream and element index.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

SEED_WEIGHTS = 0x5EED0001
SEED_PIXELS = 0x5EED0002
SEED_GRIDS = 0x5EED0003
SEED_OFFSETS = 0x5EED0004


def build(force: bool = True) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, sz, dbl, vp = ctypes.c_uint64, ctypes.c_size_t, ctypes.c_double, ctypes.c_void_p
        L.synth_u64.restype = u64
        L.synth_u64.argtypes = [u64, u64, u64]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, sz, dbl, dbl, vp]
        L.synth_normal_f32.argtypes = [u64, u64, u64, sz, dbl, dbl, vp]
        L.synth_bytes.argtypes = [u64, u64, u64, sz, vp]
        L.synth_uniform.argtypes = [u64, u64, u64, sz, vp]
        _lib = L
    return _lib


_CHUNK = 1 << 19


def _chunked(fn, n, out, *args):
    """Fill ``out`` by calling ``fn(offset, count, ptr)`` over chunks on a thread pool
    (ctypes releases the GIL; every element depends only on its own index)."""
    if n <= _CHUNK:
        fn(0, n, out.ctypes.data)
        return out
    from concurrent.futures import ThreadPoolExecutor
    starts = range(0, n, _CHUNK)
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda s: fn(s, min(_CHUNK, n - s), out.ctypes.data + s * out.itemsize),
                    starts))
    return out


def normal_bf16(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0,
                offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    return _chunked(lambda o, c, p: lib().synth_normal_bf16(seed, stream, offset + o, c,
                                                            mean, std, p), n, out)


def normal_f32(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0,
               offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    return _chunked(lambda o, c, p: lib().synth_normal_f32(seed, stream, offset + o, c,
                                                           mean, std, p), n, out)


def uniform_bytes(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    return _chunked(lambda o, c, p: lib().synth_bytes(seed, stream, offset + o, c, p), n, out)


def uniform(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform(seed, stream, offset, n, out.ctypes.data)
    return out


# --------------------------------------------------------------------------------------
# bf16 <-> fp32 bit helpers (pure data movement, used to build and inspect host arrays)
# --------------------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------
# Encoder configurations
# --------------------------------------------------------------------------------------
CLIP_MEAN = (0.48145466, 0.4578275, 0.40821073)
CLIP_STD = (0.26862954, 0.26130258, 0.27577711)


@dataclass(frozen=True)
class VitConfig:
    """Dimensions of one vision encoder plus its pixel normalisation constants."""
    layers: int = 32
    hidden: int = 1024
    heads: int = 16
    mlp: int = 4096
    patch: int = 14
    merge: int = 3
    out_hidden: int = 5120
    max_tokens_per_image: int = 1024
    ln_eps: float = 1e-6
    rope_base: float = 10000.0
    pix_mean: tuple = (0.5, 0.5, 0.5)
    pix_std: tuple = (0.5, 0.5, 0.5)
    # official-layer variant ([Z] "Comparing the DeepSeek V4.1 Flash and Qwen3-VL vision
    # towers", "Step 2", "End-to-end results"); all zero = the LayerNorm / GELU-tanh tower
    norm_kind: int = 0        # 0 LayerNorm (gamma, beta), 1 RMSNorm (gamma)
    mlp_kind: int = 0         # 0 fc1 -> GELU -> fc2, 1 SwiGLU: down(silu(gate) * up)
    gelu_kind: int = 0        # 0 tanh form, 1 erf form (MLP GELU and the aligner's GELU)
    aligner_hidden: int = 0   # 0 one projection; > 0 two, with this width between them

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def patch_dim(self) -> int:
        return 3 * self.patch * self.patch

    def tensor_shapes(self):
        """(name, shape) of every weight tensor in blob order."""
        D, F, P, Dl, m2 = self.hidden, self.mlp, self.patch_dim, self.out_hidden, self.merge ** 2
        rms = self.norm_kind == 1

        def nrm(name):
            return [(name + ".g", (D,))] + ([] if rms else [(name + ".b", (D,))])
        out = [("pe.w", (D, P)), ("pe.b", (D,))]
        for l in range(self.layers):
            out += nrm(f"l{l}.ln1")
            out += [(f"l{l}.qkv.w", (3 * D, D)), (f"l{l}.qkv.b", (3 * D,)),
                    (f"l{l}.o.w", (D, D)), (f"l{l}.o.b", (D,))]
            out += nrm(f"l{l}.ln2")
            if self.mlp_kind == 1:
                out += [(f"l{l}.gate.w", (F, D)), (f"l{l}.gate.b", (F,)),
                        (f"l{l}.up.w", (F, D)), (f"l{l}.up.b", (F,)),
                        (f"l{l}.down.w", (D, F)), (f"l{l}.down.b", (D,))]
            else:
                out += [(f"l{l}.fc1.w", (F, D)), (f"l{l}.fc1.b", (F,)),
                        (f"l{l}.fc2.w", (D, F)), (f"l{l}.fc2.b", (D,))]
        out += nrm("lnf")
        if self.aligner_hidden > 0:
            Da = self.aligner_hidden
            out += [("proj.w", (Da, m2 * D)), ("proj.b", (Da,)), ("proj2.w", (Dl, Da)), ("proj2.b", (Dl,))]
        else:
            out += [("proj.w", (Dl, m2 * D)), ("proj.b", (Dl,))]
        return out

    def blob_elems(self) -> int:
        return sum(int(np.prod(s)) for _, s in self.tensor_shapes())

    def tokens(self, gh: int, gw: int) -> int:
        m = self.merge
        return ((gh + m - 1) // m) * ((gw + m - 1) // m)


TINY = VitConfig(layers=2, hidden=64, heads=4, mlp=256, out_hidden=128, max_tokens_per_image=1024,
                 pix_mean=CLIP_MEAN, pix_std=CLIP_STD)
V41 = VitConfig()                                   # 32 layers, 1024 wide, projection to 5120
V41_ONE_LAYER = replace(V41, layers=1)
V4 = replace(V41, out_hidden=4096, max_tokens_per_image=384)
# the official-layer variant of the V4.1 tower: RMSNorm, SwiGLU MLP, erf GELU and a two-linear
# aligner whose inner width is the language hidden size (reading: the pages name the layer
# kinds, not the inner width)
V41_OFFICIAL = replace(V41, norm_kind=1, mlp_kind=1, gelu_kind=1, aligner_hidden=5120)
TINY_OFFICIAL = replace(TINY, norm_kind=1, mlp_kind=1, gelu_kind=1, aligner_hidden=192)


@dataclass
class Workload:
    """A named encoder input: configuration plus the patch grid of every image."""
    name: str
    cfg: VitConfig
    grids: list = field(default_factory=list)      # [(gh, gw), ...]
    embed_rows: int = 0                            # rows of the prompt embedding matrix (overlay)

    @property
    def n_patches(self) -> int:
        return sum(gh * gw for gh, gw in self.grids)

    @property
    def n_tokens(self) -> int:
        return sum(self.cfg.tokens(gh, gw) for gh, gw in self.grids)


# --------------------------------------------------------------------------------------
# Weights
# --------------------------------------------------------------------------------------
def make_weights(cfg: VitConfig, seed: int = SEED_WEIGHTS, perturbed: bool = False,
                 std: float = 0.02) -> np.ndarray:
    """The weight blob as bf16 bits (uint16), tensors concatenated in blob order.

    Matrices are [out][in] row-major.  Linear weights ~ N(0, std).  By default biases are 0,
    LayerNorm gamma = 1 and beta = 0; ``perturbed`` draws gamma = 1 + N(0, 0.1) and every
    beta and bias ~ N(0, 0.02), so that their indexing is exercised.
    """
    parts = []
    one = np.uint16(0x3F80)
    for stream, (name, shape) in enumerate(cfg.tensor_shapes()):
        n = int(np.prod(shape))
        kind = name.rsplit(".", 1)[1]
        if kind == "w":
            parts.append(normal_bf16(seed, stream, n, 0.0, std))
        elif kind == "g":
            parts.append(normal_bf16(seed, stream, n, 1.0, 0.1) if perturbed
                         else np.full(n, one, dtype=np.uint16))
        else:  # "b": LayerNorm beta or linear bias
            parts.append(normal_bf16(seed, stream, n, 0.0, 0.02) if perturbed
                         else np.zeros(n, dtype=np.uint16))
    return np.concatenate(parts)


def split_weights(cfg: VitConfig, blob: np.ndarray) -> dict:
    """Views into the blob by tensor name (no copies)."""
    out, off = {}, 0
    for name, shape in cfg.tensor_shapes():
        n = int(np.prod(shape))
        out[name] = blob[off:off + n].reshape(shape)
        off += n
    assert off == blob.size, (off, blob.size)
    return out


# --------------------------------------------------------------------------------------
# Images
# --------------------------------------------------------------------------------------
def make_pixels(cfg: VitConfig, grids, seed: int = SEED_PIXELS) -> np.ndarray:
    """Uniform U{0..255} uint8 images, HWC [patch*gh][patch*gw][3], packed back to back."""
    parts = []
    for i, (gh, gw) in enumerate(grids):
        n = (cfg.patch * gh) * (cfg.patch * gw) * 3
        parts.append(uniform_bytes(seed, i, n))
    return np.concatenate(parts) if parts else np.zeros(0, np.uint8)


def packed_grids_batch(seed: int = SEED_GRIDS, n_images: int = 16, merge: int = 3,
                       lo: int = 256, hi: int = 1024, max_aspect: float = 8.0,
                       total_lo: int = 7778, total_hi: int = 8704):
    """Seeded patch grids for a packed multi-image batch.

    Per image: merged-token count m log-uniform in [lo, hi] and aspect a log-uniform in
    [1/max_aspect, max_aspect]; mh = round(sqrt(m a)), mw = floor(m / mh); redraw until
    lo <= mh*mw <= hi and the aspect bound holds.  The whole batch is redrawn (next attempt
    counter) until the total merged tokens fall in [total_lo, total_hi].
    Returns [(gh, gw)] with gh = merge*mh, gw = merge*mw.
    """
    attempt = 0
    while True:
        grids, total, ctr = [], 0, 0
        for i in range(n_images):
            while True:
                u = uniform(seed, (attempt << 8) | i, 2, offset=2 * ctr)
                ctr += 1
                m = math.exp(math.log(lo) + u[0] * (math.log(hi) - math.log(lo)))
                a = math.exp(-math.log(max_aspect) + u[1] * 2 * math.log(max_aspect))
                mh = max(1, int(round(math.sqrt(m * a))))
                mw = max(1, int(m // mh))
                if lo <= mh * mw <= hi and max(mh, mw) / min(mh, mw) <= max_aspect:
                    break
            grids.append((merge * mh, merge * mw))
            total += mh * mw
        if total_lo <= total <= total_hi:
            return grids
        attempt += 1


def make_sentinels(hidden: int, seed: int = SEED_WEIGHTS, std: float = 0.02) -> np.ndarray:
    """The three learned span vectors START, NEWLINE, END as bf16 bits [3][hidden], N(0, std)
    (drawn from a stream of the weight seed that the blob does not use)."""
    return normal_bf16(seed, 1 << 20, 3 * hidden, 0.0, std).reshape(3, hidden)


def seeded_offsets(n: int, lo: int, hi: int, seed: int = SEED_OFFSETS, stream: int = 0):
    """n integers uniform in [lo, hi]."""
    u = uniform(seed, stream, n)
    return [lo + int(x * (hi - lo + 1)) for x in u]


def seeded_distinct_rows(n: int, n_rows: int, seed: int = SEED_OFFSETS, stream: int = 1):
    """n distinct row indices in [0, n_rows), by a seeded partial Fisher-Yates shuffle."""
    perm = np.arange(n_rows, dtype=np.int64)
    u = uniform(seed, stream, n)
    for i in range(n):
        j = i + int(u[i] * (n_rows - i))
        perm[i], perm[j] = perm[j], perm[i]
    return perm[:n].astype(np.int32)


# --------------------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------------------
def workload(name: str) -> Workload:
    """tiny: 84x84 image, 2-layer 64-wide encoder (6x6 patches -> 4 tokens).
    one_layer: 336x336 (24x24 -> 64 tokens), one full-width layer, 5120 projection.
    v4_384: 756x882 (54x63 -> 378 tokens), 32 layers, 4096 projection, 2048-row overlay.
    v41_1024: 1344x1344 (96x96 -> 1024 tokens), 32 layers, 5120 projection.
    packed16: 16 seeded grids (~8k tokens, >70k patches), 32 layers, 5120 projection.
    v41_official: the 1024-token image through the official-layer variant of the V4.1 tower."""
    if name == "tiny":
        return Workload(name, TINY, [(6, 6)])
    if name == "one_layer":
        return Workload(name, V41_ONE_LAYER, [(24, 24)])
    if name == "v4_384":
        return Workload(name, V4, [(54, 63)], embed_rows=2048)
    if name == "v41_1024":
        return Workload(name, V41, [(96, 96)])
    if name == "packed16":
        return Workload(name, V41, packed_grids_batch())
    if name == "v41_official":
        return Workload(name, V41_OFFICIAL, [(96, 96)])
    raise KeyError(name)


WORKLOADS = ("tiny", "one_layer", "v4_384", "v41_1024", "packed16", "v41_official")
