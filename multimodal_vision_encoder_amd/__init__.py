"""Python binding of the MI355X (gfx950) vision encoder for DeepSeek V4 / V4.1 Flash.

Argument marshalling only: every step of the encoder runs in the HIP kernels of
``libvit.so`` behind the C ABI declared in ``include/vit.h`` and ``include/vit_ops.h``.
PyTorch supplies device memory and the current stream and nothing else.  There is no CPU
fallback: if the library is missing or the GPU call fails, these functions raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvit.so")

VIT_OK, VIT_E_ARG, VIT_E_BUDGET, VIT_E_NOMEM, VIT_E_DEVICE = 0, 1, 2, 3, 4
TOK_START, TOK_IMAGE, TOK_NEWLINE, TOK_END, TOK_PAD = 1, 2, 3, 4, 5
SPAN_V41, SPAN_V4 = 0, 1
DUMP_PATCHES, DUMP_EMBED, DUMP_QKV, DUMP_ATTN, DUMP_LAYER, DUMP_FINAL_NORM, DUMP_MERGED, DUMP_ROPE = range(8)
ACT_NONE, ACT_GELU_TANH, ACT_GELU_ERF, ACT_SWIGLU = 0, 1, 2, 3

# every entry point declared in include/vit.h and include/vit_ops.h
EXPORTS = ("vit_blob_elems", "vit_create", "vit_destroy", "vit_reserve", "vit_num_tokens",
           "vit_num_patches", "vit_encode", "vit_layout", "vit_overlay", "vit_dump",
           "vit_last_error", "vit_op_linear", "vit_op_layernorm", "vit_vt_stride", "vit_op_rope",
           "vit_op_attention", "vit_op_merge_project", "vit_timing_enable", "vit_timing_read",
           "vit_set_attention_split", "vit_op_qkv_rope", "vit_set_sentinels",
           "vit_assemble", "vit_plan_image", "vit_preprocess", "vit_op_rmsnorm",
           "vit_op_linear_noalloc", "vit_layout_v4", "vit_set_span_layout",
           "vit_op_linear_residual")
STEP_NAMES = ("patch_embed", "layernorm", "qkv", "rope", "attention", "out_proj", "fc1", "fc2",
              "projector", "overlay", "attn_merge")


class VitError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"vit status {status}: {msg}")
        self.status = status


class Grid(ctypes.Structure):
    _fields_ = [("gh", ctypes.c_int32), ("gw", ctypes.c_int32)]


class Config(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("mlp", ctypes.c_int32), ("patch", ctypes.c_int32), ("merge", ctypes.c_int32),
                ("out_hidden", ctypes.c_int32), ("max_tokens_per_image", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("pix_mean", ctypes.c_float * 3), ("pix_std", ctypes.c_float * 3),
                ("norm_kind", ctypes.c_int32), ("mlp_kind", ctypes.c_int32),
                ("gelu_kind", ctypes.c_int32), ("aligner_hidden", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("cfg", Config), ("blob", ctypes.c_void_p), ("blob_elems", ctypes.c_size_t)]


_lib = None


class ImagePlan(ctypes.Structure):
    _fields_ = [("gh", ctypes.c_int32), ("gw", ctypes.c_int32), ("canvas_h", ctypes.c_int32),
                ("canvas_w", ctypes.c_int32), ("resized_h", ctypes.c_int32), ("resized_w", ctypes.c_int32),
                ("off_y", ctypes.c_int32), ("off_x", ctypes.c_int32)]


def plan_image(height, width, patch=14, merge=3, max_tokens=1024, min_pixels=295936, max_aspect=0) -> dict:
    """vit_plan_image: token grid, canvas and contain geometry of one image."""
    p = ImagePlan()
    st = lib().vit_plan_image(int(height), int(width), int(patch), int(merge), int(max_tokens),
                              int(min_pixels), int(max_aspect), ctypes.byref(p))
    if st != VIT_OK:
        raise VitError(st, lib().vit_last_error(None).decode())
    return {k: getattr(p, k) for k, _ in ImagePlan._fields_}


def lib():
    """Load libvit.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python multimodal_vision_encoder_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        P = ctypes.POINTER
        sig = {
            "vit_blob_elems": (sz, [P(Config)]),
            "vit_create": (i32, [P(Weights), P(vp)]),
            "vit_destroy": (None, [vp]),
            "vit_reserve": (i32, [vp, i64]),
            "vit_num_tokens": (i64, [vp, P(Grid), i32]),
            "vit_num_patches": (i64, [vp, P(Grid), i32]),
            "vit_encode": (i32, [vp, vp, P(Grid), i32, vp, vp]),
            "vit_layout": (i32, [P(Grid), i32, i32, vp, vp, P(i64)]),
            "vit_layout_v4": (i32, [P(Grid), i32, i32, vp, vp, P(i64)]),
            "vit_set_span_layout": (i32, [vp, i32]),
            "vit_overlay": (i32, [vp, vp, i64, vp, vp, i64, i32, vp]),
            "vit_dump": (i32, [vp, i32, i32, vp, P(Grid), i32, vp, sz, vp]),
            "vit_last_error": (ctypes.c_char_p, [vp]),
            "vit_op_linear": (i32, [vp, vp, i64, i32, vp, vp, i32, i32, i32, vp, vp]),
            "vit_op_linear_noalloc": (i32, [vp, vp, i64, i32, vp, vp, i32, i32, i32, vp, vp]),
            "vit_op_linear_residual": (i32, [vp, vp, i64, i32, vp, vp, i32, vp, vp]),
            "vit_op_layernorm": (i32, [vp, vp, vp, vp, i64, i32, vp, vp, ctypes.c_float, vp, vp]),
            "vit_op_rmsnorm": (i32, [vp, vp, vp, vp, i64, i32, vp, ctypes.c_float, vp, vp]),
            "vit_vt_stride": (i64, [P(Grid), i32]),
            "vit_op_rope": (i32, [vp, vp, vp, P(Grid), i32, vp]),
            "vit_op_qkv_rope": (i32, [vp, vp, vp, vp, P(Grid), i32, vp, vp, i32, vp]),
            "vit_set_sentinels": (i32, [vp, vp, i32]),
            "vit_plan_image": (i32, [i32, i32, i32, i32, i32, i64, i32, P(ImagePlan)]),
            "vit_preprocess": (i32, [vp, vp, i32, i32, P(ImagePlan), vp, vp]),
            "vit_assemble": (i32, [vp, vp, i64, i64, i32, P(Grid), i32, vp, vp, vp]),
            "vit_op_attention": (i32, [vp, vp, vp, P(Grid), i32, vp, vp]),
            "vit_op_merge_project": (i32, [vp, vp, P(Grid), i32, vp, vp]),
            "vit_timing_enable": (i32, [vp, i32]),
            "vit_timing_read": (i32, [vp, vp, vp]),
            "vit_set_attention_split": (i32, [vp, i32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def make_config(cfg) -> Config:
    """vit_config from any object with the encoder's dimension attributes."""
    c = Config()
    for f in ("layers", "hidden", "heads", "mlp", "patch", "merge", "out_hidden",
              "max_tokens_per_image"):
        setattr(c, f, int(getattr(cfg, f)))
    c.ln_eps = float(cfg.ln_eps)
    c.rope_base = float(cfg.rope_base)
    for i in range(3):
        c.pix_mean[i] = float(cfg.pix_mean[i])
        c.pix_std[i] = float(cfg.pix_std[i])
    for f in ("norm_kind", "mlp_kind", "gelu_kind", "aligner_hidden"):
        setattr(c, f, int(getattr(cfg, f, 0)))
    return c


def swiglu_interleave(gate, up):
    """The ACT_SWIGLU operand layout from gate and up tensors of F rows each (weights [F][K]
    or biases [F]): rows 16j .. 16j+7 = gate rows 8j .. 8j+7, rows 16j+8 .. 16j+15 = up rows
    8j .. 8j+7.  Works on numpy arrays and torch tensors (a pure row permutation)."""
    F = gate.shape[0]
    assert up.shape == gate.shape and F % 8 == 0
    rest = tuple(gate.shape[1:])
    g = gate.reshape((F // 8, 8) + rest)
    u = up.reshape((F // 8, 8) + rest)
    if hasattr(gate, "new_empty"):
        import torch
        return torch.stack([g, u], dim=1).reshape((2 * F,) + rest)
    return np.stack([g, u], axis=1).reshape((2 * F,) + rest)


def grid_array(grids):
    arr = (Grid * max(1, len(grids)))()
    for i, (gh, gw) in enumerate(grids):
        arr[i].gh, arr[i].gw = int(gh), int(gw)
    return arr


def layout(grids, merge: int = 3, span=SPAN_V41):
    """Span layout (types, src) of a batch, as int32 numpy arrays (vit_layout, or vit_layout_v4
    with span=SPAN_V4)."""
    L = lib()
    fn = L.vit_layout_v4 if span == SPAN_V4 else L.vit_layout
    g = grid_array(grids)
    n = ctypes.c_int64(0)
    st = fn(g, len(grids), merge, None, None, ctypes.byref(n))
    if st != VIT_OK:
        raise VitError(st, L.vit_last_error(None).decode())
    types = np.zeros(n.value, np.int32)
    src = np.zeros(n.value, np.int32)
    st = fn(g, len(grids), merge, types.ctypes.data, src.ctypes.data, ctypes.byref(n))
    if st != VIT_OK:
        raise VitError(st, L.vit_last_error(None).decode())
    return types, src


def vt_stride(grids) -> int:
    return int(lib().vit_vt_stride(grid_array(grids), len(grids)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def check_tensor(t, name, dtype, shape=None, numel=None, optional=False, gpu=True):
    """Refuse a tensor the kernels would read or write out of bounds: wrong dtype, not
    contiguous, wrong shape or element count, or (with gpu) not on a GPU (ValueError).  The
    checks run in that order, so the host-side ones can be exercised without a GPU."""
    import torch
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is None")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != int(numel):
        raise ValueError(f"{name} must hold {int(numel)} elements, got {t.numel()}")
    if gpu:
        on_gpu(**{name: t})


def on_gpu(**tensors):
    """ValueError unless every given tensor (None entries skipped) lives on a GPU."""
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU, got {t.device}")


def batch_sizes(grids, patch: int, merge: int = 3):
    """(patches, merged tokens, pixel bytes) of a batch of (gh, gw) grids: sum of gh*gw, of
    ceil(gh/merge)*ceil(gw/merge) and of 3*(patch*gh)*(patch*gw).  ValueError on a grid side
    below 1 (the library validates the rest)."""
    n = m = px = 0
    for gh, gw in grids:
        gh, gw = int(gh), int(gw)
        if gh < 1 or gw < 1:
            raise ValueError(f"grid {gh}x{gw}: sides must be >= 1")
        n += gh * gw
        m += -(-gh // merge) * -(-gw // merge)
        px += 3 * patch * gh * patch * gw
    return n, m, px


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Encoder:
    """A vision-encoder context on the current GPU (weights uploaded once)."""

    def __init__(self, cfg, blob: np.ndarray):
        L = lib()
        self.cfg = cfg
        self.out_hidden = int(cfg.out_hidden)
        blob = np.ascontiguousarray(blob, dtype=np.uint16)
        w = Weights()
        w.cfg = make_config(cfg)
        w.blob = blob.ctypes.data
        w.blob_elems = blob.size
        ctx = ctypes.c_void_p()
        st = L.vit_create(ctypes.byref(w), ctypes.byref(ctx))
        if st != VIT_OK:
            raise VitError(st, L.vit_last_error(None).decode())
        self._ctx = ctx

    def close(self):
        if getattr(self, "_ctx", None):
            lib().vit_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st):
        if st != VIT_OK:
            raise VitError(st, lib().vit_last_error(self._ctx).decode())

    # ---- queries ---------------------------------------------------------------------
    def num_tokens(self, grids) -> int:
        return int(lib().vit_num_tokens(self._ctx, grid_array(grids), len(grids)))

    def num_patches(self, grids) -> int:
        return int(lib().vit_num_patches(self._ctx, grid_array(grids), len(grids)))

    def reserve(self, max_patches: int):
        self._check(lib().vit_reserve(self._ctx, int(max_patches)))

    def timing(self, enable: bool):
        self._check(lib().vit_timing_enable(self._ctx, 1 if enable else 0))

    def timing_read(self):
        """{step: (total ms, launches)} since the last read (waits for the recorded events)."""
        ms = np.zeros(len(STEP_NAMES), np.float32)
        n = np.zeros(len(STEP_NAMES), np.int64)
        self._check(lib().vit_timing_read(self._ctx, ms.ctypes.data, n.ctypes.data))
        return {k: (float(ms[i]), int(n[i])) for i, k in enumerate(STEP_NAMES)}

    # ---- the encoder -----------------------------------------------------------------
    def encode(self, pixels, grids, out=None, stream=None):
        """pixels: uint8 CUDA tensor (packed HWC images); returns fp32 [tokens][out_hidden]."""
        import torch
        _, M, npx = batch_sizes(grids, int(self.cfg.patch), int(self.cfg.merge))
        check_tensor(pixels, "pixels", torch.uint8, numel=npx, gpu=False)
        if out is None:
            out = torch.empty((M, self.out_hidden), dtype=torch.float32, device=pixels.device)
        check_tensor(out, "out", torch.float32, shape=(M, self.out_hidden), gpu=False)
        on_gpu(pixels=pixels, out=out)
        self._check(lib().vit_encode(self._ctx, _ptr(pixels), grid_array(grids), len(grids),
                                     _ptr(out), _stream(stream)))
        return out

    def dump(self, boundary: int, pixels, grids, arg: int = 0, stream=None):
        import torch
        D, ps = int(self.cfg.hidden), int(self.cfg.patch)
        N, M, npx = batch_sizes(grids, ps, int(self.cfg.merge))
        check_tensor(pixels, "pixels", torch.uint8, numel=npx)
        if boundary == DUMP_ROPE:   # fp32 [N][hd]: cos of the hd/2 angles, then their sin
            dst = torch.empty((N, D // int(self.cfg.heads)), dtype=torch.float32, device=pixels.device)
            self._check(lib().vit_dump(self._ctx, boundary, arg, _ptr(pixels), grid_array(grids),
                                       len(grids), _ptr(dst), dst.numel() * 4, _stream(stream)))
            return dst
        shape = {DUMP_PATCHES: (N, 3 * ps * ps), DUMP_EMBED: (N, D), DUMP_QKV: (N, 3 * D),
                 DUMP_ATTN: (N, D), DUMP_LAYER: (N, D), DUMP_FINAL_NORM: (N, D),
                 DUMP_MERGED: (M, 9 * D)}[boundary]
        dst = torch.empty(shape, dtype=torch.bfloat16, device=pixels.device)
        self._check(lib().vit_dump(self._ctx, boundary, arg, _ptr(pixels), grid_array(grids),
                                   len(grids), _ptr(dst), dst.numel() * 2, _stream(stream)))
        return dst

    def overlay(self, embeds, rows, visual_rows, stream=None):
        """embeds: bf16 CUDA tensor [R][out_hidden] (modified in place); rows: host ints
        (negative = skip); visual_rows: fp32 CUDA tensor [len(rows)][out_hidden]."""
        import torch
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1))
        if embeds is None or embeds.dim() != 2:
            raise ValueError("embeds must be a 2-D tensor [rows][out_hidden]")
        check_tensor(embeds, "embeds", torch.bfloat16, shape=(embeds.shape[0], self.out_hidden), gpu=False)
        check_tensor(visual_rows, "visual_rows", torch.float32, shape=(r.size, self.out_hidden), gpu=False)
        on_gpu(embeds=embeds, visual_rows=visual_rows)
        self._check(lib().vit_overlay(self._ctx, _ptr(embeds), embeds.shape[0], r.ctypes.data,
                                      _ptr(visual_rows), r.size, int(embeds.shape[1]),
                                      _stream(stream)))
        return embeds

    def preprocess(self, src, height, width, plan: dict, stream=None):
        """The gray canvas of `plan` (uint8 CUDA tensor [canvas_h][canvas_w][3]) from src (uint8
        CUDA tensor, HWC height x width x 3)."""
        import torch
        check_tensor(src, "src", torch.uint8, numel=int(height) * int(width) * 3)
        p = ImagePlan(**plan)
        canvas = torch.empty((plan["canvas_h"], plan["canvas_w"], 3), dtype=torch.uint8, device=src.device)
        self._check(lib().vit_preprocess(self._ctx, _ptr(src), int(height), int(width), ctypes.byref(p),
                                         _ptr(canvas), _stream(stream)))
        return canvas

    def set_span_layout(self, span: int):
        """Span geometry of assemble(): SPAN_V41 or SPAN_V4 (starts at multiples of 4)."""
        self._check(lib().vit_set_span_layout(self._ctx, int(span)))

    def set_sentinels(self, sentinels: np.ndarray):
        """Learned START, NEWLINE, END rows: bf16 bits [3][out_hidden] (host)."""
        s = np.ascontiguousarray(sentinels, dtype=np.uint16)
        assert s.shape == (3, self.out_hidden)
        self._check(lib().vit_set_sentinels(self._ctx, s.ctypes.data, self.out_hidden))

    def assemble(self, chunk, chunk_lo, grids, span_start, visual_rows, stream=None):
        """Write the span positions inside [chunk_lo, chunk_lo + len(chunk)) into chunk (bf16
        CUDA tensor [rows][out_hidden], row j = prompt position chunk_lo + j)."""
        import torch
        st = np.ascontiguousarray(np.asarray(span_start, dtype=np.int64).reshape(-1))
        if len(st) != len(grids):
            raise ValueError("span_start needs one entry per image")
        _, M, _ = batch_sizes(grids, int(self.cfg.patch), int(self.cfg.merge))
        if chunk is None or chunk.dim() != 2:
            raise ValueError("chunk must be a 2-D tensor [rows][out_hidden]")
        check_tensor(chunk, "chunk", torch.bfloat16, shape=(chunk.shape[0], self.out_hidden), gpu=False)
        check_tensor(visual_rows, "visual_rows", torch.float32, shape=(M, self.out_hidden), gpu=False)
        on_gpu(chunk=chunk, visual_rows=visual_rows)
        self._check(lib().vit_assemble(self._ctx, _ptr(chunk), int(chunk_lo),
                                       int(chunk_lo) + int(chunk.shape[0]), int(chunk.shape[1]),
                                       grid_array(grids), len(grids), st.ctypes.data,
                                       _ptr(visual_rows), _stream(stream)))
        return chunk

    # ---- single steps (include/vit_ops.h) ---------------------------------------------
    def op_linear(self, A, W, b, act=ACT_NONE, out_f32=False, stream=None):
        """act = ACT_SWIGLU takes W, b in the swiglu_interleave layout and returns [M][N/2]."""
        import torch
        if A is None or A.dim() != 2 or W is None or W.dim() != 2:
            raise ValueError("A and W must be 2-D tensors")
        M, K = A.shape
        N = W.shape[0]
        check_tensor(A, "A", torch.bfloat16, shape=(M, K), gpu=False)
        check_tensor(W, "W", torch.bfloat16, shape=(N, K), gpu=False)
        check_tensor(b, "b", torch.bfloat16, shape=(N,), optional=True, gpu=False)
        on_gpu(A=A, W=W, b=b)
        n_out = N // 2 if act == ACT_SWIGLU else N
        out = torch.empty((M, n_out), dtype=torch.float32 if out_f32 else torch.bfloat16, device=A.device)
        self._check(lib().vit_op_linear(self._ctx, _ptr(A), M, K, _ptr(W), _ptr(b), N, act,
                                        1 if out_f32 else 0, _ptr(out), _stream(stream)))
        return out

    def op_linear_residual(self, A, W, b, x, stream=None):
        """x = bf16(x + bf16(A W^T + b)) in place on x; returns x."""
        import torch
        if A is None or A.dim() != 2 or W is None or W.dim() != 2:
            raise ValueError("A and W must be 2-D tensors")
        M, K = A.shape
        N = W.shape[0]
        check_tensor(A, "A", torch.bfloat16, shape=(M, K), gpu=False)
        check_tensor(W, "W", torch.bfloat16, shape=(N, K), gpu=False)
        check_tensor(b, "b", torch.bfloat16, shape=(N,), optional=True, gpu=False)
        check_tensor(x, "x", torch.bfloat16, shape=(M, N), gpu=False)
        on_gpu(A=A, W=W, b=b, x=x)
        self._check(lib().vit_op_linear_residual(self._ctx, _ptr(A), M, K, _ptr(W), _ptr(b), N, _ptr(x),
                                                 _stream(stream)))
        return x

    def op_layernorm(self, x, g, b, eps, delta=None, xout=None, out=None, stream=None):
        import torch
        M, D = self._check_rows(x, delta, xout)
        check_tensor(g, "g", torch.bfloat16, shape=(D,), gpu=False)
        check_tensor(b, "b", torch.bfloat16, shape=(D,), gpu=False)
        check_tensor(out, "out", torch.bfloat16, shape=x.shape, optional=True, gpu=False)
        on_gpu(x=x, delta=delta, xout=xout, g=g, b=b, out=out)
        if out is None:
            out = torch.empty_like(x)
        self._check(lib().vit_op_layernorm(self._ctx, _ptr(x), _ptr(delta), _ptr(xout), M, D,
                                           _ptr(g), _ptr(b), float(eps), _ptr(out),
                                           _stream(stream)))
        return out

    @staticmethod
    def _check_rows(x, delta, xout):
        import torch
        if x is None or x.dim() != 2:
            raise ValueError("x must be a 2-D tensor [rows][D]")
        check_tensor(x, "x", torch.bfloat16, shape=x.shape, gpu=False)
        check_tensor(delta, "delta", torch.bfloat16, shape=x.shape, optional=True, gpu=False)
        check_tensor(xout, "xout", torch.bfloat16, shape=x.shape, optional=delta is None, gpu=False)
        return x.shape

    def op_rmsnorm(self, x, g, eps, delta=None, xout=None, stream=None):
        import torch
        M, D = self._check_rows(x, delta, xout)
        check_tensor(g, "g", torch.bfloat16, shape=(D,), gpu=False)
        on_gpu(x=x, delta=delta, xout=xout, g=g)
        out = torch.empty_like(x)
        self._check(lib().vit_op_rmsnorm(self._ctx, _ptr(x), _ptr(delta), _ptr(xout), M, D,
                                         _ptr(g), float(eps), _ptr(out), _stream(stream)))
        return out

    def op_rope(self, qkv, grids, stream=None):
        """In place on qkv (q bf16, k then binary16); returns the transposed-V buffer
        (torch.float16)."""
        import torch
        H, D = int(self.cfg.heads), int(self.cfg.hidden)
        N, _, _ = batch_sizes(grids, int(self.cfg.patch), int(self.cfg.merge))
        check_tensor(qkv, "qkv", torch.bfloat16, shape=(N, 3 * D))
        vt = torch.empty((H, D // H, vt_stride(grids)), dtype=torch.float16, device=qkv.device)
        self._check(lib().vit_op_rope(self._ctx, _ptr(qkv), _ptr(vt), grid_array(grids),
                                      len(grids), _stream(stream)))
        return vt

    def op_qkv_rope(self, x, W, b, grids, store_v=False, stream=None):
        """Fused QKV projection + RoPE + V^T relayout; returns (qkv bf16 [N][3D] with k as
        binary16 bits and v only with store_v, vt torch.float16 [H][hd][vt_stride])."""
        import torch
        H, D = int(self.cfg.heads), int(self.cfg.hidden)
        N, _, _ = batch_sizes(grids, int(self.cfg.patch), int(self.cfg.merge))
        check_tensor(x, "x", torch.bfloat16, shape=(N, D), gpu=False)
        check_tensor(W, "W", torch.bfloat16, shape=(3 * D, D), gpu=False)
        check_tensor(b, "b", torch.bfloat16, shape=(3 * D,), optional=True, gpu=False)
        on_gpu(x=x, W=W, b=b)
        qkv = torch.zeros((x.shape[0], 3 * D), dtype=torch.bfloat16, device=x.device)
        vt = torch.empty((H, D // H, vt_stride(grids)), dtype=torch.float16, device=x.device)
        self._check(lib().vit_op_qkv_rope(self._ctx, _ptr(x), _ptr(W), _ptr(b), grid_array(grids),
                                          len(grids), _ptr(qkv), _ptr(vt), 1 if store_v else 0,
                                          _stream(stream)))
        return qkv, vt

    def set_attention_split(self, n):
        """Key slices of the attention: 0 = chosen per batch, 1..4 = fixed."""
        self._check(lib().vit_set_attention_split(self._ctx, int(n)))

    def op_attention(self, qkv, vt, grids, stream=None):
        import torch
        H, D = int(self.cfg.heads), int(self.cfg.hidden)
        N, _, _ = batch_sizes(grids, int(self.cfg.patch), int(self.cfg.merge))
        check_tensor(qkv, "qkv", torch.bfloat16, shape=(N, 3 * D), gpu=False)
        check_tensor(vt, "vt", torch.float16, shape=(H, D // H, vt_stride(grids)), gpu=False)
        on_gpu(qkv=qkv, vt=vt)
        o = torch.empty((qkv.shape[0], int(self.cfg.hidden)), dtype=torch.bfloat16, device=qkv.device)
        self._check(lib().vit_op_attention(self._ctx, _ptr(qkv), _ptr(vt), grid_array(grids),
                                           len(grids), _ptr(o), _stream(stream)))
        return o

    def op_merge_project(self, y, grids, stream=None):
        import torch
        N, M, _ = batch_sizes(grids, int(self.cfg.patch), int(self.cfg.merge))
        check_tensor(y, "y", torch.bfloat16, shape=(N, int(self.cfg.hidden)))
        out = torch.empty((M, self.out_hidden), dtype=torch.float32, device=y.device)
        self._check(lib().vit_op_merge_project(self._ctx, _ptr(y), grid_array(grids), len(grids),
                                               _ptr(out), _stream(stream)))
        return out
