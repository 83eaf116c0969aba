"""Helpers shared by the GPU parity tests (host <-> device marshalling and tolerances)."""
import numpy as np

import synth


def require_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch


def raw_encode(enc, pixels, grids, out) -> int:
    """vit_encode straight through the C ABI, bypassing the binding's own tensor checks, so
    that the library's validation of grids and budgets is what is tested; returns the status."""
    import ctypes
    import torch
    import multimodal_vision_encoder_amd as vit
    return vit.lib().vit_encode(enc._ctx, ctypes.c_void_p(pixels.data_ptr()), vit.grid_array(grids),
                                len(grids), ctypes.c_void_p(out.data_ptr()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def to_dev_bf16(bits: np.ndarray):
    """uint16 bf16 bits (numpy) -> torch.bfloat16 CUDA tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev_bf16(t) -> np.ndarray:
    """torch.bfloat16 CUDA tensor -> float32 numpy (exact widening)."""
    import torch
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f32(bits).reshape(t.shape)


def qkv_after_rope(t, D: int) -> np.ndarray:
    """qkv rows after RoPE -> float32 numpy: q and v columns are bf16, the k columns
    (D .. 2D-1) hold binary16 bit patterns (the attention's score operand type)."""
    import torch
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(t.shape)
    out = synth.bf16_bits_to_f32(bits).reshape(t.shape)
    out[:, D:2 * D] = bits[:, D:2 * D].view(np.float16).astype(np.float32)
    return out


def f16_of(x: np.ndarray) -> np.ndarray:
    """float32 values -> binary16 (round to nearest even, saturating at +-65504) -> float32."""
    return np.clip(np.asarray(x, np.float32), -65504, 65504).astype(np.float16).astype(np.float32)


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """float32 values that are already bf16 -> their bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not a bf16 value"
    return (u >> 16).astype(np.uint16)


def seeded_bf16(shape, seed, stream=0, std=1.0, mean=0.0):
    n = int(np.prod(shape))
    return synth.normal_bf16(seed, stream, n, mean, std).reshape(shape)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def assert_bf16_close(got, want, ulps: float = 1.0, atol: float = 0.0, what: str = ""):
    """Every element within `ulps` bf16 ulps of the reference (a bf16 rounding decided the
    other way after a differently ordered fp32 sum moves a value by exactly one ulp)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    tol = ulps * 2.0 ** -7 * np.abs(want) + atol
    bad = np.abs(got - want) > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements off; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} want {want[tuple(i)]!r}")


def assert_projector_gate(got, want, what=""):
    """The parity gate on fp32 projector outputs: rel-L2 <= 1e-2 and max-abs <= 5e-2."""
    r = rel_l2(got, want)
    m = float(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)).max()) if np.size(want) else 0.0
    assert r <= 1e-2 and m <= 5e-2, f"{what}: rel_l2={r:.3e} max_abs={m:.3e}"
    return r, m
