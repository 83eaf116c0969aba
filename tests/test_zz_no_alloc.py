"""vit_op_linear_noalloc, the linear entry point that allocates nothing (its split-K partials
live in the library's fixed device scratch), against vit_op_linear on the same operands: two
calls in a row, the second smaller, both with the K split that uses the scratch, plus an fp32
output and the argument checks.  Called through the C ABI."""
import ctypes

import numpy as np
import pytest

import multimodal_vision_encoder_amd as vit
import synth
from tests.gpu_util import require_gpu, seeded_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu


def noalloc_fn():
    return vit.lib().vit_op_linear_noalloc


def call_noalloc(enc, A, W, b, act, out_f32):
    import torch
    M, K = A.shape
    N = W.shape[0]
    out = torch.full((M, N), 3.0, dtype=torch.float32 if out_f32 else torch.bfloat16, device=A.device)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = noalloc_fn()(enc._ctx, p(A), M, K, p(W), p(b), N, act, 1 if out_f32 else 0, p(out),
                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, out


# (M, K, N, act, fp32 out): every shape below takes the split-K path, whose partial tiles the
# scratch holds: long-K launches under one round of 256 x 128 tiles (4 slices of 48 tiles,
# 24 MiB, then 8 slices of 16 tiles, 16 MiB); a 9216-deep fp32 projection (2 slices of 96
# tiles, 24 MiB) then the 384-token image's projector (4 slices of 64 tiles, the whole
# 32 MiB); 128 x 128 tiles with GELU (4 slices, 8 MiB then 4 MiB).
@pytest.mark.parametrize("shapes", [[(768, 4096, 2048, vit.ACT_NONE, False),
                                     (512, 4096, 1024, vit.ACT_NONE, False)],
                                    [(640, 9216, 4096, vit.ACT_NONE, True),
                                     (378, 9216, 4096, vit.ACT_NONE, True)],
                                    [(256, 2048, 2048, vit.ACT_GELU_TANH, False),
                                     (200, 2048, 1024, vit.ACT_GELU_TANH, False)]],
                         ids=["long_k_shapes", "projector_shapes_fp32", "small_tiles_gelu"])
def test_noalloc_linear_equals_linear(shapes):
    torch = require_gpu()
    cfg = synth.TINY
    enc = vit.Encoder(cfg, synth.make_weights(cfg))
    for i, (M, K, N, act, out_f32) in enumerate(shapes):
        print(f"[noalloc] call {i}: M={M} K={K} N={N} act={act} fp32={out_f32}", flush=True)
        A = to_dev_bf16(seeded_bf16((M, K), 301, i))
        W = to_dev_bf16(seeded_bf16((N, K), 301, 10 + i, std=0.02))
        b = to_dev_bf16(seeded_bf16((N,), 301, 20 + i, std=0.02))
        want = enc.op_linear(A, W, b, act, out_f32)
        st, got = call_noalloc(enc, A, W, b, act, out_f32)
        torch.cuda.synchronize()
        assert st == vit.VIT_OK, vit.lib().vit_last_error(enc._ctx)
        assert torch.equal(got.view(torch.int32) if out_f32 else got.view(torch.int16),
                           want.view(torch.int32) if out_f32 else want.view(torch.int16)), (M, K, N)
    enc.close()


def test_noalloc_linear_rejects_bad_arguments():
    torch = require_gpu()
    cfg = synth.TINY
    enc = vit.Encoder(cfg, synth.make_weights(cfg))
    A = to_dev_bf16(seeded_bf16((8, 64), 302))
    W = to_dev_bf16(seeded_bf16((16, 64), 302, 1))
    st, out = call_noalloc(enc, A, W, None, vit.ACT_GELU_TANH, True)
    assert st == vit.VIT_E_ARG
    st, _ = call_noalloc(enc, A, to_dev_bf16(seeded_bf16((24, 64), 302, 2)), None, vit.ACT_SWIGLU, False)
    assert st == vit.VIT_E_ARG
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    enc.close()
