"""The Python binding refuses tensors that the kernels would read or write out of bounds, before
any call into the library (CPU tests: the checks run before the device check, and the device
check refuses host tensors)."""
import numpy as np
import pytest
import torch

import multimodal_vision_encoder_amd as vit
import synth


def host_encoder(cfg=synth.TINY):
    """An Encoder object without a device context: enough to run the binding's checks."""
    enc = object.__new__(vit.Encoder)
    enc.cfg = cfg
    enc.out_hidden = int(cfg.out_hidden)
    enc._ctx = None
    return enc


def test_batch_sizes():
    assert vit.batch_sizes([(6, 6), (5, 7)], 14) == (36 + 35, 4 + 6, 3 * 14 * 14 * (36 + 35))
    assert vit.batch_sizes([], 14) == (0, 0, 0)
    with pytest.raises(ValueError):
        vit.batch_sizes([(6, 0)], 14)


def test_check_tensor_order_and_messages():
    t = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="bfloat16"):
        vit.check_tensor(t, "x", torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous"):
        vit.check_tensor(t.T, "x", torch.float32)
    with pytest.raises(ValueError, match="shape"):
        vit.check_tensor(t, "x", torch.float32, shape=(4, 9))
    with pytest.raises(ValueError, match="elements"):
        vit.check_tensor(t, "x", torch.float32, numel=33)
    with pytest.raises(ValueError, match="GPU"):
        vit.check_tensor(t, "x", torch.float32, shape=(4, 8), numel=32)
    with pytest.raises(ValueError, match="None"):
        vit.check_tensor(None, "x", torch.float32)
    vit.check_tensor(None, "x", torch.float32, optional=True)
    with pytest.raises(ValueError, match="torch tensor"):
        vit.check_tensor(np.zeros(3), "x", torch.float32)


def test_encode_refusals():
    enc = host_encoder()
    grids = [(6, 6)]
    n_px = 3 * 84 * 84
    px = torch.zeros(n_px, dtype=torch.uint8)
    out = torch.zeros((4, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="uint8"):
        enc.encode(px.to(torch.int16), grids, out=out)
    with pytest.raises(ValueError, match="elements"):
        enc.encode(px[:-1], grids, out=out)
    with pytest.raises(ValueError, match="elements"):
        enc.encode(torch.zeros(n_px + 3, dtype=torch.uint8), grids, out=out)
    with pytest.raises(ValueError, match="sides"):
        enc.encode(px, [(6, 6), (0, 3)], out=out)
    with pytest.raises(ValueError, match="GPU"):       # right size, but a host tensor
        enc.encode(px, grids, out=out)


def test_encode_out_refusals(monkeypatch):
    """The output checks, with the pixel check passed (a stand-in that skips the device test)."""
    enc = host_encoder()
    real = vit.check_tensor

    def host_ok(t, name, *a, **k):
        if name == "pixels":
            return
        return real(t, name, *a, **k)
    monkeypatch.setattr(vit, "check_tensor", host_ok)
    px = torch.zeros(3 * 84 * 84, dtype=torch.uint8)
    with pytest.raises(ValueError, match="float32"):
        enc.encode(px, [(6, 6)], out=torch.zeros((4, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        enc.encode(px, [(6, 6)], out=torch.zeros((3, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        enc.encode(px, [(6, 6)], out=torch.zeros((4, 64), dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        enc.encode(px, [(6, 6)], out=torch.zeros((128, 4), dtype=torch.float32).T)


def test_dump_refusals():
    enc = host_encoder()
    with pytest.raises(ValueError, match="elements"):
        enc.dump(vit.DUMP_EMBED, torch.zeros(10, dtype=torch.uint8), [(6, 6)])


def test_overlay_refusals():
    enc = host_encoder()
    emb = torch.zeros((8, 128), dtype=torch.bfloat16)
    rows = torch.zeros((2, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="bfloat16"):
        enc.overlay(emb.float(), [0, 1], rows)
    with pytest.raises(ValueError, match="shape"):
        enc.overlay(torch.zeros((8, 64), dtype=torch.bfloat16), [0, 1], rows)
    with pytest.raises(ValueError, match="2-D"):
        enc.overlay(torch.zeros(8 * 128, dtype=torch.bfloat16), [0, 1], rows)
    with pytest.raises(ValueError, match="float32"):
        enc.overlay(emb, [0, 1], rows.to(torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        enc.overlay(emb, [0, 1, 2], rows)
    with pytest.raises(ValueError, match="contiguous"):
        enc.overlay(emb, [0, 1], torch.zeros((128, 2), dtype=torch.float32).T)


def test_assemble_and_preprocess_refusals():
    enc = host_encoder()
    chunk = torch.zeros((16, 128), dtype=torch.bfloat16)
    rows = torch.zeros((4, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="span_start"):
        enc.assemble(chunk, 0, [(6, 6)], [0, 5], rows)
    with pytest.raises(ValueError, match="shape"):
        enc.assemble(chunk, 0, [(6, 6)], [0], torch.zeros((5, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="bfloat16"):
        enc.assemble(chunk.float(), 0, [(6, 6)], [0], rows)
    with pytest.raises(ValueError, match="elements"):
        enc.preprocess(torch.zeros(10, dtype=torch.uint8), 4, 4, {})


def test_op_refusals():
    enc = host_encoder()
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        enc.op_linear(bf(8, 64), bf(16, 128), None)
    with pytest.raises(ValueError, match="shape"):
        enc.op_linear(bf(8, 64), bf(16, 64), bf(15))
    with pytest.raises(ValueError, match="bfloat16"):
        enc.op_linear(bf(8, 64).float(), bf(16, 64), None)
    with pytest.raises(ValueError, match="contiguous"):
        enc.op_linear(bf(64, 8).T, bf(16, 64), None)
    with pytest.raises(ValueError, match="shape"):
        enc.op_layernorm(bf(8, 64), bf(64), bf(63), 1e-6)
    with pytest.raises(ValueError, match="shape"):
        enc.op_layernorm(bf(8, 64), bf(64), bf(64), 1e-6, delta=bf(7, 64), xout=bf(8, 64))
    with pytest.raises(ValueError, match="None"):
        enc.op_rmsnorm(bf(8, 64), bf(64), 1e-6, delta=bf(8, 64))
    grids = [(2, 3)]
    with pytest.raises(ValueError, match="shape"):
        enc.op_rope(bf(6, 64), grids)
    with pytest.raises(ValueError, match="shape"):
        enc.op_qkv_rope(bf(5, 64), bf(192, 64), None, grids)
    with pytest.raises(ValueError, match="float16"):
        enc.op_attention(bf(6, 192), bf(4, 16, 64), grids)
    with pytest.raises(ValueError, match="shape"):
        enc.op_attention(bf(6, 192), torch.zeros((4, 16, 63), dtype=torch.float16), grids)
    with pytest.raises(ValueError, match="shape"):
        enc.op_merge_project(bf(5, 64), grids)
