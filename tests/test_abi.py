"""The C ABI library loads and exports every function the public headers declare; its
host-only logic (layout, sizes, argument validation) is checked without a GPU."""
import ctypes
import os
import re
from dataclasses import replace

import numpy as np
import pytest

import multimodal_vision_encoder_amd as vit
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in ("vit.h", "vit_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(vit_\w+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 17
    L = ctypes.CDLL(vit.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert names == set(vit.EXPORTS)


def test_blob_size_agrees_with_generator():
    for cfg in (synth.TINY, synth.V41, synth.V4, synth.V41_ONE_LAYER, synth.V41_OFFICIAL,
                synth.TINY_OFFICIAL, replace(synth.TINY, norm_kind=1), replace(synth.TINY, mlp_kind=1),
                replace(synth.TINY, aligner_hidden=64), replace(synth.TINY, gelu_kind=1)):
        assert vit.lib().vit_blob_elems(vit.make_config(cfg)) == cfg.blob_elems()
    for bad in (dict(hidden=100), dict(norm_kind=2), dict(mlp_kind=-1), dict(gelu_kind=3),
                dict(aligner_hidden=100), dict(aligner_hidden=-64)):
        assert vit.lib().vit_blob_elems(vit.make_config(replace(synth.TINY, **bad))) == 0, bad


@pytest.mark.parametrize("grids", [[(96, 96)], [(54, 63)], [(6, 6), (5, 7), (1, 1), (10, 4)],
                                   synth.packed_grids_batch()])
def test_layout_matches_oracle(grids):
    t, s = vit.layout(grids)
    ot, os_ = oracle.layout(grids)
    assert np.array_equal(t, ot) and np.array_equal(s, os_)


def test_layout_v41_closed_form():
    t, s = vit.layout([(96, 96)])
    assert t.size == 1058 and (t == vit.TOK_IMAGE).sum() == 1024 and (t == vit.TOK_NEWLINE).sum() == 32


def test_vt_stride():
    assert vit.vt_stride([(96, 96)]) == 9216
    assert vit.vt_stride([(5, 7), (1, 1)]) == 64 + 64
    assert vit.vt_stride([(9, 15)]) == 192


def test_create_rejects_bad_weights_without_touching_the_device():
    L = vit.lib()
    cfg = synth.TINY
    blob = synth.make_weights(cfg)
    ctx = ctypes.c_void_p()
    for bad_cfg, n in [(replace(cfg, heads=3), blob.size), (replace(cfg, merge=2), blob.size),
                       (cfg, blob.size - 1), (replace(cfg, mlp=100), blob.size),
                       (replace(cfg, pix_std=(0.5, 0.0, 0.5)), blob.size)]:
        w = vit.Weights()
        w.cfg = vit.make_config(bad_cfg)
        w.blob = blob.ctypes.data
        w.blob_elems = n
        assert L.vit_create(ctypes.byref(w), ctypes.byref(ctx)) == vit.VIT_E_ARG
        assert not ctx.value
        assert L.vit_last_error(None)
    assert L.vit_create(None, ctypes.byref(ctx)) == vit.VIT_E_ARG


def test_create_rejects_mismatched_layer_kinds():
    """A blob laid out for the official layers is refused under the LayerNorm/GELU config and
    the other way round (their sizes differ), and invalid layer kinds are refused, all before
    any device work."""
    L = vit.lib()
    ctx = ctypes.c_void_p()
    base, off = synth.TINY, synth.TINY_OFFICIAL
    for cfg, blob_cfg in ((base, off), (off, base), (replace(off, norm_kind=3), off),
                          (replace(off, aligner_hidden=100), off)):
        blob = synth.make_weights(blob_cfg)
        w = vit.Weights()
        w.cfg = vit.make_config(cfg)
        w.blob = blob.ctypes.data
        w.blob_elems = blob.size
        assert L.vit_create(ctypes.byref(w), ctypes.byref(ctx)) == vit.VIT_E_ARG
        assert not ctx.value
        assert L.vit_last_error(None)


def test_null_context_is_rejected():
    L = vit.lib()
    g = vit.grid_array([(6, 6)])
    assert L.vit_encode(None, None, g, 1, None, None) == vit.VIT_E_ARG
    assert L.vit_num_tokens(None, g, 1) == -1
    assert L.vit_overlay(None, None, 0, None, None, 0, 128, None) == vit.VIT_E_ARG
    assert L.vit_set_sentinels(None, None, 128) == vit.VIT_E_ARG
    assert L.vit_assemble(None, None, 0, 8, 128, g, 1, None, None, None) == vit.VIT_E_ARG
    assert L.vit_op_qkv_rope(None, None, None, None, g, 1, None, None, 0, None) == vit.VIT_E_ARG
    assert L.vit_op_rmsnorm(None, None, None, None, 4, 64, None, 1e-6, None, None) == vit.VIT_E_ARG
    assert L.vit_op_linear(None, None, 4, 64, None, None, 32, vit.ACT_SWIGLU, 0, None, None) == vit.VIT_E_ARG
    assert L.vit_op_merge_project(None, None, g, 1, None, None) == vit.VIT_E_ARG


def test_plan_image_matches_oracle():
    """The library's preprocessing planner (host logic) gives the oracle's integers exactly on
    seeded sizes, the workload images and degenerate ones, for the V4.1 and V4 rules."""
    from oracle import preprocess as pp
    rng = np.random.default_rng(21)
    profiles = (dict(max_tokens=1024, min_pixels=295936, max_aspect=0),
                dict(max_tokens=384, min_pixels=147456, max_aspect=8))
    sizes = [(1344, 1344), (756, 882), (1, 1), (1, 5000), (5000, 1), (14, 14), (42, 42 * 97)]
    sizes += [tuple(int(x) for x in np.exp(rng.uniform(0, np.log(8000), 2))) for _ in range(500)]
    for prof in profiles:
        for h, w in sizes:
            assert vit.plan_image(h, w, **prof) == pp.plan_image(h, w, **prof), (h, w, prof)
    with pytest.raises(vit.VitError):
        vit.plan_image(0, 10)
    with pytest.raises(vit.VitError):
        vit.plan_image(10, 10, max_tokens=0)
