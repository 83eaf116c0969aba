"""Full-size end-to-end parity: the 32-layer workloads (and the 1024-token image through the
official-layer variant of the tower) on the GPU against rows written by the CPU oracle
(``tests/golden/make_golden.py``, which calls only the oracle and the seeded generator), plus
the overlay of those workloads into prompt embedding matrices.

Two gates:

* after the first block (full width, full sequence length): the GPU residual stream against
  the fp32 oracle within rel-L2 1e-2 and max-abs 5e-2;
* after all 32 blocks: the projector rows against the fp32 oracle within 1.5 times the spread
  between the fp32 oracle and its fp64 twin on the same rows.  Both compute the same steps
  with the same bf16 rounding points and differ only in the arithmetic between them, yet
  they end up rel-L2 ~1.4e-2 and max-abs ~0.12 apart: a value that lands next to a bf16
  rounding boundary rounds differently under any other summation order, and the residual
  stream carries and amplifies such flips through 32 blocks.  The GPU (MFMA accumulation
  order) can be no closer to the fp32 oracle than an exact implementation is, so its
  deviation is gated against that spread; the stated rel-L2 <= 1e-2 / max-abs <= 5e-2 is
  reported next to it.
"""
import os

import numpy as np
import pytest

import multimodal_vision_encoder_amd as vit
import oracle
import synth
from tests.gpu_util import assert_projector_gate, from_dev_bf16, rel_l2, require_gpu

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def golden(name):
    path = os.path.join(HERE, "golden", f"oracle_{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_golden.py {name}")
    return np.load(path)


_runs = {}


def encoded(name):
    """(workload, encoder, device pixels, fp32 rows on the GPU) for a workload, cached."""
    if name not in _runs:
        torch = require_gpu()
        wl = synth.workload(name)
        enc = vit.Encoder(wl.cfg, synth.make_weights(wl.cfg))
        px = torch.from_numpy(synth.make_pixels(wl.cfg, wl.grids)).cuda()
        out = enc.encode(px, wl.grids)
        torch.cuda.synchronize()
        _runs[name] = (wl, enc, px, out)
    return _runs[name]


@pytest.mark.parametrize("name", ["v4_384", "v41_1024", "packed16", "v41_official"])
def test_full_size_rows_match_oracle(name):
    torch = require_gpu()
    g = golden(name)
    wl, enc, px, out = encoded(name)
    assert [tuple(x) for x in g["grids"]] == [tuple(x) for x in wl.grids]
    assert out.shape == (wl.n_tokens, wl.cfg.out_hidden)
    got = out[torch.as_tensor(g["rows"], device=out.device)].cpu().numpy()
    assert np.isfinite(got).all()
    ref, ref64 = g["values"].astype(np.float64), g["values64"]
    floor_rel, floor_max = rel_l2(ref64, ref), float(np.abs(ref64 - ref).max())
    err_rel, err_max = rel_l2(got, ref), float(np.abs(got - ref).max())
    print(f"{name}: GPU vs fp32 oracle rel_l2={err_rel:.3e} max_abs={err_max:.3e}; "
          f"fp64 vs fp32 oracle rel_l2={floor_rel:.3e} max_abs={floor_max:.3e}; "
          f"GPU vs fp64 oracle rel_l2={rel_l2(got, ref64):.3e}")
    assert err_rel <= 1.5 * floor_rel and err_max <= 1.5 * floor_max, \
        (name, err_rel, floor_rel, err_max, floor_max)


@pytest.mark.parametrize("name", ["v4_384", "v41_1024", "packed16", "v41_official"])
def test_full_size_first_block_matches_oracle(name):
    """Residual stream after the first block, every image at full length, on sampled rows."""
    torch = require_gpu()
    g = golden(name)
    wl, enc, px, _ = encoded(name)
    x1 = enc.dump(vit.DUMP_LAYER, px, wl.grids, 0)
    torch.cuda.synchronize()
    got = from_dev_bf16(x1[torch.as_tensor(g["layer0_rows"], device=x1.device)])
    assert_projector_gate(got, g["layer0_values"], f"{name} first block")


def test_v41_token_stream_layout():
    """1344x1344 -> 1024 tokens; the span is START, 32 x (32 IMAGE + NEWLINE), END."""
    wl, enc, _, out = encoded("v41_1024")
    types, src = vit.layout(wl.grids)
    assert out.shape[0] == 1024 == (types == vit.TOK_IMAGE).sum()
    assert types.size == 1058 and types[0] == vit.TOK_START and types[-1] == vit.TOK_END
    assert (types[1 + 32::33] == vit.TOK_NEWLINE).all()


@pytest.mark.parametrize("placement", ["span", "scattered"])
def test_v4_overlay_into_prompt(placement):
    """The 378 visual rows replace placeholder rows of a seeded 2048 x 4096 bf16 prompt: at
    the IMAGE positions of a span starting at a seeded offset, then at 378 seeded distinct
    rows.  Untouched rows stay bitwise; overlaid rows are the round-to-nearest-even bf16 of
    the visual rows (torch conversion as the reference)."""
    torch = require_gpu()
    wl, enc, _, out = encoded("v4_384")
    R, Dl = wl.embed_rows, wl.cfg.out_hidden
    emb0 = synth.normal_bf16(synth.SEED_OFFSETS, 5, R * Dl).reshape(R, Dl)
    types, src = vit.layout(wl.grids)
    if placement == "span":
        start = synth.seeded_offsets(1, 0, R - types.size)[0]
        rows = np.full(out.shape[0], -1, np.int32)
        img = np.nonzero(types == vit.TOK_IMAGE)[0]
        rows[src[img]] = start + img
    else:
        rows = synth.seeded_distinct_rows(out.shape[0], R)
    d_emb = torch.from_numpy(emb0.view(np.int16)).cuda().view(torch.bfloat16)
    enc.overlay(d_emb, rows, out)
    torch.cuda.synchronize()
    got = d_emb.view(torch.int16).cpu().numpy().view(np.uint16)
    touched = np.zeros(R, bool)
    touched[rows[rows >= 0]] = True
    assert np.array_equal(got[~touched], emb0[~touched])
    want = out.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[rows], want)


def test_packed16_overlay_into_one_prompt():
    """All 8k visual rows of the packed batch go to the IMAGE positions of one packed prompt
    (text rows between spans); every IMAGE row gets its own visual row, nothing else moves."""
    torch = require_gpu()
    wl, enc, _, out = encoded("packed16")
    types, src = vit.layout(wl.grids)
    text = 16
    R = types.size + text
    rows = np.full(out.shape[0], -1, np.int32)
    img = np.nonzero(types == vit.TOK_IMAGE)[0]
    rows[src[img]] = text + img
    emb = torch.zeros((R, wl.cfg.out_hidden), dtype=torch.bfloat16, device="cuda")
    enc.overlay(emb, rows, out)
    torch.cuda.synchronize()
    e = emb.float().cpu().numpy()
    want = out.to(torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(e[text + img], want[src[img]])
    others = np.ones(R, bool)
    others[text + img] = False
    assert not e[others].any()


def test_packed16_assemble_in_chunks():
    """The packed batch's 8k visual rows and learned span rows assembled into one prompt (text
    runs between spans) in prefill chunks of 1024 positions, the pages' cap with a projector
    loaded: bitwise the oracle's assembly of the same rows."""
    torch = require_gpu()
    wl, enc, _, out = encoded("packed16")
    Dl = wl.cfg.out_hidden
    sent = synth.make_sentinels(Dl)
    enc.set_sentinels(sent)
    gaps = synth.seeded_offsets(len(wl.grids) + 1, 0, 64, stream=9)
    starts, pos = [], 0
    for (gh, gw), g in zip(wl.grids, gaps):
        pos += g
        starts.append(pos)
        pos += 2 + -(-gh // 3) * (-(-gw // 3) + 1)
    R = pos + gaps[-1]
    rows = out.cpu().numpy()
    emb = np.zeros((R, Dl), np.uint16)
    want = oracle.assemble(emb, 0, R, wl.grids, starts, rows, sent)
    got = np.zeros_like(emb)
    for a in range(0, R, 1024):
        b = min(R, a + 1024)
        d = torch.zeros((b - a, Dl), dtype=torch.bfloat16, device="cuda")
        enc.assemble(d, a, wl.grids, starts, out)
        torch.cuda.synchronize()
        got[a:b] = d.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)



def test_official_variant_first_block_full_length():
    """The official-layer variant at the 1024-token image (96 x 96 = 9216 patches, one block):
    the residual stream after the first block on sampled rows against the oracle, which
    computes q, k, v for every patch and the rest of the block for the sampled rows only
    (attention rows are independent of one another; the other steps act row by row)."""
    from dataclasses import replace
    torch = require_gpu()
    cfg = replace(synth.V41_OFFICIAL, layers=1)
    gh = gw = 96
    blob = synth.make_weights(cfg, perturbed=True)
    px = synth.make_pixels(cfg, [(gh, gw)])
    enc = vit.Encoder(cfg, blob)
    x1 = enc.dump(vit.DUMP_LAYER, torch.from_numpy(px).cuda(), [(gh, gw)], 0)
    torch.cuda.synchronize()
    rows = np.r_[0:2, 95:98, 4600:4602, 9214:9216]
    got = from_dev_bf16(x1)[rows]
    want = first_block_rows(cfg, oracle.Weights(cfg, blob), px, gh, gw, rows)
    assert_projector_gate(got, want, "official first block")


def first_block_rows(cfg, W, px, gh, gw, rows):
    """Residual stream after the first block for some rows of one image, from the oracle: q, k,
    v for every patch, the rest of the block for those rows only (attention rows are
    independent of one another; the other steps act row by row)."""
    kw = dict(workers=16)
    D, H = cfg.hidden, cfg.heads
    x0 = oracle.linear(oracle.patchify(px, gh, gw, cfg), None, W["pe.b"], Wt=W.T("pe.w"), **kw)
    ln = oracle.norm(cfg, x0, W, "l0.ln1", **kw)
    qkv = oracle.rope_qk(oracle.linear(ln, None, W["l0.qkv.b"], Wt=W.T("l0.qkv.w"), **kw), gw, D, H,
                         cfg.rope_base, **kw)
    o = np.stack([oracle.attention(qkv, D, H, rows=(r, r + 1))[r] for r in rows])
    a = oracle.linear(o, None, W["l0.o.b"], Wt=W.T("l0.o.w"))
    x = oracle.add_round(x0[rows], a)
    return oracle.add_round(x, oracle.mlp(cfg, oracle.norm(cfg, x, W, "l0.ln2"), W, 0))


def test_extreme_aspect_images_first_block():
    """The longest grids the token cap allows: 3 x 3072 and 3072 x 3 patches (1024 merged tokens
    each, RoPE positions up to 3071 on one axis), packed in one batch; the residual stream
    after the first block on rows at both ends and in the middle of each image."""
    from dataclasses import replace
    torch = require_gpu()
    cfg = replace(synth.V41, layers=1)
    grids = [(3, 3072), (3072, 3)]
    blob = synth.make_weights(cfg, perturbed=True)
    px = synth.make_pixels(cfg, grids)
    enc = vit.Encoder(cfg, blob)
    x1 = from_dev_bf16(enc.dump(vit.DUMP_LAYER, torch.from_numpy(px).cuda(), grids, 0))
    torch.cuda.synchronize()
    W = oracle.Weights(cfg, blob)
    n = 9216
    rows = np.r_[0:2, 3070:3074, 6143:6145, n - 2:n]
    split = 14 * 3 * 14 * 3072 * 3
    for i, (gh, gw) in enumerate(grids):
        want = first_block_rows(cfg, W, px[i * split:(i + 1) * split], gh, gw, rows)
        assert_projector_gate(x1[i * n + rows], want, f"grid {gh}x{gw} first block")
    out = enc.encode(torch.from_numpy(px).cuda(), grids)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (2048, cfg.out_hidden) and bool(torch.isfinite(out).all())
