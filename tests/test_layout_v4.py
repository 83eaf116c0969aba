"""The V4 Flash span layout (a reading of [G] "V4 Flash Vision-Exp": row-pair interleave and
pos % 4 alignment, which V4.1 drops; [L] DS4V: the projector's tile permutation applied once
at assembly).  Parity with the official model is unpinned: the pages give no formula.  The
oracle's reading is pinned by closed forms and the C ABI's host layout is checked against it."""
import numpy as np
import pytest

import multimodal_vision_encoder_amd as vit
import oracle
import synth

GRIDS = [[(6, 9), (3, 3)], [(54, 63)], [(96, 96)], [(5, 7), (1, 1), (12, 3), (4, 30)],
         synth.packed_grids_batch()]


def merged(g):
    return -(-g[0] // 3), -(-g[1] // 3)


@pytest.mark.parametrize("grids", GRIDS, ids=["small", "v4_384", "v41_1024", "ragged", "packed16"])
def test_v4_layout_closed_forms(grids):
    """Catches a row-major stream (no interleave), a NEWLINE per row instead of per pair, and a
    missing or misplaced compress_pad: every span has 4 ceil((2 + ceil(mh/2) + mh mw) / 4)
    positions, merged token (r, c) sits at 1 + (r // 2)(2 mw + 1) + 2c + r % 2 inside a full
    pair and at 1 + (mh // 2)(2 mw + 1) + c in a last lone row, and IMAGE positions cover the
    visual rows exactly once."""
    types, src = oracle.layout_v4(grids)
    pos, first = 0, 0
    for g in grids:
        mh, mw = merged(g)
        core = 2 + -(-mh // 2) + mh * mw
        n = -(-core // 4) * 4
        t, s = types[pos:pos + n], src[pos:pos + n]
        assert t[0] == oracle.TOK_START and t[core - 1] == oracle.TOK_END
        assert (t[core:] == oracle.TOK_PAD).all() and len(t) % 4 == 0
        assert (t == oracle.TOK_NEWLINE).sum() == -(-mh // 2)
        for r in range(mh):
            for c in range(mw):
                k = 1 + (r // 2) * (2 * mw + 1) + 2 * c + r % 2 if r < mh - mh % 2 else \
                    1 + (mh // 2) * (2 * mw + 1) + c
                assert t[k] == oracle.TOK_IMAGE and s[k] == first + r * mw + c
        pos += n
        first += mh * mw
    assert pos == len(types)
    img = src[types == oracle.TOK_IMAGE]
    assert np.array_equal(np.sort(img), np.arange(first))


def test_v4_layout_special_cases():
    """One merged row: the V4.1 stream followed by padding.  The 54x63 (384-token) image: 378
    IMAGE, 9 NEWLINE, 389 positions padded to 392."""
    for g in [(3, 12), (1, 30), (2, 2)]:
        t4, s4 = oracle.layout_v4([g])
        t1, s1 = oracle.layout([g])
        assert np.array_equal(t4[:len(t1)], t1) and np.array_equal(s4[:len(s1)], s1)
        assert (t4[len(t1):] == oracle.TOK_PAD).all()
    t, s = oracle.layout_v4([(54, 63)])
    assert len(t) == 392 and (t == oracle.TOK_IMAGE).sum() == 378 and (t == oracle.TOK_NEWLINE).sum() == 9
    assert (t == oracle.TOK_PAD).sum() == 3


@pytest.mark.parametrize("grids", GRIDS, ids=["small", "v4_384", "v41_1024", "ragged", "packed16"])
def test_c_abi_v4_layout_matches_oracle(grids):
    t, s = vit.layout(grids, span=vit.SPAN_V4)
    ot, os_ = oracle.layout_v4(grids)
    assert np.array_equal(t, ot) and np.array_equal(s, os_)
    assert vit.TOK_PAD == oracle.TOK_PAD
