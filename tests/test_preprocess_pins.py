"""Pins of the preprocessing oracle (planner, contain geometry, bicubic resize) against what the
pages fix and against closed forms; no GPU."""
import math

import numpy as np
import pytest

import synth
from oracle import preprocess as pp

V41 = dict(max_tokens=1024, min_pixels=295936, max_aspect=0)
V4 = dict(max_tokens=384, min_pixels=147456, max_aspect=8)


def test_plan_of_the_workload_images():
    """The 1344 x 1344 image of the 1024-token workload fills the V4.1 budget exactly (96 x 96
    patches, 32 x 32 tokens); the 756 x 882 image of the V4 workload gives 54 x 63 patches and
    378 tokens, under the 384 cap.  Both are already multiples of 42 pixels: no resize offset."""
    p = pp.plan_image(1344, 1344, **V41)
    assert (p["gh"], p["gw"], p["canvas_h"], p["canvas_w"]) == (96, 96, 1344, 1344)
    assert (p["resized_h"], p["resized_w"], p["off_y"], p["off_x"]) == (1344, 1344, 0, 0)
    p = pp.plan_image(756, 882, **V4)
    assert (p["gh"], p["gw"], p["canvas_h"], p["canvas_w"]) == (54, 63, 756, 882)
    assert (p["resized_h"], p["resized_w"], p["off_y"], p["off_x"]) == (756, 882, 0, 0)


def test_budget_minimum_and_aspect_on_many_sizes():
    """Seeded sizes from 1 to 6000 pixels a side: the token grid never exceeds the budget, an
    image with enough pixels for the budget uses at least 90% of it, small images reach the
    minimum pixel count (within the 42-pixel grid rounding), the grid keeps the image's aspect
    (or 8:1 under the V4 clamp), and the resized image fits the canvas, touches it on one axis
    and is centred."""
    rng = np.random.default_rng(5)
    for prof in (V41, V4):
        for _ in range(400):
            h, w = (int(x) for x in np.exp(rng.uniform(0, math.log(6000), 2)))
            p = pp.plan_image(h, w, **prof)
            mh, mw = p["gh"] // 3, p["gw"] // 3
            assert 1 <= mh * mw <= prof["max_tokens"]
            if h * w >= 4 * prof["max_tokens"] * 42 * 42 and max(h, w) / min(h, w) < 20:
                assert mh * mw >= 0.9 * prof["max_tokens"]
            if h * w < prof["min_pixels"] and mh * mw < prof["max_tokens"] and max(h, w) / min(h, w) < 4:
                assert (mh + 1) * (mw + 1) * 42 * 42 >= prof["min_pixels"]
            asp = w / h
            if prof["max_aspect"]:
                asp = min(max(asp, 1 / prof["max_aspect"]), prof["max_aspect"])
            if mh >= 4 and mw >= 4:
                assert abs(math.log(mw / mh) - math.log(asp)) < 0.3
            ch, cw, rh, rw = p["canvas_h"], p["canvas_w"], p["resized_h"], p["resized_w"]
            assert (ch, cw) == (p["gh"] * 14, p["gw"] * 14)
            assert 1 <= rh <= ch and 1 <= rw <= cw and (rh == ch or rw == cw)
            assert p["off_y"] == (ch - rh) // 2 and p["off_x"] == (cw - rw) // 2
            # contain: one side is the canvas side, the other its rounded proportional length
            assert ((rw == cw and (abs(rh - h * cw / w) <= 0.5 or rh == 1)) or
                    (rh == ch and (abs(rw - w * ch / h) <= 0.5 or rw == 1)))


def test_contain_rounding_ties_to_even():
    """The second side of the contain step is the exact rational rounded half to even: a
    1000 x 999 image in a 1008 x 1008 canvas gives 1008 x round(999 * 1008 / 1000) = 1007, and
    exact halves go to the even neighbour."""
    assert pp._round_half_even_div(1007 * 2 + 1, 2) == 1008
    assert pp._round_half_even_div(1006 * 2 + 1, 2) == 1006
    p = pp.plan_image(1000, 999, **V41)
    assert p["canvas_h"] == p["canvas_w"] == p["resized_h"]
    assert p["resized_w"] == round(999 * p["canvas_h"] / 1000)


def test_keys_kernel_values():
    """The Keys cubic (a = -0.5): 1 at 0, 0 at the other integers, 0.5625 at 1/2 and -0.0625 at
    3/2 (closed forms of the two polynomial pieces), symmetric, partition of unity."""
    k = pp.keys_cubic(np.array([0.0, 1.0, 2.0, 0.5, 1.5, -0.5, 2.5]))
    assert np.allclose(k, [1.0, 0.0, 0.0, 0.5625, -0.0625, 0.5625, 0.0])
    t = np.linspace(0, 1, 11)
    s = sum(pp.keys_cubic(t + j) for j in (-2, -1, 0, 1))
    assert np.allclose(s, 1.0)


def test_resize_identity_constant_and_linear():
    """Same size: a copy.  A constant image stays constant at any size.  Enlarging reproduces a
    linear ramp exactly away from the borders (the Keys cubic interpolates linear functions)."""
    img = synth.uniform_bytes(11, 0, 37 * 23 * 3).reshape(37, 23, 3)
    assert np.array_equal(pp.resize_bicubic(img, 37, 23), img)
    const = np.full((30, 17, 3), 200, np.uint8)
    for oh, ow in ((61, 40), (9, 5), (30, 100)):
        assert (pp.resize_bicubic(const, oh, ow) == 200).all()
    ramp = np.tile((np.arange(64) * 3).astype(np.uint8)[None, :, None], (4, 1, 3))
    Wx = pp.resize_weights(64, 160)
    out = Wx @ ramp[0, :, 0].astype(np.float64)
    c = (np.arange(160) + 0.5) * 64 / 160 - 0.5          # source coordinate of each output
    inner = (c > 2) & (c < 61)
    assert np.allclose(out[inner], 3 * c[inner], atol=1e-9)


def test_resize_one_output_by_hand():
    """One output pixel of a 2x shrink written out: centre (i + 0.5) * 2, kernel stretched by 2,
    taps j with weights k((j + 0.5 - centre) / 2), normalised."""
    src = synth.uniform_bytes(12, 0, 8 * 8).reshape(8, 8, 1)
    out = pp.resize_bicubic(src, 4, 4)
    i, x = 1, 2
    def axis(n, i):
        c = (i + 0.5) * 2
        js = [j for j in range(n) if abs(j + 0.5 - c) < 4]
        w = np.array([pp.keys_cubic(np.array([(j + 0.5 - c) / 2]))[0] for j in js])
        return js, w / w.sum()
    jy, wy = axis(8, i)
    jx, wx = axis(8, x)
    v = sum(wy[a] * wx[b] * float(src[jy[a], jx[b], 0]) for a in range(len(jy)) for b in range(len(jx)))
    assert out[i, x, 0] == np.clip(np.rint(v), 0, 255)


def test_canvas_is_gray_outside_the_image():
    img = synth.uniform_bytes(13, 0, 300 * 900 * 3).reshape(300, 900, 3)
    p = pp.plan_image(300, 900, **V41)
    cv = pp.preprocess(img, p)
    assert cv.shape == (p["canvas_h"], p["canvas_w"], 3)
    y0, x0, rh, rw = p["off_y"], p["off_x"], p["resized_h"], p["resized_w"]
    mask = np.ones(cv.shape[:2], bool)
    mask[y0:y0 + rh, x0:x0 + rw] = False
    assert (cv[mask] == 127).all()
    assert not (cv[~mask] == 127).all()
