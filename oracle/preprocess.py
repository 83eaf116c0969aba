"""CPU oracle of the image preprocessing before the encoder (TEST INFRASTRUCTURE ONLY, like
the rest of this package).

[Z] "DeepSeek V4.1 Flash Engineering, Part 3: Integrating Vision", "Step 1": the largest grid
that fits the image's aspect ratio and the token budget, dimensions constrained to the patch
and merge grid, a contain resize (bicubic) whose second dimension comes from a branch on the
aspect ratio and a rounding, the result centred on RGB 127 gray padding; images below the
minimum pixel count are first enlarged proportionally.  [G] ds4-learning "glossary/vision":
the V4.1 row (1024 tokens, minimum 295,936 pixels, no aspect clamp) and the V4 Flash row (384
tokens, minimum 147,456 pixels, aspect clamped to 8:1, gray 127 canvas).

The pages leave the exact growth, clamp and tie rules open; the readings taken here:
  * enlargement: both sides scaled by sqrt(min_pixels / (H W)) (real-valued, no rounding);
  * aspect clamp: the planning aspect is limited to max_aspect:1 by lengthening the short side
    (the contain step then pads the image);
  * grid: with a = H/(patch*merge), b = W/(patch*merge), the nearest integers (at least 1) when
    a*b fits the budget; otherwise floor(a r) x floor(b r) with r = sqrt(budget / (a b)), then
    grown one row or column at a time while the budget allows, each time the step that keeps
    log(columns/rows) closest to log(b/a) (rows first on a tie);
  * contain: the side that limits the fit is the canvas side, the other is
    round(other * canvas side / limiting side), ties to even, at least 1;
  * centring: offsets floor((canvas - resized) / 2);
  * bicubic: the Keys cubic with a = -0.5 as a separable convolution, sample centres at
    (i + 0.5) * in/out, the kernel stretched by in/out when shrinking (support 2 * in/out),
    taps outside the image dropped and the weights renormalised; horizontal pass first,
    intermediate kept unrounded; result rounded half to even and clamped to 0..255.
Byte-exact agreement with any particular imaging library is not claimed (parity unpinned).
"""
from __future__ import annotations

import math

import numpy as np


def _round_half_even_div(num: int, den: int) -> int:
    """round(num / den) for non-negative integers, ties to even, exactly."""
    q, r = divmod(num, den)
    if 2 * r > den or (2 * r == den and q % 2 == 1):
        q += 1
    return q


def plan_image(height: int, width: int, patch: int = 14, merge: int = 3, max_tokens: int = 1024,
               min_pixels: int = 295936, max_aspect: int = 0) -> dict:
    """Token grid, canvas and contain geometry of one image (see the module docstring)."""
    assert height >= 1 and width >= 1 and max_tokens >= 1
    u = patch * merge
    H1, W1 = float(height), float(width)
    if height * width < min_pixels:
        s = math.sqrt(min_pixels / (height * width))
        H1, W1 = H1 * s, W1 * s
    if max_aspect:
        if W1 > max_aspect * H1:
            H1 = W1 / max_aspect
        elif H1 > max_aspect * W1:
            W1 = H1 / max_aspect
    a, b = H1 / u, W1 / u
    mh = mw = 0
    if a * b <= max_tokens:
        mh, mw = max(1, round(a)), max(1, round(b))
    if mh * mw == 0 or mh * mw > max_tokens:
        r = math.sqrt(max_tokens / (a * b))
        mh, mw = max(1, math.floor(a * r)), max(1, math.floor(b * r))
        target = math.log(b / a)
        while True:
            best = None
            for cand in ((mh + 1, mw), (mh, mw + 1)):
                if cand[0] * cand[1] > max_tokens:
                    continue
                err = abs(math.log(cand[1] / cand[0]) - target)
                if best is None or err < best[0]:
                    best = (err, cand)
            if best is None:
                break
            mh, mw = best[1]
    gh, gw = mh * merge, mw * merge
    ch, cw = gh * patch, gw * patch
    if width * ch >= height * cw:    # the image is relatively wider: its width fills the canvas
        rw, rh = cw, max(1, _round_half_even_div(height * cw, width))
    else:
        rh, rw = ch, max(1, _round_half_even_div(width * ch, height))
    return {"gh": gh, "gw": gw, "canvas_h": ch, "canvas_w": cw, "resized_h": rh, "resized_w": rw,
            "off_y": (ch - rh) // 2, "off_x": (cw - rw) // 2}


def keys_cubic(x: np.ndarray, a: float = -0.5) -> np.ndarray:
    """The Keys cubic convolution kernel (support 2)."""
    x = np.abs(np.asarray(x, np.float64))
    out = np.zeros_like(x)
    m1 = x < 1
    m2 = (x >= 1) & (x < 2)
    out[m1] = ((a + 2) * x[m1] - (a + 3)) * x[m1] * x[m1] + 1
    out[m2] = ((a * x[m2] - 5 * a) * x[m2] + 8 * a) * x[m2] - 4 * a
    return out


def resize_weights(n_in: int, n_out: int) -> np.ndarray:
    """[n_out][n_in] normalised bicubic weights of one axis."""
    scale = n_in / n_out
    fs = max(scale, 1.0)
    support = 2.0 * fs
    Wt = np.zeros((n_out, n_in), np.float64)
    for i in range(n_out):
        c = (i + 0.5) * scale
        lo = max(0, int(math.floor(c - support)))
        hi = min(n_in, int(math.ceil(c + support)) + 1)
        j = np.arange(lo, hi)
        k = keys_cubic((j + 0.5 - c) / fs)
        Wt[i, lo:hi] = k / k.sum()
    return Wt


def resize_bicubic(img: np.ndarray, out_h: int, out_w: int) -> np.ndarray:
    """uint8 HWC image -> uint8 [out_h][out_w][C]: horizontal pass, then vertical, in fp64."""
    x = img.astype(np.float64)
    Wx = resize_weights(img.shape[1], out_w)
    Wy = resize_weights(img.shape[0], out_h)
    tmp = np.einsum("ij,hjc->hic", Wx, x)
    out = np.einsum("ij,jwc->iwc", Wy, tmp)
    return np.clip(np.rint(out), 0, 255).astype(np.uint8)


def preprocess(img: np.ndarray, plan: dict) -> np.ndarray:
    """The gray-127 canvas [canvas_h][canvas_w][3] with the contained, centred image."""
    canvas = np.full((plan["canvas_h"], plan["canvas_w"], 3), 127, np.uint8)
    rh, rw, y0, x0 = plan["resized_h"], plan["resized_w"], plan["off_y"], plan["off_x"]
    canvas[y0:y0 + rh, x0:x0 + rw] = resize_bicubic(img, rh, rw)
    return canvas
