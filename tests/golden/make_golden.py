#!/usr/bin/env python3
"""Write oracle reference rows for the full-size encoder workloads.

The fp32 CPU oracle needs minutes for a 32-layer pass over thousands of patches, too long
for a test, so this script runs it once and stores, in ``tests/golden/oracle_<workload>.npz``:

  rows, values        sampled visual rows (global token index) and the fp32 oracle's values;
  values64            the same rows from the fp64 twin of the oracle (same algorithm and bf16
                      rounding points, fp64 arithmetic between them): the spread between the
                      two is the method's own sensitivity to summation order at full depth;
  layer0_rows/values  sampled patch rows of the residual stream after the first block (fp32
                      oracle), for a one-block end-to-end check at full size;
  spread_all_rel/max  rel-L2 and max-abs between the fp64 twin and the fp32 oracle over ALL
                      visual rows of the stored images (the gate of an all-rows comparison).

It calls only ``oracle`` and the seeded input generator ``synth``; the GPU tests regenerate
the same inputs from the same seeds.

    python tests/golden/make_golden.py [workload ...] [--workers N]
"""
import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

# images of the packed batch whose rows are stored (the two smallest and the two largest)
PACKED_IMAGES = 4
ROWS_PER_IMAGE = 8
LAYER0_ROWS_PER_IMAGE = 64


def sample_rows(m: int, k: int, seed: int):
    """First, last and k-2 seeded distinct rows of an image with m merged tokens."""
    rest = [int(r) for r in synth.seeded_distinct_rows(min(k, m), m, seed=seed, stream=7)]
    rows = sorted(set([0, m - 1] + rest))[:k]
    return np.array(rows, np.int64)


def run(name: str, workers: int):
    wl = synth.workload(name)
    cfg, grids = wl.cfg, wl.grids
    blob = synth.make_weights(cfg)
    px = synth.make_pixels(cfg, grids)
    W = oracle.Weights(cfg, blob)
    offs = np.cumsum([0] + [(cfg.patch * gh) * (cfg.patch * gw) * 3 for gh, gw in grids])
    tok_offs = np.cumsum([0] + [cfg.tokens(gh, gw) for gh, gw in grids])
    if name == "packed16":
        order = np.argsort([gh * gw for gh, gw in grids], kind="stable")
        images = sorted(set(order[:2].tolist() + order[-2:].tolist()))[:PACKED_IMAGES]
    else:
        images = list(range(len(grids)))
    patch_offs = np.cumsum([0] + [gh * gw for gh, gw in grids])
    out = {"images": np.array(images, np.int64)}
    all_rows, all_vals, all_vals64, l0_rows, l0_vals = [], [], [], [], []
    every32, every64 = [], []
    for i in images:
        gh, gw = grids[i]
        img = px[offs[i]:offs[i + 1]]
        t = time.time()
        dumps = {}
        rows = oracle.encode_image(cfg, W, img, gh, gw, workers=workers, dumps=dumps)
        m = rows.shape[0]
        sel = sample_rows(m, ROWS_PER_IMAGE, seed=1000 + i)
        all_rows.append(tok_offs[i] + sel)
        all_vals.append(rows[sel])
        psel = sample_rows(gh * gw, LAYER0_ROWS_PER_IMAGE, seed=2000 + i)
        l0_rows.append(patch_offs[i] + psel)
        l0_vals.append(np.asarray(dumps["layer0"])[psel])
        del dumps
        rows64 = oracle.encode_image(cfg, W, img, gh, gw, prec="f64", workers=workers)
        all_vals64.append(rows64[sel])
        every32.append(np.asarray(rows, np.float64))
        every64.append(np.asarray(rows64, np.float64))
        print(f"{name} image {i} ({gh}x{gw}): {time.time() - t:.0f} s", flush=True)
    out["rows"] = np.concatenate(all_rows)
    out["values"] = np.concatenate(all_vals).astype(np.float32)
    out["values64"] = np.concatenate(all_vals64).astype(np.float64)
    out["layer0_rows"] = np.concatenate(l0_rows)
    out["layer0_values"] = np.concatenate(l0_vals).astype(np.float32)
    out["grids"] = np.array(grids, np.int64)
    e32, e64 = np.concatenate(every32), np.concatenate(every64)
    out["spread_all_rel"] = np.float64(np.linalg.norm(e64 - e32) / np.linalg.norm(e64))
    out["spread_all_max"] = np.float64(np.abs(e64 - e32).max())
    print(f"{name}: fp64 vs fp32 over all {e32.shape[0]} rows: rel_l2={float(out['spread_all_rel']):.3e} "
          f"max_abs={float(out['spread_all_max']):.3e}", flush=True)
    path = os.path.join(HERE, f"oracle_{name}.npz")
    np.savez_compressed(path, **out)
    print("wrote", path, out["values"].shape, flush=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="*", default=["v4_384", "v41_1024", "packed16", "v41_official"])
    ap.add_argument("--workers", type=int, default=os.cpu_count() or 1)
    a = ap.parse_args()
    for w in a.workloads:
        run(w, a.workers)
