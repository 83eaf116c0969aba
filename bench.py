#!/usr/bin/env python3
"""Throughput of the vision-encoder hot path on one MI355X.

One step = one whole pass of the hot path over one synthetic batch: vit_encode (patchify,
patch projection, the ViT blocks, final LayerNorm, 3x3 merge + projector), the span layout
and vit_overlay of the visual rows into a prompt embedding matrix.  Inputs are resident in
HBM before the timed region starts.  Prints one JSON line on stdout; progress on stderr.

Default workload: one 1344x1344 image (96x96 = 9216 patches, 32 layers of width 1024 with
16 heads and MLP 4096, 1024 merged tokens projected to 5120).  Besides the headline line's
figures, the JSON carries per-kernel times, the steps around the path (preprocessing, chunk
assembly) and the same images through the official-layer variant of the tower (RMSNorm,
SwiGLU, erf GELU, two-linear aligner).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# HBM bytes per attention launch, from rocprofv3 FETCH_SIZE and WRITE_SIZE passes scaled by
# the same counters on a plain copy of known size; valid while the kernel source is unchanged
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_v41_1024_hbm_traffic.md")
ATTN_SOURCE = os.path.join(ROOT, "multimodal_vision_encoder_amd", "csrc", "attention.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_per_pass(cfg, grids):
    """Algorithmic MFMA FLOPs: patch projection at K = 588, per layer QKV + out-proj + MLP +
    attention (QK^T and PV over each image's own patches only), projector at K = 9D.  The
    official-layer variant's SwiGLU step computes two F-wide projections (gate and up), and
    its aligner adds the second projection."""
    D, F, L, Dl = cfg.hidden, cfg.mlp, cfg.layers, cfg.out_hidden
    Da = cfg.aligner_hidden or Dl
    nf1 = 2 if cfg.mlp_kind == 1 else 1
    tot = {"patch_embed": 0, "qkv": 0, "attention": 0, "out_proj": 0, "fc1": 0, "fc2": 0,
           "projector": 0}
    for gh, gw in grids:
        n, m = gh * gw, cfg.tokens(gh, gw)
        tot["patch_embed"] += 2 * n * cfg.patch_dim * D
        tot["qkv"] += L * 6 * n * D * D
        tot["attention"] += L * 4 * n * n * D
        tot["out_proj"] += L * 2 * n * D * D
        tot["fc1"] += L * 2 * n * D * F * nf1
        tot["fc2"] += L * 2 * n * F * D
        tot["projector"] += 2 * m * 9 * D * Da + (2 * m * Da * Dl if cfg.aligner_hidden else 0)
    return tot


def bytes_per_pass(cfg, grids, vt_cols):
    """Algorithmic HBM bytes of the memory-bound steps (one read and one write of each
    tensor a step must touch)."""
    D, L, Dl = cfg.hidden, cfg.layers, cfg.out_hidden
    N = sum(gh * gw for gh, gw in grids)
    M = sum(cfg.tokens(gh, gw) for gh, gw in grids)
    # every norm reads x and writes its output (the residual adds run in the epilogues of the
    # out-projection and fc2): two per layer and the final one
    ln = (2 * L + 1) * 2 * N * D * 2
    rope = L * (8 * N * D + 2 * N * D + 2 * vt_cols * D)   # q,k in+out, v in, v^T out
    overlay = M * Dl * (4 + 2) + 4 * M
    return {"layernorm": ln, "rope": rope, "overlay": overlay}


def cpu_baseline(cfg, blob, px, grids):
    """The CPU oracle on the host's cores: fixed part (patchify, patch projection, final LN,
    merge, projector) plus one of the layers, all patches of the first image; the full pass
    is extrapolated as T_fixed + layers * T_layer."""
    import oracle
    cores = min(16, len(os.sched_getaffinity(0)))
    gh, gw = grids[0]
    W = oracle.Weights(cfg, blob)
    for name, _ in cfg.tensor_shapes():
        if name.endswith(".w") and (name.startswith("l0.") or not name.startswith("l")):
            W.T(name)
    n_img = (cfg.patch * gh) * (cfg.patch * gw) * 3
    img = px[:n_img]
    t0 = time.perf_counter()
    oracle.encode_image(cfg, W, img, gh, gw, workers=cores, layers=0)
    t_fixed = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.encode_image(cfg, W, img, gh, gw, workers=cores, layers=1)
    t_one = time.perf_counter() - t0
    t_layer = max(t_one - t_fixed, 0.0)
    t_pass = t_fixed + cfg.layers * t_layer
    tokens = cfg.tokens(gh, gw)
    return {"value": tokens / t_pass, "unit": "visual tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"first image ({gh}x{gw} patches): patch projection + final LN + merge + "
                       f"projector timed ({t_fixed:.2f} s) and 1 of {cfg.layers} layers timed "
                       f"({t_layer:.2f} s) on all patches, fp32 oracle, rows split over {cores} "
                       f"threads; full pass extrapolated as T_fixed + {cfg.layers} T_layer = "
                       f"{t_pass:.1f} s"),
            "seconds_per_pass": t_pass}


def norm_isolated(enc, cfg, n_rows, launches=100, replays=5):
    """The LayerNorm kernel alone at the pass's shape (n_rows x hidden): `launches` launches of
    vit_op_layernorm on fixed buffers captured in one HIP graph and replayed under a single
    event pair, so that the event pair the per-step timing puts around every launch (about 2 us
    on an 8-10 us kernel) does not count.  The graph holds kernel launches only.  After the
    replays, and between them beside eager launches, the output is compared bitwise with an
    eager launch.  Bytes as in bytes_per_pass: read x, write the norm."""
    import torch
    D = cfg.hidden
    gen = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn(n_rows, D, device="cuda", generator=gen).bfloat16()
    ga = (1.0 + 0.1 * torch.randn(D, device="cuda", generator=gen)).bfloat16()
    be = (0.1 * torch.randn(D, device="cuda", generator=gen)).bfloat16()
    ref = enc.op_layernorm(x, ga, be, cfg.ln_eps)
    out = torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            enc.op_layernorm(x, ga, be, cfg.ln_eps, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(launches):
            enc.op_layernorm(x, ga, be, cfg.ln_eps, out=out)
    ok = True
    for _ in range(2):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ok = ok and bool(torch.equal(out, ref))
        ok = ok and bool(torch.equal(enc.op_layernorm(x, ga, be, cfg.ln_eps), ref))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ok = ok and bool(torch.equal(out, ref))
    us = e0.elapsed_time(e1) / (replays * launches) * 1e3
    del graph
    by = 2 * n_rows * D * 2
    return {"avg_launch_us": us, "gbs": by / (us * 1e-6) / 1e9, "hbm_frac": by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "launches": launches * replays, "replays_match_eager": ok,
            "method": f"{launches} launches of {n_rows} x {D} rows in one graph, {replays} replays under one event pair"}


def around_the_path(enc, cfg, grids, out, reps):
    """The steps before and after the timed path, timed alone with events on the current
    stream: preprocessing of a 3000 x 2000 photo-sized image onto the first image's canvas
    (bicubic contain resize), and the chunk assembly of the visual rows plus the learned span
    rows into one prompt.  Algorithmic bytes: preprocessing reads the image and writes the
    canvas, with the fp32 intermediate [H][resized_w][3] written and read once; assembly reads
    each fp32 visual row and writes each bf16 span row."""
    import numpy as np
    import torch
    import multimodal_vision_encoder_amd as vit
    import synth
    res = {}
    gh, gw = grids[0]
    H, W = 2000, 3000
    plan = vit.plan_image(H, W, patch=cfg.patch, merge=3, max_tokens=cfg.max_tokens_per_image,
                          min_pixels=0, max_aspect=0)
    img = torch.from_numpy(synth.uniform_bytes(41, 0, H * W * 3)).cuda()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    enc.preprocess(img, H, W, plan)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        enc.preprocess(img, H, W, plan)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    by = H * W * 3 + 2 * H * plan["resized_w"] * 3 * 4 + plan["canvas_h"] * plan["canvas_w"] * 3
    res["preprocess"] = {"image": [H, W], "canvas": [plan["canvas_h"], plan["canvas_w"]], "us": us,
                         "gbs": by / (us * 1e-6) / 1e9, "hbm_frac": by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    types, _ = vit.layout(grids)
    R = 64 + types.size
    enc.set_sentinels(synth.make_sentinels(cfg.out_hidden))
    chunk = torch.zeros((R, cfg.out_hidden), dtype=torch.bfloat16, device="cuda")
    starts, pos = [], 64
    for g in grids:
        starts.append(pos)
        pos += 2 + -(-g[0] // 3) * (-(-g[1] // 3) + 1)
    enc.assemble(chunk, 0, grids, starts, out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        enc.assemble(chunk, 0, grids, starts, out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    # the kernel alone (the library's event pair around its launch): a call also uploads the
    # chunk's (row, source) pairs from pinned host memory, which the call time includes
    enc.timing(True)
    for _ in range(reps):
        enc.assemble(chunk, 0, grids, starts, out)
    torch.cuda.synchronize()
    t_ms, n = enc.timing_read()["overlay"]
    enc.timing(False)
    k_us = t_ms / max(n, 1) * 1e3
    n_img = int((types == vit.TOK_IMAGE).sum())
    by = n_img * cfg.out_hidden * (4 + 2) + (types.size - n_img) * cfg.out_hidden * 4
    res["assemble"] = {"positions": int(types.size), "us": us, "gbs": by / (us * 1e-6) / 1e9,
                       "hbm_frac": by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                       "kernel_us": k_us, "kernel_gbs": by / (k_us * 1e-6) / 1e9,
                       "kernel_hbm_frac": by / (k_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                       "note": "us and gbs per call (host metadata upload included); kernel_* the "
                               "assembly kernel alone"}
    return res


def official_variant(cfg, grids, steps, warmup):
    """The official-layer variant of the same tower (RMSNorm, SwiGLU MLP, erf GELU, two-linear
    aligner with inner width out_hidden) on the same images: encoder throughput and per-step
    kernel times.  Random N(0, 0.02) weights, gamma 1, biases 0."""
    import dataclasses
    import torch
    import multimodal_vision_encoder_amd as vit
    import synth
    vc = dataclasses.replace(cfg, norm_kind=1, mlp_kind=1, gelu_kind=1, aligner_hidden=cfg.out_hidden)
    blob = synth.make_weights(vc)
    px = torch.from_numpy(synth.make_pixels(vc, grids)).cuda()
    M = sum(vc.tokens(gh, gw) for gh, gw in grids)
    enc = vit.Encoder(vc, blob)
    del blob
    out = torch.empty((M, vc.out_hidden), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        enc.encode(px, grids, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        enc.encode(px, grids, out=out)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = el / steps * 1e3
    fl = flops_per_pass(vc, grids)
    res = {"layers": "RMSNorm, SwiGLU MLP, erf GELU, two-linear aligner",
           "aligner_hidden": vc.aligner_hidden, "visual_tokens_per_s": M * steps / el, "ms_per_step": ms,
           "images_per_s": len(grids) * steps / el, "tflops": sum(fl.values()) / (ms * 1e-3) / 1e12}
    res["mfma_frac"] = res["tflops"] / PEAK_BF16_TFLOPS
    enc.timing(True)
    for _ in range(steps):
        enc.encode(px, grids, out=out)
    torch.cuda.synchronize()
    tm = enc.timing_read()
    enc.timing(False)
    kern = {}
    for k, (t_ms, n) in tm.items():
        if n == 0:
            continue
        e = {"ms_per_step": t_ms / steps, "avg_launch_us": t_ms / n * 1e3}
        if k in fl:
            e["tflops"] = fl[k] / (t_ms / steps * 1e-3) / 1e12
            e["mfma_frac"] = e["tflops"] / PEAK_BF16_TFLOPS
        kern[k] = e
    res["kernels"] = kern
    enc.close()
    log(f"official-layer variant: {ms:.3f} ms/step, {res['visual_tokens_per_s']:.0f} tokens/s")
    return res


def pass_distribution(step, n):
    """Per-pass milliseconds of n passes, each bracketed by its own HIP event pair on the
    current stream (the stream the library launches on): median, p10, p90."""
    import numpy as np
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"passes": n, "median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90)), "min_ms": float(t.min()), "max_ms": float(t.max())}


class ClockSampler:
    """Samples the GPU core clock (the active level of the driver's sclk table in sysfs) every
    50 ms while running; None where the table is not readable."""

    def __init__(self):
        import glob
        self.files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []

    def _read(self):
        for f in self.files:
            try:
                for line in open(f):
                    if line.rstrip().endswith("*"):
                        mhz = float(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
                        if mhz > 0:
                            return mhz
            except (OSError, ValueError, IndexError):
                continue
        return None

    def __enter__(self):
        import threading
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                v = self._read()
                if v is not None:
                    self.samples.append(v)
                self._stop.wait(0.05)
        self._t = threading.Thread(target=run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        self._t.join()

    def summary(self):
        import numpy as np
        if not self.samples:
            return {"sclk_mhz": None, "note": "no readable sclk table", "peak_at_clock_tflops": None}
        mhz = float(np.median(self.samples))
        return {"sclk_mhz": mhz, "samples": len(self.samples), "source": "sysfs pp_dpm_sclk (active level)",
                "peak_at_clock_tflops": PEAK_BF16_TFLOPS * mhz / 2400.0,
                "note": "dense bf16 peak scaled from 2.4 GHz to the sampled clock"}


def measure_workload(name, steps, warmup):
    """A second workload through the same hot path (encode + layout + overlay): wall-clock
    throughput over `steps` passes, the event-timed per-pass distribution, and the per-kernel
    times that give the GEMM + attention fraction of the dense bf16 peak."""
    import numpy as np
    import torch
    import multimodal_vision_encoder_amd as vit
    import synth
    wl = synth.workload(name)
    cfg, grids = wl.cfg, wl.grids
    N, M = wl.n_patches, wl.n_tokens
    blob = synth.make_weights(cfg)
    enc = vit.Encoder(cfg, blob)
    del blob
    enc.reserve(N)
    d_px = torch.from_numpy(synth.make_pixels(cfg, grids)).cuda()
    out = torch.empty((M, cfg.out_hidden), dtype=torch.float32, device="cuda")
    types, src = vit.layout(grids)
    R = wl.embed_rows or (64 + types.size)
    start = (R - types.size) // 2
    rows = np.full(M, -1, np.int32)
    img_pos = np.nonzero(types == vit.TOK_IMAGE)[0]
    rows[src[img_pos]] = start + img_pos
    embeds = torch.zeros((R, cfg.out_hidden), dtype=torch.bfloat16, device="cuda")

    def step():
        enc.encode(d_px, grids, out=out)
        vit.layout(grids)
        enc.overlay(embeds, rows, out)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = el / steps * 1e3
    fl = flops_per_pass(cfg, grids)
    res = {"workload": name, "images": len(grids), "patches": N, "tokens": M, "out_hidden": cfg.out_hidden,
           "embed_rows": R, "ms_per_pass": ms, "visual_tokens_per_s": M * steps / el,
           "images_per_s": len(grids) * steps / el, "tflops": sum(fl.values()) / (ms * 1e-3) / 1e12}
    res["mfma_frac"] = res["tflops"] / PEAK_BF16_TFLOPS
    res["pass_ms"] = pass_distribution(step, max(20, steps))
    enc.timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    tm = enc.timing_read()
    enc.timing(False)
    gemm_attn = ("qkv", "attention", "out_proj", "fc1", "fc2")
    # the GEMM + attention time includes the merge of the attention's key-sliced items
    ga_ms = sum(tm[k][0] for k in gemm_attn + ("attn_merge",)) / steps
    res["gemm_attention_mfma_frac"] = sum(fl[k] for k in gemm_attn) / (ga_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    res["attention_ms_per_pass"] = (tm["attention"][0] + tm["attn_merge"][0]) / steps
    res["kernels_ms_per_pass"] = {k: v[0] / steps for k, v in tm.items() if v[1]}
    enc.close()
    log(f"{name}: {ms:.3f} ms/pass, {res['visual_tokens_per_s']:.0f} tokens/s, "
        f"GEMM+attention {res['gemm_attention_mfma_frac']:.3f} of peak")
    return res


def _oracle_image_child(args):
    """One packed-batch image through the single-threaded oracle in its own process: T_fixed
    (patchify, patch projection, final norm, merge, projector) and T_layer (one block), on all
    of the image's patches.  Weights of a one-layer tower with the same shapes (the values
    do not change the work)."""
    cfg, (gh, gw), i = args
    import dataclasses
    import oracle
    import synth
    c1 = dataclasses.replace(cfg, layers=1)
    W = oracle.Weights(c1, synth.make_weights(c1))
    img = synth.make_pixels(c1, [(gh, gw)], seed=synth.SEED_PIXELS + i)
    t0 = time.perf_counter()
    oracle.encode_image(c1, W, img, gh, gw, workers=1, layers=0)
    t_fixed = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.encode_image(c1, W, img, gh, gw, workers=1, layers=1)
    t_layer = max(time.perf_counter() - t0 - t_fixed, 0.0)
    return t_fixed, t_layer


def cpu_baseline_packed(cfg, grids):
    """The packed 16-image batch on the host: min(16, cores) independent single-threaded oracle
    processes, one image each; each image's pass is extrapolated as T_fixed + layers T_layer
    and the batch takes as long as its slowest image."""
    import multiprocessing as mp
    cores = min(16, len(os.sched_getaffinity(0)))
    todo = [(cfg, g, i) for i, g in enumerate(grids)]
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_oracle_image_child, todo)
    wall = time.perf_counter() - t0
    per_image = [tf + cfg.layers * tl for tf, tl in res]
    # images are dealt to the processes in order; a process runs its images back to back
    lanes = [0.0] * cores
    for t in per_image:
        k = lanes.index(min(lanes))
        lanes[k] += t
    t_batch = max(lanes)
    tokens = sum(cfg.tokens(gh, gw) for gh, gw in grids)
    return {"value": tokens / t_batch, "unit": "visual tokens/s", "cores": cores, "kind": "oracle",
            "images_per_s": len(grids) / t_batch, "seconds_per_batch": t_batch,
            "sample": (f"{len(grids)} images in {cores} single-threaded oracle processes (fp32): per image "
                       f"T_fixed and 1 of {cfg.layers} blocks timed on all its patches ({wall:.1f} s "
                       f"wall), each pass extrapolated as T_fixed + {cfg.layers} T_layer, batch time = "
                       f"the slowest process")}


def attention_traffic():
    """(bytes per launch, note) from the committed counter summary, or (None, reason)."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    fields = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    want = fields.get("attention.hip sha256")
    have = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
    if want != have:
        return None, "attention kernel changed since the counters were taken"
    return float(fields["HBM bytes per launch"]), "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled"


def copy_calibration(mib, reps=5):
    """A plain device copy of `mib` MiB, `reps` times: the reference the HBM byte counters are
    scaled by (run under rocprofv3 --pmc)."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "reps": reps, "bytes_read_per_copy": n * 4,
                      "bytes_written_per_copy": n * 4}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="v41_1024",
                    choices=["tiny", "one_layer", "v4_384", "v41_1024", "packed16"])
    ap.add_argument("--tower", default="base", choices=["base", "official"],
                    help="official: time the official-layer variant (RMSNorm, SwiGLU, erf GELU, "
                         "two-linear aligner) as the step instead of the LayerNorm/GELU tower")
    ap.add_argument("--no-variant", action="store_true",
                    help="skip the extra official-layer variant measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the 384-token and packed 16-image workloads measured after the headline")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel timing loop")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the encoder's hot path is "
                                   "measured on one MI355X (shard images across GPUs to scale "
                                   "out); run with --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch
    import multimodal_vision_encoder_amd as vit
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = synth.workload(args.workload)
    cfg, grids = wl.cfg, wl.grids
    if args.tower == "official":
        import dataclasses
        cfg = dataclasses.replace(cfg, norm_kind=1, mlp_kind=1, gelu_kind=1, aligner_hidden=cfg.out_hidden)
    N, M = wl.n_patches, wl.n_tokens
    log(f"workload {args.workload}: {len(grids)} image(s), {N} patches, {M} tokens")
    t = time.perf_counter()
    blob = synth.make_weights(cfg)
    px = synth.make_pixels(cfg, grids)
    log(f"inputs generated in {time.perf_counter() - t:.1f} s")

    enc = vit.Encoder(cfg, blob)
    enc.reserve(N)
    d_px = torch.from_numpy(px).cuda()
    out = torch.empty((M, cfg.out_hidden), dtype=torch.float32, device="cuda")
    # prompt: a run of text rows, then each image span; IMAGE positions are the placeholders
    types, src = vit.layout(grids)
    text_rows = 64
    R = text_rows + types.size
    rows = np.full(M, -1, np.int32)
    img_pos = np.nonzero(types == vit.TOK_IMAGE)[0]
    rows[src[img_pos]] = text_rows + img_pos
    embeds = torch.zeros((R, cfg.out_hidden), dtype=torch.bfloat16, device="cuda")

    def step():
        enc.encode(d_px, grids, out=out)
        vit.layout(grids)
        enc.overlay(embeds, rows, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    log(f"{args.steps} steps in {elapsed:.3f} s: {ms:.3f} ms/step")

    with ClockSampler() as clk:
        dist = pass_distribution(step, max(20, args.steps))
    log(f"event-timed passes: median {dist['median_ms']:.3f} ms, p10 {dist['p10_ms']:.3f}, "
        f"p90 {dist['p90_ms']:.3f}")

    fl = flops_per_pass(cfg, grids)
    total_flops = sum(fl.values())
    result = {
        "metric": "visual tokens/s + % bf16 MFMA peak, 32-layer ViT on 1024-token image",
        "value": M * args.steps / elapsed, "unit": "visual tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tower": args.tower, "images": len(grids),
                   "grids": grids if len(grids) <= 4 else f"{len(grids)} seeded grids",
                   "patches": N, "tokens": M, "layers": cfg.layers, "hidden": cfg.hidden,
                   "heads": cfg.heads, "mlp": cfg.mlp, "out_hidden": cfg.out_hidden,
                   "weights": "random N(0, 0.02) bf16", "pixels": "uniform u8"},
        "images_per_s": len(grids) * args.steps / elapsed,
        "tflops": total_flops / (ms * 1e-3) / 1e12,
        "mfma_frac": total_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "pass_ms": dist,
        "clock": clk.summary(),
    }
    pk = result["clock"]["peak_at_clock_tflops"]
    result["mfma_frac_at_clock"] = (total_flops / (dist["median_ms"] * 1e-3) / 1e12 / pk) if pk else None

    if not args.no_profile:
        enc.timing(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        tm = enc.timing_read()
        enc.timing(False)
        by = bytes_per_pass(cfg, grids, vit.vt_stride(grids))
        kernels = {}
        for k, (t_ms, n) in tm.items():
            if n == 0:
                continue
            per_step = t_ms / args.steps
            e = {"ms_per_step": per_step, "launches_per_step": n / args.steps,
                 "avg_launch_us": t_ms / n * 1e3}
            if k in fl:
                e["tflops"] = fl[k] / (per_step * 1e-3) / 1e12
                e["mfma_frac"] = e["tflops"] / PEAK_BF16_TFLOPS
            if k in by:
                e["gbs"] = by[k] / (per_step * 1e-3) / 1e9
                e["hbm_frac"] = e["gbs"] / PEAK_HBM_GBS
            kernels[k] = e
        if "layernorm" in kernels and args.tower == "base":
            try:
                kernels["layernorm"]["isolated"] = norm_isolated(enc, cfg, N)
            except Exception as exc:   # an extra figure: never lose the bench line for it
                torch.cuda.synchronize()
                kernels["layernorm"]["isolated"] = {"error": f"{type(exc).__name__}: {exc}"}
        result["kernels"] = kernels
        gemm_attn = ("qkv", "attention", "out_proj", "fc1", "fc2")
        # time of the GEMM and attention steps, the merge of the attention's key slices included;
        # the roofline below is the attention kernel alone (its event pair covers no merge)
        ga_ms = sum(kernels[k]["ms_per_step"] for k in gemm_attn + ("attn_merge",) if k in kernels)
        result["gemm_attention_mfma_frac"] = (sum(fl[k] for k in gemm_attn) / (ga_ms * 1e-3) / 1e12
                                              / PEAK_BF16_TFLOPS) if ga_ms else None
        a = kernels.get("attention")
        if a:
            per_launch = fl["attention"] / (cfg.layers or 1)
            achieved = per_launch / (a["avg_launch_us"] * 1e-6) / 1e12
            traffic, note = attention_traffic() if args.workload == "v41_1024" else (None, "other workload")
            result["roofline"] = {"kernel": "attention", "bound": "mfma", "achieved": achieved,
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                                  "traffic_unit": "bytes per launch", "traffic_note": note,
                                  "peak_at_clock": pk,
                                  "frac_at_clock": achieved / pk if pk else None}
        result["around_the_path"] = around_the_path(enc, cfg, grids, out, args.steps)
        log(json.dumps(kernels, indent=1))
        if args.workload in ("v4_384", "v41_1024", "packed16") and args.tower == "base" and not args.no_variant:
            result["official_layer_variant"] = official_variant(cfg, grids, args.steps, args.warmup)
    if args.workload == "v41_1024" and args.tower == "base" and not args.no_other_workloads:
        enc.close()
        # the 384-token V4 image and the packed 16-image batch, in the same run
        result["workloads"] = {w: measure_workload(w, args.steps, args.warmup) for w in ("v4_384", "packed16")}

    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(cfg, blob, px, grids)
        if "workloads" in result:
            log("timing the CPU oracle on the packed batch ...")
            pw = synth.workload("packed16")
            result["workloads"]["packed16"]["cpu_baseline"] = cpu_baseline_packed(pw.cfg, pw.grids)
    print(json.dumps(result), flush=True)
    enc.close()


if __name__ == "__main__":
    main()
