"""bench.py's host-side contract, without a GPU: the one-GPU refusal and the algorithmic work
it divides by."""
import json
import os
import subprocess
import sys
from dataclasses import replace

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_flops_of_the_1024_token_image():
    """2 n 588 D + L (8 n D^2 + 4 n D F + 4 n^2 D) + 2 m 9D D_lm at n = 9216, m = 1024."""
    n, m, D, F, L, Dl = 9216, 1024, 1024, 4096, 32, 5120
    want = 2 * n * 588 * D + L * (8 * n * D * D + 4 * n * D * F + 4 * n * n * D) + 2 * m * 9 * D * Dl
    fl = bench.flops_per_pass(synth.V41, [(96, 96)])
    assert sum(fl.values()) == want
    assert abs(want / 1e12 - 18.662) < 1e-3
    assert fl["attention"] == L * 4 * n * n * D


def test_flops_of_the_official_layer_variant():
    """SwiGLU doubles the first MLP projection; the aligner adds its second projection."""
    n, m, D, F, L, Dl = 9216, 1024, 1024, 4096, 32, 5120
    cfg = replace(synth.V41, norm_kind=1, mlp_kind=1, gelu_kind=1, aligner_hidden=Dl)
    fl = bench.flops_per_pass(cfg, [(96, 96)])
    assert fl["fc1"] == L * 2 * n * D * 2 * F
    assert fl["projector"] == 2 * m * 9 * D * Dl + 2 * m * Dl * Dl
    assert abs(sum(fl.values()) / 1e12 - 21.190) < 1e-3


def test_memory_bound_bytes():
    """LayerNorm: every one of the 2 L + 1 norms reads [N][D] bf16 and writes its output (the
    residual adds run in the out-projection and fc2 epilogues); overlay: fp32 rows in, bf16 rows
    out, one int32 index per row."""
    n, D, L, m, Dl = 9216, 1024, 32, 1024, 5120
    by = bench.bytes_per_pass(synth.V41, [(96, 96)], 9216)
    assert by["layernorm"] == (2 * L + 1) * 2 * n * D * 2
    assert by["overlay"] == m * Dl * 6 + 4 * m
