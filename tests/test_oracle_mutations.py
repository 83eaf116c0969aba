"""The pins must be able to fail: each case plants one plausible mistake in a private copy of
the oracle's C source (on the CPU, in a temporary directory), loads it in place of the real
oracle and checks that the named pin test then fails."""
import os
import subprocess

import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "vit_oracle.c")

MUTATIONS = [
    ("rope sign", "real na = a * c - b * s;", "real na = a * c + b * s;",
     pins.test_rope_vs_complex_rotation_fp64),
    ("rope interleaved angles", "double pos = i < quarter ? (double)h : (double)w;",
     "double pos = (i % 2) ? (double)w : (double)h; j = i / 2;", pins.test_rope_axis_blocks),
    ("rope wrong frequency", "double f = pow(base, -2.0 * (double)j / (double)half);",
     "double f = pow(base, -1.0 * (double)j / (double)half);", pins.test_rope_vs_complex_rotation_fp64),
    ("layernorm unbiased variance", "real var = ss / (real)D;", "real var = ss / (real)(D - 1);",
     lambda: pins.test_layernorm_vs_torch("f64")),
    ("layernorm eps outside sqrt", "sqrt((double)(var + eps))", "(sqrt((double)var) + eps)",
     lambda: pins.test_layernorm_vs_torch("f64")),
    ("attention missing scale", "p[j] = acc * scale;", "p[j] = acc;", pins.test_softmax_rows_sum_to_one),
    ("attention scale dropped", "s[j] *= scale;", "s[j] *= 1;", pins.test_attention_vs_torch_sdpa_fp64),
    ("attention drops the first key from P.V",
     "for (int64_t j = 0; j < n; ++j) {\n                const real pj = s[j];",
     "for (int64_t j = 1; j < n; ++j) {\n                const real pj = s[j];",
     pins.test_attention_vs_torch_sdpa_fp64),
    ("attention reads q as k", "ko = D + qo", "ko = qo", pins.test_attention_vs_torch_sdpa_fp64),
    ("merge row-major unfold", "dst[(int64_t)c * mm + k] = src[c];", "dst[(int64_t)k * D + c] = src[c];",
     pins.test_merge_matches_torch_unfold_with_padding),
    ("merge pads the flattened rows",
     "int t = (sy / m) * mw + (sx / m);\n            int k = (sy % m) * m + (sx % m);",
     "int f_ = sy * gw + sx, yy = f_ / (mw * m), xx = f_ % (mw * m);\n"
     "            int t = (yy / m) * mw + (xx / m);\n            int k = (yy % m) * m + (xx % m);",
     pins.test_merge_matches_torch_unfold_with_padding),
    ("patchify HWC inside the row", "row[c * ps * ps + y * ps + x]", "row[(y * ps + x) * 3 + c]",
     lambda: pins.test_patchify_closed_form(pins.synth.V41)),
    ("patchify x/y swapped", "int64_t py = (int64_t)gy * ps + y, px = (int64_t)gx * ps + x;",
     "int64_t py = (int64_t)gy * ps + x, px = (int64_t)gx * ps + y;",
     lambda: pins.test_patchify_closed_form(pins.synth.V41)),
    ("gelu constant", "const real k1 = (real)0.044715;", "const real k1 = (real)0.04471;",
     pins.test_gelu_tanh_vs_torch_and_identities),
    ("linear drops bias", "real v = acc[j] + (bias ? bias[j] : 0);", "real v = acc[j];",
     lambda: pins.test_linear_vs_numpy_fp64("f64")),
    ("linear skips last k", "for (int k = 0; k < K; ++k) {", "for (int k = 0; k < K - 1; ++k) {",
     lambda: pins.test_linear_vs_numpy_fp64("f64")),
    ("rmsnorm eps outside sqrt", "sqrt((double)(ms + eps))", "(sqrt((double)ms) + eps)",
     lambda: pins.test_rmsnorm_vs_torch("f64")),
    ("rmsnorm divides by D - 1", "real ms = ss / (real)D;", "real ms = ss / (real)(D - 1);",
     lambda: pins.test_rmsnorm_vs_torch("f64")),
    ("silu as sigmoid", "return u / ((real)1 + (ORC_IS_DOUBLE ? (real)exp(-(double)u)",
     "return (real)1 / ((real)1 + (ORC_IS_DOUBLE ? (real)exp(-(double)u)", pins.test_silu_closed_forms),
    ("swiglu gates the wrong operand", "out[i] = R(silu(g[i]) * u[i]);", "out[i] = R(silu(u[i]) * g[i]);",
     pins.test_swiglu_gate_and_up_roles),
    ("gelu erf without the sqrt 2", "(real)erf((double)(u / r2))", "(real)erf((double)u)",
     pins.test_gelu_erf_vs_torch_and_closed_form),
    ("linear erf act takes the tanh form", "else if (act == 2) v = gelu_erf(v);",
     "else if (act == 2) v = gelu_tanh(v);", pins.test_linear_gelu_erf_unrounded_and_rounded),
    ("bf16 truncation", "v.u += 0x7FFFu + ((v.u >> 16) & 1u);", "v.u += 0;",
     pins.test_bf16_rounding_matches_torch),
    ("bf16 ties away", "v.u += 0x7FFFu + ((v.u >> 16) & 1u);", "v.u += 0x8000u;",
     pins.test_bf16_rounding_matches_torch),
]


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_mutation(name, old, new, pin, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {old}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    libs = {}
    for prec, real in (("f32", "float"), ("f64", "double")):
        path = str(tmp_path / f"liboracle_{prec}.so")
        subprocess.check_call(["gcc", *oracle._FLAGS, f"-DORC_REAL={real}", "-o", path,
                               str(mutant), "-lm"])
        libs[prec] = path
    monkeypatch.setattr(oracle, "_LIBS", libs)
    monkeypatch.setattr(oracle, "_libs", {})
    with pytest.raises(AssertionError):
        pin()
