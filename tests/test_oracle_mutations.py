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


# ------------------------------------------------------------------------------------------
# mistakes in the oracle's Python layer: the order of the steps and the pixel constants
# ------------------------------------------------------------------------------------------
import types

import tests.test_oracle_composition as comp

PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")
_LN_CASE = lambda: comp.test_encoder_equals_bruteforce_composition(*comp.CASES[0])
_PAD_CASE = lambda: comp.test_encoder_equals_bruteforce_composition(*comp.CASES[1])
_OFFICIAL_CASE = lambda: comp.test_encoder_equals_bruteforce_composition(*comp.CASES[2])
_ALIGNER_CASE = lambda: comp.test_encoder_equals_bruteforce_composition(*comp.CASES[3])

PY_MUTATIONS = [
    ("residual after attention kept unrounded", "x = add_round(x, a, prec)", "x = x + a",
     comp.test_constant_values_block_closed_form),
    ("residual after the MLP kept unrounded", "x = add_round(x, f, prec)", "x = x + f",
     comp.test_uniform_image_block_closed_form),
    ("block without LN1", 'ln = norm(cfg, x, W, f"l{l}.ln1", **kw)', "ln = x",
     comp.test_uniform_image_block_closed_form),
    ("block without LN2", 'ln2 = norm(cfg, x, W, f"l{l}.ln2", **kw)', "ln2 = x",
     comp.test_constant_values_block_closed_form),
    ("post-norm block", "x = add_round(x, a, prec)",
     'x = norm(cfg, add_round(x, a, prec), W, f"l{l}.ln1", **kw)', _LN_CASE),
    ("sublayer output replaces the residual", "x = add_round(x, f, prec)", "x = f",
     comp.test_zero_output_projections_keep_the_patch_embedding),
    ("no final norm", 'y = norm(cfg, x, W, "lnf", **kw)', "y = x",
     comp.test_zero_output_projections_keep_the_patch_embedding),
    ("RoPE skipped", "qkv = rope_qk(qkv, gw, D, H, cfg.rope_base, **kw)", "qkv = qkv", _LN_CASE),
    ("RoPE given the grid height as the row length", "qkv = rope_qk(qkv, gw, D, H",
     "qkv = rope_qk(qkv, gh, D, H", _LN_CASE),
    ("merge of the transposed grid", "A = merge(y, gh, gw, cfg.merge, prec)",
     "A = merge(y, gw, gh, cfg.merge, prec)", _PAD_CASE),
    ("SwiGLU gate and up exchanged", 'h = swiglu(g, u, kw.get("prec", "f32"))',
     'h = swiglu(u, g, kw.get("prec", "f32"))', _OFFICIAL_CASE),
    ("aligner inner layer left unrounded", 'a1 = linear(A, None, W["proj.b"], act=act, Wt=W.T("proj.w"), **kw)',
     'a1 = linear(A, None, W["proj.b"], act=act, round_out=False, Wt=W.T("proj.w"), **kw)', _ALIGNER_CASE),
    ("V4 layout without the row-pair interleave",
     "            for c in range(mw):\n                for r in rows_of_pair:",
     "            for r in rows_of_pair:\n                for c in range(mw):",
     lambda: __import__("tests.test_layout_v4", fromlist=["x"]).test_v4_layout_closed_forms([(6, 9), (3, 3)])),
    ("V4 layout without compress_pad", "        while len(span_t) % align:", "        while False:",
     lambda: __import__("tests.test_layout_v4", fromlist=["x"]).test_v4_layout_closed_forms([(6, 9), (3, 3)])),
    ("pixel map with mean and std exchanged",
     "m32 = [float(np.float32(m)) for m in mean]\n    s32 = [float(np.float32(sd)) for sd in std]",
     "m32 = [float(np.float32(m)) for m in std]\n    s32 = [float(np.float32(sd)) for sd in mean]",
     comp.test_clip_pixel_map_endpoints_by_hand),
    ("pixel map without the 1/255", "s = np.array([1.0 / (255.0 * sd) for sd in s32], dtype=np.float32)",
     "s = np.array([1.0 / sd for sd in s32], dtype=np.float32)", comp.test_clip_pixel_map_endpoints_by_hand),
]


@pytest.mark.parametrize("name,old,new,pin", PY_MUTATIONS, ids=[m[0] for m in PY_MUTATIONS])
def test_pin_catches_python_mutation(name, old, new, pin, monkeypatch):
    """The oracle's Python module with one mistake planted is executed as a private module,
    and its functions replace the real module's for the duration of the named pin."""
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = PY_SRC
    exec(compile(src.replace(old, new), PY_SRC + " (mutant)", "exec"), mod.__dict__)
    for k, v in vars(mod).items():
        if isinstance(v, (types.FunctionType, type)) and getattr(v, "__module__", None) == "oracle_mutant":
            monkeypatch.setattr(oracle, k, v)
    with pytest.raises(AssertionError):
        pin()


@pytest.mark.parametrize("pin", sorted({m[3] for m in PY_MUTATIONS}, key=id), ids=lambda p: getattr(p, "__name__", "case"))
def test_python_mutation_harness_control(pin, monkeypatch):
    """Control: the same harness with no mistake planted leaves every pin passing."""
    src = open(PY_SRC).read()
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = PY_SRC
    exec(compile(src, PY_SRC + " (copy)", "exec"), mod.__dict__)
    for k, v in vars(mod).items():
        if isinstance(v, (types.FunctionType, type)) and getattr(v, "__module__", None) == "oracle_mutant":
            monkeypatch.setattr(oracle, k, v)
    pin()
