"""The oracle's pins have teeth: plant one plausible mistake at a time in a
copy of oracle.c (CPU only), build it, and require at least one pin to fail."""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "rope_sign": ("v[i] = a * c - b * s;", "v[i] = a * c + b * s;"),
    "rope_freq": ("pow(base, -2.0 * (double)i / (double)d)", "pow(base, -1.0 * (double)i / (double)d)"),
    "rope_pairing": ("double a = v[i], b = v[i + half];", "double a = v[i], b = v[(i + 1) % d];"),
    "nibble_order": ("(k % 2 == 0) ? (byte & 0xf) : (byte >> 4)", "(k % 2 == 0) ? (byte >> 4) : (byte & 0xf)"),
    "int4_offset": ("scale * (double)(u - 8)", "scale * (double)(u - 7)"),
    "scale_group": ("s[r * (cols / 64) + k / 64]", "s[r * (cols / 64) + k / 128]"),
    "gqa_mapping": ("int32_t g = hh / group;", "int32_t g = hh % nkv;"),
    "attn_scale": ("1.0 / sqrt((double)d)", "1.0 / (double)d"),
    "softmax_no_max": ("sc[t] = exp(sc[t] - m);", "sc[t] = exp(sc[t] - 0.5 * m);"),
    "attn_excludes_current": ("Vl + (int64_t)g * ctx * d, pos + 1,", "Vl + (int64_t)g * ctx * d, pos > 0 ? pos : 1,"),
    "rms_no_eps": ("sqrt(ss / (double)n + eps)", "sqrt(ss / (double)n)"),
    "rms_no_gain": ("y[i] = x[i] * inv * orc_bf16_value(gain[i]);", "y[i] = x[i] * inv;"),
    "silu_sign": ("z / (1.0 + exp(-z))", "z / (1.0 + exp(z))"),
    "swiglu_swap": ("orc_silu(gu[r]) * gu[I + r]", "orc_silu(gu[I + r]) * gu[r]"),
    "residual_o_dropped": ("for (int32_t i = 0; i < H; ++i) x[i] += y[i];\n        if (tr && tr->x_mid)",
                           "for (int32_t i = 0; i < H; ++i) x[i] = y[i];\n        if (tr && tr->x_mid)"),
    "bias_dropped": ("qkv[r] += orc_bf16_value(L->b_qkv[r]);", "qkv[r] += 0.0;"),
    "k_not_roped": ("for (int32_t g = 0; g < nkv; ++g) orc_rope(qkv + qd + g * d, d, pos, c->rope_theta);", ""),
    "v_from_k": ("orc_round_bf16(qkv[qd + kvd + g * d + i]);", "orc_round_bf16(qkv[qd + g * d + i]);"),
    "argmax_last_tie": ("if (best < 0 || v > bv)", "if (best < 0 || v >= bv)"),
    "bf16_round_truncates": ("if (rest > 0x8000u || (rest == 0x8000u && (top & 1u))) top += 1u;", ""),
    "route_last_tie": ("if (best < 0 || bv < v)", "if (best < 0 || bv <= v)"),
    "route_unnormalised": ("weights[j] = exp(z[best] - m) / sum;", "weights[j] = exp(z[best] - m);"),
    "route_smallest": ("if (best < 0 || bv < v)", "if (best < 0 || bv > v)"),
    "moe_swiglu_swap": ("gu[I + r] * orc_silu(gu[r])", "gu[r] * orc_silu(gu[I + r])"),
    "moe_unweighted": ("ysum[i] += wts[j] * y[i];", "ysum[i] += y[i];"),
    "moe_residual_dropped": ("for (int32_t i = 0; i < H; ++i) x[i] += ysum[i];",
                             "for (int32_t i = 0; i < H; ++i) x[i] = ysum[i];"),
    "moe_expert_offset": ("return (const uint16_t*)w + (int64_t)e * rows * cols;",
                          "return (const uint16_t*)w + (int64_t)e * cols;"),
    "moe_scale_offset": ("return s + (int64_t)e * rows * (cols / 64);", "return s;"),
}

PINS = [
    (P.test_round_bf16_matches_torch_rne, {}),
    (P.test_rmsnorm_constant_vector_closed_form, {"c": 1e-3}),
    (P.test_rmsnorm_scale_invariance_and_rms_one, {}),
    (P.test_linear_one_hot_returns_column, {}),
    (P.test_int4_nibble_order_hand_built, {}),
    (P.test_int4_one_hot_is_exact_dequant_all_codes_and_scales, {}),
    (P.test_rope_preserves_pair_norms, {}),
    (P.test_rope_relative_position, {}),
    (P.test_rope_d2_is_plane_rotation_and_pairs_are_half_split, {}),
    (P.test_attention_single_entry_returns_v_exactly, {}),
    (P.test_attention_brute_force_scipy_softmax, {"n": 5}),
    (P.test_silu_properties_and_library, {}),
    (P.test_argmax_lowest_id_on_ties_and_errors, {}),
    (P.test_zero_block_model_reduces_to_embedding_dot, {}),
    (P.test_decode_matches_full_sequence_reference, {"name": "tiny", "over": {}}),
    (P.test_decode_matches_full_sequence_reference,
     {"name": "gqa4_bias_int4", "over": dict(n_q_heads=8, n_kv_heads=2, qkv_bias=True,
                                             weight_format=oracle.WF_INT4_G64, tied=False, hidden=128,
                                             intermediate=192, vocab=500, head_dim=32)}),
    (P.test_route_closed_form_example, {}),
    (P.test_moe_identical_experts_reduce_to_dense, {}),
    (P.test_moe_decode_matches_full_sequence_reference, {"name": "moe_bf16", "over": dict(n_experts=8, top_k=2)}),
    (P.test_moe_decode_matches_full_sequence_reference,
     {"name": "moe_int4", "over": dict(n_experts=6, top_k=3, weight_format=oracle.WF_INT4_G64, hidden=128,
                                       intermediate=192, tied=False)}),
]


def _build_mutant(name, tmpdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = os.path.join(tmpdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmpdir, f"{name}.so")
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                           "-I", os.path.dirname(SRC), "-o", so, path, "-lm"])
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    with tempfile.TemporaryDirectory() as d:
        so = _build_mutant(name, d)
        real = oracle.lib()
        monkeypatch.setattr(oracle, "_SO", so)
        monkeypatch.setattr(oracle, "_lib", None)
        caught = []
        try:
            for fn, kw in PINS:
                try:
                    fn(**kw)
                except (AssertionError, ValueError, FloatingPointError):
                    caught.append(fn.__name__)
                    break
        finally:
            monkeypatch.setattr(oracle, "_lib", real)
        assert caught, f"no pin caught mutant {name}"
