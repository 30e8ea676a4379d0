"""The byte accounting behind the bandwidth metric reproduces the pages' counts."""
import json
import os

from decode_persistent_megakernel_amd import accounting as A
import synth

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "byte_counts.json")))


def test_llama1b_bytes_match_tiles():
    c = synth.CONFIGS["llama1b"]
    layers = c.n_layers * A.layer_weight_bytes(c)
    full = layers + c.vocab * c.hidden * 2 + c.hidden * 2   # tied table stored once + final norm
    assert full == G["llama32_1b_bf16_weight_bytes"]["value"]
    assert A.kv_bytes_per_position(c) == G["llama32_1b_kv_bytes_per_position"]["value"]
    assert round(4096 * A.kv_bytes_per_position(c) / 1e6) == G["llama32_1b_kv_bytes_4096"]["value_mb"]
    mm = A.layer_weight_bytes(c) - 2 * c.hidden * 2
    assert round(mm / 1e6, 1) == G["llama32_1b_layer_matmul_mb"]["value_mb"]
    mlp = A.linear_bytes(2 * c.intermediate, c.hidden, 0) + A.linear_bytes(c.hidden, c.intermediate, 0)
    assert round(mlp / mm, 2) == G["llama32_1b_layer_matmul_mb"]["mlp_share"]
    assert round(A.head_bytes(c) / 1e6) == G["llama32_1b_lm_head_mb"]["value_mb"]
    assert round(A.head_bytes(c) / full, 1) == G["llama32_1b_lm_head_mb"]["share"]
    assert c.qkv_rows == G["llama32_1b_qkv_rows"]["value"]


def test_tinyllama_bytes_match_tinyinfer():
    c4 = synth.CONFIGS["tinyllama_int4"]
    c16 = synth.shrink(c4, weight_format=A.WF_BF16)
    # bytes a token reads: all layers and the head (no norms needed at this precision)
    b16 = c16.n_layers * A.layer_weight_bytes(c16) + A.head_bytes(c16)
    assert round(b16 / 1e9, 2) == G["tinyllama_bytes_per_token_16bit_gb"]["value_gb"]
    b4 = c4.n_layers * A.layer_weight_bytes(c4) + A.linear_bytes(c4.vocab, c4.hidden, A.WF_INT4_G64)
    assert round(b4 / 1e9, 2) == G["tinyllama_bytes_per_token_4bit_gb"]["value_gb"]
    assert c4.qkv_rows == G["tinyllama_qkv_rows"]["value"]


def test_model_storage_matches_accounting():
    for name in ("tiny",):
        c = synth.CONFIGS[name]
        m = synth.make_model(c)
        assert m.nbytes() == c.n_layers * A.layer_weight_bytes(c) + c.vocab * c.hidden * 2 + c.hidden * 2


def test_step_bytes_grow_by_one_kv_row_per_position():
    c = synth.CONFIGS["llama1b"]
    assert A.step_bytes(c, 513) - A.step_bytes(c, 512) == A.kv_bytes_per_position(c)
    assert abs(A.mean_step_bytes(c, 512, 128) - 2491069440) < 1
