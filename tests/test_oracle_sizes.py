"""KV-cache size closed forms ("Out-of-Core Flash Streaming & Speculative Decode (1M Context)",
Sec. 1 and Sec. 5; "Core Architecture & The 4-Brick Pipeline", Sec. 5) against the numbers the
pages print (tests/golden/kv_cache_sizes.json)."""
import json
import os

import numpy as np

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_cache_sizes.json")))
P = GOLD["printed"]
W = GOLD["workload"]


def test_printed_totals_are_one_32_head_layer(orc):
    f16 = orc.kv_bytes(1, W["heads"], W["tokens"], W["head_dim"], "f16")
    q8 = orc.kv_bytes(1, W["heads"], W["tokens"], W["head_dim"], "q8_0")
    assert f16 == 8_589_934_592 and round(f16 / 1e9, 2) == P["f16_total_GB"]
    assert q8 == 4_563_402_752 and round(q8 / 1e9, 2) == P["q8_0_total_GB"]


def test_printed_formula_is_16x_the_printed_total(orc):
    layers = W["layers_as_labelled"]
    f16 = orc.kv_bytes(layers, W["heads"], W["tokens"], W["head_dim"], "f16")
    q8 = orc.kv_bytes(layers, W["heads"], W["tokens"], W["head_dim"], "q8_0")
    assert f16 == 16 * 8_589_934_592 and q8 == 16 * 4_563_402_752


def test_printed_single_layer_is_one_sixteenth(orc):
    f16 = orc.kv_bytes(1, W["heads"], W["tokens"], W["head_dim"], "f16") // 16
    q8 = orc.kv_bytes(1, W["heads"], W["tokens"], W["head_dim"], "q8_0") // 16
    assert round(f16 / 1e6, 2) == P["f16_single_layer_MB"]
    assert round(q8 / 1e6, 2) == P["q8_0_single_layer_MB"]


def test_block_and_reduction(orc):
    x = np.zeros((1, 32), dtype=np.float32)
    assert orc.q8_0_pack(x).shape[-1] == P["q8_0_block_bytes"]
    ratio = orc.kv_bytes(1, 1, 1, 64, "q8_0") / orc.kv_bytes(1, 1, 1, 64, "f16")
    assert ratio == 68 / 128
    assert round((1 - ratio) * 100, 2) == P["q8_0_reduction_percent"]


def test_million_token_figure(orc):
    # Sec. 5 quotes 4.3 GB for 1,000,000 tokens of Q8_0 KV (one 32-head layer, truncated)
    q8 = orc.kv_bytes(1, W["heads"], 1_000_000, W["head_dim"], "q8_0")
    assert int(q8 / 1e8) / 10 == P["q8_0_at_1e6_tokens_GB"]
