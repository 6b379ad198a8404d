"""The pages' printed size figures (tests/golden/page_figures.json, each cited there) pin the
serving layer shape used everywhere else: a 4 MiB fp32 state per sequence per layer is
H*P*N*4 bytes at 128 heads x 64 x 128, and it equals 8,192 fp8 KV tokens of 0.5 KiB."""
import json
import os

import workload

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_state_size_is_serving_shape():
    s = workload.SERVING
    assert s["H"] * s["P"] * s["N"] * 4 == GOLD["fp32_state_bytes_per_sequence_per_layer"]
    shp = GOLD["serving_layer_shape"]
    assert (shp["nheads"], shp["headdim"], shp["dstate"]) == (s["H"], s["P"], s["N"])
    assert s["L"] == GOLD["buffer_len"]


def test_kv_equivalents():
    st = GOLD["fp32_state_bytes_per_sequence_per_layer"]
    kv = GOLD["fp8_kv_bytes_per_token"]
    assert st // kv == GOLD["state_as_kv_tokens"]
    assert GOLD["state_as_kv_tokens"] * GOLD["ssm_layers_per_attention_layer"] == \
        GOLD["state_as_kv_tokens_per_attention_layer"]
    assert 2 * GOLD["state_as_kv_tokens_per_attention_layer"] == \
        GOLD["load_and_store_as_kv_tokens_per_attention_layer"]
