"""The byte and roofline calculator against the pages' printed arithmetic
(tests/golden/speed_of_light.json)."""
import json
import os

import pytest

import synth
from decode_megakernel_02_amd import roofline as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "speed_of_light.json")))


def test_llama_1b_weight_bytes_match_printed_size():
    g = GOLD["llama_1b_h100"]
    gb = R.weight_bytes_read(synth.LLAMA_1B, 1) / 1e9
    assert abs(gb - g["weights_gb"]) / g["weights_gb"] < 0.01  # printed as "about 2.48 GB"


def test_llama_1b_h100_floor_and_rate():
    g = GOLD["llama_1b_h100"]
    us = R.floor_us(R.weight_bytes_read(synth.LLAMA_1B, 1), g["bandwidth_tbps"] * 1000)
    assert abs(us - g["floor_us"]) / g["floor_us"] < 0.01
    assert abs(1e6 / us - g["tokens_per_s"]) / g["tokens_per_s"] < 0.02


def test_llama_1b_b200_rate_close_to_3000():
    g = GOLD["llama_1b_b200"]
    rate = 1e6 / R.floor_us(R.weight_bytes_read(synth.LLAMA_1B, 1), g["bandwidth_tbps_assumed"] * 1000)
    assert 0.9 * g["tokens_per_s_close_to"] < rate < 1.1 * 3300


@pytest.mark.parametrize("row", GOLD["gemma_26b_a4b"]["rows"], ids=lambda r: r["hardware"])
def test_speed_of_light_table(row):
    # tokens/s = bandwidth / bytes per token; the printed rows imply ~7.84 GB
    bytes_per_token = GOLD["gemma_26b_a4b"]["gb_per_token"] * 1e9
    rate = 1e6 / R.floor_us(bytes_per_token, row["bandwidth_tbps"] * 1000)
    assert abs(rate - row["tokens_per_s"]) / row["tokens_per_s"] < 0.01


def test_mpk_floor():
    g = GOLD["mpk_a100"]
    assert abs(R.floor_us(g["weights_gb"] * 1e9, g["bandwidth_tbps"] * 1000) / 1000 - g["floor_ms"]) < 1e-9


def test_launch_stall_cap():
    g = GOLD["launch_stall_cap"]
    floor = GOLD["llama_1b_h100"]["floor_us"]
    stall = g["launches_per_layer"] * g["layers"] * g["stall_us"]
    assert abs(1e6 / (floor + stall) - g["forwards_per_s_about"]) / g["forwards_per_s_about"] < 0.01


def test_kv_bytes_and_mean_keys():
    m = synth.LLAMA_1B
    # 32 KB of K+V per position per row for the 1B shape
    assert R.kv_bytes_read(m, 1, 1) == 32768
    # steps 0..255 after a 1024-token prompt attend 1025..1280 keys
    assert R.mean_keys(1024, 0, 256) == (1025 + 1280) / 2
    total = R.step_bytes(m, 1, R.mean_keys(1024, 0, 256))
    assert abs(total - 2.4716e9 - 37.77e6) / total < 1e-3


def test_8b_model_about_16_gb_and_bytes_read_per_step():
    # untied: the model stores ~16 GB, a step reads the LM head but only B embedding rows
    assert abs(synth.LLAMA_8B.weight_bytes() / 1e9 - 16.06) < 0.01
    assert R.weight_bytes_read(synth.LLAMA_8B, 1) == 15009857536
