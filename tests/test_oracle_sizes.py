"""Closed-form cache sizes against the numbers printed on the pages
(tests/golden/page_numbers.json, each entry with its citation)."""
import json
import os

import pytest

from oracle import mla_oracle as O

with open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")) as f:
    G = json.load(f)


def test_deepseek_values_per_token():
    e = G["deepseek_v3_values_per_token_layer"]
    assert O.latent_values_per_token(**e["dims"]) == e["value"]


def test_glm53_values_and_bytes():
    e = G["glm53_flash_values_per_token_layer"]
    v = O.latent_values_per_token(**e["dims"])
    assert v == e["value"]
    b = G["glm53_flash_bytes_per_token"]
    assert b["dims"]["latent_layers"] * v * b["dims"]["bytes_per_value"] == b["value"]
    gb = G["glm53_flash_gb_at_1m_tokens"]
    assert abs(b["value"] * gb["tokens"] / 1e9 - gb["value"]) <= gb["tolerance_rel"] * gb["value"]
    after = G["glm53_flash_after_estimate"]
    got = b["value"] * after["tokens"] / 1e9
    assert round(got, 1) == after["value_gb"]
    assert after["tokens"] // 1000 == after["tokens_k"]


def test_absorb_reduction_ratio():
    e = G["absorb_kv_reduction"]
    full = O.full_head_values_per_token(128, 128, 64, 128)
    lat = O.latent_values_per_token(512, 64)
    assert abs(full / lat - e["value"]) <= e["tolerance_rel"] * e["value"]


@pytest.mark.parametrize("r,g,d_r,d_idx,want", [
    (512, 32, 64, 0, 320),     # 128 codes + 64 scale/zero + 128 rope
    (512, 32, 64, 64, 448),    # + 128 bytes of bf16 indexer key
    (64, 16, 16, 0, 64),       # 16 + 16 + 32
])
def test_int2_physical_bytes(r, g, d_r, d_idx, want):
    assert O.int2_cache_bytes_per_token(r, g, d_r, d_idx) == want
    # logical entry is r + d_r (+ d_idx) values
    assert O.latent_values_per_token(r, d_r, d_idx) == r + d_r + d_idx
