"""The byte model behind the bench's GB/s figure, pinned to the pages' worked examples."""
import json
import os

import pytest

from gqa_decode_attention_mqa_amd.traffic import (decode_step_flops, decode_step_kv_bytes, decode_step_quant_bytes,
                                                  kv_cache_bytes, max_context_tokens)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_cache_worked_examples.json")))


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: c["name"])
def test_kv_cache_bytes_worked_examples(case):
    got = kv_cache_bytes(case["layers"], case["kv_heads"], case["head_dim"], case["bytes_per_elem"],
                         case["tokens"], case["batch"])
    if case.get("keys_only"):
        got //= 2
    if case["rel_tol"] == 0.0:
        assert got == case["printed"]
    else:
        assert abs(got - case["printed"]) <= case["rel_tol"] * case["printed"]


@pytest.mark.parametrize("case", GOLDEN["max_context"], ids=lambda c: c["name"])
def test_table1_max_context(case):
    got = max_context_tokens(case["hbm_bytes"], case["kv_fraction"], case["batch"], case["layers"],
                             case["kv_heads"], case["head_dim"], case["bytes_per_elem"])
    assert abs(got - case["printed"]) <= case["rel_tol"] * case["printed"]


def test_decode_step_bytes_for_the_five_workloads():
    # valid K+V bytes per step: 2 (K and V) * Hkv * D * 2 bytes * sum(len)
    assert decode_step_kv_bytes([128], 1, 64) == 32768
    assert decode_step_kv_bytes([2048] * 64, 1, 256) == 128 * 2 ** 20
    assert decode_step_kv_bytes([4096] * 32, 8, 128) == 512 * 2 ** 20
    assert decode_step_kv_bytes([131072] * 4, 1, 256) == 512 * 2 ** 20
    assert decode_step_kv_bytes([1, 8192], 8, 128) == 8193 * 4096
    assert decode_step_flops([2048] * 64, 48, 256) == 4 * 48 * 256 * 2048 * 64


def test_decode_step_bytes_of_an_8bit_cache():
    # per position and kv head: D codes of K and of V (one byte each) plus one fp32 scale each
    assert decode_step_quant_bytes([2048] * 64, 1, 256) == 64 * 2048 * (512 + 8)
    assert decode_step_quant_bytes([4096] * 32, 8, 128) == 32 * 4096 * 8 * 264
    # half of the bf16 bytes plus the scales
    assert decode_step_quant_bytes([100], 2, 64) == decode_step_kv_bytes([100], 2, 64) // 2 + 100 * 2 * 8
