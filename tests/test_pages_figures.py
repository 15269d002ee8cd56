"""Host-side arithmetic pinned to numbers the pages print (tests/golden)."""

import json
import math
import os

import pytest
import torch

import oracle
import synthetic_inputs as si

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_score_matrix_memory_table():
    g = GOLD["score_matrix_memory"]
    assert si.score_matrix_bytes(1, 1, 4096, g["elem_bytes"]) == g["per_head_bytes_at_4096"]
    for n, gib in g["per_layer_GiB"].items():
        assert si.score_matrix_bytes(1, g["heads"], int(n), g["elem_bytes"]) == gib * 2**30


def test_yolo_sequence_and_block_count():
    g = GOLD["yolo_tiling"]
    assert g["map_h"] * g["map_w"] == g["seq_len"] == si.WORKLOADS["c1_yolo_n400"].N
    assert math.ceil(g["seq_len"] / g["block"]) == g["blocks"]


def test_gqa_cache_cut():
    g = GOLD["gqa_cache"]
    assert 1 - g["kv_heads"] / g["q_heads"] == g["cache_cut"]


def test_workload_flop_and_byte_counts():
    w = si.WORKLOADS["c3_causal_7b"]
    assert w.pairs() == 4096 * 4097 // 2
    assert abs(w.fwd_flops() - 4 * 128 * 4096 * 4097 / 2 * 64) < 1
    assert w.bwd_flops() == 2.5 * w.fwd_flops()
    assert w.fwd_bytes() == 2 * (64 * 4096 * 128 * 2) + 2 * 2 * 32 * 4096 * 128 * 2 + 2 * 32 * 4096 * 4
    w1 = si.WORKLOADS["c1_yolo_n400"]
    assert w1.pairs() == 400 * 400
    assert abs(w1.scale - 0.125) == 0
    assert si.WORKLOADS["c5_bwd_d80"].scale == float(torch.tensor(1 / math.sqrt(80), dtype=torch.float32))


def test_inputs_are_seeded_bf16_and_ordered():
    a = si.make_inputs(1, 2, 1, 5, 8, 7, with_do=True)
    b = si.make_inputs(1, 2, 1, 5, 8, 7, with_do=True)
    for key in ("q", "k", "v", "do"):
        assert a[key].dtype == torch.bfloat16 and a[key].is_contiguous()
        assert torch.equal(a[key], b[key])
    assert a["k"].shape == (1, 1, 5, 8) and a["do"].shape == (1, 2, 5, 8)
    g = torch.Generator().manual_seed(7)
    q = torch.randn((1, 2, 5, 8), generator=g).to(torch.bfloat16)
    assert torch.equal(q, a["q"])


@pytest.mark.parametrize("N,W", [(1, 1), (10, 1), (10, 3), (10, 10), (10, 25), (333, 64), (1000, 999)])
def test_window_pair_count(N, W):
    """The flop credit of a sliding-window workload counts exactly the pairs the
    oracle's mask allows (keys i-W < j <= i)."""
    w = si.Workload("t", 1, 1, 1, N, 64, True, False, 0, window=W)
    assert w.pairs() == int(oracle.allowed_mask(0, N, N, True, W).sum())
