"""The work counts behind the roofline (CPU only): against the page's per-token figure and
against brute-force enumeration of the unmasked (row, key) pairs and live pool rows."""
import json
import os

import pytest

import workloads
from workloads.accounting import attention_work, kv_bytes_per_token, write_work

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_kv_bytes_per_token_page_figures():
    g = json.load(open(os.path.join(GOLDEN, "kv_bytes_per_token.json")))
    for c in g["cases"]:
        assert kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["bytes"]) == c["per_token"]
        if "tokens" in c:
            assert round(c["per_token"] * c["tokens"] / 2 ** 30, 1) == c["gib_approx"]


def _brute(batch, ids, window):
    pairs, slots = 0, set()
    for r in ids:
        req = batch.requests[r]
        for i in range(req.new):
            pos = req.computed + i
            for key in range(pos + 1):
                if window > 0 and key <= pos - window:
                    continue
                pairs += 1
                slots.add(req.blocks[key // batch.block_size] * batch.block_size + key % batch.block_size)
    return pairs, len(slots)


@pytest.mark.parametrize("window", [0, 1, 3, 17, 64, 1000])
def test_attention_work_matches_enumeration(window):
    b = workloads.small_batch([(30, 4), (9, 9), (64, 1), (17, 17), (12, 1)], dtype="bf16", num_heads=8,
                              num_kv_heads=2, head_dim=16, block_size=4, seed=3, shared_prefix_blocks=2)
    for ids in (None, [0, 2], [1, 3]):
        sel = list(range(len(b.requests))) if ids is None else ids
        w = attention_work(b, ids, window=window)
        pairs, live = _brute(b, sel, window)
        assert w["scores_per_head"] == pairs
        assert w["flops"] == 4.0 * b.num_heads * b.head_dim * pairs
        assert w["kv_bytes"] == live * b.num_kv_heads * b.head_dim * 2 * 2


def test_write_work():
    b = workloads.small_batch([(5, 3), (0, 2)], dtype="f32", num_heads=4, num_kv_heads=2, head_dim=8, seed=1)
    assert write_work(b)["bytes"] == 5 * (2 * 2 * 2 * 8 * 4) + 8 * 5
