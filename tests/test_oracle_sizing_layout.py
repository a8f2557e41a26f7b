"""Pins for the oracle's sizing closed forms and hybrid-group layout (CPU)."""

import json
import os

import numpy as np
import pytest

from oracle import layout, sizing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_llama70b_per_token_bytes_from_the_page_factors():
    g = _golden("kv_sizing_examples.json")["llama70b_per_token"]
    b = sizing.kv_bytes_per_token(g["num_layers"], g["num_kv_heads"], g["head_dim"], "bf16")
    product = g["num_layers"] * g["num_kv_heads"] * g["head_dim"] * g["kv_factor"] * g["element_bytes_fp16"]
    assert b == product == 327680                 # 320 KiB
    # the page's "about 640 KB" is the same product with 4-byte elements
    assert sizing.kv_bytes_per_token(80, 8, 128, "f32") == 655360
    # FP8 halves it
    assert sizing.kv_bytes_per_token(80, 8, 128, "fp8") * 2 == b
    # 4096-token request and 32 of them (the page's 2.5 GB / 80 GB are 2x)
    assert b * 4096 == 1.25 * 2 ** 30
    assert b * 4096 * 32 == 40 * 2 ** 30


def test_pool_and_block_bytes():
    # one block of one LLaMA-70B-shaped layer: 16 tokens * 8 heads * 128 * 2 * 2 B
    assert sizing.block_bytes(16, 8, 128, "bf16") == 64 * 1024
    # 16384-block pool for 80 layers = 80 GiB
    assert sizing.pool_bytes(16384, 80, 16, 8, 128, "bf16") == 80 * 2 ** 30
    assert sizing.pool_bytes(16384, 80, 16, 8, 128, "fp8") == 40 * 2 ** 30


def test_block_count_from_budget():
    # brute force: the largest n with n * bytes_per_block * layers <= available
    total, util, non_kv = 288 * 10 ** 9, 0.9, 20 * 10 ** 9
    per = sizing.block_bytes(16, 8, 128, "bf16") * 12
    n = sizing.num_blocks_for_budget(total, util, non_kv, 12, 16, 8, 128, "bf16")
    avail = int(total * util) - non_kv
    assert n * per <= avail < (n + 1) * per
    assert sizing.num_blocks_for_budget(10, 0.5, 100, 1, 16, 8, 128, "bf16") == 0


def test_hybrid_example_groups_and_tensors():
    g = _golden("kv_sizing_examples.json")["hybrid_example"]
    m = layout.group_slot_tensor(g["groups"])
    assert m["L0"] == (0, 0, 0) and m["L2"] == (0, 1, 1)
    assert m["L1"] == (1, 0, 0) and m["L3"] == (1, 1, 1)
    assert layout.tensors_from_groups(g["groups"]) == g["tensors"]
    # layers of one group sit in different tensors; one tensor mixes groups
    for grp in g["groups"]:
        assert len({m[x][2] for x in grp}) == len(grp)
    for t in g["tensors"]:
        assert len({m[x][0] for x in t}) == len(t)


@pytest.mark.parametrize("bs", [4, 16, 32])
def test_swa_first_live_block_against_brute_force(bs):
    for W in (1, 5, 16, 17, 64, 4096):
        for nc in range(0, 300, 7):
            b = layout.swa_first_live_block(nc, W, bs)
            # brute force: smallest block holding any position >= nc - W + 1
            lo = max(0, nc - W + 1)
            assert b == lo // bs
            if b > 0:
                assert (b * bs) - 1 < nc - W + 1      # previous block wholly out
    assert layout.swa_first_live_block(10_000, 0, 16) == 0   # full attention keeps all


def test_swa_cap_is_tight_and_exceeds_the_pages_w_over_bs():
    bs, W = 16, 4096
    worst = 0
    for nc in range(W, W + 64):
        for ql in (1, 3, 512):
            first = layout.swa_first_live_block(nc, W, bs)
            need = -(-(nc + ql) // bs)
            live = need - first
            assert live <= layout.swa_block_cap(W, ql, bs)
            if ql == 1:
                worst = max(worst, live)
    assert worst == layout.swa_block_cap(W, 1, bs) == W // bs + 1


def test_check_group_tables_accepts_valid_and_rejects_mistakes():
    bs, W, nb = 4, 6, 32
    seq = [13]
    nc = [12]
    first = layout.swa_first_live_block(12, W, bs)        # window 7..12 -> block 1
    assert first == 1
    full = np.array([[0, 1, 2, 3]], dtype=np.int32)
    swa = np.array([[-1, 5, 6, 7]], dtype=np.int32)
    layout.check_group_tables([full, swa], seq, nc, [0, W], bs, nb)
    with pytest.raises(AssertionError):   # not released
        layout.check_group_tables([full, np.array([[4, 5, 6, 7]])], seq, nc, [0, W], bs, nb)
    with pytest.raises(AssertionError):   # released too early
        layout.check_group_tables([full, np.array([[-1, -1, 6, 7]])], seq, nc, [0, W], bs, nb)
    with pytest.raises(AssertionError):   # id shared across groups
        layout.check_group_tables([full, np.array([[-1, 1, 6, 7]])], seq, nc, [0, W], bs, nb)
