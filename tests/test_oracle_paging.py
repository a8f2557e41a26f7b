"""Pins for the oracle's slot mapping, cache write and gather (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import paging

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _slots_by_enumeration(row, block_size, length):
    """Brute force: list every physical slot of the row in logical order."""
    flat = []
    for phys in row:
        for o in range(block_size):
            flat.append(int(phys) * block_size + o)
    return flat[:length]


def test_token7_example_from_page():
    g = _golden("slot_mapping_examples.json")["token7"]
    bs = g["block_size"]
    assert g["position"] // bs == g["logical_block"]
    assert g["position"] % bs == g["offset"]
    bt = np.array([[g["physical_block"]]], dtype=np.int32)
    # one request, nothing cached before position 7, eight tokens this step
    slots, err = paging.slot_mapping(bt, [0, 8], [0], bs)
    assert err == 0
    assert slots[g["position"]] == g["slot"]


def test_48_tokens_need_3_blocks():
    g = _golden("slot_mapping_examples.json")["tokens48"]
    assert paging.num_logical_blocks(g["num_tokens"], g["block_size"]) == g["logical_blocks"]
    assert paging.num_logical_blocks(g["num_tokens"] + 1, g["block_size"]) == g["logical_blocks"] + 1


def test_four_word_phrase_paging():
    g = _golden("slot_mapping_examples.json")["four_word_phrase"]
    bs = g["block_size"]
    rng = np.random.default_rng(0)
    phys = rng.permutation(8)[:2]  # the page prints no ids: any two blocks
    bt = np.array([phys], dtype=np.int32)
    words = g["tokens"]
    assert paging.num_logical_blocks(len(words), bs) == g["logical_blocks_for_4_tokens"]
    slots, err = paging.slot_mapping(bt, [0, 4], [0], bs)
    assert err == 0
    # the four words fill block 0 at offsets 0..3
    assert list(slots) == [int(phys[0]) * bs + o for o in range(4)]
    # the fifth token, generated next step, opens logical block 1 at offset 0
    slots5, err = paging.slot_mapping(bt, [0, 1], [4], bs)
    assert err == 0
    assert slots5[0] == int(phys[1]) * bs + 0
    assert slots5[0] // bs == phys[g["fifth_token_logical_block"]]
    assert slots5[0] % bs == g["fifth_token_offset"]


def test_page_block_table_rows_against_enumeration():
    rows = _golden("slot_mapping_examples.json")["block_table_rows"]["rows"]
    bs = 16
    width = max(len(r) for r in rows)
    bt = np.full((len(rows), width), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    lens = [len(r) * bs for r in rows]
    qsl = np.concatenate([[0], np.cumsum(lens)])
    slots, err = paging.slot_mapping(bt, qsl, [0] * len(rows), bs)
    assert err == 0
    for i, r in enumerate(rows):
        assert list(slots[qsl[i]:qsl[i + 1]]) == _slots_by_enumeration(r, bs, lens[i])
    # the 7th-token example again on the [37, 12, 44] row
    assert slots[qsl[3] + 7] == 599


@pytest.mark.parametrize("seed", range(6))
def test_random_tables_against_enumeration(seed):
    rng = np.random.default_rng(100 + seed)
    bs = int(rng.choice([4, 8, 16, 32]))
    R = int(rng.integers(1, 7))
    nb = 128
    perm = rng.permutation(nb)
    nc = rng.integers(0, 40, size=R)
    ql = rng.integers(0, 12, size=R)
    maxb = max(int(np.max(-(-(nc + ql) // bs))), 1)
    bt = np.full((R, maxb), -1, dtype=np.int32)
    k = 0
    for r in range(R):
        n = -(-(int(nc[r]) + int(ql[r])) // bs)
        bt[r, :n] = perm[k:k + n]
        k += n
    qsl = np.concatenate([[0], np.cumsum(ql)])
    pad = int(rng.integers(0, 3))
    slots, err = paging.slot_mapping(bt, qsl, nc, bs, num_tokens=qsl[-1] + pad, num_blocks=nb)
    assert err == 0
    for r in range(R):
        full = _slots_by_enumeration(bt[r][bt[r] >= 0], bs, int(nc[r] + ql[r]))
        assert list(slots[qsl[r]:qsl[r + 1]]) == full[int(nc[r]):]
    assert (slots[qsl[-1]:] == -1).all()  # padding tokens


def test_slot_mapping_errors():
    bt = np.array([[3, -1], [70, 1]], dtype=np.int32)
    slots, err = paging.slot_mapping(bt, [0, 3, 5], [2, 0], 4, num_blocks=64)
    # r0 positions 2,3 -> block 0 (id 3); position 4 -> logical 1 = -1 -> error
    assert list(slots[:3]) == [14, 15, -1]
    # r1 positions 0,1 -> logical 0 = 70 >= num_blocks -> errors
    assert list(slots[3:]) == [-1, -1]
    assert err == 3
    # past the end of the row
    slots, err = paging.slot_mapping(np.array([[5]], dtype=np.int32), [0, 2], [3], 4)
    assert list(slots) == [23, -1] and err == 1


def test_cache_write_round_trip_and_untouched_cells():
    rng = np.random.default_rng(7)
    nb, bs, H, D = 12, 4, 2, 8
    kp = np.full((nb, bs, H, D), np.nan, dtype=np.float32)
    vp = np.full((nb, bs, H, D), np.nan, dtype=np.float32)
    T = 9
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[3] = -1
    key = rng.standard_normal((T, H, D)).astype(np.float32)
    val = rng.standard_normal((T, H, D)).astype(np.float32)
    k2, v2 = paging.cache_write(kp, vp, key, val, slots, "f32", "f32")
    written = np.zeros((nb, bs), dtype=bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        np.testing.assert_array_equal(k2[blk, off], key[t])
        np.testing.assert_array_equal(v2[blk, off], val[t])
        written[blk, off] = True
    assert np.isnan(k2[~written]).all() and np.isnan(v2[~written]).all()
    assert np.isnan(kp).all()  # inputs not modified
    with pytest.raises(ValueError):
        paging.cache_write(kp, vp, key[:2], val[:2], np.array([5, 5]), "f32", "f32")


def test_gather_follows_table_and_rejects_missing_blocks():
    nb, bs = 6, 2
    plane = np.arange(nb * bs, dtype=np.float32).reshape(nb, bs, 1, 1)
    row = np.array([4, 0, -1])
    got = paging.gather_positions(plane, row, [0, 1, 2, 3], bs)[:, 0, 0]
    assert list(got) == [8, 9, 0, 1]
    with pytest.raises(IndexError):
        paging.gather_positions(plane, row, [4], bs)
    with pytest.raises(IndexError):
        paging.gather_positions(plane, row, [6], bs)


def test_unused_slot_mask():
    bt = np.array([[2, 0], [1, -1]], dtype=np.int32)
    m = paging.unused_slot_mask(4, 4, bt, [6, 3])
    live = ~m
    assert live[2].all() and list(live[0]) == [True, True, False, False]
    assert list(live[1]) == [True, True, True, False]
    assert not live[3].any()
