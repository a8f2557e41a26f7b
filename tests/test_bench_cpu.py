"""CPU checks of bench.py's own arithmetic -- the byte and flop counts that its
throughput, roofline and prefill figures divide by -- against closed forms
worked out by hand, and its one-GPU contract."""

import os
import subprocess
import sys
import types

import numpy as np

import bench
from paged_kv_cache_mapping_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and r.stdout == ""
    assert "one GPU" in r.stderr


def test_decode_step_bytes_on_the_llama8b_batch():
    """64 sequences, Hq 32, Hkv 8, D 128, block 16, bf16: the split kernel
    reads each visible K and V row once (2 x 2 B per element), the queries and
    one 4-B table entry per visible block and a 4-B length per sequence."""
    w = workloads.llama8b_decode()
    L = w.seq_lens.astype(np.int64)
    assert len(L) == 64 and int(L.sum()) == 73505          # the workload's seed-2 lengths
    kv = int(L.sum()) * 8 * 128 * 2 * 2
    nblk = int(((L + 15) // 16).sum())
    ab = bench.algorithmic_bytes(w)
    assert ab["kv"] == kv == 301076480
    assert ab["split"] == kv + 64 * 32 * 128 * 2 + 4 * nblk + 4 * 64 == 301619516
    assert ab["combine"] == 64 * 32 * 128 * 2                # the output rows
    # one new K and V row per sequence: read as bf16, written as bf16; the int64 slot
    assert ab["write"] == 64 * 8 * 128 * 2 * (2 + 2) + 64 * 8
    # per token: query start pair, computed count, table entry (4 B each) and the slot
    assert ab["slot"] == 64 * (4 * 4 + 8)
    assert ab["step"] == ab["split"] + ab["combine"] + ab["slot"] + ab["write"]


def _tiny_hybrid():
    # request 0: one decode token at position 9 (10 keys); request 1: a chunk of
    # 4 query tokens at positions 4..7 (8 keys); Hq 4, Hkv 2, D 4
    return types.SimpleNamespace(query_start_loc=np.array([0, 1, 5], np.int32),
                                 seq_lens=np.array([10, 8], np.int32), num_kv_heads=2, head_dim=4,
                                 num_q_heads=4, num_tokens=5)


def test_hybrid_layer_bytes_and_flops_full_attention():
    rd, wr, fl = bench.hybrid_layer_bytes(_tiny_hybrid(), 0)
    row = 2 * 4 * 2 * 2                     # K and V of one token: Hkv x D x 2 planes x 2 B
    assert rd == (10 + 8) * row + 5 * 4 * 4 * 2 * 2            # keys once + q and out
    assert wr == 5 * row * 2 + 5 * 8                            # read + write new rows, slots
    # only the chunk counts as prefill: its queries see 5, 6, 7 and 8 keys
    assert fl == (5 + 6 + 7 + 8) * 4 * 4 * 4


def test_hybrid_layer_bytes_and_flops_sliding_window():
    rd, _, fl = bench.hybrid_layer_bytes(_tiny_hybrid(), 2)
    row = 2 * 4 * 2 * 2
    # window 2: the decode token sees keys 8..9; the chunk's queries see keys 3..7
    assert rd == (2 + 5) * row + 5 * 4 * 4 * 2 * 2
    assert fl == 4 * 2 * 4 * 4 * 4
