"""Shared helpers for the GPU parity tests (test-side plumbing only)."""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from oracle import attention, paging


def say(*a):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pkv.load()


def host_bits(t):
    """Device tensor -> numpy array of its raw storage (bf16 as uint16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_f64(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.to(torch.float64).numpy()
    return t.numpy().astype(np.float64)


def max_err(got, ref):
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - ref).max())


def run_decode_step(w, d):
    """Slot mapping -> cache write -> decode attention on the device."""
    slots = pkv.slot_mapping(d.block_table, d.query_start_loc, d.num_computed, w.block_size,
                             w.num_blocks)
    pkv.cache_write(d.new_k, d.new_v, slots, d.cache)
    out = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len,
                                     w.scale, sliding_window=w.window)
    torch.cuda.synchronize()
    return slots, out


def oracle_decode_step(w, src_dtype):
    slots, errs = paging.slot_mapping(w.block_table, w.query_start_loc, w.num_computed,
                                      w.block_size, num_blocks=w.num_blocks)
    assert errs == 0
    kp, vp = paging.cache_write(w.k_plane, w.v_plane, w.new_k, w.new_v, slots, src_dtype,
                                w.cache_dtype, w.k_scale, w.v_scale)
    out = attention.paged_decode(w.q, w.q_dtype, kp, vp, w.cache_dtype, w.block_table,
                                 w.seq_lens, w.scale, sliding_window=w.window,
                                 k_scale=w.k_scale, v_scale=w.v_scale)
    return slots, kp, vp, out


def compact_planes(k_plane_dev, v_plane_dev, tables, rows):
    """Host copies of just the blocks that the given table rows reference.

    Returns (k, v, remapped tables) with ids renumbered 0..n-1 (-1 kept).
    """
    ids = np.unique(np.concatenate([t[rows][t[rows] >= 0] for t in tables]))
    idx = torch.from_numpy(ids.astype(np.int64)).to(k_plane_dev.device)
    k = host_bits(k_plane_dev.index_select(0, idx))
    v = host_bits(v_plane_dev.index_select(0, idx))
    remap = np.full(int(max(t.max() for t in tables)) + 2, -1, dtype=np.int64)
    remap[ids] = np.arange(len(ids))
    out = []
    for t in tables:
        sub = t[rows].astype(np.int64)
        out.append(np.where(sub >= 0, remap[np.maximum(sub, 0)], -1).astype(np.int32))
    return k, v, out
