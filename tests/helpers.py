"""Shared helpers for the GPU parity tests (test-side plumbing only)."""

import json
import os
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


# ---- element-wise bounds at the output's precision, logged

PARITY_LOG = os.environ.get("PKV_PARITY_LOG")
BF16_REL = 2.0 ** -8     # half an ulp of bfloat16, relative to the value


def check_close(name, got, ref, max_abs, floor):
    """Compare a bf16 (or f32) output with the fp64 oracle element by element.

    Two bounds, both asserted: the spec max-abs bound (2e-3 bf16 KV,
    3e-2 fp8 KV) and a per-element bound at the output's own precision,
    |got - ref| <= 2^-8 |ref| + floor: rounding to bf16 moves a value by at
    most half an ulp (2^-8 of it), and `floor` covers the float32 arithmetic
    before that rounding (stated per test from the data's scale).  Logs the
    max-abs and max-relative errors (to stdout, and to $PKV_PARITY_LOG as a
    JSON line when set).
    """
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite output"
    assert np.isfinite(ref).all(), "non-finite oracle output"
    diff = np.abs(got - ref)
    bound = BF16_REL * np.abs(ref) + floor
    mask = np.abs(ref) > 100 * floor
    rec = dict(case=name, n=int(got.size), max_abs=float(diff.max()),
               max_rel=float((diff[mask] / np.abs(ref[mask])).max()) if mask.any() else 0.0,
               worst_vs_bound=float((diff / bound).max()), floor=floor, max_abs_bound=max_abs,
               ref_max=float(np.abs(ref).max()), ref_std=float(ref.std()))
    say("parity", json.dumps(rec))
    if PARITY_LOG:
        try:
            with open(PARITY_LOG, "a") as f:
                f.write(json.dumps(rec) + "\n")
        except OSError:
            pass
    assert rec["max_abs"] <= max_abs, rec
    bad = np.argwhere(diff > bound)
    assert len(bad) == 0, "%d elements beyond |d| <= 2^-8 |ref| + %g, first %s: got %r ref %r" % (
        len(bad), floor, bad[0].tolist(), got[tuple(bad[0])], ref[tuple(bad[0])])
    return rec
