"""Block tables, slot mapping and the KV-cache write (oracle, test-only).

Definitions followed:

* A request's KV is split into fixed-size blocks; a block table row maps the
  request's logical block index to a physical block id (Worker-Side KV Init,
  § PagedAttention and Block Management and § Block Table Multi-Level Mapping
  Mechanism; Engine-to-Worker card, § GPU worker가 하는 일).
* A token at sequence position ``pos`` lives in logical block ``pos // bs`` at
  offset ``pos % bs``; with physical id ``p`` its slot is ``p * bs + pos % bs``
  (Worker-Side KV Init, § Pinpointing the Token Slot: the position-7 example
  with block 37 and block size 16; Engine-to-Worker card, § Slot mapping은 왜
  필요한가: position -> logical block + offset -> physical id -> slot).
* Tokens computed in one step: ``num_new = num_tokens_with_spec -
  num_computed``; they occupy positions ``num_computed ..`` in order
  (Engine-to-Worker card, § EngineCore가 하는 일).
* The write step stores each new token's K/V at its slot; attention later reads
  past K/V through the block table (Engine-to-Worker card, § Slot mapping은 왜
  필요한가, and § Forward 직전의 metadata).

Readings where the pages are silent:

* slots count token positions, not bytes (the page's "base + 37*16 + 7" has no
  element size); positions are 0-based;
* a token whose lookup falls outside the row or hits a negative or
  out-of-range id gets slot -1 and counts as an error; tokens past the last
  request (padding) get slot -1 and are not errors;
* a write with slot -1 is skipped; every slot not written keeps its old bytes.
"""

import numpy as np

from . import bf16 as _bf16
from . import e4m3 as _e4m3
from . import int4 as _int4


def num_logical_blocks(num_tokens, block_size):
    """Blocks needed to hold ``num_tokens`` tokens: ceil(n / bs)."""
    return -(-int(num_tokens) // int(block_size))


def slot_mapping(block_table, query_start_loc, num_computed, block_size,
                 num_tokens=None, num_blocks=None):
    """Per-token write slots for one step.

    block_table     int[R, max_blocks]  physical ids (-1 = no block)
    query_start_loc int[R+1]            token range of request r: [q[r], q[r+1])
    num_computed    int[R]              tokens already in the cache
    Returns (slots int64[num_tokens], error_count).
    """
    bt = np.asarray(block_table)
    qsl = np.asarray(query_start_loc)
    nc = np.asarray(num_computed)
    R = len(nc)
    T = int(qsl[R]) if num_tokens is None else int(num_tokens)
    slots = np.full(T, -1, dtype=np.int64)
    errors = 0
    for r in range(R):
        for t in range(int(qsl[r]), int(qsl[r + 1])):
            pos = int(nc[r]) + (t - int(qsl[r]))
            logical = pos // block_size
            offset = pos % block_size
            if logical >= bt.shape[1]:
                errors += 1
                continue
            phys = int(bt[r, logical])
            if phys < 0 or (num_blocks is not None and phys >= num_blocks):
                errors += 1
                continue
            slots[t] = phys * block_size + offset
    return slots, errors


def convert_for_cache(x, src_dtype, cache_dtype, scale=1.0):
    """Source elements -> the cache's storage bits.

    src_dtype: 'f32' (float32 values) or 'bf16' (uint16 bit patterns).
    cache_dtype: 'f32', 'bf16', 'fp8' (uint8 E4M3 codes) or 'int4' (rows of
    D / 2 bytes, two 4-bit codes each).
    Same type: a bit copy.  f32 -> bf16: round to nearest even.
    -> fp8 / int4: quantise the float32 value with the per-tensor scale.
    """
    x = np.asarray(x)
    if src_dtype == "bf16":
        as_f32 = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif src_dtype == "f32":
        as_f32 = x.astype(np.float32)
    else:
        raise ValueError(src_dtype)
    if cache_dtype == src_dtype:
        return x.copy()
    if cache_dtype == "bf16":
        return _bf16.from_f32(as_f32)
    if cache_dtype == "fp8":
        return _e4m3.quantize(as_f32, scale)
    if cache_dtype == "int4":
        return _int4.quantize_packed(as_f32, scale)
    raise ValueError((src_dtype, cache_dtype))


def cache_write(k_plane, v_plane, key, value, slots, src_dtype, cache_dtype,
                k_scale=1.0, v_scale=1.0):
    """Scatter one step's K/V rows into copies of the paged planes.

    Planes are [num_blocks, bs, Hkv, D] arrays of storage bits; key/value are
    [T, Hkv, D].  Slot s (>= 0) addresses plane[s // bs, s % bs].
    Returns the new (k_plane, v_plane); the inputs are not modified.
    """
    kp = np.array(k_plane, copy=True)
    vp = np.array(v_plane, copy=True)
    bs = kp.shape[1]
    seen = set()
    for t, s in enumerate(np.asarray(slots)):
        s = int(s)
        if s < 0:
            continue
        if s in seen:
            raise ValueError("two tokens of one step map to slot %d" % s)
        seen.add(s)
        kp[s // bs, s % bs] = convert_for_cache(key[t], src_dtype, cache_dtype, k_scale)
        vp[s // bs, s % bs] = convert_for_cache(value[t], src_dtype, cache_dtype, v_scale)
    return kp, vp


def plane_to_f64(plane, cache_dtype, scale=1.0):
    """Storage bits -> float64 values (fp8 and int4 codes are dequantised;
    an int4 row of D / 2 bytes becomes D values)."""
    if cache_dtype == "bf16":
        return _bf16.to_f64(plane)
    if cache_dtype == "f32":
        return np.asarray(plane, dtype=np.float32).astype(np.float64)
    if cache_dtype == "f64":  # already-widened values (test constructions)
        return np.asarray(plane, dtype=np.float64)
    if cache_dtype == "fp8":
        return _e4m3.dequantize(plane, scale)
    if cache_dtype == "int4":
        return _int4.dequantize(plane, scale)
    raise ValueError(cache_dtype)


def gather_positions(plane, table_row, positions_, block_size):
    """Rows of one request at the given sequence positions, in that order.

    Follows the block table row: position j -> physical block
    table_row[j // bs], offset j % bs.  Raises if a needed entry is missing.
    Returns plane[...] rows of shape [len(positions), Hkv, D].
    """
    out = []
    nb = plane.shape[0]
    for j in positions_:
        j = int(j)
        logical = j // block_size
        if logical >= len(table_row):
            raise IndexError("position %d beyond the block table row" % j)
        phys = int(table_row[logical])
        if phys < 0 or phys >= nb:
            raise IndexError("position %d needs block entry %d = %d" % (j, logical, phys))
        out.append(plane[phys, j % block_size])
    if not out:
        return plane[:0, 0]
    return np.stack(out)


def unused_slot_mask(num_blocks, block_size, block_table, seq_lens):
    """Boolean [num_blocks, bs]: True where no request holds a live token.

    A slot is live if some row r has, at logical block b < ceil(L_r / bs), the
    physical id of that slot's block and the offset's position b*bs + o is
    below L_r.  Everything else (unreferenced blocks, tails of last blocks,
    table entries past a request's length) is unused.  Tests poison these slots
    with NaN to prove kernels never read them.
    """
    bt = np.asarray(block_table)
    live = np.zeros((num_blocks, block_size), dtype=bool)
    for r, L in enumerate(np.asarray(seq_lens)):
        L = int(L)
        for b in range(num_logical_blocks(L, block_size)):
            phys = int(bt[r, b])
            if phys < 0:
                continue
            for o in range(block_size):
                if b * block_size + o < L:
                    live[phys, o] = True
    return ~live


# --------------------------------------------------------------------------
# Prefix sharing (Chinese worker-side page, § PagedAttention与Block管理:
# requests that start with the same prompt point the leading entries of
# their block tables at the same physical blocks; each block counts the
# logical entries that reference it and returns to the pool only when that
# count reaches zero).  Reading where the page is silent: a request that must
# write into a block it shares first moves to a private copy of it.


def refcounts(tables, num_blocks):
    """References to each physical block: the number of table entries, over
    every row of every table given, that hold its id (entries < 0 hold none)."""
    counts = np.zeros(num_blocks, dtype=np.int64)
    for t in tables:
        for row in np.atleast_2d(np.asarray(t)):
            for e in row:
                e = int(e)
                if e >= 0:
                    counts[e] += 1
    return counts


def copy_blocks(k_plane, v_plane, src, dst):
    """Block dst[i] of each plane becomes a copy of block src[i] of the
    plane as it was before the call (the pairs are independent); a pair
    with an id outside [0, num_blocks) changes nothing and is counted.

    Returns (k_plane', v_plane', error count)."""
    nb = k_plane.shape[0]
    k_out, v_out = k_plane.copy(), v_plane.copy()
    errors = 0
    for s_, d_ in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        if not (0 <= s_ < nb and 0 <= d_ < nb):
            errors += 1
            continue
        k_out[d_] = k_plane[s_]
        v_out[d_] = v_plane[s_]
    return k_out, v_out, errors
