"""Torch-facing binding of libpagedkv.so: argument marshalling only.

Every function checks dtypes/shapes that the C ABI cannot see (torch tensor
metadata), passes raw device pointers and torch's current HIP stream, and
raises :class:`PkvError` on a non-zero status.  All computation happens in the
library's HIP kernels.
"""

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (PKV_BF16, PKV_F32, PKV_FP8_E4M3, PKV_INT4, PKV_PLAN_BLOCKS_NOT_SHARED,
                   PKV_PLAN_BLOCKS_SHARED, PkvCache,
                   PkvDecodePlan, check, load)

_DTYPES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.uint8: PKV_FP8_E4M3}
if hasattr(torch, "float8_e4m3fn"):
    _DTYPES[torch.float8_e4m3fn] = PKV_FP8_E4M3


def _dt(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError("unsupported dtype %s" % t.dtype)


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _i32(t, name):
    _need(t.dtype == torch.int32 and t.is_contiguous(), "%s must be a contiguous int32 tensor" % name)
    return t


@dataclass
class CacheView:
    """One attention layer's paged K/V planes (see ``pkv_cache`` in pagedkv.h).

    k, v: tensors whose storage holds ``num_blocks`` blocks of
    [block_size, num_kv_heads, head_dim] elements, block b starting
    ``block_stride`` elements after block b-1.  Typically views
    ``[num_blocks, block_size, num_kv_heads, head_dim]`` of one byte buffer.
    fp8 caches use dtype uint8 (or float8_e4m3fn) with per-tensor scales.
    int4 caches are uint8 planes of head_dim / 2 bytes per row (two elements
    a byte) with per-tensor scales; head_dim and block_stride count elements.
    """
    k: torch.Tensor
    v: torch.Tensor
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    block_stride: int
    k_scale: float = 1.0
    v_scale: float = 1.0
    int4: bool = False

    @classmethod
    def from_planes(cls, k, v, k_scale=1.0, v_scale=1.0, int4=False):
        """Planes shaped [num_blocks, block_size, num_kv_heads, head_dim]
        (int4: uint8 planes [..., head_dim / 2])."""
        _need(k.dim() == 4 and k.shape == v.shape and k.dtype == v.dtype, "k/v planes mismatch")
        _need(k.stride(3) == 1 and k.stride(2) == k.shape[3] and k.stride(1) == k.shape[2] * k.shape[3],
              "each block must be contiguous [block_size, heads, dim]")
        _need(k.stride() == v.stride(), "k and v strides differ")
        nb, bs, h, d = k.shape
        if int4:
            _need(k.dtype == torch.uint8, "int4 planes are uint8 bytes")
            return cls(k, v, nb, bs, h, 2 * d, 2 * k.stride(0), float(k_scale), float(v_scale), True)
        return cls(k, v, nb, bs, h, d, k.stride(0), float(k_scale), float(v_scale))

    @property
    def dtype(self):
        return PKV_INT4 if self.int4 else _dt(self.k)

    def c_struct(self):
        return PkvCache(k=self.k.data_ptr(), v=self.v.data_ptr(), block_stride=self.block_stride,
                        num_blocks=self.num_blocks, block_size=self.block_size,
                        num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                        dtype=self.dtype, k_scale=self.k_scale, v_scale=self.v_scale)


def status_string(status):
    return load().pkv_status_string(status).decode()


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype):
    """Closed form of the per-token KV footprint (host arithmetic in the library)."""
    dt = {"f32": PKV_F32, "bf16": PKV_BF16, "fp8": PKV_FP8_E4M3, "int4": PKV_INT4}[dtype]
    return int(load().pkv_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dt))


def slot_mapping(block_table, query_start_loc, num_computed, block_size, num_blocks,
                 num_tokens=None, out=None, err_count=None):
    """Per-token write slots (int64), -1 for padding / invalid lookups."""
    lib = load()
    _i32(block_table, "block_table")
    _i32(query_start_loc, "query_start_loc")
    _i32(num_computed, "num_computed")
    num_reqs = num_computed.numel()
    _need(query_start_loc.numel() == num_reqs + 1, "query_start_loc needs num_reqs + 1 entries")
    _need(block_table.dim() == 2 and block_table.shape[0] >= num_reqs, "block_table must be [R, max_blocks]")
    if num_tokens is None:
        num_tokens = out.numel() if out is not None else int(query_start_loc[-1].item())
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=block_table.device)
    _need(out.dtype == torch.int64 and out.is_contiguous() and out.numel() >= num_tokens, "bad out")
    if err_count is not None:
        _need(err_count.dtype == torch.int32, "err_count must be int32")
    check("pkv_slot_mapping", lib.pkv_slot_mapping(
        _ptr(block_table), block_table.shape[1], num_reqs, _ptr(query_start_loc), _ptr(num_computed),
        block_size, num_blocks, num_tokens, _ptr(out), _ptr(err_count), _stream(block_table.device)))
    return out


def cache_write(key, value, slot_mapping_, cache):
    """Scatter key/value [T, Hkv, D] rows into the cache at the given slots."""
    lib = load()
    _need(key.shape == value.shape and key.dim() == 3 and key.dtype == value.dtype, "key/value mismatch")
    _need(key.stride() == value.stride() and key.stride(2) == 1, "key/value need unit dim stride")
    _need(slot_mapping_.dtype == torch.int64 and slot_mapping_.is_contiguous(), "slot_mapping must be int64")
    T = key.shape[0]
    _need(slot_mapping_.numel() >= T, "slot_mapping shorter than key")
    c = cache.c_struct()
    check("pkv_cache_write", lib.pkv_cache_write(
        _ptr(key), _ptr(value), _dt(key), key.stride(0), key.stride(1), _ptr(slot_mapping_), T,
        ctypes.byref(c), _stream(key.device)))


def slot_mapping_cache_write(block_table, query_start_loc, num_computed, key, value, cache,
                             out=None, err_count=None):
    """slot_mapping followed by cache_write in one launch; returns the slots
    (int64 [T], T = key rows)."""
    lib = load()
    _i32(block_table, "block_table")
    _i32(query_start_loc, "query_start_loc")
    _i32(num_computed, "num_computed")
    num_reqs = num_computed.numel()
    _need(query_start_loc.numel() == num_reqs + 1, "query_start_loc needs num_reqs + 1 entries")
    _need(block_table.dim() == 2 and block_table.shape[0] >= num_reqs, "block_table must be [R, max_blocks]")
    _need(key.shape == value.shape and key.dim() == 3 and key.dtype == value.dtype, "key/value mismatch")
    _need(key.stride() == value.stride() and key.stride(2) == 1, "key/value need unit dim stride")
    T = key.shape[0]
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=key.device)
    _need(out.dtype == torch.int64 and out.is_contiguous() and out.numel() >= T, "bad out")
    if err_count is not None:
        _need(err_count.dtype == torch.int32, "err_count must be int32")
    c = cache.c_struct()
    check("pkv_slot_mapping_cache_write", lib.pkv_slot_mapping_cache_write(
        _ptr(block_table), block_table.shape[1], num_reqs, _ptr(query_start_loc), _ptr(num_computed), T,
        _ptr(out), _ptr(err_count), _ptr(key), _ptr(value), _dt(key), key.stride(0), key.stride(1),
        ctypes.byref(c), _stream(key.device)))
    return out


def copy_blocks(src_ids, dst_ids, cache, err_count=None):
    """Copy blocks src_ids[i] -> dst_ids[i] (int32 device tensors) in both planes."""
    lib = load()
    _i32(src_ids, "src_ids")
    _i32(dst_ids, "dst_ids")
    _need(src_ids.numel() == dst_ids.numel(), "src_ids and dst_ids differ in length")
    if err_count is not None:
        _need(err_count.dtype == torch.int32, "err_count must be int32")
    c = cache.c_struct()
    check("pkv_copy_blocks", lib.pkv_copy_blocks(
        ctypes.byref(c), _ptr(src_ids), _ptr(dst_ids), src_ids.numel(), _ptr(err_count),
        _stream(src_ids.device)))


def decode_plan(num_rows, num_q_heads, cache, max_seq_len, sliding_window=0, blocks_not_shared=False,
                blocks_shared=False):
    """The library's plan (pkv_decode_plan_make); blocks_not_shared sets
    PKV_PLAN_BLOCKS_NOT_SHARED (no block is read by two rows of a call),
    blocks_shared PKV_PLAN_BLOCKS_SHARED (many rows read the same blocks)."""
    lib = load()
    plan = PkvDecodePlan()
    flags = (PKV_PLAN_BLOCKS_NOT_SHARED if blocks_not_shared else 0) | (PKV_PLAN_BLOCKS_SHARED if blocks_shared else 0)
    check("pkv_decode_plan_make", lib.pkv_decode_plan_make(
        num_rows, num_q_heads, cache.num_kv_heads, cache.head_dim, cache.block_size,
        cache.dtype, max_seq_len, sliding_window, flags, ctypes.byref(plan)))
    return plan


def tune_plan(plan, num_rows, num_q_heads, cache, max_seq_len, sliding_window=0,
              split_blocks=None, num_workers=None, lead_workers=None, trail_share_pct=None,
              heads_per_item=None):
    """Override a plan's tuning fields; the library recomputes the sizes they
    imply (pkv_decode_plan_resize).

    Scheme 0: split_blocks = blocks per split.  Scheme 1: split_blocks =
    least blocks per worker, num_workers = workers launched, lead_workers /
    trail_share_pct = unequal shares (see pagedkv.h).  Changing num_workers
    alone keeps the half-and-half lead split when the plan had one.
    """
    if split_blocks is not None:
        plan.split_blocks = int(split_blocks)
    if num_workers is not None:
        plan.num_workers = int(num_workers)
        if lead_workers is None:
            plan.lead_workers = plan.num_workers // 2 if plan.lead_workers else 0
    if lead_workers is not None:
        plan.lead_workers = int(lead_workers)
    if trail_share_pct is not None:
        plan.trail_share_pct = int(trail_share_pct)
    if heads_per_item is not None:
        plan.heads_per_item = int(heads_per_item)
    check("pkv_decode_plan_resize", load().pkv_decode_plan_resize(
        num_rows, num_q_heads, cache.head_dim, cache.block_size, max_seq_len, sliding_window,
        ctypes.byref(plan)))
    return plan


def new_workspace(nbytes, device):
    """A workspace for the attention calls (at least 16 bytes; its contents
    need no initialisation)."""
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return workspace, 0
    if workspace is None:
        workspace = new_workspace(nbytes, device)
    _need(workspace.numel() * workspace.element_size() >= nbytes, "workspace too small")
    return workspace, workspace.numel() * workspace.element_size()


def paged_attention_decode(q, cache, block_table, seq_lens, max_seq_len, softmax_scale,
                           sliding_window=0, workspace=None, out=None):
    """One query token per sequence: q [B, Hq, D] -> out [B, Hq, D]."""
    lib = load()
    _need(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [B, Hq, D]")
    _i32(block_table, "block_table")
    _i32(seq_lens, "seq_lens")
    B, Hq, D = q.shape
    _need(D == cache.head_dim and seq_lens.numel() == B and block_table.shape[0] >= B, "shape mismatch")
    plan = decode_plan(B, Hq, cache, max_seq_len, sliding_window)
    ws, wsb = _workspace(plan.workspace_bytes, q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "bad out")
    c = cache.c_struct()
    check("pkv_paged_attention_decode", lib.pkv_paged_attention_decode(
        _ptr(out), _ptr(q), _dt(q), B, Hq, ctypes.byref(c), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), max_seq_len, softmax_scale, sliding_window, _ptr(ws), wsb, _stream(q.device)))
    return out


def paged_attention_decode_partials(q, cache, block_table, seq_lens, max_seq_len, softmax_scale,
                                    plan, workspace, out, sliding_window=0):
    """Phase 1 of the decode (see pagedkv.h); `plan` from :func:`decode_plan`."""
    lib = load()
    B, Hq, _ = q.shape
    c = cache.c_struct()
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("pkv_paged_attention_decode_partials", lib.pkv_paged_attention_decode_partials(
        _ptr(out), _ptr(q), _dt(q), B, Hq, ctypes.byref(c), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), max_seq_len, softmax_scale, sliding_window, ctypes.byref(plan),
        _ptr(workspace), wsb, _stream(q.device)))


def paged_attention_decode_combine(out, seq_lens, block_size, plan, workspace, sliding_window=0):
    """Phase 2 of the decode: merge the splits of multi-split rows into out."""
    lib = load()
    B, Hq, D = out.shape
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("pkv_paged_attention_decode_combine", lib.pkv_paged_attention_decode_combine(
        _ptr(out), _dt(out), B, Hq, D, block_size, _ptr(seq_lens), sliding_window,
        ctypes.byref(plan), _ptr(workspace), wsb, _stream(out.device)))


def paged_attention_decode_step(q, new_k, new_v, cache, block_table, seq_lens, max_seq_len,
                                softmax_scale, plan, workspace, out, slots=None, sliding_window=0):
    """One decode step (see pagedkv.h): the new K/V rows [B, Hkv, D] bf16 are
    written at position seq_lens - 1 and attended to with the cache; `slots`
    (int64 [B], optional) receives their slots."""
    lib = load()
    B, Hq, _ = q.shape
    _need(new_k.is_contiguous() and new_v.is_contiguous() and new_k.dtype == torch.bfloat16
          and new_v.dtype == torch.bfloat16, "new_k / new_v must be contiguous bf16 [B, Hkv, D]")
    c = cache.c_struct()
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("pkv_paged_attention_decode_step", lib.pkv_paged_attention_decode_step(
        _ptr(out), _ptr(q), _dt(q), _ptr(new_k), _ptr(new_v), B, Hq, ctypes.byref(c), _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), max_seq_len, softmax_scale, sliding_window,
        ctypes.byref(plan), _ptr(workspace), wsb, _ptr(slots) if slots is not None else None,
        _stream(q.device)))


def chunked_workspace_size(num_tokens, num_reqs, num_q_heads, cache, max_query_len, max_seq_len,
                           sliding_window=0):
    lib = load()
    n = ctypes.c_size_t(0)
    check("pkv_chunked_workspace_size", lib.pkv_chunked_workspace_size(
        num_tokens, num_reqs, num_q_heads, cache.num_kv_heads, cache.head_dim, cache.block_size,
        cache.dtype, max_query_len, max_seq_len, sliding_window, ctypes.byref(n)))
    return n.value


def paged_attention_chunked(q, query_start_loc, seq_lens, max_query_len, cache, block_table,
                            max_seq_len, softmax_scale, causal=True, sliding_window=0,
                            workspace=None, out=None, blocks_not_shared=False, blocks_shared=False):
    """Mixed prefill/decode step: q [T, Hq, D] -> out [T, Hq, D];
    blocks_not_shared passes PKV_PLAN_BLOCKS_NOT_SHARED (no block read by
    two requests of the call), blocks_shared PKV_PLAN_BLOCKS_SHARED (many
    requests read the same blocks)."""
    lib = load()
    _need(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [T, Hq, D]")
    _i32(query_start_loc, "query_start_loc")
    _i32(seq_lens, "seq_lens")
    _i32(block_table, "block_table")
    T, Hq, D = q.shape
    R = seq_lens.numel()
    _need(query_start_loc.numel() == R + 1 and block_table.shape[0] >= R, "shape mismatch")
    nbytes = chunked_workspace_size(T, R, Hq, cache, max_query_len, max_seq_len, sliding_window)
    ws, wsb = _workspace(nbytes, q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    c = cache.c_struct()
    check("pkv_paged_attention_chunked", lib.pkv_paged_attention_chunked(
        _ptr(out), _ptr(q), _dt(q), T, Hq, _ptr(query_start_loc), _ptr(seq_lens), R, max_query_len,
        ctypes.byref(c), _ptr(block_table), block_table.shape[1], max_seq_len, softmax_scale,
        1 if causal else 0, sliding_window,
        (PKV_PLAN_BLOCKS_NOT_SHARED if blocks_not_shared else 0) | (PKV_PLAN_BLOCKS_SHARED if blocks_shared else 0),
        _ptr(ws), wsb, _stream(q.device)))
    return out


def fp8_quantize(x, scale, out=None):
    lib = load()
    _need(x.is_contiguous(), "x must be contiguous")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    check("pkv_fp8_e4m3_quantize", lib.pkv_fp8_e4m3_quantize(
        _ptr(x), _dt(x), x.numel(), float(scale), _ptr(out), _stream(x.device)))
    return out


def int4_quantize(x, scale, out=None):
    """x [..., n] (n even) -> packed uint8 [..., n / 2]."""
    lib = load()
    _need(x.is_contiguous() and x.shape[-1] % 2 == 0, "x must be contiguous with an even last dimension")
    if out is None:
        out = torch.empty(x.shape[:-1] + (x.shape[-1] // 2,), dtype=torch.uint8, device=x.device)
    check("pkv_int4_quantize", lib.pkv_int4_quantize(
        _ptr(x), _dt(x), x.numel(), float(scale), _ptr(out), _stream(x.device)))
    return out


def int4_dequantize(packed, scale, out=None):
    """packed uint8 [..., m] -> float32 [..., 2 m]."""
    lib = load()
    _need(packed.dtype == torch.uint8 and packed.is_contiguous(), "packed must be contiguous uint8")
    if out is None:
        out = torch.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=torch.float32,
                          device=packed.device)
    check("pkv_int4_dequantize", lib.pkv_int4_dequantize(
        _ptr(packed), 2 * packed.numel(), float(scale), PKV_F32, _ptr(out), _stream(packed.device)))
    return out


def fp8_dequantize(codes, scale=1.0, out_dtype=torch.float32, out=None):
    lib = load()
    _need(codes.dtype == torch.uint8 and codes.is_contiguous(), "codes must be contiguous uint8")
    if out is None:
        out = torch.empty(codes.shape, dtype=out_dtype, device=codes.device)
    check("pkv_fp8_e4m3_dequantize", lib.pkv_fp8_e4m3_dequantize(
        _ptr(codes), codes.numel(), float(scale), _DTYPES[out.dtype], _ptr(out), _stream(codes.device)))
    return out
