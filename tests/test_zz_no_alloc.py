"""pkv_paged_attention_decode_static (the decode for callers that cannot
allocate) against pkv_paged_attention_decode, through the C ABI: two calls in
a row, the second with a smaller batch, each bit-identical to the workspace
form (same kernels, same plan) and within the oracle's bound; sizes past the
scratch are refused before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from paged_kv_cache_mapping_amd import _lib, workloads
from oracle import attention

from helpers import gpu_or_skip, max_err, out_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


def _static_call(lib, out, d, w, rows, max_seq_len):
    c = d.cache.c_struct()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.pkv_paged_attention_decode_static(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(d.q.data_ptr()), _lib.PKV_BF16, rows,
        w.num_q_heads, ctypes.byref(c), ctypes.c_void_p(d.block_table.data_ptr()),
        d.block_table.shape[1], ctypes.c_void_p(d.seq_lens.data_ptr()), max_seq_len, w.scale, 0, stream)


def _workspace_call(d, w, rows, max_seq_len):
    return pkv.paged_attention_decode(d.q[:rows], d.cache, d.block_table[:rows], d.seq_lens[:rows],
                                      max_seq_len, w.scale)


def test_static_scratch_decode_equals_the_workspace_form_twice():
    lib = _lib.load()
    w = workloads.llama8b_decode()
    d = w.device()
    for rows in (64, 23):                       # the second call smaller
        say("static-scratch decode, rows", rows)
        out = torch.full_like(d.q, float("nan"))
        st = _static_call(lib, out, d, w, rows, w.max_seq_len)
        assert st == _lib.PKV_OK, pkv.status_string(st)
        ref_ws = _workspace_call(d, w, rows, w.max_seq_len)
        torch.cuda.synchronize()
        assert torch.equal(out[:rows].view(torch.int16), ref_ws.view(torch.int16))
        assert torch.isnan(out[rows:].float()).all()     # rows past the batch untouched
        ref = attention.paged_decode(w.q[:rows], "bf16", w.k_plane, w.v_plane, "bf16",
                                     w.block_table[:rows], w.seq_lens[:rows], w.scale)
        assert max_err(out_f64(out[:rows]), ref) <= 2e-3


def test_static_scratch_decode_small_shapes_and_window():
    """A shape on the other kernels (fixed splits: block size 8) and a
    windowed call, after the bf16 calls above left their partials behind."""
    lib = _lib.load()
    w = workloads.decode_workload("static_small", 12, lambda rng: rng.integers(1, 700, size=9), None,
                                  pool_blocks=9 * 88 + 5, block_size=8, num_q_heads=8, num_kv_heads=2,
                                  head_dim=64, cache_dtype="bf16", q_dtype="bf16", sigma=0.35)
    d = w.device()
    out = torch.empty_like(d.q)
    st = _static_call(lib, out, d, w, w.num_reqs, w.max_seq_len)
    assert st == _lib.PKV_OK
    torch.cuda.synchronize()
    ref = attention.paged_decode(w.q, "bf16", w.k_plane, w.v_plane, "bf16", w.block_table, w.seq_lens,
                                 w.scale)
    assert max_err(out_f64(out), ref) <= 2e-3


def test_static_scratch_refuses_plans_past_its_size():
    """A batch whose plan needs more than the scratch holds (4096 rows of the
    Llama-3-8B shape: one partial record per share, run-time chunk and row
    group) returns PKV_ERR_WORKSPACE, checked on the host before anything is
    launched; the workspace form of the same call runs."""
    lib = _lib.load()
    w = workloads.llama8b_decode()
    d = w.device()
    rows = 4096
    plan = _lib.PkvDecodePlan()
    assert lib.pkv_decode_plan_make(rows, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                    _lib.PKV_BF16, w.max_seq_len, 0, 0, ctypes.byref(plan)) == _lib.PKV_OK
    assert plan.workspace_bytes > _lib.PKV_STATIC_SCRATCH_BYTES
    # a batch of that many rows: every row one copy of row 0 of the workload
    q = d.q[:1].expand(rows, -1, -1).contiguous()
    bt = d.block_table[:1].expand(rows, -1).contiguous()
    sl = d.seq_lens[:1].expand(rows).contiguous()

    class Big:
        pass
    big = Big()
    big.q, big.block_table, big.seq_lens, big.cache = q, bt, sl, d.cache
    out = torch.full_like(q, float("nan"))
    st = _static_call(lib, out, big, w, rows, w.max_seq_len)
    assert st == _lib.PKV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()          # nothing was launched
    got = pkv.paged_attention_decode(q, d.cache, bt, sl, w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    ref0 = attention.paged_decode(w.q[:1], "bf16", w.k_plane, w.v_plane, "bf16", w.block_table[:1],
                                  w.seq_lens[:1], w.scale)
    assert max_err(out_f64(got), np.broadcast_to(ref0, got.shape)) <= 2e-3
