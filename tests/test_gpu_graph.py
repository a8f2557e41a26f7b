"""GPU: the decode step and the chunked call recorded in a HIP graph.

A serving loop replays a recorded step instead of launching its kernels one
by one.  The library's calls allocate nothing, copy nothing and clear no
memory (workspace slots are written before they are read), so a recorded
call must give, on every replay, the bits the eager call gave: the outputs,
the slots and the cache planes (a replayed decode step writes the same new
tokens to the same slots again).  Each replay follows eager work on the
device and a synchronisation, with the outputs poisoned in between, and is
checked on its own ([W] § Pinpointing the Token Slot, [P] § Handling
Softmax Across Blocks).  The chunked call's prefill part runs on a second
stream forked from and joined to the caller's, which the recording follows.
The decode entry point that allocates nothing (its partials in the
library's static scratch) is recorded too: it exists for such callers.
"""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from paged_kv_cache_mapping_amd import _lib, workloads

from helpers import gpu_or_skip, host_bits, say
from test_gpu_chunked import _chunk_case

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


def _eager_work():
    # unrelated work on the device between replays, then a full stop
    x = torch.randn(1 << 22, device="cuda")
    x.mul_(3.0).add_(1.0)
    float(x[:4096].sum())
    torch.cuda.synchronize()


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["llama8b", "fp8", "int4"])
def test_decode_step_replays_give_the_eager_bits(name):
    say("graph decode step", name)
    w = workloads.ALL[name]()
    d = w.device()
    plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len, blocks_not_shared=True)
    ws = pkv.new_workspace(plan.workspace_bytes, "cuda")
    out = torch.empty_like(d.q)
    slots = torch.full((w.num_reqs,), 12345, dtype=torch.int64, device="cuda")

    def step():
        pkv.paged_attention_decode_step(d.q, d.new_k, d.new_v, d.cache, d.block_table, d.seq_lens,
                                        w.max_seq_len, w.scale, plan, ws, out, slots=slots)

    step()
    torch.cuda.synchronize()
    ref_out, ref_slots = out.clone(), slots.clone()
    ref_k, ref_v = host_bits(d.cache.k).tobytes(), host_bits(d.cache.v).tobytes()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        slots.fill_(-7)
        _eager_work()
        g.replay()
        torch.cuda.synchronize()
        say("replay", i)
        assert _same_bits(out, ref_out)
        assert torch.equal(slots, ref_slots)
        assert host_bits(d.cache.k).tobytes() == ref_k
        assert host_bits(d.cache.v).tobytes() == ref_v


@pytest.mark.parametrize("qmax,W", [(1, 0), (4, 0), (64, 0), (64, 300)])
def test_chunked_replays_give_the_eager_bits(qmax, W):
    """Single-query rows (decode items), multi-token items, and prefill
    tiles on the second stream beside the decode items, with and without a
    window."""
    say("graph chunked", qmax, W)
    c = _chunk_case(4400 + qmax + W, R=12, Lmax=1500, qmax=qmax, Hq=32, Hkv=8, D=128, bs=16)

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    q = dev16(c["q"])
    qsl = torch.from_numpy(c["qsl"]).cuda()
    L = torch.from_numpy(c["L"]).cuda()
    bt = torch.from_numpy(c["bt"]).cuda()
    qmax_got, lmax = int(np.diff(c["qsl"]).max()), int(c["L"].max())
    T, Hq, _ = q.shape
    nbytes = pkv.chunked_workspace_size(T, L.numel(), Hq, cache, qmax_got, lmax, W)
    ws = pkv.new_workspace(nbytes, "cuda")
    out = torch.empty_like(q)

    def call():
        pkv.paged_attention_chunked(q, qsl, L, qmax_got, cache, bt, lmax, 0.125, causal=True,
                                    sliding_window=W, workspace=ws, out=out)

    call()
    torch.cuda.synchronize()
    ref = out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        _eager_work()
        g.replay()
        torch.cuda.synchronize()
        say("replay", i)
        assert _same_bits(out, ref)


def test_static_scratch_decode_replays_give_the_eager_bits():
    say("graph static-scratch decode")
    lib = _lib.load()
    w = workloads.llama8b_decode()
    d = w.device()
    out = torch.empty_like(d.q)

    def call():
        c = d.cache.c_struct()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        st = lib.pkv_paged_attention_decode_static(
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(d.q.data_ptr()), _lib.PKV_BF16, w.num_reqs,
            w.num_q_heads, ctypes.byref(c), ctypes.c_void_p(d.block_table.data_ptr()),
            d.block_table.shape[1], ctypes.c_void_p(d.seq_lens.data_ptr()), w.max_seq_len, w.scale, 0, stream)
        assert st == _lib.PKV_OK, pkv.status_string(st)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    ws_form = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    assert _same_bits(ref, ws_form)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        _eager_work()
        g.replay()
        torch.cuda.synchronize()
        say("replay", i)
        assert _same_bits(out, ref)
