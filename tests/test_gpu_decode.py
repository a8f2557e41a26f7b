"""GPU parity: paged decode attention against the fp64 oracle.

Tolerances (max-abs): bf16 output with bf16 KV 2e-3; fp8 KV 3e-2 (against the
oracle over the same dequantised cache); f32 everything 1e-5 (float32
accumulation over at most a few thousand terms of unit-size values).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from paged_kv_cache_mapping_amd import workloads
from oracle import attention, paging

from helpers import (check_close, gpu_or_skip, host_bits, max_err, oracle_decode_step, out_f64,
                     run_decode_step, say)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8": 3e-2}


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


@pytest.mark.parametrize("name", ["tiny", "llama8b", "llama70b", "fp8"])
def test_full_decode_step_matches_oracle(name):
    say("decode step", name)
    w = workloads.ALL[name]()
    d = w.device()
    slots, out = run_decode_step(w, d)
    ref_slots, kp, vp, ref = oracle_decode_step(w, w.q_dtype)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert host_bits(d.cache.k).tobytes() == kp.tobytes()
    assert host_bits(d.cache.v).tobytes() == vp.tobytes()
    if w.q_dtype == "f32":
        err = max_err(out_f64(out), ref)
        say(name, "max abs err", err)
        assert err <= TOL[w.cache_dtype]
    else:
        check_close("decode_step_" + name, out_f64(out), ref, TOL[w.cache_dtype],
                    1e-4 if w.cache_dtype == "fp8" else 1e-5)


def _small(seed, B, Lmax, Hq, Hkv, D, bs, dtype="bf16", Lmin=1, pool=None):
    def lengths(rng):
        return rng.integers(Lmin, Lmax + 1, size=B)
    nb = pool or int(B * (-(-Lmax // bs)) + 7)
    return workloads.decode_workload(
        "small", seed, lengths, None, pool_blocks=nb, block_size=bs, num_q_heads=Hq,
        num_kv_heads=Hkv, head_dim=D, cache_dtype=dtype, q_dtype="f32" if dtype == "f32" else "bf16",
        sigma=1.0 if dtype == "f32" else 0.35)


def _check_attention_only(w, window=0, plan_split=None, not_shared=False):
    """Decode attention over the planes as given (no write) vs the oracle."""
    d = w.device()
    if plan_split is None and not not_shared:
        out = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len,
                                         w.scale, sliding_window=window)
    else:
        plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len, window,
                               blocks_not_shared=not_shared)
        if plan_split is not None:
            workers = None if plan.scheme == 0 else max(1, plan.num_workers // plan_split)
            pkv.tune_plan(plan, w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len, window,
                          split_blocks=plan_split, num_workers=workers)
        ws = pkv.new_workspace(plan.workspace_bytes, "cuda")
        out = torch.empty_like(d.q)
        pkv.paged_attention_decode_partials(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len,
                                            w.scale, plan, ws, out, sliding_window=window)
        pkv.paged_attention_decode_combine(out, d.seq_lens, w.block_size, plan, ws,
                                           sliding_window=window)
    torch.cuda.synchronize()
    ref = attention.paged_decode(w.q, w.q_dtype, w.k_plane, w.v_plane, w.cache_dtype,
                                 w.block_table, w.seq_lens, w.scale, sliding_window=window,
                                 k_scale=w.k_scale, v_scale=w.v_scale)
    return out, max_err(out_f64(out), ref)


@pytest.mark.parametrize("D", [8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("bs", [4, 16, 32])
def test_head_dims_and_block_sizes(D, bs):
    say("decode D", D, "bs", bs)
    w = _small(40 + D + bs, B=5, Lmax=300, Hq=4, Hkv=2, D=D, bs=bs)
    _, err = _check_attention_only(w)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("B,scheme", [(1500, 1), (4096, 1), (4097, 0)])
def test_many_rows(B, scheme):
    """Batches past the rows whose records the balanced kernel keeps in LDS
    (1024), at its limit (4096 rows of prefix sums in LDS), and one row past
    it, where the plan falls back to fixed splits.  Rows of at least 32 keys
    keep the outputs under 0.3, where bf16 rounding of the output stays
    inside the tolerance (a row of one or two keys returns V rows near 1,
    whose bf16 half-ulp alone is 3.9e-3)."""
    say("decode rows", B)
    w = _small(200 + B, B=B, Lmax=96, Hq=8, Hkv=2, D=128, bs=16, Lmin=32)
    plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, w.device().cache, w.max_seq_len)
    assert plan.scheme == scheme
    _, err = _check_attention_only(w)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 1), (8, 2), (16, 2), (32, 8), (64, 8), (16, 1)])
def test_group_sizes(Hq, Hkv):
    say("decode group", Hq, Hkv)
    w = _small(70 + Hq, B=6, Lmax=500, Hq=Hq, Hkv=Hkv, D=64, bs=16)
    _, err = _check_attention_only(w)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "fp8"])
def test_f32_and_fp8_small(dtype):
    say("decode small", dtype)
    if dtype == "fp8":
        w = workloads.decode_workload(
            "small_fp8", 91, lambda rng: rng.integers(1, 900, size=7), lambda n: n + 5,
            block_size=8, num_q_heads=8, num_kv_heads=2, head_dim=64, cache_dtype="fp8",
            q_dtype="bf16", sigma=1.0)
    else:
        w = _small(92, B=7, Lmax=900, Hq=4, Hkv=1, D=16, bs=8, dtype="f32")
    _, err = _check_attention_only(w)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("W", [1, 2, 5, 16, 17, 100, 4096])
def test_sliding_window(W):
    say("decode window", W)
    w = _small(120 + W, B=9, Lmax=700, Hq=8, Hkv=2, D=128, bs=16)
    _, err = _check_attention_only(w, window=W)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("split", [1, 2, 3, 8, 64])
@pytest.mark.parametrize("not_shared", [False, True])
def test_any_split_plan_gives_the_same_answer(split, not_shared):
    say("decode split", split, "blocks not shared", not_shared)
    w = _small(150, B=6, Lmax=1500, Hq=32, Hkv=8, D=128, bs=16, Lmin=200)
    _, err = _check_attention_only(w, plan_split=split, not_shared=not_shared)
    assert err <= TOL["bf16"]
    _, err = _check_attention_only(w, window=333, plan_split=split, not_shared=not_shared)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("not_shared", [False, True])
@pytest.mark.parametrize("Hq,Hkv,dtype", [(64, 4, "bf16"), (64, 8, "bf16"), (32, 8, "fp8"), (64, 8, "fp8")])
def test_item_heights_and_dtypes(not_shared, Hq, Hkv, dtype):
    """Items of 16 and 8 rows (matrix-core and vector-ALU P.V) and fp8 items,
    with and without the non-temporal loads of unshared blocks (which fp8
    does not take)."""
    say("decode item heights", not_shared, Hq, Hkv, dtype)
    w = _small(160 + Hq + Hkv, B=7, Lmax=1300, Hq=Hq, Hkv=Hkv, D=128, bs=16, dtype=dtype, Lmin=100)
    _, err = _check_attention_only(w, plan_split=2, not_shared=not_shared)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("split", [1, 8, 64])
def test_vector_alu_fixed_split_path(split):
    """The vector-ALU kernels behind scheme 0 on a shape the matrix path would take."""
    say("decode fixed-split vector path", split)
    w = _small(151, B=5, Lmax=900, Hq=32, Hkv=8, D=128, bs=32, Lmin=100)
    d = w.device()
    plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len)
    if plan.scheme != 0:
        # build the equivalent scheme-0 plan by hand: vector kernels, fixed splits
        plan.scheme, plan.num_workers, plan.heads_per_item = 0, 0, 4
    pkv.tune_plan(plan, w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len, split_blocks=split)
    ws = pkv.new_workspace(plan.workspace_bytes, "cuda")
    out = torch.empty_like(d.q)
    pkv.paged_attention_decode_partials(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len,
                                        w.scale, plan, ws, out)
    pkv.paged_attention_decode_combine(out, d.seq_lens, w.block_size, plan, ws)
    torch.cuda.synchronize()
    ref = attention.paged_decode(w.q, "bf16", w.k_plane, w.v_plane, "bf16", w.block_table,
                                 w.seq_lens, w.scale)
    assert max_err(out_f64(out), ref) <= TOL["bf16"]


def test_phases_equal_the_one_call_form_bit_for_bit():
    say("decode phases vs one call")
    w = workloads.llama8b_decode()
    d = w.device()
    one = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale)
    plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len)
    ws = pkv.new_workspace(plan.workspace_bytes, "cuda")
    two = torch.empty_like(d.q)
    pkv.paged_attention_decode_partials(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len,
                                        w.scale, plan, ws, two)
    pkv.paged_attention_decode_combine(two, d.seq_lens, w.block_size, plan, ws)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


@pytest.mark.parametrize("split", [None, 4, 32])
def test_fp8_phases_called_separately(split):
    """fp8 cache through the two phases as separate calls: the merge phase
    takes no cache, so the partials must already carry the V scale.  Rows
    with several pieces are forced by small shares; the fixed-split vector
    kernels are covered as well (split 32 with scheme 0)."""
    say("decode fp8 phases", split)
    w = workloads.decode_workload(
        "fp8_phases", 93, lambda rng: rng.integers(200, 1500, size=9), lambda n: n + 5,
        block_size=16, num_q_heads=32, num_kv_heads=8, head_dim=128, cache_dtype="fp8",
        q_dtype="bf16", sigma=1.0)
    d = w.device()
    plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len)
    if split == 32:
        plan.scheme, plan.num_workers, plan.heads_per_item = 0, 0, 4
        pkv.tune_plan(plan, w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len, split_blocks=8)
    elif split is not None:
        pkv.tune_plan(plan, w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len,
                      num_workers=max(1, plan.num_workers // split))
    ws = pkv.new_workspace(plan.workspace_bytes, "cuda")
    out = torch.empty_like(d.q)
    pkv.paged_attention_decode_partials(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len,
                                        w.scale, plan, ws, out)
    pkv.paged_attention_decode_combine(out, d.seq_lens, w.block_size, plan, ws)
    one = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    ref = attention.paged_decode(w.q, w.q_dtype, w.k_plane, w.v_plane, w.cache_dtype,
                                 w.block_table, w.seq_lens, w.scale, k_scale=w.k_scale,
                                 v_scale=w.v_scale)
    assert max_err(out_f64(out), ref) <= TOL["fp8"]
    if split is None:
        assert torch.equal(one.view(torch.int16), out.view(torch.int16))


def test_physical_placement_does_not_change_a_single_bit():
    say("decode permutation invariance")
    w = workloads.llama8b_decode()
    d = w.device()
    base = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale)
    rng = np.random.default_rng(77)
    perm = rng.permutation(w.num_blocks)
    pt = torch.from_numpy(perm.astype(np.int64)).cuda()
    k2 = torch.empty_like(d.cache.k)
    v2 = torch.empty_like(d.cache.v)
    k2.index_copy_(0, pt, d.cache.k)
    v2.index_copy_(0, pt, d.cache.v)
    bt = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    cache2 = pkv.CacheView.from_planes(k2, v2)
    out = pkv.paged_attention_decode(d.q, cache2, torch.from_numpy(bt).cuda(), d.seq_lens,
                                     w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), out.view(torch.int16))


def test_unused_slots_poisoned_with_nan_are_never_read():
    say("decode NaN poison")
    w = _small(160, B=11, Lmax=777, Hq=8, Hkv=2, D=128, bs=16)
    clean, err = _check_attention_only(w)
    assert err <= TOL["bf16"]
    mask = paging.unused_slot_mask(w.num_blocks, w.block_size, w.block_table, w.seq_lens)
    w.k_plane[mask] = 0x7FC0
    w.v_plane[mask] = 0x7FC0
    poisoned, err2 = _check_attention_only(w)
    assert torch.equal(clean.view(torch.int16), poisoned.view(torch.int16))


def test_window_skips_blocks_before_the_window():
    say("decode window ignores released blocks")
    W = 40
    w = _small(170, B=5, Lmax=600, Hq=4, Hkv=1, D=64, bs=8, Lmin=100)
    clean, err = _check_attention_only(w, window=W)
    assert err <= TOL["bf16"]
    # release every block wholly before the window: -1 in the table, NaN data
    for r, L in enumerate(w.seq_lens):
        first = max(0, int(L) - W) // w.block_size
        for b in range(first):
            w.k_plane[w.block_table[r, b]] = 0x7FC0
            w.v_plane[w.block_table[r, b]] = 0x7FC0
            w.block_table[r, b] = -1
    rel, err2 = _check_attention_only(w, window=W)
    assert torch.equal(clean.view(torch.int16), rel.view(torch.int16))


def test_edge_cases_empty_batch_length_one_and_invalid_rows():
    say("decode edge cases")
    w = _small(180, B=6, Lmax=64, Hq=4, Hkv=2, D=64, bs=16)
    d = w.device()
    empty = pkv.paged_attention_decode(d.q[:0], d.cache, d.block_table[:0], d.seq_lens[:0],
                                       w.max_seq_len, w.scale)
    assert empty.shape[0] == 0
    lens = w.seq_lens.copy()
    lens[0] = 1                 # a single key: output is that value row
    lens[1] = 0                 # invalid: no keys -> NaN
    lens[2] = w.max_seq_len + 1  # beyond max_seq_len -> NaN
    bt = w.block_table.copy()
    bt[3, 0] = w.num_blocks + 3  # missing block -> NaN, never dereferenced
    out = pkv.paged_attention_decode(d.q, d.cache, torch.from_numpy(bt).cuda(),
                                     torch.from_numpy(lens).cuda(), w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    o = out_f64(out)
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all() and np.isnan(o[3]).all()
    assert np.isfinite(o[[0, 4, 5]]).all()
    v0 = attention.paged_decode(w.q[:1], "bf16", w.k_plane, w.v_plane, "bf16", w.block_table[:1],
                                [1], w.scale)
    assert max_err(o[:1], v0) <= TOL["bf16"]
    ref = attention.paged_decode(w.q[4:], "bf16", w.k_plane, w.v_plane, "bf16", w.block_table[4:],
                                 w.seq_lens[4:], w.scale)
    assert max_err(o[4:], ref) <= TOL["bf16"]


@pytest.mark.parametrize("rows", [23, 64])
def test_stale_workspace_gives_the_same_bits(rows):
    """A workspace that a larger call used before (its partial records and
    row-group entries left behind) gives exactly the bits of a fresh one:
    every record a merge reads was written by the same call.  Batches with
    fewer units than the workers could take leave static shares empty."""
    say("decode stale workspace", rows)
    w = workloads.llama8b_decode()
    d = w.device()
    big = pkv.decode_plan(w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len)
    ws = pkv.new_workspace(big.workspace_bytes, "cuda")
    junk = torch.empty_like(d.q)
    pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale,
                               workspace=ws, out=junk)
    stale = pkv.paged_attention_decode(d.q[:rows], d.cache, d.block_table[:rows], d.seq_lens[:rows],
                                       w.max_seq_len, w.scale, workspace=ws)
    fresh = pkv.paged_attention_decode(d.q[:rows], d.cache, d.block_table[:rows], d.seq_lens[:rows],
                                       w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(stale.view(torch.int16), fresh.view(torch.int16))
    ref = attention.paged_decode(w.q[:rows], "bf16", w.k_plane, w.v_plane, "bf16", w.block_table[:rows],
                                 w.seq_lens[:rows], w.scale)
    check_close("stale_ws_%d" % rows, out_f64(stale), ref, 2e-3, 1e-5)
