"""GPU parity for the INT4 KV cache (half a byte per element; Worker-Side KV
Init (zh), § KV Cache技术背景): the codec, the cache write and block copies
bit-exact against the oracle; decode, short multi-query and prefill-chunk
attention against the oracle's attention over the same codes.

Tolerance: the oracle attends over the dequantised codes in float64, so the
kernels differ from it only by their own arithmetic -- bf16 query, exact
bf16 K values (192 + u), float32 accumulation, the bf16 output -- which is
the arithmetic of the bf16 path; the bf16 bound 2e-3 applies, read as an
absolute bound for outputs below 1 (every case keeps |value| <= 8 * scale < 1,
since a one-key window returns a V value itself, rounded to bf16).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from paged_kv_cache_mapping_amd import workloads
from oracle import attention, int4, paging

from helpers import (check_close, gpu_or_skip, host_bits, max_err, oracle_decode_step, out_f64, run_decode_step,
                     say)

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


def _bits_to_f32(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.0567, 2.5e-3, 40.0])
def test_codec_every_bf16_pattern(scale):
    say("int4 codec bf16", scale)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = pkv.int4_quantize(x, scale).cpu().numpy()
    np.testing.assert_array_equal(got, int4.quantize_packed(_bits_to_f32(bits), scale))


def test_codec_f32_source_and_dequantize():
    say("int4 codec f32")
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(40000) * 5).astype(np.float32)
    x[:8] = [np.nan, np.inf, -np.inf, 0.0, -0.0, 7.5, -8.5, 6.5]
    got = pkv.int4_quantize(torch.from_numpy(x).cuda(), 0.7).cpu().numpy()
    np.testing.assert_array_equal(got, int4.quantize_packed(x, 0.7))
    packed = rng.integers(0, 256, size=5000, dtype=np.uint8)
    for s in (0.3, 1.7e-3):
        deq = pkv.int4_dequantize(torch.from_numpy(packed).cuda(), s).cpu().numpy()
        np.testing.assert_array_equal(deq, int4.dequantize(packed, s).astype(np.float32))


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_cache_write_bit_exact(src):
    """Scatter into an int4 cache: every byte as the oracle writes it; padding
    slots, slots past the pool and untouched blocks keep their bytes."""
    say("int4 cache write", src)
    rng = np.random.default_rng(31)
    nb, bs, H, D, T = 40, 16, 8, 128, 300
    kp = rng.integers(0, 256, size=(nb, bs, H, D // 2), dtype=np.uint8)
    vp = rng.integers(0, 256, size=(nb, bs, H, D // 2), dtype=np.uint8)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[[3, 50, 120]] = [-1, nb * bs, nb * bs + 77]
    kx = (rng.standard_normal((T, H, D)) * 0.4).astype(np.float32)
    vx = (rng.standard_normal((T, H, D)) * 0.4).astype(np.float32)
    kx[0, 0, :4] = [np.nan, np.inf, -np.inf, 0.0]
    ks, vs = 0.11, 0.07
    if src == "bf16":
        key, val = workloads.bf16_bits(kx), workloads.bf16_bits(vx)
        tk = torch.from_numpy(key.view(np.int16)).view(torch.bfloat16).cuda()
        tv = torch.from_numpy(val.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        key, val = kx, vx
        tk, tv = torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda()
    kd, vd = torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda()
    cache = pkv.CacheView.from_planes(kd, vd, ks, vs, int4=True)
    pkv.cache_write(tk, tv, torch.from_numpy(slots).cuda(), cache)
    torch.cuda.synchronize()
    ok = np.where((slots >= 0) & (slots < nb * bs), slots, -1)
    k_ref, v_ref = paging.cache_write(kp, vp, key, val, ok, src, "int4", ks, vs)
    np.testing.assert_array_equal(kd.cpu().numpy(), k_ref)
    np.testing.assert_array_equal(vd.cpu().numpy(), v_ref)


def test_copy_blocks_bit_exact():
    say("int4 copy blocks")
    rng = np.random.default_rng(41)
    nb, bs, H, D = 300, 16, 8, 128
    kp = rng.integers(0, 256, size=(nb, bs, H, D // 2), dtype=np.uint8)
    vp = rng.integers(0, 256, size=(nb, bs, H, D // 2), dtype=np.uint8)
    perm = rng.permutation(nb)
    src, dst = perm[:100].astype(np.int32), perm[100:200].astype(np.int32)
    kd, vd = torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda()
    cache = pkv.CacheView.from_planes(kd, vd, 0.5, 0.5, int4=True)
    pkv.copy_blocks(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), cache)
    torch.cuda.synchronize()
    k_ref, v_ref, bad = paging.copy_blocks(kp, vp, src, dst)
    assert bad == 0
    np.testing.assert_array_equal(kd.cpu().numpy(), k_ref)
    np.testing.assert_array_equal(vd.cpu().numpy(), v_ref)


def _small(seed, B, Lmin, Lmax, Hq, Hkv, bs):
    return workloads.decode_workload(
        "small_int4", seed, lambda rng: rng.integers(Lmin, Lmax + 1, size=B), None,
        pool_blocks=int(B * (-(-Lmax // bs)) + 7), block_size=bs, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=128, cache_dtype="int4", q_dtype="bf16", sigma=0.2)   # values within +-0.8


def _attend(w, window=0, split=None):
    d = w.device()
    if split is None:
        out = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale,
                                         sliding_window=window)
    else:
        plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len, window)
        pkv.tune_plan(plan, w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len, window, split_blocks=split,
                      num_workers=max(1, plan.num_workers // split))
        ws = pkv.new_workspace(plan.workspace_bytes, "cuda")
        out = torch.empty_like(d.q)
        pkv.paged_attention_decode_partials(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale,
                                            plan, ws, out, sliding_window=window)
        pkv.paged_attention_decode_combine(out, d.seq_lens, w.block_size, plan, ws, sliding_window=window)
    torch.cuda.synchronize()
    ref = attention.paged_decode(w.q, "bf16", w.k_plane, w.v_plane, "int4", w.block_table, w.seq_lens,
                                 w.scale, sliding_window=window, k_scale=w.k_scale, v_scale=w.v_scale)
    return out, ref


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (16, 8), (64, 8), (32, 2), (64, 4), (12, 3)])
@pytest.mark.parametrize("bs", [16, 32])
def test_decode_groups_and_block_sizes(Hq, Hkv, bs):
    """Groups 1, 2, 4 (items over two KV heads), 8, 16 (two items of 8 heads)
    and an odd KV head count (single-head items) over ragged lengths 1..700
    (single tokens, partial blocks, several pieces per row)."""
    say("int4 decode", Hq, Hkv, bs)
    w = _small(700 + Hq + Hkv + bs, 9, 1, 700, Hq, Hkv, bs)
    out, ref = _attend(w)
    assert max_err(out_f64(out), ref) <= TOL


@pytest.mark.parametrize("W", [1, 17, 300])
def test_decode_sliding_window(W):
    say("int4 decode window", W)
    w = _small(800 + W, 11, 1, 900, 32, 8, 16)
    out, ref = _attend(w, window=W)
    assert max_err(out_f64(out), ref) <= TOL


@pytest.mark.parametrize("split", [1, 2, 8])
def test_decode_split_plans(split):
    """Finer and coarser balanced shares (more or fewer pieces to merge)."""
    say("int4 decode split", split)
    w = _small(900 + split, 13, 200, 1500, 32, 8, 16)
    out, ref = _attend(w, split=split)
    assert max_err(out_f64(out), ref) <= TOL


@pytest.mark.parametrize("hpi", [4, 8])
def test_single_head_and_pair_items_agree_with_the_oracle(hpi):
    """Group 4: the planner's items over two KV heads (8 rows) and forced
    single-head items (4 rows) both match the oracle."""
    say("int4 items", hpi)
    w = _small(990, 10, 100, 1200, 32, 8, 16)
    d = w.device()
    plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len)
    assert plan.heads_per_item == 8
    pkv.tune_plan(plan, w.num_reqs, w.num_q_heads, d.cache, w.max_seq_len, heads_per_item=hpi)
    ws = pkv.new_workspace(plan.workspace_bytes, "cuda")
    out = torch.empty_like(d.q)
    pkv.paged_attention_decode_partials(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale,
                                        plan, ws, out)
    pkv.paged_attention_decode_combine(out, d.seq_lens, w.block_size, plan, ws)
    torch.cuda.synchronize()
    ref = attention.paged_decode(w.q, "bf16", w.k_plane, w.v_plane, "int4", w.block_table, w.seq_lens,
                                 w.scale, k_scale=w.k_scale, v_scale=w.v_scale)
    assert max_err(out_f64(out), ref) <= TOL


def test_unmapped_block_gives_nan_row_only():
    say("int4 unmapped")
    w = _small(950, 6, 100, 400, 32, 8, 16)
    w.block_table[2, 1] = -1
    d = w.device()
    out = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    o = out_f64(out)
    assert np.isnan(o[2]).all()
    rows = [0, 1, 3, 4, 5]
    ref = attention.paged_decode(w.q[rows], "bf16", w.k_plane, w.v_plane, "int4", w.block_table[rows],
                                 w.seq_lens[rows], w.scale, k_scale=w.k_scale, v_scale=w.v_scale)
    assert max_err(o[rows], ref) <= TOL


def test_full_int4_decode_step():
    """The full-size INT4 workload (64 Llama-3-8B-shaped sequences of
    128..2048 tokens): slot mapping, the write of each new token into the
    INT4 cache and the decode, as the bench runs them."""
    say("int4 full step")
    w = workloads.int4_decode()
    d = w.device()
    slots, out = run_decode_step(w, d)
    ref_slots, kp, vp, ref = oracle_decode_step(w, "bf16")
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert host_bits(d.cache.k).tobytes() == kp.tobytes()
    assert host_bits(d.cache.v).tobytes() == vp.tobytes()
    check_close("int4_decode_step", out_f64(out), ref, TOL, 1e-5)


def _int4_chunk_case(seed, R, Lmax, qmax, Hq, Hkv, bs=16):
    rng = np.random.default_rng(seed)
    L = rng.integers(1, Lmax + 1, size=R)
    ql = np.minimum(rng.integers(1, qmax + 1, size=R), L)
    nb = int(sum(-(-int(x) // bs) for x in L)) + 5
    perm = rng.permutation(nb)
    bt = np.full((R, int(max(-(-int(x) // bs) for x in L))), -1, np.int32)
    k = 0
    for r in range(R):
        n = -(-int(L[r]) // bs)
        bt[r, :n] = perm[k:k + n]
        k += n
    kp = workloads.int4_history(rng, (nb, bs, Hkv, 128))
    vp = workloads.int4_history(rng, (nb, bs, Hkv, 128))
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    q = workloads.bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, 128)).astype(np.float32) * 0.4)
    return dict(L=L.astype(np.int32), qsl=qsl, bt=bt, kp=kp, vp=vp, q=q)


def _run_int4_chunked(c, causal, W, ks=0.06, vs=0.05):
    cache = pkv.CacheView.from_planes(torch.from_numpy(c["kp"]).cuda(), torch.from_numpy(c["vp"]).cuda(),
                                      ks, vs, int4=True)
    q = torch.from_numpy(c["q"].view(np.int16)).view(torch.bfloat16).cuda()
    out = pkv.paged_attention_chunked(q, torch.from_numpy(c["qsl"]).cuda(), torch.from_numpy(c["L"]).cuda(),
                                      int(np.diff(c["qsl"]).max()), cache, torch.from_numpy(c["bt"]).cuda(),
                                      int(c["L"].max()), 0.125, causal=causal, sliding_window=W)
    torch.cuda.synchronize()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "int4", c["bt"], c["L"], c["qsl"], 0.125,
                                    causal=causal, sliding_window=W, k_scale=ks, v_scale=vs)
    return out, ref


@pytest.mark.parametrize("Hq,Hkv,qmax", [(32, 8, 4), (8, 8, 8), (64, 8, 2), (16, 1, 3)])
@pytest.mark.parametrize("causal,W", [(True, 0), (False, 45)])
def test_chunked_short_multi_query_requests(Hq, Hkv, qmax, causal, W):
    """Chunked steps with 1..8 query tokens per request: single-query rows
    on the decode kernels, the rest as multi-token items (8 MFMA rows)."""
    say("int4 chunked", Hq, Hkv, qmax, causal, W)
    c = _int4_chunk_case(1200 + Hq + qmax + W, 12, 1300, qmax, Hq, Hkv)
    out, ref = _run_int4_chunked(c, causal, W)
    assert max_err(out_f64(out), ref) <= TOL


@pytest.mark.parametrize("causal,W", [(True, 0), (True, 64), (False, 0)])
def test_chunked_prefill_chunks(causal, W):
    """Requests with up to 90 query tokens: the matrix-core prefill kernel
    stages INT4 tiles widened to the integers u - 8 (scales on the scores and
    the output); single-query rows on the decode kernels."""
    say("int4 chunked prefill", causal, W)
    c = _int4_chunk_case(1300 + W + causal, 6, 600, 90, 32, 8)
    out, ref = _run_int4_chunked(c, causal, W)
    assert max_err(out_f64(out), ref) <= TOL
