"""GPU parity: chunked (mixed prefill + decode) paged attention and the hybrid
two-group workload."""

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from paged_kv_cache_mapping_amd import workloads
from paged_kv_cache_mapping_amd.workloads import bf16_bits
from oracle import attention

from helpers import gpu_or_skip, max_err, out_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


def _chunk_case(seed, R, Lmax, qmax, Hq, Hkv, D, bs, v_sigma=0.4):
    rng = np.random.default_rng(seed)
    L = rng.integers(1, Lmax + 1, size=R)
    ql = np.minimum(rng.integers(1, qmax + 1, size=R), L)
    ql[0] = 1
    nb = int(sum(-(-int(x) // bs) for x in L)) + 5
    perm = rng.permutation(nb)
    width = int(max(-(-int(x) // bs) for x in L))
    bt = np.full((R, width), -1, np.int32)
    k = 0
    for r in range(R):
        n = -(-int(L[r]) // bs)
        bt[r, :n] = perm[k:k + n]
        k += n
    shape = (nb, bs, Hkv, D)
    kp = bf16_bits(rng.standard_normal(shape).astype(np.float32) * 0.4)
    vp = bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(v_sigma))
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    q = bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32) * 0.4)
    return dict(L=L.astype(np.int32), qsl=qsl, bt=bt, kp=kp, vp=vp, q=q, nb=nb, bs=bs, Hkv=Hkv, D=D)


def _run_chunked(c, causal, W, scale=0.125):
    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    out = pkv.paged_attention_chunked(dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(),
                                      torch.from_numpy(c["L"]).cuda(), int(np.diff(c["qsl"]).max()),
                                      cache, torch.from_numpy(c["bt"]).cuda(), int(c["L"].max()),
                                      scale, causal=causal, sliding_window=W)
    torch.cuda.synchronize()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"],
                                    c["qsl"], scale, causal=causal, sliding_window=W)
    return out, ref


@pytest.mark.parametrize("R", [4096, 4100])
def test_chunked_many_requests(R):
    """Requests of one or two query tokens: 4096 of them run as multi-token
    decode items (the balanced scheme's row limit); 4100 fall back to the
    prefill tile for the two-token requests and to fixed splits for the
    others.  V is scaled so that outputs stay under 0.5 (a request of one
    or two keys returns V rows), where bf16 output rounding fits the
    tolerance."""
    say("chunked many requests", R)
    c = _chunk_case(900 + R, R=R, Lmax=64, qmax=2, Hq=8, Hkv=2, D=128, bs=16, v_sigma=0.1)
    out, ref = _run_chunked(c, True, 0)
    assert max_err(out_f64(out), ref) <= 2e-3


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("W", [0, 1, 7, 64, 1000])
def test_chunked_small_cases(causal, W):
    say("chunked small causal", causal, "W", W)
    c = _chunk_case(500 + W + causal, R=7, Lmax=400, qmax=70, Hq=8, Hkv=2, D=128, bs=16)
    out, ref = _run_chunked(c, causal, W)
    assert max_err(out_f64(out), ref) <= 2e-3


@pytest.mark.parametrize("D,bs,Hq,Hkv", [(64, 8, 4, 4), (128, 32, 16, 2), (256, 4, 8, 1)])
def test_chunked_shapes(D, bs, Hq, Hkv):
    say("chunked shapes", D, bs, Hq, Hkv)
    c = _chunk_case(600 + D + bs, R=5, Lmax=260, qmax=40, Hq=Hq, Hkv=Hkv, D=D, bs=bs)
    out, ref = _run_chunked(c, True, 0)
    assert max_err(out_f64(out), ref) <= 2e-3


def test_single_token_chunks_equal_decode_bit_for_bit():
    say("chunked q_len 1 == decode")
    w = workloads.llama8b_decode(batch=16)
    d = w.device()
    dec = pkv.paged_attention_decode(d.q, d.cache, d.block_table, d.seq_lens, w.max_seq_len, w.scale)
    chk = pkv.paged_attention_chunked(d.q, d.query_start_loc, d.seq_lens, 1, d.cache, d.block_table,
                                      w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(dec.view(torch.int16), chk.view(torch.int16))


def test_padding_rows_are_left_untouched():
    say("chunked padding rows")
    c = _chunk_case(700, R=3, Lmax=50, qmax=5, Hq=2, Hkv=1, D=64, bs=8)
    T = int(c["qsl"][-1])
    qpad = np.concatenate([c["q"], np.zeros((4,) + c["q"].shape[1:], np.uint16)])

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    out = torch.full((T + 4, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_chunked(dev16(qpad), torch.from_numpy(c["qsl"]).cuda(),
                                torch.from_numpy(c["L"]).cuda(), 5, cache,
                                torch.from_numpy(c["bt"]).cuda(), 50, 0.1, out=out)
    torch.cuda.synchronize()
    assert (out[T:].float() == 7.0).all()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"],
                                    c["qsl"], 0.1)
    assert max_err(out_f64(out[:T]), ref) <= 2e-3


def _chunk_case_fp8(seed, R, Lmax, qmax, Hq, Hkv, D, bs):
    """As _chunk_case, with K/V stored as E4M3 codes under per-tensor scales."""
    c = _chunk_case(seed, R, Lmax, qmax, Hq, Hkv, D, bs)
    rng = np.random.default_rng(seed + 1)
    shape = (c["nb"], bs, Hkv, D)
    kx = rng.standard_normal(shape).astype(np.float32)
    vx = rng.standard_normal(shape).astype(np.float32)
    c["k_scale"] = float(np.float32(np.abs(kx).max() / 448.0))
    c["v_scale"] = float(np.float32(np.abs(vx).max() / 448.0))
    c["kp"] = workloads.fp8_codes(kx, c["k_scale"])
    c["vp"] = workloads.fp8_codes(vx, c["v_scale"])
    return c


@pytest.mark.parametrize("D,bs,Hq,Hkv", [(128, 16, 8, 2), (64, 32, 16, 1)])
def test_chunked_fp8_cache(D, bs, Hq, Hkv):
    """E4M3 cache through the chunked call: prefill rows on the matrix-core
    kernel (fp8 widened to bf16 while staging), against the oracle on the
    dequantised cache."""
    say("chunked fp8", D, bs, Hq, Hkv)
    c = _chunk_case_fp8(810 + D, R=5, Lmax=300, qmax=90, Hq=Hq, Hkv=Hkv, D=D, bs=bs)

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(torch.from_numpy(c["kp"]).cuda(), torch.from_numpy(c["vp"]).cuda(),
                                      c["k_scale"], c["v_scale"])
    out = pkv.paged_attention_chunked(dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(),
                                      torch.from_numpy(c["L"]).cuda(), int(np.diff(c["qsl"]).max()),
                                      cache, torch.from_numpy(c["bt"]).cuda(), int(c["L"].max()), 0.09)
    torch.cuda.synchronize()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "fp8", c["bt"], c["L"],
                                    c["qsl"], 0.09, k_scale=c["k_scale"], v_scale=c["v_scale"])
    assert np.isfinite(out_f64(out)).all()
    assert max_err(out_f64(out), ref) <= 3e-2


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (16, 2), (16, 1)])
@pytest.mark.parametrize("causal,W", [(True, 0), (True, 300), (False, 100)])
def test_chunked_long_queries_span_several_tiles(Hq, Hkv, causal, W):
    """Queries of up to 600 tokens: several query tiles per request (ragged
    last tile), keys over many 32-key tiles, windows that start mid-tile.
    Early causal rows see one or two keys, so their outputs are single V
    values; V ~ N(0, 0.2^2) keeps every output below 1, where bf16's own
    rounding of the output stays inside the 2e-3 bound."""
    say("chunked long queries", Hq, Hkv, causal, W)
    c = _chunk_case(900 + Hq + Hkv + W, R=4, Lmax=900, qmax=600, Hq=Hq, Hkv=Hkv, D=128, bs=16,
                    v_sigma=0.2)
    out, ref = _run_chunked(c, causal, W)
    assert max_err(out_f64(out), ref) <= 2e-3


def test_chunked_stale_workspace_contents_do_not_matter():
    """The chunked call on a workspace that a different step used before
    (all requests single-query, so every row left a piece count and output
    row behind): rows of multi-query requests are skipped by the
    single-query pass, which must still leave a piece count of 0 for them so
    that the merge phase never reads the stale counts.  The workspace starts
    zeroed, as the contract asks, and is never cleared again."""
    say("chunked stale workspace")
    c = _chunk_case(1700, R=9, Lmax=400, qmax=60, Hq=8, Hkv=2, D=128, bs=16)

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    T, R = int(c["qsl"][-1]), len(c["L"])
    qmax, Lmax = int(np.diff(c["qsl"]).max()), int(c["L"].max())
    n = pkv.chunked_workspace_size(T, R, 8, cache, qmax, Lmax)
    ws = pkv.new_workspace(n, "cuda")
    # the earlier step: one query per request, at each request's last position
    qsl1 = np.arange(R + 1, dtype=np.int32)
    q1 = c["q"][c["qsl"][1:] - 1].copy()
    pkv.paged_attention_chunked(dev16(q1), torch.from_numpy(qsl1).cuda(), torch.from_numpy(c["L"]).cuda(),
                                qmax, cache, torch.from_numpy(c["bt"]).cuda(), Lmax, 0.125, workspace=ws)
    for _ in range(2):
        out = pkv.paged_attention_chunked(dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(),
                                          torch.from_numpy(c["L"]).cuda(), qmax, cache,
                                          torch.from_numpy(c["bt"]).cuda(), Lmax, 0.125, workspace=ws)
        torch.cuda.synchronize()
        ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"],
                                        c["qsl"], 0.125)
        assert max_err(out_f64(out), ref) <= 2e-3


def test_chunked_unmapped_block_poisons_only_rows_that_reach_it():
    """A prefill request whose table has an unmapped entry: causal rows whose
    keys stop before that block are exact, rows that reach it are NaN."""
    say("chunked unmapped block")
    bs, D, Hq, Hkv = 16, 128, 8, 2
    rng = np.random.default_rng(77)
    L = np.array([10, 200], np.int32)
    ql = np.array([1, 40], np.int32)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    nb = 64
    perm = rng.permutation(nb)
    bt = np.full((2, 13), -1, np.int32)
    bt[0, :1] = perm[:1]
    bt[1, :13] = perm[1:14]
    shape = (nb, bs, Hkv, D)
    kp = bf16_bits(rng.standard_normal(shape).astype(np.float32) * 0.4)
    vp = bf16_bits(rng.standard_normal(shape).astype(np.float32) * 0.4)
    q = bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32) * 0.4)
    ref = attention.paged_attention(q, "bf16", kp, vp, "bf16", bt, L, qsl, 0.125)
    bad = bt.copy()
    bad[1, 11] = -1                       # keys 176..191

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(kp), dev16(vp))
    out = pkv.paged_attention_chunked(dev16(q), torch.from_numpy(qsl).cuda(), torch.from_numpy(L).cuda(),
                                      40, cache, torch.from_numpy(bad).cuda(), 200, 0.125)
    torch.cuda.synchronize()
    got = out_f64(out)
    pos = 160 + np.arange(40)             # positions of request 1's queries
    reach = pos >= 176
    rows = 1 + np.arange(40)
    assert np.isnan(got[rows[reach]]).all()
    assert max_err(got[rows[~reach]], ref[rows[~reach]]) <= 2e-3
    assert max_err(got[:1], ref[:1]) <= 2e-3


def test_chunked_requests_with_inconsistent_lengths_get_nan_rows():
    """Requests whose lengths contradict the arguments (q_len > seq_len, or
    seq_len > max_seq_len), among valid single- and multi-query requests:
    their rows are NaN, every other row is exact.  The reference uses the
    valid lengths, so only the rows of the two broken requests differ."""
    say("chunked inconsistent lengths")
    c = _chunk_case(1900, R=7, Lmax=300, qmax=50, Hq=8, Hkv=2, D=128, bs=16)
    ql = np.diff(c["qsl"])
    multi = [r for r in range(1, 7) if ql[r] >= 2]
    assert len(multi) >= 2
    short, long_ = multi[0], multi[1]
    Lmax = int(c["L"].max())
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"], c["qsl"], 0.125)
    L = c["L"].copy()
    L[short] = ql[short] - 1              # fewer keys than queries
    L[long_] = Lmax + 5                   # past max_seq_len

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    out = pkv.paged_attention_chunked(dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(), torch.from_numpy(L).cuda(),
                                      int(ql.max()), cache, torch.from_numpy(c["bt"]).cuda(), Lmax, 0.125)
    torch.cuda.synchronize()
    got = out_f64(out)
    broken = np.zeros(int(c["qsl"][-1]), bool)
    for r in (short, long_):
        broken[c["qsl"][r]:c["qsl"][r + 1]] = True
    assert np.isnan(got[broken]).all()
    assert max_err(got[~broken], ref[~broken]) <= 2e-3


def test_chunked_one_long_item_cut_by_every_share():
    """One prefill item (64 queries, one KV head) over 20,000 keys: the
    balanced partition cuts it at every share boundary, so the merge combines
    one piece from every share."""
    say("chunked one item over every share")
    bs, D, Hq, Hkv = 16, 128, 8, 1
    rng = np.random.default_rng(2024)
    L = np.array([20000], np.int32)
    ql = np.array([64], np.int32)
    qsl = np.array([0, 64], np.int32)
    nblk = -(-int(L[0]) // bs)
    nb = nblk + 7
    bt = rng.permutation(nb)[:nblk].astype(np.int32).reshape(1, nblk)
    shape = (nb, bs, Hkv, D)
    kp = bf16_bits(rng.standard_normal(shape).astype(np.float32) * 0.4)
    vp = bf16_bits(rng.standard_normal(shape).astype(np.float32) * 0.4)
    q = bf16_bits(rng.standard_normal((64, Hq, D)).astype(np.float32) * 0.4)
    ref = attention.paged_attention(q, "bf16", kp, vp, "bf16", bt, L, qsl, 0.125)

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(kp), dev16(vp))
    out = pkv.paged_attention_chunked(dev16(q), torch.from_numpy(qsl).cuda(), torch.from_numpy(L).cuda(), 64,
                                      cache, torch.from_numpy(bt).cuda(), int(L[0]), 0.125)
    torch.cuda.synchronize()
    assert max_err(out_f64(out), ref) <= 2e-3


def _long_prefill_case(seed, lens, qlens, Hq, Hkv, D, bs):
    """Prefill chunks at the end of very long contexts; V carries a +-1 offset
    per group of 64 positions (and K, Q plain noise), so that a dropped or
    repeated key tile shows at several times the per-element bound."""
    rng = np.random.default_rng(seed)
    R = len(lens)
    L = np.asarray(lens, np.int32)
    ql = np.asarray(qlens, np.int32)
    nb = int(sum(-(-int(x) // bs) for x in L)) + 3
    perm = rng.permutation(nb)
    width = int(max(-(-int(x) // bs) for x in L))
    bt = np.full((R, width), -1, np.int32)
    kp = np.zeros((nb, bs, Hkv, D), np.uint16)
    vp = np.zeros((nb, bs, Hkv, D), np.uint16)
    k = 0
    for r in range(R):
        n = -(-int(L[r]) // bs)
        bt[r, :n] = perm[k:k + n]
        k += n
        pos = int(L[r])
        kr = rng.standard_normal((pos, Hkv, D), dtype=np.float32) * np.float32(0.35)
        sig = rng.choice([-1.0, 1.0], size=(-(-pos // 64), Hkv, D)).astype(np.float32)
        vr = rng.standard_normal((pos, Hkv, D), dtype=np.float32) * np.float32(0.35) + \
            np.repeat(sig, 64, axis=0)[:pos]
        pad = n * bs - pos
        kr = np.concatenate([kr, np.zeros((pad, Hkv, D), np.float32)]).reshape(n, bs, Hkv, D)
        vr = np.concatenate([vr, np.zeros((pad, Hkv, D), np.float32)]).reshape(n, bs, Hkv, D)
        kp[bt[r, :n]] = bf16_bits(kr)
        vp[bt[r, :n]] = bf16_bits(vr)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    q = bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32) * 0.35)
    return dict(L=L, qsl=qsl, bt=bt, kp=kp, vp=vp, q=q, nb=nb, bs=bs, Hkv=Hkv, D=D)


def test_prefill_tile_takes_long_contexts():
    """Contexts whose table slice takes the prefill tile past 64 KiB of LDS
    (about 120K tokens at head size 128, block size 16) stay on the tile:
    the chunked call's workspace for the multi-query part is the tile's, the
    same as for a short context, and the output is within the per-element
    bound of every element."""
    from helpers import check_close
    props = torch.cuda.get_device_properties(0)
    say("long-context prefill, LDS per block", getattr(props, "shared_memory_per_block", None))
    lens, qlens = [125000, 119001], [40, 17]
    Hq, Hkv, D, bs = 4, 2, 128, 16
    c = _long_prefill_case(4100, lens, qlens, Hq, Hkv, D, bs)
    cache = pkv.CacheView.from_planes(
        torch.from_numpy(c["kp"].view(np.int16)).view(torch.bfloat16).cuda(),
        torch.from_numpy(c["vp"].view(np.int16)).view(torch.bfloat16).cuda())

    def multi_part(max_seq_len):
        T, R = int(c["qsl"][-1]), len(lens)
        return (pkv.chunked_workspace_size(T, R, Hq, cache, max(qlens), max_seq_len, 0)
                - pkv.chunked_workspace_size(T, R, Hq, cache, 1, max_seq_len, 0))
    assert multi_part(max(lens)) == multi_part(4096)
    out = pkv.paged_attention_chunked(
        torch.from_numpy(c["q"].view(np.int16)).view(torch.bfloat16).cuda(), torch.from_numpy(c["qsl"]).cuda(),
        torch.from_numpy(c["L"]).cuda(), max(qlens), cache, torch.from_numpy(c["bt"]).cuda(), max(lens), 0.125)
    torch.cuda.synchronize()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"], c["qsl"], 0.125)
    # floor: the fp32 sums over 120K keys of unit-scale V (outputs ~0.02);
    # a dropped or repeated 32-key tile moves an output by about 3e-4
    check_close("long_context_prefill", out_f64(out), ref, 2e-3, 5e-5)
