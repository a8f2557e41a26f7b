"""GPU parity: short multi-query requests (speculative decode, 2..8 query
tokens) in the chunked call, which runs them as decode work items holding a
request's query tokens for a whole group of heads (MFMA rows = tokens x
heads), against the oracle."""

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from oracle import attention

from helpers import gpu_or_skip, max_err, out_f64, say
from test_gpu_chunked import _chunk_case, _chunk_case_fp8, _run_chunked

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


# (Hq, Hkv, max query tokens): items of 8 or 16 MFMA rows, groups 1 .. 16
SHAPES = [(32, 8, 2), (32, 8, 4), (64, 8, 2), (8, 4, 8), (16, 8, 8), (8, 8, 8), (32, 8, 3),
          (64, 4, 4), (64, 8, 8)]   # last two: groups split into items of 4 and 2 heads


@pytest.mark.parametrize("Hq,Hkv,qmax", SHAPES)
@pytest.mark.parametrize("causal,W", [(True, 0), (True, 100), (False, 0), (False, 37)])
def test_multitoken_requests_match_the_oracle(Hq, Hkv, qmax, causal, W):
    """Twelve requests of up to 1500 keys (several pieces per item, so the
    merge runs), one to qmax query tokens each (single-query requests take
    the decode pass)."""
    say("multi-token", Hq, Hkv, qmax, causal, W)
    c = _chunk_case(3000 + Hq + Hkv + qmax + W + causal, R=12, Lmax=1500, qmax=qmax, Hq=Hq, Hkv=Hkv,
                    D=128, bs=16, v_sigma=0.2)
    out, ref = _run_chunked(c, causal, W)
    assert max_err(out_f64(out), ref) <= 2e-3


def test_multitoken_fp8_cache():
    say("multi-token fp8")
    c = _chunk_case_fp8(3100, R=10, Lmax=1200, qmax=4, Hq=32, Hkv=8, D=128, bs=16)

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(torch.from_numpy(c["kp"]).cuda(), torch.from_numpy(c["vp"]).cuda(),
                                      c["k_scale"], c["v_scale"])
    qmax = int(np.diff(c["qsl"]).max())
    out = pkv.paged_attention_chunked(dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(),
                                      torch.from_numpy(c["L"]).cuda(), qmax, cache,
                                      torch.from_numpy(c["bt"]).cuda(), int(c["L"].max()), 0.125)
    torch.cuda.synchronize()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "fp8", c["bt"], c["L"], c["qsl"], 0.125,
                                    k_scale=c["k_scale"], v_scale=c["v_scale"])
    assert max_err(out_f64(out), ref) <= 3e-2


def test_multitoken_inconsistent_lengths_get_nan_rows():
    """A multi-token request with more query tokens than keys: its rows are
    NaN, the other requests' rows exact."""
    say("multi-token inconsistent lengths")
    c = _chunk_case(3200, R=8, Lmax=400, qmax=4, Hq=32, Hkv=8, D=128, bs=16)
    ql = np.diff(c["qsl"])
    r = int(np.nonzero(ql >= 2)[0][0])
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"], c["qsl"], 0.125)
    L = c["L"].copy()
    L[r] = ql[r] - 1

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    out = pkv.paged_attention_chunked(dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(), torch.from_numpy(L).cuda(),
                                      int(ql.max()), cache, torch.from_numpy(c["bt"]).cuda(), int(c["L"].max()),
                                      0.125)
    torch.cuda.synchronize()
    got = out_f64(out)
    broken = np.zeros(int(c["qsl"][-1]), bool)
    broken[c["qsl"][r]:c["qsl"][r + 1]] = True
    assert np.isnan(got[broken]).all()
    assert max_err(got[~broken], ref[~broken]) <= 2e-3


def test_single_query_requests_ride_in_the_items():
    """A step declared with up to 4 query tokens whose requests all have one:
    every request runs as a multi-token item, and the output equals the
    oracle and the decode form's output for the same queries."""
    say("multi-token single-query requests")
    c = _chunk_case(3300, R=12, Lmax=900, qmax=1, Hq=32, Hkv=8, D=128, bs=16, v_sigma=0.2)
    assert (np.diff(c["qsl"]) == 1).all()

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    args = (torch.from_numpy(c["qsl"]).cuda(), torch.from_numpy(c["L"]).cuda())
    out = pkv.paged_attention_chunked(dev16(c["q"]), *args, 4, cache, torch.from_numpy(c["bt"]).cuda(),
                                      int(c["L"].max()), 0.125)
    dec = pkv.paged_attention_decode(dev16(c["q"]), cache, torch.from_numpy(c["bt"]).cuda(), args[1],
                                     int(c["L"].max()), 0.125)
    torch.cuda.synchronize()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"], c["qsl"], 0.125)
    assert max_err(out_f64(out), ref) <= 2e-3
    assert max_err(out_f64(dec), ref) <= 2e-3


def test_empty_requests_among_multi_token_requests():
    """Requests with no query tokens in a multi-token step: nothing is written
    for them and every other row matches the oracle."""
    say("multi-token empty requests")
    c = _chunk_case(3400, R=10, Lmax=700, qmax=4, Hq=32, Hkv=8, D=128, bs=16, v_sigma=0.2)
    ql = np.diff(c["qsl"])
    ql[[2, 5]] = 0
    c["qsl"] = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    T = int(c["qsl"][-1])
    c["q"] = c["q"][:T]

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    out = pkv.paged_attention_chunked(dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(),
                                      torch.from_numpy(c["L"]).cuda(), int(ql.max()), cache,
                                      torch.from_numpy(c["bt"]).cuda(), int(c["L"].max()), 0.125)
    torch.cuda.synchronize()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"], c["qsl"], 0.125)
    assert max_err(out_f64(out), ref) <= 2e-3


@pytest.mark.parametrize("qmax,W", [(1, 0), (4, 0), (4, 100), (64, 0)])
def test_blocks_not_shared_gives_the_same_bits(qmax, W):
    """The promise that no block is read by two requests only changes how
    the decode items load the cache (past the caches); single-query rows,
    multi-token items and prefill tiles return the same bits either way."""
    say("blocks not shared", qmax, W)
    c = _chunk_case(3300 + qmax + W, R=12, Lmax=1500, qmax=qmax, Hq=32, Hkv=8, D=128, bs=16, v_sigma=0.2)

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    args = (dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(), torch.from_numpy(c["L"]).cuda(),
            int(np.diff(c["qsl"]).max()), cache, torch.from_numpy(c["bt"]).cuda(), int(c["L"].max()), 0.125)
    plain = pkv.paged_attention_chunked(*args, causal=True, sliding_window=W)
    ntl = pkv.paged_attention_chunked(*args, causal=True, sliding_window=W, blocks_not_shared=True)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), ntl.view(torch.int16))
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"], c["qsl"], 0.125,
                                    causal=True, sliding_window=W)
    assert max_err(out_f64(ntl), ref) <= 2e-3


@pytest.mark.parametrize("qmax,W", [(1, 0), (4, 0), (4, 100), (64, 0)])
def test_blocks_shared_chunked_calls_match_the_oracle(qmax, W):
    """PKV_PLAN_BLOCKS_SHARED on a chunked call: its single-query rows and
    multi-token items run an eighth of their units per XCD (prefill tiles
    are unaffected); every output stays within the bound of the oracle."""
    say("blocks shared, chunked", qmax, W)
    c = _chunk_case(3500 + qmax + W, R=12, Lmax=1500, qmax=qmax, Hq=32, Hkv=8, D=128, bs=16, v_sigma=0.2)

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    cache = pkv.CacheView.from_planes(dev16(c["kp"]), dev16(c["vp"]))
    out = pkv.paged_attention_chunked(dev16(c["q"]), torch.from_numpy(c["qsl"]).cuda(),
                                      torch.from_numpy(c["L"]).cuda(), int(np.diff(c["qsl"]).max()), cache,
                                      torch.from_numpy(c["bt"]).cuda(), int(c["L"].max()), 0.125, causal=True,
                                      sliding_window=W, blocks_shared=True)
    torch.cuda.synchronize()
    ref = attention.paged_attention(c["q"], "bf16", c["kp"], c["vp"], "bf16", c["bt"], c["L"], c["qsl"], 0.125,
                                    causal=True, sliding_window=W)
    assert max_err(out_f64(out), ref) <= 2e-3
