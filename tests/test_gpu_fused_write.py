"""GPU parity: slot mapping and the cache write in one launch
(pkv_slot_mapping_cache_write) against the oracle's slot mapping followed by
its cache write -- slots, error counts and every byte of both planes
(Worker-Side KV Init, § Pinpointing the Token Slot and § Summary)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from paged_kv_cache_mapping_amd import workloads
from oracle import paging

from helpers import gpu_or_skip, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


def _planes_equal(cache, kp, vp):
    assert host_bits(cache.k).tobytes() == np.ascontiguousarray(kp).tobytes()
    assert host_bits(cache.v).tobytes() == np.ascontiguousarray(vp).tobytes()


@pytest.mark.parametrize("name", ["tiny", "llama8b", "fp8", "int4"])
def test_fused_step_write_matches_the_oracle(name):
    say("fused write", name)
    w = workloads.ALL[name]()
    d = w.device()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    slots = pkv.slot_mapping_cache_write(d.block_table, d.query_start_loc, d.num_computed, d.new_k, d.new_v,
                                         d.cache, err_count=err)
    torch.cuda.synchronize()
    ref_slots, werr = paging.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, w.block_size,
                                          num_blocks=w.num_blocks)
    assert np.array_equal(slots.cpu().numpy(), ref_slots) and int(err.item()) == werr == 0
    kp, vp = paging.cache_write(w.k_plane, w.v_plane, w.new_k, w.new_v, ref_slots, w.q_dtype, w.cache_dtype,
                                w.k_scale, w.v_scale)
    _planes_equal(d.cache, kp, vp)


def _random_case(seed, R, max_q, nb, bs, extra_tokens):
    rng = np.random.default_rng(seed)
    ql = rng.integers(0, max_q + 1, size=R)
    nc = rng.integers(0, 200, size=R)
    width = int(np.max(-(-(nc + ql) // bs))) + 1
    bt = rng.integers(-1, nb + 20, size=(R, width)).astype(np.int32)      # some bad ids
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    T = int(qsl[-1]) + extra_tokens                                        # padding tokens
    return rng, bt, qsl, nc.astype(np.int32), T


@pytest.mark.parametrize("R,max_q", [(37, 40), (1500, 2)])
def test_fused_bad_lookups_padding_and_many_requests(R, max_q):
    """Bad table entries (counted, not written), padding tokens past the last
    request, empty requests; 1500 requests exceed the metadata a workgroup
    stages in LDS."""
    say("fused write random", R, max_q)
    bs, nb, H, D = 16, 400, 4, 128
    rng, bt, qsl, nc, T = _random_case(500 + R, R, max_q, nb, bs, 9)
    kp0 = rng.integers(0, 1 << 16, size=(nb, bs, H, D), dtype=np.uint16)
    vp0 = rng.integers(0, 1 << 16, size=(nb, bs, H, D), dtype=np.uint16)
    key = workloads.bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    val = workloads.bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    kd, vd = dev16(kp0.copy()), dev16(vp0.copy())
    cache = pkv.CacheView.from_planes(kd, vd)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    slots = pkv.slot_mapping_cache_write(torch.from_numpy(bt).cuda(), torch.from_numpy(qsl).cuda(),
                                         torch.from_numpy(nc).cuda(), dev16(key), dev16(val), cache,
                                         err_count=err)
    torch.cuda.synchronize()
    ref, werr = paging.slot_mapping(bt, qsl, nc, bs, num_tokens=T, num_blocks=nb)
    assert np.array_equal(slots.cpu().numpy(), ref)
    assert int(err.item()) == werr and (werr > 0 or R > 1000)
    # two tokens may not share a slot in one call; the random ids allow it, so
    # the oracle writes the first and the comparison skips later duplicates
    seen, keep = set(), np.full(T, -1, np.int64)
    for t, s_ in enumerate(ref):
        if s_ >= 0 and int(s_) not in seen:
            seen.add(int(s_))
            keep[t] = s_
    dup = np.array([t for t in range(T) if ref[t] >= 0 and keep[t] < 0], dtype=np.int64)
    kp, vp = paging.cache_write(kp0, vp0, key, val, keep, "bf16", "bf16")
    got_k, got_v = host_bits(kd), host_bits(vd)
    mask = np.ones(nb * bs, bool)
    mask[ref[dup]] = False                                                # slots written twice: racy
    np.testing.assert_array_equal(got_k.reshape(nb * bs, -1)[mask], kp.reshape(nb * bs, -1)[mask])
    np.testing.assert_array_equal(got_v.reshape(nb * bs, -1)[mask], vp.reshape(nb * bs, -1)[mask])


def test_fused_equals_the_two_calls_bit_for_bit():
    say("fused vs two calls")
    w = workloads.llama8b_decode()
    d1, d2 = w.device(), w.device()
    s1 = pkv.slot_mapping(d1.block_table, d1.query_start_loc, d1.num_computed, w.block_size, w.num_blocks)
    pkv.cache_write(d1.new_k, d1.new_v, s1, d1.cache)
    s2 = pkv.slot_mapping_cache_write(d2.block_table, d2.query_start_loc, d2.num_computed, d2.new_k,
                                      d2.new_v, d2.cache)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(d1.cache.k.view(torch.int16), d2.cache.k.view(torch.int16))
    assert torch.equal(d1.cache.v.view(torch.int16), d2.cache.v.view(torch.int16))
