"""GPU parity: block copies for prefix sharing, and decode over tables whose
leading entries are shared (Chinese worker-side page, § PagedAttention与Block
管理: a common prompt's blocks are shared by reference; copy-on-write before a
private write is this build's reading)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from paged_kv_cache_mapping_amd import kv_cache
from paged_kv_cache_mapping_amd.workloads import bf16_bits
from oracle import attention, paging

from helpers import gpu_or_skip, host_bits, max_err, out_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_copy_blocks_bit_exact(dtype):
    say("copy_blocks", dtype)
    rng = np.random.default_rng(40)
    nb, bs, H, D = 600, 16, 8, 128
    npdt = {"bf16": np.uint16, "fp8": np.uint8, "f32": np.uint32}[dtype]
    kp = rng.integers(0, np.iinfo(npdt).max, size=(nb, bs, H, D), dtype=npdt)
    vp = rng.integers(0, np.iinfo(npdt).max, size=(nb, bs, H, D), dtype=npdt)
    perm = rng.permutation(nb)
    src = perm[:250].astype(np.int32)                  # sources and destinations disjoint
    dst = perm[250:500].astype(np.int32)
    src[7], dst[19], src[100] = -3, nb + 4, nb        # three bad pairs
    tdt = {"bf16": torch.bfloat16, "fp8": torch.uint8, "f32": torch.float32}[dtype]
    kd = torch.from_numpy(kp.view({"bf16": np.int16, "fp8": np.uint8, "f32": np.float32}[dtype])).cuda()
    vd = torch.from_numpy(vp.view({"bf16": np.int16, "fp8": np.uint8, "f32": np.float32}[dtype])).cuda()
    if dtype == "bf16":
        kd, vd = kd.view(tdt), vd.view(tdt)
    cache = pkv.CacheView.from_planes(kd, vd, 0.5, 0.25) if dtype == "fp8" else pkv.CacheView.from_planes(kd, vd)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.copy_blocks(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), cache, err_count=err)
    torch.cuda.synchronize()
    k_ref, v_ref, n_bad = paging.copy_blocks(kp, vp, src, dst)
    assert int(err.item()) == n_bad == 3
    np.testing.assert_array_equal(kd.cpu().view({"bf16": torch.int16, "fp8": torch.uint8,
                                                 "f32": torch.float32}[dtype]).numpy().view(npdt), k_ref)
    np.testing.assert_array_equal(vd.cpu().view({"bf16": torch.int16, "fp8": torch.uint8,
                                                 "f32": torch.float32}[dtype]).numpy().view(npdt), v_ref)


def _shared_prefix_run(share, prompt=200, R=16, seed=50):
    """Write a prompt once, fork it to R requests (or write it R times when
    share is False), append private suffixes (copy-on-write of the shared
    partial block), then one decode step over every request.  Returns the
    GPU output, the GPU planes, the oracle's planes and output, the tables."""
    bs, Hq, Hkv, D = 16, 32, 8, 128
    rng = np.random.default_rng(seed)
    nb = 512
    pool = kv_cache.BlockPool(nb, order=rng.permutation(nb))
    tabs = kv_cache.GroupBlockTables(pool, [0], bs)
    suffix = rng.integers(1, 41, size=R)
    kprompt = bf16_bits((rng.standard_normal((prompt, Hkv, D)) / np.sqrt(D)).astype(np.float32))
    vprompt = bf16_bits((rng.standard_normal((prompt, Hkv, D)) / np.sqrt(D)).astype(np.float32))
    ksuf = bf16_bits((rng.standard_normal((int(suffix.sum()), Hkv, D)) / np.sqrt(D)).astype(np.float32))
    vsuf = bf16_bits((rng.standard_normal((int(suffix.sum()), Hkv, D)) / np.sqrt(D)).astype(np.float32))
    q = bf16_bits((rng.standard_normal((R, Hq, D)) / np.sqrt(D)).astype(np.float32))

    nan = np.full((nb, bs, Hkv, D), 0x7FC0, np.uint16)
    kd, vd = _dev(nan.copy()), _dev(nan.copy())
    cache = pkv.CacheView.from_planes(kd, vd)
    k_or, v_or = nan.copy(), nan.copy()

    def write(reqs, starts, ks, vs):
        """One step: tokens of reqs at positions starts[i] .. (host tables)."""
        lens = [len(x) for x in ks]
        qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        nc = np.array(starts, np.int32)
        width = max(len(tabs.rows[0][r]) for r in reqs)
        bt = tabs.table(0, reqs, width)
        k_all, v_all = np.concatenate(ks), np.concatenate(vs)
        slots = pkv.slot_mapping(_dev(bt), _dev(qsl), _dev(nc), bs, nb)
        pkv.cache_write(_dev(k_all), _dev(v_all), slots, cache)
        s_ref, e = paging.slot_mapping(bt, qsl, nc, bs)
        assert e == 0
        return paging.cache_write(k_or, v_or, k_all, v_all, s_ref, "bf16", "bf16")

    reqs = list(range(R))
    for r in reqs:
        tabs.add_request(r)
    if share:
        assert tabs.prepare_write(0, 0, prompt) == []
        k_or, v_or = write([0], [0], [kprompt], [vprompt])
        for r in reqs[1:]:
            tabs.fork(0, r, prompt)
    else:
        for r in reqs:
            assert tabs.prepare_write(r, 0, prompt) == []
        k_or, v_or = write(reqs, [0] * R, [kprompt] * R, [vprompt] * R)
    pairs = []
    for r in reqs:
        pairs += tabs.prepare_write(r, prompt, prompt + int(suffix[r]))
    if share:
        assert len(pairs) == R - 1            # all but the last holder copy the partial block
    if pairs:
        src = np.array([p[0] for p in pairs], np.int32)
        dst = np.array([p[1] for p in pairs], np.int32)
        pkv.copy_blocks(_dev(src), _dev(dst), cache)
        k_or, v_or, e = paging.copy_blocks(k_or, v_or, src, dst)
        assert e == 0
    offs = np.concatenate([[0], np.cumsum(suffix)])
    k_or, v_or = write(reqs, [prompt] * R, [ksuf[offs[r]:offs[r + 1]] for r in reqs],
                       [vsuf[offs[r]:offs[r + 1]] for r in reqs])
    L = (prompt + suffix).astype(np.int32)
    bt = tabs.table(0, reqs)
    out = pkv.paged_attention_decode(_dev(q), cache, _dev(bt), _dev(L), int(L.max()), 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    ref = attention.paged_decode(q, "bf16", k_or, v_or, "bf16", bt, L, 1.0 / np.sqrt(D))
    return out, (host_bits(kd), host_bits(vd)), (k_or, v_or), ref, bt


def test_shared_prefix_decode_matches_oracle_and_private_copies():
    say("shared prefix decode")
    out, planes, planes_ref, ref, bt = _shared_prefix_run(True)
    np.testing.assert_array_equal(planes[0], planes_ref[0])
    np.testing.assert_array_equal(planes[1], planes_ref[1])
    assert max_err(out_f64(out), ref) <= 2e-3
    # the prompt's full blocks are one set of ids in every row
    assert (bt[:, :12] == bt[0, :12]).all()
    say("private prompt copies")
    out2, _, _, ref2, bt2 = _shared_prefix_run(False)
    assert not (bt2[:, :12] == bt2[0, :12]).all()
    np.testing.assert_array_equal(ref, ref2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
