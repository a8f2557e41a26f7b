"""GPU parity: slot mapping, cache write and the FP8 codec (bit-exact)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_mapping_amd as pkv
from paged_kv_cache_mapping_amd import workloads
from oracle import bf16, e4m3, paging

from helpers import gpu_or_skip, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gpu_or_skip()


# ------------------------------------------------------------------ codec

@pytest.mark.parametrize("scale", [1.0, 0.37, 0.0069196428])
def test_fp8_quantize_all_bf16_patterns(scale):
    say("fp8 quantize, all bf16 patterns, scale", scale)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = pkv.fp8_quantize(x, scale).cpu().numpy()
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    want = e4m3.quantize(vals, scale)
    nan = np.isnan(vals)
    assert (got[~nan] == want[~nan]).all()
    assert ((got[nan] & 0x7F) == 0x7F).all() and (got[nan] == want[nan]).all()


def test_fp8_quantize_f32_edge_values():
    say("fp8 quantize f32 edges")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.uniform(-5, 3, 100000),
                        [0.0, -0.0, 448.0, 449.0, 464.0, 480.0, 1e30, -1e30, np.inf, -np.inf,
                         2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 17.0, 19.0,
                         2.0 ** -130]]).astype(np.float32)
    got = pkv.fp8_quantize(torch.from_numpy(x).cuda(), 0.5).cpu().numpy()
    assert (got == e4m3.quantize(x, 0.5)).all()


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.3])
def test_fp8_dequantize_all_codes_f32(scale):
    say("fp8 dequantize f32, scale", scale)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    got = pkv.fp8_dequantize(codes, scale).cpu().numpy()
    want = (e4m3.decode(np.arange(256)) * np.float64(np.float32(scale))).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert (got[~nan] == want[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(want[~nan])).all()


def test_fp8_dequantize_all_codes_bf16_exact():
    say("fp8 dequantize bf16")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    got = pkv.fp8_dequantize(codes, 1.0, out_dtype=torch.bfloat16).cpu().to(torch.float64).numpy()
    want = e4m3.decode(np.arange(256))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert (got[~nan] == want[~nan]).all()


# ------------------------------------------------------------------ slot mapping

def _slot_case(w_tables, qsl, nc, bs, nb, num_tokens=None):
    bt = torch.from_numpy(w_tables).cuda()
    q = torch.from_numpy(np.asarray(qsl, np.int32)).cuda()
    n = torch.from_numpy(np.asarray(nc, np.int32)).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = pkv.slot_mapping(bt, q, n, bs, nb, num_tokens=num_tokens, err_count=err)
    torch.cuda.synchronize()
    want, werr = paging.slot_mapping(w_tables, qsl, nc, bs, num_tokens=num_tokens, num_blocks=nb)
    return got.cpu().numpy(), int(err.item()), want, werr


@pytest.mark.parametrize("name", ["tiny", "llama8b", "llama70b", "fp8"])
def test_slot_mapping_decode_workloads(name):
    say("slot mapping", name)
    w = workloads.ALL[name]()
    got, err, want, werr = _slot_case(w.block_table, w.query_start_loc, w.num_computed,
                                      w.block_size, w.num_blocks)
    assert werr == 0 and err == 0
    assert np.array_equal(got, want)


def test_slot_mapping_hybrid_both_groups():
    say("slot mapping hybrid")
    w = workloads.hybrid_chunked()
    for g in range(2):
        got, err, want, werr = _slot_case(w.tables[g], w.query_start_loc, w.num_computed,
                                          w.block_size, w.num_blocks)
        assert werr == 0 and err == 0
        assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(4))
def test_slot_mapping_random_with_errors_padding_and_empty_requests(seed):
    say("slot mapping random", seed)
    rng = np.random.default_rng(300 + seed)
    R, bs, nb = 37, int(rng.choice([4, 8, 16, 32])), 500
    ql = rng.integers(0, 40, size=R)
    ql[rng.integers(0, R, 5)] = 0
    nc = rng.integers(0, 300, size=R)
    width = int(np.max(-(-(nc + ql) // bs))) + 1
    bt = rng.integers(-1, nb + 20, size=(R, width)).astype(np.int32)   # some invalid ids
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    got, err, want, werr = _slot_case(bt, qsl, nc.astype(np.int32), bs, nb,
                                      num_tokens=int(qsl[-1]) + 7)
    assert np.array_equal(got, want)
    assert err == werr and werr > 0


# ------------------------------------------------------------------ cache write

def _compare_planes(cache, kp, vp):
    assert host_bits(cache.k).tobytes() == np.ascontiguousarray(kp).tobytes()
    assert host_bits(cache.v).tobytes() == np.ascontiguousarray(vp).tobytes()


@pytest.mark.parametrize("name,src", [("tiny", "f32"), ("llama8b", "bf16"), ("fp8", "bf16")])
def test_cache_write_workloads_bit_exact(name, src):
    say("cache write", name)
    w = workloads.ALL[name]()
    d = w.device()
    slots = pkv.slot_mapping(d.block_table, d.query_start_loc, d.num_computed, w.block_size,
                             w.num_blocks)
    pkv.cache_write(d.new_k, d.new_v, slots, d.cache)
    torch.cuda.synchronize()
    ref_slots, _ = paging.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, w.block_size)
    kp, vp = paging.cache_write(w.k_plane, w.v_plane, w.new_k, w.new_v, ref_slots, src,
                                w.cache_dtype, w.k_scale, w.v_scale)
    _compare_planes(d.cache, kp, vp)


@pytest.mark.parametrize("src,dst,D", [("f32", "bf16", 128), ("f32", "fp8", 64), ("bf16", "fp8", 8),
                                       ("bf16", "bf16", 8), ("f32", "f32", 16), ("bf16", "bf16", 256)])
def test_cache_write_conversions_and_strided_sources(src, dst, D):
    say("cache write", src, dst, D)
    rng = np.random.default_rng(11)
    nb, bs, H, T = 40, 8, 3, 50
    k_scale, v_scale = 0.02, 0.03
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
    from paged_kv_cache_mapping_amd.workloads import nan_plane, bf16_bits
    kp0 = nan_plane((nb, bs, H, D), dst)
    vp0 = nan_plane((nb, bs, H, D), dst)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[[3, 17]] = -1
    slots[20] = nb * bs + 5          # out of range: skipped
    x = (rng.standard_normal((T, H + 1, D)) * 4).astype(np.float32)   # one extra head: strided
    y = (rng.standard_normal((T, H + 1, D)) * 4).astype(np.float32)
    xs = x if src == "f32" else bf16_bits(x)
    ys = y if src == "f32" else bf16_bits(y)

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a if a.dtype != np.uint16 else a.view(np.int16)))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).cuda()
    key = dev(xs)[:, :H]
    val = dev(ys)[:, :H]
    kd = torch.from_numpy(kp0 if dst != "bf16" else kp0.view(np.int16)).cuda()
    vd = torch.from_numpy(vp0 if dst != "bf16" else vp0.view(np.int16)).cuda()
    if dst == "bf16":
        kd, vd = kd.view(torch.bfloat16), vd.view(torch.bfloat16)
    cache = pkv.CacheView.from_planes(kd, vd, k_scale, v_scale)
    pkv.cache_write(key, val, torch.from_numpy(slots).cuda(), cache)
    torch.cuda.synchronize()
    kp, vp = paging.cache_write(kp0, vp0, xs[:, :H], ys[:, :H], np.where(slots < nb * bs, slots, -1),
                                src, dst, k_scale, v_scale)
    _compare_planes(cache, kp, vp)


def _fp8_cache_write_case(x, y, src, k_scale, v_scale):
    """Write rows x (K) and y (V), [T, 1, D], into an fp8 cache through
    pkv.cache_write (slot t = token t) and compare both planes with the
    oracle's write, byte for byte."""
    from paged_kv_cache_mapping_amd.workloads import nan_plane
    T, _, D = x.shape
    bs = 16
    nb = (T + bs - 1) // bs
    kp0 = nan_plane((nb, bs, 1, D), "fp8")
    vp0 = nan_plane((nb, bs, 1, D), "fp8")
    slots = np.arange(T, dtype=np.int64)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    cache = pkv.CacheView.from_planes(torch.from_numpy(kp0).cuda(), torch.from_numpy(vp0).cuda(),
                                      k_scale, v_scale)
    pkv.cache_write(dev(x), dev(y), torch.from_numpy(slots).cuda(), cache)
    torch.cuda.synchronize()
    kp, vp = paging.cache_write(kp0, vp0, x, y, slots, src, "fp8", k_scale, v_scale)
    _compare_planes(cache, kp, vp)


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.37, 2.5), (0.0069196428, 0.011)])
def test_fp8_cache_write_all_bf16_patterns(scales):
    """Every bfloat16 bit pattern through the cache write into an fp8 cache:
    K in bit order (the NaN patterns fill whole chunks), V in a seeded
    permutation (NaNs scattered among finite values of every size)."""
    say("fp8 cache write, all bf16 patterns, scales", scales)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    perm = np.random.default_rng(5).permutation(65536)
    x = bits.reshape(512, 1, 128)
    y = np.ascontiguousarray(bits[perm]).reshape(512, 1, 128)
    _fp8_cache_write_case(x, y, "bf16", *scales)


def test_fp8_cache_write_f32_edge_values():
    """f32 sources: magnitudes over eight decades, the saturation edge
    (448, 464, 480, infinities), ties at the subnormal and normal spacing,
    values below the smallest code, and NaNs in a few rows."""
    say("fp8 cache write f32 edges")
    rng = np.random.default_rng(9)
    n = 64 * 128
    edges = np.array([0.0, -0.0, 448.0, 449.0, 464.0, 465.0, 480.0, -464.0, 1e30, -1e30, np.inf,
                      -np.inf, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 2.0 ** -6,
                      2.0 ** -6 - 2.0 ** -10, 1.0625, 1.1875, 17.0, 19.0, 2.0 ** -130, -2.0 ** -11],
                     np.float32)
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 3, n)).astype(np.float32)
    x[:len(edges)] = edges
    y = -x[::-1].copy()
    x[5000] = np.nan
    y[77] = -np.nan
    _fp8_cache_write_case(x.reshape(64, 1, 128), y.reshape(64, 1, 128), "f32", 0.5, 0.25)
