"""Pins for the oracle's paged attention (CPU only).

The oracle follows block tables and applies the textbook softmax; these tests
tie it to things it does not compute itself: torch's scaled-dot-product
attention on contiguous tensors (a library routine for the special case of an
unpaged cache), closed forms, hand-computable examples and invariances.
"""

import numpy as np
import pytest
import torch

from oracle import attention, paging


def _paginate(kc, vc, table, bs, nb, fill=np.nan):
    """Lay contiguous [L, Hkv, D] rows out into planes by a block table."""
    L, H, D = kc.shape
    kp = np.full((nb, bs, H, D), fill)
    vp = np.full((nb, bs, H, D), fill)
    for j in range(L):
        kp[table[j // bs], j % bs] = kc[j]
        vp[table[j // bs], j % bs] = vc[j]
    return kp, vp


def _case(rng, L_list, qlen_list, Hq, Hkv, D, bs, nb):
    R = len(L_list)
    kcs, vcs = [], []
    tables = []
    perm = rng.permutation(nb)
    k = 0
    maxb = max(-(-L // bs) for L in L_list)
    bt = np.full((R, maxb), -1, dtype=np.int32)
    for r, L in enumerate(L_list):
        n = -(-L // bs)
        bt[r, :n] = perm[k:k + n]
        k += n
        # float32-representable values: the oracle reads 'f32' planes
        kcs.append(rng.standard_normal((L, Hkv, D)).astype(np.float32).astype(np.float64))
        vcs.append(rng.standard_normal((L, Hkv, D)).astype(np.float32).astype(np.float64))
    kp = np.full((nb, bs, Hkv, D), np.nan)
    vp = np.full((nb, bs, Hkv, D), np.nan)
    for r in range(R):
        a, b = _paginate(kcs[r], vcs[r], bt[r], bs, nb)
        used = ~np.isnan(a)
        kp[used] = a[used]
        vp[used] = b[used]
    qsl = np.concatenate([[0], np.cumsum(qlen_list)]).astype(np.int64)
    q = rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32).astype(np.float64)
    return q, kp, vp, bt, qsl, kcs, vcs


def _sdpa(q, kc, vc, mask, scale, G):
    """torch SDPA in float64 on contiguous K/V (GQA by repeating KV heads)."""
    qt = torch.from_numpy(q).permute(1, 0, 2)                    # [Hq, ql, D]
    kt = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(G, 0)
    m = torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("seed", range(8))
def test_matches_torch_sdpa_on_contiguous_kv(seed):
    rng = np.random.default_rng(200 + seed)
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4]))
    Hq = Hkv * G
    D = int(rng.choice([4, 8]))
    bs = int(rng.choice([4, 8, 16]))
    R = int(rng.integers(1, 4))
    L_list = [int(x) for x in rng.integers(1, 70, size=R)]
    qlen = [int(rng.integers(1, L + 1)) for L in L_list]
    causal = bool(rng.integers(0, 2))
    W = int(rng.choice([0, 0, 1, 3, 17, 200]))
    scale = float(rng.uniform(0.2, 1.5))
    q, kp, vp, bt, qsl, kcs, vcs = _case(rng, L_list, qlen, Hq, Hkv, D, bs, 128)
    got = attention.paged_attention(q, "f32", kp.astype(np.float32), vp.astype(np.float32),
                                    "f32", bt, L_list, qsl, scale, causal=causal,
                                    sliding_window=W)
    for r, L in enumerate(L_list):
        ql = qlen[r]
        mask = np.zeros((ql, L), dtype=bool)
        for i in range(ql):
            p = L - ql + i
            for j in range(L):
                ok = (j <= p) if causal else True
                if W > 0:
                    ok = ok and j > p - W
                mask[i, j] = ok
        ref = _sdpa(q[qsl[r]:qsl[r + 1]], kcs[r], vcs[r], mask, scale, G)
        np.testing.assert_allclose(got[qsl[r]:qsl[r + 1]], ref, rtol=0, atol=1e-12)


def test_hand_computed_three_key_example():
    # scores 0, ln 2, ln 3 -> weights 1:2:3; values 6, 0, 12 -> 42 / 6 = 7
    # (keys are stored as float32, so ln 2 and ln 3 carry float32 rounding)
    kc = np.array([[[0.0]], [[np.log(2.0)]], [[np.log(3.0)]]])
    vc = np.array([[[6.0]], [[0.0]], [[12.0]]])
    bt = np.array([[5, 2]], dtype=np.int32)
    kp, vp = _paginate(kc, vc, bt[0], 2, 8)
    q = np.array([[[1.0]]])
    out = attention.paged_attention(q, "f32", kp, vp, "f32", bt, [3], [0, 1], 1.0)
    assert abs(out[0, 0, 0] - 7.0) < 1e-6


def test_window_of_one_returns_own_value_and_window_of_two_is_a_sigmoid_mix():
    rng = np.random.default_rng(11)
    L, D = 9, 4
    q, kp, vp, bt, qsl, kcs, vcs = _case(rng, [L], [3], 1, 1, D, 4, 16)
    out1 = attention.paged_attention(q, "f32", kp, vp, "f32", bt, [L], qsl, 0.7,
                                     causal=True, sliding_window=1)
    for i in range(3):
        np.testing.assert_allclose(out1[i, 0], vcs[0][L - 3 + i, 0], rtol=0, atol=1e-15)
    out2 = attention.paged_attention(q, "f32", kp, vp, "f32", bt, [L], qsl, 0.7,
                                     causal=True, sliding_window=2)
    for i in range(3):
        p = L - 3 + i
        z_prev = 0.7 * q[i, 0] @ kcs[0][p - 1, 0]  # all float32-representable
        z_self = 0.7 * q[i, 0] @ kcs[0][p, 0]
        a = 1.0 / (1.0 + np.exp(z_prev - z_self))
        want = a * vcs[0][p, 0] + (1 - a) * vcs[0][p - 1, 0]
        np.testing.assert_allclose(out2[i, 0], want, rtol=0, atol=1e-12)


def test_equal_keys_give_the_mean_of_visible_values():
    rng = np.random.default_rng(12)
    L, D, bs = 23, 8, 4
    kc = np.tile(rng.standard_normal((1, 1, D)), (L, 1, 1)).astype(np.float32).astype(np.float64)
    vc = rng.standard_normal((L, 1, D)).astype(np.float32).astype(np.float64)
    bt = np.array([rng.permutation(12)[:6]], dtype=np.int32)
    kp, vp = _paginate(kc, vc, bt[0], bs, 12)
    q = rng.standard_normal((1, 2, D))  # two query heads share the KV head
    out = attention.paged_decode(q, "f32", kp, vp, "f32", bt, [L], 0.3)
    np.testing.assert_allclose(out[0, 0], vc[:, 0].mean(axis=0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[0, 1], vc[:, 0].mean(axis=0), rtol=0, atol=1e-13)
    outw = attention.paged_decode(q, "f32", kp, vp, "f32", bt, [L], 0.3, sliding_window=5)
    np.testing.assert_allclose(outw[0, 0], vc[L - 5:, 0].mean(axis=0), rtol=0, atol=1e-13)


def test_window_at_least_length_equals_full_attention():
    rng = np.random.default_rng(13)
    q, kp, vp, bt, qsl, _, _ = _case(rng, [30, 7], [4, 7], 4, 2, 8, 8, 32)
    full = attention.paged_attention(q, "f32", kp, vp, "f32", bt, [30, 7], qsl, 0.5)
    wide = attention.paged_attention(q, "f32", kp, vp, "f32", bt, [30, 7], qsl, 0.5,
                                     sliding_window=30)
    np.testing.assert_array_equal(full, wide)


def test_physical_placement_does_not_change_the_result():
    rng = np.random.default_rng(14)
    L_list = [37, 5, 64]
    Hq, Hkv, D, bs, nb = 4, 2, 8, 8, 48
    kcs = [rng.standard_normal((L, Hkv, D)) for L in L_list]
    vcs = [rng.standard_normal((L, Hkv, D)) for L in L_list]
    q = rng.standard_normal((3, Hq, D))
    outs = []
    for trial in range(3):
        perm = np.random.default_rng(trial).permutation(nb)
        bt = np.full((3, 8), -1, dtype=np.int32)
        kp = np.full((nb, bs, Hkv, D), np.nan)
        vp = np.full((nb, bs, Hkv, D), np.nan)
        k = 0
        for r, L in enumerate(L_list):
            n = -(-L // bs)
            bt[r, :n] = perm[k:k + n]
            k += n
            for j in range(L):
                kp[bt[r, j // bs], j % bs] = kcs[r][j]
                vp[bt[r, j // bs], j % bs] = vcs[r][j]
        outs.append(attention.paged_decode(q, "f32", kp, vp, "f32", bt, L_list, 0.35))
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_chunk_of_one_query_equals_decode():
    rng = np.random.default_rng(15)
    q, kp, vp, bt, qsl, _, _ = _case(rng, [19, 40, 3], [1, 1, 1], 2, 1, 8, 4, 64)
    a = attention.paged_attention(q, "f32", kp, vp, "f32", bt, [19, 40, 3], qsl, 0.4)
    b = attention.paged_decode(q, "f32", kp, vp, "f32", bt, [19, 40, 3], 0.4)
    np.testing.assert_array_equal(a, b)


def test_unused_slots_are_never_read():
    # every unused cell is NaN in _case; the outputs must be finite
    rng = np.random.default_rng(16)
    q, kp, vp, bt, qsl, _, _ = _case(rng, [13, 29], [13, 2], 2, 2, 4, 8, 16)
    out = attention.paged_attention(q, "f32", kp, vp, "f32", bt, [13, 29], qsl, 0.5)
    assert np.isfinite(out).all()


def test_split_and_merge_equals_the_whole_softmax():
    rng = np.random.default_rng(17)
    D, L = 16, 300
    keys = rng.standard_normal((L, D))
    vals = rng.standard_normal((L, D))
    qrow = rng.standard_normal(D) * 2
    whole = attention.softmax_attend(qrow, keys, vals, 0.25)
    for S in (1, 2, 7, 300):
        cuts = np.sort(rng.choice(np.arange(1, L), size=S - 1, replace=False)) if S > 1 else []
        parts = np.split(np.arange(L), cuts)
        accs, ms, ls = [], [], []
        for idx in parts:
            # arbitrary (non-maximal) reference values are allowed too
            ref_m = None if len(accs) % 2 == 0 else 3.0
            a, m, l = attention.partial_softmax(qrow, keys[idx], vals[idx], 0.25, m=ref_m)
            accs.append(a), ms.append(m), ls.append(l)
        np.testing.assert_allclose(attention.merge_partials(accs, ms, ls), whole,
                                   rtol=0, atol=1e-12)


def test_bf16_and_fp8_caches_are_widened_exactly():
    from oracle import bf16, e4m3
    rng = np.random.default_rng(18)
    L, D, bs = 10, 8, 4
    kc = rng.standard_normal((L, 1, D)).astype(np.float32)
    vc = rng.standard_normal((L, 1, D)).astype(np.float32)
    bt = np.array([[3, 0, 7]], dtype=np.int32)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    # bf16: oracle on bits == oracle on the exactly widened float planes
    kb, vb = bf16.from_f32(kc), bf16.from_f32(vc)
    kpb, vpb = _paginate(kb.astype(np.float64), vb.astype(np.float64), bt[0], bs, 8, fill=0)
    out_b = attention.paged_decode(bf16.from_f32(q), "bf16", kpb.astype(np.uint16),
                                   vpb.astype(np.uint16), "bf16", bt, [L], 0.3)
    kf, vf = _paginate(bf16.to_f64(kb), bf16.to_f64(vb), bt[0], bs, 8)
    out_f = attention.paged_decode(bf16.to_f64(bf16.from_f32(q)).astype(np.float32), "f32",
                                   kf, vf, "f32", bt, [L], 0.3)
    np.testing.assert_array_equal(out_b, out_f)
    # fp8: codes times scale
    ks, vs = np.float32(0.01), np.float32(0.02)
    kq, vq = e4m3.quantize(kc, ks), e4m3.quantize(vc, vs)
    kp8, vp8 = _paginate(kq.astype(np.float64), vq.astype(np.float64), bt[0], bs, 8, fill=0)
    out8 = attention.paged_decode(q, "f32", kp8.astype(np.uint8), vp8.astype(np.uint8), "fp8",
                                  bt, [L], 0.3, k_scale=ks, v_scale=vs)
    kd, vd = _paginate(e4m3.decode(kq) * np.float64(ks), e4m3.decode(vq) * np.float64(vs),
                       bt[0], bs, 8)
    outd = attention.paged_decode(q, "f32", kd, vd, "f64", bt, [L], 0.3)
    np.testing.assert_array_equal(out8, outd)
