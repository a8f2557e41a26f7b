"""Softmax attention over a paged KV cache, in float64 (oracle, test-only).

What is computed (the plain definition; no tiling, no online softmax):

For request r with sequence length L (the tokens already cached plus this
step's tokens) and q_len query tokens, query i sits at position
p = L - q_len + i.  It attends keys j with
    j <= p                      (causal; without it, j <= L - 1)
    j >= p - W + 1              (sliding window of W keys, W > 0)
and, for query head h, uses KV head h // G where G = Hq / Hkv (grouped-query
attention: consecutive query heads share one KV head).
    z_j = scale * <q_h, k_j>,   out = sum_j softmax(z)_j v_j.
K and V are gathered in logical order by following the request's block table
row; fp8 and int4 caches are dequantised exactly (code value times the per-tensor
scale), bf16 widened exactly.

Sources: attention reads past K/V through the block table, never assuming one
contiguous tensor (Engine-to-Worker card, § Slot mapping은 왜 필요한가 and
§ Forward 직전의 metadata); blocks sit at arbitrary physical places and the
softmax normaliser needs all of them (PageAttention blog, § Understanding
PageAttention Memory Optimization and § Handling Softmax Across Blocks, whose
formula did not survive -- the textbook softmax is used); kernels tile and use
an online softmax (Worker-Side KV Init (zh), § Worker与ModelRunner的协作),
which is a reordering of the same sum; GQA and a 4096-token sliding window
(Worker-Side KV Init, § Hybrid Attention Mechanisms).

Readings where the pages are silent:

* softmax scale is an explicit argument (1/sqrt(D) by convention);
* the window holds the W most recent positions including the query's own,
  i.e. keys p-W+1 .. p;
* "context length" includes this step's token(s), which are written to the
  cache before attention reads it;
* every query sees at least one key (L >= q_len >= 1).

``merge_partials`` is the log-sum-exp merge of partial softmax results over
disjoint key sets (the split-K combine); partials use base-2 exponents:
    acc = sum_j 2**(s_j - m) v_j,  l = sum_j 2**(s_j - m)
for any reference value m; out = sum_s 2**(m_s-M) acc_s / sum_s 2**(m_s-M) l_s.
"""

import numpy as np

from . import bf16 as _bf16
from . import paging as _paging


def q_to_f64(q, q_dtype):
    if q_dtype == "bf16":
        return _bf16.to_f64(q)
    if q_dtype == "f32":
        return np.asarray(q, dtype=np.float32).astype(np.float64)
    raise ValueError(q_dtype)


def key_range(L, q_len, i, causal, window):
    """Inclusive key positions [lo, hi] seen by query i of a request."""
    p = L - q_len + i
    hi = p if causal else L - 1
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, hi


def softmax_attend(qrow, keys, values, scale):
    """One query vector against rows of keys/values (all float64)."""
    z = scale * (keys @ qrow)
    z = z - z.max()
    w = np.exp(z)
    return (w[:, None] * values).sum(axis=0) / w.sum()


def paged_attention(q, q_dtype, k_plane, v_plane, cache_dtype, block_table,
                    seq_lens, query_start_loc, scale, causal=True,
                    sliding_window=0, k_scale=1.0, v_scale=1.0):
    """Attention of every query token of a step against the paged cache.

    q: [T, Hq, D]; planes: [num_blocks, bs, Hkv, D] storage bits;
    block_table: [R, max_blocks]; seq_lens, query_start_loc as in the ABI.
    Returns float64 [T, Hq, D]; rows of tokens outside every request are NaN.
    """
    qf = q_to_f64(q, q_dtype)
    T, Hq, D = qf.shape
    bs = k_plane.shape[1]
    Hkv = k_plane.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    bt = np.asarray(block_table)
    qsl = np.asarray(query_start_loc)
    out = np.full((T, Hq, D), np.nan)
    for r in range(len(seq_lens)):
        L = int(seq_lens[r])
        t0, t1 = int(qsl[r]), int(qsl[r + 1])
        q_len = t1 - t0
        if q_len == 0:
            continue
        if q_len > L:
            raise ValueError("request %d has more queries than tokens" % r)
        lo_all = key_range(L, q_len, 0, causal, sliding_window)[0]
        pos = np.arange(lo_all, L)
        kr = _paging.gather_positions(k_plane, bt[r], pos, bs)
        vr = _paging.gather_positions(v_plane, bt[r], pos, bs)
        kr = _paging.plane_to_f64(kr, cache_dtype, k_scale)
        vr = _paging.plane_to_f64(vr, cache_dtype, v_scale)
        for i in range(q_len):
            lo, hi = key_range(L, q_len, i, causal, sliding_window)
            a, b = lo - lo_all, hi - lo_all + 1
            for h in range(Hq):
                kvh = h // G
                out[t0 + i, h] = softmax_attend(qf[t0 + i, h], kr[a:b, kvh],
                                                vr[a:b, kvh], scale)
    return out


def paged_decode(q, q_dtype, k_plane, v_plane, cache_dtype, block_table,
                 seq_lens, scale, sliding_window=0, k_scale=1.0, v_scale=1.0):
    """Decode form: one query token per sequence, q is [B, Hq, D]."""
    B = len(seq_lens)
    qsl = np.arange(B + 1)
    return paged_attention(q, q_dtype, k_plane, v_plane, cache_dtype,
                           block_table, seq_lens, qsl, scale, causal=True,
                           sliding_window=sliding_window, k_scale=k_scale,
                           v_scale=v_scale)


def partial_softmax(qrow, keys, values, scale, m=None):
    """Base-2 partial (acc, m, l) of one query over a key subset.

    m defaults to the subset's largest scaled score in log2 units.
    """
    s = (scale * (keys @ qrow)) / np.log(2.0)
    if m is None:
        m = s.max()
    w = np.exp2(s - m)
    return (w[:, None] * values).sum(axis=0), m, w.sum()


def merge_partials(acc, m, l):
    """Log-sum-exp merge: acc [S, D], m [S], l [S] -> out [D]."""
    acc = np.asarray(acc, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    M = m.max()
    w = np.exp2(m - M)
    return (w[:, None] * acc).sum(axis=0) / (w * l).sum()
