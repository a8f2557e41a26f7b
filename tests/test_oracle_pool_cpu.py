"""The test plumbing that runs the oracle over every row in worker processes
gives exactly the oracle's own result: cutting a causal request's queries
into sub-requests (queries i0 .. i1 - 1 of a request of length L with q_len
queries are a request of length L - q_len + i1 with i1 - i0 queries) and
renumbering the blocks each task carries changes nothing."""

import numpy as np
import pytest

import oracle_pool
from oracle import attention
from paged_kv_cache_mapping_amd import workloads


@pytest.mark.parametrize("window,causal", [(0, True), (40, True), (0, False), (25, False)])
def test_all_rows_equal_the_oracle(window, causal):
    rng = np.random.default_rng(5 + window)
    bs, Hkv, Hq, D = 16, 2, 4, 32
    L = np.array([130, 1, 77, 200, 33], np.int32)
    ql = np.array([70, 1, 1, 150, 33], np.int32)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    nb = int(sum(-(-int(x) // bs) for x in L)) + 5
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(L), max(-(-int(x) // bs) for x in L)), -1, np.int32)
    k = 0
    for r, x in enumerate(L):
        n = -(-int(x) // bs)
        bt[r, :n] = perm[k:k + n]
        k += n
    kp = workloads.bf16_bits(rng.standard_normal((nb, bs, Hkv, D), dtype=np.float32))
    vp = workloads.bf16_bits(rng.standard_normal((nb, bs, Hkv, D), dtype=np.float32))
    q = workloads.bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, D), dtype=np.float32))
    ref = attention.paged_attention(q, "bf16", kp, vp, "bf16", bt, L, qsl, 0.2, causal=causal,
                                    sliding_window=window)
    got = oracle_pool.paged_attention_all_rows(
        q, "bf16", oracle_pool.host_block_fetcher(kp, vp, bt, bs), "bf16", bt, L, qsl, 0.2,
        causal=causal, window=window, query_chunk=32)
    np.testing.assert_array_equal(got, ref)
