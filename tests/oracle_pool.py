"""CPU worker processes that run the oracle on the full-size workloads (test
plumbing only).

The full-size parity tests compare every output row with the fp64 oracle.
One query of the hybrid workload costs the oracle a few milliseconds, so a
layer of 2144 tokens x 32 heads takes minutes on one core; the rows are
independent, so they are farmed out to worker processes.

The workers are fresh interpreters (the "spawn" start method), started by
``start()`` before the test process touches the GPU (tests/conftest.py does
this after collection when a selected test asks for the pool), so no worker
inherits the GPU state.  Each task carries just the blocks its request
references, renumbered from 0, and calls ``oracle.attention.paged_attention``
unchanged.  If the pool could not be started before the GPU was initialised,
tasks run in threads of the test process instead (slower, same results).
"""

import atexit
import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

_POOL = None


def available_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, n)


def _limit_blas():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _warm(_):
    import oracle.attention  # noqa: F401
    return os.getpid()


def start(workers=None):
    """Start the worker processes (idempotent).  Must run before the GPU is
    initialised in this process."""
    global _POOL
    if _POOL is not None:
        return _POOL
    workers = workers or min(8, available_cores())
    ctx = mp.get_context("spawn")
    _POOL = cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_limit_blas)
    list(_POOL.map(_warm, range(workers)))    # start every worker now
    atexit.register(_POOL.shutdown)
    return _POOL


def executor():
    if _POOL is not None:
        return _POOL
    return cf.ThreadPoolExecutor(max_workers=min(8, available_cores()))


def _task(args):
    from oracle import attention
    (q, q_dtype, k, v, cache_dtype, table, seq_lens, qsl, scale, causal, window, k_scale,
     v_scale) = args
    return attention.paged_attention(q, q_dtype, k, v, cache_dtype, table, seq_lens, qsl, scale,
                                     causal=causal, sliding_window=window, k_scale=k_scale,
                                     v_scale=v_scale)


def paged_attention_all_rows(q_bits, q_dtype, fetch_blocks, cache_dtype, block_table, seq_lens,
                             query_start_loc, scale, causal=True, window=0, k_scale=1.0,
                             v_scale=1.0, query_chunk=64):
    """oracle.attention.paged_attention over every request, in the pool.

    fetch_blocks(r, lo, L) -> (k, v, first, bs): host arrays (storage bits,
    [n, bs, Hkv, ...]) of the blocks of request r that hold positions lo ..
    L - 1, the first of them logical block `first`.  Causal requests with many
    queries are cut into sub-requests of at most `query_chunk` queries (query
    i of a request of length L with q_len queries sits at L - q_len + i, so
    queries i0 .. i1 - 1 are exactly a request of length L - q_len + i1 with
    i1 - i0 queries).  Returns float64 [T, Hq, D].
    """
    q_bits = np.asarray(q_bits)
    bt = np.asarray(block_table)
    qsl = np.asarray(query_start_loc)
    T, Hq, D = q_bits.shape
    futures = []
    ex = executor()
    for r in range(len(seq_lens)):
        L = int(seq_lens[r])
        t0, t1 = int(qsl[r]), int(qsl[r + 1])
        ql = t1 - t0
        if ql == 0:
            continue
        # blocks from the first key any query sees to the last
        p0 = L - ql
        lo = max(0, p0 - window + 1) if window > 0 else 0
        futures_r = []
        cuts = range(0, ql, query_chunk) if causal else range(0, ql, ql)
        for i0 in cuts:
            i1 = min(ql, i0 + query_chunk) if causal else ql
            Lsub = p0 + i1 if causal else L
            futures_r.append((i0, i1, Lsub))
        # one fetch per request: blocks lo // bs .. (L - 1) // bs
        k_blk, v_blk, first, _ = fetch_blocks(r, lo, L)
        n = k_blk.shape[0]
        table = np.full((1, first + n), -1, dtype=np.int32)
        table[0, first:] = np.arange(n, dtype=np.int32)
        for i0, i1, Lsub in futures_r:
            args = (q_bits[t0 + i0:t0 + i1], q_dtype, k_blk, v_blk, cache_dtype, table,
                    np.array([Lsub], np.int32), np.array([0, i1 - i0], np.int32), scale, causal,
                    window, k_scale, v_scale)
            futures.append((t0 + i0, t0 + i1, ex.submit(_task, args)))
    out = np.full((T, Hq, D), np.nan)
    for a, b, f in futures:
        out[a:b] = f.result()
    return out


def host_block_fetcher(k_plane, v_plane, block_table, block_size):
    """fetch_blocks over host planes (storage bits)."""
    bt = np.asarray(block_table)

    def fetch(r, lo, L):
        first = lo // block_size
        last = (L - 1) // block_size
        ids = bt[r, first:last + 1].astype(np.int64)
        assert (ids >= 0).all(), "a visible block is unmapped"
        return k_plane[ids], v_plane[ids], first, block_size
    return fetch
