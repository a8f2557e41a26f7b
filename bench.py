"""Benchmark of the paged KV-cache hot path on one MI355X.

One step = one decode step of the Llama-3-8B-shaped layer (bf16, 32 query /
8 KV heads, head_dim 128, block 16, 64 sequences with 128..2048 tokens):
slot mapping -> KV cache write -> paged decode attention (split phase +
combine).  Steps rotate over three KV pools that hold the same logical data
under different physical block permutations (3 GiB in total), so the 256 MB
last-level cache cannot serve the KV reads.

Prints one JSON line: the whole step's algorithmic HBM bytes per second
(value), the split kernel's roofline (HIP events around back-to-back launches of it),
bulk KV-write rates, the same steps recorded in a HIP graph and replayed
(graph_replay; `value` stays the eager step), and the CPU oracle on a bounded
sample of the same step.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench_profiles  # noqa: E402

HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E, AMD's published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
DATA_NOTE = {
    "llama8b": "synthetic (seeded N(0,1)/sqrt(128) bf16 K/V/Q; lengths uniform 128..2048)",
    "llama70b": "synthetic (seeded N(0,1)/sqrt(128) bf16 K/V/Q; 32 sequences of 4096 tokens)",
    "fp8": "synthetic (seeded N(0,1) K/V quantised to e4m3 with amax/448 scales, N(0,1) bf16 Q; "
           "lognormal lengths, median 1024, clipped to 16..32768)",
    "hybrid": "synthetic (seeded N(0,1)/sqrt(128) bf16; 96 decode requests 1k..16k + 4 prefill "
              "chunks of 512, full and sliding-window groups over shared tensors)",
    "prefix": "synthetic (seeded N(0,1)/sqrt(128) bf16; 100 requests sharing the blocks of one "
              "2000-token prompt, 1..64 private tokens each)",
    "spec": "synthetic (seeded N(0,1)/sqrt(128) bf16; 64 requests, lengths uniform 128..2048, "
            "4 query (draft) tokens each)",
    "int4": "synthetic (seeded INT4 K/V codes round(2 N(0,1)) in [-8, 7] with scales 0.5/sqrt(128), "
            "N(0,1)/sqrt(128) bf16 Q and new K/V; lengths uniform 128..2048)",
}
POOLS = 3
SPLIT_KERNEL = "decode_flat_kernel"     # the split phase's kernels (1- and 2-wave forms)
MERGE_KERNEL = "decode_merge_kernel"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", default="llama8b",
                   choices=["llama8b", "llama70b", "fp8", "hybrid", "prefix", "spec", "int4"],
                   help="llama8b (default line), llama70b (80 allocated layers), fp8, hybrid, "
                        "prefix (shared prompt blocks), spec (4 query tokens per request)")
    p.add_argument("--layers", type=int, default=80, help="llama70b: layers allocated and rotated")
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--split-blocks", type=int, default=0, help="override the decode split (tuning)")
    p.add_argument("--three-call", action="store_true",
                   help="time the step as slot mapping + write, split, merge (three calls) instead of "
                        "one pkv_paged_attention_decode_step call")
    p.add_argument("--shared-blocks", action="store_true",
                   help="plan as if blocks could be shared (no PKV_PLAN_BLOCKS_NOT_SHARED); "
                        "the prefix workload always is")
    p.add_argument("--workers", type=int, default=0, help="balanced-scheme workers (tuning)")
    p.add_argument("--lead", type=int, default=-1, help="balanced scheme: full-share workers (tuning)")
    p.add_argument("--trail-pct", type=int, default=0, help="balanced scheme: other share %% (tuning)")
    p.add_argument("--heads-per-item", type=int, default=0, help="balanced scheme: query heads per item")
    p.add_argument("--no-prefill-part", action="store_true",
                   help="hybrid: skip the leg that times the prefill requests in calls of their own")
    p.add_argument("--calibration-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (scale reference for HBM counters)")
    return p.parse_args()


def algorithmic_bytes(w):
    """HBM bytes a decode step must move, by kernel (see the roofline notes)."""
    B, Hq, D, Hkv = w.num_reqs, w.num_q_heads, w.head_dim, w.num_kv_heads
    nblk = int(sum(-(-int(L) // w.block_size) for L in w.seq_lens))
    # with shared prompt blocks, HBM need deliver each distinct row only once
    kv = w.info.get("unique_kv_bytes", w.kv_read_bytes())
    q = B * Hq * D * 2
    out = B * Hq * D * 2
    split = kv + q + nblk * 4 + B * 4
    combine = out
    slot = B * (4 * 3 + 4 + 8)            # qsl, computed, table entry, slot out
    elt = {"f32": 4, "bf16": 2, "fp8": 1, "int4": 0.5}[w.cache_dtype]
    src = 4 if w.q_dtype == "f32" else 2
    write = int(B * Hkv * D * 2 * (src + elt)) + B * 8  # read + write K and V rows, slots
    return dict(kv=kv, split=split, combine=combine, slot=slot, write=write,
                step=split + combine + slot + write)


def decode_plan_for(pkv, w, cache, shared_blocks=False, **tune):
    """The plan the decode line times: the library's plan for the workload,
    declaring PKV_PLAN_BLOCKS_NOT_SHARED unless blocks are shared (the
    prefix workload, which declares PKV_PLAN_BLOCKS_SHARED instead) or the
    caller says they may be; `tune` overrides fields through pkv.tune_plan
    (None keeps the library's value)."""
    shares = w.info.get("shares_blocks", False)
    not_shared = not shared_blocks and not shares
    plan = pkv.decode_plan(w.num_reqs, w.num_q_heads, cache, w.max_seq_len,
                           blocks_not_shared=not_shared, blocks_shared=shares)
    if any(v is not None for v in tune.values()):
        pkv.tune_plan(plan, w.num_reqs, w.num_q_heads, cache, w.max_seq_len, **tune)
    return plan


def decode_step_fn(pkv, w, base, plan, ws, out, slots, one_call=True):
    """One timed decode step over a (cache view, block table) pair: with
    one_call (balanced plans; the default) the decode step call, whose split
    attends to the cached keys and writes the step's K/V rows and slots and
    whose merge adds each row's own token; otherwise slot mapping and the
    write of the step's K/V rows in one launch, then the decode attention's
    two phases."""
    def step(cache, bt):
        pkv.paged_attention_decode_step(base.q, base.new_k, base.new_v, cache, bt, base.seq_lens,
                                        w.max_seq_len, w.scale, plan, ws, out, slots=slots)

    def step3(cache, bt):
        pkv.slot_mapping_cache_write(bt, base.query_start_loc, base.num_computed, base.new_k,
                                     base.new_v, cache, out=slots)
        pkv.paged_attention_decode_partials(base.q, cache, bt, base.seq_lens, w.max_seq_len, w.scale,
                                            plan, ws, out)
        pkv.paged_attention_decode_combine(out, base.seq_lens, w.block_size, plan, ws)
    return step if one_call and plan.scheme == 1 else step3


def cpu_baseline(w, sample_seqs, min_seconds=10.0):
    """The oracle, as it stands, on the first `sample_seqs` sequences of the
    step, repeated until about `min_seconds` of CPU work have been timed."""
    from oracle import attention, paging
    import copy
    sub = copy.copy(w)
    sel = np.arange(sample_seqs)
    sub.seq_lens = w.seq_lens[sel]
    sub.block_table = w.block_table[sel]
    sub.query_start_loc = np.arange(sample_seqs + 1, dtype=np.int32)
    sub.num_computed = w.num_computed[sel]
    sub.new_k, sub.new_v, sub.q = w.new_k[sel], w.new_v[sel], w.q[sel]
    t0 = time.perf_counter()
    reps = 0
    while True:
        slots, _ = paging.slot_mapping(sub.block_table, sub.query_start_loc, sub.num_computed,
                                       sub.block_size)
        kp, vp = paging.cache_write(sub.k_plane, sub.v_plane, sub.new_k, sub.new_v, slots, "bf16",
                                    sub.cache_dtype, k_scale=sub.k_scale, v_scale=sub.v_scale)
        attention.paged_decode(sub.q, "bf16", kp, vp, sub.cache_dtype, sub.block_table, sub.seq_lens,
                               sub.scale, k_scale=sub.k_scale, v_scale=sub.v_scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    ab = algorithmic_bytes(sub)["step"] * reps
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    except Exception:
        threads = 1
    return dict(value=round(ab / dt / 1e9, 4), unit="GB/s", cores=int(threads), kind="oracle",
                sample="%d of %d sequences of one step (%d tokens of context), %d repeats, %.1f s"
                       % (sample_seqs, w.num_reqs, int(sub.seq_lens.sum()), reps, dt),
                seconds=round(dt, 2), bytes=ab)


def stream_probe(w, pools, dev, steps):
    """The streaming-read probe (libpkvprobe.so): the K/V bytes of the decode
    step's (KV head, row, block) units, read in the decode's order (head
    group first; here one KV head per group) by single-wave workers with
    nothing else to do, rotating over the same
    pools; and the same number of units read block-contiguously.  Returns
    GB/s of the bytes read (whole 16-token blocks) per setting and the best,
    the practical ceiling the split kernel is held against."""
    import ctypes
    import torch
    from paged_kv_cache_mapping_amd import build as pkv_build
    lib = ctypes.CDLL(pkv_build.PROBE_LIB)
    fn = lib.pkvprobe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                   ctypes.c_void_p]
    elt = {"bf16": 2, "fp8": 1}.get(w.cache_dtype)
    if elt is None or w.head_dim * elt != 256 or w.block_size != 16:
        return None
    row_bytes = w.num_kv_heads * w.head_dim * elt
    nb = pools[0][0].num_blocks
    blk_bytes = pools[0][0].block_stride * elt
    lists = {"decode_order": [], "contiguous": []}
    for p, (cache, bt) in enumerate(pools):
        bt_h = bt.cpu().numpy()
        offs = []
        for h in range(w.num_kv_heads):
            for r, L in enumerate(w.seq_lens):
                n = -(-int(L) // w.block_size)
                phys = bt_h[r, :n].astype(np.int64)
                offs.append(phys * blk_bytes + h * w.head_dim * elt)
        offs = np.concatenate(offs)
        lists["decode_order"].append(torch.from_numpy(offs).to(dev))
        u = np.arange(len(offs), dtype=np.int64)
        first = (p * (nb // len(pools))) % max(1, nb - len(offs) // w.num_kv_heads - 1)
        lists["contiguous"].append(torch.from_numpy((first + u // w.num_kv_heads) * blk_bytes
                                                    + (u % w.num_kv_heads) * w.head_dim * elt).to(dev))
    units = int(lists["decode_order"][0].numel())
    nbytes = units * w.block_size * w.head_dim * elt * 2
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    res = {"bytes_per_launch": nbytes, "units": units, "settings": {}}
    for name, offs in lists.items():
        for workers, depth in ((2048, 1), (1024, 1), (1024, 2), (2048, 2)):
            def launch(i):
                cache = pools[i % len(pools)][0]
                st = fn(ctypes.c_void_p(cache.k.data_ptr()), ctypes.c_void_p(cache.v.data_ptr()),
                        ctypes.c_void_p(offs[i % len(pools)].data_ptr()), units, row_bytes, 256, 16,
                        workers, depth, ctypes.c_void_p(sink.data_ptr()), stream)
                assert st == 0, st
            for i in range(5):
                launch(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for i in range(steps):
                launch(i)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / steps * 1e3
            res["settings"]["%s_w%d_d%d" % (name, workers, depth)] = dict(
                us=round(us, 2), GBps=round(nbytes / (us * 1e-6) / 1e9, 1))
    best = max(res["settings"].items(), key=lambda kv: kv[1]["GBps"] if kv[0].startswith("decode") else 0)
    res["best_decode_order"] = dict(setting=best[0], **best[1])
    bestc = max((v["GBps"] for k, v in res["settings"].items() if k.startswith("contiguous")))
    res["best_contiguous_GBps"] = bestc
    return res


def rotating_pools(w, base, dev, count):
    """`count` KV pools holding the same logical data under different physical
    block permutations (so the last-level cache cannot serve the reads)."""
    import torch
    import paged_kv_cache_mapping_amd as pkv
    nb = w.num_blocks
    pools = [(base.cache, base.block_table)]
    rng = np.random.default_rng(1234)
    for _ in range(count - 1):
        perm = rng.permutation(nb)
        pt = torch.from_numpy(perm.astype(np.int64)).to(dev)
        k2 = torch.empty_like(base.cache.k)
        v2 = torch.empty_like(base.cache.v)
        k2.index_copy_(0, pt, base.cache.k)
        v2.index_copy_(0, pt, base.cache.v)
        bt = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
        pools.append((pkv.CacheView.from_planes(k2, v2, base.cache.k_scale, base.cache.v_scale,
                                                int4=base.cache.int4),
                      torch.from_numpy(bt).to(dev)))
    return pools


def layer_pools(w, base, dev, layers):
    """The whole model's cache at once: one byte buffer per layer (the pages'
    allocation), each layer's used blocks filled with the workload's data
    under its own block permutation; returns the per-layer (view, table)
    pairs and the allocation size and time."""
    import torch
    from paged_kv_cache_mapping_amd import kv_cache
    spec = kv_cache.KVCacheSpec(w.block_size, w.num_kv_heads, w.head_dim, w.cache_dtype)
    names = ["layer%d" % i for i in range(layers)]
    cfg = kv_cache.hybrid_config([kv_cache.KVCacheGroupSpec(names, spec)], w.num_blocks)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    views, bufs = kv_cache.allocate(cfg, dev)
    torch.cuda.synchronize()
    alloc_s = time.perf_counter() - t0
    used = np.unique(w.block_table[w.block_table >= 0]).astype(np.int64)
    used_t = torch.from_numpy(used).to(dev)
    ksrc = base.cache.k.index_select(0, used_t)
    vsrc = base.cache.v.index_select(0, used_t)
    rng = np.random.default_rng(4321)
    pools = []
    for name in names:
        perm = rng.permutation(w.num_blocks)
        dst = torch.from_numpy(perm[used]).to(dev)
        v = views[name]
        v.k.index_copy_(0, dst, ksrc)
        v.v.index_copy_(0, dst, vsrc)
        bt = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
        pools.append((v, torch.from_numpy(bt).to(dev)))
    torch.cuda.synchronize()
    total = sum(t.size for t in cfg.tensors)
    return pools, {"layers_allocated": layers, "allocated_bytes": int(total),
                   "allocation_s": round(alloc_s, 3)}


def calibration_copy(dev):
    """Three plain 1 GiB device-to-device copies: the known-size reference
    that turns HBM counter values of the same run into bytes."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def hybrid_layer_bytes(w, W):
    """Algorithmic bytes of one hybrid layer's attention: every request reads
    the keys its queries can see once (K and V), plus q and out."""
    ql = np.diff(w.query_start_loc)
    kv = 0
    flops = 0
    for L, q in zip(w.seq_lens.astype(np.int64), ql.astype(np.int64)):
        p0 = L - q
        lo = max(0, p0 - W + 1) if W > 0 else 0
        kv += (L - lo) * w.num_kv_heads * w.head_dim * 2 * 2
        if q > 1:
            pos = p0 + np.arange(q)
            vis = pos + 1 - (np.maximum(0, pos - W + 1) if W > 0 else 0)
            flops += int(vis.sum()) * w.num_q_heads * w.head_dim * 4
    T = w.num_tokens
    qo = T * w.num_q_heads * w.head_dim * 2 * 2
    write = T * w.num_kv_heads * w.head_dim * 2 * 2 * 2 + T * 8
    return kv + qo, write, flops


def bench_spec(args, dev):
    """Speculative decode: every request checks 4 draft tokens at once; one
    step = slot mapping + cache write of the 4 tokens + chunked attention
    (multi-token decode items).  Rotates over 3 pools like the decode line."""
    import torch
    import paged_kv_cache_mapping_amd as pkv
    from paged_kv_cache_mapping_amd import workloads
    w = workloads.spec_decode()
    base = w.device(dev)
    pools = rotating_pools(w, base, dev, POOLS)
    T, R = w.num_tokens, w.num_reqs
    nbytes = pkv.chunked_workspace_size(T, R, w.num_q_heads, base.cache, w.max_query_len, w.max_seq_len)
    ws = pkv.new_workspace(nbytes, dev)
    out = torch.empty_like(base.q)
    slots = torch.empty(T, dtype=torch.int64, device=dev)

    def attend(i):
        cache, bt = pools[i % len(pools)]
        pkv.paged_attention_chunked(base.q, base.query_start_loc, base.seq_lens, w.max_query_len, cache, bt,
                                    w.max_seq_len, w.scale, causal=True, out=out, workspace=ws,
                                    blocks_not_shared=True)

    def step(i):
        cache, bt = pools[i % len(pools)]
        pkv.slot_mapping_cache_write(bt, base.query_start_loc, base.num_computed, base.new_k, base.new_v,
                                     cache, out=slots)
        attend(i)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_step = timed(step)
    ms_attn = timed(attend)
    kv = w.kv_read_bytes()                      # each request's keys once (all 4 queries share them)
    qo = T * w.num_q_heads * w.head_dim * 2 * 2
    attn_bytes = kv + qo
    step_bytes = attn_bytes + T * w.num_kv_heads * w.head_dim * 2 * 2 * 2 + T * 8
    gbps = attn_bytes / (ms_attn * 1e-3) / 1e9
    if args.calibration_copy:
        calibration_copy(dev)
    res = {
        "metric": "paged decode attention HBM GB/s (% of peak) + KV cache writes tokens/s, 1 GPU",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": DATA_NOTE["spec"],
        "config": {"workload": w.name, "batch": R, "query_tokens": T, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "pool_blocks": w.num_blocks, "rotating_pools": len(pools),
                   "context_tokens": int(w.seq_lens.sum()), "parallelism": "none (1 GPU)"},
        "attention": {"us": round(ms_attn * 1e3, 2), "GBps": round(gbps, 1), "kv_bytes": kv},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": bench_profiles.traffic(bench_profiles.WORKLOAD_SET["spec"],
                                                       [SPLIT_KERNEL, MERGE_KERNEL]),
                     "kernel": "chunked attention (multi-token decode items + merge)"},
    }
    print(json.dumps(res), flush=True)


def bench_hybrid(args, dev):
    """Hybrid KV groups with chunked prefill: four layers (full, SWA, full,
    SWA) over two shared tensors and two group tables; one step = per group
    slot mapping, then per layer cache write + chunked attention."""
    import torch
    import paged_kv_cache_mapping_amd as pkv
    from paged_kv_cache_mapping_amd import workloads
    w = workloads.hybrid_chunked()
    cfg, views, bufs = w.device_tensors(dev)
    qsl = torch.from_numpy(w.query_start_loc).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    nc = torch.from_numpy(w.num_computed).to(dev)
    tables = [torch.from_numpy(t).to(dev) for t in w.tables]
    layers = [name for grp in w.groups for name in grp]
    layers.sort()
    group_of = {name: g for g, grp in enumerate(w.groups) for name in grp}
    inputs = {name: w.step_inputs(int(name[1:]), dev) for name in layers}
    slots = [torch.empty(w.num_tokens, dtype=torch.int64, device=dev) for _ in w.groups]
    outs = {name: torch.empty_like(inputs[name][0]) for name in layers}
    ws = {}
    for g, W in enumerate(w.windows):
        nbytes = pkv.chunked_workspace_size(w.num_tokens, len(w.seq_lens), w.num_q_heads, views[layers[0]],
                                            w.max_query_len, w.max_seq_len, W)
        ws[g] = pkv.new_workspace(nbytes, dev)

    def attend(name):
        g = group_of[name]
        q, nk, nv = inputs[name]
        pkv.cache_write(nk, nv, slots[g], views[name])
        pkv.paged_attention_chunked(q, qsl, sl, w.max_query_len, views[name], tables[g], w.max_seq_len,
                                    w.scale, causal=True, sliding_window=w.windows[g], out=outs[name],
                                    workspace=ws[g], blocks_not_shared=True)

    def step():
        for g in range(len(w.groups)):
            pkv.slot_mapping(tables[g], qsl, nc, w.block_size, w.num_blocks, out=slots[g])
        for name in layers:
            attend(name)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    per_layer = {}
    for name in layers:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            attend(name)
        b.record()
        torch.cuda.synchronize()
        per_layer[name] = a.elapsed_time(b) / args.steps
    # the prefill requests alone, in a chunked call of their own (the prefill
    # tile and its merge): the matrix-core share of the prefill part
    ql_h = np.diff(w.query_start_loc).astype(np.int64)
    pre = np.nonzero(ql_h > 1)[0]
    pre_tok = np.concatenate([np.arange(w.query_start_loc[r], w.query_start_loc[r + 1]) for r in pre])
    pre_qsl = torch.from_numpy(np.concatenate([[0], np.cumsum(ql_h[pre])]).astype(np.int32)).to(dev)
    pre_sl = torch.from_numpy(w.seq_lens[pre].astype(np.int32)).to(dev)
    pre_tok_t = torch.from_numpy(pre_tok.astype(np.int64)).to(dev)
    pre_t = torch.from_numpy(pre.astype(np.int64)).to(dev)
    pre_mql = int(ql_h[pre].max())
    prefill_ms = {}
    # (--no-prefill-part skips this leg: a kernel trace then holds only the
    # whole-layer calls)
    for name in ([] if args.no_prefill_part else layers):
        g = group_of[name]
        pq = inputs[name][0].index_select(0, pre_tok_t).contiguous()
        ptab = tables[g].index_select(0, pre_t).contiguous()
        pout = torch.empty_like(pq)
        nbytes = pkv.chunked_workspace_size(len(pre_tok), len(pre), w.num_q_heads, views[name], pre_mql,
                                            w.max_seq_len, w.windows[g])
        pws = pkv.new_workspace(nbytes, dev)

        def prefill_call():
            pkv.paged_attention_chunked(pq, pre_qsl, pre_sl, pre_mql, views[name], ptab, w.max_seq_len,
                                        w.scale, causal=True, sliding_window=w.windows[g], out=pout,
                                        workspace=pws, blocks_not_shared=True)
        for _ in range(args.warmup):
            prefill_call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            prefill_call()
        b.record()
        torch.cuda.synchronize()
        prefill_ms[name] = a.elapsed_time(b) / args.steps
    step_bytes = 0
    layer_rec = {}
    total_flops = 0
    prefill_total_ms = 0.0
    for name in layers:
        W = w.windows[group_of[name]]
        rd, wr, fl = hybrid_layer_bytes(w, W)
        step_bytes += rd + wr
        total_flops += fl
        layer_rec[name] = {"window": W, "us": round(per_layer[name] * 1e3, 1),
                           "GBps": round((rd + wr) / (per_layer[name] * 1e-3) / 1e9, 1),
                           "prefill_gflop": round(fl / 1e9, 2)}
        if name in prefill_ms:
            prefill_total_ms += prefill_ms[name]
            pt = fl / (prefill_ms[name] * 1e-3) / 1e12
            layer_rec[name].update({"prefill_alone_us": round(prefill_ms[name] * 1e3, 1),
                                    "prefill_TFLOPs": round(pt, 1),
                                    "prefill_mfma_frac": round(pt / MFMA_BF16_PEAK_TFLOPS, 4)})
    prefill_tflops = total_flops / (prefill_total_ms * 1e-3) / 1e12 if prefill_ms else None
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    if args.calibration_copy:
        calibration_copy(dev)
    dom = max(layers, key=lambda n: per_layer[n])
    rd, wr, _ = hybrid_layer_bytes(w, w.windows[group_of[dom]])
    gbps = (rd + wr) / (per_layer[dom] * 1e-3) / 1e9
    # HBM bytes of one whole step from the counter passes: each kernel's bytes
    # per launch (averaged over the four layers' launches) times its launches
    # per step (slot mapping once per group, the others once per layer)
    per_step = [(len(w.groups), "slot_mapping_kernel"), (len(layers), "cache_write_kernel"),
                (len(layers), "prefill_tile_kernel"), (len(layers), "prefill_merge_kernel"),
                (len(layers), SPLIT_KERNEL), (len(layers), MERGE_KERNEL)]
    parts = [bench_profiles.traffic(bench_profiles.WORKLOAD_SET["hybrid"], [frag]) for _, frag in per_step]
    step_traffic = (sum(n * t for (n, _), t in zip(per_step, parts))
                    if all(t is not None for t in parts) else None)
    res = {
        "metric": "paged decode attention HBM GB/s (% of peak) + KV cache writes tokens/s, 1 GPU",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": DATA_NOTE["hybrid"],
        "config": {"workload": "hybrid_groups_chunked_prefill_96dec_4x512", "layers": layers,
                   "num_tokens": w.num_tokens, "requests": int(len(w.seq_lens)),
                   "windows": list(w.windows), "pool_blocks": int(w.num_blocks),
                   "context_tokens": int(w.seq_lens.sum()), "parallelism": "none (1 GPU)"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "layers": layer_rec,
        "prefill_gflop_per_step": round(total_flops / 1e9, 1),
        **({"prefill_part": {"requests": int(len(pre)), "query_tokens": int(len(pre_tok)),
                             "us_per_step": round(prefill_total_ms * 1e3, 1),
                             "TFLOPs": round(prefill_tflops, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                             "mfma_frac": round(prefill_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "flops": "4 D per visible (query token, key, query head): scores and P.V"}}
           if prefill_ms else {}),
        # the unit is the whole step (its kernels are timed together; the
        # counters give bytes per kernel averaged over the layers)
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": step_traffic,
                     "algorithmic_bytes": int(step_bytes),
                     "kernel": "whole step: 4 layers of cache write + chunked attention, and the slot "
                               "mappings"},
        "dominant_layer": {"layer": dom, "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)},
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_kv_cache_mapping_amd as pkv
    from paged_kv_cache_mapping_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "hybrid":
        return bench_hybrid(args, dev)
    if args.workload == "spec":
        return bench_spec(args, dev)
    w = {"llama8b": workloads.llama8b_decode, "llama70b": workloads.llama70b_decode,
         "fp8": workloads.fp8_decode, "prefix": workloads.shared_prefix_decode,
         "int4": workloads.int4_decode}[args.workload]()
    base = w.device(dev)
    nb = w.num_blocks
    extra = {}
    if args.workload == "llama70b":
        pools, extra = layer_pools(w, base, dev, args.layers)
    else:
        pools = rotating_pools(w, base, dev, POOLS)
    npools = len(pools)

    plan = decode_plan_for(pkv, w, base.cache, shared_blocks=args.shared_blocks,
                           split_blocks=args.split_blocks or None, num_workers=args.workers or None,
                           lead_workers=args.lead if args.lead >= 0 else None,
                           trail_share_pct=args.trail_pct or None,
                           heads_per_item=args.heads_per_item or None)
    ws = pkv.new_workspace(plan.workspace_bytes, dev)
    out = torch.empty_like(base.q)
    slots = torch.empty(w.num_reqs, dtype=torch.int64, device=dev)
    run_step = decode_step_fn(pkv, w, base, plan, ws, out, slots, one_call=not args.three_call)

    def step(i):
        run_step(*pools[i % npools])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps between synchronised events
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # split kernel alone: `steps` back-to-back launches over the same pool
    # rotation between two events (no event inside, so no per-event overhead)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(args.steps):
        cache, bt = pools[i % npools]
        pkv.paged_attention_decode_partials(base.q, cache, bt, base.seq_lens, w.max_seq_len, w.scale,
                                            plan, ws, out)
    b.record()
    torch.cuda.synchronize()
    split_ms = a.elapsed_time(b) / args.steps

    # the same steps recorded once in a HIP graph (one step per pool of the
    # rotation) and replayed: what a serving loop that replays its step sees
    graph = None
    if plan.scheme == 1 and not args.three_call:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(npools):
                step(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, -(-args.steps // npools))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        gms = a.elapsed_time(b) / (reps * npools)
        graph = dict(us_per_step=round(gms * 1e3, 2), steps_per_graph=npools, replays=reps)
        del g

    ab = algorithmic_bytes(w)
    value = ab["step"] / (ms_per_step * 1e-3) / 1e9
    if graph is not None:
        graph["GBps"] = round(ab["step"] / (graph["us_per_step"] * 1e-6) / 1e9, 1)
    split_gbps = ab["split"] / (split_ms * 1e-3) / 1e9

    # bulk KV writes: distinct random slots, bf16 -> bf16 and bf16 -> fp8
    writes = {}
    for T in ((16384, 131072) if args.workload == "llama8b" else ()):
        gen = torch.Generator(device=dev).manual_seed(T)
        kx = torch.randn((T, w.num_kv_heads, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
        vx = torch.randn((T, w.num_kv_heads, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
        sl = torch.randperm(nb * w.block_size, generator=gen, device=dev)[:T]
        for dst in ("bf16", "fp8"):
            if dst == "bf16":
                cache = pools[0][0]
            else:
                k8 = torch.empty(base.cache.k.shape, dtype=torch.uint8, device=dev)
                v8 = torch.empty(base.cache.v.shape, dtype=torch.uint8, device=dev)
                cache = pkv.CacheView.from_planes(k8, v8, 0.01, 0.01)
            for _ in range(3):
                pkv.cache_write(kx, vx, sl, cache)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 20
            a.record()
            for _ in range(reps):
                pkv.cache_write(kx, vx, sl, cache)
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            elt = 2 if dst == "bf16" else 1
            nbytes = T * w.num_kv_heads * w.head_dim * 2 * (2 + elt) + T * 8
            writes["%s_T%d" % (dst, T)] = dict(tokens_per_s=round(T / (ms * 1e-3)),
                                              GBps=round(nbytes / (ms * 1e-3) / 1e9, 1),
                                              us=round(ms * 1e3, 2))
    # one decode step's 64-token write (launch-latency bound)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(50):
        pkv.cache_write(base.new_k, base.new_v, slots, pools[0][0])
    b.record()
    torch.cuda.synchronize()
    writes["bf16_T64_step"] = dict(us=round(a.elapsed_time(b) / 50 * 1e3, 2))
    # the same with its slot mapping in the one launch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(50):
        pkv.slot_mapping_cache_write(pools[0][1], base.query_start_loc, base.num_computed, base.new_k,
                                     base.new_v, pools[0][0], out=slots)
    b.record()
    torch.cuda.synchronize()
    writes["slot_mapping_and_write_T64_step"] = dict(us=round(a.elapsed_time(b) / 50 * 1e3, 2))

    sharing = {}
    if args.workload == "prefix":
        # logical reads (every request's whole context) and the block saving
        logical = w.kv_read_bytes()
        sharing = dict(logical_kv_bytes=logical, unique_kv_bytes=w.info["unique_kv_bytes"],
                       logical_split_GBps=round(logical / (split_ms * 1e-3) / 1e9, 1),
                       blocks_with_sharing=w.info["blocks_used"],
                       blocks_without_sharing=w.info["blocks_without_sharing"],
                       cow_pairs=w.info["cow_pairs"])
        # copy-on-write throughput: 4096 disjoint block pairs, both planes
        gen = torch.Generator(device=dev).manual_seed(7)
        perm = torch.randperm(nb, generator=gen, device=dev).to(torch.int32)
        src, dst = perm[:4096].contiguous(), perm[4096:8192].contiguous()
        cache = pools[0][0]
        for _ in range(3):
            pkv.copy_blocks(src, dst, cache)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            pkv.copy_blocks(src, dst, cache)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 20
        blk = w.block_size * w.num_kv_heads * w.head_dim * 2
        sharing["copy_blocks_4096_pairs"] = dict(us=round(ms * 1e3, 2),
                                                 GBps=round(4096 * blk * 2 * 2 / (ms * 1e-3) / 1e9, 1))

    if args.calibration_copy:
        calibration_copy(dev)

    probe = stream_probe(w, pools, dev, min(args.steps, 100)) if args.workload == "llama8b" else None
    traffic = bench_profiles.traffic(bench_profiles.WORKLOAD_SET[args.workload], [SPLIT_KERNEL])
    res = {
        "metric": "paged decode attention HBM GB/s (% of peak) + KV cache writes tokens/s, 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "e4m3 KV, bf16 q/out", "int4": "int4 KV, bf16 q/out"}[w.cache_dtype],
        "data": DATA_NOTE[args.workload],
        "config": {"workload": w.name, "batch": w.num_reqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "pool_blocks": nb, "rotating_pools": npools,
                   "context_tokens": int(w.seq_lens.sum()), "parallelism": "none (1 GPU)",
                   "scheme": int(plan.scheme), "workers": int(plan.num_workers),
                   "split_blocks": int(plan.split_blocks), "max_splits": int(plan.max_splits),
                   "lead_workers": int(plan.lead_workers), "trail_share_pct": int(plan.trail_share_pct),
                   "plan_flags": int(plan.flags),
                   "step_calls": ("decode_step" if not args.three_call and plan.scheme == 1
                                  else "slot_mapping_cache_write + decode_partials + decode_combine"),
                   **extra},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_attention": {"split_kernel_us": round(split_ms * 1e3, 2),
                             "split_GBps": round(split_gbps, 1),
                             "kv_bytes": ab["kv"], "step_bytes": ab["step"]},
        **({"graph_replay": graph} if graph else {}),
        "kv_write": writes,
        # the split kernel's GB/s (algorithmic bytes) against the probe's
        # (every byte of the blocks it reads): a conservative fraction
        **({"stream_probe": probe,
            "split_pct_of_probe": round(100 * split_gbps / probe["best_decode_order"]["GBps"], 2)}
           if probe else {}),
        **({"prefix_sharing": sharing} if sharing else {}),
        "roofline": {"bound": "hbm", "achieved": round(split_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(split_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": SPLIT_KERNEL,
                     "algorithmic_bytes_per_launch": ab["split"]},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, sample_seqs=w.num_reqs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
