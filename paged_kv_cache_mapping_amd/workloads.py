"""Seeded synthetic workloads (inputs only; no arithmetic of the method).

Both the HIP path and the oracle read the arrays made here.  Every array is
drawn from ``numpy.random.default_rng(seed)`` (PCG64) in a fixed order:
lengths -> block-pool permutation -> K history -> V history -> new K/V -> Q.
float32 draws become bfloat16 by round-to-nearest-even (torch's conversion)
and FP8 history by torch's E4M3 conversion after clamping to +-448 with the
per-tensor scale amax/448.  INT4 history is drawn as integer codes directly:
round(2 z) for standard normal z, limited to [-8, 7], with scales sigma / 2,
stored as nibbles (element 2j low, 2j + 1 high).  Blocks no request owns are
filled with NaN (INT4, which has no NaN: 0xFF, the largest value) so that
any stray read shows up.

Block tables come from a shuffled free pool, as a scheduler would hand them
out; the hybrid workload drives :class:`kv_cache.GroupBlockTables` so that
sliding-window blocks are released and re-drawn by other requests.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

from . import kv_cache

NAN_BITS = {"bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F), "int4": np.uint8(0xFF)}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "int4": np.uint8}


def bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns (torch RNE conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def fp8_codes(x, scale):
    """float32 array -> E4M3 codes of clamp(x / scale) (torch conversion)."""
    y = np.clip(np.asarray(x, np.float32) * (np.float32(1) / np.float32(scale)), -448.0, 448.0)
    return torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def int4_history(rng, shape):
    """Packed INT4 rows [..., D / 2] of codes round(2 z) in [-8, 7]."""
    k = np.clip(np.rint(rng.standard_normal(shape, dtype=np.float32) * np.float32(2.0)), -8, 7)
    u = (k + 8).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def nan_plane(shape, dtype):
    if dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, NAN_BITS[dtype], dtype=STORAGE[dtype])


@dataclass
class Workload:
    name: str
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    cache_dtype: str          # storage of the planes
    q_dtype: str              # q, new K/V and output
    k_plane: np.ndarray       # [nb, bs, Hkv, D] storage bits
    v_plane: np.ndarray
    new_k: np.ndarray         # [T, Hkv, D] (float32 or bf16 bits)
    new_v: np.ndarray
    q: np.ndarray             # [T, Hq, D]
    block_table: np.ndarray   # [R, width] int32
    seq_lens: np.ndarray      # [R] int32, including this step's tokens
    query_start_loc: np.ndarray  # [R + 1] int32
    num_computed: np.ndarray  # [R] int32
    scale: float
    window: int = 0
    causal: bool = True
    k_scale: float = 1.0
    v_scale: float = 1.0
    decode: bool = True       # one query token per request
    info: dict = field(default_factory=dict)

    @property
    def num_reqs(self):
        return len(self.seq_lens)

    @property
    def num_tokens(self):
        return int(self.query_start_loc[-1])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    @property
    def max_query_len(self):
        return int(np.diff(self.query_start_loc).max()) if len(self.seq_lens) else 0

    def kv_read_bytes(self):
        """Cache bytes an attention pass must read: visible keys x Hkv x D x 2."""
        elt = {"f32": 4, "bf16": 2, "fp8": 1, "int4": 0.5}[self.cache_dtype]
        total = 0
        for L, q0, q1 in zip(self.seq_lens, self.query_start_loc[:-1], self.query_start_loc[1:]):
            p0 = int(L) - int(q1 - q0)
            lo = max(0, p0 - self.window + 1) if self.window > 0 else 0
            total += int(L) - lo
        return int(total * self.num_kv_heads * self.head_dim * 2 * elt)

    def device(self, device="cuda"):
        """Device copies: a one-layer KV tensor (byte buffer + typed views)."""
        spec = kv_cache.KVCacheSpec(self.block_size, self.num_kv_heads, self.head_dim, self.cache_dtype)
        cfg = kv_cache.hybrid_config([kv_cache.KVCacheGroupSpec(["layer0"], spec)], self.num_blocks)
        views, bufs = kv_cache.allocate(cfg, device, k_scale=self.k_scale, v_scale=self.v_scale)
        cache = views["layer0"]
        tdt = kv_cache.TORCH_DTYPE[self.cache_dtype]
        cache.k.copy_(_to_torch(self.k_plane, tdt))
        cache.v.copy_(_to_torch(self.v_plane, tdt))
        qdt = kv_cache.TORCH_DTYPE[self.q_dtype]
        d = dict(
            cache=cache, buffers=bufs,
            q=_to_torch(self.q, qdt).to(device),
            new_k=_to_torch(self.new_k, qdt).to(device),
            new_v=_to_torch(self.new_v, qdt).to(device),
            block_table=torch.from_numpy(self.block_table).to(device),
            seq_lens=torch.from_numpy(self.seq_lens).to(device),
            query_start_loc=torch.from_numpy(self.query_start_loc).to(device),
            num_computed=torch.from_numpy(self.num_computed).to(device),
        )
        return type("DeviceWorkload", (), d)


def _to_torch(a, tdt):
    if tdt == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def _tables_from_pool(lengths, block_size, perm, width=None):
    """Rows drawn in order from the shuffled pool: request r takes ceil(L_r / bs)."""
    need = [-(-int(L) // block_size) for L in lengths]
    width = width or max(need + [1])
    bt = np.full((len(lengths), width), -1, dtype=np.int32)
    k = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[k:k + n]
        k += n
    return bt, k


def _fill_history(rng, plane, ids, shape_tail, dtype, sigma, scale=None):
    n = len(ids)
    x = rng.standard_normal((n,) + shape_tail, dtype=np.float32) * np.float32(sigma)
    if dtype == "f32":
        plane[ids] = x
    elif dtype == "bf16":
        plane[ids] = bf16_bits(x)
    else:
        plane[ids] = fp8_codes(x, scale)
    return x


def decode_workload(name, seed, lengths_fn, num_blocks_fn, *, block_size, num_q_heads,
                    num_kv_heads, head_dim, cache_dtype, q_dtype, sigma, window=0,
                    fp8_amax_scale=False, pool_blocks=None):
    """Generic decode step: one new token per sequence at position L - 1."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths_fn(rng), dtype=np.int32)                       # lengths
    needed = int(sum(-(-int(L) // block_size) for L in lengths))
    nb = pool_blocks if pool_blocks is not None else num_blocks_fn(needed)
    perm = rng.permutation(nb).astype(np.int32)                                 # permutation
    bt, used = _tables_from_pool(lengths, block_size, perm)
    ids = perm[:used]
    shape = (nb, block_size, num_kv_heads, head_dim)
    tail = shape[1:]
    pshape = shape[:3] + (head_dim // 2,) if cache_dtype == "int4" else shape
    kp, vp = nan_plane(pshape, cache_dtype), nan_plane(pshape, cache_dtype)
    B = len(lengths)
    if cache_dtype == "int4":
        kp[ids] = int4_history(rng, (used,) + tail)                             # K history
        vp[ids] = int4_history(rng, (used,) + tail)                             # V history
        nk = rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32) * np.float32(sigma)
        nv = rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32) * np.float32(sigma)
        new_k, new_v = bf16_bits(nk), bf16_bits(nv)
        k_scale = v_scale = float(np.float32(sigma / 2.0))
    elif cache_dtype == "fp8":
        kx = rng.standard_normal((used,) + tail, dtype=np.float32) * np.float32(sigma)   # K history
        vx = rng.standard_normal((used,) + tail, dtype=np.float32) * np.float32(sigma)   # V history
        nk = rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32) * np.float32(sigma)
        nv = rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32) * np.float32(sigma)
        new_k, new_v = bf16_bits(nk), bf16_bits(nv)
        # per-tensor scales from the largest magnitude of everything the cache holds
        k_scale = float(np.float32(max(np.abs(kx).max(), np.abs(nk).max()) / 448.0))
        v_scale = float(np.float32(max(np.abs(vx).max(), np.abs(nv).max()) / 448.0))
        kp[ids] = fp8_codes(kx, k_scale)
        vp[ids] = fp8_codes(vx, v_scale)
    else:
        _fill_history(rng, kp, ids, tail, cache_dtype, sigma)                   # K history
        _fill_history(rng, vp, ids, tail, cache_dtype, sigma)                   # V history
        nk = rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32) * np.float32(sigma)
        nv = rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32) * np.float32(sigma)
        new_k = nk if q_dtype == "f32" else bf16_bits(nk)
        new_v = nv if q_dtype == "f32" else bf16_bits(nv)
        k_scale = v_scale = 1.0
    qx = rng.standard_normal((B, num_q_heads, head_dim), dtype=np.float32) * np.float32(
        1.0 if cache_dtype == "fp8" else sigma)                                  # Q
    q = qx if q_dtype == "f32" else bf16_bits(qx)
    return Workload(
        name=name, block_size=block_size, num_blocks=nb, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, cache_dtype=cache_dtype, q_dtype=q_dtype,
        k_plane=kp, v_plane=vp, new_k=new_k, new_v=new_v, q=q, block_table=bt,
        seq_lens=lengths, query_start_loc=np.arange(B + 1, dtype=np.int32),
        num_computed=(lengths - 1).astype(np.int32), scale=float(1.0 / np.sqrt(head_dim)),
        window=window, k_scale=k_scale, v_scale=v_scale, decode=True,
        info=dict(seed=seed, blocks_used=used))


# ---------------------------------------------------------------------------
# The five workloads.

def tiny(seed=1):
    """fp32, block 4, 2 query heads on 1 KV head, head_dim 8, 16 blocks,
    context lengths 5 and 11 (including the decode token)."""
    return decode_workload(
        "tiny_fp32_bs4_gqa2_d8", seed, lambda rng: [5, 11], None, pool_blocks=16,
        block_size=4, num_q_heads=2, num_kv_heads=1, head_dim=8, cache_dtype="f32",
        q_dtype="f32", sigma=1.0)


def llama8b_decode(seed=2, batch=64, lo=128, hi=2048, pool=16384):
    """Llama-3-8B-shaped decode layer: bf16, 32/8 heads, D 128, block 16,
    64 sequences with lengths uniform in [128, 2048], 16384-block pool."""
    return decode_workload(
        "llama3_8b_decode_b64_L128-2048", seed, lambda rng: rng.integers(lo, hi + 1, size=batch),
        None, pool_blocks=pool, block_size=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
        cache_dtype="bf16", q_dtype="bf16", sigma=1.0 / np.sqrt(128.0))


def llama70b_decode(seed=3, batch=32, length=4096, pool=16384):
    """LLaMA-70B-shaped decode layer: bf16, 64/8 heads, D 128, block 16,
    32 sequences of 4096 tokens from a shuffled 16384-block pool."""
    return decode_workload(
        "llama70b_decode_b32_L4096", seed, lambda rng: np.full(batch, length), None,
        pool_blocks=pool, block_size=16, num_q_heads=64, num_kv_heads=8, head_dim=128,
        cache_dtype="bf16", q_dtype="bf16", sigma=1.0 / np.sqrt(128.0))


def fp8_decode(seed=4, batch=128, sigma_len=1.0):
    """E4M3 KV with per-tensor scales, bf16 Q/out, 32/8 heads, D 128,
    block 16, 128 sequences, lognormal lengths (median 1024) in [16, 32768]."""
    def lengths(rng):
        return np.clip(np.round(np.exp(rng.normal(np.log(1024.0), sigma_len, size=batch))), 16, 32768)
    return decode_workload(
        "fp8_e4m3_decode_b128_lognormal1024", seed, lengths, lambda n: int(np.ceil(n * 1.25)),
        block_size=16, num_q_heads=32, num_kv_heads=8, head_dim=128, cache_dtype="fp8",
        q_dtype="bf16", sigma=1.0, fp8_amax_scale=True)


def int4_decode(seed=8, batch=64, lo=128, hi=2048, pool=16384):
    """The Llama-3-8B decode layer with an INT4 cache (half a byte per
    element): 32/8 heads, D 128, block 16, 64 sequences with lengths uniform
    in [128, 2048], 16384-block pool, per-tensor scales sigma / 2."""
    return decode_workload(
        "int4_decode_b64_L128-2048", seed, lambda rng: rng.integers(lo, hi + 1, size=batch),
        None, pool_blocks=pool, block_size=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
        cache_dtype="int4", q_dtype="bf16", sigma=1.0 / np.sqrt(128.0))


def spec_decode(seed=7, batch=64, q_len=4, lo=128, hi=2048, pool=16384):
    """Speculative decode step on the Llama-3-8B shape: 64 requests with
    contexts uniform in [lo, hi] (including this step's tokens), each
    checking q_len draft tokens at once (q_len query tokens at positions
    L - q_len .. L - 1, causal).  bf16, 32/8 heads, D 128, block 16."""
    D, Hq, Hkv, bs = 128, 32, 8, 16
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, size=batch).astype(np.int32)            # lengths
    perm = rng.permutation(pool).astype(np.int32)                               # permutation
    bt, used = _tables_from_pool(lengths, bs, perm)
    ids = perm[:used]
    shape = (pool, bs, Hkv, D)
    sigma = 1.0 / np.sqrt(D)
    kp, vp = nan_plane(shape, "bf16"), nan_plane(shape, "bf16")
    _fill_history(rng, kp, ids, shape[1:], "bf16", sigma)                       # K history
    _fill_history(rng, vp, ids, shape[1:], "bf16", sigma)                       # V history
    T = batch * q_len
    nk = bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32) * np.float32(sigma))
    nv = bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32) * np.float32(sigma))
    q = bf16_bits(rng.standard_normal((T, Hq, D), dtype=np.float32) * np.float32(sigma))   # Q
    return Workload(
        name="spec_decode_b%d_q%d_L%d-%d" % (batch, q_len, lo, hi), block_size=bs, num_blocks=pool,
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, cache_dtype="bf16", q_dtype="bf16",
        k_plane=kp, v_plane=vp, new_k=nk, new_v=nv, q=q, block_table=bt, seq_lens=lengths,
        query_start_loc=(np.arange(batch + 1) * q_len).astype(np.int32),
        num_computed=(lengths - q_len).astype(np.int32), scale=float(1.0 / np.sqrt(D)), decode=False,
        info=dict(seed=seed, blocks_used=used, q_len=q_len))


def shared_prefix_decode(seed=6, num_reqs=100, prompt=2000, suffix_hi=64, pool=16384, block_size=16):
    """Prefix sharing (Chinese worker-side page, § PagedAttention与Block管理:
    100 requests opening with one 2000-token system prompt): every request's
    table starts with the prompt's blocks, held once in the pool by
    reference; each request then has 1..suffix_hi private tokens, the last
    being this step's decode token.  bf16, 32/8 heads, D 128, block 16.

    The tables come from the host pool: request 0 writes the prompt, the
    others fork it, and every request makes its suffix blocks private
    (copy-on-write pairs only arise when the prompt ends inside a block)."""
    D, Hq, Hkv = 128, 32, 8
    rng = np.random.default_rng(seed)
    suffix = rng.integers(1, suffix_hi + 1, size=num_reqs)                      # lengths
    lengths = (prompt + suffix).astype(np.int32)
    perm = rng.permutation(pool)                                                # permutation
    bp = kv_cache.BlockPool(pool, order=perm)
    tabs = kv_cache.GroupBlockTables(bp, [0], block_size)
    tabs.add_request(0)
    tabs.prepare_write(0, 0, prompt)
    for r in range(1, num_reqs):
        tabs.add_request(r)
        tabs.fork(0, r, prompt)
    cow = []
    for r in range(num_reqs):
        cow += tabs.prepare_write(r, prompt, int(lengths[r]))
    bt = tabs.table(0, list(range(num_reqs)))
    ids = np.nonzero(bp.refcount)[0].astype(np.int32)
    shape = (pool, block_size, Hkv, D)
    sigma = 1.0 / np.sqrt(D)
    kp, vp = nan_plane(shape, "bf16"), nan_plane(shape, "bf16")
    _fill_history(rng, kp, ids, shape[1:], "bf16", sigma)                       # K history
    _fill_history(rng, vp, ids, shape[1:], "bf16", sigma)                       # V history
    for src, dst in cow:                                                        # copied blocks
        kp[dst], vp[dst] = kp[src], vp[src]
    nk = bf16_bits(rng.standard_normal((num_reqs, Hkv, D), dtype=np.float32) * np.float32(sigma))
    nv = bf16_bits(rng.standard_normal((num_reqs, Hkv, D), dtype=np.float32) * np.float32(sigma))
    q = bf16_bits(rng.standard_normal((num_reqs, Hq, D), dtype=np.float32) * np.float32(sigma))  # Q
    without = int(sum(-(-int(L) // block_size) for L in lengths))
    unique_rows = prompt + int(suffix.sum())
    return Workload(
        name="shared_prefix_decode_b%d_prompt%d" % (num_reqs, prompt), block_size=block_size,
        num_blocks=pool, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, cache_dtype="bf16",
        q_dtype="bf16", k_plane=kp, v_plane=vp, new_k=nk, new_v=nv, q=q, block_table=bt,
        seq_lens=lengths, query_start_loc=np.arange(num_reqs + 1, dtype=np.int32),
        num_computed=(lengths - 1).astype(np.int32), scale=float(1.0 / np.sqrt(D)), decode=True,
        info=dict(seed=seed, shares_blocks=True, blocks_used=int(len(ids)), blocks_without_sharing=without,
                  cow_pairs=len(cow), unique_kv_bytes=unique_rows * Hkv * D * 2 * 2))


# ---------------------------------------------------------------------------
# Hybrid groups with chunked prefill.

@dataclass
class HybridWorkload:
    """Four layers: group 0 (L0, L2) full attention, group 1 (L1, L3) sliding
    window; tensor 0 holds L0 and L1, tensor 1 holds L2 and L3; one shared
    block pool.  Per-group block tables; one step mixes decode requests
    (one query) and prefill chunks (causal)."""
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int
    groups: list              # layer names per group
    windows: list             # per group
    tables: list              # per group [R, width] int32
    seq_lens: np.ndarray
    query_start_loc: np.ndarray
    num_computed: np.ndarray
    scale: float
    seed: int
    live_ids: np.ndarray      # every id some table holds
    info: dict = field(default_factory=dict)

    @property
    def num_tokens(self):
        return int(self.query_start_loc[-1])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max())

    @property
    def max_query_len(self):
        return int(np.diff(self.query_start_loc).max())

    def config(self):
        spec0 = kv_cache.KVCacheSpec(self.block_size, self.num_kv_heads, self.head_dim, "bf16", 0)
        spec1 = kv_cache.KVCacheSpec(self.block_size, self.num_kv_heads, self.head_dim, "bf16", self.window)
        return kv_cache.hybrid_config([kv_cache.KVCacheGroupSpec(self.groups[0], spec0),
                                       kv_cache.KVCacheGroupSpec(self.groups[1], spec1)],
                                      self.num_blocks)

    def device_tensors(self, device="cuda"):
        """Allocate both tensors; fill every live block with N(0, 1/D) bf16
        (torch generator seeded per tensor), every other block with NaN."""
        cfg = self.config()
        views, bufs = kv_cache.allocate(cfg, device)
        live = torch.from_numpy(self.live_ids.astype(np.int64)).to(device)
        for t, tensor in enumerate(cfg.tensors):
            cache = views[tensor.shared_by[0]]
            gen = torch.Generator(device=device).manual_seed(self.seed * 1000 + t)
            for plane in (cache.k, cache.v):
                plane.view(torch.int16).fill_(0x7FC0)
                vals = torch.randn((len(self.live_ids),) + tuple(plane.shape[1:]), generator=gen,
                                   device=device, dtype=torch.float32) / np.sqrt(self.head_dim)
                plane.index_copy_(0, live, vals.to(torch.bfloat16))
        return cfg, views, bufs

    def step_inputs(self, layer, device="cuda"):
        """Q and new K/V [T, heads, D] bf16 for one layer (seeded per layer)."""
        gen = torch.Generator(device=device).manual_seed(self.seed * 1000 + 100 + layer)
        T = self.num_tokens
        s = 1.0 / np.sqrt(self.head_dim)
        new_k = (torch.randn((T, self.num_kv_heads, self.head_dim), generator=gen, device=device) * s)
        new_v = (torch.randn((T, self.num_kv_heads, self.head_dim), generator=gen, device=device) * s)
        q = (torch.randn((T, self.num_q_heads, self.head_dim), generator=gen, device=device) * s)
        return q.to(torch.bfloat16), new_k.to(torch.bfloat16), new_v.to(torch.bfloat16)


def hybrid_chunked(seed=5, num_decode=96, num_prefill=4, chunk=512, window=4096,
                   decode_lo=1024, decode_hi=16384, prefill_hi=8192, history_chunk=512,
                   block_size=16, slack=1.10):
    """Hybrid KV groups with chunked prefill (see :class:`HybridWorkload`).

    Decode requests: context uniform in [1024, 16384] including the new token.
    Prefill chunks: cached offset uniform in [0, 8192], 512 new tokens, causal.
    History is built step-wise: requests grow by 512-token chunks in a
    shuffled round-robin, and the sliding-window group gives back blocks that
    leave the window after each chunk, so released ids are drawn again by
    other requests.  Batch order is shuffled.
    """
    rng = np.random.default_rng(seed)
    L_dec = rng.integers(decode_lo, decode_hi + 1, size=num_decode)
    c_pre = rng.integers(0, prefill_hi + 1, size=num_prefill)
    seq = np.concatenate([L_dec, c_pre + chunk]).astype(np.int64)
    ql = np.concatenate([np.ones(num_decode, np.int64), np.full(num_prefill, chunk, np.int64)])
    R = len(seq)
    full_blocks = int(sum(-(-int(L) // block_size) for L in seq))
    swa_blocks = int(sum(min(-(-int(L) // block_size), -(-(window + int(q) - 1) // block_size) + 2)
                         for L, q in zip(seq, ql)))
    nb = int(np.ceil((full_blocks + swa_blocks) * slack))
    pool = kv_cache.BlockPool(nb, order=rng.permutation(nb))
    tables = kv_cache.GroupBlockTables(pool, [0, window], block_size)
    cached = seq - ql
    progress = np.zeros(R, np.int64)
    for r in range(R):
        tables.add_request(r)
    while (progress < cached).any():
        for r in rng.permutation(R):
            if progress[r] < cached[r]:
                new = min(int(progress[r]) + history_chunk, int(cached[r]))
                tables.grow(r, new)
                progress[r] = new
                tables.release_out_of_window(r, new)
    for r in range(R):
        tables.grow(r, int(seq[r]))
    order = rng.permutation(R)                                              # batch order
    width = max(-(-int(L) // block_size) for L in seq)
    t_full = tables.table(0, list(order), width)
    t_swa = tables.table(1, list(order), width)
    seq_o = seq[order].astype(np.int32)
    ql_o = ql[order]
    qsl = np.concatenate([[0], np.cumsum(ql_o)]).astype(np.int32)
    live = np.unique(np.concatenate([t_full[t_full >= 0], t_swa[t_swa >= 0]]))
    return HybridWorkload(
        block_size=block_size, num_blocks=nb, num_q_heads=32, num_kv_heads=8, head_dim=128,
        window=window, groups=[["L0", "L2"], ["L1", "L3"]], windows=[0, window],
        tables=[t_full, t_swa], seq_lens=seq_o, query_start_loc=qsl,
        num_computed=(seq_o - ql_o).astype(np.int32), scale=float(1.0 / np.sqrt(128.0)), seed=seed,
        live_ids=live, info=dict(pool_free=pool.num_free, full_blocks=full_blocks,
                                 order=order, decode_requests=num_decode))


ALL = {"tiny": tiny, "llama8b": llama8b_decode, "llama70b": llama70b_decode,
       "fp8": fp8_decode, "hybrid": hybrid_chunked, "int4": int4_decode}
