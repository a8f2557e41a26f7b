"""Host-side KV-cache layout: configs, byte-buffer allocation, typed views,
the physical block pool and per-group block tables (no kernels here).

Sources:

* A worker's KV-cache "resource contract" holds the block count, the groups
  (layers sharing one logical block table) and the physical tensors with the
  layers that share each (page "Deep Dive into vLLM Worker-Side GPU KV Cache
  Initialization", section "Composition of KVCacheConfig").
* Each tensor is allocated once as an untyped byte buffer and reinterpreted
  per layer without copying (same page, sections "Step 1: Physical
  Allocation" and "Step 2: View Transformation (reshape)"); block starts keep
  an alignment that suits the memory system (Chinese original, section
  "第一步：物理分配").
* Layers at the same position ("slot") of different groups share one tensor;
  layers of one group sit in different tensors (sections "Model View:
  Grouping" and "Physical View: Two KVCacheTensors").
* The scheduler keeps a free block pool and per-request tables mapping
  logical to physical blocks; ids return to the pool when released
  ("vLLM의 KV cache 연결 흐름", section on the KV cache manager); sliding-window
  layers release blocks that fall wholly before the window (Chinese original,
  section "混合注意力机制"); blocks can be shared between requests with a
  reference count (section "PagedAttention与Block管理").
"""

from dataclasses import dataclass, field

import numpy as np
import torch

from .api import CacheView

ELEMENT_BITS = {"f32": 32, "bf16": 16, "fp8": 8, "int4": 4}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8, "int4": torch.uint8}
ALIGN = 256


@dataclass(frozen=True)
class KVCacheSpec:
    """How one layer reads its tensor: block size, heads, head size, dtype."""
    block_size: int
    num_kv_heads: int
    head_dim: int
    dtype: str = "bf16"
    sliding_window: int = 0

    @property
    def block_bytes(self):
        """Bytes of one block of one plane (K or V)."""
        return self.block_size * self.num_kv_heads * self.head_dim * ELEMENT_BITS[self.dtype] // 8

    @property
    def page_bytes(self):
        """K + V bytes of one block."""
        return 2 * self.block_bytes


@dataclass
class KVCacheGroupSpec:
    layer_names: list
    spec: KVCacheSpec


@dataclass
class KVCacheTensor:
    size: int            # bytes
    shared_by: list      # layer names


@dataclass
class KVCacheConfig:
    num_blocks: int
    groups: list         # [KVCacheGroupSpec]
    tensors: list = field(default_factory=list)   # [KVCacheTensor]

    def layer_group(self, name):
        for g, grp in enumerate(self.groups):
            if name in grp.layer_names:
                return g
        raise KeyError(name)


def hybrid_config(groups, num_blocks):
    """Config for groups of layers; tensor i holds the i-th layer of every group.

    All groups must have the same page size (they share tensors and one id
    space).  Returns a KVCacheConfig with one tensor per slot.
    """
    pages = {grp.spec.page_bytes for grp in groups}
    if len(pages) != 1:
        raise ValueError("groups sharing tensors need one page size")
    page = pages.pop()
    nslots = max(len(grp.layer_names) for grp in groups)
    tensors = []
    for slot in range(nslots):
        shared = [grp.layer_names[slot] for grp in groups if slot < len(grp.layer_names)]
        tensors.append(KVCacheTensor(size=num_blocks * page, shared_by=shared))
    return KVCacheConfig(num_blocks=num_blocks, groups=list(groups), tensors=tensors)


def num_blocks_for_budget(total_bytes, utilization, non_kv_bytes, spec, num_tensors):
    """Blocks a memory budget holds (PageAttention blog, § Memory
    Pre-allocation Logic), computed by the library: floor(total *
    utilisation) less the non-KV bytes, over one block's K+V bytes times the
    KV tensors that share the pool."""
    from . import _lib
    code = {"f32": _lib.PKV_F32, "bf16": _lib.PKV_BF16, "fp8": _lib.PKV_FP8_E4M3,
            "int4": _lib.PKV_INT4}[spec.dtype]
    n = _lib.load().pkv_num_blocks_for_budget(int(total_bytes), float(utilization), int(non_kv_bytes),
                                              int(num_tensors), spec.block_size, spec.num_kv_heads,
                                              spec.head_dim, code)
    if n < 0:
        raise ValueError("bad budget arguments (%s)" % _lib.load().pkv_status_string(int(n)).decode())
    return int(n)


def budget_config(groups, total_bytes, utilization, non_kv_bytes):
    """hybrid_config with as many blocks as the budget holds: every slot's
    tensor gets num_blocks pages."""
    nslots = max(len(grp.layer_names) for grp in groups)
    n = num_blocks_for_budget(total_bytes, utilization, non_kv_bytes, groups[0].spec, nslots)
    return hybrid_config(groups, n)


def allocate(config, device, zero=False, k_scale=1.0, v_scale=1.0):
    """Allocate every tensor as a byte buffer and return {layer: CacheView}.

    Each buffer is laid out as [2 (K, V), num_blocks, block_size, kv_heads,
    head_dim] of the layer's dtype (int4: bytes [..., head_dim / 2]); all
    layers sharing it get the same view.
    """
    views = {}
    buffers = []
    for t in config.tensors:
        alloc = torch.zeros if zero else torch.empty
        raw = alloc(t.size + ALIGN, dtype=torch.uint8, device=device)
        off = (-raw.data_ptr()) % ALIGN      # start the tensor on an ALIGN boundary
        buf = raw[off:off + t.size]
        buffers.append(buf)
        for name in t.shared_by:
            spec = config.groups[config.layer_group(name)].spec
            # The kernels need 16-byte aligned blocks; blocks of a multiple of
            # ALIGN bytes (every realistic shape) also start on ALIGN.
            if spec.block_bytes % 16:
                raise ValueError("block bytes %d are not a multiple of 16" % spec.block_bytes)
            n = 2 * config.num_blocks * spec.block_bytes
            if n > t.size:
                raise ValueError("tensor too small for layer %s" % name)
            i4 = spec.dtype == "int4"
            typed = buf[:n].view(TORCH_DTYPE[spec.dtype]).view(
                2, config.num_blocks, spec.block_size, spec.num_kv_heads,
                spec.head_dim // 2 if i4 else spec.head_dim)
            views[name] = CacheView.from_planes(typed[0], typed[1], k_scale, v_scale, int4=i4)
    return views, buffers


class PoolExhausted(RuntimeError):
    pass


class BlockPool:
    """Free physical block ids with reference counts.

    Ids are handed out in the order given (a shuffled order models a pool whose
    free list has been churned); released ids are reused first.
    """

    def __init__(self, num_blocks, order=None):
        self.num_blocks = int(num_blocks)
        order = list(range(num_blocks)) if order is None else [int(x) for x in order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of the block ids")
        self._free = order[::-1]          # stack: the next id is at the end
        self.refcount = np.zeros(num_blocks, dtype=np.int64)

    @property
    def num_free(self):
        return len(self._free)

    def allocate(self, n):
        if n > len(self._free):
            raise PoolExhausted("need %d blocks, %d free" % (n, len(self._free)))
        ids = [self._free.pop() for _ in range(n)]
        self.refcount[ids] += 1
        return ids

    def share(self, ids):
        """Another owner takes references to already-live ids."""
        for i in ids:
            if self.refcount[i] <= 0:
                raise ValueError("block %d is not live" % i)
            self.refcount[i] += 1

    def release(self, ids):
        for i in ids:
            if self.refcount[i] <= 0:
                raise ValueError("block %d released twice" % i)
            self.refcount[i] -= 1
            if self.refcount[i] == 0:
                self._free.append(i)


class GroupBlockTables:
    """Per-group, per-request logical -> physical tables over one shared pool.

    windows[g] is 0 for a full-attention group or the window W of a
    sliding-window group.  Released entries are -1.
    """

    def __init__(self, pool, windows, block_size):
        self.pool = pool
        self.windows = list(windows)
        self.block_size = int(block_size)
        self.rows = [dict() for _ in self.windows]

    def add_request(self, req):
        for g in range(len(self.windows)):
            self.rows[g][req] = []

    def grow(self, req, num_tokens):
        """Make every group's row cover positions 0 .. num_tokens - 1."""
        need = -(-int(num_tokens) // self.block_size)
        for g in range(len(self.windows)):
            row = self.rows[g][req]
            if need > len(row):
                row.extend(self.pool.allocate(need - len(row)))

    def release_out_of_window(self, req, num_computed):
        """Give back sliding-window blocks no later query can read.

        With num_computed tokens done, every later query looks back no further
        than num_computed - W + 1; blocks ending before that are dead.
        """
        for g, W in enumerate(self.windows):
            if W <= 0:
                continue
            start = int(num_computed) - W + 1
            first_live = start // self.block_size if start > 0 else 0
            row = self.rows[g][req]
            for b in range(min(first_live, len(row))):
                if row[b] >= 0:
                    self.pool.release([row[b]])
                    row[b] = -1

    def fork(self, src_req, dst_req, num_tokens):
        """Start dst_req with src_req's first num_tokens positions, sharing
        their physical blocks (Chinese worker-side page, § PagedAttention与
        Block管理: requests with a common prompt point their leading table
        entries at the same blocks, each block counting its references)."""
        need = -(-int(num_tokens) // self.block_size)
        for g in range(len(self.windows)):
            row = self.rows[g][src_req]
            if need > len(row):
                raise ValueError("request %r holds fewer than %d positions" % (src_req, num_tokens))
            shared = list(row[:need])
            self.pool.share([i for i in shared if i >= 0])
            self.rows[g][dst_req] = shared

    def prepare_write(self, req, pos_lo, pos_hi):
        """Make the blocks that positions pos_lo .. pos_hi - 1 fall in private
        to req before its tokens are written there: the row grows as needed,
        and a block other tables still reference is replaced by a fresh one.
        Returns the (old id, new id) pairs whose contents must be copied
        (pkv_copy_blocks) before the write; the old ids stay live."""
        self.grow(req, pos_hi)
        pairs = []
        lo, hi = int(pos_lo) // self.block_size, -(-int(pos_hi) // self.block_size)
        for g in range(len(self.windows)):
            row = self.rows[g][req]
            for b in range(lo, min(hi, len(row))):
                old = row[b]
                if old >= 0 and self.pool.refcount[old] > 1:
                    new = self.pool.allocate(1)[0]
                    self.pool.release([old])
                    row[b] = new
                    pairs.append((old, new))
        return pairs

    def finish(self, req):
        for g in range(len(self.windows)):
            self.pool.release([i for i in self.rows[g].pop(req) if i >= 0])

    def table(self, g, reqs, width=None):
        rows = [self.rows[g][r] for r in reqs]
        width = width or max([len(r) for r in rows] + [1])
        out = np.full((len(reqs), width), -1, dtype=np.int32)
        for i, r in enumerate(rows):
            out[i, :len(r)] = r
        return out
