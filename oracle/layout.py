"""Hybrid KV groups, shared tensors and sliding-window block release (oracle).

Test-only.  Sources:

* Layers using the same attention type form a group and share one logical
  block table; a layer's *slot* is its index inside its group; the layers that
  sit in the same slot of different groups share one physical KV tensor
  (Worker-Side KV Init, § Hybrid Attention Mechanisms, § Model View: Grouping,
  § Physical View: Two KVCacheTensors -- the 4-layer example: group 0 = L0, L2
  full attention, group 1 = L1, L3 sliding window; tensor 0 holds L0 and L1,
  tensor 1 holds L2 and L3).
* Each group keeps its own logical -> physical table (Worker-Side KV Init,
  § Block Table Multi-Level Mapping Mechanism).
* A sliding-window layer only looks at the last W tokens, so blocks that fall
  wholly before the window can go back to the pool and the number of blocks
  it holds stays bounded (Worker-Side KV Init (zh), § 混合注意力机制).

Readings:

* Groups whose layers share a tensor draw physical ids from one pool, so an
  id is live in at most one group at a time (otherwise two layers of one
  tensor would write the same bytes).
* With ``nc`` tokens already computed, every later query sits at p >= nc and
  looks back to p - W + 1 >= nc - W + 1.  Logical block b is dead once its last
  position is before that: (b + 1) * bs - 1 < nc - W + 1.
* The live blocks of a step with q_len queries then cover positions
  nc - W + 1 .. nc + q_len - 1, which straddle at most
  ceil((W + q_len - 1) / bs) + 1 blocks.  The page's W / block_size is one
  short whenever the window is not block-aligned.
"""

import numpy as np


def group_slot_tensor(groups):
    """Map layer -> (group index, slot index, tensor index).

    groups: list of lists of layer names, each inner list one KV group in
    layer order.  Slot = index inside the group; tensor index = slot.
    """
    out = {}
    for g, layers in enumerate(groups):
        for slot, name in enumerate(layers):
            out[name] = (g, slot, slot)
    return out


def tensors_from_groups(groups):
    """Tensor index -> list of layers sharing it (ordered by group)."""
    mapping = group_slot_tensor(groups)
    n = max(t for (_, _, t) in mapping.values()) + 1
    tensors = [[] for _ in range(n)]
    for g, layers in enumerate(groups):
        for name in layers:
            tensors[mapping[name][2]].append(name)
    return tensors


def swa_first_live_block(num_computed, window, block_size):
    """Smallest logical block index that a future query may still read."""
    start = int(num_computed) - int(window) + 1
    if window <= 0 or start <= 0:
        return 0
    b = 0
    while (b + 1) * block_size - 1 < start:  # block b ends before the window
        b += 1
    return b


def swa_block_cap(window, q_len, block_size):
    """Most blocks a sliding-window request can hold during one step."""
    return -(-(int(window) + int(q_len) - 1) // int(block_size)) + 1


def check_group_tables(tables, seq_lens, num_computed, windows, block_size,
                       num_blocks):
    """Validate hybrid block tables; raise AssertionError on any violation.

    tables:       list over groups of int[R, max_blocks] (-1 = no block)
    seq_lens:     int[R] tokens including this step's
    num_computed: int[R] tokens cached before this step
    windows:      per group, 0 for full attention or W
    Checks: every block a query of this step can read is present and in range;
    every sliding-window block before the first live one has been released
    (-1); no entry exists past the blocks the sequence needs; no physical id
    is used twice across all groups and requests; live SWA rows respect the cap.
    """
    used = {}
    for g, (bt, W) in enumerate(zip(tables, windows)):
        bt = np.asarray(bt)
        for r, L in enumerate(np.asarray(seq_lens)):
            L = int(L)
            nc = int(num_computed[r])
            need = -(-L // block_size)
            first = swa_first_live_block(nc, W, block_size) if W > 0 else 0
            row = bt[r]
            for b in range(len(row)):
                phys = int(row[b])
                if b < first or b >= need:
                    assert phys == -1, (g, r, b, phys, "should be released/empty")
                    continue
                assert 0 <= phys < num_blocks, (g, r, b, phys, "missing block")
                assert phys not in used, (g, r, b, phys, "id used twice", used.get(phys))
                used[phys] = (g, r, b)
            if W > 0:
                live = need - first
                assert live <= swa_block_cap(W, L - nc, block_size), (g, r, live)
    return used
