"""KV-cache sizing closed forms (oracle, test-only).

Per-token KV bytes = layers * KV heads * head_dim * 2 (K and V) * element
bytes (Worker-Side KV Init (zh), § KV Cache技术背景, the LLaMA-70B worked
example: 80 layers, 8 KV heads, head_dim 128, FP16).  An FP8 cache stores one
byte per element and halves it; an INT4 cache stores half a byte and quarters
it (same section, next paragraph).

The page prints about 640 KB for that product; its factors give
80*8*128*2*2 = 327,680 bytes.  The factors are taken as authoritative; the
printed figure (and the 2.5 GB/request, 80 GB/32 requests that follow from it)
equals the product with 4-byte elements.

One physical block of one layer holds block_size tokens of K and V:
    block_size * KV heads * head_dim * 2 * element bytes.
A pool of num_blocks blocks for n layers: num_blocks * n * that.
The number of blocks a budget allows (PageAttention blog, § Memory
Pre-allocation Logic): budget = total * utilisation; available = budget -
non-KV bytes; blocks = floor(available / (bytes per block per layer * layers)).
"""

ELEMENT_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1, "int4": 0.5}
ELEMENT_BITS = {"f32": 32, "bf16": 16, "f16": 16, "fp8": 8, "int4": 4}


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype):
    bits = int(num_layers) * int(num_kv_heads) * int(head_dim) * 2 * ELEMENT_BITS[dtype]
    return bits // 8


def block_bytes(block_size, num_kv_heads, head_dim, dtype):
    """K+V bytes of one block of one layer."""
    bits = int(block_size) * int(num_kv_heads) * int(head_dim) * 2 * ELEMENT_BITS[dtype]
    return bits // 8


def pool_bytes(num_blocks, num_layers, block_size, num_kv_heads, head_dim, dtype):
    return int(num_blocks) * int(num_layers) * block_bytes(block_size, num_kv_heads, head_dim, dtype)


def num_blocks_for_budget(total_bytes, utilization, non_kv_bytes, num_layers,
                          block_size, num_kv_heads, head_dim, dtype):
    budget = int(total_bytes * utilization)
    available = budget - int(non_kv_bytes)
    if available <= 0:
        return 0
    return available // (block_bytes(block_size, num_kv_heads, head_dim, dtype) * int(num_layers))
