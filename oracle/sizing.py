"""Closed forms of the pages' capacity arithmetic (test infrastructure only).

Each function is the definition the pages state, written out with Python
integers (exact) or floats where the pages print a ratio.
"""

from __future__ import annotations


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    """KV bytes per token = 2 * L * h_kv * d * s.

    The factor 2 is one K and one V vector per layer and KV head.
    "The pantry of pigeonholes", "The maths that matter" (first formula);
    the first page's budget paragraph uses the same quantity (128 KiB/token
    for Llama-3-8B), its formula being lost from the extracted text.
    """
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def blocks_for_bytes(pool_bytes: int, bytes_per_token: int, block_size: int) -> int:
    """Blocks that fit in a pool: two floor divisions, bytes -> tokens -> blocks.

    "PagedAttention: fragmentation, blocks, block tables", budget paragraph
    (52.32 GiB carved into 16-token blocks).
    """
    if bytes_per_token <= 0 or block_size <= 0 or pool_bytes < 0:
        raise ValueError("sizes must be positive")
    return (pool_bytes // bytes_per_token) // block_size


def blocks_for_tokens(n: int, block_size: int) -> int:
    """A sequence of n tokens occupies ceil(n / B) blocks.

    "Memory management", Maths; the first page's slot-mapping walk
    (cdiv(4097, 16) = 257).
    """
    if n < 0 or block_size <= 0:
        raise ValueError("n >= 0 and B > 0 required")
    return -(-n // block_size)


def tail_waste(n: int, block_size: int) -> int:
    """Unused slots of the last block: B * ceil(n / B) - n (< B).

    "Memory management", Maths; equals (B - n % B) % B as in the first
    page's tail-waste paragraph.
    """
    return block_size * blocks_for_tokens(n, block_size) - n


def expected_tail_waste(lengths, probs, block_size: int) -> float:
    """Expected tail waste: sum over lengths of p * ((B - n % B) % B).

    First page, "Tail waste has a distribution".
    """
    return float(sum(p * ((block_size - n % block_size) % block_size)
                     for n, p in zip(lengths, probs)))


def contiguous_waste(n: int, n_max: int) -> int:
    """Slots wasted by a contiguous reservation of n_max for n tokens.

    "Memory management", Maths (n_max - n).
    """
    return n_max - n


def shared_full_blocks(prefix_len: int, block_size: int) -> int:
    """Full blocks shared outright by sequences with a common prefix: floor(p / B).

    "Memory management", Maths (the tail block is copied on first write).
    """
    return prefix_len // block_size


def block_table_bytes(num_reqs: int, max_len: int, block_size: int,
                      index_bytes: int = 4) -> int:
    """Bytes of a rectangular [num_reqs, ceil(max_len / B)] index table.

    First page, "2. The block table" (256 x 2048 x 4 B = 2 MiB); with B = 1
    and one padding row it is SGLang's req_to_token (257 x 32768 x 4 B).
    """
    return num_reqs * blocks_for_tokens(max_len, block_size) * index_bytes
