"""KV-cache write and block copy on numpy arrays (test infrastructure only).

Both operations move bits, so they work on any dtype; bf16 caches are
passed as uint16 arrays of bit patterns and the results are bit-exact.
"""

from __future__ import annotations

import numpy as np

from oracle import fp8


PAD_SLOT = -1


def slot_mapping(block_tables: np.ndarray, query_start_loc, seq_lens, block_size: int,
                 num_tokens: int) -> np.ndarray:
    """Slots of a step's new tokens, from the block table.

    "PagedAttention: fragmentation, blocks, block tables", 3. The slot
    mapping: with one context-parallel rank the kernel's arithmetic reduces
    to slot = block_table[req][pos // B] * B + pos % B, and positions that
    have no slot get the padding id.  Request i's step tokens are rows
    query_start_loc[i] .. query_start_loc[i+1]-1 and are the last q_i of its
    seq_lens[i] positions (the attention-metadata section).

    Readings: rows past query_start_loc[-1] (padding up to num_tokens), a
    position below 0 and a table index past the row get the padding id -1.
    """
    bt = np.asarray(block_tables)
    qsl = [int(x) for x in query_start_loc]
    out = np.full(num_tokens, PAD_SLOT, dtype=np.int64)
    for i in range(len(qsl) - 1):
        q = qsl[i + 1] - qsl[i]
        first = int(seq_lens[i]) - q
        for j in range(q):
            t = qsl[i] + j
            if t >= num_tokens:
                break
            pos = first + j
            if pos < 0 or pos // block_size >= bt.shape[1]:
                continue
            out[t] = int(bt[i, pos // block_size]) * block_size + pos % block_size
    return out


def decode_append(block_tables: np.ndarray, seq_lens: np.ndarray, key_cache: np.ndarray,
                  value_cache: np.ndarray, key: np.ndarray, value: np.ndarray, slots, positions) -> None:
    """One decode token per row, written and entered into a device mirror of
    the block tables (arrays are updated in place).

    Row i's new token sits at position p = positions[i] (the row's length
    before the step, which the host pool knows) and at slot slots[i], which
    the pool returned for it.  By the slot formula
    (the pool page, 3. The slot mapping) its block is slots[i] // B and that
    block is entry p // B of the row, so the mirror learns a newly allocated
    block, and the in-place redirect of a copied tail (copy-on-write
    section), from the slot alone: table[i][p // B] = slots[i] // B.  The K/V
    rows are written as reshape_and_cache does, and seq_lens[i] becomes p + 1.

    Reading: a negative slot (the padding id) leaves row i unchanged; the row
    has room for entry p // B (the caller sizes the table).
    """
    B = key_cache.shape[1]
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        p = int(positions[i])
        block_tables[i, p // B] = int(slot) // B
        seq_lens[i] = p + 1
    reshape_and_cache(key_cache, value_cache, key, value, np.asarray(slots, dtype=np.int64))


def map_to_kernel_blocks(block_ids, blocks_per_alloc: int) -> np.ndarray:
    """Allocation-block ids -> kernel-block ids.

    "PagedAttention: fragmentation, blocks, block tables", the block-table
    append (the hybrid-blocks branch) and the decoupling paragraph: an
    allocation block of B_alloc tokens is split into k = B_alloc / B_kernel
    kernel blocks, so the allocator and the attention kernel may use
    different block sizes.  Reading: allocation block b is the same memory as
    kernel blocks b*k .. b*k + k - 1 of the cache viewed with B_kernel-token
    blocks, and every allocation id of a row expands, in order, to its k
    kernel ids (so a row of n ids becomes n*k ids).
    """
    ids = np.asarray(block_ids, dtype=np.int64).reshape(-1)
    k = int(blocks_per_alloc)
    out = []
    for b in ids:
        for j in range(k):
            out.append(int(b) * k + j)
    return np.array(out, dtype=np.int64)


def reshape_and_cache(key_cache: np.ndarray, value_cache: np.ndarray,
                      key: np.ndarray, value: np.ndarray,
                      slot_mapping: np.ndarray) -> None:
    """Write token t's K and V rows to flat row slot_mapping[t] of the cache.

    The cache is block-major [num_blocks, B, Hkv, D]; viewed as
    [num_blocks * B, Hkv, D], flat row s belongs to block s // B at offset
    s % B.  "PagedAttention: fragmentation, blocks, block tables": 3. The
    slot mapping (the padding id is written for tokens that have no slot;
    block i owns a contiguous range of the backing storage) and step 9 of
    the worked allocation (each layer's write stores the token at its flat
    row).

    Reading: a slot that is negative (the padding id, -1) or past the end
    of the pool is skipped.  Slots are unique within a call.
    """
    nb, bs, hkv, d = key_cache.shape
    assert value_cache.shape == key_cache.shape
    kflat = key_cache.reshape(nb * bs, hkv, d)
    vflat = value_cache.reshape(nb * bs, hkv, d)
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if 0 <= s < nb * bs:
            kflat[s] = key[t]
            vflat[s] = value[t]


def copy_blocks(caches, pairs, num_blocks: int) -> None:
    """cache[dst] <- cache[src] for every (src, dst) pair, whole blocks.

    Axis 0 of each cache indexes blocks; all sources are read
    before any destination is written, as the fancy-index assignment in
    the copy-on-write section of "PagedAttention: fragmentation, blocks,
    block tables" does (one block copy covers every byte of the block).

    Reading: a destination named twice, or a destination that is also a
    source, makes the result order-dependent and is rejected; ids must lie
    in [0, num_blocks).
    """
    pairs = [(int(s), int(d)) for s, d in pairs]
    srcs = [s for s, _ in pairs]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block is named twice")
    if set(dsts) & set(srcs):
        raise ValueError("a destination block is also a source")
    for b in srcs + dsts:
        if not 0 <= b < num_blocks:
            raise ValueError(f"block id {b} out of range")
    if not pairs:
        return
    for cache in caches:
        # axis 0 indexes blocks; each block row holds all of its bytes, and
        # indexing a (possibly strided) view writes through to its base
        if cache.shape[0] != num_blocks:
            raise ValueError("axis 0 of every cache must index the blocks")
        rows = cache[srcs].copy()
        cache[dsts] = rows


def reshape_and_cache_fp8(key_cache: np.ndarray, value_cache: np.ndarray,
                          key: np.ndarray, value: np.ndarray, slot_mapping: np.ndarray,
                          k_scale: float, v_scale: float) -> None:
    """The slot write of reshape_and_cache into E4M3 caches (uint8): each
    bf16 element is stored as its E4M3 code at the cache's scale
    (oracle.fp8.quantize_bf16), then written at its slot exactly as above."""
    assert key_cache.dtype == np.uint8 and value_cache.dtype == np.uint8
    reshape_and_cache(key_cache, value_cache, fp8.quantize_bf16(key, k_scale),
                      fp8.quantize_bf16(value, v_scale), slot_mapping)
