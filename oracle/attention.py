"""fp64 paged attention by explicit block-table gather (test infrastructure only).

For every sequence the oracle walks its block-table row in logical order
for ceil(len / B) entries, copies the valid rows of each physical block
into one contiguous K (and V) matrix, converts bf16 to fp64 exactly, and
computes softmax(q K^T * scale) V in fp64.

Sources
  * "PagedAttention: fragmentation, blocks, block tables": the attention
    metadata section (block_table [num_reqs, W] int32; the kernel gathers
    past K/V by walking row r for ceil(seq_lens[r] / B) entries; seq_lens
    counts the computed tokens; query_start_loc delimits each request's
    queries) and the VM-analogy paragraph (a straight gather, lookup per
    query).
  * "The pantry of pigeonholes", "The mechanism": the attention kernel
    visits a sequence's physical blocks in logical order, so the gathered
    K and V behave like one contiguous sequence.
  * "Memory management", Concept: the kernel follows the block table to
    gather keys and values.

Readings where the pages are silent
  * GQA grouping is contiguous: query head h reads KV head h // (Hq / Hkv).
  * seq_lens includes the tokens written in the current step.
  * A chunk of q_i queries of a sequence of length L sits at positions
    L - q_i .. L - 1; with the causal mask query j sees keys 0 .. L - q_i + j.
  * A sequence of length 0 yields a zero output and lse = -inf.
"""

from __future__ import annotations

import numpy as np

from oracle import fp8


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp64: a bf16 pattern is the upper half of an fp32."""
    u = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def gather_sequence(cache: np.ndarray, table_row, seq_len: int, kv_head: int,
                    scale: float = 1.0) -> np.ndarray:
    """Contiguous [seq_len, D] fp64 rows of one KV head, gathered through the
    table: logical position p is row p % B of physical block table_row[p // B].

    A uint16 cache holds bf16 bits (scale must be 1); a uint8 cache holds
    E4M3 codes whose values are decode(code) * scale (oracle.fp8)."""
    B = cache.shape[1]
    nblk = -(-seq_len // B)
    pieces = []
    for j in range(nblk):
        blk = int(table_row[j])
        valid = min(B, seq_len - j * B)
        pieces.append(cache[blk, :valid, kv_head, :])
    if not pieces:
        return np.zeros((0, cache.shape[3]), dtype=np.float64)
    rows = np.concatenate(pieces, axis=0)
    if cache.dtype == np.uint8:
        return fp8.dequantize(rows, scale)
    assert scale == 1.0, "a bf16 cache has no scale"
    return bf16_to_f64(rows)


def softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   visible: np.ndarray | None = None):
    """out = softmax(q k^T * scale) v and lse = log sum exp(q k^T * scale).

    q [M, D], k and v [N, D] fp64; visible [M, N] bool masks keys out.
    A row that sees no key gets out = 0 and lse = -inf.
    """
    x = (q @ k.T) * scale
    if visible is not None:
        x = np.where(visible, x, -np.inf)
    m = np.max(x, axis=1, keepdims=True) if x.shape[1] else np.full((x.shape[0], 1), -np.inf)
    empty = ~np.isfinite(m[:, 0])
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(x - m_safe)
    s = w.sum(axis=1, keepdims=True)
    s_safe = np.where(s > 0, s, 1.0)
    out = (w @ v) / s_safe
    lse = (m_safe + np.log(s_safe))[:, 0]
    out[empty] = 0.0
    lse[empty] = -np.inf
    return out, lse


def paged_decode(q_bits: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                 block_tables: np.ndarray, seq_lens, scale: float,
                 k_scale: float = 1.0, v_scale: float = 1.0):
    """Single-query attention per sequence over its paged K/V.

    q_bits [S, Hq, D] bf16 bits; caches [NB, B, Hkv, D] bf16 bits, or E4M3
    codes (uint8) with per-cache scales k_scale / v_scale;
    block_tables [S, W] int32; seq_lens [S].
    Returns out [S, Hq, D] fp64 and lse [S, Hq] fp64.
    """
    S, Hq, D = q_bits.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    q = bf16_to_f64(q_bits)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    lse = np.full((S, Hq), -np.inf, dtype=np.float64)
    for s in range(S):
        n = int(seq_lens[s])
        for g in range(Hkv):
            k = gather_sequence(key_cache, block_tables[s], n, g, k_scale)
            v = gather_sequence(value_cache, block_tables[s], n, g, v_scale)
            heads = slice(g * G, (g + 1) * G)
            o, l = softmax_attend(q[s, heads], k, v, scale)
            out[s, heads] = o
            lse[s, heads] = l
    return out, lse


def paged_prefill(q_bits: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                  block_tables: np.ndarray, query_start_loc, seq_lens, scale: float,
                  causal: bool = True, rows=None, k_scale: float = 1.0, v_scale: float = 1.0):
    """Chunked-prefill attention: request i's queries are rows
    query_start_loc[i] .. query_start_loc[i+1]-1 of q and occupy the last
    q_i positions of its seq_lens[i] tokens.

    q_bits [Tq, Hq, D]; caches bf16 bits, or E4M3 codes (uint8) with
    per-cache scales k_scale / v_scale; returns out [Tq, Hq, D] fp64 (rows
    not computed stay zero).  ``rows`` optionally restricts the computation
    to a set of (request, query row within request) pairs.
    """
    Tq, Hq, D = q_bits.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    q = bf16_to_f64(q_bits)
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    qsl = [int(x) for x in query_start_loc]
    want = None
    if rows is not None:
        want = {}
        for i, j in rows:
            want.setdefault(int(i), []).append(int(j))
    for i in range(len(qsl) - 1):
        if want is not None and i not in want:
            continue
        qi = qsl[i + 1] - qsl[i]
        n = int(seq_lens[i])
        ctx = n - qi
        js = np.arange(qi) if want is None else np.array(sorted(set(want[i])))
        if js.size == 0:
            continue
        keys = np.arange(n)
        visible = None
        if causal:
            visible = keys[None, :] <= (ctx + js)[:, None]
        for g in range(Hkv):
            k = gather_sequence(key_cache, block_tables[i], n, g, k_scale)
            v = gather_sequence(value_cache, block_tables[i], n, g, v_scale)
            for h in range(g * G, (g + 1) * G):
                o, _ = softmax_attend(q[qsl[i] + js, h], k, v, scale, visible)
                out[qsl[i] + js, h] = o
    return out
