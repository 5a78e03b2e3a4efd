"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws numbers and describes workloads; it computes nothing of
the attention method itself (no slots, tables, softmax or copies).  Both
the HIP path and the CPU oracle are fed from here and from nowhere else.

Value recipe: q, k and v are drawn N(0, 1) in fp32 and rounded to bf16
(round to nearest even, as a float -> bfloat16 cast does).  bf16 travels
as uint16 bit patterns on the host.  Lengths are drawn on the host from
numpy.random.default_rng seeded with 1000 + k for workload k; physical
placement is a seeded permutation handed to the pool as its initial free
order, so every sequence's blocks are scattered through the pool.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 1000


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def seq_kv_bits(seed: int, seq: int, n_tokens: int, num_kv_heads: int, head_dim: int,
                layer: int = 0, part: int = 0):
    """K and V rows [n, Hkv, D] (bf16 bits) of one piece of one sequence:
    part 0 is its context, part 1 the tokens of the measured step.

    Each (layer, sequence, part) has its own stream, so any piece can be
    regenerated alone for a sampled check."""
    rng = np.random.default_rng([seed, 11, layer, seq, part])
    k = normal_bf16(rng, (n_tokens, num_kv_heads, head_dim))
    v = normal_bf16(rng, (n_tokens, num_kv_heads, head_dim))
    return k, v


def query_bits(seed: int, n_rows: int, num_q_heads: int, head_dim: int, layer: int = 0):
    rng = np.random.default_rng([seed, 23, layer])
    return normal_bf16(rng, (n_rows, num_q_heads, head_dim))


@dataclass
class Workload:
    """One seeded configuration.

    Every sequence first receives ``ctx_lens[i]`` context tokens (set-up),
    then ``new_lens[i]`` tokens in the measured step; attention covers all
    ``ctx_lens[i] + new_lens[i]`` tokens.  Sequences with new_lens == 1 are
    decode queries, the others prefill chunks.  ``forks`` lists (src, dst)
    sequence forks applied after the context of ``src`` is written.
    """
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    ctx_lens: list
    new_lens: list
    free_order: np.ndarray
    num_layers: int = 1
    forks: list = field(default_factory=list)
    shared_prefix: int = 0
    q_lens: list = None

    def __post_init__(self):
        if self.q_lens is None:
            self.q_lens = list(self.new_lens)

    def pieces(self, seq: int):
        """(source sequence, part, n_tokens) pieces that make up ``seq`` in
        logical order: a forked sequence starts with its source's context."""
        src = seq
        for a, b in self.forks:
            if b == seq:
                src = a
        out = []
        if self.ctx_lens[src]:
            out.append((src, 0, self.ctx_lens[src]))
        out.append((seq, 1, self.new_lens[seq]))
        return out

    def logical_kv(self, seq: int, layer: int = 0):
        ks, vs = [], []
        for src, part, n in self.pieces(seq):
            k, v = seq_kv_bits(self.seed, src, n, self.num_kv_heads, self.head_dim, layer, part)
            ks.append(k)
            vs.append(v)
        return np.concatenate(ks), np.concatenate(vs)

    def step_kv(self, seq: int, layer: int = 0):
        return seq_kv_bits(self.seed, seq, self.new_lens[seq], self.num_kv_heads, self.head_dim, layer, 1)

    def ctx_kv(self, seq: int, layer: int = 0):
        return seq_kv_bits(self.seed, seq, self.ctx_lens[seq], self.num_kv_heads, self.head_dim, layer, 0)

    def queries(self, layer: int = 0):
        """bf16 bits [sum(q_lens), Hq, D]: the step's query rows, sequence by sequence."""
        return query_bits(self.seed, int(sum(self.q_lens)), self.num_q_heads, self.head_dim, layer)

    @property
    def num_seqs(self) -> int:
        return len(self.ctx_lens)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def seq_lens(self) -> list:
        return [c + n for c, n in zip(self.ctx_lens, self.new_lens)]

    @property
    def max_seq_len(self) -> int:
        return max(self.seq_lens) if self.ctx_lens else 0


def tiny_decode() -> Workload:
    """4 sequences of lengths {1, 17, 33, 100}; 8 q heads, 2 KV heads,
    head_dim 64, B = 16, 64 physical blocks in seeded random order."""
    seed = SEED_BASE + 1
    rng = np.random.default_rng(seed)
    lens = [1, 17, 33, 100]
    return Workload("tiny_decode", seed, 8, 2, 64, 16, 64,
                    ctx_lens=[n - 1 for n in lens], new_lens=[1] * 4,
                    free_order=rng.permutation(64))


def llama_decode(seed_offset: int = 0, batch: int = 64) -> Workload:
    """Llama-3-8B-shaped decode: 32/8 heads, d 128, B 16, 8192 blocks;
    each sequence holds 512 prompt + U{0..100} generated tokens and appends
    one new token this step."""
    seed = SEED_BASE + 2 + 100 * seed_offset
    rng = np.random.default_rng(seed)
    ctx = (512 + rng.integers(0, 101, size=batch)).tolist()
    return Workload("llama3_8b_decode", seed, 32, 8, 128, 16, 8192,
                    ctx_lens=ctx, new_lens=[1] * batch,
                    free_order=rng.permutation(8192))


def long_context(num_layers: int = 32, batch: int = 8) -> Workload:
    """32-layer pool of 26,785 blocks per layer (Llama-3-8B shapes, B 16);
    8 sequences of U{16384..32768} tokens (the last token is the step's)."""
    seed = SEED_BASE + 3
    rng = np.random.default_rng(seed)
    lens = rng.integers(16384, 32769, size=batch)
    return Workload("long_context_decode", seed, 32, 8, 128, 16, 26785,
                    ctx_lens=(lens - 1).tolist(), new_lens=[1] * batch,
                    free_order=rng.permutation(26785), num_layers=num_layers)


def prefix_cow(batch: int = 256, prompt: int = 2050, num_blocks: int = 16384) -> Workload:
    """256 sequences forked from one 2050-token prompt, each then appending
    a suffix of U{1..512} tokens (its last token is the decode query)."""
    seed = SEED_BASE + 4
    rng = np.random.default_rng(seed)
    suffix = rng.integers(1, 513, size=batch).tolist()
    return Workload("prefix_cow_decode", seed, 32, 8, 128, 16, num_blocks,
                    ctx_lens=[prompt] * batch, new_lens=suffix,
                    free_order=rng.permutation(num_blocks),
                    forks=[(0, i) for i in range(1, batch)], shared_prefix=prompt,
                    q_lens=[1] * batch)


def mixed_step(block_size: int, n_chunks: int = 16, chunk: int = 512, n_decode: int = 240,
               pool_slots: int = 1 << 20) -> Workload:
    """16 prefill chunks of 512 queries over U{0..8192} context tokens plus
    240 decode sequences with lognormal lengths (median 1500, sigma 1,
    clipped to [1, 32768]); pool of 2^20 token slots."""
    seed = SEED_BASE + 5
    rng = np.random.default_rng(seed)
    ctx_p = rng.integers(0, 8193, size=n_chunks).tolist()
    dec = np.clip(np.round(rng.lognormal(np.log(1500.0), 1.0, size=n_decode)), 1, 32768)
    dec = dec.astype(np.int64).tolist()
    nb = pool_slots // block_size
    order = np.random.default_rng([seed, block_size]).permutation(nb)
    return Workload(f"mixed_step_b{block_size}", seed, 32, 8, 128, block_size, nb,
                    ctx_lens=ctx_p + [n - 1 for n in dec],
                    new_lens=[chunk] * n_chunks + [1] * n_decode,
                    free_order=order)


def custom(name: str, seed: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
           block_size: int, lens, q_lens=None, extra_blocks: int = 3, order_seed=None) -> Workload:
    """A small ad-hoc case: sequence i holds lens[i] tokens, the last
    min(q_lens[i], lens[i]) of them written in the step; q_lens[i] query rows
    (default 1 each, i.e. decode -- a sequence of length 0 still has a query)."""
    q_lens = list(q_lens) if q_lens is not None else [1] * len(lens)
    new = [min(q, n) for q, n in zip(q_lens, lens)]
    ctx = [n - q for n, q in zip(lens, new)]
    nb = sum(-(-n // block_size) for n in lens) + extra_blocks
    order = np.random.default_rng(order_seed if order_seed is not None else seed).permutation(nb)
    return Workload(name, seed, num_q_heads, num_kv_heads, head_dim, block_size, nb,
                    ctx_lens=ctx, new_lens=new, free_order=order, q_lens=q_lens)


def pool_ops(seed: int, n_ops: int = 200, max_seqs: int = 12, max_append: int = 40):
    """A replayable list of pool operations for the randomized pool test:
    ("add", s), ("append", s, n), ("fork", src, dst), ("free", s).

    Only the set of live sequence ids is tracked here (fork, add and free
    change it whether or not a later append fits)."""
    rng = np.random.default_rng([SEED_BASE, 7, seed])
    live: list[int] = []
    next_id = 0
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        if not live or (r < 0.15 and len(live) < max_seqs):
            ops.append(("add", next_id))
            live.append(next_id)
            next_id += 1
        elif r < 0.65:
            s = live[rng.integers(len(live))]
            ops.append(("append", s, int(rng.integers(1, max_append + 1))))
        elif r < 0.80 and len(live) < max_seqs:
            s = live[rng.integers(len(live))]
            ops.append(("fork", s, next_id))
            live.append(next_id)
            next_id += 1
        else:
            s = live.pop(int(rng.integers(len(live))))
            ops.append(("free", s))
    return ops


def device_seq_kv(seed: int, seq: int, n_tokens: int, num_kv_heads: int, head_dim: int,
                  layer: int = 0, part: int = 0, device="cuda"):
    """Device-side counterpart of seq_kv_bits for workloads too large to
    draw on the host: K and V [n, Hkv, D] bf16 drawn N(0, 1) by a torch
    generator seeded per (seed, layer, sequence, part).  A check copies the
    same tensors back to the host; it never redraws them with numpy."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((((seed * 131 + layer) * 1_000_003 + seq) * 7 + part) % (2**63 - 1))
    k = torch.randn((n_tokens, num_kv_heads, head_dim), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((n_tokens, num_kv_heads, head_dim), generator=g, device=device, dtype=torch.float32)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def device_query(seed: int, n_rows: int, num_q_heads: int, head_dim: int, layer: int = 0, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 977 + layer * 31 + 5) % (2**63 - 1))
    return torch.randn((n_rows, num_q_heads, head_dim), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def pool_ops_cached(seed: int, n_ops: int = 200, max_seqs: int = 10, max_append: int = 24):
    """Replayable pool operations with prefix caching, transfer pins and
    step boundaries, for the randomized pool tests:
      ("add", s), ("add_prefix", s, donor, n)  -- new sequence that asks for
        the first n tokens of sequence donor (live or finished) as a prefix,
      ("append", s, n), ("fork", src, dst), ("free", s),
      ("cache", s)  -- hash the full blocks of s,
      ("pin", s, t), ("unpin", t)  -- transfer pins,
      ("done",)  -- end of a step: pending copies and writes land.
    Only ids are tracked here; token contents are chosen by the runner."""
    rng = np.random.default_rng([SEED_BASE, 8, seed])
    live: list[int] = []
    ever: list[int] = []
    transfers: list[int] = []
    next_id = next_t = 0
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        if not live or (r < 0.10 and len(live) < max_seqs):
            ops.append(("add", next_id))
            live.append(next_id)
            ever.append(next_id)
            next_id += 1
        elif r < 0.18 and len(live) < max_seqs and ever:
            donor = ever[int(rng.integers(len(ever)))]
            ops.append(("add_prefix", next_id, donor, int(rng.integers(0, 4 * max_append))))
            live.append(next_id)
            ever.append(next_id)
            next_id += 1
        elif r < 0.48:
            s = live[int(rng.integers(len(live)))]
            ops.append(("append", s, int(rng.integers(1, max_append + 1))))
        elif r < 0.55 and len(live) < max_seqs:
            s = live[int(rng.integers(len(live)))]
            ops.append(("fork", s, next_id))
            live.append(next_id)
            ever.append(next_id)
            next_id += 1
        elif r < 0.65:
            ops.append(("cache", live[int(rng.integers(len(live)))]))
        elif r < 0.71:
            ops.append(("pin", live[int(rng.integers(len(live)))], next_t))
            transfers.append(next_t)
            next_t += 1
        elif r < 0.77 and transfers:
            ops.append(("unpin", transfers.pop(int(rng.integers(len(transfers))))))
        elif r < 0.90:
            ops.append(("done",))
        else:
            s = live.pop(int(rng.integers(len(live))))
            ops.append(("free", s))
    ops.append(("done",))
    for t in transfers:
        ops.append(("unpin", t))
    return ops


def device_rows(seed: int, tag: int, shape, device="cuda"):
    """bf16 device tensor of `shape` drawn N(0, 1) by a torch generator seeded
    per (seed, tag): step inputs (new K/V rows, queries) of the large
    workloads.  A check copies the tensor back; it never redraws it."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 2_000_003 + tag * 613 + 17) % (2**63 - 1))
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
