"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake in a copy of an oracle function (a
dropped term, a wrong sign, index or operand, an off-by-one in a mask or a
slot, a wrong rounding rule), swaps it in for the real one with
monkeypatch, and runs the pins of that function from the oracle's own test
modules: at least one pin must fail.  The unmutated oracle passes the same
pins (the last test), so a failure here means a pin stopped guarding
against that mistake.  Everything runs on the CPU.
"""

import numpy as np
import pytest

from oracle import attention, cache_ops, fp8, sizing
from oracle import pool_model as pm
from tests import test_oracle_attention as TA
from tests import test_oracle_cache_ops as TC
from tests import test_oracle_fp8 as TF
from tests import test_oracle_pool as TP
from tests import test_oracle_sizing as TS

_softmax = attention.softmax_attend
_gather = attention.gather_sequence
_reshape = cache_ops.reshape_and_cache
_copy = cache_ops.copy_blocks
_decode8 = fp8.decode
_hash = pm.block_hash


def _golden():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_numbers.json")
    with open(path) as f:
        return {e["name"]: e for e in json.load(f)["entries"]}


GOLDEN = _golden()

ATTENTION_PINS = [
    lambda: TF.test_decode_over_fp8_caches_equals_bf16_caches_of_the_same_values(0.25, 2.0),
    lambda: TA.test_decode_matches_torch_sdpa(16, (8, 2)),
    lambda: TA.test_decode_matches_torch_sdpa(1, (6, 1)),
    TA.test_lse_matches_scipy_logsumexp,
    lambda: TA.test_prefill_matches_torch_sdpa(True, 16),
    lambda: TA.test_prefill_matches_torch_sdpa(False, 1),
    TA.test_length_one_returns_v_exactly,
    TA.test_equal_keys_give_mean_of_values,
    TA.test_equal_values_give_that_value,
    lambda: TA.test_one_hot_key_selects_each_logical_position(3),
    TA.test_empty_sequence,
]
CACHE_PINS = [
    lambda: TF.test_decode_over_fp8_caches_equals_bf16_caches_of_the_same_values(0.25, 2.0),
    TC.test_scatter_round_trips_through_table_gather,
    TC.test_padding_and_out_of_range_slots_are_skipped,
    TC.test_copy_blocks_matches_fancy_index,
    lambda: TC.test_slot_mapping_worked_example(GOLDEN),
    TC.test_slot_mapping_agrees_with_the_pool_appends,
    TC.test_slot_mapping_padding_ids,
    TC.test_kernel_blocks_small_example,
    lambda: TC.test_decode_append_keeps_the_table_mirror_equal_to_the_pool(0),
]
FP8_PINS = [
    TF.test_decode_matches_torch_on_every_code,
    TF.test_format_fixed_points,
    TF.test_encode_round_trips_every_finite_code,
    TF.test_encode_matches_torch_on_ties_and_random_values,
    TF.test_ties_go_to_even,
    TF.test_saturation_and_nan,
    lambda: TF.test_quantize_is_fp32_product_then_torch_rounding(0.0173),
    lambda: TF.test_decode_over_fp8_caches_equals_bf16_caches_of_the_same_values(0.25, 2.0),
]
POOL_PINS = [
    TP.test_initial_order_and_pop_from_head,
    lambda: TP.test_r7_walk(GOLDEN),
    lambda: TP.test_partial_tail_copy_on_write(GOLDEN),
    TP.test_full_tail_shares_without_copy,
    lambda: TP.test_pagedkv_scenario(GOLDEN),
    TP.test_capacity_counts_copy_and_new_blocks,
    TP.test_free_puts_tail_block_at_head,
    TP.test_shared_blocks_survive_free,
    lambda: TP.test_randomized_against_list_model(0),
]

PREFIX_PINS = [
    TP.test_fnv1a_published_vectors,
    TP.test_block_hash_chain_captures_position,
    TP.test_prefix_hit_after_free_and_eviction_on_reuse,
    TP.test_duplicate_content_keeps_first_block,
    TP.test_pinned_sole_owner_copies_its_partial_tail,
    TP.test_pinned_blocks_are_not_reused_until_unpinned,
    TP.test_copy_endpoints_retained_until_copies_done,
    lambda: TP.test_randomized_prefix_cache_and_pins(0),
]
SIZING_PINS = [
    lambda: TS.test_bytes_per_token(GOLDEN),
    lambda: TS.test_pool_blocks_two_floor_divisions(GOLDEN),
    lambda: TS.test_contiguous_reservation_arithmetic(GOLDEN),
    lambda: TS.test_paged_concurrency_ceiling(GOLDEN),
    lambda: TS.test_internal_fragmentation_bound(GOLDEN),
    lambda: TS.test_table_metadata(GOLDEN),
    lambda: TS.test_r7_sizing(GOLDEN),
    lambda: TS.test_partial_hit_index(GOLDEN),
    lambda: TS.test_tail_waste_distribution(GOLDEN),
    lambda: TS.test_tail_waste_bound(16),
    lambda: TS.test_llama70b_sizing(GOLDEN),
    lambda: TS.test_lab_and_interactive(GOLDEN),
    TS.test_shared_prefix_blocks,
]


def failures(pins):
    """How many of the pins fail (an assertion, a pytest.raises that saw no
    error, or an error the mistake causes, e.g. an index error).  A
    TypeError does not count: it would mean the planted copy was called with
    arguments it does not take, not that a pin saw the mistake."""
    n = 0
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin()
        except TypeError:
            pass
        except (Exception, pytest.fail.Exception):  # noqa: BLE001 -- any other failure of a pin counts
            n += 1
    return n


# ---------------------------------------------------------------- attention


def softmax_unnormalised(q, k, v, scale, visible=None):
    x = (q @ k.T) * scale
    if visible is not None:
        x = np.where(visible, x, -np.inf)
    m = np.max(x, axis=1, keepdims=True) if x.shape[1] else np.full((x.shape[0], 1), -np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(x - m_safe)
    s = w.sum(axis=1, keepdims=True)
    out = w @ v                                          # planted: no division by the sum
    lse = (m_safe + np.log(np.where(s > 0, s, 1.0)))[:, 0]
    return out, lse


def softmax_lse_without_max(q, k, v, scale, visible=None):
    out, lse = _softmax(q, k, v, scale, visible)
    x = (q @ k.T) * scale
    if visible is not None:
        x = np.where(visible, x, -np.inf)
    m = np.max(x, axis=1) if x.shape[1] else np.zeros(x.shape[0])
    return out, np.where(np.isfinite(lse), lse - np.where(np.isfinite(m), m, 0.0), lse)   # planted


def gather_rows_reversed(cache, table_row, seq_len, kv_head, scale=1.0):
    B = cache.shape[1]
    pieces = []
    for j in range(-(-seq_len // B)):
        valid = min(B, seq_len - j * B)
        pieces.append(cache[int(table_row[j]), :valid, kv_head, :][::-1])   # planted: rows reversed
    if not pieces:
        return np.zeros((0, cache.shape[3]))
    rows = np.concatenate(pieces)
    return fp8.dequantize(rows, scale) if cache.dtype == np.uint8 else attention.bf16_to_f64(rows)


def gather_whole_last_block(cache, table_row, seq_len, kv_head, scale=1.0):
    B = cache.shape[1]
    return _gather(cache, table_row, -(-seq_len // B) * B, kv_head, scale)   # planted: tail rows read


def paged_decode_interleaved_gqa(q_bits, key_cache, value_cache, block_tables, seq_lens, scale,
                                 k_scale=1.0, v_scale=1.0):
    S, Hq, D = q_bits.shape
    Hkv = key_cache.shape[2]
    q = attention.bf16_to_f64(q_bits)
    out = np.zeros((S, Hq, D))
    lse = np.full((S, Hq), -np.inf)
    for s in range(S):
        n = int(seq_lens[s])
        for h in range(Hq):
            g = h % Hkv                                  # planted: h // (Hq / Hkv) is the reading
            k = _gather(key_cache, block_tables[s], n, g, k_scale)
            v = _gather(value_cache, block_tables[s], n, g, v_scale)
            o, l = _softmax(q[s, h][None], k, v, scale)
            out[s, h], lse[s, h] = o[0], l[0]
    return out, lse


def paged_prefill_mask(strict=False, shift=0):
    def run(q_bits, key_cache, value_cache, block_tables, query_start_loc, seq_lens, scale, causal=True,
            rows=None, k_scale=1.0, v_scale=1.0):
        Tq, Hq, D = q_bits.shape
        Hkv = key_cache.shape[2]
        G = Hq // Hkv
        q = attention.bf16_to_f64(q_bits)
        out = np.zeros((Tq, Hq, D))
        qsl = [int(x) for x in query_start_loc]
        for i in range(len(qsl) - 1):
            qi = qsl[i + 1] - qsl[i]
            n = int(seq_lens[i])
            ctx = n - qi + shift                         # planted (shift != 0)
            js = np.arange(qi)
            keys = np.arange(n)
            visible = None
            if causal:
                lim = (ctx + js)[:, None]
                visible = keys[None, :] < lim if strict else keys[None, :] <= lim   # planted (strict)
            for g in range(Hkv):
                k = _gather(key_cache, block_tables[i], n, g, k_scale)
                v = _gather(value_cache, block_tables[i], n, g, v_scale)
                for h in range(g * G, (g + 1) * G):
                    o, _ = _softmax(q[qsl[i] + js, h], k, v, scale, visible)
                    out[qsl[i] + js, h] = o
        return out
    return run


_decode_real = attention.paged_decode


def paged_decode_one_scale(q_bits, key_cache, value_cache, block_tables, seq_lens, scale, k_scale=1.0,
                           v_scale=1.0):
    return _decode_real(q_bits, key_cache, value_cache, block_tables, seq_lens, scale, k_scale,
                        k_scale)                         # planted: V read at K's scale


ATTENTION_MUTANTS = {
    "V read at K's scale": ("paged_decode", paged_decode_one_scale),
    "scale dropped": ("softmax_attend", lambda q, k, v, scale, visible=None: _softmax(q, k, v, 1.0, visible)),
    "scale squared": ("softmax_attend", lambda q, k, v, scale, visible=None: _softmax(q, k, v, scale * scale,
                                                                                     visible)),
    "keys paired with the wrong values": ("softmax_attend", lambda q, k, v, scale, visible=None:
                                          _softmax(q, np.roll(k, 1, axis=0), v, scale, visible)),
    "last key dropped": ("softmax_attend", lambda q, k, v, scale, visible=None:
                         _softmax(q, k[:-1], v[:-1], scale, None if visible is None else visible[:, :-1])
                         if k.shape[0] > 1 else _softmax(q, k, v, scale, visible)),
    "weights not normalised": ("softmax_attend", softmax_unnormalised),
    "lse without the maximum": ("softmax_attend", softmax_lse_without_max),
    "lse in log2 units": ("softmax_attend", lambda q, k, v, scale, visible=None:
                          (lambda o, l: (o, l / np.log(2.0)))(*_softmax(q, k, v, scale, visible))),
    "table entry of the next block": ("gather_sequence", lambda c, t, n, g, s=1.0:
                                      _gather(c, np.roll(np.asarray(t), -1), n, g, s)),
    "KV head 0 for every head": ("gather_sequence", lambda c, t, n, g, s=1.0: _gather(c, t, n, 0, s)),
    "rows of a block reversed": ("gather_sequence", gather_rows_reversed),
    "unwritten tail rows read": ("gather_sequence", gather_whole_last_block),
    "query heads interleaved over KV heads": ("paged_decode", paged_decode_interleaved_gqa),
    "causal mask strict": ("paged_prefill", paged_prefill_mask(strict=True)),
    "chunk placed one position late": ("paged_prefill", paged_prefill_mask(shift=1)),
    "chunk placed one position early": ("paged_prefill", paged_prefill_mask(shift=-1)),
    "bf16 bits shifted by 15": ("bf16_to_f64", lambda bits: (np.ascontiguousarray(bits).view(np.uint16)
                                                              .astype(np.uint32) << 15)
                                .view(np.float32).astype(np.float64)),
}


@pytest.mark.parametrize("name", list(ATTENTION_MUTANTS))
def test_attention_pins_catch(monkeypatch, name):
    attr, fn = ATTENTION_MUTANTS[name]
    monkeypatch.setattr(attention, attr, fn)
    assert failures(ATTENTION_PINS) > 0, name


# ---------------------------------------------------------------- cache ops


def slot_mapping_mutant(offset=True, from_front=False):
    def run(block_tables, query_start_loc, seq_lens, block_size, num_tokens):
        bt = np.asarray(block_tables)
        qsl = [int(x) for x in query_start_loc]
        out = np.full(num_tokens, -1, dtype=np.int64)
        for i in range(len(qsl) - 1):
            q = qsl[i + 1] - qsl[i]
            first = 0 if from_front else int(seq_lens[i]) - q       # planted (from_front)
            for j in range(q):
                t = qsl[i] + j
                if t >= num_tokens:
                    break
                pos = first + j
                if pos < 0 or pos // block_size >= bt.shape[1]:
                    continue
                out[t] = int(bt[i, pos // block_size]) * block_size + (pos % block_size if offset else 0)
        return out
    return run


def reshape_wrapping(key_cache, value_cache, key, value, slot_mapping):
    nb, bs, hkv, d = key_cache.shape
    kflat = key_cache.reshape(nb * bs, hkv, d)
    vflat = value_cache.reshape(nb * bs, hkv, d)
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < nb * bs:                                  # planted: the padding id -1 wraps to the last row
            kflat[s] = key[t]
            vflat[s] = value[t]


def reshape_kv_swapped(key_cache, value_cache, key, value, slot_mapping):
    _reshape(key_cache, value_cache, value, key, slot_mapping)


def copy_blocks_reversed(caches, pairs, num_blocks):
    _copy(caches, [(d, s) for s, d in pairs], num_blocks)   # planted: destination copied to source


def decode_append_length_kept(block_tables, seq_lens, key_cache, value_cache, key, value, slots, positions):
    B = key_cache.shape[1]
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        p = int(positions[i])
        block_tables[i, p // B] = int(slot) // B
        seq_lens[i] = p                                  # planted: the length does not advance
    _reshape(key_cache, value_cache, key, value, np.asarray(slots, dtype=np.int64))


def decode_append_table_kept(block_tables, seq_lens, key_cache, value_cache, key, value, slots, positions):
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot >= 0:
            seq_lens[i] = int(positions[i]) + 1          # planted: the table mirror is not updated
    _reshape(key_cache, value_cache, key, value, np.asarray(slots, dtype=np.int64))


def copy_blocks_first_cache_only(caches, pairs, num_blocks):
    _copy(list(caches)[:1], pairs, num_blocks)           # planted: the other caches are not copied


def reshape_fp8_one_scale(key_cache, value_cache, key, value, slot_mapping, k_scale, v_scale):
    _reshape(key_cache, value_cache, fp8.quantize_bf16(key, k_scale),
             fp8.quantize_bf16(value, k_scale), slot_mapping)   # planted: V written at K's scale


CACHE_MUTANTS = {
    "table mirror not updated by the append": ("decode_append", decode_append_table_kept),
    "only the first cache copied": ("copy_blocks", copy_blocks_first_cache_only),
    "V written at K's scale": ("reshape_and_cache_fp8", reshape_fp8_one_scale),
    "kernel ids reversed within a block": ("map_to_kernel_blocks", lambda ids, k: np.array(
        [int(b) * int(k) + (int(k) - 1 - j) for b in np.asarray(ids).reshape(-1) for j in range(int(k))],
        dtype=np.int64)),
    "slot without its offset in the block": ("slot_mapping", slot_mapping_mutant(offset=False)),
    "step tokens taken from the front": ("slot_mapping", slot_mapping_mutant(from_front=True)),
    "padding slot written": ("reshape_and_cache", reshape_wrapping),
    "K and V swapped": ("reshape_and_cache", reshape_kv_swapped),
    "copy direction reversed": ("copy_blocks", copy_blocks_reversed),
    "length not advanced by the append": ("decode_append", decode_append_length_kept),
    "kernel ids not scaled": ("map_to_kernel_blocks", lambda ids, k: np.array(
        [int(b) + j for b in np.asarray(ids).reshape(-1) for j in range(int(k))], dtype=np.int64)),
}


@pytest.mark.parametrize("name", list(CACHE_MUTANTS))
def test_cache_op_pins_catch(monkeypatch, name):
    attr, fn = CACHE_MUTANTS[name]
    monkeypatch.setattr(cache_ops, attr, fn)
    assert failures(CACHE_PINS) > 0, name


# ---------------------------------------------------------------- E4M3


def decode_bias(bias=7.0, implicit_one_subnormals=False):
    def run(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = c & 0x7
        sub = (1.0 + m / 8.0) * 2.0 ** -6 if implicit_one_subnormals else m * 2.0 ** -9   # planted (flag)
        mag = np.where(e == 0, sub, (1.0 + m / 8.0) * np.exp2(e - bias))                # planted (bias)
        mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
        return sign * mag
    return run


FP8_MUTANTS = {
    "exponent bias 8": ("decode", decode_bias(bias=8.0)),
    "subnormals read as normals": ("decode", decode_bias(implicit_one_subnormals=True)),
    "ties rounded up": ("_round_half_even", lambda x: np.floor(x + 0.5)),
    "ties rounded down": ("_round_half_even", lambda x: np.ceil(x - 0.5)),
    "scale multiplied instead of divided": ("reciprocal", lambda scale: np.float32(scale)),
    "dequantize ignores the scale": ("dequantize", lambda codes, scale: _decode8(codes)),
}


@pytest.mark.parametrize("name", list(FP8_MUTANTS))
def test_fp8_pins_catch(monkeypatch, name):
    attr, fn = FP8_MUTANTS[name]
    monkeypatch.setattr(fp8, attr, fn)
    assert failures(FP8_PINS) > 0, name


# ---------------------------------------------------------------- pool


def release_to_tail(self, blocks):
    first = [b for b in blocks if self.hash_of[b] is None]
    last = [b for b in blocks if self.hash_of[b] is not None]
    self.free.extend(first)                              # planted: freed blocks go to the tail
    self.free.extend(last)


def pop_from_tail(self):
    b = self.free.pop()                                  # planted: the tail, not the head
    if self.hash_of[b] is not None:
        del self.cached[self.hash_of[b]]
        self.hash_of[b] = None
    return b


def fork_without_refs(self, src, dst):
    if src not in self.tables:
        raise pm.InvalidArgument(f"unknown sequence {src}")
    if dst in self.tables:
        raise pm.InvalidArgument(f"sequence {dst} exists")
    self.tables[dst] = list(self.tables[src])            # planted: shared blocks gain no reference
    self.lens[dst] = self.lens[src]


def append_mutant(cow_when_full=False, capacity_without_copy=False, slot_off_by_one=False):
    def run(self, seq, n):
        if seq not in self.tables:
            raise pm.InvalidArgument(f"unknown sequence {seq}")
        if n <= 0:
            raise pm.InvalidArgument("n must be positive")
        B = self.block_size
        table = self.tables[seq]
        cur = self.lens[seq]
        needed = -(-(cur + n) // B) - len(table)
        partial = True if cow_when_full else cur % B != 0                 # planted (cow_when_full)
        cow = bool(table) and partial and (self.ref[table[-1]] > 1 or self.pins[table[-1]] > 0)
        extra = 0 if capacity_without_copy else int(cow)                   # planted (capacity)
        if needed + extra > len(self.free):
            raise pm.NoSpace("no space")
        pair = None
        if cow:
            src = table[-1]
            dst = self._pop()
            self.ref[dst] = 1
            self.ref[src] -= 1
            self.hold[src] += 1
            self.hold[dst] += 1
            self.pending.append((src, dst))
            table[-1] = dst
            pair = (src, dst)
        for _ in range(needed):
            b = self._pop()
            self.ref[b] = 1
            table.append(b)
        d = 1 if slot_off_by_one else 0                                    # planted (slot)
        slots = [table[(p + d) // B] * B + (p + d) % B if (p + d) // B < len(table) else table[-1] * B
                 for p in range(cur, cur + n)]
        self.lens[seq] = cur + n
        return slots, pair
    return run


def free_head_first(self, seq):
    if seq not in self.tables:
        raise pm.InvalidArgument(f"unknown sequence {seq}")
    released = []
    for b in self.tables[seq]:                           # planted: head first, not tail first
        self.ref[b] -= 1
        if not self._retained(b):
            released.append(b)
    self._release(released)
    del self.tables[seq]
    del self.lens[seq]


POOL_MUTANTS = {
    "free walks the table head first": ("free_seq", free_head_first),
    "freed blocks to the tail": ("_release", release_to_tail),
    "allocation from the tail": ("_pop", pop_from_tail),
    "fork takes no references": ("fork", fork_without_refs),
    "copy-on-write of a full shared tail": ("append", append_mutant(cow_when_full=True)),
    "capacity check ignores the copy": ("append", append_mutant(capacity_without_copy=True)),
    "slots one position late": ("append", append_mutant(slot_off_by_one=True)),
}


@pytest.mark.parametrize("name", list(POOL_MUTANTS))
def test_pool_pins_catch(monkeypatch, name):
    attr, fn = POOL_MUTANTS[name]
    monkeypatch.setattr(pm.PoolModel, attr, fn)
    assert failures(POOL_PINS) > 0, name


# ---------------------------------------------------------------- prefix cache and pins


def hash_without_parent(parent, tokens):
    return _hash(0, tokens)                              # planted: the chain's parent is dropped


def hash_two_byte_tokens(parent, tokens):
    h = pm.FNV_OFFSET
    data = (int(parent) & pm.MASK64).to_bytes(8, "little")
    for t in tokens:
        data += (int(t) & 0xFFFF).to_bytes(2, "little")   # planted: token ids as 2 bytes
    for byte in data:
        h = ((h ^ byte) * pm.FNV_PRIME) & pm.MASK64
    return h


def release_hashed_to_head(self, blocks):
    self.free.extendleft(reversed(list(blocks)))         # planted: cached blocks evicted first


def touch_keeps_free(self, b):
    self.ref[b] += 1                                     # planted: a reused cached block stays queued


def copies_done_keeps_holds(self):
    self.pending = []                                    # planted: copy endpoints never released


def pin_tail_only(self, seq, transfer):
    if seq not in self.tables:
        raise pm.InvalidArgument(f"unknown sequence {seq}")
    if transfer in self.transfers:
        raise pm.InvalidArgument(f"transfer {transfer} exists")
    blocks = list(self.tables[seq])[-1:]                 # planted: only the tail block pinned
    for b in blocks:
        self.pins[b] += 1
    self.transfers[transfer] = blocks
    return list(self.tables[seq])


def cache_blocks_last_wins(self, seq, tokens):
    if seq not in self.tables:
        raise pm.InvalidArgument(f"unknown sequence {seq}")
    B = self.block_size
    h = 0
    for j in range(len(tokens) // B):
        h = pm.block_hash(h, tokens[j * B:(j + 1) * B])
        b = self.tables[seq][j]
        if self.hash_of[b] is None:
            old = self.cached.get(h)
            if old is not None:
                self.hash_of[old] = None
            self.cached[h] = b                           # planted: a duplicate replaces the first block
            self.hash_of[b] = h


PREFIX_MUTANTS = {
    "FNV prime off by two": (pm, "FNV_PRIME", pm.FNV_PRIME + 2),
    "FNV offset basis zero": (pm, "FNV_OFFSET", 0),
    "chain parent dropped": (pm, "block_hash", hash_without_parent),
    "token ids hashed as two bytes": (pm, "block_hash", hash_two_byte_tokens),
    "cached blocks released to the head": (pm.PoolModel, "_release", release_hashed_to_head),
    "a prefix hit leaves the block queued": (pm.PoolModel, "_touch", touch_keeps_free),
    "copy endpoints never released": (pm.PoolModel, "copies_done", copies_done_keeps_holds),
    "pin covers the tail block only": (pm.PoolModel, "pin", pin_tail_only),
    "duplicate content replaces the first block": (pm.PoolModel, "cache_blocks", cache_blocks_last_wins),
}


@pytest.mark.parametrize("name", list(PREFIX_MUTANTS))
def test_prefix_cache_pins_catch(monkeypatch, name):
    target, attr, value = PREFIX_MUTANTS[name]
    monkeypatch.setattr(target, attr, value)
    assert failures(PREFIX_PINS) > 0, name


# ---------------------------------------------------------------- closed forms


SIZING_MUTANTS = {
    "K or V only": ("kv_bytes_per_token", lambda L, H, D, e: L * H * D * e),
    "pool blocks rounded up": ("blocks_for_bytes", lambda pool, bpt, B: -(-(pool // bpt) // B)),
    "blocks for tokens floored": ("blocks_for_tokens", lambda n, B: n // B),
    "tail waste as the remainder": ("tail_waste", lambda n, B: n % B),
    "shared blocks include the partial tail": ("shared_full_blocks", lambda n, B: -(-n // B)),
    "table bytes per request row": ("block_table_bytes", lambda r, m, B, ib=4: r * m * ib),
}


@pytest.mark.parametrize("name", list(SIZING_MUTANTS))
def test_sizing_pins_catch(monkeypatch, name):
    attr, fn = SIZING_MUTANTS[name]
    monkeypatch.setattr(sizing, attr, fn)
    assert failures(SIZING_PINS) > 0, name


def test_unmutated_oracle_passes_every_pin():
    for pins in (ATTENTION_PINS, CACHE_PINS, FP8_PINS, POOL_PINS, PREFIX_PINS, SIZING_PINS):
        assert failures(pins) == 0
