"""Pins of the oracle's closed forms against the numbers the pages print
(tests/golden/page_numbers.json carries each value with its citation)."""

import math

import pytest

from oracle import sizing

GiB = 1 << 30
MiB = 1 << 20
KiB = 1 << 10


def _r(x, nd):
    return round(x, nd)


def test_bytes_per_token(golden):
    for name in ("llama3_8b_kv_bytes_per_token", "llama70b_kv_bytes_per_token"):
        e = golden[name]
        i = e["inputs"]
        got = sizing.kv_bytes_per_token(i["layers"], i["kv_heads"], i["head_dim"], i["elem_bytes"])
        assert got == e["printed"], name
    assert sizing.kv_bytes_per_token(32, 8, 128, 2) == 128 * KiB


def test_pool_blocks_two_floor_divisions(golden):
    bpt = sizing.kv_bytes_per_token(32, 8, 128, 2)
    blocks = golden["pool_blocks_b16"]["printed"]
    slots = golden["pool_token_slots_b16"]["printed"]
    assert blocks * 16 == slots
    # The printed 52.32 GiB is rounded: a pool of 52.3155 GiB prints as
    # 52.32 and yields the printed block count, 52.32 GiB exactly does not.
    pool = int(52.3155 * GiB)
    assert _r(pool / GiB, 2) == golden["pool_gib"]["printed"]
    assert sizing.blocks_for_bytes(pool, bpt, 16) == blocks
    # every pool in [slots, slots + 16) tokens gives the same count
    assert sizing.blocks_for_bytes(slots * bpt, bpt, 16) == blocks
    assert sizing.blocks_for_bytes((slots + 16) * bpt - 1, bpt, 16) == blocks
    assert sizing.blocks_for_bytes((slots + 16) * bpt, bpt, 16) == blocks + 1
    assert sizing.blocks_for_bytes(slots * bpt - 1, bpt, 16) == blocks - 1


def test_contiguous_reservation_arithmetic(golden):
    bpt = sizing.kv_bytes_per_token(32, 8, 128, 2)
    maxlen = golden["max_model_len"]["printed"]
    assert maxlen * bpt == golden["reservation_gib"]["printed"] * GiB
    pool = golden["pool_gib"]["printed"] * GiB
    assert math.floor(pool / (maxlen * bpt)) == golden["reservations_that_fit"]["printed"]
    n = golden["chat_turn_tokens"]["printed"]
    assert n * bpt / MiB == golden["chat_turn_mib"]["printed"]
    assert _r(13 * n * bpt / GiB, 2) == golden["thirteen_live_gib"]["printed"]
    waste = sizing.contiguous_waste(n, maxlen) / maxlen
    assert _r(100 * waste, 2) == golden["reservation_waste_pct"]["printed"]


def test_paged_concurrency_ceiling(golden):
    blocks = golden["pool_blocks_b16"]["printed"]
    per_seq = sizing.blocks_for_tokens(golden["chat_turn_tokens"]["printed"], 16)
    assert per_seq == 39
    assert blocks // per_seq == golden["paged_concurrency_612"]["printed"]


def test_internal_fragmentation_bound(golden):
    bpt = sizing.kv_bytes_per_token(32, 8, 128, 2)
    for b, mib_name, gib_name, pct_name, nd in (
            (16, "tail_max_mib_b16", "tail_total_gib_b16_686", "tail_pct_b16_686", 1),
            (128, "tail_max_mib_b128", "tail_total_gib_b128_686", "tail_pct_b128_686", 0)):
        worst = max(sizing.tail_waste(n, b) for n in range(1, 4 * b))
        assert worst == b - 1
        assert worst * bpt / MiB == golden[mib_name]["printed"]
        total = 686 * worst * bpt
        assert _r(total / GiB, 1) == golden[gib_name]["printed"]
        pct = 100 * total / (golden["pool_gib"]["printed"] * GiB)
        assert _r(pct, nd) == golden[pct_name]["printed"]


def test_table_metadata(golden):
    e = golden["block_table_mib"]
    i = e["inputs"]
    assert sizing.block_table_bytes(i["num_reqs"], i["max_len"], i["block_size"]) == e["printed"] * MiB
    e = golden["req_to_token_mib"]
    i = e["inputs"]
    got = sizing.block_table_bytes(i["num_reqs"], i["max_len"], i["block_size"])
    assert _r(got / MiB, 1) == e["printed"]
    assert 16 * sizing.kv_bytes_per_token(32, 8, 128, 2) == golden["all_layer_block_mib"]["printed"] * MiB


def test_r7_sizing(golden):
    e = golden["r7_walk"]["printed"]
    req = sizing.blocks_for_tokens(e["committed"] + e["new"], e["block_size"])
    assert req == e["required"]
    assert sizing.blocks_for_tokens(e["committed"], e["block_size"]) == e["held"]
    assert max(req - e["held"], 0) == e["to_allocate"]


def test_partial_hit_index(golden):
    e = golden["partial_hit_4100"]["printed"]
    assert e["tokens"] // e["block_size"] == e["tail_index"]
    assert e["tokens"] % e["block_size"] == e["valid_slots"]
    assert sizing.tail_waste(e["tokens"], e["block_size"]) == e["block_size"] - e["valid_slots"]


def test_tail_waste_distribution(golden):
    e = golden["tail_waste_distribution"]["printed"]
    b = e["block_size"]
    got = [sizing.tail_waste(n, b) for n in e["lengths"]]
    assert got == e["waste"]
    assert got == [(b - n % b) % b for n in e["lengths"]]
    assert sizing.expected_tail_waste(e["lengths"], [0.25] * 4, b) == e["mean"]
    # uniform residues give (B - 1) / 2
    for bb in (1, 4, 16, 32):
        mean = sizing.expected_tail_waste(range(1, bb + 1), [1.0 / bb] * bb, bb)
        assert mean == pytest.approx((bb - 1) / 2)


@pytest.mark.parametrize("b", [1, 2, 4, 16, 32, 128])
def test_tail_waste_bound(b):
    for n in range(0, 5 * b + 3):
        w = sizing.tail_waste(n, b)
        assert 0 <= w < b
        assert (n + w) % b == 0
        assert sizing.blocks_for_tokens(n, b) * b == n + w
    assert sizing.tail_waste(0, b) == 0 and sizing.blocks_for_tokens(0, b) == 0


def test_llama70b_sizing(golden):
    bpt = sizing.kv_bytes_per_token(80, 8, 128, 2)
    # 16 x 327,680 B is exactly 5 MiB; the page prints 16 x 320 "KB" = 5.12 "MB"
    assert 16 * bpt == 5 * MiB
    assert 16 * (bpt // KiB) / 1000 == golden["llama70b_block_mb"]["printed"]
    tokens = 120 * 10**9 // bpt
    assert abs(tokens - golden["llama70b_tokens_in_120gb"]["printed"]) / tokens < 1e-3
    blocks = sizing.blocks_for_bytes(120 * 10**9, bpt, 16)
    assert blocks == 22888
    assert round(blocks, -2) == golden["llama70b_blocks_in_120gb"]["printed"]
    e = golden["llama70b_requests_4k"]
    assert sizing.blocks_for_tokens(e["inputs"]["context"], 16) == e["inputs"]["blocks_each"]
    assert round(blocks // e["inputs"]["blocks_each"], -1) == e["printed"]
    e = golden["half_block_residual_pct"]
    half = e["inputs"]["block_size"] / 2
    assert 100 * half / e["inputs"]["seq_len"] == e["printed"]


def test_lab_and_interactive(golden):
    e = golden["lab_blocks"]["printed"]
    assert e["blocks"] * 16 == e["slots"]
    assert sizing.blocks_for_tokens(e["prompt"], 16) == e["blocks_per_prompt"]
    e = golden["interactive_step0"]["printed"]
    assert e["pool_blocks"] * e["block_size"] == e["pool_tokens"]
    n = e["slab"] - e["contiguous_waste"]          # tokens of request #0
    assert sizing.contiguous_waste(n, e["slab"]) == e["contiguous_waste"]
    assert sizing.blocks_for_tokens(n, e["block_size"]) == e["blocks_used"]
    assert sizing.tail_waste(n, e["block_size"]) == e["paged_slack"]


def test_shared_prefix_blocks():
    # the prefix-sharing workload: a 2050-token prompt at B = 16
    assert sizing.shared_full_blocks(2050, 16) == 128
    assert sizing.blocks_for_tokens(2050, 16) == 129
    assert 2050 - 16 * sizing.shared_full_blocks(2050, 16) == 2


def test_bad_sizes_rejected():
    with pytest.raises(ValueError):
        sizing.blocks_for_bytes(10, 0, 16)
    with pytest.raises(ValueError):
        sizing.blocks_for_tokens(-1, 16)
