"""Pins of the E4M3 oracle (oracle.fp8) and of the oracle's attention over
E4M3 caches: torch's float8_e4m3fn conversion (a library routine, round to
nearest even) on every code and on values across the whole range, the
format's fixed points, saturation, the rounding error bound, and exact
agreement with bf16 caches holding the same values."""

import numpy as np
import pytest
import torch

from oracle import attention, cache_ops, fp8

ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(values):
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_matches_torch_on_every_code():
    got, want = fp8.decode(ALL), torch_decode(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_format_fixed_points():
    d = fp8.decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0x80, 0xFE, 0x7F, 0xFF], dtype=np.uint8))
    assert d[0] == 0 and d[1] == 2.0 ** -9 and d[2] == 7 * 2.0 ** -9 and d[3] == 2.0 ** -6
    assert d[4] == 1.0 and d[5] == 448.0 and d[6] == 0 and np.signbit(d[6]) and d[7] == -448.0
    assert np.isnan(d[8]) and np.isnan(d[9])
    assert np.nanmax(np.abs(fp8.decode(ALL))) == fp8.MAX_FINITE


def test_encode_round_trips_every_finite_code():
    finite = ALL[~np.isnan(fp8.decode(ALL))]
    assert np.array_equal(fp8.encode(fp8.decode(finite)), finite)


def test_encode_matches_torch_on_ties_and_random_values():
    pos = np.sort(np.unique(fp8.decode(ALL[:0x7F])))               # 0 .. 448
    mids = (pos[1:] + pos[:-1]) / 2                                 # every tie
    rng = np.random.default_rng(5)
    rand = np.concatenate([
        rng.uniform(-464, 464, 20000),
        rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, 20000)),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000),                 # subnormal range
    ]).astype(np.float32)
    rand = rand[np.abs(rand) <= 464]                                # torch gives NaN beyond
    vals = np.concatenate([pos, -pos, mids, -mids, rand, [464.0, -464.0]]).astype(np.float32)
    assert np.array_equal(fp8.encode(vals), torch_encode(vals))


def test_ties_go_to_even():
    e = fp8.encode(np.array([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -10, 3 * 2.0 ** -10], dtype=np.float32))
    assert e.tolist() == [0x38, 0x3A, 0x00, 0x01, 0x02]


def test_saturation_and_nan():
    e = fp8.encode(np.array([465.0, 1e6, np.inf, -np.inf, -500.0, np.nan], dtype=np.float32))
    assert e[:5].tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert e[5] & 0x7F == 0x7F


def test_rounding_error_bound():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(50000) * np.exp2(rng.integers(-10, 8, 50000))).astype(np.float32).astype(np.float64)
    x = x[np.abs(x) <= 448]
    err = np.abs(fp8.decode(fp8.encode(x)) - x)
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4)       # half of 2^-3 relative
    assert np.all(err[~normal] <= 2.0 ** -10)                         # half the subnormal step
    y = np.sort(x)
    assert np.all(np.diff(fp8.decode(fp8.encode(y))) >= 0)            # monotone


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 0.0173])
def test_quantize_is_fp32_product_then_torch_rounding(scale):
    rng = np.random.default_rng([7, int(scale * 1e4)])
    x = rng.standard_normal(20000).astype(np.float32) * 3
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xb = (bits.astype(np.uint32) << 16).view(np.float32)
    prod = (torch.from_numpy(xb) * torch.tensor(np.float32(1.0) / np.float32(scale))).numpy()
    ok = np.abs(prod) <= 464
    assert np.array_equal(fp8.quantize_bf16(bits, scale)[ok], torch_encode(prod[ok]))
    assert np.all(fp8.quantize_bf16(bits, scale)[~ok] & 0x7F == 0x7E)
    if scale == 0.5:
        assert fp8.quantize_bf16(np.array([0x4040], dtype=np.uint16), 0.5)[0] == 0x4C   # 3.0 / 0.5 = 6
        assert fp8.dequantize(np.array([0x4C], dtype=np.uint8), 0.5)[0] == 3.0


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.25, 2.0)])
def test_decode_over_fp8_caches_equals_bf16_caches_of_the_same_values(k_scale, v_scale):
    """With power-of-two scales every dequantised value is a bf16 value, so
    attention over the E4M3 caches must equal attention over bf16 caches
    holding those values, bit for bit."""
    rng = np.random.default_rng(8)
    nb, bs, hkv, d, S, hq = 12, 4, 2, 64, 3, 4
    kc8 = np.zeros((nb, bs, hkv, d), dtype=np.uint8)
    vc8 = kc8.copy()
    lens = [7, 1, 13]
    order = rng.permutation(nb)
    table = np.full((S, 4), 0, dtype=np.int32)
    slots, used = [], 0
    for s, n in enumerate(lens):
        blocks = order[used:used + -(-n // bs)]
        used += len(blocks)
        table[s, :len(blocks)] = blocks
        slots.append([blocks[p // bs] * bs + p % bs for p in range(n)])
    for s, n in enumerate(lens):
        k = (rng.standard_normal((n, hkv, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        v = (rng.standard_normal((n, hkv, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        cache_ops.reshape_and_cache_fp8(kc8, vc8, k, v, np.array(slots[s]), k_scale, v_scale)
        # each cache's codes are torch's E4M3 of value * fp32(1 / its own scale)
        for cache, bits, sc in ((kc8, k, k_scale), (vc8, v, v_scale)):
            x = torch.from_numpy((bits.astype(np.uint32) << 16).view(np.float32))
            want = (x * torch.tensor(np.float32(1.0) / np.float32(sc))).to(torch.float8_e4m3fn)
            got = cache.reshape(nb * bs, hkv, d)[np.array(slots[s])]
            assert np.array_equal(got, want.view(torch.uint8).numpy())

    def to_bf16_bits(codes, scale):
        f = (fp8.decode(codes) * scale).astype(np.float32)
        assert np.array_equal(f.astype(np.float64), fp8.decode(codes) * scale)
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    kcb, vcb = to_bf16_bits(kc8, k_scale), to_bf16_bits(vc8, v_scale)
    q = (rng.standard_normal((S, hq, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    o8, l8 = attention.paged_decode(q, kc8, vc8, table, lens, 0.125, k_scale, v_scale)
    ob, lb = attention.paged_decode(q, kcb, vcb, table, lens, 0.125)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)
    # and chunked prefill: each sequence's last 3 (or fewer) positions as queries
    ql = [min(3, n) for n in lens]
    qsl = np.concatenate([[0], np.cumsum(ql)])
    qp = (rng.standard_normal((int(qsl[-1]), hq, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    p8 = attention.paged_prefill(qp, kc8, vc8, table, qsl, lens, 0.125, k_scale=k_scale, v_scale=v_scale)
    pb = attention.paged_prefill(qp, kcb, vcb, table, qsl, lens, 0.125)
    assert np.array_equal(p8, pb)
    # and the E4M3 write touched only the written slots
    written = np.zeros(nb * bs, dtype=bool)
    written[np.concatenate([np.array(x) for x in slots])] = True
    assert np.all(kc8.reshape(nb * bs, -1)[~written] == 0)
