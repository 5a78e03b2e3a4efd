"""Comparison helpers for GPU-vs-oracle parity tests."""

import numpy as np
import torch

# Attention tolerance for bf16 storage with fp32 accumulation.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# The softmax weights enter p.v and their sum rounded to bf16 (8 significant
# bits, nearest-even: relative error <= 2^-8 each), so the sum's relative
# error is <= 2^-8 and the log-sum-exp's <= ln(1 + 2^-8) = 3.90e-3, plus
# fp32 rounding far below 1e-4.
LSE_ABS = 4e-3


def attention_errors(got: torch.Tensor, want: np.ndarray):
    g = got.float().cpu().numpy().astype(np.float64)
    assert g.shape == want.shape, (g.shape, want.shape)
    assert np.all(np.isfinite(g)), "non-finite output"
    err = np.abs(g - want)
    return float(err.max()), float(err.mean())


def assert_attention_close(got, want, max_abs=MAX_ABS, mean_abs=MEAN_ABS, what=""):
    mx, mean = attention_errors(got, want)
    assert mx <= max_abs and mean <= mean_abs, f"{what}: max abs {mx:.3g}, mean abs {mean:.3g}"
    return mx, mean


def assert_lse_close(got: torch.Tensor, want: np.ndarray, tol=LSE_ABS):
    g = got.cpu().numpy().astype(np.float64)
    finite = np.isfinite(want)
    assert np.array_equal(np.isfinite(g), finite)
    assert np.all(g[~finite] == want[~finite])
    if finite.any():
        assert np.max(np.abs(g[finite] - want[finite])) <= tol


def valid_table_prefix(table, seq_lens, block_size):
    """Rows of a block table cut to ceil(len / B) entries."""
    return [table[i, :-(-int(n) // block_size)].tolist() for i, n in enumerate(seq_lens)]
