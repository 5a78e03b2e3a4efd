"""GPU parity at the block sizes the library accepts beyond those the
benched workloads use (2, 8, 64, 128, 256 tokens per block): decode in
the head layout (one partition, and partitions of 2048) and the row
layouts (partitions of 512), bf16 and E4M3, and chunked prefill, on
lengths at block and tile edges, against the fp64 oracle."""

import pytest
import torch

from paged_kv_cache_327_amd import workloads
from tests import test_gpu_decode as TD
from tests import test_gpu_fp8 as T8
from tests import test_gpu_prefill as TPF

pytestmark = pytest.mark.gpu

SIZES = [2, 8, 64, 128, 256]


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"


def decode_lens(b):
    return sorted({0, 1, b - 1, b, b + 1, 3 * b + 5, 513, 700, 2049})


@pytest.mark.parametrize("block_size", SIZES)
def test_decode_block_sizes(block_size):
    wl = workloads.custom(f"bsz_decode_b{block_size}", 71, 32, 8, 128, block_size, decode_lens(block_size))
    for p in (0, 512, 2048):
        TD.run_parity(wl, p, what=f"B={block_size} P={p}")


@pytest.mark.parametrize("block_size", SIZES)
def test_fp8_decode_block_sizes(block_size):
    wl = workloads.custom(f"bsz_fp8_decode_b{block_size}", 72, 32, 8, 128, block_size, decode_lens(block_size))
    for p in (0, 512, 2048):
        T8.run_parity(wl, (0.0173, 0.05), p, what=f"B={block_size} P={p}")


@pytest.mark.parametrize("block_size", SIZES)
def test_prefill_block_sizes(block_size):
    ctx = [0, block_size - 1, block_size, 100, 0, 257]
    q = [1, 33, 64, 70, 128, 5]
    lens = [c + n for c, n in zip(ctx, q)]
    wl = workloads.custom(f"bsz_prefill_b{block_size}", 73, 32, 8, 128, block_size, lens, q_lens=q)
    TPF.run_parity(wl, causal=True, what=f"B={block_size}")
    T8.run_prefill_parity(wl, (0.0173, 0.05))
