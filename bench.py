"""Benchmark of the paged-attention decode step on one MI355X.

One step is the whole path for one batch:
  1. the host pool appends one token to each of the 64 sequences (new block
     ids, slots, copy-on-write pairs);
  2. pending copy-on-write block copies run (none arise in this workload);
  3. one pa_paged_decode_append launch writes the step's new K/V rows to
     their slots, updates the device block tables and lengths from the
     slots, which travel in the kernel arguments (the tables were copied to
     the device once, at set-up; no metadata moves host -> device per step),
     and runs paged decode (partition pass, plus the log-sum-exp merge when a
     sequence spans several partitions) over the cache.

Workload: Llama-3-8B-shaped decode (32 query / 8 KV heads, head_dim 128,
bf16, block_size 16), batch 64, each sequence 512 prompt + U{0..100}
generated tokens (+1 per step), 8192-block pool per instance with seeded
random placement, values ~N(0, 1).  Several independent instances are used
round-robin so that a step never finds its 141 MiB of K/V still in the
256 MiB last-level cache from the step before.

Prints one JSON line.  --gpus above 1 is refused: this build runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
METRIC = "paged decode KV-read GB/s (% of HBM peak) + seqs/s; prefill TFLOP/s"
DECODE_KERNEL = "decode_partition_kernel<128, 4, true, false, false>"  # D, G, B >= 16, E4M3, appending
COUNTERS = os.path.join(ROOT, "profiles", "decode_partition_llama3_8b_traffic.txt")
COPY_CALIBRATION_BYTES = 512 << 20


def decode_source_hash():
    h = hashlib.sha256()
    for rel in ("paged_kv_cache_327_amd/csrc/kernels/paged_decode.hip",
                "paged_kv_cache_327_amd/csrc/kernels/common.hpp"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kv_bytes(seq_lens, num_kv_heads, head_dim, elem_bytes=2):
    """K and V rows of every attended token (bf16, or 1-byte E4M3)."""
    return int(np.sum(np.asarray(seq_lens, dtype=np.int64))) * 2 * num_kv_heads * head_dim * elem_bytes


def decode_bytes(seq_lens, num_q_heads, num_kv_heads, head_dim, block_size, elem_bytes=2):
    """Algorithmic bytes of one decode call: K/V rows (elem_bytes per
    element), q in and out (bf16) and the block-table entries walked."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    qo = len(seq_lens) * num_q_heads * head_dim * 2 * 2
    table = int(np.sum(-(-seq_lens // block_size))) * 4
    return kv_bytes(seq_lens, num_kv_heads, head_dim, elem_bytes) + qo + table


class Instance:
    """One pool with its caches and the step's inputs.

    The device block tables and lengths are copied to the GPU once, at
    set-up.  Every step after that updates them on the device:
    pa_paged_decode_append writes the new tokens, learns new blocks (and
    copy-on-write redirects) from their slots, which travel in the kernel
    arguments with the positions, and decodes, so a step moves no metadata
    from host to device and launches one kernel (plus the merge when a
    sequence spans several partitions)."""

    def __init__(self, wl, torch, B, hip_side, workloads, max_seq_len, partition_size, workspace):
        self.wl = wl
        S = wl.num_seqs
        self.S = S
        self.width = -(-max_seq_len // wl.block_size)
        self.state = hip_side.HipStep(wl, bt_width=self.width)   # set-up: contexts + one step's token
        self.d_table = self.state.table_dev
        self.d_lens = self.state.seq_lens_dev
        self.h_lens = self.state.seq_lens.astype(np.int64).copy()  # host copy of the lengths, for the byte count
        rng = np.random.default_rng([wl.seed, 99])
        self.new_k = hip_side.to_device(workloads.normal_bf16(rng, (S, wl.num_kv_heads, wl.head_dim)))
        self.new_v = hip_side.to_device(workloads.normal_bf16(rng, (S, wl.num_kv_heads, wl.head_dim)))
        self.q = hip_side.to_device(workloads.normal_bf16(rng, (S, wl.num_q_heads, wl.head_dim)))
        self.out = torch.empty_like(self.q)
        self.seq_ids = np.arange(S, dtype=np.int64)
        self.ones = np.ones(S, dtype=np.int32)
        self.h_slots = np.empty(S, dtype=np.int64)
        self.h_pos = np.empty(S, dtype=np.int32)         # each row's length before the step
        self.pairs = np.empty((S, 2), dtype=np.int32)
        self.done = B.c_i32(0)
        kc, vc = self.state.kc, self.state.vc
        L = B.lib()
        self.lib = L
        # argument tuples of the C calls (validated once by the binding's
        # checks in HipStep; the pointers do not change)
        self.append_args = (self.state.pool.handle, self.seq_ids.ctypes.data_as(B.P_i64),
                            self.ones.ctypes.data_as(B.P_i32), S,
                            self.h_slots.ctypes.data_as(B.P_i64), self.pairs.ctypes.data_as(B.P_i32),
                            B.ctypes.byref(self.done))
        bstride = kc.stride(0)
        self.decode_args = (self.out.data_ptr(), None, self.q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bstride,
                            wl.num_blocks, self.d_table.data_ptr(), self.width, self.d_lens.data_ptr(), S,
                            wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, max_seq_len,
                            partition_size, wl.scale, workspace.data_ptr(), workspace.numel())
        # the step: new tokens written, tables updated and decode, one launch
        self.step_args = (self.out.data_ptr(), None, self.q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bstride,
                          wl.num_blocks, self.d_table.data_ptr(), self.width, self.d_lens.data_ptr(), S,
                          wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, max_seq_len,
                          partition_size, wl.scale, self.new_k.data_ptr(), self.new_k.stride(0),
                          self.new_v.data_ptr(), self.new_v.stride(0), self.h_slots.ctypes.data_as(B.P_i64),
                          self.h_pos.ctypes.data_as(B.P_i32), workspace.data_ptr(), workspace.numel())

    def decode(self, stream):
        rc = self.lib.pa_paged_decode(*self.decode_args, stream)
        if rc != 0:
            raise RuntimeError(self.lib.pa_last_error().decode())


def run_step(inst, B, stream):
    """One decode step on one instance (host pool append, copy-on-write
    copies if any, then one launch that writes the new tokens, updates the
    device tables and lengths from the slots and decodes); returns the
    attended lengths."""
    L = inst.lib
    rc = L.pa_pool_append_batch(*inst.append_args)
    if rc != 0:
        raise RuntimeError(L.pa_last_error().decode())
    cow = inst.pairs[inst.pairs[:, 0] >= 0]
    if len(cow):
        B.pa_copy_blocks([inst.state.kc, inst.state.vc], cow)
        B.pa_pool_copies_done(inst.state.pool)
    inst.h_pos[:] = inst.h_lens
    rc = L.pa_paged_decode_append(*inst.step_args, stream)
    if rc != 0:
        raise RuntimeError(L.pa_last_error().decode())
    inst.h_lens += 1
    return inst.h_lens.copy()


def cpu_baseline(wl, budget_s=12.0):
    """The oracle (numpy fp64, single thread) on the same workload: the full
    64-sequence decode batch, repeated until about budget_s of CPU time."""
    from threadpoolctl import threadpool_limits

    from oracle import attention
    from tests.oracle_side import OracleStep
    o = OracleStep(wl)
    from paged_kv_cache_327_amd import workloads
    q = workloads.query_bits(wl.seed, wl.num_seqs, wl.num_q_heads, wl.head_dim)
    reps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            attention.paged_decode(q, o.kc, o.vc, o.table, o.seq_lens, wl.scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 400:
                break
    per = el / reps
    return {"value": round(kv_bytes(o.seq_lens, wl.num_kv_heads, wl.head_dim) / per / 1e9, 4),
            "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full {wl.num_seqs}-sequence decode batch of {wl.name} (fp64 numpy, 1 BLAS thread), "
                      f"{reps} reps in {el:.1f} s; {wl.num_seqs / per:.1f} seqs/s"}


def traffic_from_counters(alg_bytes):
    """HBM bytes per decode launch from the committed FETCH_SIZE / WRITE_SIZE
    summary (each counter scaled by what it reads for a plain copy of known
    size); None when the summary is missing or was taken on other decode
    kernel sources."""
    if not os.path.exists(COUNTERS):
        return None
    vals = {}
    with open(COUNTERS) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("decode_source_hash") != decode_source_hash():
        return None
    return int(float(vals["hbm_bytes_per_launch"]))


def prefill_flops(q_lens, seq_lens, num_q_heads, head_dim):
    """Algorithmic flops of causal chunked prefill: QK^T and PV over the
    visible keys only, 4 * D * Hq * (q * c + q (q + 1) / 2) per chunk."""
    total = 0
    for q, n in zip(q_lens, seq_lens):
        c = n - q
        total += 4 * head_dim * num_q_heads * (q * c + q * (q + 1) // 2)
    return total


def measure_prefill(torch, B, hip_side, workloads, block_size=16, reps=10):
    """The mixed step's prefill: 16 chunks of 512 queries over U{0..8192}
    context tokens, Llama-3-8B head shapes, one launch timed back to back."""
    wl = workloads.mixed_step(block_size, n_decode=0)
    h = hip_side.HipStep(wl)
    q = hip_side.to_device(workloads.query_bits(wl.seed, sum(wl.q_lens), wl.num_q_heads, wl.head_dim))
    out = torch.empty_like(q)
    qsl = torch.tensor(np.concatenate([[0], np.cumsum(wl.q_lens)]), dtype=torch.int32, device="cuda")
    msl = int(max(wl.seq_lens))

    def launch():
        B.pa_paged_prefill(out, q, h.kc, h.vc, h.table_dev, qsl, h.seq_lens_dev, max(wl.q_lens), msl, wl.scale)
    sec = time_launches(torch, launch, reps)
    flops = prefill_flops(wl.q_lens, wl.seq_lens, wl.num_q_heads, wl.head_dim)
    return {"workload": "16 prefill chunks of 512 queries over U{0..8192} context tokens",
            "block_size": block_size, "kernel": "prefill_kernel<128, 4, true, true, false>",
            "us": round(sec * 1e6, 1), "gflop": round(flops / 1e9, 2),
            "tflops": round(flops / sec / 1e12, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "frac": round(flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def measure_copy_bandwidth(torch, nbytes=1 << 30, reps=20):
    """A plain device-to-device copy of nbytes (read + write counted): the
    box's practical HBM ceiling, a second denominator beside the 8 TB/s
    published peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sec = time_launches(torch, lambda: dst.copy_(src), reps)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes": 2 * nbytes, "us": round(sec * 1e6, 1), "gbps": round(2 * nbytes / sec / 1e9, 1),
            "hbm_frac": round(2 * nbytes / sec / 1e9 / HBM_PEAK_GBPS, 4)}


def measure_tiny(torch, B, hip_side, workloads, reps=200):
    """The tiny decode (4 sequences of 1, 17, 33, 100 tokens; 8/2 heads, d 64):
    latency only, no roofline claim."""
    wl = workloads.tiny_decode()
    h = hip_side.HipStep(wl)
    q = hip_side.to_device(workloads.query_bits(wl.seed, wl.num_seqs, wl.num_q_heads, wl.head_dim))
    out = torch.empty_like(q)
    msl = max(wl.seq_lens)
    B.pa_paged_decode(out, q, h.kc, h.vc, h.table_dev, h.seq_lens_dev, msl, wl.scale, partition_size=0)  # checks
    args = (out.data_ptr(), None, q.data_ptr(), h.kc.data_ptr(), h.vc.data_ptr(), h.kc.stride(0), wl.num_blocks,
            h.table_dev.data_ptr(), h.table_dev.stride(0), h.seq_lens_dev.data_ptr(), wl.num_seqs, wl.num_q_heads,
            wl.num_kv_heads, wl.head_dim, wl.block_size, msl, 0, wl.scale, None, 0,
            torch.cuda.current_stream().cuda_stream)
    L = B.lib()
    sec = time_launches(torch, lambda: L.pa_paged_decode(*args), reps)
    return {"workload": "4 sequences of 1, 17, 33, 100 tokens, 8/2 heads, d 64, B 16", "decode_us": round(sec * 1e6, 2)}


def warm_clocks(torch, fn, seconds=0.3):
    """Keep the GPU busy with fn for about `seconds` so that its clocks have
    left their idle state before a measurement (a cold MI355X runs the first
    tens of milliseconds of work markedly slower)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_launches(torch, fn, reps, windows=3):
    """Seconds per call of fn (one or more launches on the current stream):
    the median over `windows` of one pair of HIP events around reps
    back-to-back calls, after a clock warm-up with the same calls."""
    warm_clocks(torch, fn)
    per = []
    for _ in range(windows):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / 1e3 / reps)
    return sorted(per)[len(per) // 2]


def hbm(gbps):
    return round(gbps / HBM_PEAK_GBPS, 4)


def unique_kv_bytes(table, seq_lens, block_size, num_kv_heads, head_dim):
    """K/V bytes of the distinct physical rows that a decode call attends
    (blocks shared by several sequences count once)."""
    rows = {}
    for r, n in zip(table, seq_lens):
        n = int(n)
        for j in range(-(-n // block_size)):
            b = int(r[j])
            rows[b] = max(rows.get(b, 0), min(block_size, n - j * block_size))
    return sum(rows.values()) * 2 * num_kv_heads * head_dim * 2


def measure_long_context(torch, B, hip_side, workloads, reps=3):
    """Decode over the 32-layer pool (26,785 16-token blocks per layer,
    52.3 GiB, layer-major [layer][K|V][block]); 8 sequences of
    U{16384..32768} tokens; partitions of 512 tokens plus the merge.  One
    step decodes every layer with that layer's queries."""
    wl = workloads.long_context()
    L, S, P = wl.num_layers, wl.num_seqs, 512
    kv = torch.full((L, 2, wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim), float("nan"),
                    dtype=torch.bfloat16, device="cuda")
    h = hip_side.HipStep(wl, gen="device", caches=(kv[0, 0], kv[0, 1]),
                         layers=[(l, kv[l, 0], kv[l, 1]) for l in range(L)])
    msl = max(wl.seq_lens)
    qs = [workloads.device_query(wl.seed, S, wl.num_q_heads, wl.head_dim, layer=l) for l in range(L)]
    out = torch.empty_like(qs[0])
    ws = torch.empty(B.pa_paged_decode_workspace_size(S, wl.num_q_heads, wl.head_dim, msl, P),
                     dtype=torch.uint8, device="cuda")

    def step():
        for l in range(L):
            B.pa_paged_decode(out, qs[l], kv[l, 0], kv[l, 1], h.table_dev, h.seq_lens_dev, msl, wl.scale,
                              partition_size=P, workspace=ws)
    sec = time_launches(torch, step, reps)
    per_layer = decode_bytes(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
    gbps = per_layer * L / sec / 1e9
    res = {"workload": "8 sequences of U{16384..32768} tokens over a 32-layer pool of 26,785 blocks per layer",
           "pool_gib": round(kv.numel() * 2 / 2**30, 2), "partition_size": P, "layers": L,
           "step_ms": round(sec * 1e3, 3), "layer_us": round(sec / L * 1e6, 1),
           "bytes_per_layer": per_layer, "gbps": round(gbps, 1), "hbm_frac": hbm(gbps),
           "seqs_per_s": round(S / sec, 1)}
    # the same step with partitions of 2048 tokens (fewer, longer work-groups)
    P2 = 2048
    ws2 = torch.empty(B.pa_paged_decode_workspace_size(S, wl.num_q_heads, wl.head_dim, msl, P2),
                      dtype=torch.uint8, device="cuda")

    def step2():
        for l in range(L):
            B.pa_paged_decode(out, qs[l], kv[l, 0], kv[l, 1], h.table_dev, h.seq_lens_dev, msl, wl.scale,
                              partition_size=P2, workspace=ws2)
    sec2 = time_launches(torch, step2, reps)
    res[f"partition_{P2}"] = {"step_ms": round(sec2 * 1e3, 3), "layer_us": round(sec2 / L * 1e6, 1),
                              "gbps": round(per_layer * L / sec2 / 1e9, 1),
                              "hbm_frac": hbm(per_layer * L / sec2 / 1e9), "seqs_per_s": round(S / sec2, 1)}
    del kv, h, qs
    torch.cuda.empty_cache()
    return res


def measure_prefix_cow(torch, B, hip_side, workloads, reps=20):
    """256 sequences forked from one 2050-token prompt, each with a suffix
    of U{1..512} tokens: the 255 copy-on-write copies (one layer, and all 32
    layers' 64 cache tensors in one call), the suffix writes, and decode.
    Decode GB/s is given on logical bytes (every sequence's K/V) and on
    unique bytes (shared prompt blocks once)."""
    wl = workloads.prefix_cow()
    h = hip_side.HipStep(wl, gen="device")
    S = wl.num_seqs
    pairs = np.array(h.pairs, dtype=np.int32)
    blk_bytes = wl.block_size * wl.num_kv_heads * wl.head_dim * 2
    res = {"workload": "256 forks of a 2050-token prompt, suffixes U{1..512}", "cow_pairs": len(pairs)}
    L = B.lib()
    stream = torch.cuda.current_stream().cuda_stream

    def copy_call(caches):
        # the C call with its arguments built once (the binding's argument
        # checks and marshalling in Python would otherwise be what is timed)
        B.pa_copy_blocks(caches, pairs)                                        # argument checks
        ptrs = (B.c_vp * len(caches))(*[c.data_ptr() for c in caches])
        args = (ptrs, len(caches), blk_bytes, caches[0].stride(0) * 2, caches[0].shape[0],
                pairs.ctypes.data_as(B.P_i32), len(pairs), stream)
        return lambda: L.pa_copy_blocks(*args)
    # bytes: each pair's block read and written; unique bytes: every
    # destination written and each distinct source read once (all 255 pairs
    # here copy the one shared partial tail block, which stays in cache)
    uniq = (len(set(pairs[:, 0].tolist())) + len(pairs)) * blk_bytes
    sec = time_launches(torch, copy_call([h.kc, h.vc]), reps)
    cb = 2 * len(pairs) * blk_bytes * 2
    res["copy_1_layer"] = {"us": round(sec * 1e6, 2), "bytes": cb, "gbps": round(cb / sec / 1e9, 1),
                           "unique_bytes": uniq * 2, "unique_gbps": round(uniq * 2 / sec / 1e9, 1)}
    big = torch.empty((32, 2, wl.num_blocks) + tuple(h.kc.shape[1:]), dtype=torch.bfloat16, device="cuda")
    caches = [big[l, c] for l in range(32) for c in range(2)]
    sec = time_launches(torch, copy_call(caches), 5)
    cb = 2 * len(pairs) * blk_bytes * 64
    res["copy_32_layers"] = {"us": round(sec * 1e6, 2), "bytes": cb, "gbps": round(cb / sec / 1e9, 1),
                             "unique_bytes": uniq * 64, "unique_gbps": round(uniq * 64 / sec / 1e9, 1),
                             "hbm_frac": hbm(uniq * 64 / sec / 1e9)}
    del big, caches
    torch.cuda.empty_cache()
    seqs = h.step_seqs
    n0 = np.concatenate([[0], np.cumsum([wl.new_lens[s] for s in seqs])])
    kn = torch.cat([workloads.device_seq_kv(wl.seed, s, wl.new_lens[s], wl.num_kv_heads, wl.head_dim, 0, 9)[0]
                    for s in seqs])
    slots = torch.from_numpy(np.asarray(h.step_slots, dtype=np.int64)).cuda()
    T = int(n0[-1])
    # rewriting the same rows leaves the caches as they were
    kc2, vc2 = h.kc.clone(), h.vc.clone()
    sec = time_launches(torch, lambda: B.pa_reshape_and_cache(kn, kn, kc2, vc2, slots), reps)
    rb = 2 * T * wl.num_kv_heads * wl.head_dim * 2 * 2
    res["reshape"] = {"tokens": T, "us": round(sec * 1e6, 2), "bytes": rb, "gbps": round(rb / sec / 1e9, 1),
                      "hbm_frac": hbm(rb / sec / 1e9)}
    del kc2, vc2
    q = workloads.device_query(wl.seed, S, wl.num_q_heads, wl.head_dim)
    out = torch.empty_like(q)
    msl = max(wl.seq_lens)
    logical = decode_bytes(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
    uniq = unique_kv_bytes(h.table, h.seq_lens, wl.block_size, wl.num_kv_heads, wl.head_dim)
    for P in (0, 512):
        ws = torch.empty(max(256, B.pa_paged_decode_workspace_size(S, wl.num_q_heads, wl.head_dim, msl, P)),
                         dtype=torch.uint8, device="cuda")
        sec = time_launches(torch, lambda: B.pa_paged_decode(out, q, h.kc, h.vc, h.table_dev, h.seq_lens_dev,
                                                             msl, wl.scale, partition_size=P, workspace=ws), reps)
        res[f"decode_p{P}"] = {"us": round(sec * 1e6, 2), "logical_gbps": round(logical / sec / 1e9, 1),
                               "unique_gbps": round(uniq / sec / 1e9, 1), "unique_hbm_frac": hbm(uniq / sec / 1e9),
                               "seqs_per_s": round(S / sec, 1)}
    res["logical_bytes"], res["unique_kv_bytes"] = logical, uniq
    del h
    torch.cuda.empty_cache()
    return res


def measure_mixed(torch, B, hip_side, workloads, block_size, reps=10):
    """The mixed step at one block size: the step's slots from the block
    table, writes of its 8,432 new tokens, prefill of 16 chunks of 512
    queries, decode of 240 sequences (partitions of 2048 tokens), on one
    stream; each call timed alone and the four together."""
    P = 2048
    wl = workloads.mixed_step(block_size)
    h = hip_side.HipStep(wl, gen="device")
    chunks = [s for s in range(wl.num_seqs) if wl.q_lens[s] > 1]
    dec = [s for s in range(wl.num_seqs) if wl.q_lens[s] == 1]
    seqs = h.step_seqs
    T = int(sum(wl.new_lens[s] for s in seqs))
    kn = workloads.device_query(wl.seed, T, wl.num_kv_heads, wl.head_dim, layer=3)
    qp = workloads.device_query(wl.seed, int(sum(wl.q_lens[s] for s in chunks)), wl.num_q_heads, wl.head_dim)
    op = torch.empty_like(qp)
    qsl = torch.tensor(np.concatenate([[0], np.cumsum([wl.q_lens[s] for s in chunks])]), dtype=torch.int32,
                       device="cuda")
    bt_p = h.table_dev[chunks].contiguous()
    sl_p = h.seq_lens_dev[chunks].contiguous()
    msl_p = int(max(wl.seq_lens[s] for s in chunks))
    qd = workloads.device_query(wl.seed, len(dec), wl.num_q_heads, wl.head_dim, layer=1)
    od = torch.empty_like(qd)
    bt_d = h.table_dev[dec].contiguous()
    sl_d = h.seq_lens_dev[dec].contiguous()
    dl = [wl.seq_lens[s] for s in dec]
    msl_d = int(max(dl))
    ws = torch.empty(B.pa_paged_decode_workspace_size(len(dec), wl.num_q_heads, wl.head_dim, msl_d, P),
                     dtype=torch.uint8, device="cuda")
    # the timed writes go to scratch copies of the caches: same slots, same bytes
    kc2, vc2 = h.kc.clone(), h.vc.clone()
    # the step's slots computed on the device from the block table (they equal
    # the host pool's, checked by the tests)
    qsl_all = torch.tensor(np.concatenate([[0], np.cumsum([wl.new_lens[s] for s in range(wl.num_seqs)])]),
                           dtype=torch.int32, device="cuda")
    dslots = torch.empty(T, dtype=torch.int64, device="cuda")

    def slot_mapping():
        B.pa_slot_mapping(h.table_dev, qsl_all, h.seq_lens_dev, block_size, T, out=dslots)

    def reshape():
        B.pa_reshape_and_cache(kn, kn, kc2, vc2, dslots)

    def prefill():
        B.pa_paged_prefill(op, qp, h.kc, h.vc, bt_p, qsl, sl_p, max(wl.q_lens), msl_p, wl.scale)

    def decode():
        B.pa_paged_decode(od, qd, h.kc, h.vc, bt_d, sl_d, msl_d, wl.scale, partition_size=P, workspace=ws)

    def step():
        slot_mapping()
        reshape()
        prefill()
        decode()

    # the same step with the decode on a second stream (default priority):
    # the HBM-bound decode can use compute units the MFMA-bound prefill leaves
    # idle; both wait for the cache writes
    side = torch.cuda.Stream()
    written = torch.cuda.Event()

    def step_two_streams():
        slot_mapping()
        reshape()
        written.record()
        side.wait_event(written)
        with torch.cuda.stream(side):
            decode()
        prefill()
        torch.cuda.current_stream().wait_stream(side)
    slot_mapping()
    t_m = time_launches(torch, slot_mapping, reps)
    t_r = time_launches(torch, reshape, reps)
    t_p = time_launches(torch, prefill, reps)
    t_d = time_launches(torch, decode, reps)
    t_s = time_launches(torch, step, reps)
    t_s2 = time_launches(torch, step_two_streams, reps)
    flops = prefill_flops([wl.q_lens[s] for s in chunks], [wl.seq_lens[s] for s in chunks], wl.num_q_heads,
                          wl.head_dim)
    db = decode_bytes(dl, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, block_size)
    rb = 2 * T * wl.num_kv_heads * wl.head_dim * 2 * 2
    res = {"block_size": block_size, "decode_partition_size": P, "step_ms": round(t_s * 1e3, 3),
           "step_two_streams_ms": round(t_s2 * 1e3, 3), "tokens_written": T,
           "slot_mapping_us": round(t_m * 1e6, 2),
           "reshape_us": round(t_r * 1e6, 2), "reshape_gbps": round(rb / t_r / 1e9, 1),
           "prefill_us": round(t_p * 1e6, 1), "prefill_gflop": round(flops / 1e9, 2),
           "prefill_tflops": round(flops / t_p / 1e12, 1),
           "prefill_mfma_frac": round(flops / t_p / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "decode_us": round(t_d * 1e6, 1), "decode_bytes": db, "decode_gbps": round(db / t_d / 1e9, 1),
           "decode_hbm_frac": hbm(db / t_d / 1e9), "decode_seqs_per_s": round(len(dec) / t_d, 1)}
    del h, kc2, vc2
    torch.cuda.empty_cache()
    return res


def measure_host_pool(B, num_blocks=26_785, block_size=16, prompt=8192, batch=64, reps=200):
    """Host cost of the pool calls a serving step makes, on a pool the size of
    the 52.32 GiB Llama-3-8B budget: one decode step's append for `batch`
    sequences, hashing a prompt's full blocks into the prefix cache, a fully
    hitting prefix lookup of the same prompt, and freeing it again."""
    L = B.lib()
    pool = B.pa_pool_create(num_blocks, block_size)
    h = pool.handle
    toks = np.arange(prompt, dtype=np.int32)
    tp = toks.ctypes.data_as(B.P_i32)
    hit = B.c_i64()
    B.pa_pool_add_seq(pool, 0)
    B.pa_pool_append(pool, 0, prompt)
    t0 = time.perf_counter()
    for _ in range(reps):
        if L.pa_pool_cache_blocks(h, 0, tp, prompt) != 0:
            raise RuntimeError(L.pa_last_error().decode())
    t_cache = (time.perf_counter() - t0) / reps
    t_hit = t_free = 0.0
    for r in range(reps):
        t0 = time.perf_counter()
        rc = L.pa_pool_add_seq_cached(h, 1 + r, tp, prompt, B.ctypes.byref(hit))
        t1 = time.perf_counter()
        rc |= L.pa_pool_free_seq(h, 1 + r)
        t2 = time.perf_counter()
        if rc != 0 or hit.value != prompt:
            raise RuntimeError("prefix lookup did not hit the whole prompt")
        t_hit += t1 - t0
        t_free += t2 - t1
    ids = np.arange(1000, 1000 + batch, dtype=np.int64)
    ones = np.full(batch, 1, dtype=np.int32)
    slots = np.empty(batch, dtype=np.int64)
    pairs = np.empty((batch, 2), dtype=np.int32)
    done = B.c_i32()
    for i in ids:
        B.pa_pool_add_seq(pool, int(i))
        B.pa_pool_append(pool, int(i), 600)
    args = (h, ids.ctypes.data_as(B.P_i64), ones.ctypes.data_as(B.P_i32), batch,
            slots.ctypes.data_as(B.P_i64), pairs.ctypes.data_as(B.P_i32), B.ctypes.byref(done))
    n = 1000
    t0 = time.perf_counter()
    for _ in range(n):
        if L.pa_pool_append_batch(*args) != 0:
            raise RuntimeError(L.pa_last_error().decode())
    t_app = (time.perf_counter() - t0) / n
    B.pa_pool_check(pool)
    return {"num_blocks": num_blocks, "block_size": block_size, "prompt_tokens": prompt,
            "cache_blocks_us": round(t_cache * 1e6, 1),
            "hash_mtok_per_s": round(prompt / t_cache / 1e6, 1),
            "prefix_hit_us": round(t_hit / reps * 1e6, 1), "free_seq_us": round(t_free / reps * 1e6, 1),
            f"append_batch_{batch}x1_us": round(t_app * 1e6, 2)}


def measure_fp8_decode(torch, B, hip_side, workloads, scales=(0.05, 0.05), instances=8, reps=48):
    """Decode over E4M3 caches: the 64-sequence Llama-3-8B decode batch
    (8 pools rotated, about 590 MB of K/V codes, so that no pool stays in the
    last-level cache between its calls) and the 32-layer long-context pool;
    plus the quantising cache write of one decode step's 64 tokens."""
    wls = [workloads.llama_decode(seed_offset=i) for i in range(instances)]
    hs = [hip_side.HipStep(w, gen="device", fp8=scales) for w in wls]
    wl = wls[0]
    S = wl.num_seqs
    qs = [workloads.device_query(w.seed, S, w.num_q_heads, w.head_dim) for w in wls]
    msl = max(max(w.seq_lens) for w in wls)
    out = torch.empty_like(qs[0])
    rot = [0]

    def nxt():
        i = rot[0] % instances
        B.pa_paged_decode_fp8(out, qs[i], hs[i].kc, hs[i].vc, hs[i].table_dev, hs[i].seq_lens_dev, msl,
                              wl.scale, *scales, partition_size=0)
        rot[0] += 1
    sec = time_launches(torch, nxt, reps)
    alg = np.mean([decode_bytes(w.seq_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, 1)
                   for w in wls])
    gbps = alg / sec / 1e9
    # one step's write: 64 new tokens quantised into their slots
    k = hip_side.to_device(workloads.normal_bf16(np.random.default_rng(1), (S, wl.num_kv_heads, wl.head_dim)))
    slots = torch.from_numpy(hs[0].step_slots.astype(np.int64)).cuda()
    B.pa_reshape_and_cache_fp8(k, k, hs[0].kc, hs[0].vc, slots, *scales)          # argument checks
    w_args = (k.data_ptr(), k.stride(0), k.data_ptr(), k.stride(0), hs[0].kc.data_ptr(), hs[0].vc.data_ptr(),
              hs[0].kc.stride(0), wl.num_blocks, slots.data_ptr(), S, wl.num_kv_heads, wl.head_dim, wl.block_size,
              scales[0], scales[1], torch.cuda.current_stream().cuda_stream)
    L = B.lib()
    t_w = time_launches(torch, lambda: L.pa_reshape_and_cache_fp8(*w_args), 200)
    res = {"workload": f"{wl.name}, E4M3 K/V with per-cache scales", "scales": list(scales),
           "kernel": "decode_partition_kernel<128, 4, true, true, false>", "decode_us": round(sec * 1e6, 2),
           "bytes_per_launch": int(alg), "gbps": round(gbps, 1), "hbm_frac": hbm(gbps),
           "seqs_per_s": round(S / sec, 1), "write_64_tokens_us": round(t_w * 1e6, 2)}
    del hs, qs
    torch.cuda.empty_cache()

    # the mixed step's prefill chunks over E4M3 caches
    pw = workloads.mixed_step(16, n_decode=0)
    ph = hip_side.HipStep(pw, gen="device", fp8=scales)
    pq = hip_side.to_device(workloads.query_bits(pw.seed, sum(pw.q_lens), pw.num_q_heads, pw.head_dim))
    pout = torch.empty_like(pq)
    pqsl = torch.tensor(np.concatenate([[0], np.cumsum(pw.q_lens)]), dtype=torch.int32, device="cuda")
    pmsl = int(max(pw.seq_lens))
    B.pa_paged_prefill_fp8(pout, pq, ph.kc, ph.vc, ph.table_dev, pqsl, ph.seq_lens_dev, max(pw.q_lens), pmsl,
                           pw.scale, *scales)                                   # argument checks
    p_args = (pout.data_ptr(), pq.data_ptr(), ph.kc.data_ptr(), ph.vc.data_ptr(), ph.kc.stride(0), pw.num_blocks,
              ph.table_dev.data_ptr(), ph.table_dev.stride(0), pqsl.data_ptr(), ph.seq_lens_dev.data_ptr(),
              pw.num_seqs, max(pw.q_lens), pmsl, pw.num_q_heads, pw.num_kv_heads, pw.head_dim, pw.block_size,
              pw.scale, scales[0], scales[1], 1, torch.cuda.current_stream().cuda_stream)
    t_p = time_launches(torch, lambda: L.pa_paged_prefill_fp8(*p_args), 10)
    pflops = prefill_flops(pw.q_lens, pw.seq_lens, pw.num_q_heads, pw.head_dim)
    res["prefill"] = {"workload": "16 prefill chunks of 512 queries over U{0..8192} context tokens",
                      "kernel": "prefill_kernel<128, 4, true, true, true>", "us": round(t_p * 1e6, 1),
                      "tflops": round(pflops / t_p / 1e12, 1),
                      "frac": round(pflops / t_p / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    del ph, pq, pout
    torch.cuda.empty_cache()

    # the 32-layer long-context pool in E4M3 (half the bytes of the bf16 pool)
    wl = workloads.long_context()
    L, S, P = wl.num_layers, wl.num_seqs, 2048
    kv = torch.full((L, 2, wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim), 0x7F,
                    dtype=torch.uint8, device="cuda")
    h = hip_side.HipStep(wl, gen="device", caches=(kv[0, 0], kv[0, 1]),
                         layers=[(l, kv[l, 0], kv[l, 1]) for l in range(L)], fp8=scales)
    msl = max(wl.seq_lens)
    qs = [workloads.device_query(wl.seed, S, wl.num_q_heads, wl.head_dim, layer=l) for l in range(L)]
    out = torch.empty_like(qs[0])
    ws = torch.empty(B.pa_paged_decode_workspace_size(S, wl.num_q_heads, wl.head_dim, msl, P),
                     dtype=torch.uint8, device="cuda")

    def step():
        for l in range(L):
            B.pa_paged_decode_fp8(out, qs[l], kv[l, 0], kv[l, 1], h.table_dev, h.seq_lens_dev, msl, wl.scale,
                                  *scales, partition_size=P, workspace=ws)
    sec = time_launches(torch, step, 3)
    per_layer = decode_bytes(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, 1)
    gbps = per_layer * L / sec / 1e9
    res["long_context"] = {"pool_gib": round(kv.numel() / 2**30, 2), "partition_size": P,
                           "step_ms": round(sec * 1e3, 3), "layer_us": round(sec / L * 1e6, 1),
                           "bytes_per_layer": per_layer, "gbps": round(gbps, 1), "hbm_frac": hbm(gbps),
                           "seqs_per_s": round(S / sec, 1)}
    del kv, h, qs
    torch.cuda.empty_cache()
    return res


def counter_run(kind, reps):
    """Launch only one kernel kind, for rocprofv3 --pmc passes:
    'decode' = the decode call of this workload on rotating pools,
    'copy' = a plain device copy of COPY_CALIBRATION_BYTES (calibration),
    'prefill' = the mixed step's prefill chunks (MFMA counters)."""
    import torch

    from paged_kv_cache_327_amd import binding as B
    from paged_kv_cache_327_amd import workloads
    from tests import hip_side
    if kind == "prefill":
        wl = workloads.mixed_step(16, n_decode=0)
        h = hip_side.HipStep(wl)
        q = hip_side.to_device(workloads.query_bits(wl.seed, sum(wl.q_lens), wl.num_q_heads, wl.head_dim))
        out = torch.empty_like(q)
        qsl = torch.tensor(np.concatenate([[0], np.cumsum(wl.q_lens)]), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        for _ in range(reps):
            B.pa_paged_prefill(out, q, h.kc, h.vc, h.table_dev, qsl, h.seq_lens_dev, max(wl.q_lens),
                               int(max(wl.seq_lens)), wl.scale)
        torch.cuda.synchronize()
        print(f"prefill x {reps}; {prefill_flops(wl.q_lens, wl.seq_lens, 32, 128):.0f} flop per launch", flush=True)
        return
    if kind == "copy":
        x = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(reps):
            y.copy_(x)
        torch.cuda.synchronize()
        print(f"copy of {COPY_CALIBRATION_BYTES} bytes x {reps}", flush=True)
        return
    wls = [workloads.llama_decode(seed_offset=i) for i in range(4)]
    msl = max(max(w.seq_lens) for w in wls) + 1
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    insts = [Instance(w, torch, B, hip_side, workloads, msl + 1, 0, ws) for w in wls]
    stream = torch.cuda.current_stream().cuda_stream
    lens = [run_step(i, B, stream) for i in insts]      # stage tables and lengths (one decode step each)
    torch.cuda.synchronize()
    for k in range(reps):
        insts[k % 4].decode(stream)
    torch.cuda.synchronize()
    print(f"decode x {reps}; algorithmic bytes per launch "
          f"{np.mean([decode_bytes(lens[k % 4], 32, 8, 128, 16) for k in range(reps)]):.0f}", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--partition-size", type=int, default=0,
                    help="decode split-K partition (0 = one partition per sequence)")
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--kernel-reps", type=int, default=48,
                    help="back-to-back decode launches timed with HIP events for the roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the long-context, prefix-sharing and mixed-step measurements")
    ap.add_argument("--counter-run", choices=["decode", "copy", "prefill"],
                    help="only launch one kernel kind (for rocprofv3 --pmc passes) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; there is no multi-GPU path. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.counter_run:
        counter_run(args.counter_run, 12)
        return

    import torch

    from paged_kv_cache_327_amd import binding as B
    from paged_kv_cache_327_amd import workloads
    from tests import hip_side

    B.lib()  # fail loudly if the library is missing
    wls = [workloads.llama_decode(seed_offset=i) for i in range(args.instances)]
    max_seq_len = max(max(w.seq_lens) for w in wls) + args.warmup + args.steps + 1
    wl = wls[0]
    S = wl.num_seqs
    ws_bytes = B.pa_paged_decode_workspace_size(S, wl.num_q_heads, wl.head_dim, max_seq_len,
                                                args.partition_size)
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    print(f"[bench] set-up: {args.instances} instances of {wl.name}", file=sys.stderr, flush=True)
    insts = [Instance(w, torch, B, hip_side, workloads, max_seq_len, args.partition_size, workspace)
             for w in wls]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    for i in range(max(args.warmup, len(insts))):    # every pool staged at least once
        run_step(insts[i % len(insts)], B, stream)
    torch.cuda.synchronize()
    # bring the clocks up with decode launches on the staged pools (they leave
    # the pools unchanged)
    warm_clocks(torch, lambda: [inst.decode(stream) for inst in insts], 0.5)
    print("[bench] warm-up done", file=sys.stderr, flush=True)

    # whole-step throughput
    step_lens = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step_lens.append(run_step(insts[k % len(insts)], B, stream))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print("[bench] timed steps done", file=sys.stderr, flush=True)

    # dominant kernel: back-to-back decode launches on the same stream,
    # rotating over the pools, bracketed by one pair of HIP events per window
    # (an event between launches adds its own cost to every launch)
    rot = [0]

    def decode_next():
        insts[rot[0] % len(insts)].decode(stream)
        rot[0] += 1
    dec_s = time_launches(torch, decode_next, args.kernel_reps)
    cur_lens = [np.array(i.h_lens) for i in insts]
    alg_per_launch = np.mean([decode_bytes(cur_lens[k], wl.num_q_heads, wl.num_kv_heads,
                                           wl.head_dim, wl.block_size) for k in range(len(insts))])
    achieved = alg_per_launch / dec_s / 1e9
    # the step's cache write alone (no table update): 64 new tokens' K and V
    # rows to their slots
    w_inst = insts[0]
    w_slots = torch.from_numpy(w_inst.h_slots.copy()).cuda()
    kc0 = w_inst.state.kc
    w_args = (w_inst.new_k.data_ptr(), w_inst.new_k.stride(0), w_inst.new_v.data_ptr(), w_inst.new_v.stride(0),
              kc0.data_ptr(), w_inst.state.vc.data_ptr(), kc0.stride(0), wl.num_blocks, w_slots.data_ptr(), S,
              wl.num_kv_heads, wl.head_dim, wl.block_size, stream)
    res_s = time_launches(torch, lambda: w_inst.lib.pa_reshape_and_cache(*w_args), 200)

    ms_per_step = elapsed / args.steps * 1e3
    kv_per_step = np.mean([kv_bytes(l, wl.num_kv_heads, wl.head_dim) for l in step_lens])
    value = kv_per_step / (ms_per_step / 1e3) / 1e9
    nparts = -(-max_seq_len // args.partition_size) if args.partition_size else 1

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": S, "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "num_blocks": wl.num_blocks, "context": "512 + U{0..100} (+1 per step)",
                   "partition_size": args.partition_size, "pool_instances": args.instances},
        "seqs_per_s": round(S / (ms_per_step / 1e3), 1),
        "step_hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "decode_kernel_us": round(dec_s * 1e6, 2),
        "decode_seqs_per_s": round(S / dec_s, 1),
        "reshape_64_tokens_us": round(res_s * 1e6, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": DECODE_KERNEL + (" + decode_merge_kernel<128>" if nparts > 1 else ""),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_counters(alg_per_launch),
            "algorithmic_bytes_per_launch": int(alg_per_launch),
        },
        "cpu_baseline": None,
    }
    if not args.no_prefill:
        print("[bench] prefill", file=sys.stderr, flush=True)
        del insts
        torch.cuda.empty_cache()
        line["prefill"] = measure_prefill(torch, B, hip_side, workloads)
    if not args.no_configs:
        cfg = {}
        print("[bench] tiny decode, copy bandwidth", file=sys.stderr, flush=True)
        cfg["tiny_decode"] = measure_tiny(torch, B, hip_side, workloads)
        cfg["d2d_copy"] = measure_copy_bandwidth(torch)
        print("[bench] long-context 32-layer pool", file=sys.stderr, flush=True)
        cfg["long_context_decode"] = measure_long_context(torch, B, hip_side, workloads)
        print("[bench] prefix sharing + copy-on-write", file=sys.stderr, flush=True)
        cfg["prefix_cow_decode"] = measure_prefix_cow(torch, B, hip_side, workloads)
        for bs in (1, 16, 32):
            print(f"[bench] mixed step, block size {bs}", file=sys.stderr, flush=True)
            cfg[f"mixed_step_b{bs}"] = measure_mixed(torch, B, hip_side, workloads, bs)
        print("[bench] E4M3 KV cache decode", file=sys.stderr, flush=True)
        cfg["fp8_decode"] = measure_fp8_decode(torch, B, hip_side, workloads)
        line["configs"] = cfg
    line["host_pool"] = measure_host_pool(B)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
