"""Benchmark of paged attention on one MI355X.

Headline step: long-context decode over a 32-layer pool.  Eight sequences
of U{16384..32768} tokens (Llama-3-8B head shapes: 32 query / 8 KV heads,
head_dim 128, bf16, block_size 16) live in a 32-layer pool of 26,785
blocks per layer (the 52.32 GiB pool of the budget paragraph of
"PagedAttention: fragmentation, blocks, block tables"), every sequence's
blocks scattered through it by a seeded placement.  One step is the whole
decode path for the batch:
  1. the host pool appends one token to each sequence (new block ids,
     slots, copy-on-write pairs);
  2. pending copy-on-write block copies run over all 64 cache tensors
     (none arise in this workload);
  3. for each of the 32 layers one pa_paged_decode_append call: the layer's
     new K/V rows go to their slots, the device block-table entries and
     lengths follow from the slots (kernel arguments; the tables were copied
     to the device once, at set-up), split-K decode runs over partitions of
     --partition-size tokens and the log-sum-exp merge combines them.
value = K/V bytes attended per step / step time (whole-job throughput; the
K/V are resident in HBM).  Every layer reads ~780 MB, far beyond the 256 MiB
last-level cache, so no layer finds its K/V cached.

The other workloads (the Llama-3-8B batch of 64, prefix sharing with
copy-on-write, the mixed chunked-prefill + decode step at block sizes 1, 16
and 32, the tiny decode, E4M3 caches) are reported under "configs"; the
oracle (numpy fp64) is timed on the host for each of them under
"cpu_baseline".

Prints one JSON line.  --gpus above 1 is refused: this build runs on one GPU.

Profiling helpers (the summaries under profiles/ are written by them):
  --counter-run KIND     launch only one kernel kind, for rocprofv3 --pmc
  --counter-summary      FETCH_SIZE / WRITE_SIZE CSVs -> traffic summary
  --trace-summary        kernel-trace stats CSV -> markdown table
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
METRIC = "paged decode KV-read GB/s (% of HBM peak) + seqs/s; prefill TFLOP/s"
# template arguments: head_dim, query heads per KV head, block size >= 16, E4M3 caches, appending
# the long-context step's appending decode (row layout: explicit partitions
# of up to 1024 tokens) and the Llama batch's (head layout: one partition
# per sequence)
APPEND_KERNEL = "decode_rows_kernel<4, true, true>"
LLAMA_APPEND_KERNEL = "decode_partition_kernel<128, 4, true, false, true>"
LLAMA_PLAIN_KERNEL = "decode_partition_kernel<128, 4, true, false, false>"
MERGE_KERNEL = "decode_merge_kernel<128>"
FP8_KERNEL = "decode_partition_kernel<128, 4, true, true, false>"
FP8_LONG_CONTEXT_KERNEL = "decode_rows8_kernel<4, true>"
# head_dim, query heads per work-group, causal, block size >= 16, E4M3 caches, 32-bit key offsets
PREFILL_KERNEL = "prefill_kernel<128, 4, true, true, false, 0>"
HEADLINE_PARTITION = 512
FP8_SCALES = (0.05, 0.05)        # E4M3 k_scale, v_scale of the E4M3 workloads
FP8_LONG_CONTEXT_PARTITION = 512
COUNTERS = {
    "long_context": os.path.join(ROOT, "profiles", "decode_append_long_context_traffic.txt"),
    "decode": os.path.join(ROOT, "profiles", "decode_append_llama3_8b_traffic.txt"),
    "fp8_long_context": os.path.join(ROOT, "profiles", "decode_fp8_long_context_traffic.txt"),
}
COPY_CALIBRATION_BYTES = 512 << 20
DECODE_SOURCES = ("paged_kv_cache_327_amd/csrc/kernels/paged_decode.hip",
                  "paged_kv_cache_327_amd/csrc/kernels/decode_body.hpp",
                  "paged_kv_cache_327_amd/csrc/kernels/common.hpp",
                  "paged_kv_cache_327_amd/csrc/internal.hpp",
                  "paged_kv_cache_327_amd/csrc/api.cpp",
                  "paged_kv_cache_327_amd/build.py")


def decode_source_hash():
    """Hash of every source that shapes the decode kernels' code (kernel,
    helpers, argument layout, host launch set-up, compiler flags)."""
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ work formulas


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


def prefill_flops(q_lens, seq_lens, num_q_heads, head_dim):
    """Algorithmic flops of causal chunked prefill: QK^T and PV over the
    visible keys only, 4 * D * Hq * (q * c + q (q + 1) / 2) per chunk."""
    total = 0
    for q, n in zip(q_lens, seq_lens):
        c = n - q
        total += 4 * head_dim * num_q_heads * (q * c + q * (q + 1) // 2)
    return total


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


def hbm(gbps):
    return round(gbps / HBM_PEAK_GBPS, 4)


# ------------------------------------------------------------------ timing


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
    """Seconds per call of fn (one or more launches on torch's current
    stream, which every call here launches on): the median over `windows` of
    one pair of HIP events around reps back-to-back calls, after a clock
    warm-up with the same calls."""
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


def _check(L, rc):
    if rc != 0:
        raise RuntimeError(L.pa_last_error().decode())


# ------------------------------------------------------------ step classes


class LongContextStep:
    """The 32-layer long-context decode step (the headline).

    Set-up: the 32-layer pool (layer-major [layer][K|V][block][B][Hkv][D]),
    every sequence's context written to every layer at the slots the host
    pool gave it, the block tables copied to the device once.  Step inputs
    (queries and new K/V rows per layer) come in ROT seeded sets used in
    turn.  A step is append() (host pool) followed by launch() (one
    pa_paged_decode_append call per layer on `stream`); outputs go to
    out[layer] (and lse[layer] when asked for)."""

    ROT = 4

    def __init__(self, torch, B, hip_side, workloads, partition_size=HEADLINE_PARTITION, max_steps=64,
                 lse=False):
        wl = workloads.long_context()
        self.wl, self.B, self.torch = wl, B, torch
        L, S = wl.num_layers, wl.num_seqs
        Hq, Hkv, D = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
        self.L, self.S, self.P = L, S, partition_size
        self.kv = torch.full((L, 2, wl.num_blocks, wl.block_size, Hkv, D), float("nan"), dtype=torch.bfloat16,
                             device="cuda")
        self.max_seq_len = max(wl.seq_lens) + max_steps + 1
        self.width = -(-self.max_seq_len // wl.block_size)
        self.h = hip_side.HipStep(wl, gen="device", caches=(self.kv[0, 0], self.kv[0, 1]),
                                  layers=[(l, self.kv[l, 0], self.kv[l, 1]) for l in range(L)], bt_width=self.width)
        self.lens = self.h.seq_lens.astype(np.int64).copy()
        self.q = workloads.device_rows(wl.seed, 1, (self.ROT, L, S, Hq, D))
        self.new_k = workloads.device_rows(wl.seed, 2, (self.ROT, L, S, Hkv, D))
        self.new_v = workloads.device_rows(wl.seed, 3, (self.ROT, L, S, Hkv, D))
        self.out = torch.empty((L, S, Hq, D), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((L, S, Hq), dtype=torch.float32, device="cuda") if lse else None
        ws = B.pa_paged_decode_workspace_size(S, Hq, D, self.max_seq_len, partition_size)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda")
        self.seq_ids = np.arange(S, dtype=np.int64)
        self.ones = np.ones(S, dtype=np.int32)
        self.slots = np.empty(S, dtype=np.int64)
        self.pos = np.empty(S, dtype=np.int32)
        self.pairs = np.empty((S, 2), dtype=np.int32)
        self.done = B.c_i32(0)
        self.lib = B.lib()
        self.steps = 0
        self.stream = torch.cuda.current_stream().cuda_stream
        # validate every argument once through the binding (a plain decode
        # call with the same geometry), then keep the raw C argument tuples
        B.pa_paged_decode(self.out[0], self.q[0, 0], self.kv[0, 0], self.kv[0, 1], self.h.table_dev,
                          self.h.seq_lens_dev, self.max_seq_len, wl.scale, partition_size=partition_size,
                          workspace=self.ws)
        self.append_args = (self.h.pool.handle, self.seq_ids.ctypes.data_as(B.P_i64),
                            self.ones.ctypes.data_as(B.P_i32), S, self.slots.ctypes.data_as(B.P_i64),
                            self.pairs.ctypes.data_as(B.P_i32), B.ctypes.byref(self.done))
        bstride = self.kv.stride(2)
        self.args = []
        for r in range(self.ROT):
            row = []
            for l in range(L):
                kc, vc = self.kv[l, 0], self.kv[l, 1]
                row.append((self.out[l].data_ptr(), self.lse[l].data_ptr() if lse else None,
                            self.q[r, l].data_ptr(), kc.data_ptr(), vc.data_ptr(), bstride, wl.num_blocks,
                            self.h.table_dev.data_ptr(), self.width, self.h.seq_lens_dev.data_ptr(), S, Hq, Hkv,
                            D, wl.block_size, self.max_seq_len, partition_size, wl.scale,
                            self.new_k[r, l].data_ptr(), self.new_k.stride(2), self.new_v[r, l].data_ptr(),
                            self.new_v.stride(2), self.slots.ctypes.data_as(B.P_i64),
                            self.pos.ctypes.data_as(B.P_i32), self.ws.data_ptr(), self.ws.numel(), self.stream))
            self.args.append(row)
        self.caches = [self.kv[l, c] for l in range(L) for c in range(2)]

    def append(self):
        """Host pool: one token for every sequence; copy-on-write copies (if
        any) for all 64 cache tensors."""
        if self.steps + 1 > self.max_seq_len - max(self.wl.seq_lens) - 1:
            raise RuntimeError("more steps than the tables were sized for")
        _check(self.lib, self.lib.pa_pool_append_batch(*self.append_args))
        cow = self.pairs[self.pairs[:, 0] >= 0]
        if len(cow):
            self.B.pa_copy_blocks(self.caches, cow)
            self.B.pa_pool_copies_done(self.h.pool)
        self.pos[:] = self.lens

    def launch(self):
        """The step's device work: one appending decode call per layer."""
        r = self.steps % self.ROT
        f = self.lib.pa_paged_decode_append
        for a in self.args[r]:
            _check(self.lib, f(*a))
        self.lens += 1
        self.steps += 1

    def relaunch(self):
        """The last step's device work again (same slots, positions and
        inputs): idempotent, so the layer launches can be timed back to
        back."""
        r = (self.steps - 1) % self.ROT
        f = self.lib.pa_paged_decode_append
        for a in self.args[r]:
            _check(self.lib, f(*a))

    def step(self):
        self.append()
        self.launch()

    def step_inputs(self):
        """(queries, new K rows, new V rows) of the last step, all layers."""
        r = (self.steps - 1) % self.ROT
        return self.q[r], self.new_k[r], self.new_v[r]

    def bytes_per_layer(self):
        """Algorithmic bytes of one layer's decode at the current lengths."""
        w = self.wl
        return decode_bytes(self.lens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size)

    def close(self):
        del self.kv, self.h, self.caches, self.args
        self.torch.cuda.empty_cache()


class LlamaDecodeInstance:
    """One Llama-3-8B-shaped decode batch (64 sequences of 512 + U{0..100}
    tokens, 8192-block pool): the device tables and lengths are copied once,
    at set-up; every step after that is one pa_paged_decode_append launch
    (plus the merge when a sequence spans several partitions).  Step inputs
    (new K/V rows and queries) come in ROT seeded host draws used in turn."""

    ROT = 4

    def __init__(self, wl, torch, B, hip_side, workloads, max_seq_len, partition_size, workspace, lse=False):
        self.wl = wl
        S = wl.num_seqs
        self.S = S
        self.width = -(-max_seq_len // wl.block_size)
        self.state = hip_side.HipStep(wl, bt_width=self.width)   # set-up: contexts + one step's token
        self.d_table = self.state.table_dev
        self.d_lens = self.state.seq_lens_dev
        self.h_lens = self.state.seq_lens.astype(np.int64).copy()
        rng = np.random.default_rng([wl.seed, 99])
        Hq, Hkv, D = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
        self.k_bits = [workloads.normal_bf16(rng, (S, Hkv, D)) for _ in range(self.ROT)]
        self.v_bits = [workloads.normal_bf16(rng, (S, Hkv, D)) for _ in range(self.ROT)]
        self.q_bits = [workloads.normal_bf16(rng, (S, Hq, D)) for _ in range(self.ROT)]
        self.new_k = [hip_side.to_device(b) for b in self.k_bits]
        self.new_v = [hip_side.to_device(b) for b in self.v_bits]
        self.q = [hip_side.to_device(b) for b in self.q_bits]
        self.out = torch.empty_like(self.q[0])
        self.lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda") if lse else None
        self.seq_ids = np.arange(S, dtype=np.int64)
        self.ones = np.ones(S, dtype=np.int32)
        self.h_slots = np.empty(S, dtype=np.int64)
        self.h_pos = np.empty(S, dtype=np.int32)         # each row's length before the step
        self.pairs = np.empty((S, 2), dtype=np.int32)
        self.done = B.c_i32(0)
        self.steps = 0
        kc, vc = self.state.kc, self.state.vc
        self.lib = B.lib()
        self.B = B
        self.append_args = (self.state.pool.handle, self.seq_ids.ctypes.data_as(B.P_i64),
                            self.ones.ctypes.data_as(B.P_i32), S,
                            self.h_slots.ctypes.data_as(B.P_i64), self.pairs.ctypes.data_as(B.P_i32),
                            B.ctypes.byref(self.done))
        bstride = kc.stride(0)
        lse_p = self.lse.data_ptr() if lse else None
        self.decode_args = [(self.out.data_ptr(), lse_p, q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bstride,
                             wl.num_blocks, self.d_table.data_ptr(), self.width, self.d_lens.data_ptr(), S, Hq, Hkv,
                             D, wl.block_size, max_seq_len, partition_size, wl.scale, workspace.data_ptr(),
                             workspace.numel()) for q in self.q]
        self.step_args = [(self.out.data_ptr(), lse_p, self.q[r].data_ptr(), kc.data_ptr(), vc.data_ptr(), bstride,
                           wl.num_blocks, self.d_table.data_ptr(), self.width, self.d_lens.data_ptr(), S, Hq, Hkv,
                           D, wl.block_size, max_seq_len, partition_size, wl.scale, self.new_k[r].data_ptr(),
                           self.new_k[r].stride(0), self.new_v[r].data_ptr(), self.new_v[r].stride(0),
                           self.h_slots.ctypes.data_as(B.P_i64), self.h_pos.ctypes.data_as(B.P_i32),
                           workspace.data_ptr(), workspace.numel()) for r in range(self.ROT)]

    def step(self, stream):
        """Host pool append, copy-on-write copies if any, then one launch that
        writes the new tokens, updates the device tables and lengths from the
        slots and decodes; returns the attended lengths."""
        L = self.lib
        _check(L, L.pa_pool_append_batch(*self.append_args))
        cow = self.pairs[self.pairs[:, 0] >= 0]
        if len(cow):
            self.B.pa_copy_blocks([self.state.kc, self.state.vc], cow)
            self.B.pa_pool_copies_done(self.state.pool)
        self.h_pos[:] = self.h_lens
        _check(L, L.pa_paged_decode_append(*self.step_args[self.steps % self.ROT], stream))
        self.steps += 1
        self.h_lens += 1
        return self.h_lens.copy()

    def relaunch(self, stream):
        """The last step's launch again (idempotent: same slots, positions and
        inputs)."""
        _check(self.lib, self.lib.pa_paged_decode_append(*self.step_args[(self.steps - 1) % self.ROT], stream))

    def decode(self, stream):
        """A plain decode launch over the current tables."""
        _check(self.lib, self.lib.pa_paged_decode(*self.decode_args[0], stream))


class MixedStep:
    """The mixed chunked-prefill + decode step at one block size: the step's
    slots from the block table (pa_slot_mapping), the cache writes of its
    8,432 new tokens (pa_reshape_and_cache), prefill of the 16 chunks of 512
    queries and decode of the 240 sequences (partitions of P tokens).  The
    new tokens written are the ones the set-up drew for the step, so a step
    leaves the caches as it found them and can be repeated."""

    def __init__(self, torch, B, hip_side, workloads, block_size, partition_size=2048):
        self.torch, self.B = torch, B
        wl = workloads.mixed_step(block_size)
        self.wl, self.P = wl, partition_size
        h = hip_side.HipStep(wl, gen="device")
        self.h = h
        self.chunks = [s for s in range(wl.num_seqs) if wl.q_lens[s] > 1]
        self.dec = [s for s in range(wl.num_seqs) if wl.q_lens[s] == 1]
        seqs = h.step_seqs
        self.T = int(sum(wl.new_lens[s] for s in seqs))
        # the step's new K/V rows, token by token in step_seqs order (the order
        # of the host pool's slots and of query_start_loc below)
        kv = [workloads.device_seq_kv(wl.seed, s, wl.new_lens[s], wl.num_kv_heads, wl.head_dim, 0, 1) for s in seqs]
        self.kn = torch.cat([k for k, _ in kv])
        self.vn = torch.cat([v for _, v in kv])
        self.qp = workloads.device_query(wl.seed, int(sum(wl.q_lens[s] for s in self.chunks)), wl.num_q_heads,
                                         wl.head_dim)
        self.op = torch.empty_like(self.qp)
        self.qsl = torch.tensor(np.concatenate([[0], np.cumsum([wl.q_lens[s] for s in self.chunks])]),
                                dtype=torch.int32, device="cuda")
        self.bt_p = h.table_dev[self.chunks].contiguous()
        self.sl_p = h.seq_lens_dev[self.chunks].contiguous()
        self.msl_p = int(max(wl.seq_lens[s] for s in self.chunks))
        self.qd = workloads.device_query(wl.seed, len(self.dec), wl.num_q_heads, wl.head_dim, layer=1)
        self.od = torch.empty_like(self.qd)
        self.lsed = torch.empty(self.qd.shape[:2], dtype=torch.float32, device="cuda")
        self.bt_d = h.table_dev[self.dec].contiguous()
        self.sl_d = h.seq_lens_dev[self.dec].contiguous()
        self.dl = [wl.seq_lens[s] for s in self.dec]
        self.msl_d = int(max(self.dl))
        self.ws = torch.empty(max(256, B.pa_paged_decode_workspace_size(len(self.dec), wl.num_q_heads, wl.head_dim,
                                                                        self.msl_d, partition_size)),
                              dtype=torch.uint8, device="cuda")
        assert seqs == list(range(wl.num_seqs))
        self.qsl_all = torch.tensor(np.concatenate([[0], np.cumsum(wl.new_lens)]), dtype=torch.int32, device="cuda")
        self.dslots = torch.empty(self.T, dtype=torch.int64, device="cuda")
        self.side = torch.cuda.Stream()          # default priority
        self.written = torch.cuda.Event()
        # the same attention as one mixed batch, decode rows first
        # (pa_paged_attention): one launch plus the decode rows' merge
        order = self.dec + self.chunks
        self.qv = torch.cat([self.qd, self.qp])
        self.ov = torch.empty_like(self.qv)
        self.bt_v = h.table_dev[order].contiguous()
        self.sl_v = h.seq_lens_dev[order].contiguous()
        self.qsl_v_host = np.concatenate([[0], np.cumsum([wl.q_lens[s] for s in order])]).astype(np.int32)
        self.qsl_v = torch.from_numpy(self.qsl_v_host).cuda()
        self.msl_v = int(max(wl.seq_lens))
        self.ws_v = torch.empty(max(256, B.pa_paged_attention_workspace_size(self.qsl_v_host, wl.num_q_heads,
                                                                             wl.head_dim, self.msl_v, partition_size)),
                                dtype=torch.uint8, device="cuda")

    def slot_mapping(self):
        self.B.pa_slot_mapping(self.h.table_dev, self.qsl_all, self.h.seq_lens_dev, self.wl.block_size, self.T,
                               out=self.dslots)

    def reshape(self):
        self.B.pa_reshape_and_cache(self.kn, self.vn, self.h.kc, self.h.vc, self.dslots)

    def prefill(self):
        w = self.wl
        self.B.pa_paged_prefill(self.op, self.qp, self.h.kc, self.h.vc, self.bt_p, self.qsl, self.sl_p,
                                max(w.q_lens), self.msl_p, w.scale)

    def decode(self, stream=None):
        self.B.pa_paged_decode(self.od, self.qd, self.h.kc, self.h.vc, self.bt_d, self.sl_d, self.msl_d, self.wl.scale,
                               partition_size=self.P, workspace=self.ws, lse=self.lsed, stream=stream)

    def step(self):
        """All four on one stream."""
        self.slot_mapping()
        self.reshape()
        self.prefill()
        self.decode()

    def step_two_streams(self):
        """The decode on a second stream beside the prefill (the HBM-bound
        decode can use compute units the MFMA-bound prefill leaves idle);
        both wait for the cache writes, and the current stream waits for
        both."""
        torch = self.torch
        self.slot_mapping()
        self.reshape()
        self.written.record()
        self.side.wait_event(self.written)
        with torch.cuda.stream(self.side):
            self.decode()
        self.prefill()
        torch.cuda.current_stream().wait_stream(self.side)

    def varlen(self):
        w = self.wl
        self.B.pa_paged_attention(self.ov, self.qv, self.h.kc, self.h.vc, self.bt_v, self.qsl_v, self.qsl_v_host,
                                  self.sl_v, max(w.q_lens), self.msl_v, w.scale, partition_size=self.P,
                                  workspace=self.ws_v)

    def step_varlen(self):
        """The step's slots and writes, then its whole attention as one mixed
        batch."""
        self.slot_mapping()
        self.reshape()
        self.varlen()

    def close(self):
        del self.h, self.kn, self.vn
        self.torch.cuda.empty_cache()


# ------------------------------------------------------------ measurements


def traffic_from_counters(kind):
    """HBM bytes per launch from a committed FETCH_SIZE / WRITE_SIZE summary
    (each counter scaled by what it reads for a plain copy of known size);
    None when the summary is missing or was taken on other decode sources."""
    path = COUNTERS[kind]
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("decode_source_hash") != decode_source_hash():
        return None
    return int(float(vals["hbm_bytes_per_launch"]))


def measure_headline(torch, B, hip_side, workloads, steps, warmup, partition_size, kernel_reps=3):
    """The 32-layer long-context step: warm-up steps, then `steps` timed
    steps bracketed by synchronisation; then the layer launches of the last
    step repeated back to back under HIP events for the kernel roofline."""
    print("[bench] set-up: 32-layer long-context pool", file=sys.stderr, flush=True)
    st = LongContextStep(torch, B, hip_side, workloads, partition_size, max_steps=warmup + steps + 2)
    wl = st.wl
    torch.cuda.synchronize()
    for _ in range(max(warmup, 1)):
        st.step()
    torch.cuda.synchronize()
    warm_clocks(torch, st.relaunch, 0.5)
    print("[bench] warm-up done", file=sys.stderr, flush=True)
    kv_step = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.step()
        kv_step.append(kv_bytes(st.lens, wl.num_kv_heads, wl.head_dim) * st.L)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print("[bench] timed steps done", file=sys.stderr, flush=True)
    # the dominant kernels: the last step's 32 appending launches (partition
    # pass + merge each) again, back to back on the same stream
    sec = time_launches(torch, st.relaunch, kernel_reps)
    layer_s = sec / st.L
    alg = st.bytes_per_layer()
    nparts = -(-int(st.lens.max()) // partition_size)
    res = {"elapsed": elapsed, "kv_per_step": float(np.mean(kv_step)), "layer_s": layer_s, "alg": alg,
           "nparts": nparts, "S": st.S, "L": st.L, "max_seq_len": st.max_seq_len,
           "lens": [int(x) for x in st.lens]}
    st.close()
    return res


def measure_llama_decode(torch, B, hip_side, workloads, steps=40, warmup=4, instances=4, kernel_reps=48):
    """The Llama-3-8B decode batch of 64: the step (host pool append + one
    appending launch) over `instances` pools used in turn, so a step never
    finds its 141 MiB of K/V in the last-level cache from the step before;
    the appending launch alone and the plain decode launch, back to back."""
    wls = [workloads.llama_decode(seed_offset=i) for i in range(instances)]
    max_seq_len = max(max(w.seq_lens) for w in wls) + warmup + steps + 4
    wl = wls[0]
    S = wl.num_seqs
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    insts = [LlamaDecodeInstance(w, torch, B, hip_side, workloads, max_seq_len, 0, ws) for w in wls]
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(max(warmup, instances)):
        insts[i % instances].step(stream)
    torch.cuda.synchronize()
    warm_clocks(torch, lambda: [i.decode(stream) for i in insts], 0.5)
    step_lens = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step_lens.append(insts[k % instances].step(stream))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    rot = [0]

    def relaunch():
        insts[rot[0] % instances].relaunch(stream)
        rot[0] += 1

    def plain():
        insts[rot[0] % instances].decode(stream)
        rot[0] += 1
    t_app = time_launches(torch, relaunch, kernel_reps)
    t_plain = time_launches(torch, plain, kernel_reps)
    alg = float(np.mean([decode_bytes(i.h_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
                         for i in insts]))
    # the step's cache write alone: 64 new tokens' K and V rows to their slots
    w = insts[0]
    w_slots = torch.from_numpy(w.h_slots.copy()).cuda()
    kc0 = w.state.kc
    w_args = (w.new_k[0].data_ptr(), w.new_k[0].stride(0), w.new_v[0].data_ptr(), w.new_v[0].stride(0),
              kc0.data_ptr(), w.state.vc.data_ptr(), kc0.stride(0), wl.num_blocks, w_slots.data_ptr(), S,
              wl.num_kv_heads, wl.head_dim, wl.block_size, stream)
    t_w = time_launches(torch, lambda: w.lib.pa_reshape_and_cache(*w_args), 200)
    ms = el / steps * 1e3
    kv = float(np.mean([kv_bytes(l, wl.num_kv_heads, wl.head_dim) for l in step_lens]))
    res = {"workload": "64 sequences of 512 + U{0..100} tokens (+1 per step), 32/8 heads, d 128, B 16, "
                       f"8192-block pools, {instances} pools used in turn",
           "steps": steps, "ms_per_step": round(ms, 4), "step_gbps": round(kv / ms / 1e6, 1),
           "step_hbm_frac": hbm(kv / ms / 1e6), "seqs_per_s": round(S / ms * 1e3, 1),
           "roofline": {"bound": "hbm", "kernel": LLAMA_APPEND_KERNEL, "achieved": round(alg / t_app / 1e9, 2),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": hbm(alg / t_app / 1e9),
                        "traffic": traffic_from_counters("decode"), "algorithmic_bytes_per_launch": int(alg),
                        "launch_us": round(t_app * 1e6, 2)},
           "plain_kernel": {"kernel": LLAMA_PLAIN_KERNEL, "us": round(t_plain * 1e6, 2),
                            "gbps": round(alg / t_plain / 1e9, 1), "hbm_frac": hbm(alg / t_plain / 1e9),
                            "seqs_per_s": round(S / t_plain, 1)},
           "reshape_64_tokens_us": round(t_w * 1e6, 2)}
    del insts
    torch.cuda.empty_cache()
    return res


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
    del h
    torch.cuda.empty_cache()
    return {"workload": "16 prefill chunks of 512 queries over U{0..8192} context tokens",
            "block_size": block_size, "kernel": PREFILL_KERNEL,
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


def measure_long_context_partitions(torch, B, hip_side, workloads, sizes=(256, 1024, 2048), reps=3):
    """Plain decode over the 32-layer pool (no token write) at several
    partition sizes (up to 1024 tokens the row layout, above it the head
    layout): every layer with its own queries, per layer and per 32-layer
    pass."""
    st = LongContextStep(torch, B, hip_side, workloads, sizes[0], max_steps=2)
    wl = st.wl
    L, S = st.L, st.S
    msl = st.max_seq_len
    per_layer = st.bytes_per_layer()
    res = {"workload": "8 sequences of U{16384..32768} tokens over a 32-layer pool of 26,785 blocks per layer",
           "pool_gib": round(st.kv.numel() * 2 / 2**30, 2), "layers": L, "bytes_per_layer": per_layer}
    for P in sizes:
        ws = torch.empty(max(256, B.pa_paged_decode_workspace_size(S, wl.num_q_heads, wl.head_dim, msl, P)),
                         dtype=torch.uint8, device="cuda")

        def one_pass():
            for l in range(L):
                B.pa_paged_decode(st.out[l], st.q[0, l], st.kv[l, 0], st.kv[l, 1], st.h.table_dev,
                                  st.h.seq_lens_dev, msl, wl.scale, partition_size=P, workspace=ws)
        sec = time_launches(torch, one_pass, reps)
        res[f"plain_p{P}"] = {"layout": "rows" if P <= 1024 else "heads",
                              "pass_ms": round(sec * 1e3, 3), "layer_us": round(sec / L * 1e6, 1),
                              "gbps": round(per_layer * L / sec / 1e9, 1),
                              "hbm_frac": hbm(per_layer * L / sec / 1e9), "seqs_per_s": round(S / sec, 1)}
        del ws
    st.close()
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
    kn = torch.cat([workloads.device_seq_kv(wl.seed, s, wl.new_lens[s], wl.num_kv_heads, wl.head_dim, 0, 9)[0]
                    for s in seqs])
    slots = torch.from_numpy(np.asarray(h.step_slots, dtype=np.int64)).cuda()
    T = int(kn.shape[0])
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
    """The mixed step at one block size: each call timed alone and the step
    on one stream and with the decode on a second stream."""
    m = MixedStep(torch, B, hip_side, workloads, block_size)
    wl = m.wl
    m.slot_mapping()
    t_m = time_launches(torch, m.slot_mapping, reps)
    t_r = time_launches(torch, m.reshape, reps)
    t_p = time_launches(torch, m.prefill, reps)
    t_d = time_launches(torch, m.decode, reps)
    t_s = time_launches(torch, m.step, reps)
    t_s2 = time_launches(torch, m.step_two_streams, reps)
    t_v = time_launches(torch, m.varlen, reps)
    t_sv = time_launches(torch, m.step_varlen, reps)
    flops = prefill_flops([wl.q_lens[s] for s in m.chunks], [wl.seq_lens[s] for s in m.chunks], wl.num_q_heads,
                          wl.head_dim)
    db = decode_bytes(m.dl, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, block_size)
    rb = 2 * m.T * wl.num_kv_heads * wl.head_dim * 2 * 2
    res = {"block_size": block_size, "decode_partition_size": m.P, "step_ms": round(t_s * 1e3, 3),
           "step_two_streams_ms": round(t_s2 * 1e3, 3), "step_one_launch_ms": round(t_sv * 1e3, 3),
           "attention_one_launch_us": round(t_v * 1e6, 1),
           "attention_one_launch_note": "prefill chunks and decode rows in one pa_paged_attention launch "
                                        "(+ the decode merge)", "tokens_written": m.T,
           "slot_mapping_us": round(t_m * 1e6, 2),
           "reshape_us": round(t_r * 1e6, 2), "reshape_gbps": round(rb / t_r / 1e9, 1),
           "prefill_us": round(t_p * 1e6, 1), "prefill_gflop": round(flops / 1e9, 2),
           "prefill_tflops": round(flops / t_p / 1e12, 1),
           "prefill_mfma_frac": round(flops / t_p / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "decode_us": round(t_d * 1e6, 1), "decode_bytes": db, "decode_gbps": round(db / t_d / 1e9, 1),
           "decode_hbm_frac": hbm(db / t_d / 1e9), "decode_seqs_per_s": round(len(m.dec) / t_d, 1)}
    m.close()
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
        _check(L, L.pa_pool_cache_blocks(h, 0, tp, prompt))
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
        _check(L, L.pa_pool_append_batch(*args))
    t_app = (time.perf_counter() - t0) / n
    B.pa_pool_check(pool)
    return {"num_blocks": num_blocks, "block_size": block_size, "prompt_tokens": prompt,
            "cache_blocks_us": round(t_cache * 1e6, 1),
            "hash_mtok_per_s": round(prompt / t_cache / 1e6, 1),
            "prefix_hit_us": round(t_hit / reps * 1e6, 1), "free_seq_us": round(t_free / reps * 1e6, 1),
            f"append_batch_{batch}x1_us": round(t_app * 1e6, 2)}


def measure_fp8_decode(torch, B, hip_side, workloads, scales=FP8_SCALES, instances=8, reps=48):
    """Decode over E4M3 caches: the 64-sequence Llama-3-8B decode batch
    (8 pools rotated, about 590 MB of K/V codes, so that no pool stays in the
    last-level cache between its calls) and the 32-layer long-context pool;
    plus the quantising cache write of one decode step's 64 tokens and the
    mixed step's prefill chunks over E4M3 caches."""
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
    k = hip_side.to_device(workloads.normal_bf16(np.random.default_rng(1), (S, wl.num_kv_heads, wl.head_dim)))
    slots = torch.from_numpy(hs[0].step_slots.astype(np.int64)).cuda()
    B.pa_reshape_and_cache_fp8(k, k, hs[0].kc, hs[0].vc, slots, *scales)          # argument checks
    w_args = (k.data_ptr(), k.stride(0), k.data_ptr(), k.stride(0), hs[0].kc.data_ptr(), hs[0].vc.data_ptr(),
              hs[0].kc.stride(0), wl.num_blocks, slots.data_ptr(), S, wl.num_kv_heads, wl.head_dim, wl.block_size,
              scales[0], scales[1], torch.cuda.current_stream().cuda_stream)
    L = B.lib()
    t_w = time_launches(torch, lambda: L.pa_reshape_and_cache_fp8(*w_args), 200)
    res = {"workload": f"{wl.name}, E4M3 K/V with per-cache scales", "scales": list(scales),
           "kernel": FP8_KERNEL, "decode_us": round(sec * 1e6, 2),
           "bytes_per_launch": int(alg), "gbps": round(gbps, 1), "hbm_frac": hbm(gbps),
           "seqs_per_s": round(S / sec, 1), "write_64_tokens_us": round(t_w * 1e6, 2)}
    del hs, qs
    torch.cuda.empty_cache()

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
                      "kernel": "prefill_kernel<128, 4, true, true, true, 0>", "us": round(t_p * 1e6, 1),
                      "tflops": round(pflops / t_p / 1e12, 1),
                      "frac": round(pflops / t_p / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    del ph, pq, pout
    torch.cuda.empty_cache()

    wl = workloads.long_context()
    L_, S, P = wl.num_layers, wl.num_seqs, FP8_LONG_CONTEXT_PARTITION
    kv = torch.full((L_, 2, wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim), 0x7F,
                    dtype=torch.uint8, device="cuda")
    h = hip_side.HipStep(wl, gen="device", caches=(kv[0, 0], kv[0, 1]),
                         layers=[(l, kv[l, 0], kv[l, 1]) for l in range(L_)], fp8=scales)
    msl = max(wl.seq_lens)
    qs = [workloads.device_query(wl.seed, S, wl.num_q_heads, wl.head_dim, layer=l) for l in range(L_)]
    out = torch.empty_like(qs[0])
    ws = torch.empty(B.pa_paged_decode_workspace_size(S, wl.num_q_heads, wl.head_dim, msl, P),
                     dtype=torch.uint8, device="cuda")

    def one_pass():
        for l in range(L_):
            B.pa_paged_decode_fp8(out, qs[l], kv[l, 0], kv[l, 1], h.table_dev, h.seq_lens_dev, msl, wl.scale,
                                  *scales, partition_size=P, workspace=ws)
    sec = time_launches(torch, one_pass, 3)
    per_layer = decode_bytes(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, 1)
    gbps = per_layer * L_ / sec / 1e9
    res["long_context"] = {"pool_gib": round(kv.numel() / 2**30, 2), "partition_size": P,
                           "kernel": f"{FP8_LONG_CONTEXT_KERNEL} + {MERGE_KERNEL}",
                           "pass_ms": round(sec * 1e3, 3), "layer_us": round(sec / L_ * 1e6, 1),
                           "bytes_per_layer": per_layer, "gbps": round(gbps, 1), "hbm_frac": hbm(gbps),
                           "seqs_per_s": round(S / sec, 1),
                           "roofline": {"bound": "hbm", "kernel": f"{FP8_LONG_CONTEXT_KERNEL} + {MERGE_KERNEL}",
                                        "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                        "frac": hbm(gbps), "traffic": traffic_from_counters("fp8_long_context"),
                                        "algorithmic_bytes_per_launch": per_layer,
                                        "launch": "one layer's decode call (partition pass + merge), timed over "
                                                  "back-to-back passes of the 32 layer calls"}}
    del kv, h, qs
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ oracle timing


def oracle_threads():
    """Threads the oracle may use: the cores this process may run on, capped
    by OMP_NUM_THREADS when the environment sets it (the machine's CPU share)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return n


def blas_vendor():
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:                                   # noqa: BLE001 (informational only)
        return "unknown"


def _median_of_3(fn):
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts)


def cpu_baseline():
    """The oracle (numpy fp64, as committed) timed on the host, median of 3
    per workload, in the GPU's units.  The headline entry is one layer of
    the long-context step (all 8 sequences); the others time the tiny decode,
    the Llama-3-8B batch of 64, the 256 forked sequences, and a sample of the
    mixed step (2 of its 16 prefill chunks, 24 of its 240 decode sequences,
    with their drawn lengths)."""
    from threadpoolctl import threadpool_limits

    from oracle import attention
    from paged_kv_cache_327_amd import workloads
    from tests.oracle_side import OracleStep
    threads = oracle_threads()
    vendor = blas_vendor()
    out = {}
    with threadpool_limits(limits=threads):
        def decode_case(wl, label, sample):
            o = OracleStep(wl)
            q = workloads.query_bits(wl.seed, wl.num_seqs, wl.num_q_heads, wl.head_dim)
            t = _median_of_3(lambda: attention.paged_decode(q, o.kc, o.vc, o.table, o.seq_lens, wl.scale))
            b = decode_bytes(o.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
            out[label] = {"value": round(b / t / 1e9, 4), "unit": "GB/s", "s_per_call": round(t, 4),
                          "seqs_per_s": round(wl.num_seqs / t, 2), "sample": sample}
            del o

        print("[bench] oracle: long-context layer", file=sys.stderr, flush=True)
        decode_case(workloads.long_context(), "long_context_decode",
                    "one layer of the long-context step: all 8 sequences of U{16384..32768} tokens")
        print("[bench] oracle: tiny, Llama batch, prefix sharing", file=sys.stderr, flush=True)
        decode_case(workloads.tiny_decode(), "tiny_decode", "the whole tiny decode")
        decode_case(workloads.llama_decode(), "llama3_8b_decode", "the whole 64-sequence batch")
        decode_case(workloads.prefix_cow(), "prefix_cow_decode", "all 256 forked sequences (logical bytes)")

        print("[bench] oracle: mixed-step sample", file=sys.stderr, flush=True)
        m = workloads.mixed_step(16)
        chunks = [s for s in range(m.num_seqs) if m.q_lens[s] > 1][:2]
        dec = [s for s in range(m.num_seqs) if m.q_lens[s] == 1][:24]
        seqs = chunks + dec
        lens = [m.seq_lens[s] for s in seqs]
        qls = [m.q_lens[s] for s in seqs]
        wl = workloads.custom("mixed_step_sample", m.seed, m.num_q_heads, m.num_kv_heads, m.head_dim, 16, lens,
                              q_lens=qls)
        o = OracleStep(wl)
        npre = len(chunks)
        q = workloads.query_bits(wl.seed, int(sum(qls[:npre])), wl.num_q_heads, wl.head_dim)
        qsl = np.concatenate([[0], np.cumsum(qls[:npre])])
        t_p = _median_of_3(lambda: attention.paged_prefill(q, o.kc, o.vc, o.table[:npre], qsl, o.seq_lens[:npre],
                                                           wl.scale))
        fl = prefill_flops(qls[:npre], lens[:npre], wl.num_q_heads, wl.head_dim)
        qd = workloads.query_bits(wl.seed, len(dec), wl.num_q_heads, wl.head_dim, layer=1)
        t_d = _median_of_3(lambda: attention.paged_decode(qd, o.kc, o.vc, o.table[npre:], o.seq_lens[npre:],
                                                          wl.scale))
        db = decode_bytes(lens[npre:], wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 16)
        out["mixed_step_b16"] = {"prefill_tflops": round(fl / t_p / 1e12, 5), "prefill_s": round(t_p, 3),
                                 "decode_gbps": round(db / t_d / 1e9, 4), "decode_s": round(t_d, 4),
                                 "decode_seqs_per_s": round(len(dec) / t_d, 2),
                                 "sample": f"prefill chunks {chunks} (512 queries over {lens[0] - 512} and "
                                           f"{lens[1] - 512} context tokens) and decode sequences {dec[0]}.."
                                           f"{dec[-1]} of the mixed step, B 16"}
        del o
    head = out.pop("long_context_decode")
    return {"value": head["value"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{head['sample']}; median of 3 calls of {head['s_per_call']} s; numpy fp64 with "
                      f"{threads} BLAS threads ({vendor})",
            "seqs_per_s": head["seqs_per_s"], "blas": vendor, "configs": out}


# ------------------------------------------------------------ profiling


def counter_run(kind, reps):
    """Launch one kernel kind, for rocprofv3 --pmc passes:
    'long_context' = two steps of the headline (appending decode + merge per
    layer), 'decode' = the Llama batch's appending launch on rotating pools,
    'copy' = a plain device copy of COPY_CALIBRATION_BYTES (calibration),
    'prefill' = the mixed step's prefill chunks (MFMA counters),
    'fp8_long_context' = two passes over the 32-layer E4M3 pool (decode +
    merge per layer)."""
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
    if kind == "fp8_long_context":
        wl = workloads.long_context()
        L_, S, P = wl.num_layers, wl.num_seqs, FP8_LONG_CONTEXT_PARTITION
        kv = torch.full((L_, 2, wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim), 0x7F,
                        dtype=torch.uint8, device="cuda")
        h = hip_side.HipStep(wl, gen="device", caches=(kv[0, 0], kv[0, 1]),
                             layers=[(l, kv[l, 0], kv[l, 1]) for l in range(L_)], fp8=FP8_SCALES)
        msl = max(wl.seq_lens)
        qs = [workloads.device_query(wl.seed, S, wl.num_q_heads, wl.head_dim, layer=l) for l in range(L_)]
        out = torch.empty_like(qs[0])
        ws = torch.empty(B.pa_paged_decode_workspace_size(S, wl.num_q_heads, wl.head_dim, msl, P),
                         dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        print("E4M3 long-context set-up done", flush=True)
        for _ in range(2):
            for l in range(L_):
                B.pa_paged_decode_fp8(out, qs[l], kv[l, 0], kv[l, 1], h.table_dev, h.seq_lens_dev, msl, wl.scale,
                                      *FP8_SCALES, partition_size=P, workspace=ws)
        torch.cuda.synchronize()
        print(f"E4M3 long-context passes x 2 ({L_} layers each, partitions of {P}); algorithmic bytes per layer "
              f"{decode_bytes(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, 1)}",
              flush=True)
        return
    if kind == "long_context":
        st = LongContextStep(torch, B, hip_side, workloads, HEADLINE_PARTITION, max_steps=4)
        torch.cuda.synchronize()
        print("long-context set-up done", flush=True)
        for _ in range(2):
            st.step()
        torch.cuda.synchronize()
        print(f"long-context steps x 2 ({st.L} layers each); algorithmic bytes per layer "
              f"{st.bytes_per_layer()} after the second step", flush=True)
        return
    wls = [workloads.llama_decode(seed_offset=i) for i in range(4)]
    msl = max(max(w.seq_lens) for w in wls) + reps + 8
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    insts = [LlamaDecodeInstance(w, torch, B, hip_side, workloads, msl, 0, ws) for w in wls]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    algs = []
    for k in range(reps):
        lens = insts[k % 4].step(stream)
        algs.append(decode_bytes(lens, 32, 8, 128, 16))
    torch.cuda.synchronize()
    print(f"decode steps x {reps}; algorithmic bytes per launch {np.mean(algs):.0f}", flush=True)


def _read_counter_csv(d):
    """{kernel name: [counter value per dispatch]} from the counter CSV(s)
    rocprofv3 wrote under directory d (one counter per run)."""
    rows = {}
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return rows


def _kernel_avg(rows, *keys):
    """Average per dispatch over the kernels whose name contains every key."""
    vals = [v for k, vs in rows.items() if all(key in k for key in keys) for v in vs]
    if not vals:
        raise SystemExit(f"no dispatch of {keys}")
    return sum(vals) / len(vals), len(vals)


def counter_summary(kind, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, alg, command):
    """Write the traffic summary of `kind` ('long_context' or 'decode') from
    four rocprofv3 --pmc output directories (FETCH_SIZE and WRITE_SIZE of the
    counter run, and of the copy calibration run); `alg` is the run's
    algorithmic bytes per layer (or launch), `command` the profiling
    commands."""
    copy_f, _ = _kernel_avg(_read_counter_csv(copy_fetch_dir))
    copy_w, _ = _kernel_avg(_read_counter_csv(copy_write_dir))
    kib = COPY_CALIBRATION_BYTES / 1024
    ff, wf = kib / copy_f, kib / copy_w
    fr, wr = _read_counter_csv(fetch_dir), _read_counter_csv(write_dir)
    # every appending launch of the run (their bytes differ by one token)
    kernel = {"long_context": APPEND_KERNEL, "decode": LLAMA_APPEND_KERNEL, "fp8_long_context": FP8_LONG_CONTEXT_KERNEL}[kind]
    f_app, n_app = _kernel_avg(fr, kernel + "(")
    w_app, _ = _kernel_avg(wr, kernel + "(")
    f_mrg, n_mrg = _kernel_avg(fr, "decode_merge") if any("decode_merge" in k for k in fr) else (0.0, 0)
    w_mrg, _ = _kernel_avg(wr, "decode_merge") if any("decode_merge" in k for k in wr) else (0.0, 0)
    per_launch = (f_app + f_mrg) * 1024 * ff + (w_app + w_mrg) * 1024 * wf
    name = {"long_context": "one layer of the 32-layer long-context step (appending decode + merge)",
            "decode": "the Llama-3-8B batch of 64 (appending decode launch)",
            "fp8_long_context": "one layer of the 32-layer E4M3 long-context pool (decode + merge, partitions of "
                                f"{FP8_LONG_CONTEXT_PARTITION})"}[kind]
    lines = [
        f"# HBM traffic of {name}",
        f"# kernels: {kernel}" + (f" and {MERGE_KERNEL}" if n_mrg else ""),
        "#",
        "# Commands (from /tmp, TMPDIR=/tmp), one counter per run:",
        *[f"#   {c}" for c in command.split(" ;; ")],
        "#",
        f"# Calibration: a plain device copy of {COPY_CALIBRATION_BYTES} bytes reads FETCH_SIZE = {copy_f:.1f} KiB",
        f"# and WRITE_SIZE = {copy_w:.1f} KiB per dispatch: fetch factor {ff:.3f}, write factor {wf:.3f}.",
        f"# Averages over {n_app} " + ("decode" if kind == "fp8_long_context" else "appending") + " launches" +
        (f" and {n_mrg} merge launches" if n_mrg else "") +
        " (KiB per dispatch).",
        f"fetch_size_kib = {f_app:.2f}",
        f"write_size_kib = {w_app:.2f}",
        f"merge_fetch_size_kib = {f_mrg:.2f}",
        f"merge_write_size_kib = {w_mrg:.2f}",
        f"fetch_factor = {ff:.4f}",
        f"write_factor = {wf:.4f}",
        f"hbm_bytes_per_launch = {per_launch:.0f}",
        f"algorithmic_bytes_per_launch = {alg}",
        f"ratio = {per_launch / alg:.4f}",
        f"decode_source_hash = {decode_source_hash()}",
    ]
    path = COUNTERS[kind]
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(path).read())


def trace_summary(stats_csv, title, command):
    """Markdown table of a rocprofv3 --stats kernel summary."""
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    print(f"# {title}\n\nCommand:\n\n    {command}\n")
    print("| kernel | calls | avg us | min us | max us | % time |\n|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"]
        for pre in ("pa::(anonymous namespace)::", "pa::"):
            name = name.replace(pre, "")
        print(f"| {name[:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")


# ------------------------------------------------------------------ main


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--partition-size", type=int, default=HEADLINE_PARTITION,
                    help="split-K partition of the headline step's decode")
    ap.add_argument("--kernel-reps", type=int, default=3,
                    help="back-to-back repeats of the headline step's 32 layer launches for the roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads")
    ap.add_argument("--counter-run", choices=["long_context", "decode", "copy", "prefill", "fp8_long_context"],
                    help="only launch one kernel kind (for rocprofv3 --pmc passes) and exit")
    ap.add_argument("--counter-summary", nargs=5, metavar=("KIND", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write profiles/<kind> traffic summary from four rocprofv3 --pmc output dirs")
    ap.add_argument("--alg-bytes", type=int, help="algorithmic bytes per launch of the counter run")
    ap.add_argument("--command", default="", help="profiling commands for a summary (';;'-separated)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "TITLE"))
    args = ap.parse_args()
    if args.counter_summary:
        counter_summary(*args.counter_summary, args.alg_bytes, args.command)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary, args.command)
        return
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
    P = args.partition_size
    r = measure_headline(torch, B, hip_side, workloads, args.steps, args.warmup, P, args.kernel_reps)
    ms_per_step = r["elapsed"] / args.steps * 1e3
    value = r["kv_per_step"] / (ms_per_step / 1e3) / 1e9
    achieved = r["alg"] / r["layer_s"] / 1e9
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
        "config": {"workload": "long_context_decode", "layers": r["L"], "batch": r["S"], "num_q_heads": 32,
                   "num_kv_heads": 8, "head_dim": 128, "block_size": 16, "num_blocks_per_layer": 26785,
                   "pool_gib": 52.31, "context": "U{16384..32768} (+1 per step)", "partition_size": P,
                   "step": "host pool append + 32 x pa_paged_decode_append (token write, table update, "
                           "split-K decode, merge)"},
        "seqs_per_s": round(r["S"] / (ms_per_step / 1e3), 1),
        "step_hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "layer_us": round(r["layer_s"] * 1e6, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": f"{APPEND_KERNEL} + {MERGE_KERNEL}" if r["nparts"] > 1 else APPEND_KERNEL,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_counters("long_context"),
            "algorithmic_bytes_per_launch": int(r["alg"]),
            "launch": "one layer's appending decode call (partition pass + merge), timed over back-to-back "
                      "repeats of the step's 32 layer calls",
        },
        "cpu_baseline": None,
    }
    print(f"[bench] headline {value:.0f} GB/s", file=sys.stderr, flush=True)
    if not args.no_prefill:
        print("[bench] prefill", file=sys.stderr, flush=True)
        line["prefill"] = measure_prefill(torch, B, hip_side, workloads)
    if not args.no_configs:
        cfg = {}
        print("[bench] Llama-3-8B decode batch", file=sys.stderr, flush=True)
        cfg["llama3_8b_decode"] = measure_llama_decode(torch, B, hip_side, workloads)
        print("[bench] tiny decode, copy bandwidth", file=sys.stderr, flush=True)
        cfg["tiny_decode"] = measure_tiny(torch, B, hip_side, workloads)
        cfg["d2d_copy"] = measure_copy_bandwidth(torch)
        print("[bench] long-context plain decode", file=sys.stderr, flush=True)
        cfg["long_context_decode"] = measure_long_context_partitions(torch, B, hip_side, workloads)
        print("[bench] prefix sharing + copy-on-write", file=sys.stderr, flush=True)
        cfg["prefix_cow_decode"] = measure_prefix_cow(torch, B, hip_side, workloads)
        for bs in (1, 16, 32):
            print(f"[bench] mixed step, block size {bs}", file=sys.stderr, flush=True)
            cfg[f"mixed_step_b{bs}"] = measure_mixed(torch, B, hip_side, workloads, bs)
        print("[bench] E4M3 KV cache", file=sys.stderr, flush=True)
        cfg["fp8_decode"] = measure_fp8_decode(torch, B, hip_side, workloads)
        line["configs"] = cfg
    line["host_pool"] = measure_host_pool(B)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
