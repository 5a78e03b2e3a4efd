"""Thin ctypes binding of libpagedattn with the C-ABI's names.

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream, numpy arrays supply host buffers; every computation
runs in the library.  Loading fails loudly when the library is not built.
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np

PA_OK, PA_ERR_INVALID, PA_ERR_NO_SPACE, PA_ERR_HIP, PA_ERR_NO_MEMORY = 0, -1, -2, -3, -4

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pagedattn.h")


class PagedAttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class InvalidArgument(PagedAttnError):
    pass


class NoSpace(PagedAttnError):
    pass


class HipError(PagedAttnError):
    pass


class NoMemory(PagedAttnError):
    pass


_ERRORS = {PA_ERR_INVALID: InvalidArgument, PA_ERR_NO_SPACE: NoSpace, PA_ERR_HIP: HipError, PA_ERR_NO_MEMORY: NoMemory}

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
P_i32, P_i64 = ctypes.POINTER(c_i32), ctypes.POINTER(c_i64)

_SIGS = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_pool_create": (c_i32, [c_i32, c_i32, P_i32, ctypes.POINTER(c_vp)]),
    "pa_pool_destroy": (None, [c_vp]),
    "pa_pool_add_seq": (c_i32, [c_vp, c_i64]),
    "pa_pool_add_seq_cached": (c_i32, [c_vp, c_i64, P_i32, c_i64, P_i64]),
    "pa_pool_cache_blocks": (c_i32, [c_vp, c_i64, P_i32, c_i64]),
    "pa_pool_pin": (c_i32, [c_vp, c_i64, c_i64, P_i32, c_i32, P_i32]),
    "pa_pool_unpin": (c_i32, [c_vp, c_i64]),
    "pa_pool_copies_done": (c_i32, [c_vp]),
    "pa_pool_num_cached": (c_i32, [c_vp, P_i32]),
    "pa_pool_stats": (c_i32, [c_vp, P_i64, c_i32]),
    "pa_pool_block_state": (c_i32, [c_vp, c_i32, P_i32, P_i32, ctypes.POINTER(ctypes.c_uint64), P_i32]),
    "pa_pool_fork": (c_i32, [c_vp, c_i64, c_i64]),
    "pa_pool_append": (c_i32, [c_vp, c_i64, c_i32, P_i64, P_i32]),
    "pa_pool_append_batch": (c_i32, [c_vp, P_i64, P_i32, c_i32, P_i64, P_i32, P_i32]),
    "pa_pool_free_seq": (c_i32, [c_vp, c_i64]),
    "pa_pool_block_table": (c_i32, [c_vp, P_i64, c_i32, P_i32, c_i32, P_i32]),
    "pa_pool_kernel_block_table": (c_i32, [c_vp, P_i64, c_i32, c_i32, P_i32, c_i32, P_i32]),
    "pa_pool_num_free": (c_i32, [c_vp, P_i32]),
    "pa_pool_refcount": (c_i32, [c_vp, c_i32, P_i32]),
    "pa_pool_seq_len": (c_i32, [c_vp, c_i64, P_i64]),
    "pa_pool_free_order": (c_i32, [c_vp, P_i32, c_i32, P_i32]),
    "pa_pool_check": (c_i32, [c_vp]),
    "pa_blocks_for_bytes": (c_i64, [c_i64, c_i64, c_i32]),
    "pa_slot_mapping": (c_i32, [c_vp, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_vp]),
    "pa_reshape_and_cache": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_i32, c_vp,
                                     c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pa_reshape_and_cache_fp8": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_i32, c_vp,
                                         c_i32, c_i32, c_i32, c_i32, c_f32, c_f32, c_vp]),
    "pa_decode_append": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_vp, P_i64,
                                 P_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pa_copy_blocks_device": (c_i32, [ctypes.POINTER(c_vp), c_i32, c_i64, c_i64, c_i32, c_vp, c_i32, c_vp]),
    "pa_copy_blocks": (c_i32, [ctypes.POINTER(c_vp), c_i32, c_i64, c_i64, c_i32, P_i32, c_i32, c_vp]),
    "pa_paged_decode_workspace_size": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_paged_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_vp,
                                c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_vp, c_sz, c_vp]),
    "pa_paged_decode_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_vp,
                                        c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_vp]),
    "pa_paged_decode_append": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_vp,
                                       c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32,
                                       c_vp, c_i64, c_vp, c_i64, P_i64, P_i32, c_vp, c_sz, c_vp]),
    "pa_paged_decode_fp8": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_vp,
                                    c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_f32, c_f32,
                                    c_vp, c_sz, c_vp]),
    "pa_paged_prefill_fp8": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_vp, c_vp,
                                     c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_f32, c_f32,
                                     c_i32, c_vp]),
    "pa_paged_attention_workspace_size": (c_sz, [P_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_paged_attention": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_vp, P_i32, c_vp,
                                   c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_i32,
                                   c_vp, c_sz, c_vp]),
    "pa_paged_prefill": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_vp, c_vp,
                                 c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp]),
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m paged_kv_cache_327_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_symbols():
    """Names of the functions include/pagedattn.h declares."""
    with open(HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def _check(rc):
    if rc != PA_OK:
        msg = lib().pa_last_error().decode()
        raise _ERRORS.get(rc, PagedAttnError)(rc, msg)


def _i32p(a):
    return a.ctypes.data_as(P_i32)


def _i64p(a):
    return a.ctypes.data_as(P_i64)


# ---------------------------------------------------------------- host pool


class Pool:
    """Owner of a pa_pool handle (destroyed with the object)."""

    def __init__(self, handle, num_blocks, block_size):
        self.handle = handle
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.pa_pool_destroy(h)


def pa_pool_create(num_blocks, block_size, initial_free_order=None) -> Pool:
    h = c_vp()
    order = None
    if initial_free_order is not None:
        order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
        if order.shape != (num_blocks,):
            raise InvalidArgument(PA_ERR_INVALID, "initial_free_order must have num_blocks entries")
    _check(lib().pa_pool_create(num_blocks, block_size, _i32p(order) if order is not None else None,
                                ctypes.byref(h)))
    return Pool(h.value, num_blocks, block_size)


def pa_pool_destroy(pool: Pool):
    h, pool.handle = pool.handle, None
    if h:
        lib().pa_pool_destroy(h)


def pa_pool_add_seq(pool, seq_id):
    _check(lib().pa_pool_add_seq(pool.handle, seq_id))


def pa_pool_add_seq_cached(pool, seq_id, tokens):
    """Registers seq_id with its cached prefix blocks; returns the hit tokens."""
    t = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
    hit = c_i64()
    _check(lib().pa_pool_add_seq_cached(pool.handle, seq_id, _i32p(t), len(t), ctypes.byref(hit)))
    return hit.value


def pa_pool_cache_blocks(pool, seq_id, tokens):
    t = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
    _check(lib().pa_pool_cache_blocks(pool.handle, seq_id, _i32p(t), len(t)))


def pa_pool_pin(pool, seq_id, transfer_id):
    """Pins seq_id's blocks for transfer_id; returns the pinned ids (list)."""
    n = c_i32()
    cap = -(-pa_pool_seq_len(pool, seq_id) // pool.block_size)
    out = np.empty(max(cap, 1), dtype=np.int32)
    _check(lib().pa_pool_pin(pool.handle, seq_id, transfer_id, _i32p(out), cap, ctypes.byref(n)))
    return out[:n.value].tolist()


def pa_pool_unpin(pool, transfer_id):
    _check(lib().pa_pool_unpin(pool.handle, transfer_id))


def pa_pool_copies_done(pool):
    _check(lib().pa_pool_copies_done(pool.handle))


def pa_pool_stats(pool):
    """dict(used_blocks, free_blocks, cached_blocks, tokens, tail_waste_slots)."""
    out = np.zeros(5, dtype=np.int64)
    _check(lib().pa_pool_stats(pool.handle, _i64p(out), 5))
    return dict(zip(("used_blocks", "free_blocks", "cached_blocks", "tokens", "tail_waste_slots"),
                    out.tolist()))


def pa_pool_num_cached(pool):
    out = c_i32()
    _check(lib().pa_pool_num_cached(pool.handle, ctypes.byref(out)))
    return out.value


def pa_pool_block_state(pool, block_id):
    """Returns (pins, pending copies, hash or None)."""
    pins, pend, hashed = c_i32(), c_i32(), c_i32()
    h = ctypes.c_uint64()
    _check(lib().pa_pool_block_state(pool.handle, block_id, ctypes.byref(pins), ctypes.byref(pend),
                                     ctypes.byref(h), ctypes.byref(hashed)))
    return pins.value, pend.value, (h.value if hashed.value else None)


def pa_pool_fork(pool, src_seq, dst_seq):
    _check(lib().pa_pool_fork(pool.handle, src_seq, dst_seq))


def pa_pool_append(pool, seq_id, n_tokens):
    """Returns (slots int64 [n], (src, dst) or None)."""
    slots = np.empty(max(n_tokens, 0), dtype=np.int64)
    pair = np.empty(2, dtype=np.int32)
    _check(lib().pa_pool_append(pool.handle, seq_id, n_tokens, _i64p(slots), _i32p(pair)))
    return slots, (None if pair[0] < 0 else (int(pair[0]), int(pair[1])))


def pa_pool_append_batch(pool, seq_ids, n_tokens):
    """Returns (slots concatenated int64, pairs int32 [n, 2]); raises on the
    first failing sequence with .n_done set on the exception."""
    ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    nt = np.ascontiguousarray(n_tokens, dtype=np.int32)
    slots = np.empty(int(nt.sum()), dtype=np.int64)
    pairs = np.empty((len(ids), 2), dtype=np.int32)
    done = c_i32(0)
    rc = lib().pa_pool_append_batch(pool.handle, _i64p(ids), _i32p(nt), len(ids), _i64p(slots),
                                    _i32p(pairs), ctypes.byref(done))
    try:
        _check(rc)
    except PagedAttnError as e:
        e.n_done = done.value
        raise
    return slots, pairs


def pa_pool_free_seq(pool, seq_id):
    _check(lib().pa_pool_free_seq(pool.handle, seq_id))


def pa_pool_block_table(pool, seq_ids, bt_stride, out=None, fill=0):
    """Returns (table int32 [n, bt_stride], seq_lens int32 [n]); entries past
    each row's blocks keep `fill` (or the content of `out`)."""
    ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    table = out if out is not None else np.full((len(ids), bt_stride), fill, dtype=np.int32)
    assert table.dtype == np.int32 and table.flags.c_contiguous and table.shape == (len(ids), bt_stride)
    lens = np.empty(len(ids), dtype=np.int32)
    _check(lib().pa_pool_block_table(pool.handle, _i64p(ids), len(ids), _i32p(table), bt_stride, _i32p(lens)))
    return table, lens


def pa_pool_kernel_block_table(pool, seq_ids, kernel_block_size, bt_stride, fill=0):
    """Returns (table int32 [n, bt_stride] of kernel-block ids, seq_lens
    int32 [n])."""
    ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    table = np.full((len(ids), bt_stride), fill, dtype=np.int32)
    lens = np.empty(len(ids), dtype=np.int32)
    _check(lib().pa_pool_kernel_block_table(pool.handle, _i64p(ids), len(ids), kernel_block_size, _i32p(table),
                                            bt_stride, _i32p(lens)))
    return table, lens


def pa_pool_num_free(pool):
    out = c_i32()
    _check(lib().pa_pool_num_free(pool.handle, ctypes.byref(out)))
    return out.value


def pa_pool_refcount(pool, block_id):
    out = c_i32()
    _check(lib().pa_pool_refcount(pool.handle, block_id, ctypes.byref(out)))
    return out.value


def pa_pool_seq_len(pool, seq_id):
    out = c_i64()
    _check(lib().pa_pool_seq_len(pool.handle, seq_id, ctypes.byref(out)))
    return out.value


def pa_pool_free_order(pool):
    n = pa_pool_num_free(pool)
    out = np.empty(max(n, 1), dtype=np.int32)
    got = c_i32()
    _check(lib().pa_pool_free_order(pool.handle, _i32p(out), n, ctypes.byref(got)))
    return out[:got.value].tolist()


def pa_pool_check(pool):
    _check(lib().pa_pool_check(pool.handle))


def pa_blocks_for_bytes(pool_bytes, bytes_per_token, block_size):
    return lib().pa_blocks_for_bytes(pool_bytes, bytes_per_token, block_size)


# ------------------------------------------------------------- device calls


def _stream(t, stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _bf16(t, name):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise InvalidArgument(PA_ERR_INVALID, f"{name} must be a bf16 device tensor")


def _scratch(nbytes, device, stream):
    """A workspace allocated here for a launch on `stream`: marked as used on
    that stream, so the caching allocator does not hand its memory to other
    work before the launch's kernels have finished with it."""
    import torch
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None:
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=device)
        ws.record_stream(s)
    return ws


def _cache_geometry(kc, vc, fp8=False):
    """[NB, B, Hkv, D] views whose inner three dims are contiguous (bf16, or
    one-byte E4M3 codes as uint8 / float8_e4m3fn with fp8); returns
    (num_blocks, block_size, num_kv_heads, head_dim, block_stride)."""
    import torch
    if fp8:
        for t, name in ((kc, "key_cache"), (vc, "value_cache")):
            if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or not t.is_cuda:
                raise InvalidArgument(PA_ERR_INVALID, f"{name} must be a uint8 or float8_e4m3fn device tensor")
    else:
        _bf16(kc, "key_cache")
        _bf16(vc, "value_cache")
    if kc.dim() != 4 or kc.shape != vc.shape or kc.stride() != vc.stride():
        raise InvalidArgument(PA_ERR_INVALID, "caches must be matching [NB, B, Hkv, D] views")
    nb, bs, hkv, d = kc.shape
    if kc.stride()[1:] != (hkv * d, d, 1):
        raise InvalidArgument(PA_ERR_INVALID, "cache blocks must be contiguous [B, Hkv, D]")
    return nb, bs, hkv, d, kc.stride(0)


def pa_slot_mapping(block_tables, query_start_loc, seq_lens, block_size, num_tokens, out=None, stream=None):
    """Slots of a step's tokens computed on the device: block_tables int32
    [S, W] (unit column stride), query_start_loc int32 [S+1], seq_lens int32
    [S], all device tensors; returns (or fills) an int64 device tensor
    [num_tokens]."""
    import torch
    S = seq_lens.shape[0]
    for t, name in ((block_tables, "block_tables"), (query_start_loc, "query_start_loc"), (seq_lens, "seq_lens")):
        if t.dtype != torch.int32 or not t.is_cuda:
            raise InvalidArgument(PA_ERR_INVALID, f"{name} must be an int32 device tensor")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or block_tables.stride(1) != 1 \
            or query_start_loc.shape != (S + 1,) or not query_start_loc.is_contiguous() \
            or not seq_lens.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "need block_tables [S, W], query_start_loc [S+1], seq_lens [S]")
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=seq_lens.device)
    elif out.dtype != torch.int64 or out.shape != (num_tokens,) or not out.is_contiguous() or not out.is_cuda:
        raise InvalidArgument(PA_ERR_INVALID, "out must be a contiguous int64 device tensor [num_tokens]")
    _check(lib().pa_slot_mapping(out.data_ptr(), num_tokens, block_tables.data_ptr(), block_tables.stride(0),
                                 query_start_loc.data_ptr(), seq_lens.data_ptr(), S, block_size,
                                 _stream(seq_lens, stream)))
    return out


def pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, stream=None):
    """key/value [T, Hkv, D] bf16 (heads and dims contiguous); slot_mapping
    int64 [T] device tensor."""
    _reshape(key, value, key_cache, value_cache, slot_mapping, stream, False, 1.0, 1.0)


def pa_reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale=1.0, v_scale=1.0,
                             stream=None):
    """As pa_reshape_and_cache into E4M3 caches (uint8 or float8_e4m3fn
    [NB, B, Hkv, D]) with per-cache scales."""
    _reshape(key, value, key_cache, value_cache, slot_mapping, stream, True, k_scale, v_scale)


def _reshape(key, value, key_cache, value_cache, slot_mapping, stream, fp8, k_scale, v_scale):
    import torch
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache, fp8)
    _bf16(key, "key")
    _bf16(value, "value")
    T = key.shape[0]
    for t in (key, value):
        if t.dim() != 3 or tuple(t.shape[1:]) != (hkv, d) or t.stride()[1:] != (d, 1):
            raise InvalidArgument(PA_ERR_INVALID, "key/value must be [T, Hkv, D] with contiguous rows")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_cuda or slot_mapping.shape != (T,) \
            or not slot_mapping.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "slot_mapping must be a contiguous int64 device tensor [T]")
    args = (key.data_ptr(), key.stride(0), value.data_ptr(), value.stride(0), key_cache.data_ptr(),
            value_cache.data_ptr(), bstride, nb, slot_mapping.data_ptr(), T, hkv, d, bs)
    if fp8:
        _check(lib().pa_reshape_and_cache_fp8(*args, k_scale, v_scale, _stream(key_cache, stream)))
    else:
        _check(lib().pa_reshape_and_cache(*args, _stream(key_cache, stream)))


def pa_decode_append(key, value, key_cache, value_cache, block_tables, seq_lens, slots, positions, stream=None):
    """key/value [S, Hkv, D] bf16 device rows (one new token per row);
    block_tables int32 [S, W] and seq_lens int32 [S] device tensors, updated
    in place; slots: host int64 [S] (the pool's slots for the new tokens);
    positions: host int32 [S] (each row's length before the step)."""
    import torch
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    _bf16(key, "key")
    _bf16(value, "value")
    S = key.shape[0]
    for t in (key, value):
        if t.dim() != 3 or tuple(t.shape[1:]) != (hkv, d) or t.stride()[1:] != (d, 1):
            raise InvalidArgument(PA_ERR_INVALID, "key/value must be [S, Hkv, D] with contiguous rows")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] < S \
            or block_tables.stride(1) != 1 or not block_tables.is_cuda:
        raise InvalidArgument(PA_ERR_INVALID, "block_tables must be a device int32 [>= S, W] tensor")
    if seq_lens.dtype != torch.int32 or seq_lens.shape[0] < S or not seq_lens.is_contiguous() or not seq_lens.is_cuda:
        raise InvalidArgument(PA_ERR_INVALID, "seq_lens must be a contiguous device int32 [>= S] tensor")
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    if sl.shape != (S,) or pos.shape != (S,):
        raise InvalidArgument(PA_ERR_INVALID, "slots and positions must have one entry per row")
    _check(lib().pa_decode_append(key.data_ptr(), key.stride(0), value.data_ptr(), value.stride(0),
                                  key_cache.data_ptr(), value_cache.data_ptr(), bstride, nb, block_tables.data_ptr(),
                                  block_tables.stride(0), seq_lens.data_ptr(), _i64p(sl), _i32p(pos), S, hkv, d, bs,
                                  _stream(key_cache, stream)))


def pa_copy_blocks(caches, pairs, stream=None):
    """caches: list of device tensors whose dim 0 indexes blocks (each block's
    bytes contiguous); pairs: host [n, 2] (src, dst)."""
    if not caches:
        return
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    c0 = caches[0]
    nb = c0.shape[0]
    block_bytes = c0[0].numel() * c0.element_size()
    stride_bytes = c0.stride(0) * c0.element_size()
    for c in caches:
        if c.shape != c0.shape or c.stride() != c0.stride() or c.dtype != c0.dtype or not c.is_cuda:
            raise InvalidArgument(PA_ERR_INVALID, "caches must share shape, strides and dtype")
        if not c[0].is_contiguous():
            raise InvalidArgument(PA_ERR_INVALID, "each block of a cache must be contiguous")
    ptrs = (c_vp * len(caches))(*[c.data_ptr() for c in caches])
    _check(lib().pa_copy_blocks(ptrs, len(caches), block_bytes, stride_bytes, nb, _i32p(pairs), len(pairs),
                                _stream(c0, stream)))


def pa_copy_blocks_device(caches, pairs, stream=None):
    """caches: list of device tensors whose dim 0 indexes blocks; pairs: a
    device int32 tensor [n, 2] (src, dst), ids outside the pool skipped."""
    import torch
    if not caches:
        return
    c0 = caches[0]
    for c in caches:
        if c.shape != c0.shape or c.stride() != c0.stride() or c.dtype != c0.dtype or not c.is_cuda:
            raise InvalidArgument(PA_ERR_INVALID, "caches must share shape, strides and dtype")
        if not c[0].is_contiguous():
            raise InvalidArgument(PA_ERR_INVALID, "each block of a cache must be contiguous")
    if pairs.dtype != torch.int32 or not pairs.is_cuda or pairs.dim() != 2 or pairs.shape[1] != 2 \
            or not pairs.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "pairs must be a contiguous device int32 [n, 2] tensor")
    ptrs = (c_vp * len(caches))(*[c.data_ptr() for c in caches])
    _check(lib().pa_copy_blocks_device(ptrs, len(caches), c0[0].numel() * c0.element_size(),
                                       c0.stride(0) * c0.element_size(), c0.shape[0], pairs.data_ptr(),
                                       pairs.shape[0], _stream(c0, stream)))


def pa_paged_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size):
    return lib().pa_paged_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size)


def pa_paged_decode(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale,
                    partition_size=512, lse=None, workspace=None, stream=None):
    """out/q [S, Hq, D] bf16 contiguous; block_tables int32 [S, W] (row
    stride bt_stride = its stride(0)); seq_lens int32 [S]; lse fp32 [S, Hq]
    or None; workspace a uint8 device tensor (allocated here if None)."""
    _decode(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale, partition_size, lse,
            workspace, stream, False, 1.0, 1.0)


def pa_paged_decode_noalloc(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale,
                            partition_size=512, lse=None, stream=None):
    """pa_paged_decode with the split-K partials in the library's static
    device scratch (no workspace; nothing is allocated)."""
    _decode(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale, partition_size, lse,
            None, stream, False, 1.0, 1.0, noalloc=True)


def pa_paged_decode_fp8(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale,
                        k_scale=1.0, v_scale=1.0, partition_size=512, lse=None, workspace=None, stream=None):
    """pa_paged_decode over E4M3 caches (uint8 or float8_e4m3fn) with
    per-cache scales."""
    _decode(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale, partition_size, lse,
            workspace, stream, True, k_scale, v_scale)


def pa_paged_decode_append(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale,
                           key, value, slots, positions, partition_size=512, lse=None, workspace=None,
                           stream=None):
    """pa_decode_append + pa_paged_decode in one launch: key/value [S, Hkv, D]
    bf16 device rows of the new tokens; slots (host int64 [S]) and positions
    (host int32 [S]); block_tables and seq_lens are updated in place."""
    for t, name in ((key, "key"), (value, "value")):
        _bf16(t, name)
        if t.dim() != 3 or t.shape[0] != q.shape[0] or tuple(t.shape[1:]) != tuple(key_cache.shape[2:]) \
                or t.stride()[1:] != (t.shape[2], 1):
            raise InvalidArgument(PA_ERR_INVALID, f"{name} must be [S, Hkv, D] with contiguous rows")
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    if sl.shape != (q.shape[0],) or pos.shape != (q.shape[0],):
        raise InvalidArgument(PA_ERR_INVALID, "slots and positions must have one entry per sequence")
    _decode(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale, partition_size, lse,
            workspace, stream, False, 1.0, 1.0, append=(key, value, sl, pos))


def _decode(out, q, key_cache, value_cache, block_tables, seq_lens, max_seq_len, scale, partition_size, lse,
            workspace, stream, fp8, k_scale, v_scale, append=None, noalloc=False):
    import torch
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache, fp8)
    _bf16(q, "q")
    _bf16(out, "out")
    S, hq = q.shape[0], q.shape[1]
    if q.shape != (S, hq, d) or out.shape != q.shape or not q.is_contiguous() or not out.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "q and out must be contiguous [S, Hq, D]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.stride(1) != 1 \
            or block_tables.shape[0] != S:
        raise InvalidArgument(PA_ERR_INVALID, "block_tables must be int32 [S, W] with unit column stride")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (S,) or not seq_lens.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "seq_lens must be contiguous int32 [S]")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (S, hq) or not lse.is_contiguous()):
        raise InvalidArgument(PA_ERR_INVALID, "lse must be contiguous fp32 [S, Hq]")
    args = (out.data_ptr(), lse.data_ptr() if lse is not None else None, q.data_ptr(), key_cache.data_ptr(),
            value_cache.data_ptr(), bstride, nb, block_tables.data_ptr(), block_tables.stride(0),
            seq_lens.data_ptr(), S, hq, hkv, d, bs, max_seq_len, partition_size, scale)
    if noalloc:
        _check(lib().pa_paged_decode_noalloc(*args, _stream(q, stream)))
        return
    need = pa_paged_decode_workspace_size(S, hq, d, max_seq_len, partition_size)
    if workspace is None and need > 0:
        workspace = _scratch(need, q.device, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if append is not None:
        k, v, sl, pos = append
        _check(lib().pa_paged_decode_append(*args, k.data_ptr(), k.stride(0), v.data_ptr(), v.stride(0), _i64p(sl),
                                            _i32p(pos), ws_ptr, ws_bytes, _stream(q, stream)))
    elif fp8:
        _check(lib().pa_paged_decode_fp8(*args, k_scale, v_scale, ws_ptr, ws_bytes, _stream(q, stream)))
    else:
        _check(lib().pa_paged_decode(*args, ws_ptr, ws_bytes, _stream(q, stream)))


def pa_paged_prefill(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens,
                     max_query_len, max_seq_len, scale, causal=True, stream=None):
    """out/q [Tq, Hq, D] bf16 contiguous; query_start_loc int32 [S+1];
    seq_lens int32 [S]; block_tables int32 [S, W]."""
    _prefill(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, max_query_len, max_seq_len,
             scale, causal, stream, None)


def pa_paged_prefill_fp8(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens,
                         max_query_len, max_seq_len, scale, k_scale=1.0, v_scale=1.0, causal=True, stream=None):
    """pa_paged_prefill over E4M3 caches (uint8 or float8_e4m3fn) with
    per-cache scales."""
    _prefill(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, max_query_len, max_seq_len,
             scale, causal, stream, (k_scale, v_scale))


def _prefill(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, max_query_len, max_seq_len,
             scale, causal, stream, fp8):
    import torch
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache, fp8 is not None)
    _bf16(q, "q")
    _bf16(out, "out")
    hq = q.shape[1]
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or not q.is_contiguous() \
            or not out.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "q and out must be contiguous [Tq, Hq, D]")
    S = seq_lens.shape[0]
    if query_start_loc.dtype != torch.int32 or query_start_loc.shape != (S + 1,) \
            or seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "query_start_loc int32 [S+1] and seq_lens int32 [S] required")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.stride(1) != 1 \
            or block_tables.shape[0] != S:
        raise InvalidArgument(PA_ERR_INVALID, "block_tables must be int32 [S, W] with unit column stride")
    args = (out.data_ptr(), q.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), bstride, nb,
            block_tables.data_ptr(), block_tables.stride(0), query_start_loc.data_ptr(), seq_lens.data_ptr(), S,
            max_query_len, max_seq_len, hq, hkv, d, bs, scale)
    if fp8 is None:
        _check(lib().pa_paged_prefill(*args, int(bool(causal)), _stream(q, stream)))
    else:
        _check(lib().pa_paged_prefill_fp8(*args, fp8[0], fp8[1], int(bool(causal)), _stream(q, stream)))


def pa_paged_attention_workspace_size(query_start_loc_host, num_q_heads, head_dim, max_seq_len, partition_size):
    qsl = np.ascontiguousarray(query_start_loc_host, dtype=np.int32)
    return lib().pa_paged_attention_workspace_size(_i32p(qsl), len(qsl) - 1, num_q_heads, head_dim, max_seq_len,
                                                   partition_size)


def pa_paged_attention(out, q, key_cache, value_cache, block_tables, query_start_loc, query_start_loc_host, seq_lens,
                       max_query_len, max_seq_len, scale, partition_size=512, causal=True, workspace=None,
                       stream=None):
    """A mixed batch (decode rows first, then prefill chunks) in one launch:
    out/q [Tq, Hq, D] bf16 contiguous; query_start_loc int32 [S+1] on the
    device and query_start_loc_host the same values on the host; seq_lens
    int32 [S]; block_tables int32 [S, W]; workspace a uint8 device tensor
    (allocated here if None)."""
    import torch
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    _bf16(q, "q")
    _bf16(out, "out")
    hq = q.shape[1]
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or not q.is_contiguous() \
            or not out.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "q and out must be contiguous [Tq, Hq, D]")
    S = seq_lens.shape[0]
    qsl_h = np.ascontiguousarray(query_start_loc_host, dtype=np.int32)
    if query_start_loc.dtype != torch.int32 or query_start_loc.shape != (S + 1,) or qsl_h.shape != (S + 1,) \
            or seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise InvalidArgument(PA_ERR_INVALID, "query_start_loc int32 [S+1] (device and host) and seq_lens int32 [S]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.stride(1) != 1 \
            or block_tables.shape[0] != S:
        raise InvalidArgument(PA_ERR_INVALID, "block_tables must be int32 [S, W] with unit column stride")
    need = lib().pa_paged_attention_workspace_size(_i32p(qsl_h), S, hq, d, max_seq_len, partition_size)
    if workspace is None and need > 0:
        workspace = _scratch(need, q.device, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_paged_attention(out.data_ptr(), q.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), bstride,
                                    nb, block_tables.data_ptr(), block_tables.stride(0), query_start_loc.data_ptr(),
                                    _i32p(qsl_h), seq_lens.data_ptr(), S, max_query_len, max_seq_len, hq, hkv, d, bs,
                                    partition_size, scale, int(bool(causal)), ws_ptr, ws_bytes, _stream(q, stream)))
