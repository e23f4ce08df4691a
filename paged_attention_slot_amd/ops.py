"""Torch-facing binding of the device entry points of ``libpkv``.

Marshalling only: tensors are checked for device, dtype, shape and layout,
then their data pointers, sizes and the current HIP stream go to the C ABI.
Every step of the path runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (PKV_BF16, PKV_F32, PKV_FP8_E4M3, PKV_INT8, PkvGeom, PkvHostPool, PkvKvScales,
                   check, lib)

_DTYPES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.float8_e4m3fn: PKV_FP8_E4M3,
           torch.int8: PKV_INT8}
_QUANT = (torch.float8_e4m3fn, torch.int8)


def geom_of(k_cache: torch.Tensor) -> PkvGeom:
    """Geometry of a pool tensor [num_blocks, block_size, num_kv_heads, head_dim]."""
    if k_cache.dim() != 4:
        raise ValueError("cache must be [num_blocks, block_size, num_kv_heads, head_dim]")
    if k_cache.dtype not in _DTYPES:
        raise TypeError(f"unsupported cache dtype {k_cache.dtype}")
    nb, B, H, D = k_cache.shape
    return PkvGeom(nb, B, H, D, _DTYPES[k_cache.dtype])


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def set_tuning(name: str, value: int) -> None:
    """Set a tuning knob of the attention entry points (pkv_set_tuning; 0 =
    the library's heuristic)."""
    check(lib().pkv_set_tuning(name.encode(), int(value)), "pkv_set_tuning")


def get_tuning(name: str) -> int:
    v = lib().pkv_get_tuning(name.encode())
    if v < 0:
        raise KeyError(name)
    return int(v)


def _scratch(nbytes: int, dev, stream, phases: int = 3) -> torch.Tensor:
    """A workspace for one call, when the caller passes none.  A call of one
    phase alone needs the caller's workspace (the other phase reads what this
    one leaves there).  On a side stream the buffer is recorded on it, so the
    caching allocator does not hand it out again before the call's kernels
    have finished with it."""
    if (phases & 3) != 3:
        raise ValueError("a single-phase call needs the caller's workspace "
                         "(the two phases communicate through it)")
    t = torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=dev)
    if stream is not None:
        t.record_stream(stream)
    return t


def _out_like(q: torch.Tensor, stream) -> torch.Tensor:
    out = torch.empty_like(q)
    if stream is not None:
        out.record_stream(stream)
    return out


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def write(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Scatter token rows k/v [T, H_kv, D] into the pools at ``slot_mapping``
    (int32 [T], negative = skip)."""
    g = geom_of(k_cache)
    dev = k_cache.device
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k, "k"), (v, "v")):
        _need(t, n, k_cache.dtype, dev)
    _need(slot_mapping, "slot_mapping", torch.int32, dev)
    T = slot_mapping.numel()
    if k.shape != (T, g.num_kv_heads, g.head_dim) or v.shape != k.shape:
        raise ValueError("k/v must be [T, num_kv_heads, head_dim]")
    if v_cache.shape != k_cache.shape:
        raise ValueError("pool shapes differ")
    check(lib().pkv_write(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache),
                          ctypes.byref(g), _stream(stream)), "pkv_write")


def copy_blocks(pairs, k_cache, v_cache, stream=None) -> None:
    """Whole-block copies for int32 [P, 2] (src, dst) pairs."""
    g = geom_of(k_cache)
    dev = k_cache.device
    _need(k_cache, "k_cache", None, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    _need(pairs, "pairs", torch.int32, dev)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [P, 2]")
    if v_cache.shape != k_cache.shape:
        raise ValueError("pool shapes differ")
    check(lib().pkv_copy_blocks(_ptr(pairs), pairs.shape[0], _ptr(k_cache), _ptr(v_cache),
                                ctypes.byref(g), _stream(stream)), "pkv_copy_blocks")


def partition_tokens(num_seqs: int, num_q_heads: int, max_seq_len: int, k_cache) -> int:
    """The library's automatic split-KV partition length for these sizes."""
    g = geom_of(k_cache)
    return int(lib().pkv_attention_partition_tokens(num_seqs, num_q_heads, max_seq_len,
                                                    ctypes.byref(g)))


def piece_tokens(num_seqs: int, num_q_heads: int, max_seq_len: int, k_cache,
                 partition_tokens: int = 0) -> int:
    """Positions one split-KV piece covers (pkv_attention_piece_tokens; 0 on
    the balanced split)."""
    g = geom_of(k_cache)
    return int(lib().pkv_attention_piece_tokens(num_seqs, num_q_heads, max_seq_len,
                                                int(partition_tokens), ctypes.byref(g)))


ROUTES = {0: "partitions", 1: "balanced", 2: "matrix", 3: "matrix-balanced"}


def decode_route(num_seqs: int, num_q_heads: int, max_seq_len: int, k_cache,
                 partition_tokens: int = 0) -> str:
    """Which kernels pkv_attention_decode runs for these sizes: "partitions",
    "balanced" or "matrix" (pkv_attention_decode_route)."""
    g = geom_of(k_cache)
    r = lib().pkv_attention_decode_route(num_seqs, num_q_heads, max_seq_len,
                                         int(partition_tokens), ctypes.byref(g))
    if r < 0:
        check(1, "pkv_attention_decode_route")
    return ROUTES[int(r)]


def append_folded(num_seqs: int, num_q_heads: int, max_seq_len: int, k_cache,
                  partition_tokens: int = 0, kv_shared: bool = False) -> bool:
    """Whether pkv_attention_decode_append stores the new rows from inside the
    attention kernel (True) or launches a row-copy kernel first (False)
    (pkv_attention_decode_append_folded)."""
    g = geom_of(k_cache)
    r = lib().pkv_attention_decode_append_folded(num_seqs, num_q_heads, max_seq_len,
                                                 int(partition_tokens), int(bool(kv_shared)),
                                                 ctypes.byref(g))
    if r < 0:
        check(1, "pkv_attention_decode_append_folded")
    return bool(r)


def workspace_bytes(num_seqs: int, num_q_heads: int, max_seq_len: int, k_cache,
                    partition_tokens: int = 0) -> int:
    g = geom_of(k_cache)
    n = lib().pkv_attention_workspace_bytes(num_seqs, num_q_heads, max_seq_len,
                                            partition_tokens, ctypes.byref(g))
    if n == ctypes.c_size_t(-1).value:
        check(1, "pkv_attention_workspace_bytes")
    return int(n)


def _scales(k_cache, k_scale, v_scale, k_scales, v_scales) -> PkvKvScales:
    if k_cache.dtype == torch.int8:
        dev = k_cache.device
        nb, B, H, _ = k_cache.shape
        for t, n in ((k_scales, "k_scales"), (v_scales, "v_scales")):
            if t is None:
                raise ValueError(f"INT8 pools need {n}")
            _need(t, n, torch.float32, dev)
            if t.numel() != nb * B * H:
                raise ValueError(f"{n} must hold [num_blocks * block_size, num_kv_heads] floats")
    return PkvKvScales(float(k_scale), float(v_scale), _ptr(k_scales).value or None,
                       _ptr(v_scales).value or None)


KV_SHARED = 4  # PKV_KV_SHARED: or-ed into phases when sequences share blocks


def _attention(q, k_cache, v_cache, block_tables, seq_lens, scale, out, max_seq_len,
               partition_tokens, workspace, stream, phases, scales, new=None, kv_shared=False):
    g = geom_of(k_cache)
    dev = k_cache.device
    quant = k_cache.dtype in _QUANT
    _need(k_cache, "k_cache", None, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    _need(q, "q", torch.bfloat16 if quant else k_cache.dtype, dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(seq_lens, "seq_lens", torch.int32, dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("pool shapes differ")
    N, Hq, D = q.shape
    if D != g.head_dim or block_tables.dim() != 2 or block_tables.shape[0] != N or \
            seq_lens.shape != (N,):
        raise ValueError("shape mismatch between q, block_tables, seq_lens and the pools")
    max_blocks = block_tables.shape[1]
    if max_seq_len is None:
        max_seq_len = max_blocks * g.block_size
    if out is None:
        out = _out_like(q, stream)
    else:
        _need(out, "out", q.dtype, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    need = workspace_bytes(N, Hq, max_seq_len, k_cache, partition_tokens)
    if need and workspace is None:
        workspace = _scratch(need, dev, stream, phases)
    if workspace is not None:
        _need(workspace, "workspace", None, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    common = (_ptr(block_tables), max_blocks, _ptr(seq_lens), float(scale), _ptr(out), N, Hq,
              int(max_seq_len), int(partition_tokens), _ptr(workspace), ws_bytes,
              ctypes.byref(g), _stream(stream))
    phases = int(phases) | (KV_SHARED if kv_shared else 0)
    if new is not None:
        k_new, v_new, slots = new
        check(lib().pkv_attention_decode_append(int(phases), _ptr(q), _ptr(k_new), _ptr(v_new),
                                                _ptr(slots), _ptr(k_cache), _ptr(v_cache),
                                                *common), "pkv_attention_decode_append")
    elif quant:
        check(lib().pkv_attention_decode_quant(int(phases), _ptr(q), _ptr(k_cache),
                                               _ptr(v_cache), ctypes.byref(scales), *common),
              "pkv_attention_decode_quant")
    else:
        check(lib().pkv_attention_decode_phase(int(phases), _ptr(q), _ptr(k_cache),
                                               _ptr(v_cache), *common), "pkv_attention_decode")
    return out


def attention_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, out=None,
                     max_seq_len=None, partition_tokens=0, workspace=None, stream=None,
                     phases=3, kv_shared=False):
    """Decode attention; returns ``out`` [N, H_q, D] (allocated if None).

    ``max_seq_len`` is the host-known bound of ``seq_lens`` (default: the
    capacity of the block tables).  A workspace is allocated here only when the
    caller passes none and the split needs one; callers that must not
    allocate pass their own (size from ``workspace_bytes``).  ``phases``: 1 =
    partition kernel only, 2 = merge only, 3 = both (see include/pkv.h)."""
    if k_cache.dtype in _QUANT:
        raise TypeError("quantized pools: use attention_decode_quant")
    return _attention(q, k_cache, v_cache, block_tables, seq_lens, scale, out, max_seq_len,
                      partition_tokens, workspace, stream, phases, None, kv_shared=kv_shared)


def attention_decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, scale, out,
                             max_seq_len=None, partition_tokens=0, stream=None):
    """pkv_attention_decode_noalloc: decode attention with the library's own
    device scratch as the workspace (nothing is allocated; ``out`` is the
    caller's).  Calls that may overlap on one GPU race on that scratch."""
    if k_cache.dtype in _QUANT:
        raise TypeError("attention_decode_noalloc takes bf16 or f32 pools")
    g = geom_of(k_cache)
    dev = k_cache.device
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (q, "q"), (out, "out")):
        _need(t, n, k_cache.dtype, dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(seq_lens, "seq_lens", torch.int32, dev)
    N, Hq, D = q.shape
    if v_cache.shape != k_cache.shape or out.shape != q.shape or D != g.head_dim or \
            block_tables.dim() != 2 or block_tables.shape[0] != N or seq_lens.shape != (N,):
        raise ValueError("shape mismatch between q, out, block_tables, seq_lens and the pools")
    max_blocks = block_tables.shape[1]
    if max_seq_len is None:
        max_seq_len = max_blocks * g.block_size
    check(lib().pkv_attention_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(block_tables), max_blocks, _ptr(seq_lens),
                                             float(scale), _ptr(out), N, Hq, int(max_seq_len),
                                             int(partition_tokens), ctypes.byref(g),
                                             _stream(stream)), "pkv_attention_decode_noalloc")
    return out


def attention_decode_append(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                            seq_lens, scale, out=None, max_seq_len=None, partition_tokens=0,
                            workspace=None, stream=None, phases=3, kv_shared=False):
    """The step's KV append and decode attention in one computation
    (pkv_attention_decode_append): k_new/v_new [N, H_kv, D] in the pool dtype,
    slot_mapping int32 [N] the slot of each sequence's newest position; the
    pools are written at those slots.  Returns ``out``."""
    if k_cache.dtype in _QUANT:
        raise TypeError("attention_decode_append takes bf16 or f32 pools")
    dev = k_cache.device
    _need(k_new, "k_new", k_cache.dtype, dev)
    _need(v_new, "v_new", k_cache.dtype, dev)
    _need(slot_mapping, "slot_mapping", torch.int32, dev)
    N = seq_lens.shape[0]
    g = geom_of(k_cache)
    if k_new.shape != (N, g.num_kv_heads, g.head_dim) or v_new.shape != k_new.shape or \
            slot_mapping.shape != (N,):
        raise ValueError("k_new/v_new must be [N, H_kv, D] and slot_mapping [N]")
    return _attention(q, k_cache, v_cache, block_tables, seq_lens, scale, out, max_seq_len,
                      partition_tokens, workspace, stream, phases, None,
                      new=(k_new, v_new, slot_mapping), kv_shared=kv_shared)


def attention_decode_quant(q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale=1.0,
                           v_scale=1.0, k_scales=None, v_scales=None, out=None,
                           max_seq_len=None, partition_tokens=0, workspace=None, stream=None,
                           phases=3, kv_shared=False):
    """Decode attention over an FP8 e4m3 (``torch.float8_e4m3fn`` pools,
    per-tensor ``k_scale``/``v_scale``) or INT8 (``torch.int8`` pools, fp32
    ``k_scales``/``v_scales`` [num_blocks * block_size, num_kv_heads]) cache;
    q and out are bf16."""
    if k_cache.dtype not in _QUANT:
        raise TypeError("attention_decode_quant needs float8_e4m3fn or int8 pools")
    sc = _scales(k_cache, k_scale, v_scale, k_scales, v_scales)
    return _attention(q, k_cache, v_cache, block_tables, seq_lens, scale, out, max_seq_len,
                      partition_tokens, workspace, stream, phases, sc, kv_shared=kv_shared)


def attention_multi(q, q_offsets, k_cache, v_cache, block_tables, seq_lens, scale,
                    max_q_per_seq, out=None, max_seq_len=None, partition_tokens=0,
                    workspace=None, stream=None, k_scale=1.0, v_scale=1.0, k_scales=None,
                    v_scales=None):
    """Attention of several new query tokens per sequence (see include/pkv.h,
    pkv_attention_multi; with FP8/INT8 pools pkv_attention_multi_quant and the
    scales).  q [total_q, H_q, D] bf16; q_offsets int32 [N+1] on the device;
    ``max_q_per_seq`` bounds the queries of any sequence."""
    g = geom_of(k_cache)
    dev = k_cache.device
    quant = k_cache.dtype in _QUANT
    _need(k_cache, "k_cache", None if quant else torch.bfloat16, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    _need(q, "q", torch.bfloat16, dev)
    _need(q_offsets, "q_offsets", torch.int32, dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(seq_lens, "seq_lens", torch.int32, dev)
    total, Hq, D = q.shape
    N = seq_lens.shape[0]
    if D != g.head_dim or q_offsets.shape != (N + 1,) or block_tables.shape[0] != N:
        raise ValueError("shape mismatch between q, q_offsets, block_tables and seq_lens")
    max_blocks = block_tables.shape[1]
    if max_seq_len is None:
        max_seq_len = max_blocks * g.block_size
    if out is None:
        out = _out_like(q, stream)
    else:
        _need(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    need = lib().pkv_attention_multi_workspace_bytes(N, Hq, total, int(max_q_per_seq),
                                                     int(max_seq_len), int(partition_tokens),
                                                     ctypes.byref(g))
    if need == ctypes.c_size_t(-1).value:
        check(1, "pkv_attention_multi_workspace_bytes")
    if need and workspace is None:
        workspace = _scratch(need, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if quant:
        sc = _scales(k_cache, k_scale, v_scale, k_scales, v_scales)
        check(lib().pkv_attention_multi_quant(
            _ptr(q), _ptr(q_offsets), _ptr(k_cache), _ptr(v_cache), ctypes.byref(sc),
            _ptr(block_tables), max_blocks, _ptr(seq_lens), float(scale), _ptr(out), N, Hq, total,
            int(max_q_per_seq), int(max_seq_len), int(partition_tokens), _ptr(workspace),
            ws_bytes, ctypes.byref(g), _stream(stream)), "pkv_attention_multi_quant")
        return out
    check(lib().pkv_attention_multi(_ptr(q), _ptr(q_offsets), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(block_tables), max_blocks, _ptr(seq_lens), float(scale),
                                    _ptr(out), N, Hq, total, int(max_q_per_seq),
                                    int(max_seq_len), int(partition_tokens), _ptr(workspace),
                                    ws_bytes, ctypes.byref(g), _stream(stream)),
          "pkv_attention_multi")
    return out


def write_quant(k, v, slot_mapping, k_cache, v_cache, k_scale=1.0, v_scale=1.0, k_scales=None,
                v_scales=None, stream=None) -> None:
    """Quantize bf16 token rows k/v [T, H_kv, D] into FP8 / INT8 pools at
    ``slot_mapping`` (INT8 also writes each row's scale)."""
    g = geom_of(k_cache)
    dev = k_cache.device
    if k_cache.dtype not in _QUANT:
        raise TypeError("write_quant needs float8_e4m3fn or int8 pools")
    _need(k_cache, "k_cache", None, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, dev)
    _need(slot_mapping, "slot_mapping", torch.int32, dev)
    T = slot_mapping.numel()
    if k.shape != (T, g.num_kv_heads, g.head_dim) or v.shape != k.shape:
        raise ValueError("k/v must be [T, num_kv_heads, head_dim]")
    if v_cache.shape != k_cache.shape:
        raise ValueError("pool shapes differ")
    sc = _scales(k_cache, k_scale, v_scale, k_scales, v_scales)
    check(lib().pkv_write_quant(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache),
                                _ptr(v_cache), ctypes.byref(sc), ctypes.byref(g),
                                _stream(stream)), "pkv_write_quant")


def copy_blocks_quant(pairs, k_cache, v_cache, k_scales=None, v_scales=None,
                      stream=None) -> None:
    """Whole-block copies of codes (and INT8 scale rows) for int32 [P, 2] pairs."""
    g = geom_of(k_cache)
    dev = k_cache.device
    _need(k_cache, "k_cache", None, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    _need(pairs, "pairs", torch.int32, dev)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [P, 2]")
    sc = _scales(k_cache, 1.0, 1.0, k_scales, v_scales)
    check(lib().pkv_copy_blocks_quant(_ptr(pairs), pairs.shape[0], _ptr(k_cache), _ptr(v_cache),
                                      ctypes.byref(sc), ctypes.byref(g), _stream(stream)),
          "pkv_copy_blocks_quant")


def prefix_groups(block_tables, seq_lens, block_size: int):
    """Shared-prefix groups of a batch from host tables (see include/pkv.h,
    pkv_prefix_groups).  Returns (group_starts int32 [G+1], prefix_lens int32
    [G], max_group_size, max_prefix_len, max_suffix_len)."""
    import numpy as np
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    n = int(L.size)
    mb = int(t.shape[1]) if t.ndim == 2 else 0
    starts = np.empty(n + 1, np.int32)
    plens = np.empty(max(n, 1), np.int32)
    ng, mg, mp, ms = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    P = ctypes.POINTER(ctypes.c_int32)
    check(lib().pkv_prefix_groups(t.ctypes.data_as(P), n, mb, L.ctypes.data_as(P),
                                  int(block_size), starts.ctypes.data_as(P),
                                  plens.ctypes.data_as(P), ctypes.byref(ng), ctypes.byref(mg),
                                  ctypes.byref(mp), ctypes.byref(ms)), "pkv_prefix_groups")
    return (starts[:ng.value + 1].copy(), plens[:ng.value].copy(), mg.value, mp.value,
            ms.value)


def shared_workspace_bytes(num_seqs, num_q_heads, num_groups, max_group_size, max_prefix_len,
                           max_suffix_len, max_seq_len, k_cache) -> int:
    g = geom_of(k_cache)
    n = lib().pkv_attention_shared_workspace_bytes(int(num_seqs), int(num_q_heads),
                                                   int(num_groups), int(max_group_size),
                                                   int(max_prefix_len), int(max_suffix_len),
                                                   int(max_seq_len), ctypes.byref(g))
    if n == ctypes.c_size_t(-1).value:
        check(1, "pkv_attention_shared_workspace_bytes")
    return int(n)


def attention_decode_shared(q, k_cache, v_cache, block_tables, seq_lens, scale, group_starts,
                            prefix_lens, max_group_size, max_prefix_len, max_suffix_len=0,
                            out=None, max_seq_len=None, workspace=None, stream=None,
                            k_scale=1.0, v_scale=1.0, k_scales=None, v_scales=None):
    """Decode attention reading each group's shared prefix once (see
    include/pkv.h, pkv_attention_decode_shared).  group_starts / prefix_lens are
    int32 device tensors as pkv_prefix_groups returns them."""
    g = geom_of(k_cache)
    dev = k_cache.device
    quant = k_cache.dtype in _QUANT
    kdt = k_cache.dtype if quant else torch.bfloat16
    for t, n, dt in ((k_cache, "k_cache", kdt), (v_cache, "v_cache", kdt),
                     (q, "q", torch.bfloat16), (block_tables, "block_tables", torch.int32),
                     (seq_lens, "seq_lens", torch.int32), (group_starts, "group_starts", torch.int32),
                     (prefix_lens, "prefix_lens", torch.int32)):
        _need(t, n, dt, dev)
    N, Hq, D = q.shape
    if D != g.head_dim or block_tables.shape[0] != N or seq_lens.shape != (N,):
        raise ValueError("shape mismatch between q, block_tables and seq_lens")
    ng = int(prefix_lens.shape[0])
    if group_starts.shape != (ng + 1,):
        raise ValueError("group_starts must hold num_groups + 1 entries")
    max_blocks = block_tables.shape[1]
    if max_seq_len is None:
        max_seq_len = max_blocks * g.block_size
    if out is None:
        out = _out_like(q, stream)
    need = shared_workspace_bytes(N, Hq, ng, max_group_size, max_prefix_len, max_suffix_len,
                                  max_seq_len, k_cache)
    if workspace is None:
        workspace = _scratch(need, dev, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    if quant:
        sc = _scales(k_cache, k_scale, v_scale, k_scales, v_scales)
        check(lib().pkv_attention_decode_shared_quant(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(sc), _ptr(block_tables),
            max_blocks, _ptr(seq_lens), _ptr(group_starts), _ptr(prefix_lens), ng,
            int(max_group_size), int(max_prefix_len), int(max_suffix_len), float(scale), _ptr(out),
            N, Hq, int(max_seq_len), _ptr(workspace), ws_bytes, ctypes.byref(g), _stream(stream)),
            "pkv_attention_decode_shared_quant")
        return out
    check(lib().pkv_attention_decode_shared(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), max_blocks, _ptr(seq_lens),
        _ptr(group_starts), _ptr(prefix_lens), ng, int(max_group_size), int(max_prefix_len),
        int(max_suffix_len), float(scale), _ptr(out), N, Hq, int(max_seq_len), _ptr(workspace),
        ws_bytes,
        ctypes.byref(g), _stream(stream)), "pkv_attention_decode_shared")
    return out


class HostPool:
    """Pinned host blocks laid out like a device pool pair (K, V and, for INT8
    pools, the fp32 scale pools), ``num_blocks`` blocks.  Allocated with
    torch's pinned allocator (HIP host allocation), so kernels reach it."""

    def __init__(self, num_blocks: int, like: torch.Tensor):
        _, B, H, D = like.shape
        self.num_blocks = int(num_blocks)
        self.k = torch.zeros((num_blocks, B, H, D), dtype=like.dtype, pin_memory=True)
        self.v = torch.zeros(self.k.shape, dtype=like.dtype, pin_memory=True)
        if like.dtype == torch.int8:
            self.k_scales = torch.zeros((num_blocks * B, H), dtype=torch.float32, pin_memory=True)
            self.v_scales = torch.zeros(self.k_scales.shape, dtype=torch.float32,
                                        pin_memory=True)
        else:
            self.k_scales = self.v_scales = None

    def struct(self) -> PkvHostPool:
        return PkvHostPool(self.num_blocks, _ptr(self.k), _ptr(self.v),
                           _ptr(self.k_scales).value or None, _ptr(self.v_scales).value or None)


def _swap_args(pairs, k_cache, v_cache, host, k_scales, v_scales):
    g = geom_of(k_cache)
    dev = k_cache.device
    _need(k_cache, "k_cache", None, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    if pairs.dtype != torch.int32 or not pairs.is_contiguous() or (
            pairs.dim() != 2 or pairs.shape[1] != 2):
        raise ValueError("pairs must be a contiguous int32 [P, 2] tensor")
    if not pairs.is_cuda and not pairs.is_pinned():
        raise ValueError("pairs must be a device tensor or pinned host memory")
    if host.k.dtype != k_cache.dtype or host.k.shape[1:] != k_cache.shape[1:]:
        raise ValueError("host pool blocks differ from the device pool's")
    sc = _scales(k_cache, 1.0, 1.0, k_scales, v_scales)
    return g, sc, host.struct()


def swap_out(pairs, k_cache, v_cache, host: HostPool, k_scales=None, v_scales=None,
             stream=None) -> None:
    """Copy device blocks to host blocks for (device, host) pairs."""
    g, sc, hp = _swap_args(pairs, k_cache, v_cache, host, k_scales, v_scales)
    check(lib().pkv_swap_out(_ptr(pairs), pairs.shape[0], _ptr(k_cache), _ptr(v_cache),
                             ctypes.byref(sc), ctypes.byref(hp), ctypes.byref(g), _stream(stream)),
          "pkv_swap_out")


def swap_in(pairs, host: HostPool, k_cache, v_cache, k_scales=None, v_scales=None,
            stream=None) -> None:
    """Copy host blocks back into device blocks for (host, device) pairs."""
    g, sc, hp = _swap_args(pairs, k_cache, v_cache, host, k_scales, v_scales)
    check(lib().pkv_swap_in(_ptr(pairs), pairs.shape[0], ctypes.byref(hp), _ptr(k_cache),
                            _ptr(v_cache), ctypes.byref(sc), ctypes.byref(g), _stream(stream)),
          "pkv_swap_in")


def stream_read(buf: torch.Tensor, sink: torch.Tensor, num_workgroups: int = 4096,
                stream=None) -> None:
    """Read-bandwidth calibration kernel over ``buf`` (see include/pkv.h)."""
    _need(buf, "buf", None, buf.device)
    _need(sink, "sink", torch.int32, buf.device)
    if sink.numel() < num_workgroups:
        raise ValueError("sink needs num_workgroups entries")
    nbytes = buf.numel() * buf.element_size()
    check(lib().pkv_stream_read(_ptr(buf), nbytes - nbytes % 16, _ptr(sink), int(num_workgroups),
                                _stream(stream)), "pkv_stream_read")
