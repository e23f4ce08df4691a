"""One decode step of a workload on the GPU, driven through ``libpkv``.

The library's host block manager replays the workload's operation trace
(sequence creation, context appends, prefix sharing, forks), the context K/V
are placed with one bulk ``pkv_write``, then the decode step is, in stream
order ([KVX §01]: the new token is appended before its query reads the
history; page keys in include/pkv.h):

    pkv_copy_blocks (copy-on-write pairs, if any)
    pkv_write       (one new token per sequence)
    pkv_attention_decode (+ split-KV merge)

or, with ``step(fused=True)``, the write folded into the attention
(pkv_attention_decode_append: the wave that attends a sequence's newest
position takes it from the new-token rows and stores it to its slot).

``layers`` > 1 keeps that many independent pool pairs with identical block
tables (one per transformer layer); ``step(layer)`` runs the step on one of
them, so consecutive steps read different memory as a model's layers do.

A trace that pauses sequences ("swap_out") and resumes them ("swap_in")
moves their blocks to a pinned host pool and back with pkv_swap_out /
pkv_swap_in ([KVM §19.2.6]); context writes, copy-on-write copies and swaps
then run in trace order.

``kv_dtype`` "fp8_e4m3" or "int8" keeps the pools as one-byte codes of the
workload's bf16 values ([KVM §19.2.4]; [PFX] "KV Cache 量化"): writes quantize
(pkv_write_quant), copies carry INT8 scales (pkv_copy_blocks_quant) and the
attention dequantizes (pkv_attention_decode_quant).
"""
from __future__ import annotations

import time

import numpy as np
import torch

from . import ops
from .block_manager import BlockManager


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host values (float32, or bf16 bit patterns as uint16) -> device tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array of its stored values (uint16 bits for bf16,
    uint8 codes for FP8 e4m3)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def shares_blocks(tables: np.ndarray, lens: np.ndarray, block_size: int) -> bool:
    """Whether two sequences of the batch read the same physical block (prefix
    sharing, forks): the attention then keeps K/V loads cacheable
    (PKV_KV_SHARED)."""
    used = [tables[s, :-(-int(L) // block_size)] for s, L in enumerate(lens) if L > 0]
    if not used:
        return False
    ids = np.concatenate(used)
    return np.unique(ids).size < ids.size


_CACHE_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16,
                 "fp8_e4m3": torch.float8_e4m3fn, "int8": torch.int8}


class DecodeStep:
    def __init__(self, wl, device=None, layers: int = 1, partition_tokens: int | None = None,
                 keep_context: bool = False, kv_dtype: str | None = None, k_scale: float = 1.0,
                 v_scale: float = 1.0):
        self.wl = wl
        self.device = torch.device(device or "cuda")
        self.torch_dtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        self.layers = int(layers)
        self.kv_dtype = kv_dtype or wl.dtype
        self.quant = self.kv_dtype in ("fp8_e4m3", "int8")
        if self.quant and wl.dtype != "bf16":
            raise ValueError("quantized caches take bf16 workloads")
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)

        # -- host: block manager replays the trace --------------------------
        bm = BlockManager(wl.num_blocks, wl.block_size, wl.free_order, wl.num_host_blocks,
                          wl.host_free_order)
        ctx_slots = np.empty(wl.ctx_tokens, dtype=np.int32)
        cur = 0
        # device work of the trace, in order: ("write", first, end) over
        # context rows, ("copy", pairs), ("swap_out", pairs), ("swap_in", pairs)
        events = []
        for op in wl.ops:
            kind = op[0]
            if kind == "add":
                bm.add_seq(op[1])
            elif kind == "append":
                slots, cow = bm.append_slots([op[1]], op[2])
                if len(cow):
                    events.append(("copy", cow))
                ctx_slots[cur:cur + op[2]] = slots
                if events and events[-1][0] == "write" and events[-1][2] == cur:
                    events[-1] = ("write", events[-1][1], cur + op[2])
                else:
                    events.append(("write", cur, cur + op[2]))
                cur += op[2]
            elif kind == "share_prefix":
                bm.share_prefix(op[1], op[2], op[3])
            elif kind == "fork":
                bm.fork(op[1], op[2])
            elif kind == "swap_out":
                events.append(("swap_out", bm.swap_out(list(op[1]))))
            elif kind == "swap_in":
                events.append(("swap_in", bm.swap_in(list(op[1]))))
            elif kind == "free":
                bm.free_seq(op[1])
                # the freed slots may be written again by later appends:
                # those writes must not join the same launch as earlier ones
                # (one pkv_write takes distinct slots)
                events.append(("free", None))
            else:
                raise ValueError(f"unknown op {kind}")
        assert cur == wl.ctx_tokens
        self.ctx_slots = ctx_slots
        self.swap_events = [(k, p) for k, p in ((e[0], e[1]) for e in events)
                            if k in ("swap_out", "swap_in")]

        # decode step, host part: one slot per sequence, CoW pairs, tables
        t0 = time.perf_counter()
        slots, cow = bm.append_slots(wl.decode_seqs, 1)
        tables, lens = bm.export(wl.decode_seqs, wl.max_blocks_per_seq)
        self.host_tables_s = time.perf_counter() - t0
        self.bm = bm
        self.slot_mapping_h, self.cow_pairs_h = slots, cow
        self.block_tables_h, self.seq_lens_h = tables, lens
        self.kv_shared = shares_blocks(tables, lens, wl.block_size)
        if not np.array_equal(lens, wl.seq_lens):
            raise RuntimeError("block manager lengths differ from the workload's")

        # -- device ------------------------------------------------------------
        dev = self.device
        shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
        cdt = _CACHE_DTYPES[self.kv_dtype]
        if wl.pool_init is not None and not self.quant:
            # the bits never-written slots hold (stale data of earlier owners)
            self.k_caches = [to_device(wl.pool_init[0], wl.dtype, dev)]
            self.v_caches = [to_device(wl.pool_init[1], wl.dtype, dev)]
        else:
            self.k_caches = [torch.zeros(shape, dtype=cdt, device=dev)]
            self.v_caches = [torch.zeros(shape, dtype=cdt, device=dev)]
        sshape = (wl.num_blocks * wl.block_size, wl.num_kv_heads)
        if self.kv_dtype == "int8":
            self.k_scale_pools = [torch.zeros(sshape, dtype=torch.float32, device=dev)]
            self.v_scale_pools = [torch.zeros(sshape, dtype=torch.float32, device=dev)]
        else:
            self.k_scale_pools = self.v_scale_pools = None
        self.host = ops.HostPool(wl.num_host_blocks, self.k_caches[0]) \
            if wl.num_host_blocks else None
        if wl.ctx_tokens:
            ck = to_device(wl.ctx_k, wl.dtype, dev)
            cv = to_device(wl.ctx_v, wl.dtype, dev)
            cs = torch.from_numpy(ctx_slots).to(dev)
            for ev in events:
                if ev[0] == "write":
                    self._write(ck[ev[1]:ev[2]], cv[ev[1]:ev[2]], cs[ev[1]:ev[2]], 0)
                elif ev[0] == "free":
                    continue
                else:
                    self._trace_event(ev[0], ev[1])
            if keep_context:
                self.ctx_k_dev, self.ctx_v_dev, self.ctx_slots_dev = ck, cv, cs
            else:
                del ck, cv, cs
        for _ in range(1, self.layers):
            self.k_caches.append(self.k_caches[0].clone())
            self.v_caches.append(self.v_caches[0].clone())
            if self.k_scale_pools is not None:
                self.k_scale_pools.append(self.k_scale_pools[0].clone())
                self.v_scale_pools.append(self.v_scale_pools[0].clone())
        self.q = to_device(wl.q, wl.dtype, dev)
        self.new_k = to_device(wl.new_k, wl.dtype, dev)
        self.new_v = to_device(wl.new_v, wl.dtype, dev)
        self.slot_mapping = torch.from_numpy(slots).to(dev)
        self.cow_pairs = torch.from_numpy(np.ascontiguousarray(cow).reshape(-1, 2)).to(dev)
        self.block_tables = torch.from_numpy(tables).to(dev)
        self.seq_lens = torch.from_numpy(lens).to(dev)
        self.max_seq_len = int(lens.max()) if lens.size else 0
        pt = wl.partition_tokens if partition_tokens is None else partition_tokens
        self.partition_tokens = int(pt or 0)
        self.out = torch.empty_like(self.q)
        n = ops.workspace_bytes(wl.num_seqs, wl.num_q_heads, self.max_seq_len, self.k_caches[0],
                                self.partition_tokens)
        self.workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=dev) if n else None
        torch.cuda.synchronize(dev)

    def _trace_event(self, kind, pairs, layer=0):
        pd = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2))
        pd = pd.to(self.device)
        if kind == "copy":
            self.copy(layer, pairs=pd)
            return
        ks, vs = self._scales(layer)
        kc, vc = self.k_caches[layer], self.v_caches[layer]
        if kind == "swap_out":
            ops.swap_out(pd, kc, vc, self.host, ks, vs)
        else:
            ops.swap_in(pd, self.host, kc, vc, ks, vs)

    @property
    def k_cache(self):
        return self.k_caches[0]

    @property
    def v_cache(self):
        return self.v_caches[0]

    def _scales(self, layer):
        if self.k_scale_pools is None:
            return None, None
        return self.k_scale_pools[layer], self.v_scale_pools[layer]

    def _write(self, k, v, slots, layer, stream=None):
        if self.quant:
            ks, vs = self._scales(layer)
            ops.write_quant(k, v, slots, self.k_caches[layer], self.v_caches[layer],
                            self.k_scale, self.v_scale, ks, vs, stream=stream)
        else:
            ops.write(k, v, slots, self.k_caches[layer], self.v_caches[layer], stream=stream)

    def copy(self, layer=0, stream=None, pairs=None):
        pairs = self.cow_pairs if pairs is None else pairs
        if pairs.shape[0]:
            if self.quant:
                ks, vs = self._scales(layer)
                ops.copy_blocks_quant(pairs, self.k_caches[layer], self.v_caches[layer],
                                      ks, vs, stream=stream)
            else:
                ops.copy_blocks(pairs, self.k_caches[layer], self.v_caches[layer],
                                stream=stream)

    def write(self, layer=0, stream=None):
        self._write(self.new_k, self.new_v, self.slot_mapping, layer, stream)

    def attention(self, layer=0, stream=None, out=None, partition_tokens=None, phases=3):
        pt = self.partition_tokens if partition_tokens is None else partition_tokens
        ws = self.workspace
        if pt != self.partition_tokens:
            ws = None  # let the binding size a workspace for this split
        kw = dict(out=self.out if out is None else out, max_seq_len=self.max_seq_len,
                  partition_tokens=pt, workspace=ws, stream=stream, phases=phases,
                  kv_shared=self.kv_shared)
        if self.quant:
            ks, vs = self._scales(layer)
            return ops.attention_decode_quant(self.q, self.k_caches[layer], self.v_caches[layer],
                                              self.block_tables, self.seq_lens, self.wl.scale,
                                              self.k_scale, self.v_scale, ks, vs, **kw)
        return ops.attention_decode(self.q, self.k_caches[layer], self.v_caches[layer],
                                    self.block_tables, self.seq_lens, self.wl.scale, **kw)

    def attention_append(self, layer=0, stream=None, out=None, phases=3):
        """The new token's append and the attention in one computation
        (pkv_attention_decode_append; bf16/f32 pools)."""
        if self.quant:
            raise ValueError("the fused append takes bf16 or f32 pools")
        return ops.attention_decode_append(
            self.q, self.new_k, self.new_v, self.slot_mapping, self.k_caches[layer],
            self.v_caches[layer], self.block_tables, self.seq_lens, self.wl.scale,
            out=self.out if out is None else out, max_seq_len=self.max_seq_len,
            partition_tokens=self.partition_tokens, workspace=self.workspace, stream=stream,
            phases=phases, kv_shared=self.kv_shared)

    def shared_groups(self):
        """Shared-prefix groups of the step's tables (pkv_prefix_groups), as
        device tensors plus their host bounds; computed once."""
        if getattr(self, "_groups", None) is None:
            starts, plens, mg, mp, ms = ops.prefix_groups(self.block_tables_h, self.seq_lens_h,
                                                          self.wl.block_size)
            self._groups = (torch.from_numpy(starts).to(self.device),
                            torch.from_numpy(plens).to(self.device), mg, mp, ms)
            n = ops.shared_workspace_bytes(self.wl.num_seqs, self.wl.num_q_heads, plens.size, mg,
                                           mp, ms, self.max_seq_len, self.k_caches[0])
            self._shared_ws = torch.empty(max(n, 16), dtype=torch.uint8, device=self.device)
        return self._groups

    def attention_shared(self, layer=0, stream=None, out=None):
        """Decode attention reading each shared prefix once
        (pkv_attention_decode_shared, or its _quant form for FP8/INT8 pools)."""
        gs, pl, mg, mp, ms = self.shared_groups()
        ks, vs = self._scales(layer)
        return ops.attention_decode_shared(
            self.q, self.k_caches[layer], self.v_caches[layer], self.block_tables, self.seq_lens,
            self.wl.scale, gs, pl, mg, mp, ms, out=self.out if out is None else out,
            max_seq_len=self.max_seq_len, workspace=self._shared_ws, stream=stream,
            k_scale=self.k_scale, v_scale=self.v_scale, k_scales=ks, v_scales=vs)

    @property
    def split(self) -> dict:
        """How pkv_attention_decode runs this batch: the kernels ("route":
        vector kernels with fixed partitions or the balanced split, or the
        matrix-core pass) and the partition length and count; on the
        matrix-core route also the workgroups per (sequence, KV head), each of
        which folds its positions into one piece."""
        route = ops.decode_route(self.wl.num_seqs, self.wl.num_q_heads, self.max_seq_len,
                                 self.k_caches[0], self.partition_tokens)
        if route in ("balanced", "matrix-balanced"):
            return {"mode": route}
        pt = self.partition_tokens or ops.partition_tokens(
            self.wl.num_seqs, self.wl.num_q_heads, self.max_seq_len, self.k_caches[0])
        split = {"mode": "matrix" if route == "matrix" else "partitions", "partition_tokens": pt,
                 "num_partitions": max(1, -(-self.max_seq_len // pt)),
                 "piece_tokens": ops.piece_tokens(self.wl.num_seqs, self.wl.num_q_heads,
                                                  self.max_seq_len, self.k_caches[0],
                                                  self.partition_tokens)}
        if route == "matrix":
            # one workspace row of D + 2 floats per (sequence, query head, run)
            ws = ops.workspace_bytes(self.wl.num_seqs, self.wl.num_q_heads, self.max_seq_len,
                                     self.k_caches[0], self.partition_tokens)
            row = self.wl.num_seqs * self.wl.num_q_heads * (self.wl.head_dim + 2) * 4
            split["workgroups_per_history"] = ws // row if ws else 1
        return split

    @property
    def append_folded(self) -> bool:
        """Whether attention_append() stores the new rows from inside the
        attention kernel (else a row-copy kernel runs first)."""
        return ops.append_folded(self.wl.num_seqs, self.wl.num_q_heads, self.max_seq_len,
                                 self.k_caches[0], self.partition_tokens or 0, self.kv_shared)

    def step(self, layer=0, stream=None, fused=False):
        """copy -> write -> attention on one layer's pools (enqueue only);
        ``fused``: copy -> append + attention (pkv_attention_decode_append)."""
        self.copy(layer, stream)
        if fused:
            return self.attention_append(layer, stream)
        self.write(layer, stream)
        return self.attention(layer, stream)
