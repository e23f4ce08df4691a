"""Drive a ``workloads.Workload`` through the oracle.  Test infrastructure.

Order of one decode step ([KVX §01]: the new token's K/V are appended before
its query reads the history): copy-on-write block copies, then the slot-scatter
write of the new tokens, then attention over every sequence's whole history.

The context trace may also pause sequences by swapping them out to the host
pool and bring them back ([KVM §19.2.6]); context appends into a block shared
after a fork copy the block first, as the decode step does.
"""
from __future__ import annotations

import numpy as np

from .block_manager import BlockManager
from .cache_ops import copy_blocks, swap_blocks, write


class OracleState:
    """Pools, manager and the decode step's tables, as the oracle computes them."""

    def __init__(self, wl, keep_values=True):
        self.wl = wl
        dt = np.float32 if wl.dtype == "f32" else np.uint16
        shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
        if wl.pool_init is not None:
            # slots never written keep these bits ([ENG §3.2]: nothing clears
            # a block)
            self.k_pool = np.array(wl.pool_init[0], dtype=dt, copy=True).reshape(shape)
            self.v_pool = np.array(wl.pool_init[1], dtype=dt, copy=True).reshape(shape)
        else:
            self.k_pool = np.zeros(shape, dtype=dt)
            self.v_pool = np.zeros(shape, dtype=dt)
        hshape = (wl.num_host_blocks,) + shape[1:]
        self.k_host = np.zeros(hshape, dtype=dt)
        self.v_host = np.zeros(hshape, dtype=dt)
        self.bm = BlockManager(wl.num_blocks, wl.block_size, wl.free_order,
                               wl.num_host_blocks, wl.host_free_order)
        self.ctx_slots = []
        self.swaps = []            # (kind, pairs) of every swap in the trace
        # Token-order histories of every sequence (for the contiguous check).
        self.keep_values = keep_values
        self.hist_k: dict[int, list] = {}
        self.hist_v: dict[int, list] = {}

    # context build --------------------------------------------------------
    def build_context(self):
        wl, bm = self.wl, self.bm
        cursor = 0
        for op in wl.ops:
            kind = op[0]
            if kind == "add":
                bm.add_seq(op[1])
                self._hist_init(op[1])
            elif kind == "append":
                s, n = op[1], op[2]
                slots, cow = bm.append_slots([s], n)
                self._copy(cow)
                self._write(wl.ctx_k[cursor:cursor + n], wl.ctx_v[cursor:cursor + n], slots)
                self.ctx_slots.extend(slots)
                if self.keep_values:
                    self.hist_k[s].extend(range(cursor, cursor + n))
                    self.hist_v[s].extend(range(cursor, cursor + n))
                cursor += n
            elif kind == "share_prefix":
                dst, src, n = op[1], op[2], op[3]
                bm.share_prefix(dst, src, n)
                if self.keep_values:
                    self.hist_k[dst] = list(self.hist_k[src][:n])
                    self.hist_v[dst] = list(self.hist_v[src][:n])
            elif kind == "fork":
                p, c = op[1], op[2]
                bm.fork(p, c)
                if self.keep_values:
                    self.hist_k[c] = list(self.hist_k[p])
                    self.hist_v[c] = list(self.hist_v[p])
            elif kind == "swap_out":
                pairs = bm.swap_out(list(op[1]))
                self._swap(pairs, to_host=True)
                self.swaps.append((kind, pairs))
            elif kind == "swap_in":
                pairs = bm.swap_in(list(op[1]))
                self._swap(pairs, to_host=False)
                self.swaps.append((kind, pairs))
            elif kind == "free":
                bm.free_seq(op[1])
                if self.keep_values:
                    del self.hist_k[op[1]], self.hist_v[op[1]]
            else:
                raise ValueError(f"unknown op {kind}")
            bm.check()
        assert cursor == wl.ctx_tokens

    def _hist_init(self, s):
        if self.keep_values:
            self.hist_k[s] = []
            self.hist_v[s] = []

    # decode step ----------------------------------------------------------
    def decode_tables(self):
        """Host part of the step: one appended slot per sequence, the CoW pairs,
        then the exported tables and lengths."""
        wl = self.wl
        slots, cow = self.bm.append_slots([int(s) for s in wl.decode_seqs], 1)
        self.bm.check()
        rows, lens = self.bm.export([int(s) for s in wl.decode_seqs], wl.max_blocks_per_seq)
        self.slot_mapping = np.asarray(slots, dtype=np.int32)
        self.cow_pairs = np.asarray(cow, dtype=np.int32).reshape(-1, 2)
        self.block_tables = np.asarray(rows, dtype=np.int32)
        self.seq_lens = np.asarray(lens, dtype=np.int32)
        assert np.array_equal(self.seq_lens, wl.seq_lens)
        if self.keep_values:
            for i, s in enumerate(wl.decode_seqs):
                self.hist_k[int(s)].append(("new", i))
                self.hist_v[int(s)].append(("new", i))

    def _write(self, k, v, slots):
        write(k, v, slots, self.k_pool, self.v_pool)

    def _copy(self, pairs):
        copy_blocks(pairs, self.k_pool, self.v_pool)

    def _swap(self, pairs, to_host):
        for dev, host in ((self.k_pool, self.k_host), (self.v_pool, self.v_host)):
            if to_host:
                swap_blocks(pairs, dev, host)
            else:
                swap_blocks(pairs, host, dev)

    def decode_device_part(self):
        """copy -> write on the oracle pools."""
        self._copy(self.cow_pairs.tolist())
        self._write(self.wl.new_k, self.wl.new_v, self.slot_mapping)

    def attention(self, seqs=None):
        from .attention import attention_decode
        wl = self.wl
        return attention_decode(wl.q, self.k_pool, self.v_pool, self.block_tables,
                                self.seq_lens, wl.scale, seqs=seqs)

    def history(self, s):
        """Token-order K/V of sequence ``s`` rebuilt from the drawn values
        (no pool involved)."""
        wl = self.wl

        def rows(idx, ctx, new):
            out = []
            for r in idx:
                out.append(new[r[1]] if isinstance(r, tuple) else ctx[r])
            if not out:
                return np.zeros((0,) + ctx.shape[1:], dtype=ctx.dtype)
            return np.stack(out)
        return rows(self.hist_k[s], wl.ctx_k, wl.new_k), rows(self.hist_v[s], wl.ctx_v, wl.new_v)


def run_step(wl, keep_values=True):
    """Full oracle decode step.  Returns the ``OracleState`` after copy and write
    (attention is computed on demand with ``.attention()``)."""
    st = OracleState(wl, keep_values=keep_values)
    st.build_context()
    st.decode_tables()
    st.decode_device_part()
    return st


class QuantOracleState(OracleState):
    """The same step over a quantized cache (oracle/quant.py): writes encode
    the workload's bf16 rows, copies carry INT8 scale rows, attention reads the
    dequantized pools."""

    def __init__(self, wl, kind, k_scale=1.0, v_scale=1.0, keep_values=False):
        from . import quant
        super().__init__(wl, keep_values=keep_values)
        self.kind, self.k_scale, self.v_scale = kind, float(k_scale), float(v_scale)
        dt = np.uint8 if kind == quant.FP8 else np.int8
        self.k_pool = np.zeros(self.k_pool.shape, dtype=dt)
        self.v_pool = np.zeros(self.v_pool.shape, dtype=dt)
        self.k_host = np.zeros(self.k_host.shape, dtype=dt)
        self.v_host = np.zeros(self.v_host.shape, dtype=dt)
        if kind == quant.INT8:
            n = wl.num_blocks * wl.block_size
            self.k_scales = np.zeros((n, wl.num_kv_heads), np.float32)
            self.v_scales = np.zeros((n, wl.num_kv_heads), np.float32)
            hn = wl.num_host_blocks * wl.block_size
            self.k_scales_host = np.zeros((hn, wl.num_kv_heads), np.float32)
            self.v_scales_host = np.zeros((hn, wl.num_kv_heads), np.float32)
        else:
            self.k_scales = self.v_scales = None
            self.k_scales_host = self.v_scales_host = None

    def _write(self, k, v, slots):
        from . import quant
        quant.write_quant(k, v, slots, self.k_pool, self.v_pool, self.kind, self.k_scale,
                          self.v_scale, self.k_scales, self.v_scales)

    def _copy(self, pairs):
        from . import quant
        quant.copy_blocks_quant(pairs, self.k_pool, self.v_pool, self.kind, self.k_scales,
                                self.v_scales)

    def _swap(self, pairs, to_host):
        super()._swap(pairs, to_host)
        if self.k_scales is None:
            return
        B, H = self.wl.block_size, self.wl.num_kv_heads
        for dev, host in ((self.k_scales, self.k_scales_host),
                          (self.v_scales, self.v_scales_host)):
            d3, h3 = dev.reshape(-1, B, H), host.reshape(-1, B, H)
            if to_host:
                swap_blocks(pairs, d3, h3)
            else:
                swap_blocks(pairs, h3, d3)

    def attention(self, seqs=None):
        from . import quant
        wl = self.wl
        return quant.attention_decode_quant(wl.q, self.k_pool, self.v_pool, self.block_tables,
                                            self.seq_lens, wl.scale, self.kind, self.k_scale,
                                            self.v_scale, self.k_scales, self.v_scales, seqs=seqs)


def run_step_quant(wl, kind, k_scale=1.0, v_scale=1.0):
    """Full oracle decode step over a quantized cache (see QuantOracleState)."""
    st = QuantOracleState(wl, kind, k_scale, v_scale)
    st.build_context()
    st.decode_tables()
    st.decode_device_part()
    return st
