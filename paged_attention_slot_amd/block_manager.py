"""Python handle for the library's host block manager (``pkv_bm_*``)."""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import PKV_ERR_NO_FREE_BLOCKS, P_i32, P_i64, PkvError, check, lib


class NoFreeBlocks(PkvError):
    pass


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(P_i32)


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(P_i64)


class BlockManager:
    """Free list, reference counts and block tables, held by ``libpkv``."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None,
                 num_host_blocks: int = 0, host_free_order=None):
        self._lib = lib()
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        fo = None
        if free_order is not None:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.size != num_blocks:
                raise ValueError("free_order must have num_blocks entries")
        h = self._lib.pkv_bm_create(num_blocks, block_size, None if fo is None else _i32p(fo))
        if not h:
            check(1, "pkv_bm_create")
        self._h = ctypes.c_void_p(h)
        self.num_host_blocks = int(num_host_blocks)
        if num_host_blocks:
            ho = None
            if host_free_order is not None:
                ho = np.ascontiguousarray(host_free_order, dtype=np.int32)
                if ho.size != num_host_blocks:
                    raise ValueError("host_free_order must have num_host_blocks entries")
            self._check(self._lib.pkv_bm_add_host_pool(self._h, int(num_host_blocks),
                                                       None if ho is None else _i32p(ho)),
                        "add_host_pool")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_bm_destroy(h)
            self._h = None

    def _check(self, st, where):
        if st == PKV_ERR_NO_FREE_BLOCKS:
            raise NoFreeBlocks(st, where, self._lib.pkv_last_error().decode())
        check(st, where)

    def add_seq(self, seq: int) -> None:
        self._check(self._lib.pkv_bm_add_seq(self._h, int(seq)), "add_seq")

    def share_prefix(self, dst: int, src: int, num_tokens: int) -> None:
        self._check(self._lib.pkv_bm_share_prefix(self._h, int(dst), int(src), int(num_tokens)),
                    "share_prefix")

    def fork(self, parent: int, child: int) -> None:
        self._check(self._lib.pkv_bm_fork(self._h, int(parent), int(child)), "fork")

    def append_slots(self, seqs, tokens_each: int = 1):
        """Returns (slots int32 [n*tokens_each], cow_pairs int32 [P, 2])."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.size
        slots = np.empty(max(1, n * tokens_each), dtype=np.int32)
        cow = np.empty((max(1, n), 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        self._check(self._lib.pkv_bm_append_slots(self._h, _i64p(s), n, int(tokens_each),
                                                  _i32p(slots), _i32p(cow), ctypes.byref(ncow)),
                    "append_slots")
        return slots[:n * tokens_each].copy(), cow[:ncow.value].copy()

    def free_seq(self, seq: int) -> None:
        self._check(self._lib.pkv_bm_free_seq(self._h, int(seq)), "free_seq")

    def export(self, seqs, max_blocks: int):
        """Returns (block_tables int32 [n, max_blocks] padded with -1, lens int32 [n])."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        tables = np.empty((s.size, max_blocks), dtype=np.int32)
        lens = np.empty(s.size, dtype=np.int32)
        self._check(self._lib.pkv_bm_export(self._h, _i64p(s), s.size, int(max_blocks),
                                            _i32p(tables), _i32p(lens)), "export")
        return tables, lens

    def num_free(self) -> int:
        return int(self._lib.pkv_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pkv_bm_refcount(self._h, int(block)))

    def num_tokens(self, seq: int) -> int:
        return int(self._lib.pkv_bm_num_tokens(self._h, int(seq)))

    def free_list(self) -> np.ndarray:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int32(0)
        self._check(self._lib.pkv_bm_free_list(self._h, _i32p(out), out.size, ctypes.byref(n)),
                    "free_list")
        return out[:n.value].copy()

    def check(self) -> None:
        self._check(self._lib.pkv_bm_check(self._h), "check")

    # -- swap (host tier) -------------------------------------------------------
    def distinct_blocks(self, seqs) -> int:
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = int(self._lib.pkv_bm_distinct_blocks(self._h, _i64p(s), s.size))
        if n < 0:
            raise PkvError(1, "distinct_blocks", "unknown sequence")
        return n

    def _swap(self, fn, seqs, where):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        cap = self.distinct_blocks(s) if s.size else 0
        pairs = np.empty((max(1, cap), 2), dtype=np.int32)
        n = ctypes.c_int32(0)
        self._check(fn(self._h, _i64p(s), s.size, _i32p(pairs), cap, ctypes.byref(n)), where)
        return pairs[:n.value].copy()

    def swap_out(self, seqs) -> np.ndarray:
        """Pause the sequences; returns int32 [P, 2] (device block, host block)."""
        return self._swap(self._lib.pkv_bm_swap_out, seqs, "swap_out")

    def swap_in(self, seqs) -> np.ndarray:
        """Resume the sequences; returns int32 [P, 2] (host block, device block)."""
        return self._swap(self._lib.pkv_bm_swap_in, seqs, "swap_in")

    def is_swapped(self, seq: int) -> bool:
        r = int(self._lib.pkv_bm_is_swapped(self._h, int(seq)))
        if r < 0:
            raise PkvError(1, "is_swapped", f"unknown sequence {seq}")
        return bool(r)

    def num_free_host(self) -> int:
        return int(self._lib.pkv_bm_num_free_host(self._h))

    def host_refcount(self, block: int) -> int:
        return int(self._lib.pkv_bm_host_refcount(self._h, int(block)))

    def host_free_list(self) -> np.ndarray:
        out = np.empty(max(1, self.num_host_blocks), dtype=np.int32)
        n = ctypes.c_int32(0)
        self._check(self._lib.pkv_bm_host_free_list(self._h, _i32p(out), out.size,
                                                    ctypes.byref(n)), "host_free_list")
        return out[:n.value].copy()
