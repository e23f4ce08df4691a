"""Oracle block manager (integers only).  Test infrastructure.

State, as the pages describe it:
* one pool of ``num_blocks`` physical blocks of ``block_size`` token slots;
* a free list of block ids ([KVM §19.2.3]: initialised with every id, a block is
  taken from the end and returned to the end; [ENG §3.2]: stack order, most
  recently freed first);
* one reference count per block, kept apart from the KV data ([ENG §5.3]);
* per sequence, a block table (logical block i -> physical id) and the number of
  tokens written ([KVM §19.2.2], Fig. 19-6 "# filled"; [ENG §2.1]).

Any failing operation raises and leaves the state exactly as it was
(all-or-nothing, [KVM §19.2.6]; out-of-blocks must reach the caller, [ENG §3.2]).

Swap ([KVM §19.2.6] recovery by moving a paused request's KV cache to CPU
memory and back; [KVM §19.2.2] concept table; [ENG §8.2] CPU memory as a
second-level block pool, invisible to attention because only the table
changes): an optional host pool of ``num_host_blocks`` blocks with its own free
list and reference counts, kept exactly like the device pool.  A swapped-out
sequence's table names host blocks; it takes part in no append, fork, prefix
share or export until it is swapped back in.
"""
from __future__ import annotations

import copy


class NoFreeBlocks(RuntimeError):
    """The pool has no free block ([KVM §19.2.3]: allocation on an empty pool fails)."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None,
                 num_host_blocks: int = 0, host_free_order=None):
        if num_blocks <= 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            free_order = range(num_blocks)
        self.free = [int(b) for b in free_order]
        if sorted(self.free) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.filled: dict[int, int] = {}
        # host tier (second-level pool)
        self.num_host_blocks = int(num_host_blocks)
        if host_free_order is None:
            host_free_order = range(num_host_blocks)
        self.hfree = [int(b) for b in host_free_order]
        if sorted(self.hfree) != list(range(num_host_blocks)):
            raise ValueError("host_free_order must be a permutation of range(num_host_blocks)")
        self.href = [0] * num_host_blocks
        self.swapped: set[int] = set()

    # -- pool ---------------------------------------------------------------
    def _allocate(self) -> int:
        # [KVM §19.2.3]: fail on an empty pool; otherwise take the last free id
        # and give it one reference.
        if not self.free:
            raise NoFreeBlocks("no free physical block")
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        # [KVM §19.2.3], [SLOT §release]: drop one reference; a block whose count
        # reaches zero goes back on the free list.  Its data is left in place
        # ([ENG §3.2]).
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    # -- sequences ----------------------------------------------------------
    def _need(self, seq):
        if seq not in self.tables:
            raise KeyError(f"unknown sequence {seq}")

    def _need_resident(self, seq):
        self._need(seq)
        if seq in self.swapped:
            raise ValueError(f"sequence {seq} is swapped out")

    def add_seq(self, seq: int) -> None:
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.filled[seq] = 0

    def _append_one(self, seq: int, cow_out: list) -> int:
        """Reserve the slot of the sequence's next token and return it."""
        B = self.block_size
        n = self.filled[seq]
        table = self.tables[seq]
        lb, off = divmod(n, B)          # [SLOT §locate]: logical block, offset
        if lb == len(table):
            # [KVM §19.2.2] step 2 / [PFX §principle]: a new physical block only
            # when the previous one is full.
            table.append(self._allocate())
        elif self.ref[table[lb]] > 1:
            # [KVM §19.2.2] Fig. 19-8 step 2: writing into a block others still
            # reference -> take a new block, copy the contents, remap the entry,
            # drop one reference on the old block.
            old = table[lb]
            new = self._allocate()
            cow_out.append((old, new))
            table[lb] = new
            self._release(old)
        self.filled[seq] = n + 1
        return table[lb] * B + off      # [SLOT §locate]: token-slot equation

    def append_slots(self, seqs, tokens_each: int = 1):
        """Append ``tokens_each`` tokens to each sequence of ``seqs`` in order
        (sequence-major).  Returns (slots, cow_pairs).  All-or-nothing."""
        for s in seqs:
            self._need_resident(s)
        snap = self._snapshot()
        slots, cow = [], []
        try:
            for s in seqs:
                for _ in range(tokens_each):
                    slots.append(self._append_one(s, cow))
        except Exception:
            self._restore(snap)
            raise
        return slots, cow

    def fork(self, parent: int, child: int) -> None:
        """Child starts as a copy of the parent: same table, same length, one
        more reference on every shared block ([ENG §5.1], [KVM §19.2.2])."""
        self._need_resident(parent)
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.filled[child] = self.filled[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def share_prefix(self, dst: int, src: int, num_tokens: int) -> None:
        """Empty sequence ``dst`` takes the blocks holding ``src``'s first
        ``num_tokens`` tokens by reference ([KVM §19.2.5]; [PFX §prefix])."""
        self._need_resident(dst)
        self._need_resident(src)
        if self.tables[dst] or self.filled[dst]:
            raise ValueError("share_prefix needs an empty destination")
        if num_tokens < 0 or num_tokens > self.filled[src]:
            raise ValueError("prefix longer than the source sequence")
        nb = -(-num_tokens // self.block_size)
        self.tables[dst] = list(self.tables[src][:nb])
        self.filled[dst] = num_tokens
        for b in self.tables[dst]:
            self.ref[b] += 1

    def free_seq(self, seq: int) -> None:
        """Release every block of the sequence, the partly filled last one
        included ([KVM §19.2.3] release of all blocks; [ENG §7.1])."""
        self._need(seq)
        if seq in self.swapped:
            for h in self.tables[seq]:
                self._release_host(h)
            self.swapped.discard(seq)
        else:
            for b in self.tables[seq]:
                self._release(b)
        del self.tables[seq]
        del self.filled[seq]

    # -- swap ([KVM §19.2.6]; [ENG §8.2]) ---------------------------------------
    def _release_host(self, h: int) -> None:
        # Host pool, same rule as the device pool: a host block whose count
        # reaches zero goes back on the host free list.
        self.href[h] -= 1
        if self.href[h] == 0:
            self.hfree.append(h)

    def _distinct_blocks(self, seqs):
        """Distinct block ids named by the sequences' tables, in order of first
        appearance (sequence order, then logical block order)."""
        seen, order = set(), []
        for s in seqs:
            for b in self.tables[s]:
                if b not in seen:
                    seen.add(b)
                    order.append(b)
        return order

    def _check_swap_set(self, seqs, want_swapped):
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("repeated sequence")
        for s in seqs:
            self._need(s)
            if (s in self.swapped) != want_swapped:
                raise ValueError(f"sequence {s} is {'resident' if want_swapped else 'swapped out'}")
        return seqs

    def swap_out(self, seqs):
        """Pause the sequences and move their KV cache to the host pool.

        Every distinct device block their tables name gets one host block
        (a block shared by several of them is moved once and stays shared on
        the host); each table entry is remapped to its host block and the
        device reference it held is released, table by table in order, so a
        device block no longer referenced by any resident sequence returns to
        the free list ([KVM §19.2.6]: all of the request's blocks at once).
        Returns the (device block, host block) pairs whose contents must be
        copied, in order of first appearance.  All-or-nothing: NoFreeBlocks
        (host pool too small) leaves the state unchanged."""
        seqs = self._check_swap_set(seqs, want_swapped=False)
        blocks = self._distinct_blocks(seqs)
        if len(blocks) > len(self.hfree):
            raise NoFreeBlocks("no free host block")
        to_host = {}
        for b in blocks:
            h = self.hfree.pop()
            self.href[h] = 0
            to_host[b] = h
        for s in seqs:
            t = self.tables[s]
            for i, b in enumerate(t):
                h = to_host[b]
                self.href[h] += 1
                t[i] = h
                self._release(b)
            self.swapped.add(s)
        return [(b, to_host[b]) for b in blocks]

    def swap_in(self, seqs):
        """Resume swapped-out sequences: every distinct host block of their
        tables gets a fresh device block (shared host blocks stay shared),
        tables are remapped and the host references released in table order.
        Returns the (host block, device block) pairs to copy, in order of first
        appearance.  All-or-nothing: NoFreeBlocks (too few free device blocks)
        leaves the state unchanged."""
        seqs = self._check_swap_set(seqs, want_swapped=True)
        hblocks = self._distinct_blocks(seqs)
        if len(hblocks) > len(self.free):
            raise NoFreeBlocks("no free physical block")
        to_dev = {}
        for h in hblocks:
            b = self.free.pop()
            self.ref[b] = 0
            to_dev[h] = b
        for s in seqs:
            t = self.tables[s]
            for i, h in enumerate(t):
                b = to_dev[h]
                self.ref[b] += 1
                t[i] = b
                self._release_host(h)
            self.swapped.discard(s)
        return [(h, to_dev[h]) for h in hblocks]

    # -- export / queries -----------------------------------------------------
    def export(self, seqs, max_blocks: int):
        """Rows of block ids padded with -1, and the token counts."""
        rows, lens = [], []
        for s in seqs:
            self._need_resident(s)
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("max_blocks too small")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.filled[s])
        return rows, lens

    def num_free(self) -> int:
        return len(self.free)

    def num_free_host(self) -> int:
        return len(self.hfree)

    def is_swapped(self, seq: int) -> bool:
        self._need(seq)
        return seq in self.swapped

    def check(self) -> None:
        """Invariants ([ENG §7.1], [ENG §7.2]), held with equality here."""
        assert len(set(self.free)) == len(self.free), "duplicate free id"
        assert len(set(self.hfree)) == len(self.hfree), "duplicate free host id"
        assert self.swapped <= set(self.tables), "swapped set names an unknown sequence"
        counted = [0] * self.num_blocks
        hcounted = [0] * self.num_host_blocks
        for s, t in self.tables.items():
            assert len(t) == -(-self.filled[s] // self.block_size), "table length"
            for b in t:
                if s in self.swapped:
                    hcounted[b] += 1
                else:
                    counted[b] += 1
        for cnt, ref, free, n in ((counted, self.ref, self.free, self.num_blocks),
                                  (hcounted, self.href, self.hfree, self.num_host_blocks)):
            assert cnt == ref, "refcount != references"
            in_use = {b for b in range(n) if ref[b] > 0}
            assert not (in_use & set(free)), "referenced block on free list"
            assert len(in_use) + len(free) == n, "leaked block"

    # -- rollback -------------------------------------------------------------
    def _snapshot(self):
        return (list(self.free), list(self.ref), copy.deepcopy(self.tables), dict(self.filled),
                list(self.hfree), list(self.href), set(self.swapped))

    def _restore(self, snap):
        (self.free, self.ref, self.tables, self.filled, self.hfree, self.href,
         self.swapped) = snap
