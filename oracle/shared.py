"""Oracle for shared-prefix groups (integers only).  Test infrastructure.

Sequences that take a common prefix by reference hold the same physical block
ids at the start of their block tables ([KVM §19.2.5]: a cached prefix's blocks
are pointed to by every request that reuses it, its reference count equal to
the number of those requests; [PFX §prefix]).  Paging alone does not make the
attention kernel read those blocks once: whether the reads are shared depends
on the kernel ([KVX §04] what paging does not solve; [KVX §05] shared prefixes
dedupe storage, read reuse depends on the kernel and the caches).  A kernel
that reads a group's prefix once needs the groups; this is how they are read
off the tables.

Attention over groups computes exactly decode attention (the oracle's
``attention.attention_decode``): the group only changes which reads serve
which positions.

Grouping rule (the plainest reading):
* a group is a maximal run of consecutive sequences whose first valid table
  entry is the same block id (a sequence with no token starts a run of its
  own);
* the group's shared blocks are the longest run of leading entries that every
  member holds as valid entries (entry i is valid for a member of length L when
  i < ceil(L / B)) and that are equal across the members;
* prefix_len = shared blocks x B tokens for a group of two or more members,
  0 for a group of one (nothing to share).  A member shorter than prefix_len
  sees only its own positions of the last shared block.
"""
from __future__ import annotations

import numpy as np


def _valid(row, L, B):
    n = -(-int(L) // B)
    return [int(b) for b in row[:n]]


def prefix_groups(tables, lens, block_size):
    """Returns (group_starts int32 [G + 1], prefix_lens int32 [G])."""
    tables = np.asarray(tables)
    lens = np.asarray(lens)
    B = int(block_size)
    rows = [_valid(tables[s], lens[s], B) for s in range(lens.size)]
    starts, plens = [], []
    s = 0
    while s < len(rows):
        e = s + 1
        if rows[s]:
            while e < len(rows) and rows[e] and rows[e][0] == rows[s][0]:
                e += 1
        k = 0
        if e - s >= 2:
            limit = min(len(rows[i]) for i in range(s, e))
            while k < limit and all(rows[i][k] == rows[s][k] for i in range(s, e)):
                k += 1
        starts.append(s)
        plens.append(k * B)
        s = e
    starts.append(len(rows))
    return np.asarray(starts, np.int32), np.asarray(plens, np.int32)
