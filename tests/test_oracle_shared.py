"""Pins of the shared-prefix grouping (oracle/shared.py).

Checked against what the trace fixes, not against the rule's own code: the
configuration whose 176 sequences all take a 2048-token prefix by reference
(one group, 128 shared blocks of 16), prefixes that end inside a block (the
copy-on-write of the first append leaves only the full blocks shared),
independent sequences (no sharing), forks whose only shared blocks are the
parent's; and, on random traces, the invariants: groups tile the batch in
order, every member's table holds the shared blocks, and no longer run is
shared."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.block_manager import BlockManager
from oracle.shared import prefix_groups
from workloads import config_workload, independent_workload, shared_prefix_workload


def groups_of(wl):
    """The decode step's tables from the oracle manager replaying the trace
    (no values needed), and their groups."""
    bm = BlockManager(wl.num_blocks, wl.block_size, wl.free_order)
    for op in wl.ops:
        if op[0] == "add":
            bm.add_seq(op[1])
        elif op[0] == "append":
            bm.append_slots([op[1]], op[2])
        elif op[0] == "share_prefix":
            bm.share_prefix(*op[1:])
        elif op[0] == "fork":
            bm.fork(*op[1:])
    seqs = [int(s) for s in wl.decode_seqs]
    bm.append_slots(seqs, 1)
    rows, lens = bm.export(seqs, wl.max_blocks_per_seq)

    class T:
        block_tables = np.asarray(rows, np.int32)
        seq_lens = np.asarray(lens, np.int32)
    return T, prefix_groups(T.block_tables, T.seq_lens, wl.block_size)


def test_shared_prefix_config_is_one_group():
    wl = config_workload("shared-prefix-cow", values=False)
    _, (starts, plens) = groups_of(wl)
    assert starts.tolist() == [0, wl.num_seqs] and wl.num_seqs == 176
    assert plens.tolist() == [2048]


@pytest.mark.parametrize("prefix,B", [(40, 16), (48, 16), (7, 8), (64, 32), (1, 16)])
def test_prefix_ending_inside_a_block(prefix, B):
    """The first suffix token written into the shared partial block copies it,
    so only the full blocks stay shared: floor(prefix / B) * B tokens."""
    wl = shared_prefix_workload(prefix_tokens=prefix, suffix_lens=[3, 9, 1, 20], forking_parents=0,
                                samples_per_fork=1, num_q_heads=4, num_kv_heads=2, head_dim=8,
                                block_size=B, dtype="f32", seed=3, values=False)
    # the generator sizes pools for block-aligned prefixes; each sharer here
    # also copies the partial block
    wl.num_blocks = 64
    wl.free_order = np.random.default_rng(0).permutation(64).astype(np.int32)
    _, (starts, plens) = groups_of(wl)
    full = prefix // B
    if full:
        assert starts.tolist() == [0, 4] and plens.tolist() == [full * B]
    else:   # nothing shared: every sequence's first block is its own copy
        assert starts.tolist() == [0, 1, 2, 3, 4] and plens.tolist() == [0, 0, 0, 0]


def test_independent_sequences_share_nothing():
    wl = independent_workload([5, 40, 17, 1, 64], num_q_heads=4, num_kv_heads=2, head_dim=8,
                              block_size=16, dtype="f32", seed=4, values=False)
    _, (starts, plens) = groups_of(wl)
    assert starts.tolist() == [0, 1, 2, 3, 4, 5] and not plens.any()


def test_fork_children_share_the_parents_full_blocks():
    """Parent 0 holds 33 tokens (blocks 0-1 full, block 2 partial) and forks
    two children; the decode append copies the partial block for each writer
    but the last, so the family of three shares blocks 0-1 (32 tokens)."""
    wl = shared_prefix_workload(prefix_tokens=0, suffix_lens=[33], forking_parents=1,
                                samples_per_fork=3, num_q_heads=4, num_kv_heads=2, head_dim=8,
                                block_size=16, dtype="f32", seed=5, values=False)
    ost, (starts, plens) = groups_of(wl)
    assert starts.tolist() == [0, 3] and plens.tolist() == [32]
    assert ost.seq_lens.tolist() == [34, 34, 34]


def test_identical_tables_share_only_the_blocks_holding_tokens():
    """Two sequences on the same three blocks (40 and 33 tokens, B = 16; e.g. a
    fork before either writes again) share exactly those blocks, 48 tokens:
    the padding after them is no block.  A third one-token sequence on block 5
    shares its one block with them."""
    tables = np.asarray([[5, 7, 9, -1], [5, 7, 9, -1], [5, -1, -1, -1]], np.int32)
    starts, plens = prefix_groups(tables[:2], np.asarray([40, 33]), 16)
    assert starts.tolist() == [0, 2] and plens.tolist() == [48]
    starts, plens = prefix_groups(tables, np.asarray([40, 33, 1]), 16)
    assert starts.tolist() == [0, 3] and plens.tolist() == [16]


@settings(max_examples=80, deadline=None)
@given(st.data())
def test_groups_on_random_tables_keep_the_invariants(data):
    B = data.draw(st.sampled_from([1, 2, 4, 16]))
    n = data.draw(st.integers(0, 9))
    nb = 12
    # tables built from a few shared stems so that runs and partial sharing occur
    stems = [data.draw(st.lists(st.integers(0, nb - 1), min_size=0, max_size=5)) for _ in range(3)]
    tables = np.full((max(n, 1), 8), -1, np.int32)
    lens = np.zeros(max(n, 1), np.int32)[:n]
    for s in range(n):
        stem = list(stems[data.draw(st.integers(0, 2))])
        tail = data.draw(st.lists(st.integers(0, nb - 1), min_size=0, max_size=8 - len(stem)))
        row = (stem + tail)[:8]
        L = data.draw(st.integers(0, len(row) * B)) if row else 0
        tables[s, :len(row)] = row
        lens[s] = L
    starts, plens = prefix_groups(tables[:n], lens, B)
    assert starts[0] == 0 and starts[-1] == n and np.all(np.diff(starts) >= 1)
    for g in range(len(plens)):
        mem = range(starts[g], starts[g + 1])
        k = plens[g] // B
        assert plens[g] % B == 0
        valid = [tables[s, :-(-lens[s] // B)].tolist() for s in mem]
        if len(mem) == 1:
            assert plens[g] == 0
            continue
        assert all(v and v[0] == valid[0][0] for v in valid)      # same first block
        assert all(len(v) >= k and v[:k] == valid[0][:k] for v in valid)
        longer = all(len(v) > k for v in valid) and len({v[k] for v in valid}) == 1
        assert not longer                                          # maximal
    # maximal runs: neighbours across a group boundary differ in their first block
    for g in range(1, len(plens)):
        a, b = starts[g] - 1, starts[g]
        fa = tables[a, 0] if lens[a] else None
        fb = tables[b, 0] if lens[b] else None
        assert fa is None or fb is None or fa != fb


# -- planted mistakes -------------------------------------------------------------

def _mutant(kind):
    import oracle.shared as sh

    def groups(tables, lens, B):
        tables, lens = np.asarray(tables), np.asarray(lens)
        if kind == "padding_counts":      # compares whole rows, padding included
            rows = [[int(b) for b in tables[s]] for s in range(lens.size)]
        else:
            rows = [sh._valid(tables[s], lens[s], B) for s in range(lens.size)]
        starts, plens, s = [], [], 0
        while s < len(rows):
            e = s + 1
            while e < len(rows) and rows[s] and rows[e] and rows[e][0] == rows[s][0]:
                e += 1
            k = 0
            if e - s >= (1 if kind == "singletons_share" else 2):
                limit = min(len(rows[i]) for i in range(s, e))
                while k < limit and all(rows[i][k] == rows[s][k] for i in range(s, e)):
                    k += 1
            starts.append(s)
            plens.append((k + (1 if kind == "one_block_more" else 0)) * B if k else 0)
            s = e
        starts.append(len(rows))
        return np.asarray(starts, np.int32), np.asarray(plens, np.int32)
    return groups


@pytest.mark.parametrize("kind", ["padding_counts", "singletons_share", "one_block_more"])
def test_grouping_mistakes_fail_a_pin(kind, monkeypatch):
    import oracle.shared as sh
    monkeypatch.setattr(sh, "prefix_groups", _mutant(kind))
    monkeypatch.setitem(globals(), "prefix_groups", _mutant(kind))
    pins = [test_shared_prefix_config_is_one_group, test_independent_sequences_share_nothing,
            test_fork_children_share_the_parents_full_blocks,
            test_identical_tables_share_only_the_blocks_holding_tokens,
            lambda: test_prefix_ending_inside_a_block(40, 16)]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
