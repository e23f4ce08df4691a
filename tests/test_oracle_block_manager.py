"""Pins of the oracle block manager against the pages' worked examples,
closed forms and invariants (no GPU)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.block_manager import BlockManager, NoFreeBlocks
from tests.conftest import load_golden


def forced_free_list(num_blocks, pops):
    """A free list whose first pops (from the end) yield ``pops`` in order."""
    rest = [b for b in range(num_blocks) if b not in pops]
    return rest + list(reversed(pops))


def test_slot_example_block_size_4():
    g = load_golden("slot_example_b4.json")
    B = g["block_size"]
    bm = BlockManager(8, B, forced_free_list(8, g["block_table"]))
    bm.add_seq(0)
    slots, cow = bm.append_slots([0], g["num_tokens"])
    assert cow == []
    assert bm.tables[0] == g["block_table"]
    # every position's slot = physical id * K + offset, position by position
    exp = []
    for lb, (a, b) in enumerate(g["logical_block_positions"]):
        for t in range(a, b + 1):
            assert t // B == lb
            exp.append(g["block_table"][lb] * B + t % B)
    assert slots == exp
    t = g["traced_position"]
    assert t // B == g["traced_logical_block"] and t % B == g["traced_offset"]
    assert slots[t] == g["traced_slot"] == 30
    used_last = g["num_tokens"] - (len(bm.tables[0]) - 1) * B
    assert used_last == g["last_block_used"] and B - used_last == g["last_block_empty"]
    bm.check()


def test_lifecycle_fig_19_6():
    g = load_golden("lifecycle_b4.json")
    B = g["block_size"]
    pops = g["prompt_table"] + [g["second_generated_new_block"]]
    bm = BlockManager(8, B, forced_free_list(8, pops))
    bm.add_seq(0)
    bm.append_slots([0], g["prompt_tokens"])
    assert bm.tables[0] == g["prompt_table"]
    filled = [min(B, bm.filled[0] - i * B) for i in range(len(bm.tables[0]))]
    assert filled == g["prompt_filled"]
    (s1,), _ = bm.append_slots([0], 1)          # "fathers"
    assert s1 // B == g["first_generated_block"] and s1 == 1 * B + 3
    (s2,), _ = bm.append_slots([0], 1)          # "brought"
    assert s2 // B == g["second_generated_new_block"] and s2 == 3 * B + 0
    assert bm.tables[0] == g["table_after_second"]
    filled = [min(B, bm.filled[0] - i * B) for i in range(len(bm.tables[0]))]
    assert filled == g["filled_after_second"]
    bm.free_seq(0)
    assert bm.num_free() == 8
    bm.check()


@pytest.mark.parametrize("case", load_golden("block_counts.json")["cases"])
def test_block_counts(case):
    n, B = case["tokens"], case["block_size"]
    pops = case.get("physical")
    nb = 64
    bm = BlockManager(nb, B, forced_free_list(nb, pops) if pops else None)
    bm.add_seq(0)
    bm.append_slots([0], n)
    assert len(bm.tables[0]) == case["blocks"]
    assert len(bm.tables[0]) * B - n == case["unused"]
    if "reserved_positions" in case:
        assert len(bm.tables[0]) * B == case["reserved_positions"]
    if pops:
        assert bm.tables[0] == pops
    assert nb - bm.num_free() == case["blocks"]


def test_max_unused_is_block_size_minus_one():
    g = load_golden("block_counts.json")
    worst = 0
    for n in range(1, 200):
        bm = BlockManager(64, 16)
        bm.add_seq(0)
        bm.append_slots([0], n)
        worst = max(worst, len(bm.tables[0]) * 16 - n)
    assert worst == g["max_unused_block16"] == 15


def test_refcount_two_one_zero():
    g = load_golden("refcounts.json")
    P = g["shared_block"]
    bm = BlockManager(16, 4, forced_free_list(16, [P]))
    bm.add_seq("A")
    bm.append_slots(["A"], 4)                    # A fills P7
    bm.add_seq("B")
    bm.share_prefix("B", "A", 4)
    assert bm.ref[P] == g["counts_A_and_B"]
    bm.free_seq("A")
    assert bm.ref[P] == g["after_A_ends"] and P not in bm.free
    bm.free_seq("B")
    assert bm.ref[P] == g["after_B_ends"] and P in bm.free
    bm.check()


def test_prefix_blocks_3_and_5_shared():
    g = load_golden("refcounts.json")
    blocks = g["prefix_shared_blocks"]
    bm = BlockManager(16, 4, forced_free_list(16, blocks))
    bm.add_seq(0)
    bm.append_slots([0], 8)
    bm.add_seq(1)
    bm.share_prefix(1, 0, 8)
    assert bm.tables[0] == bm.tables[1] == blocks
    assert [bm.ref[b] for b in blocks] == [2, 2]
    bm.append_slots([1], 1)                      # next block boundary: private block
    assert bm.tables[1][:2] == blocks and bm.ref[bm.tables[1][2]] == 1
    bm.free_seq(0)
    assert [bm.ref[b] for b in blocks] == [1, 1]
    bm.free_seq(1)
    assert bm.num_free() == 16
    bm.check()


def test_copy_on_write_fig_19_8():
    g = load_golden("refcounts.json")
    bm = BlockManager(16, 4, forced_free_list(16, [9, 2, 11]))
    bm.add_seq("A1")
    bm.append_slots(["A1"], 6)                   # blocks 9 (full) and 2 (2 of 4)
    bm.fork("A1", "A2")
    assert bm.ref[9] == bm.ref[2] == g["fork_count"]
    slots, cow = bm.append_slots(["A1"], 1)      # A1 writes into shared block 2
    assert cow == [(2, 11)]                      # new block, copy of 2
    assert bm.tables["A1"] == [9, 11] and slots == [11 * 4 + 2]
    assert bm.ref[2] == 1 and bm.ref[11] == 1 and bm.ref[9] == 2
    slots, cow = bm.append_slots(["A2"], 1)      # A2 is now the only user of 2
    assert cow == [] and slots == [2 * 4 + 2] and bm.tables["A2"] == [9, 2]
    bm.check()


def test_fork_family_cow_count_and_order():
    """Parent + 3 children share a partial last block: the first three writers
    (ascending id) copy, the last writes in place."""
    bm = BlockManager(32, 4)
    bm.add_seq(0)
    bm.append_slots([0], 5)
    for c in (1, 2, 3):
        bm.fork(0, c)
    last = bm.tables[0][1]
    assert bm.ref[last] == 4
    slots, cow = bm.append_slots([0, 1, 2, 3], 1)
    assert [p[0] for p in cow] == [last] * 3
    assert bm.tables[3][1] == last and bm.ref[last] == 1
    assert len({bm.tables[s][1] for s in range(4)}) == 4
    assert all(s % 4 == 1 for s in slots)
    bm.check()


def test_exhaustion_is_all_or_nothing():
    bm = BlockManager(3, 4)
    bm.add_seq(0)
    bm.add_seq(1)
    bm.append_slots([0], 8)
    before = (list(bm.free), list(bm.ref), {k: list(v) for k, v in bm.tables.items()},
              dict(bm.filled))
    with pytest.raises(NoFreeBlocks):
        bm.append_slots([1, 0], 5)               # needs 2 + 1 blocks, 1 free
    after = (list(bm.free), list(bm.ref), {k: list(v) for k, v in bm.tables.items()},
             dict(bm.filled))
    assert before == after
    bm.check()


def test_selfcheck_pool_counts():
    g = load_golden("selfcheck_kvm.json")
    bm = BlockManager(g["num_blocks"], g["block_size"])
    bm.add_seq(0)
    for _ in range(g["tokens"]):
        bm.append_slots([0], 1)
    assert len(bm.tables[0]) == g["blocks_used"]
    bm.free_seq(0)
    assert bm.num_free() == g["free_after_release"]


def test_initial_free_list_pops_from_end():
    """[KVM §19.2.3]: the free list starts as every id and allocation takes the
    last one, so a fresh pool hands out n-1, n-2, ..."""
    bm = BlockManager(5, 2)
    bm.add_seq(0)
    bm.append_slots([0], 6)
    assert bm.tables[0] == [4, 3, 2]
    bm.free_seq(0)
    assert bm.free == [0, 1, 4, 3, 2]            # released in table order, to the end
    bm.add_seq(1)
    bm.append_slots([1], 1)
    assert bm.tables[1] == [2]                   # most recently freed first


@settings(max_examples=60, deadline=None)
@given(st.data())
def test_random_traces_keep_invariants(data):
    nb = data.draw(st.integers(4, 40))
    B = data.draw(st.sampled_from([1, 2, 4, 8, 16]))
    bm = BlockManager(nb, B, list(np.random.default_rng(data.draw(st.integers(0, 99))).permutation(nb)))
    live, nxt = [], 0
    for _ in range(data.draw(st.integers(1, 40))):
        op = data.draw(st.sampled_from(["add", "append", "fork", "free", "share"]))
        try:
            if op == "add" or not live:
                bm.add_seq(nxt); live.append(nxt); nxt += 1
            elif op == "append":
                seqs = data.draw(st.lists(st.sampled_from(live), min_size=1, max_size=4, unique=True))
                bm.append_slots(seqs, data.draw(st.integers(1, 6)))
            elif op == "fork":
                bm.fork(data.draw(st.sampled_from(live)), nxt); live.append(nxt); nxt += 1
            elif op == "free":
                s = data.draw(st.sampled_from(live)); bm.free_seq(s); live.remove(s)
            else:
                src = data.draw(st.sampled_from(live))
                bm.add_seq(nxt); live.append(nxt); nxt += 1
                bm.share_prefix(nxt - 1, src, data.draw(st.integers(0, bm.filled[src])))
        except NoFreeBlocks:
            pass
        bm.check()
    for s in list(live):
        bm.free_seq(s)
    assert bm.num_free() == nb
