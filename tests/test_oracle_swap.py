"""Pins of the oracle's swap path (block manager host tier + block movement).

What the pages fix ([KVM §19.2.6]: a paused request releases all of its blocks
at once and its KV cache is moved to CPU memory and back; [ENG §8.2]: the block
table makes the move invisible to attention) is checked here against facts
that do not come from the swap code:
  * token-order histories rebuilt from the drawn values alone (no pool), read
    back through the final tables with the token-slot equation;
  * block counts in closed form (ceil(L / B) per independent sequence);
  * the free lists and reference counts of both pools against a brute-force
    recount, and the exact state restore of a failed call.
A set of planted mistakes (copies of the manager, on the CPU) must each fail
one of these pins.
"""
import copy

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.block_manager import BlockManager, NoFreeBlocks
from oracle.cache_ops import swap_blocks
from oracle.replay import run_step
from workloads import preemption_workload


def slot_rows(pool, table, n, B):
    """Rows of tokens 0..n-1 read through a table (slot = block * B + offset)."""
    return np.stack([pool[table[t // B], t % B] for t in range(n)]) if n else pool[:0, 0]


def history_matches(st, wl):
    B = wl.block_size
    rows, lens = st.bm.export([int(s) for s in wl.decode_seqs], wl.max_blocks_per_seq)
    for i, s in enumerate(wl.decode_seqs):
        K, V = st.history(int(s))
        if not (np.array_equal(slot_rows(st.k_pool, rows[i], lens[i], B), K)
                and np.array_equal(slot_rows(st.v_pool, rows[i], lens[i], B), V)):
            return False
    return True


SCENARIOS = {
    # independent sequences; the two latecomers are paused while the others grow
    "latecomers": dict(lens_before=[20, 7, 33, 16, 9], swapped=[3, 4], grow=[13, 30, 5, 0, 0]),
    # a forked pair swapped together (its blocks move once and stay shared)
    "fork-pair": dict(lens_before=[18, 11, 30], forks=[0], swapped=[0, 3], grow=[0, 21, 9, 0]),
    # only the child of a fork is swapped; the parent keeps the shared blocks
    "fork-child": dict(lens_before=[18, 11], forks=[0], swapped=[2], grow=[6, 3, 0]),
    # every sequence paused, nothing grows: the blocks come back in a new order
    "all": dict(lens_before=[5, 12, 1, 8], swapped=[0, 1, 2, 3], grow=[0, 0, 0, 0]),
    # empty and whole-block lengths
    "edges": dict(lens_before=[0, 8, 4, 16], swapped=[0, 1, 3], grow=[0, 0, 9, 0]),
}


def scenario(name, dtype="f32", B=4, seed=5, **kw):
    args = dict(SCENARIOS[name])
    args.update(kw)
    return preemption_workload(num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=B,
                               dtype=dtype, seed=seed, **args)


@pytest.mark.parametrize("name", sorted(SCENARIOS))
@pytest.mark.parametrize("B", [1, 4, 8])
def test_round_trip_restores_every_history(name, B):
    wl = scenario(name, B=B)
    st = run_step(wl)
    st.bm.check()
    assert history_matches(st, wl)


def test_released_blocks_are_really_overwritten():
    """The residents' growth takes the blocks the swap released (most recently
    freed first), so the restored values cannot come from the device pool."""
    wl = scenario("latecomers")
    st = run_step(wl)
    (k0, out_pairs), (k1, in_pairs) = st.swaps
    assert (k0, k1) == ("swap_out", "swap_in")
    released = {b for b, _ in out_pairs}
    rows, _ = st.bm.export([0, 1, 2], wl.max_blocks_per_seq)
    taken_by_residents = {b for r in rows for b in r if b >= 0}
    assert released & taken_by_residents
    # and the swapped sequences came back in other blocks than they left
    back = {b for _, b in in_pairs}
    assert back - released


def test_block_counts_closed_form():
    lens = [20, 7, 33, 16, 9, 1, 64]
    B = 8
    bm = BlockManager(40, B, num_host_blocks=30)
    for s, L in enumerate(lens):
        bm.add_seq(s)
        bm.append_slots([s], L)
    used = sum(-(-L // B) for L in lens)
    out = [1, 4, 6]
    k = sum(-(-lens[s] // B) for s in out)
    pairs = bm.swap_out(out)
    assert len(pairs) == k
    assert len({b for b, _ in pairs}) == k and len({h for _, h in pairs}) == k
    assert bm.num_free() == 40 - used + k and bm.num_free_host() == 30 - k
    bm.check()
    back = bm.swap_in(out)
    assert len(back) == k and {h for h, _ in back} == {h for _, h in pairs}
    assert bm.num_free() == 40 - used and bm.num_free_host() == 30
    assert [bm.filled[s] for s in out] == [lens[s] for s in out]
    bm.check()


def test_shared_blocks_move_once_and_stay_shared():
    B = 4
    bm = BlockManager(20, B, num_host_blocks=20)
    bm.add_seq(0)
    bm.append_slots([0], 10)               # blocks: 2 full + 1 partial
    bm.fork(0, 1)
    t = list(bm.tables[0])
    pairs = bm.swap_out([0, 1])
    assert [b for b, _ in pairs] == t       # first appearance order, each once
    for _, h in pairs:
        assert bm.href[h] == 2
    assert all(bm.ref[b] == 0 for b in t) and bm.num_free() == 20
    back = bm.swap_in([0, 1])
    assert bm.tables[0] == bm.tables[1]
    assert all(bm.ref[b] == 2 for b in bm.tables[0])
    # the next token of either one copies the shared partial block
    _, cow = bm.append_slots([1], 1)
    assert cow == [(bm.tables[0][2], bm.tables[1][2])]
    assert len(back) == 3
    bm.check()


def test_swapping_one_sharer_keeps_the_other_resident():
    bm = BlockManager(12, 4, num_host_blocks=8)
    bm.add_seq(0)
    bm.append_slots([0], 9)
    bm.fork(0, 1)
    t = list(bm.tables[0])
    free0 = bm.num_free()
    pairs = bm.swap_out([1])
    assert [b for b, _ in pairs] == t
    assert all(bm.ref[b] == 1 for b in t) and bm.num_free() == free0
    bm.swap_in([1])
    assert not set(bm.tables[1]) & set(t)     # private copies now
    bm.check()


def state_of(bm):
    return (list(bm.free), list(bm.ref), copy.deepcopy(bm.tables), dict(bm.filled),
            list(bm.hfree), list(bm.href), set(bm.swapped))


def test_exhaustion_is_all_or_nothing_both_ways():
    bm = BlockManager(10, 4, num_host_blocks=3)
    for s, L in enumerate([8, 7, 5]):
        bm.add_seq(s)
        bm.append_slots([s], L)              # 2 + 2 + 2 blocks
    snap = state_of(bm)
    with pytest.raises(NoFreeBlocks):
        bm.swap_out([0, 1])                  # needs 4 host blocks, 3 free
    assert state_of(bm) == snap
    bm.swap_out([0])
    bm.add_seq(9)
    bm.append_slots([9], 24)                 # 6 blocks: the device pool is full
    assert bm.num_free() == 0
    snap = state_of(bm)
    with pytest.raises(NoFreeBlocks):
        bm.swap_in([0])
    assert state_of(bm) == snap
    bm.free_seq(9)
    bm.swap_in([0])
    bm.check()


def test_swapped_sequences_take_no_other_operation():
    bm = BlockManager(10, 4, num_host_blocks=10)
    for s in (0, 1):
        bm.add_seq(s)
        bm.append_slots([s], 5)
    bm.swap_out([0])
    for call in (lambda: bm.append_slots([0], 1), lambda: bm.export([0], 4),
                 lambda: bm.fork(0, 7), lambda: bm.swap_out([0]), lambda: bm.swap_in([1]),
                 lambda: bm.swap_out([1, 1]), lambda: bm.share_prefix(1, 0, 1)):
        with pytest.raises(ValueError):
            call()
    bm.add_seq(8)
    with pytest.raises(ValueError):
        bm.share_prefix(8, 0, 2)
    assert bm.is_swapped(0) and not bm.is_swapped(1)
    bm.free_seq(0)                            # releases host blocks
    assert bm.num_free_host() == 10
    bm.check()


def test_swap_blocks_moves_whole_blocks_only_where_named():
    rng = np.random.default_rng(1)
    dev = rng.integers(0, 2**16, (6, 4, 2, 8)).astype(np.uint16)
    host = np.zeros((5, 4, 2, 8), np.uint16)
    swap_blocks([(3, 0), (1, 4), (3, 2)], dev, host)    # a src may repeat
    for h, b in ((0, 3), (4, 1), (2, 3)):
        assert np.array_equal(host[h], dev[b])
    assert not host[[1, 3]].any()
    back = np.zeros_like(dev)
    swap_blocks([(4, 5), (0, 0)], host, back)
    assert np.array_equal(back[5], dev[1]) and np.array_equal(back[0], dev[3])
    assert not back[1:5].any()
    for bad in ([(6, 0)], [(0, 5)], [(-1, 0)]):
        with pytest.raises(IndexError):
            swap_blocks(bad, dev, host)
    with pytest.raises(ValueError):
        swap_blocks([(0, 1), (2, 1)], dev, host)
    with pytest.raises(ValueError):
        swap_blocks([(0, 1)], dev, host.astype(np.float32))


@settings(max_examples=60, deadline=None)
@given(st.data())
def test_random_traces_with_swaps_keep_invariants(data):
    nb, nh = data.draw(st.integers(2, 30)), data.draw(st.integers(0, 30))
    B = data.draw(st.sampled_from([1, 2, 4, 8]))
    bm = BlockManager(nb, B, num_host_blocks=nh)
    nxt = 0
    for _ in range(data.draw(st.integers(1, 40))):
        res = [s for s in bm.tables if s not in bm.swapped]
        swp = sorted(bm.swapped)
        op = data.draw(st.sampled_from(["add", "append", "fork", "free", "out", "in"]))
        snap = state_of(bm)
        try:
            if op == "add" or not bm.tables:
                bm.add_seq(nxt)
                nxt += 1
            elif op == "append" and res:
                bm.append_slots(data.draw(st.lists(st.sampled_from(res), min_size=1, max_size=3)),
                                data.draw(st.integers(1, 6)))
            elif op == "fork" and res:
                bm.fork(data.draw(st.sampled_from(res)), nxt)
                nxt += 1
            elif op == "free":
                bm.free_seq(data.draw(st.sampled_from(sorted(bm.tables))))
            elif op == "out" and res:
                bm.swap_out(data.draw(st.lists(st.sampled_from(res), min_size=1, unique=True)))
            elif op == "in" and swp:
                bm.swap_in(data.draw(st.lists(st.sampled_from(swp), min_size=1, unique=True)))
        except NoFreeBlocks:
            assert state_of(bm) == snap
        bm.check()


# -- planted mistakes ---------------------------------------------------------

class NoDedup(BlockManager):
    """Gives every table entry its own host block (shared blocks move twice)."""

    def _distinct_blocks(self, seqs):
        return [b for s in seqs for b in self.tables[s]]

    def swap_out(self, seqs):
        seqs = self._check_swap_set(seqs, want_swapped=False)
        pairs = []
        for s in seqs:
            t = self.tables[s]
            for i, b in enumerate(t):
                if not self.hfree:
                    raise NoFreeBlocks("no free host block")
                h = self.hfree.pop()
                self.href[h] = 1
                pairs.append((b, h))
                t[i] = h
                self._release(b)
            self.swapped.add(s)
        return pairs


class KeepsHostRefs(BlockManager):
    """Forgets to release the host blocks on swap-in."""

    def _release_host(self, h):
        if any(h in self.tables[s] for s in self.swapped):
            super()._release_host(h)


class ReversedPairs(BlockManager):
    """Returns (host, device) from swap_out instead of (device, host)."""

    def swap_out(self, seqs):
        return [(h, b) for b, h in super().swap_out(seqs)]


class NoDeviceRelease(BlockManager):
    """Keeps the device references of swapped-out sequences."""

    def _release(self, b):
        if getattr(self, "_in_swap", False):
            return
        super()._release(b)

    def swap_out(self, seqs):
        self._in_swap = True
        try:
            return super().swap_out(seqs)
        finally:
            self._in_swap = False


def pins_pass(cls):
    import oracle.replay as replay
    saved = replay.BlockManager
    replay.BlockManager = cls
    try:
        for name in sorted(SCENARIOS):
            for B in (1, 4):
                wl = scenario(name, B=B)
                try:
                    st = replay.run_step(wl)
                    st.bm.check()
                except (AssertionError, IndexError, ValueError, NoFreeBlocks):
                    return False
                if not history_matches(st, wl):
                    return False
        try:
            test_block_counts_closed_form_for(cls)
            test_shared_for(cls)
        except (AssertionError, IndexError, ValueError, NoFreeBlocks):
            return False
        return True
    finally:
        replay.BlockManager = saved


def test_block_counts_closed_form_for(cls):
    bm = cls(12, 4, num_host_blocks=12)
    for s, L in enumerate([9, 4, 1]):
        bm.add_seq(s)
        bm.append_slots([s], L)
    pairs = bm.swap_out([0, 2])
    assert len(pairs) == 4 and bm.num_free_host() == 8 and bm.num_free() == 12 - 1
    bm.swap_in([0, 2])
    assert bm.num_free_host() == 12 and bm.num_free() == 12 - 5
    bm.check()


def test_shared_for(cls):
    bm = cls(10, 4, num_host_blocks=10)
    bm.add_seq(0)
    bm.append_slots([0], 6)
    bm.fork(0, 1)
    assert len(bm.swap_out([0, 1])) == 2 and bm.num_free_host() == 8
    bm.swap_in([0, 1])
    bm.check()


test_block_counts_closed_form_for.__test__ = False
test_shared_for.__test__ = False


def test_reference_manager_passes_swap_pins():
    assert pins_pass(BlockManager)


@pytest.mark.parametrize("cls", [NoDedup, KeepsHostRefs, ReversedPairs, NoDeviceRelease],
                         ids=lambda c: c.__name__)
def test_swap_mistake_caught(cls):
    assert not pins_pass(cls)
