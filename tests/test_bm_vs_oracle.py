"""The library's C++ block manager against the oracle's on the same operation
traces: identical slots, copy-on-write pairs, tables, lengths, reference
counts and free lists, bit for bit (no GPU)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.block_manager import BlockManager as OracleBM
from oracle.block_manager import NoFreeBlocks as OracleNoFree
from workloads import CONFIG_ORDER, config_workload

pkv = pytest.importorskip("paged_attention_slot_amd")


def same_state(o: OracleBM, c, seqs):
    assert c.num_free() == o.num_free()
    assert np.array_equal(c.free_list(), np.asarray(o.free, dtype=np.int32))
    for b in range(o.num_blocks):
        assert c.refcount(b) == o.ref[b]
    if seqs:
        mb = max(1, max(len(o.tables[s]) for s in seqs))
        rows, lens = o.export(seqs, mb)
        ct, cl = c.export(seqs, mb)
        assert np.array_equal(ct, np.asarray(rows, dtype=np.int32))
        assert np.array_equal(cl, np.asarray(lens, dtype=np.int32))
    c.check()
    o.check()


@settings(max_examples=80, deadline=None)
@given(st.data())
def test_random_traces_match(data):
    nb = data.draw(st.integers(2, 48))
    B = data.draw(st.sampled_from([1, 2, 4, 8, 16, 32]))
    perm = np.random.default_rng(data.draw(st.integers(0, 10**6))).permutation(nb)
    o = OracleBM(nb, B, perm)
    c = pkv.BlockManager(nb, B, perm)
    live, nxt = [], 0
    for _ in range(data.draw(st.integers(1, 50))):
        op = data.draw(st.sampled_from(["add", "append", "append", "fork", "free", "share"]))
        if op == "add" or not live:
            o.add_seq(nxt)
            c.add_seq(nxt)
            live.append(nxt)
            nxt += 1
        elif op == "append":
            seqs = data.draw(st.lists(st.sampled_from(live), min_size=1, max_size=5))
            k = data.draw(st.integers(1, 7))
            try:
                so, co = o.append_slots(seqs, k)
                failed_o = False
            except OracleNoFree:
                failed_o = True
            try:
                sc, cc = c.append_slots(seqs, k)
                failed_c = False
            except pkv.NoFreeBlocks:
                failed_c = True
            assert failed_o == failed_c
            if not failed_o:
                assert np.array_equal(sc, np.asarray(so, dtype=np.int32))
                assert np.array_equal(cc.reshape(-1, 2), np.asarray(co, dtype=np.int32).reshape(-1, 2))
        elif op == "fork":
            p = data.draw(st.sampled_from(live))
            o.fork(p, nxt)
            c.fork(p, nxt)
            live.append(nxt)
            nxt += 1
        elif op == "free":
            s = data.draw(st.sampled_from(live))
            o.free_seq(s)
            c.free_seq(s)
            live.remove(s)
        else:
            src = data.draw(st.sampled_from(live))
            n = data.draw(st.integers(0, o.filled[src]))
            for m in (o, c):
                m.add_seq(nxt)
                m.share_prefix(nxt, src, n)
            live.append(nxt)
            nxt += 1
        same_state(o, c, live)


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_config_traces_match(name):
    """Every configuration's context build and decode step."""
    wl = config_workload(name, values=False)
    o = OracleBM(wl.num_blocks, wl.block_size, wl.free_order)
    c = pkv.BlockManager(wl.num_blocks, wl.block_size, wl.free_order)
    for op in wl.ops:
        if op[0] == "add":
            o.add_seq(op[1])
            c.add_seq(op[1])
        elif op[0] == "append":
            so, _ = o.append_slots([op[1]], op[2])
            sc, _ = c.append_slots([op[1]], op[2])
            assert np.array_equal(sc, np.asarray(so, dtype=np.int32))
        elif op[0] == "share_prefix":
            o.share_prefix(*op[1:])
            c.share_prefix(*op[1:])
        else:
            o.fork(*op[1:])
            c.fork(*op[1:])
    seqs = [int(s) for s in wl.decode_seqs]
    so, co = o.append_slots(seqs, 1)
    sc, cc = c.append_slots(seqs, 1)
    assert np.array_equal(sc, np.asarray(so, dtype=np.int32))
    assert np.array_equal(cc.reshape(-1, 2), np.asarray(co, dtype=np.int32).reshape(-1, 2))
    if name == "shared-prefix-cow":
        assert len(cc) == 48
    same_state(o, c, seqs)
    ct, cl = c.export(seqs, wl.max_blocks_per_seq)
    assert np.array_equal(cl, wl.seq_lens)


def same_tiers(o: OracleBM, c):
    assert c.num_free_host() == o.num_free_host()
    assert np.array_equal(c.host_free_list(), np.asarray(o.hfree, dtype=np.int32))
    for h in range(o.num_host_blocks):
        assert c.host_refcount(h) == o.href[h]
    for s in o.tables:
        assert c.is_swapped(s) == (s in o.swapped)


@settings(max_examples=80, deadline=None)
@given(st.data())
def test_random_traces_with_swaps_match(data):
    nb, nh = data.draw(st.integers(2, 40)), data.draw(st.integers(1, 40))
    B = data.draw(st.sampled_from([1, 2, 4, 8, 16]))
    rng = np.random.default_rng(data.draw(st.integers(0, 10**6)))
    perm, hperm = rng.permutation(nb), rng.permutation(nh)
    o = OracleBM(nb, B, perm, nh, hperm)
    c = pkv.BlockManager(nb, B, perm, nh, hperm)
    nxt = 0
    for _ in range(data.draw(st.integers(1, 50))):
        res = [s for s in o.tables if s not in o.swapped]
        swp = sorted(o.swapped)
        op = data.draw(st.sampled_from(["add", "append", "append", "fork", "free", "out",
                                        "out", "in", "in"]))
        if op == "add" or not o.tables:
            o.add_seq(nxt)
            c.add_seq(nxt)
            nxt += 1
            continue
        if op in ("append", "fork", "out") and not res or op == "in" and not swp:
            continue
        if op == "append":
            seqs, k = data.draw(st.lists(st.sampled_from(res), min_size=1, max_size=4)), \
                data.draw(st.integers(1, 7))
            f = lambda m: m.append_slots(seqs, k)  # noqa: E731
        elif op == "fork":
            p, child = data.draw(st.sampled_from(res)), nxt
            f = lambda m: m.fork(p, child)  # noqa: E731
            nxt += 1
        elif op == "free":
            s = data.draw(st.sampled_from(sorted(o.tables)))
            f = lambda m: m.free_seq(s)  # noqa: E731
        else:
            pool = res if op == "out" else swp
            seqs = data.draw(st.lists(st.sampled_from(pool), min_size=1, unique=True))
            f = (lambda m: m.swap_out(seqs)) if op == "out" else (lambda m: m.swap_in(seqs))
        try:
            ro, fo = f(o), False
        except OracleNoFree:
            fo = True
        try:
            rc, fc = f(c), False
        except pkv.NoFreeBlocks:
            fc = True
        assert fo == fc, op
        if not fo and op in ("out", "in"):
            assert np.array_equal(rc, np.asarray(ro, dtype=np.int32).reshape(-1, 2))
        res = [s for s in o.tables if s not in o.swapped]
        same_state(o, c, res)
        same_tiers(o, c)
