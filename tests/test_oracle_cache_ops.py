"""Pins of the oracle write / block copy and of the workload byte accounting
(no GPU)."""
import numpy as np
import pytest

from oracle.block_manager import BlockManager
from oracle.cache_ops import copy_blocks, write
from oracle.replay import run_step
from tests.conftest import load_golden
from workloads import (CONFIGS, attention_kv_bytes, config_workload, kv_cache_bytes)


def test_write_places_rows_at_slots_worked_example():
    """10 tokens at block size 4 on P7, P1, P5: token t lands at block
    table[t//4], offset t%4 -- its flattened slot row holds exactly its K/V."""
    g = load_golden("slot_example_b4.json")
    B, H, D = 4, 2, 3
    pops = g["block_table"]
    bm = BlockManager(8, B, [b for b in range(8) if b not in pops] + pops[::-1])
    bm.add_seq(0)
    slots, _ = bm.append_slots([0], 10)
    k = np.arange(10 * H * D, dtype=np.float32).reshape(10, H, D)
    v = -k
    kp = np.zeros((8, B, H, D), np.float32)
    vp = np.zeros_like(kp)
    write(k, v, slots, kp, vp)
    assert np.array_equal(kp[7, 2], k[2])              # position 2 -> slot 30
    assert np.array_equal(kp.reshape(32, H, D)[30], k[2])
    assert np.array_equal(kp[5, :2], k[8:10]) and not kp[5, 2:].any()
    assert np.array_equal(vp[1], v[4:8])
    touched = {7, 1, 5}
    for b in range(8):
        if b not in touched:
            assert not kp[b].any() and not vp[b].any()


def test_write_skips_negative_and_rejects_bad_slots():
    kp = np.zeros((2, 4, 1, 2), np.uint16)
    vp = np.zeros_like(kp)
    k = np.array([[[1, 2]], [[3, 4]]], np.uint16)
    write(k, k, [-1, 5], kp, vp)
    assert kp.reshape(8, 1, 2)[5].tolist() == [[3, 4]] and kp.sum() == 7
    with pytest.raises(ValueError):
        write(k, k, [3, 3], kp, vp)
    with pytest.raises(IndexError):
        write(k, k, [0, 8], kp, vp)
    with pytest.raises(TypeError):
        write(k.astype(np.float32), k, [0, 1], kp, vp)


def test_copy_blocks_copies_whole_block_including_stale_slots():
    rng = np.random.default_rng(1)
    kp = rng.integers(0, 65535, (6, 4, 2, 8)).astype(np.uint16)
    vp = rng.integers(0, 65535, (6, 4, 2, 8)).astype(np.uint16)
    k0, v0 = kp.copy(), vp.copy()
    copy_blocks([(1, 4), (2, 5)], kp, vp)
    assert np.array_equal(kp[4], k0[1]) and np.array_equal(vp[5], v0[2])
    for b in (0, 1, 2, 3):
        assert np.array_equal(kp[b], k0[b]) and np.array_equal(vp[b], v0[b])
    with pytest.raises(ValueError):
        copy_blocks([(1, 1)], kp, vp)
    with pytest.raises(ValueError):
        copy_blocks([(1, 4), (2, 4)], kp, vp)
    with pytest.raises(ValueError):
        copy_blocks([(1, 4), (4, 5)], kp, vp)


def test_cow_then_write_keeps_sharers_intact():
    """Fig. 19-8: after A1's copy-on-write append, A2 still sees the original
    block; A1 sees the copy plus its new token."""
    B, H, D = 4, 1, 2
    bm = BlockManager(8, B)
    kp = np.zeros((8, B, H, D), np.float32)
    vp = np.zeros_like(kp)
    bm.add_seq(0)
    s, _ = bm.append_slots([0], 6)
    ctx = np.arange(6 * H * D, dtype=np.float32).reshape(6, H, D) + 1
    write(ctx, ctx, s, kp, vp)
    bm.fork(0, 1)
    s, cow = bm.append_slots([0], 1)
    copy_blocks(cow, kp, vp)
    new = np.full((1, H, D), 99, np.float32)
    write(new, new, s, kp, vp)
    old, cpy = cow[0]
    assert np.array_equal(kp[cpy, :2], kp[old, :2])
    assert kp[cpy, 2, 0, 0] == 99 and kp[old, 2, 0, 0] == 0
    assert bm.tables[1][1] == old and bm.tables[0][1] == cpy


@pytest.mark.parametrize("case", load_golden("kv_bytes.json")["cases"], ids=lambda c: c["what"])
def test_kv_byte_formula_closed_forms(case):
    b = kv_cache_bytes(case["layers"], case["seqs"], case["tokens"], case["kv_heads"],
                       case["head_dim"], case["elem_bytes"])
    if "bytes" in case:
        assert b == case["bytes"]
    for unit, sh in (("gib", 30), ("mib", 20), ("kib", 10)):
        if unit in case:
            assert b == case[unit] * (1 << sh)


def test_byte_accounting_small_facts():
    g = load_golden("kv_bytes.json")
    per_tok = g["per_token_kib"] * 1024
    assert 10 * per_tok == g["ten_tokens_mib"] * (1 << 20)
    assert 12 * per_tok == g["twelve_positions_mib"] * (1 << 20)
    assert g["table_entries"] * np.dtype(np.int32).itemsize == g["table_bytes"]
    q = g["gqa"]
    full = kv_cache_bytes(1, 1, 100, q["q_heads"], 128, 2)
    gqa = kv_cache_bytes(1, 1, 100, q["kv_heads"], 128, 2)
    assert gqa / full == q["ratio"]
    # variable-length form: sum over sequences of the per-sequence formula
    lens = [3, 10, 7]
    assert attention_kv_bytes(lens, 8, 128, 2) == sum(kv_cache_bytes(1, 1, L, 8, 128, 2)
                                                     for L in lens)


def test_shared_prefix_config_structure():
    """176 sequences after the fork; prefix blocks (128) referenced by all of
    them; one CoW pair per sharer but the last of each forked family (48)."""
    wl = config_workload("shared-prefix-cow")
    c = CONFIGS["shared-prefix-cow"]
    assert wl.num_seqs == 128 + 16 * 3
    st = run_step(wl, keep_values=False)
    assert len(st.cow_pairs) == 48
    prefix = st.block_tables[0][:128]
    assert all(np.array_equal(st.block_tables[i][:128], prefix) for i in range(wl.num_seqs))
    assert all(st.bm.ref[int(b)] == 176 for b in prefix)
    assert np.all(st.seq_lens[:128] >= c.prefix_tokens + 2)
    assert np.all(st.seq_lens[:128] <= c.prefix_tokens + 513)
    st.bm.check()
