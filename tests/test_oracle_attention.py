"""Pins of the oracle attention (no GPU): paging invariance, the block-wise
online form and the split-KV merge against the plain definition, closed-form
special cases, an independent library routine and a pure-Python brute force."""
import math

import numpy as np
import pytest
import torch

from oracle.attention import (attention_blockwise_online, attention_contiguous,
                              attention_decode, attention_split, to_f64)
from oracle.block_manager import BlockManager
from oracle.cache_ops import write
from oracle.replay import run_step
from tests.conftest import load_golden
from workloads import config_workload, independent_workload, shared_prefix_workload


def small_wl(dtype="bf16", lens=(1, 5, 16, 17, 40, 77), hq=8, hkv=2, d=64, B=16, seed=11,
             **kw):
    return independent_workload(list(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                block_size=B, dtype=dtype, seed=seed, **kw)


def contiguous_of(st):
    ks, vs = [], []
    for s in st.wl.decode_seqs:
        k, v = st.history(int(s))
        ks.append(k)
        vs.append(v)
    return ks, vs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B", [1, 4, 16, 32])
def test_paged_equals_contiguous_bitwise(dtype, B):
    st = run_step(small_wl(dtype=dtype, B=B))
    paged = st.attention()
    ks, vs = contiguous_of(st)
    cont = attention_contiguous(st.wl.q, ks, vs, st.wl.scale)
    assert np.array_equal(paged, cont)


def test_paged_equals_contiguous_shared_prefix_and_cow():
    wl = shared_prefix_workload(prefix_tokens=48, suffix_lens=[3, 16, 7, 1, 12, 30],
                                forking_parents=3, samples_per_fork=4, num_q_heads=8,
                                num_kv_heads=2, head_dim=32, block_size=16, dtype="bf16",
                                seed=5)
    st = run_step(wl)
    assert len(st.cow_pairs) == 3 * 3
    paged = st.attention()
    ks, vs = contiguous_of(st)
    assert np.array_equal(paged, attention_contiguous(wl.q, ks, vs, wl.scale))


def test_physical_permutation_does_not_change_result():
    a = run_step(small_wl(seed=3))
    wl2 = small_wl(seed=3)
    wl2.free_order = np.random.default_rng(99).permutation(wl2.num_blocks).astype(np.int32)
    b = run_step(wl2)
    assert not np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.attention(), b.attention())


@pytest.mark.parametrize("B", [1, 4, 16, 32])
def test_blockwise_online_equals_definition(B):
    st = run_step(small_wl(B=B, lens=(1, 2, 31, 33, 64, 100)))
    ref = st.attention()
    for i in range(st.wl.num_seqs):
        nb = -(-int(st.seq_lens[i]) // B)
        got = attention_blockwise_online(st.wl.q[i], st.k_pool, st.v_pool,
                                         st.block_tables[i][:nb], st.seq_lens[i], st.wl.scale)
        np.testing.assert_allclose(got, ref[i], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T", [16, 32, 48, 4096])
def test_split_merge_equals_definition(T):
    st = run_step(small_wl(lens=(1, 15, 16, 17, 200, 333)))
    ref = st.attention()
    got = attention_split(st.wl.q, st.k_pool, st.v_pool, st.block_tables, st.seq_lens,
                          st.wl.scale, T)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    if T >= int(st.seq_lens.max()):
        assert np.array_equal(got, ref)


def test_single_token_returns_its_value_exactly():
    st = run_step(small_wl(lens=(1, 1, 1)))
    out = st.attention()
    G = st.wl.num_q_heads // st.wl.num_kv_heads
    for i in range(3):
        for h in range(st.wl.num_q_heads):
            assert np.array_equal(out[i, h], to_f64(st.wl.new_v[i, h // G]))


def test_zero_scale_gives_mean_of_values():
    wl = small_wl(scale=0.0)
    st = run_step(wl)
    out = st.attention()
    ks, vs = contiguous_of(st)
    G = wl.num_q_heads // wl.num_kv_heads
    for i in range(wl.num_seqs):
        V = to_f64(vs[i])
        for h in range(wl.num_q_heads):
            np.testing.assert_allclose(out[i, h], V[:, h // G].mean(axis=0), rtol=1e-12,
                                       atol=1e-15)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(0)
    B, H, D, L = 4, 2, 8, 11
    bm = BlockManager(8, B)
    bm.add_seq(0)
    slots, _ = bm.append_slots([0], L)
    kp = np.zeros((8, B, H, D))
    vp = np.zeros((8, B, H, D))
    key = rng.standard_normal((H, D))
    V = rng.standard_normal((L, H, D))
    write(np.broadcast_to(key, (L, H, D)).copy(), V, slots, kp, vp)
    q = rng.standard_normal((1, 4, D))
    rows, lens = bm.export([0], 3)
    out = attention_decode(q, kp, vp, rows, lens, 0.7)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], V[:, h // 2].mean(axis=0), rtol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (8, 1), (12, 4)])
def test_matches_torch_sdpa_with_gqa(hq, hkv):
    """Library routine: torch's scaled_dot_product_attention (float64, CPU) on
    the contiguous history, with its grouped-query option (query head h reads
    KV head h // G)."""
    st = run_step(small_wl(hq=hq, hkv=hkv, d=32, lens=(3, 20, 50)))
    out = st.attention()
    ks, vs = contiguous_of(st)
    for i in range(st.wl.num_seqs):
        q = torch.from_numpy(to_f64(st.wl.q[i]))[:, None, :]           # [Hq, 1, D]
        K = torch.from_numpy(to_f64(ks[i])).permute(1, 0, 2).contiguous()  # [Hkv, L, D]
        V = torch.from_numpy(to_f64(vs[i])).permute(1, 0, 2).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None], K[None], V[None], scale=st.wl.scale, enable_gqa=True)[0, :, 0]
        np.testing.assert_allclose(out[i], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_pure_python_brute_force_tiny():
    """Scalar loops with math.exp, no numpy linear algebra."""
    st = run_step(small_wl(hq=4, hkv=2, d=8, lens=(1, 6, 9), B=4, dtype="f32"))
    out = st.attention()
    wl = st.wl
    G = wl.num_q_heads // wl.num_kv_heads
    for i in range(wl.num_seqs):
        L = int(st.seq_lens[i])
        for h in range(wl.num_q_heads):
            g = h // G
            rows = []
            for t in range(L):
                phys = int(st.block_tables[i][t // wl.block_size])
                off = t % wl.block_size
                k = [float(x) for x in st.k_pool[phys, off, g]]
                v = [float(x) for x in st.v_pool[phys, off, g]]
                z = wl.scale * sum(float(a) * b for a, b in zip(wl.q[i, h], k))
                rows.append((z, v))
            m = max(z for z, _ in rows)
            w = [math.exp(z - m) for z, _ in rows]
            tot = sum(w)
            exp = [sum(w[t] * rows[t][1][d] for t in range(L)) / tot for d in range(wl.head_dim)]
            np.testing.assert_allclose(out[i, h], exp, rtol=1e-12, atol=1e-14)


def test_selfcheck_paged_vs_standard_fp32():
    """The page's self-check: fp32 values, 16 blocks x 4 slots, 8 heads, D=32,
    10 tokens -> 3 blocks; standard softmax attention over the stacked K/V in
    float32 agrees with the paged result within 1e-5."""
    g = load_golden("selfcheck_kvm.json")
    rng = np.random.default_rng(7)
    H, D, B, n = g["num_heads"], g["head_dim"], g["block_size"], g["tokens"]
    bm = BlockManager(g["num_blocks"], B)
    bm.add_seq(0)
    kp = np.zeros((g["num_blocks"], B, H, D), np.float32)
    vp = np.zeros_like(kp)
    Ks, Vs = [], []
    for _ in range(n):
        k = rng.standard_normal((1, H, D)).astype(np.float32)
        v = rng.standard_normal((1, H, D)).astype(np.float32)
        slots, _ = bm.append_slots([0], 1)
        write(k, v, slots, kp, vp)
        Ks.append(k[0])
        Vs.append(v[0])
    assert len(bm.tables[0]) == g["blocks_used"]
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    rows, lens = bm.export([0], 3)
    paged = attention_decode(q, kp, vp, rows, lens, 1.0 / math.sqrt(D))[0]
    K = torch.from_numpy(np.stack(Ks))
    V = torch.from_numpy(np.stack(Vs))
    qt = torch.from_numpy(q[0])
    w = torch.softmax(torch.einsum("hd,shd->hs", qt, K) / math.sqrt(D), dim=-1)
    std = torch.einsum("hs,shd->hd", w, V).numpy()
    assert np.abs(paged - std).max() < g["max_abs_err_bound"]
    bm.free_seq(0)
    assert bm.num_free() == g["free_after_release"]


def test_tiny_config_structure_and_paging_invariance():
    wl = config_workload("tiny")
    st = run_step(wl)
    assert wl.num_blocks == 64
    assert [len([b for b in r if b >= 0]) for r in st.block_tables] == [1, 3, 7, 2]
    assert 64 - st.bm.num_free() == 13
    ks, vs = contiguous_of(st)
    assert np.array_equal(st.attention(), attention_contiguous(wl.q, ks, vs, wl.scale))
