"""The library's pkv_prefix_groups against the oracle's grouping rule
(oracle/shared.py) on the configurations' decode tables and on random
tables, and host-side validation of pkv_attention_decode_shared (no GPU)."""
import ctypes

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.shared import prefix_groups as oracle_groups
from tests.test_oracle_shared import groups_of
from workloads import CONFIG_ORDER, config_workload, shared_prefix_workload

pkv = pytest.importorskip("paged_attention_slot_amd")
from paged_attention_slot_amd import _lib, ops  # noqa: E402
from paged_attention_slot_amd._lib import PkvGeom  # noqa: E402


def same(tables, lens, B):
    s0, p0 = oracle_groups(tables, lens, B)
    s1, p1, mg, mp, ms = ops.prefix_groups(tables, lens, B)
    assert np.array_equal(s0, s1) and np.array_equal(p0, p1)
    pre = np.repeat(np.where(np.diff(s0) >= 2, p0, 0), np.diff(s0))   # each sequence's prefix
    assert ms == (int(np.max(lens - np.minimum(pre, lens))) if lens.size else 0)
    assert mg == (int(np.diff(s0).max()) if lens.size else 0)
    assert mp == (int(p0.max()) if p0.size else 0)


@pytest.mark.parametrize("name", [c for c in CONFIG_ORDER if c != "llama3.1-70b-longctx"])
def test_configs(name):
    wl = config_workload(name, values=False)
    T, _ = groups_of(wl)
    same(T.block_tables, T.seq_lens, wl.block_size)


def test_partial_prefix_family():
    wl = shared_prefix_workload(prefix_tokens=40, suffix_lens=[3, 9, 1, 20, 33], forking_parents=2,
                                samples_per_fork=3, num_q_heads=4, num_kv_heads=2, head_dim=8,
                                block_size=16, dtype="f32", seed=3, values=False)
    wl.num_blocks = 96
    wl.free_order = np.random.default_rng(1).permutation(96).astype(np.int32)
    T, _ = groups_of(wl)
    same(T.block_tables, T.seq_lens, wl.block_size)


@settings(max_examples=120, deadline=None)
@given(st.data())
def test_random_tables(data):
    B = data.draw(st.sampled_from([1, 2, 8, 16]))
    n = data.draw(st.integers(0, 10))
    mb = data.draw(st.integers(1, 6))
    stems = [data.draw(st.lists(st.integers(0, 9), min_size=0, max_size=mb)) for _ in range(2)]
    tables = np.full((n, mb), -1, np.int32)
    lens = np.zeros(n, np.int32)
    for s in range(n):
        stem = stems[data.draw(st.integers(0, 1))]
        row = (stem + data.draw(st.lists(st.integers(0, 9), max_size=mb)))[:mb]
        tables[s, :len(row)] = row
        lens[s] = data.draw(st.integers(0, len(row) * B))
    same(tables, lens, B)


def test_shared_attention_validates_on_the_host():
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)
    g = PkvGeom(16, 16, 2, 128, _lib.PKV_BF16)

    def call(geo=g, ng=1, mg=4, mp=32, N=4, ws=x, wsb=1 << 30, scale=0.1, q=x):
        return lib.pkv_attention_decode_shared(q, x, x, x, 8, x, x, x, ng, mg, mp, 0, scale, x, N,
                                               4, 128, ws, wsb, ctypes.byref(geo), None)
    assert call(geo=PkvGeom(16, 16, 2, 128, _lib.PKV_F32)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(geo=PkvGeom(16, 4, 2, 128, _lib.PKV_BF16)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(geo=PkvGeom(16, 16, 2, 96, _lib.PKV_BF16)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(ng=0) == _lib.PKV_ERR_INVALID_ARG            # groups must cover the batch
    assert call(mg=-1) == _lib.PKV_ERR_INVALID_ARG
    assert call(scale=float("inf")) == _lib.PKV_ERR_INVALID_ARG
    assert call(ws=None) == _lib.PKV_ERR_INVALID_ARG and "workspace" in \
        lib.pkv_last_error().decode()
    assert call(wsb=16) == _lib.PKV_ERR_INVALID_ARG
    assert call(q=ctypes.c_void_p(0x1004)) == _lib.PKV_ERR_INVALID_ARG
    assert call(N=0, ng=0) == _lib.PKV_OK                     # empty batch: nothing enqueued
    need = lib.pkv_attention_shared_workspace_bytes(4, 4, 1, 4, 32, 0, 128, ctypes.byref(g))
    assert 0 < need < (1 << 30)
    n = ctypes.c_int32()
    assert lib.pkv_prefix_groups(None, 2, 4, None, 16, None, None, None, None, None, None) == \
        _lib.PKV_ERR_INVALID_ARG
    out = (ctypes.c_int32 * 8)()
    assert lib.pkv_prefix_groups(None, 0, 0, None, 16, out, out, ctypes.byref(n), out, out,
                                 out) == _lib.PKV_OK and n.value == 0
