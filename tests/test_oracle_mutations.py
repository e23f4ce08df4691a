"""Planted mistakes: each plausible bug in an oracle-shaped function must fail at
least one of the independent pins (library routine, pure-Python brute force,
closed forms, the pages' worked examples).  Mistakes are planted in copies of
the oracle on the CPU; the oracle itself is untouched."""
import math

import numpy as np
import pytest
import torch

from oracle.attention import gather_history, to_f64
from oracle.block_manager import BlockManager
from oracle.replay import run_step
from tests.conftest import load_golden
from workloads import independent_workload


# -- attention mutants ------------------------------------------------------

def make_attn(gmap="div", drop_last=False, use_scale=True, score_from_v=False,
              reverse_offset=False, neg_exp=False):
    def attn(q, k_pool, v_pool, tables, lens, scale):
        N, Hq, D = q.shape
        B, Hkv = k_pool.shape[1], k_pool.shape[2]
        G = Hq // Hkv
        out = np.zeros((N, Hq, D))
        for s in range(N):
            L = int(lens[s]) - (1 if drop_last and lens[s] > 1 else 0)
            t = np.arange(L)
            off = (B - 1 - t % B) if reverse_offset else t % B
            phys = np.asarray(tables[s])[t // B]
            K, V = to_f64(k_pool[phys, off]), to_f64(v_pool[phys, off])
            for h in range(Hq):
                g = h // G if gmap == "div" else h % Hkv
                kk = V[:, g] if score_from_v else K[:, g]
                z = (scale if use_scale else 1.0) * (kk @ to_f64(q[s, h]))
                m = z.max()
                p = np.exp(m - z) if neg_exp else np.exp(z - m)
                out[s, h] = p @ V[:, g] / p.sum()
        return out
    return attn


def attention_pins_pass(attn):
    """Independent pins; returns True iff all hold for ``attn``."""
    wl = independent_workload([1, 5, 20, 37], num_q_heads=8, num_kv_heads=2, head_dim=16,
                              block_size=4, dtype="f32", seed=21)
    st = run_step(wl)
    out = attn(wl.q, st.k_pool, st.v_pool, st.block_tables, st.seq_lens, wl.scale)
    G = wl.num_q_heads // wl.num_kv_heads
    for i in range(wl.num_seqs):
        K, V = st.history(int(wl.decode_seqs[i]))
        qt = torch.from_numpy(to_f64(wl.q[i]))[None, :, None, :]
        Kt = torch.from_numpy(to_f64(K)).permute(1, 0, 2)[None].contiguous()
        Vt = torch.from_numpy(to_f64(V)).permute(1, 0, 2)[None].contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, Kt, Vt, scale=wl.scale, enable_gqa=True)[0, :, 0].numpy()
        if not np.allclose(out[i], ref, rtol=1e-10, atol=1e-12):
            return False
        if wl.seq_lens[i] == 1:
            for h in range(wl.num_q_heads):
                if not np.array_equal(out[i, h], to_f64(V[0, h // G])):
                    return False
    return True


ATTN_MUTANTS = {
    "gqa head map h % H_kv": dict(gmap="mod"),
    "last token dropped": dict(drop_last=True),
    "scale missing": dict(use_scale=False),
    "scores from V (operand mix-up)": dict(score_from_v=True),
    "offset reversed inside a block": dict(reverse_offset=True),
    "exp sign flipped": dict(neg_exp=True),
}


def test_reference_shape_passes_pins():
    assert attention_pins_pass(make_attn())


@pytest.mark.parametrize("name", list(ATTN_MUTANTS))
def test_attention_mutant_caught(name):
    assert not attention_pins_pass(make_attn(**ATTN_MUTANTS[name])), name


# -- block-manager mutants ----------------------------------------------------

class PopFront(BlockManager):
    def _allocate(self):
        if not self.free:
            raise RuntimeError
        b = self.free.pop(0)
        self.ref[b] = 1
        return b


class CowNoDecrement(BlockManager):
    def _release(self, b):
        import inspect
        if inspect.stack()[1].function == "_append_one":
            return
        super()._release(b)


class ForkNoIncrement(BlockManager):
    def fork(self, parent, child):
        self.tables[child] = list(self.tables[parent])
        self.filled[child] = self.filled[parent]


class SlotMinusOffset(BlockManager):
    def _append_one(self, seq, cow_out):
        s = super()._append_one(seq, cow_out)
        off = s % self.block_size
        return s - 2 * off


def block_manager_pins_pass(cls):
    try:
        g = load_golden("slot_example_b4.json")
        pops = g["block_table"]
        bm = cls(8, 4, [b for b in range(8) if b not in pops] + pops[::-1])
        bm.add_seq(0)
        slots, _ = bm.append_slots([0], 10)
        if slots[2] != 30 or bm.tables[0] != pops:
            return False
        r = load_golden("refcounts.json")
        bm = cls(16, 4)
        bm.add_seq("A1")
        bm.append_slots(["A1"], 6)
        bm.fork("A1", "A2")
        if bm.ref[bm.tables["A1"][1]] != r["fork_count"]:
            return False
        _, cow = bm.append_slots(["A1"], 1)
        old = cow[0][0]
        if bm.ref[old] != 1:
            return False
        bm.check()
        return True
    except (AssertionError, RuntimeError, IndexError, KeyError):
        return False


def test_reference_manager_passes_pins():
    assert block_manager_pins_pass(BlockManager)


@pytest.mark.parametrize("cls", [PopFront, CowNoDecrement, ForkNoIncrement, SlotMinusOffset],
                         ids=lambda c: c.__name__)
def test_block_manager_mutant_caught(cls):
    assert not block_manager_pins_pass(cls)


def test_brute_force_catches_gqa_mutant_independently():
    """The pure-Python loop (no library) separates h // G from h % H_kv."""
    wl = independent_workload([7], num_q_heads=4, num_kv_heads=2, head_dim=4, block_size=4,
                              dtype="f32", seed=2)
    st = run_step(wl)
    K, V = gather_history(st.k_pool, st.v_pool, st.block_tables[0], st.seq_lens[0])
    good = make_attn()(wl.q, st.k_pool, st.v_pool, st.block_tables, st.seq_lens, wl.scale)
    bad = make_attn(gmap="mod")(wl.q, st.k_pool, st.v_pool, st.block_tables, st.seq_lens,
                                wl.scale)
    h = 1                                    # G = 2: h // G = 0, h % H_kv = 1
    z = [wl.scale * sum(float(a) * float(b) for a, b in zip(wl.q[0, h], K[t, 0]))
         for t in range(7)]
    m = max(z)
    w = [math.exp(x - m) for x in z]
    ref = [sum(w[t] * float(V[t, 0, d]) for t in range(7)) / sum(w) for d in range(4)]
    assert np.allclose(good[0, h], ref, rtol=1e-12)
    assert not np.allclose(bad[0, h], ref, rtol=1e-6)
