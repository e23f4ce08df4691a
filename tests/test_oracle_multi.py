"""Pins of the multi-token-query oracle (oracle.attention.attention_multi):
each query equals the pinned decode definition over the history cut at its own
position; the whole batch equals torch's scaled_dot_product_attention with the
causal mask offset by the history before the new tokens (an independent
library routine); P < 0 rows are zero; one query per sequence is decode."""
import numpy as np
import pytest

from oracle.attention import attention_decode, attention_multi, gather_history, to_f64

torch = pytest.importorskip("torch")


def make(seed, lens, nq, Hq=8, Hkv=2, D=16, B=4):
    rng = np.random.default_rng(seed)
    N = len(lens)
    maxb = max(-(-L // B) for L in lens) + 1
    nb = N * maxb + 3
    perm = rng.permutation(nb)
    tables = np.full((N, maxb), -1, np.int32)
    k = 0
    for s, L in enumerate(lens):
        for b in range(-(-L // B)):
            tables[s, b] = perm[k]; k += 1
    kp = rng.normal(0, 1, (nb, B, Hkv, D))
    vp = rng.normal(0, 1, (nb, B, Hkv, D))
    offs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = rng.normal(0, 1, (int(offs[-1]), Hq, D))
    return q, offs, kp, vp, tables, np.asarray(lens, np.int32)


def test_each_query_is_decode_over_its_prefix():
    q, offs, kp, vp, tables, lens = make(1, [9, 1, 23, 5], [3, 1, 7, 5])
    out = attention_multi(q, offs, kp, vp, tables, lens, 0.3)
    for s in range(len(lens)):
        n = offs[s + 1] - offs[s]
        for j in range(n):
            P = lens[s] - n + j
            ref = attention_decode(q[offs[s] + j][None], kp, vp, tables[s:s + 1],
                                   np.array([P + 1]), 0.3)[0]
            assert np.allclose(out[offs[s] + j], ref, rtol=0, atol=1e-14)


def test_matches_torch_sdpa_with_offset_causal_mask():
    q, offs, kp, vp, tables, lens = make(2, [16, 30, 7], [4, 11, 7], Hq=12, Hkv=4, D=8, B=8)
    out = attention_multi(q, offs, kp, vp, tables, lens, 0.5)
    for s in range(len(lens)):
        n, L = int(offs[s + 1] - offs[s]), int(lens[s])
        K, V = gather_history(kp, vp, tables[s], L)
        qt = torch.from_numpy(to_f64(q[offs[s]:offs[s + 1]])).permute(1, 0, 2)[None].contiguous()
        Kt = torch.from_numpy(to_f64(K)).permute(1, 0, 2)[None].contiguous()
        Vt = torch.from_numpy(to_f64(V)).permute(1, 0, 2)[None].contiguous()
        pos = np.arange(L)[None, :]
        qpos = (L - n + np.arange(n))[:, None]
        mask = torch.from_numpy(pos <= qpos)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, Kt, Vt, attn_mask=mask, scale=0.5, enable_gqa=True)[0].permute(1, 0, 2).numpy()
        assert np.allclose(out[offs[s]:offs[s + 1]], ref, rtol=1e-12, atol=1e-13)


def test_more_queries_than_history_gives_zero_rows():
    q, offs, kp, vp, tables, lens = make(3, [3, 5], [5, 2])
    out = attention_multi(q, offs, kp, vp, tables, lens, 1.0)
    assert not out[0].any() and not out[1].any()          # positions -2, -1
    assert out[2].any() and out[4].any()


def test_one_query_per_sequence_is_decode():
    q, offs, kp, vp, tables, lens = make(4, [1, 17, 40], [1, 1, 1])
    assert np.array_equal(attention_multi(q, offs, kp, vp, tables, lens, 0.2),
                          attention_decode(q, kp, vp, tables, lens, 0.2))


def _mutant(off_by_one=False, from_start=False):
    from oracle.attention import attend, _heads_of_group

    def multi(q, q_offsets, kp, vp, tables, lens, scale):
        q = to_f64(q)
        Hkv = kp.shape[2]
        out = np.zeros(q.shape)
        for s in range(len(q_offsets) - 1):
            n, L = int(q_offsets[s + 1] - q_offsets[s]), int(lens[s])
            K, V = gather_history(kp, vp, tables[s], L)
            for j in range(n):
                P = j if from_start else L - n + j
                hi = P if off_by_one else P + 1
                if hi <= 0:
                    continue
                for g in range(Hkv):
                    hs = list(_heads_of_group(q.shape[1], Hkv, g))
                    out[q_offsets[s] + j, hs] = attend(q[q_offsets[s] + j, hs], K[:hi, g],
                                                       V[:hi, g], scale)
        return out
    return multi


@pytest.mark.parametrize("kw", [{"off_by_one": True}, {"from_start": True}])
def test_planted_causal_mistakes_fail_the_decode_pin(kw):
    q, offs, kp, vp, tables, lens = make(5, [9, 23], [3, 7])
    out = _mutant(**kw)(q, offs, kp, vp, tables, lens, 0.3)
    ok = True
    for s in range(len(lens)):
        n = offs[s + 1] - offs[s]
        for j in range(n):
            P = lens[s] - n + j
            ref = attention_decode(q[offs[s] + j][None], kp, vp, tables[s:s + 1],
                                   np.array([P + 1]), 0.3)[0]
            ok &= np.allclose(out[offs[s] + j], ref, rtol=0, atol=1e-14)
    assert not ok
