"""Oracle decode attention in float64.  Test infrastructure.

Definition ([KVX §01], new-token attention equation; [KVM §19.2.3]): the query
of sequence s, head h attends every cached position t < L_s of its sequence:

    z_t = scale * <q[s,h], K_s[t]>,  out[s,h] = sum_t softmax(z)_t * V_s[t]

where K_s[t] / V_s[t] are read through the block table: position t lives in
physical block table[floor(t/B)] at offset t mod B ([SLOT §locate]).  Grouped
query attention ([KVX §02] GQA ratio, [KVX §03] table): query heads are split
into H_kv contiguous groups of G = H_q / H_kv heads and group g reads KV head g,
i.e. g = h // G (a reading; the pages say only "grouped").  An empty history
gives a zero output (a reading; the pages are silent).

Functions:
  attention_decode           the plain definition above (gather, then softmax)
  attention_contiguous       the same over K/V stacked in token order, no paging
  attention_blockwise_online block by block: each block's own (max, sum,
                             weighted sum) folded into a running state, the
                             online-softmax form of [KVM §19.2.3], Fig. 19-5
  attention_split            split-KV: per-partition (max, sum, weighted sum)
                             merged by log-sum-exp rescaling
  attention_multi            several new query tokens per sequence (a prefill
                             chunk or tokens to verify), each attending the
                             history up to and including its own position
"""
from __future__ import annotations

import numpy as np


def to_f64(a: np.ndarray) -> np.ndarray:
    """Stored values -> float64, exactly (uint16 holds bfloat16 bits)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gather_history(k_pool, v_pool, table, length):
    """K/V rows of positions 0..length-1, in token order: position t is in
    block table[t // B] at offset t % B ([SLOT §locate])."""
    B = k_pool.shape[1]
    t = np.arange(int(length))
    phys = np.asarray(table, dtype=np.int64)[t // B]
    off = t % B
    return k_pool[phys, off], v_pool[phys, off]          # [L, H_kv, D]


def attend(q_rows, K, V, scale):
    """softmax(scale * q K^T) V for a few query rows sharing one K/V history.
    q_rows [R, D], K/V [L, D] (float64) -> [R, D]."""
    R, D = q_rows.shape
    if K.shape[0] == 0:
        return np.zeros((R, D))
    z = scale * (q_rows @ K.T)                     # [R, L]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def _heads_of_group(num_q_heads, num_kv_heads, g):
    G = num_q_heads // num_kv_heads
    return range(g * G, (g + 1) * G)


def attention_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, seqs=None):
    """Plain definition over the paged pools.  q [N, H_q, D] stored values;
    pools [nb, B, H_kv, D]; block_tables rows of physical ids.  Returns float64
    [N, H_q, D] (rows outside ``seqs`` are left at zero)."""
    N, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    out = np.zeros((N, Hq, D))
    for s in (range(N) if seqs is None else seqs):
        K, V = gather_history(k_pool, v_pool, block_tables[s], seq_lens[s])
        K, V = to_f64(K), to_f64(V)
        for g in range(Hkv):
            hs = list(_heads_of_group(Hq, Hkv, g))
            out[s, hs] = attend(to_f64(q[s, hs]), K[:, g], V[:, g], scale)
    return out


def attention_contiguous(q, k_seqs, v_seqs, scale):
    """The same math over per-sequence K/V arrays [L_s, H_kv, D] already in
    token order ([KVM §19.2.3] self-check: standard attention over the stacked
    history)."""
    N, Hq, D = q.shape
    out = np.zeros((N, Hq, D))
    for s in range(N):
        K, V = to_f64(k_seqs[s]), to_f64(v_seqs[s])
        Hkv = K.shape[1]
        for g in range(Hkv):
            hs = list(_heads_of_group(Hq, Hkv, g))
            out[s, hs] = attend(to_f64(q[s, hs]), K[:, g], V[:, g], scale)
    return out


def attention_blockwise_online(q_s, k_pool, v_pool, table, length, scale):
    """One sequence, one physical block at a time (the way [KVM §19.2.3] and
    Fig. 19-5 walk a request): the filled slots of each block give that
    block's own state (``partition_state``), and a running state absorbs it by
    ``fold_states``, so no score row longer than a block is ever held.  The
    result is the running state's weighted sum over its sum.
    q_s [H_q, D] -> [H_q, D] float64."""
    Hq, D = q_s.shape
    B, Hkv = k_pool.shape[1], k_pool.shape[2]
    L = int(length)
    out = np.zeros((Hq, D))
    if L == 0:
        return out
    qf = to_f64(q_s)
    nblk = -(-L // B)
    for g in range(Hkv):
        hs = list(_heads_of_group(Hq, Hkv, g))
        state = None
        for j in range(nblk):
            filled = min(B, L - j * B)          # slots of block j inside the history
            blk = int(table[j])
            piece = partition_state(qf[hs], to_f64(k_pool[blk, :filled, g]),
                                    to_f64(v_pool[blk, :filled, g]), scale)
            state = piece if state is None else fold_states(state, piece)
        m, l, acc = state
        out[hs] = acc / l[:, None]
    return out


def fold_states(a, b):
    """Two (max, sum, weighted sum) states of disjoint position sets -> the
    state of their union: both are rescaled to the larger max, exp(m - M)."""
    M = np.maximum(a[0], b[0])
    wa, wb = np.exp(a[0] - M), np.exp(b[0] - M)
    return M, wa * a[1] + wb * b[1], wa[:, None] * a[2] + wb[:, None] * b[2]


def partition_state(q_rows, K, V, scale):
    """(m, l, acc) of one partition: m = max score, l = sum exp(score - m),
    acc = sum exp(score - m) V.  q_rows [R, D], K/V [n, D] float64, n >= 1."""
    z = scale * (q_rows @ K.T)
    m = z.max(axis=1)
    p = np.exp(z - m[:, None])
    return m, p.sum(axis=1), p @ V


def merge_partitions(states):
    """Combine partition states by rescaling each to the common maximum:
    M = max_p m_p, w_p = exp(m_p - M), out = sum_p w_p acc_p / sum_p w_p l_p
    (the running-rescale rule of [KVM §19.2.3] applied across partitions)."""
    ms = np.stack([s[0] for s in states])          # [P, R]
    M = ms.max(axis=0)
    w = np.exp(ms - M)
    num = sum(w[i][:, None] * states[i][2] for i in range(len(states)))
    den = sum(w[i] * states[i][1] for i in range(len(states)))
    return num / den[:, None]


def attention_split(q, k_pool, v_pool, block_tables, seq_lens, scale, partition_tokens,
                    seqs=None):
    """Split-KV: sequence s is cut into partitions of ``partition_tokens``
    positions [p*T, min((p+1)*T, L_s)); each yields (m, l, acc); the partition
    states are merged as in ``merge_partitions``."""
    N, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    T = int(partition_tokens)
    out = np.zeros((N, Hq, D))
    for s in (range(N) if seqs is None else seqs):
        L = int(seq_lens[s])
        if L == 0:
            continue
        K, V = gather_history(k_pool, v_pool, block_tables[s], L)
        K, V = to_f64(K), to_f64(V)
        for g in range(Hkv):
            hs = list(_heads_of_group(Hq, Hkv, g))
            qr = to_f64(q[s, hs])
            states = [partition_state(qr, K[a:a + T, g], V[a:a + T, g], scale)
                      for a in range(0, L, T)]
            out[s, hs] = merge_partitions(states)
    return out


def attention_multi(q, q_offsets, k_pool, v_pool, block_tables, seq_lens, scale):
    """Multi-token queries.  Sequence s owns query rows q_offsets[s] ..
    q_offsets[s+1]-1: its n_s newest tokens, already in the cache, so history
    length L_s counts them.  Query j of s sits at position P = L_s - n_s + j
    and attends positions 0..P, the causal rule of [KVX §01] (a token sees the
    history up to itself) applied to each new token; P < 0 (more queries than
    history) attends nothing and gives zeros.  GQA mapping as for decode.
    q [total_q, H_q, D] -> out [total_q, H_q, D] (float64)."""
    q = to_f64(q)
    total, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    G = Hq // Hkv
    out = np.zeros((total, Hq, D))
    offs = np.asarray(q_offsets, dtype=np.int64)
    for s in range(offs.size - 1):
        n = int(offs[s + 1] - offs[s])
        if n == 0:
            continue
        L = int(seq_lens[s])
        K, V = gather_history(k_pool, v_pool, block_tables[s], L)
        K, V = to_f64(K), to_f64(V)
        for j in range(n):
            P = L - n + j
            if P < 0:
                continue
            for g in range(Hkv):
                hs = list(_heads_of_group(Hq, Hkv, g))
                out[offs[s] + j, hs] = attend(q[offs[s] + j, hs], K[:P + 1, g], V[:P + 1, g], scale)
    return out
