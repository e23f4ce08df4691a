"""Oracle cache writes and block copies (bit copies).  Test infrastructure.

Pool layout ([KVM §19.2.3]): K and V pools are each
``[num_blocks, block_size, num_kv_heads, head_dim]``; token slot ``s`` is row
``s`` of the pool viewed as ``[num_blocks * block_size, num_kv_heads,
head_dim]`` ([SLOT §locate], token-slot equation).  Values are carried as their
stored bits (uint16 for bf16, float32 for fp32), so every copy here is exact.
"""
from __future__ import annotations

import numpy as np


def write(k, v, slot_mapping, k_pool, v_pool) -> None:
    """Scatter token i's K/V rows into slot ``slot_mapping[i]``; a negative slot
    means "skip".  In place.  Rejects dtype mismatches, out-of-range slots and
    repeated slots (whose result would depend on write order)."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if k.dtype != k_pool.dtype or v.dtype != v_pool.dtype:
        raise TypeError("token and pool dtypes differ")
    nb, B, H, D = k_pool.shape
    if k.shape != (slots.size, H, D) or v.shape != (slots.size, H, D):
        raise ValueError("k/v must be [T, num_kv_heads, head_dim]")
    live = slots >= 0
    if np.any(slots[live] >= nb * B):
        raise IndexError("slot out of range")
    if np.unique(slots[live]).size != int(live.sum()):
        raise ValueError("repeated slot")
    kf = k_pool.reshape(nb * B, H, D)
    vf = v_pool.reshape(nb * B, H, D)
    assert np.shares_memory(kf, k_pool) and np.shares_memory(vf, v_pool)
    # Slots are distinct (checked above), so the scatter order is irrelevant.
    kf[slots[live]] = k[live]
    vf[slots[live]] = v[live]


def copy_blocks(pairs, k_pool, v_pool) -> None:
    """For each (src, dst): the whole dst block (all slots, K and V) becomes a
    copy of the src block ([KVM §19.2.2] Fig. 19-8: "copy the original
    contents").  In place.  Rejects src == dst, repeated dst and a dst that is
    also some src (those would make the result order-dependent)."""
    pairs = [(int(a), int(b)) for a, b in pairs]
    srcs = [a for a, _ in pairs]
    dsts = [b for _, b in pairs]
    nb = k_pool.shape[0]
    for a, b in pairs:
        if not (0 <= a < nb and 0 <= b < nb):
            raise IndexError("block id out of range")
        if a == b:
            raise ValueError("src == dst")
    if len(set(dsts)) != len(dsts):
        raise ValueError("repeated dst")
    if set(dsts) & set(srcs):
        raise ValueError("a dst is also a src")
    for a, b in pairs:
        k_pool[b] = k_pool[a]
        v_pool[b] = v_pool[a]


def swap_blocks(pairs, src_pool, dst_pool) -> None:
    """For each (src, dst): block ``dst`` of ``dst_pool`` (every slot, stale
    ones included) becomes a copy of block ``src`` of ``src_pool``.  This is
    the data movement of a swap between the device pool and the host pool
    ([KVM §19.2.6]: the paused request's KV cache goes to CPU memory and comes
    back; [ENG §8.2]), one pool at a time: K, V, and for INT8 caches the scale
    pools viewed as [blocks][block_size][heads].  In place.  Rejects pools of
    different block shape or dtype, ids out of range and a repeated dst."""
    pairs = [(int(a), int(b)) for a, b in pairs]
    if src_pool.shape[1:] != dst_pool.shape[1:] or src_pool.dtype != dst_pool.dtype:
        raise ValueError("pools differ in block shape or dtype")
    ns, nd = src_pool.shape[0], dst_pool.shape[0]
    for a, b in pairs:
        if not (0 <= a < ns and 0 <= b < nd):
            raise IndexError("block id out of range")
    dsts = [b for _, b in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("repeated dst")
    for a, b in pairs:
        dst_pool[b] = src_pool[a]
