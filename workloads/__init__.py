"""Seeded synthetic workloads for the paged decode hot path.

This module only *describes and draws inputs*.  It holds none of the method's
arithmetic: no slot mapping, no block allocation, no copy-on-write decision and
no attention.  Both the HIP path (through ``bench.py`` and the GPU tests) and
the CPU oracle (through the tests) consume the same ``Workload`` object; each
side then builds its own block tables from the operation trace with its own
block manager.

Pages cited (titles as they appear on each page):

* [KVM]  "19.2 KV Cache 系统化管理" -- book chapter (LLM full-stack book), sections
  19.2.1-19.2.6 and figures 19-3..19-8.
* [KVX]  "KV Cache：长上下文为什么吃显存，PagedAttention 怎么救" -- explainer,
  numbered sections 00-07.
* [SLOT] "推理与 KV Cache 02:分页、共享与回收如何协作" -- blog post; sections
  "从一个位置找到缓存块" (locate), "按整块分配,会多占多少空间" (whole-block),
  "请求结束后,缓存会立刻消失吗" (release).
* [PFX]  "学习大模型推理的显存优化：PagedAttention 与前缀缓存" -- blog post; sections
  "PagedAttention 原理" (principle), "前缀缓存" (prefix).
* [ENG]  the PagedAttention engineering article served under the page title
  "企业官网建设流程全解析"; numbered sections 1.1-8.3.

Value recipe (every configuration): q, context K/V and new-token K/V are drawn
i.i.d. N(0, 1) in float32 and, for bf16 configurations, rounded to bfloat16
with round-to-nearest-even.  bf16 arrays are carried as ``uint16`` bit
patterns.  Each array has its own child of ``numpy.random.SeedSequence(seed)``
(spawn order: lengths, suffixes, permutation, q, context K, context V, new K,
new V); large arrays are drawn in fixed 4 Mi-value chunks, each chunk with its
own grandchild seed, so the values do not depend on the number of threads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_CHUNK = 1 << 22

# Spawn slots of the per-workload SeedSequence (the draw order).
_S_LENS, _S_SUFFIX, _S_PERM, _S_Q, _S_CTXK, _S_CTXV, _S_NEWK, _S_NEWV = range(8)


# ----------------------------------------------------------------------------
# KV byte accounting (used for throughput figures; pinned in the tests against
# the pages' closed forms).
# ----------------------------------------------------------------------------

def kv_cache_bytes(layers: int, seqs: int, tokens: int, kv_heads: int,
                   head_dim: int, elem_bytes: float) -> float:
    """Logical KV-cache size: 2 (K and V) x layers x sequences x tokens x
    KV heads x head dim x bytes per element ([KVX §02] memory formula;
    [KVM §19.2.1] formula with the KV width written as heads x head dim)."""
    return 2 * layers * seqs * tokens * kv_heads * head_dim * elem_bytes


def attention_kv_bytes(seq_lens, kv_heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    """Bytes of history K and V one decode step must read: every cached token of
    every sequence, once, for K and for V (variable-length form of the memory
    formula, [KVX §02]; paging does not reduce the logical reads, [KVX §04])."""
    return int(np.sum(np.asarray(seq_lens, dtype=np.int64))) * 2 * kv_heads * head_dim * elem_bytes


def attention_io_bytes(seq_lens, num_q_heads: int, kv_heads: int, head_dim: int,
                       elem_bytes: int, block_size: int) -> int:
    """Algorithmic bytes of one decode-attention launch: K/V history, the query
    and output rows, the used block-table entries and the length vector."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    n = lens.size
    kv = attention_kv_bytes(lens, kv_heads, head_dim, elem_bytes)
    qo = 2 * n * num_q_heads * head_dim * elem_bytes
    tables = 4 * int(np.sum((lens + block_size - 1) // block_size))
    return kv + qo + tables + 4 * n


def write_bytes(num_tokens: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes moved by a slot-scatter append of ``num_tokens`` tokens: K and V
    rows read and written once, plus the int32 slot list."""
    row = kv_heads * head_dim * elem_bytes
    return 2 * 2 * num_tokens * row + 4 * num_tokens


def copy_bytes(num_pairs: int, block_size: int, kv_heads: int, head_dim: int,
               elem_bytes: int) -> int:
    """Bytes moved by a whole-block copy of ``num_pairs`` (src, dst) pairs for K
    and V (read once, written once)."""
    blk = block_size * kv_heads * head_dim * elem_bytes
    return 2 * 2 * num_pairs * blk + 8 * num_pairs


# ----------------------------------------------------------------------------
# Configurations
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f32" or "bf16"
    num_seqs: int = 0               # independent sequences (not shared-prefix)
    fixed_lens: tuple = ()          # final lengths (after the decode append)
    len_range: tuple = ()           # (lo, hi) inclusive, final lengths
    pool_blocks: int = 0            # fixed pool size; 0 = need + 10 % slack
    partition_tokens: int = 0       # split-KV partition; 0 = library heuristic
    # shared-prefix + copy-on-write family
    prefix_tokens: int = 0
    base_seqs: int = 0
    suffix_range: tuple = ()
    forking_parents: int = 0
    samples_per_fork: int = 0       # parent + children

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


CONFIGS = {
    "tiny": Config(name="tiny", seed=1, num_q_heads=8, num_kv_heads=2, head_dim=64,
                   block_size=16, dtype="f32", num_seqs=4, fixed_lens=(10, 35, 100, 17),
                   pool_blocks=64),
    "qwen3-0.6b-layer": Config(name="qwen3-0.6b-layer", seed=2, num_q_heads=16,
                               num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                               num_seqs=64, len_range=(128, 4096)),
    "llama3-8b-layer": Config(name="llama3-8b-layer", seed=3, num_q_heads=32,
                              num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                              num_seqs=256, len_range=(512, 8192)),
    "shared-prefix-cow": Config(name="shared-prefix-cow", seed=4, num_q_heads=32,
                                num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                                prefix_tokens=2048, base_seqs=128, suffix_range=(1, 512),
                                forking_parents=16, samples_per_fork=4),
    "llama3.1-70b-longctx": Config(name="llama3.1-70b-longctx", seed=5, num_q_heads=64,
                                   num_kv_heads=8, head_dim=128, block_size=32,
                                   dtype="bf16", num_seqs=4, fixed_lens=(131072,) * 4,
                                   partition_tokens=512),
}
CONFIG_ORDER = ["tiny", "qwen3-0.6b-layer", "llama3-8b-layer", "shared-prefix-cow",
                "llama3.1-70b-longctx"]


# ----------------------------------------------------------------------------
# Seeded draws
# ----------------------------------------------------------------------------

def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_array(seed_seq: np.random.SeedSequence, shape, dtype: str) -> np.ndarray:
    """i.i.d. N(0,1) float32 draws, chunked for threading; bf16 -> uint16 bits."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    nch = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = seed_seq.spawn(nch)

    def work(k):
        lo = k * _CHUNK
        hi = min(n, lo + _CHUNK)
        if hi <= lo:
            return
        g = np.random.Generator(np.random.PCG64(kids[k]))
        f = g.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = f if dtype == "f32" else round_to_bf16_bits(f)

    if nch == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nch)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# Workload: operation trace + values
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    """One decode step's inputs.

    ``ops`` builds the cache state before the step.  Kinds:
      ("add", seq)                       new empty sequence
      ("append", seq, n)                 n context tokens; their K/V are the next
                                         n rows of ``ctx_k``/``ctx_v``
      ("share_prefix", dst, src, ntok)   dst starts with src's first ntok tokens
      ("fork", parent, child)            child starts as a copy of parent
      ("swap_out", (seq, ...))           the sequences are paused together and
                                         their KV cache moves to the host pool
      ("swap_in", (seq, ...))            swapped-out sequences come back
      ("free", seq)                      the sequence ends; its blocks go back to
                                         the free list with their data in place
    The decode step then appends one token to every sequence of
    ``decode_seqs`` in that order (K/V rows ``new_k``/``new_v``), and every
    sequence's query row ``q[i]`` attends its whole history including that
    token.  ``seq_lens[i]`` is the length of ``decode_seqs[i]`` after the
    append.  ``free_order`` is the initial free list of physical block ids;
    blocks are taken from its end.  ``num_host_blocks`` and
    ``host_free_order`` describe the host pool the swaps use (none if 0).
    ``pool_init`` (None: zeros) holds the bits both pools start with, as
    (k_init, v_init) arrays of the pool's shape and stored type: the content
    of slots never written in the trace.
    """
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    num_blocks: int
    free_order: np.ndarray
    ops: list
    ctx_tokens: int
    decode_seqs: np.ndarray
    seq_lens: np.ndarray
    q: np.ndarray
    ctx_k: np.ndarray
    ctx_v: np.ndarray
    new_k: np.ndarray
    new_v: np.ndarray
    scale: float
    partition_tokens: int = 0
    seed: int = 0
    meta: dict = field(default_factory=dict)
    num_host_blocks: int = 0
    host_free_order: np.ndarray | None = None
    pool_init: tuple | None = None

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def num_seqs(self) -> int:
        return int(self.decode_seqs.size)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(max(1, -(-int(self.seq_lens.max()) // self.block_size)))

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    def kv_read_bytes(self) -> int:
        return attention_kv_bytes(self.seq_lens, self.num_kv_heads, self.head_dim, self.elem_bytes)


def _ceil_div(a, b):
    return -(-a // b)


def _slack_pool(need: int) -> int:
    """Pool sized to the blocks the workload needs plus 10 % slack, rounded up."""
    return _ceil_div(need * 11, 10)


def _draw_values(ss_kids, n_seqs, n_ctx, hq, hkv, d, dtype, values=True):
    if not values:
        z = np.zeros(0, dtype=np.float32 if dtype == "f32" else np.uint16)
        return z, z, z, z, z
    q = normal_array(ss_kids[_S_Q], (n_seqs, hq, d), dtype)
    ck = normal_array(ss_kids[_S_CTXK], (n_ctx, hkv, d), dtype)
    cv = normal_array(ss_kids[_S_CTXV], (n_ctx, hkv, d), dtype)
    nk = normal_array(ss_kids[_S_NEWK], (n_seqs, hkv, d), dtype)
    nv = normal_array(ss_kids[_S_NEWV], (n_seqs, hkv, d), dtype)
    return q, ck, cv, nk, nv


def independent_workload(lens, *, num_q_heads, num_kv_heads, head_dim, block_size,
                         dtype, seed, pool_blocks=0, partition_tokens=0, name="custom",
                         scale=None, kids=None, values=True) -> Workload:
    """Independent sequences with the given final lengths (context = len - 1
    tokens, then one decode append each).  Physical ids come from a seeded
    random permutation of the pool."""
    lens = np.asarray(lens, dtype=np.int64)
    if np.any(lens < 1):
        raise ValueError("every final length must be >= 1 (the decode token)")
    if kids is None:
        kids = np.random.SeedSequence(seed).spawn(8)
    need = int(np.sum(_ceil_div(lens, block_size)))
    nb = pool_blocks or _slack_pool(need)
    if nb < need:
        raise ValueError(f"pool of {nb} blocks < {need} needed")
    perm = np.random.Generator(np.random.PCG64(kids[_S_PERM])).permutation(nb).astype(np.int32)
    ops = []
    for s, L in enumerate(lens):
        ops.append(("add", s))
        if L > 1:
            ops.append(("append", s, int(L - 1)))
    n_ctx = int(np.sum(lens - 1))
    q, ck, cv, nk, nv = _draw_values(kids, lens.size, n_ctx, num_q_heads, num_kv_heads,
                                     head_dim, dtype, values)
    return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size, dtype=dtype, num_blocks=nb,
                    free_order=perm, ops=ops, ctx_tokens=n_ctx,
                    decode_seqs=np.arange(lens.size, dtype=np.int64),
                    seq_lens=lens.astype(np.int32), q=q, ctx_k=ck, ctx_v=cv, new_k=nk,
                    new_v=nv, scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                    partition_tokens=partition_tokens, seed=seed)


def shared_prefix_workload(*, prefix_tokens, suffix_lens, forking_parents, samples_per_fork,
                           num_q_heads, num_kv_heads, head_dim, block_size, dtype, seed,
                           partition_tokens=0, name="shared-prefix", kids=None,
                           values=True) -> Workload:
    """Base sequences 0..n-1 share one prefix (sequence 0 writes it, the others
    take it by reference), then each appends its own suffix.  The first
    ``forking_parents`` base sequences whose last block is partially filled fork
    ``samples_per_fork - 1`` children each (ids after all base sequences, in
    parent order).  The decode step appends one token to every sequence in
    ascending id order."""
    suffix = np.asarray(suffix_lens, dtype=np.int64)
    nbase = suffix.size
    if kids is None:
        kids = np.random.SeedSequence(seed).spawn(8)
    partial = [s for s in range(nbase) if (prefix_tokens + suffix[s]) % block_size != 0]
    parents = partial[:forking_parents]
    if len(parents) < forking_parents:
        raise ValueError("not enough sequences with a partially filled last block")
    nchild = samples_per_fork - 1
    ops = [("add", 0), ("append", 0, int(prefix_tokens))]
    for s in range(1, nbase):
        ops.append(("add", s))
        ops.append(("share_prefix", s, 0, int(prefix_tokens)))
    for s in range(nbase):
        if suffix[s] > 0:
            ops.append(("append", s, int(suffix[s])))
    child_of = {}
    nxt = nbase
    for p in parents:
        for _ in range(nchild):
            ops.append(("fork", p, nxt))
            child_of[nxt] = p
            nxt += 1
    nseq = nxt
    lens = np.empty(nseq, dtype=np.int64)
    lens[:nbase] = prefix_tokens + suffix + 1
    for c, p in child_of.items():
        lens[c] = lens[p]
    # Blocks needed: shared prefix once, each base sequence's own blocks after
    # the decode append, plus one private copy for every sharer but the last
    # of each forked partial block.
    pre_blocks = _ceil_div(prefix_tokens, block_size)
    need = pre_blocks + int(np.sum(_ceil_div(lens[:nbase], block_size) - pre_blocks))
    need += len(parents) * nchild
    nb = _slack_pool(need)
    perm = np.random.Generator(np.random.PCG64(kids[_S_PERM])).permutation(nb).astype(np.int32)
    n_ctx = int(prefix_tokens + np.sum(suffix))
    q, ck, cv, nk, nv = _draw_values(kids, nseq, n_ctx, num_q_heads, num_kv_heads, head_dim,
                                     dtype, values)
    return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size, dtype=dtype, num_blocks=nb,
                    free_order=perm, ops=ops, ctx_tokens=n_ctx,
                    decode_seqs=np.arange(nseq, dtype=np.int64), seq_lens=lens.astype(np.int32),
                    q=q, ctx_k=ck, ctx_v=cv, new_k=nk, new_v=nv,
                    scale=1.0 / math.sqrt(head_dim), partition_tokens=partition_tokens,
                    seed=seed, meta={"parents": parents, "children": child_of})


def preemption_workload(lens_before, *, swapped, grow, num_q_heads, num_kv_heads, head_dim,
                        block_size, dtype, seed, forks=(), host_blocks=0, partition_tokens=0,
                        name="preempt-swap", values=True) -> Workload:
    """Pause-and-resume trace.  Base sequences 0..n-1 write ``lens_before[s]``
    context tokens each; then each parent in ``forks`` forks one child (ids n,
    n+1, ... in order); the sequences of ``swapped`` are swapped out together;
    every other sequence s appends ``grow[s]`` more tokens (``grow`` covers
    every id, 0 for the swapped ones), taking first the blocks the swap
    released; the swapped sequences are swapped back in together; the decode
    step appends one token to every sequence in id order.  The device pool is
    sized for every sequence's final length with no sharing, plus 10 %; the
    host pool (``host_blocks``, default: the swapped sequences' blocks plus
    10 %) and both free orders are seeded permutations."""
    lens_before = np.asarray(lens_before, dtype=np.int64)
    n = lens_before.size
    forks = [int(p) for p in forks]
    nseq = n + len(forks)
    grow = np.asarray(grow, dtype=np.int64)
    swapped = [int(s) for s in swapped]
    if grow.size != nseq or np.any(grow < 0) or np.any(lens_before < 0):
        raise ValueError("grow must give a non-negative count for every sequence")
    if any(grow[s] for s in swapped):
        raise ValueError("a swapped-out sequence cannot grow")
    kids = np.random.SeedSequence(seed).spawn(9)
    ops = []
    for s in range(n):
        ops.append(("add", s))
        if lens_before[s]:
            ops.append(("append", s, int(lens_before[s])))
    before = list(lens_before)
    for i, p in enumerate(forks):
        ops.append(("fork", p, n + i))
        before.append(before[p])
    before = np.asarray(before, dtype=np.int64)
    if swapped:
        ops.append(("swap_out", tuple(swapped)))
    for s in range(nseq):
        if grow[s]:
            ops.append(("append", s, int(grow[s])))
    if swapped:
        ops.append(("swap_in", tuple(swapped)))
    lens = before + grow + 1
    need = int(np.sum(_ceil_div(lens, block_size)))
    nb = _slack_pool(need)
    hneed = int(sum(_ceil_div(before[s], block_size) for s in swapped))
    nh = host_blocks or _slack_pool(max(hneed, 1))
    perm = np.random.Generator(np.random.PCG64(kids[_S_PERM])).permutation(nb).astype(np.int32)
    hperm = np.random.Generator(np.random.PCG64(kids[8])).permutation(nh).astype(np.int32)
    n_ctx = int(np.sum(lens_before) + np.sum(grow))
    q, ck, cv, nk, nv = _draw_values(kids, nseq, n_ctx, num_q_heads, num_kv_heads, head_dim,
                                     dtype, values)
    return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size, dtype=dtype, num_blocks=nb,
                    free_order=perm, ops=ops, ctx_tokens=n_ctx,
                    decode_seqs=np.arange(nseq, dtype=np.int64), seq_lens=lens.astype(np.int32),
                    q=q, ctx_k=ck, ctx_v=cv, new_k=nk, new_v=nv,
                    scale=1.0 / math.sqrt(head_dim), partition_tokens=partition_tokens,
                    seed=seed, meta={"swapped": swapped, "forks": forks},
                    num_host_blocks=nh, host_free_order=hperm)


def preemption_config_workload(name: str, swap_fraction: float = 0.25, grow_tokens: int = 64,
                               seed: int | None = None, values: bool = True) -> Workload:
    """A pause-and-resume trace on a named independent-sequence configuration:
    its sequences (at the configuration's lengths minus the decode token)
    are built, the latest ``swap_fraction`` of them are swapped out together
    (latecomers first, [KVM §19.2.6]), every other one grows by
    ``grow_tokens`` tokens into the released blocks, the paused ones come back
    and the decode step runs over all of them."""
    c = CONFIGS[name]
    if c.prefix_tokens or c.fixed_lens and len(c.fixed_lens) < 2:
        raise ValueError("needs a configuration of several independent sequences")
    seed = c.seed if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(8)
    if c.fixed_lens:
        lens = np.asarray(c.fixed_lens, dtype=np.int64)
    else:
        g = np.random.Generator(np.random.PCG64(kids[_S_LENS]))
        lens = g.integers(c.len_range[0], c.len_range[1] + 1, size=c.num_seqs)
    n = lens.size
    k = max(1, int(round(n * swap_fraction)))
    swapped = list(range(n - k, n))
    grow = np.where(np.arange(n) < n - k, grow_tokens, 0)
    return preemption_workload(lens - 1, swapped=swapped, grow=grow, num_q_heads=c.num_q_heads,
                               num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
                               block_size=c.block_size, dtype=c.dtype, seed=seed,
                               partition_tokens=c.partition_tokens, name=f"{c.name}-preempt",
                               values=values)


# Non-finite and extreme bit patterns of each stored type: quiet NaN, +Inf,
# -Inf, the largest finite value and its negation.
_STALE_BITS = {
    "bf16": np.array([0x7FC0, 0x7F80, 0xFF80, 0x7F7F, 0xFF7F], dtype=np.uint16),
    "f32": np.array([0x7FC00000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF],
                    dtype=np.uint32),
}


def stale_pool_bits(shape, dtype: str, seed: int):
    """Pool contents before any write ([ENG §3.2] and the release section of
    [SLOT]: freed blocks keep whatever they held): every element one of
    NaN, +Inf, -Inf, +max, -max, drawn uniformly from SeedSequence(seed).
    Returns (k_init, v_init) in the stored type (uint16 bf16 bits or
    float32)."""
    kids = np.random.SeedSequence(seed).spawn(2)
    pats = _STALE_BITS[dtype]
    out = []
    for kid in kids:
        g = np.random.Generator(np.random.PCG64(kid))
        bits = pats[g.integers(0, pats.size, size=int(np.prod(shape)))].reshape(shape)
        out.append(bits if dtype == "bf16" else bits.view(np.float32))
    return tuple(out)


def with_stale_pools(wl: Workload, seed: int | None = None) -> Workload:
    """The same workload with both pools starting from stale non-finite bits
    (``stale_pool_bits``, seed defaults to the workload's + 2000)."""
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
    wl.pool_init = stale_pool_bits(shape, wl.dtype, (wl.seed + 2000) if seed is None else seed)
    wl.name = f"{wl.name}+stale"
    return wl


def churn_workload(first_lens, freed, second_lens, *, num_q_heads, num_kv_heads, head_dim,
                   block_size, dtype, seed, forks=(), name="churn", values=True) -> Workload:
    """A pool that has been used before.  Sequences 0..n1-1 write
    ``first_lens`` context tokens; the sequences in ``freed`` end (their
    blocks return to the free list, data left in place); sequences n1.. then
    write ``second_lens`` tokens each, taking the freed blocks first (most
    recently freed first); each sequence of ``forks`` (live ones, in order)
    forks one child (ids after all others), so the child shares its parent's
    partly filled last block; the decode step appends one token to every live
    sequence in ascending id.  The pool holds the blocks of the first round
    plus 10 %, or the peak need if that is larger."""
    first = np.asarray(first_lens, dtype=np.int64)
    second = np.asarray(second_lens, dtype=np.int64)
    n1, n2 = first.size, second.size
    freed = sorted(int(s) for s in freed)
    forks = [int(p) for p in forks]
    kids = np.random.SeedSequence(seed).spawn(8)
    ops = []
    for s in range(n1):
        ops.append(("add", s))
        if first[s]:
            ops.append(("append", s, int(first[s])))
    for s in freed:
        ops.append(("free", s))
    for i in range(n2):
        s = n1 + i
        ops.append(("add", s))
        if second[i]:
            ops.append(("append", s, int(second[i])))
    live = [s for s in range(n1) if s not in freed] + list(range(n1, n1 + n2))
    length = {s: int(first[s]) for s in range(n1)}
    length.update({n1 + i: int(second[i]) for i in range(n2)})
    nxt = n1 + n2
    for p in forks:
        if p not in live:
            raise ValueError("only a live sequence can fork")
        ops.append(("fork", p, nxt))
        length[nxt] = length[p]
        live.append(nxt)
        nxt += 1
    lens = np.array([length[s] + 1 for s in live], dtype=np.int64)
    # peak need: the first round, and the end state with a private copy for
    # every fork (copy-on-write at the decode append)
    need_first = int(np.sum(_ceil_div(first, block_size)))
    need_end = int(np.sum(_ceil_div(lens, block_size)))
    nb = max(_slack_pool(need_first), _slack_pool(need_end))
    perm = np.random.Generator(np.random.PCG64(kids[_S_PERM])).permutation(nb).astype(np.int32)
    n_ctx = int(np.sum(first) + np.sum(second))
    q, ck, cv, nk, nv = _draw_values(kids, len(live), n_ctx, num_q_heads, num_kv_heads,
                                     head_dim, dtype, values)
    return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size, dtype=dtype, num_blocks=nb,
                    free_order=perm, ops=ops, ctx_tokens=n_ctx,
                    decode_seqs=np.asarray(live, dtype=np.int64), seq_lens=lens.astype(np.int32),
                    q=q, ctx_k=ck, ctx_v=cv, new_k=nk, new_v=nv,
                    scale=1.0 / math.sqrt(head_dim), seed=seed,
                    meta={"freed": freed, "forks": forks})


def multi_queries(wl: Workload, n: int):
    """Queries for n new tokens per sequence of ``wl`` (its n newest cached
    tokens; fewer when a history is shorter): bf16 bit patterns
    [total, num_q_heads, head_dim] drawn N(0, 1) from SeedSequence(seed + 1000),
    and the int32 offsets [num_seqs + 1] of each sequence's rows."""
    nq = np.minimum(int(n), wl.seq_lens.astype(np.int64))
    offs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = normal_array(np.random.SeedSequence(wl.seed + 1000),
                     (int(offs[-1]), wl.num_q_heads, wl.head_dim), wl.dtype)
    return q, offs


def config_workload(name: str, seed: int | None = None, values: bool = True) -> Workload:
    """The named configuration's workload (seed defaults to the config's).
    ``values=False`` skips drawing q/K/V (trace and sizes only)."""
    c = CONFIGS[name]
    seed = c.seed if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(8)
    common = dict(num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
                  head_dim=c.head_dim, block_size=c.block_size, dtype=c.dtype, seed=seed,
                  partition_tokens=c.partition_tokens, name=c.name, kids=kids, values=values)
    if c.prefix_tokens:
        g = np.random.Generator(np.random.PCG64(kids[_S_SUFFIX]))
        suffix = g.integers(c.suffix_range[0], c.suffix_range[1] + 1, size=c.base_seqs)
        return shared_prefix_workload(prefix_tokens=c.prefix_tokens, suffix_lens=suffix,
                                      forking_parents=c.forking_parents,
                                      samples_per_fork=c.samples_per_fork, **common)
    if c.fixed_lens:
        lens = np.asarray(c.fixed_lens, dtype=np.int64)
    else:
        g = np.random.Generator(np.random.PCG64(kids[_S_LENS]))
        lens = g.integers(c.len_range[0], c.len_range[1] + 1, size=c.num_seqs)
    return independent_workload(lens, pool_blocks=c.pool_blocks, **common)
