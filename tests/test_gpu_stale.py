"""GPU parity on pools whose unwritten slots hold stale, non-finite bits.

Nothing clears a block when it is freed or before it is first used ([ENG §3.2];
the release section of [SLOT]): a partly filled last block keeps whatever its
remaining slots held, a block taken over from a finished sequence keeps that
sequence's values, and a copy-on-write copy carries the source block's unused
slots along.  Here both pools start as NaN, +-Inf and +-max bits
(``workloads.stale_pool_bits``); sequences write their contexts, some end, new
ones take their blocks, some fork, and the decode step runs.  Every route of the
attention must give the oracle's result (which reads positions < L only), and
write and copy must leave pools identical to the oracle's bit for bit, stale
bits included.  Routes: balanced split, fixed partitions, the append folded
into the attention, cacheable loads (forked batches), the matrix-core route
(groups of 8), the shared-prefix kernels, multi-token queries.  A hand case
runs the shared-prefix kernels on a fork family that shares a partly written
last block before any append (every member shorter than the shared blocks).
Every case prints its shape first."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.attention import attention_decode, attention_multi, attention_split, to_f64  # noqa: E402
from oracle.replay import run_step  # noqa: E402
from tests.parity import assert_gate  # noqa: E402
from workloads import (churn_workload, multi_queries, shared_prefix_workload,  # noqa: E402
                       stale_pool_bits, with_stale_pools)

pytestmark = pytest.mark.gpu

FIRST = [37, 100, 16, 250, 5, 64, 130, 17, 1, 300]
FREED = [1, 3, 6, 8]
SECOND = [45, 200, 31, 9, 160, 2]
FORKS = [0, 7, 12]   # live sequences whose last block is partly filled at B = 8, 16, 32


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()


def bits(a):
    """Stored values as integers (NaN payloads compare bit for bit)."""
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def host_bits(t):
    from paged_attention_slot_amd.runtime import to_host_bits
    return to_host_bits(t)


def stale_churn(Hq, Hkv, D, B, dtype, forks, seed):
    wl = churn_workload(FIRST, FREED, SECOND, forks=forks if forks else (), num_q_heads=Hq,
                        num_kv_heads=Hkv, head_dim=D, block_size=B, dtype=dtype, seed=seed,
                        name=f"churn-{dtype}-H{Hq}x{Hkv}-D{D}-B{B}{'-forks' if forks else ''}")
    return with_stale_pools(wl)


def build(wl, partition_tokens=None):
    from paged_attention_slot_amd.runtime import DecodeStep
    say(f"  case {wl.name}: N={wl.num_seqs} lens={wl.seq_lens.tolist()} pool={wl.num_blocks} "
        f"seed={wl.seed}")
    step = DecodeStep(wl, partition_tokens=partition_tokens)
    ost = run_step(wl, keep_values=False)
    assert np.array_equal(step.block_tables_h, ost.block_tables)
    assert np.array_equal(step.slot_mapping_h, ost.slot_mapping)
    return step, ost


def check_pools(step, ost):
    assert np.array_equal(bits(host_bits(step.k_cache)), bits(ost.k_pool)), "K pool differs"
    assert np.array_equal(bits(host_bits(step.v_cache)), bits(ost.v_pool)), "V pool differs"


def check_out(out_t, ref, dtype, what):
    out = to_f64(host_bits(out_t))
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    r = assert_gate(out, ref, dtype, what)
    say("  gate", what, r)


ROUTES = [  # id, Hq, Hkv, D, B, dtype, mode env, forks, fused
    ("balanced-bf16", 16, 8, 128, 16, "bf16", "2", False, False),
    ("balanced-bf16-append-folded", 16, 8, 128, 16, "bf16", "2", False, True),
    ("balanced-bf16-G4-append", 32, 8, 128, 16, "bf16", "2", False, True),
    ("balanced-f32", 8, 2, 64, 16, "f32", "2", False, False),
    ("balanced-f32-append-folded", 4, 2, 64, 16, "f32", "2", False, True),
    ("partitions-bf16", 16, 8, 128, 16, "bf16", "1", False, False),
    ("partitions-bf16-append", 32, 8, 128, 32, "bf16", "1", False, True),
    ("partitions-f32", 6, 2, 128, 16, "f32", "1", False, False),
    ("balanced-bf16-forks-cacheable", 32, 8, 128, 16, "bf16", "2", True, True),
    ("partitions-f32-forks", 8, 2, 64, 8, "f32", "1", True, False),
    ("matrix-bf16", 64, 8, 128, 16, "bf16", None, False, False),
    ("matrix-balanced-bf16", 32, 8, 128, 16, "bf16", "4", False, True),
    ("matrix-balanced-bf16-forks", 16, 8, 128, 32, "bf16", "4", True, False),
    ("matrix-bf16-B32-forks", 64, 8, 128, 32, "bf16", None, True, True),
]


@pytest.mark.parametrize("rid,Hq,Hkv,D,B,dtype,mode,forks,fused", ROUTES, ids=[r[0] for r in ROUTES])
def test_decode_routes_on_stale_pools(rid, Hq, Hkv, D, B, dtype, mode, forks, fused, tuning):
    tuning("PKV_ATTN_PARTS_PER_WG", 0)
    tuning("PKV_ATTN_MODE", int(mode) if mode else 0)
    wl = stale_churn(Hq, Hkv, D, B, dtype, FORKS if forks else None, seed=300 + Hq + B + D)
    step, ost = build(wl)
    say(f"  route {step.split} kv_shared={step.kv_shared} fused={fused} "
        f"folded={step.append_folded if fused else None} cow={len(ost.cow_pairs)}")
    if forks:
        assert len(ost.cow_pairs) == len(FORKS)
    if "folded" in rid:
        assert step.append_folded
    step.step(fused=fused)
    torch.cuda.synchronize()
    check_pools(step, ost)
    ref = attention_decode(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    check_out(step.out, ref, dtype, rid)


@pytest.mark.parametrize("pt", [32, 64])
def test_split_partitions_on_stale_pools(pt, tuning):
    """Given partitions (vector and matrix-core routes) against the oracle's
    split attention."""
    tuning("PKV_ATTN_MODE", 0)
    tuning("PKV_ATTN_PARTS_PER_WG", 0)
    for Hq in (16, 64):
        wl = stale_churn(Hq, 8, 128, 16, "bf16", None, seed=400 + pt + Hq)
        step, ost = build(wl, partition_tokens=pt)
        say(f"  route {step.split}")
        step.step()
        torch.cuda.synchronize()
        check_pools(step, ost)
        ref = attention_split(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                              wl.scale, pt)
        check_out(step.out, ref, "bf16", f"split pt={pt} Hq={Hq}")


SHARED = [  # prefix, suffix lens, forking parents, samples, Hq, Hkv, B
    (40, [3, 9, 1, 20, 33], 2, 3, 32, 8, 16),     # prefix ends inside a block
    (64, [3, 16, 7, 1, 12, 30, 9], 4, 4, 16, 4, 32),
]


@pytest.mark.parametrize("prefix,suffix,fp,spf,Hq,Hkv,B", SHARED, ids=lambda v: str(v))
def test_shared_prefix_kernels_on_stale_pools(prefix, suffix, fp, spf, Hq, Hkv, B):
    """The shared-prefix kernels on a family that shares a prefix and forks
    (copy-on-write copies carry stale tails), after the decode append."""
    wl = shared_prefix_workload(prefix_tokens=prefix, suffix_lens=suffix, forking_parents=fp,
                                samples_per_fork=spf, num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim=128, block_size=B, dtype="bf16", seed=500 + prefix + B,
                                name=f"family-p{prefix}")
    # a prefix ending inside a block is copied once per sharer
    wl.num_blocks += len(suffix) + 8
    wl.free_order = np.random.default_rng(prefix).permutation(wl.num_blocks).astype(np.int32)
    wl = with_stale_pools(wl)
    step, ost = build(wl)
    step.copy()
    step.write()
    gs, pl, mg, mp, ms = step.shared_groups()
    say(f"  groups={pl.numel()} max_group={mg} max_prefix={mp} max_suffix={ms}")
    assert mp > 0
    step.attention_shared()
    torch.cuda.synchronize()
    check_pools(step, ost)
    ref = attention_decode(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    check_out(step.out, ref, "bf16", f"shared {wl.name} Hq={Hq} B={B}")


def test_multi_token_queries_on_stale_pools():
    from paged_attention_slot_amd import ops
    wl = stale_churn(32, 8, 128, 16, "bf16", None, seed=601)
    step, ost = build(wl)
    step.step()
    torch.cuda.synchronize()
    q, offs = multi_queries(wl, 4)
    from paged_attention_slot_amd.runtime import to_device
    out = ops.attention_multi(to_device(q, "bf16", step.device),
                              torch.from_numpy(offs).to(step.device), step.k_cache, step.v_cache,
                              step.block_tables, step.seq_lens, wl.scale, 4,
                              max_seq_len=step.max_seq_len)
    torch.cuda.synchronize()
    ref = attention_multi(q, offs, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                          wl.scale)
    check_out(out, ref, "bf16", "multi-token, 4 per sequence")


def test_shared_partial_last_block_before_any_append(tuning):
    """A fork family (and a second group) whose shared last block is only
    partly written and no member has appended since: every member is shorter
    than the shared blocks, whose remaining slots hold NaN / Inf.  The
    shared-prefix kernels and every decode route must ignore those slots."""
    from paged_attention_slot_amd import ops
    B, Hq, Hkv, D, nb = 16, 32, 8, 128, 16
    tables = np.full((8, 4), -1, np.int32)
    tables[0:4, :3] = [5, 7, 9]            # family of 4: 40 tokens each (block 9 holds 8)
    tables[4:7, :2] = [2, 3]               # family of 3: 20, 20, 19 tokens
    tables[7, :3] = [11, 0, 13]            # on its own
    lens = np.array([40, 40, 40, 40, 20, 20, 19, 35], np.int32)
    rng = np.random.default_rng(77)
    kp, vp = stale_pool_bits((nb, B, Hkv, D), "bf16", 78)
    written = {5: 16, 7: 16, 9: 8, 2: 16, 3: 4, 11: 16, 0: 16, 13: 3}
    for blk, n in written.items():
        for pool in (kp, vp):
            u = rng.normal(0, 1, (n, Hkv, D)).astype(np.float32).view(np.uint32)
            pool[blk, :n] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    u = rng.normal(0, 1, (8, Hq, D)).astype(np.float32).view(np.uint32)
    q = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    scale = 1 / np.sqrt(D)
    ref = attention_decode(q, kp, vp, tables, lens, scale)
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    qd, kd, vd = t(q), t(kp), t(vp)
    tb, ln = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    starts, plens, mg, mp, ms = ops.prefix_groups(tables, lens, B)
    say(f"  groups {starts.tolist()} prefixes {plens.tolist()}")
    assert starts.tolist() == [0, 4, 7, 8] and plens.tolist() == [48, 32, 0]
    out = ops.attention_decode_shared(qd, kd, vd, tb, ln, scale,
                                      torch.from_numpy(starts).to(dev),
                                      torch.from_numpy(plens).to(dev), mg, mp, ms,
                                      max_seq_len=int(lens.max()))
    torch.cuda.synchronize()
    check_out(out, ref, "bf16", "shared kernels, partly written shared block")
    for mode in (1, 2):
        tuning("PKV_ATTN_MODE", mode)
        o = ops.attention_decode(qd, kd, vd, tb, ln, scale, max_seq_len=int(lens.max()))
        torch.cuda.synchronize()
        check_out(o, ref, "bf16", f"decode mode {mode}, partly written shared block")
