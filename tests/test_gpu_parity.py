"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Write and copy: bit-exact full pools.  Attention: the gate of tests/parity.py
against the fp64 oracle, plus exact special cases (a single position returns
its value; a different physical placement gives bit-identical output; an empty
history gives zeros).  Small cases span several tiles with ragged tails; the
full-size configurations run in the launch configuration the bench times.
"""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.attention import attention_decode as oracle_attention  # noqa: E402
from oracle.attention import attention_split as oracle_split  # noqa: E402
from oracle.attention import to_f64  # noqa: E402
from oracle.replay import run_step  # noqa: E402
from tests.parity import assert_gate  # noqa: E402
from workloads import config_workload, independent_workload, shared_prefix_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()  # fail loudly if the library is missing
    return torch.device("cuda:0")


def run_both(wl, partition_tokens=None, attention=True):
    from paged_attention_slot_amd.runtime import DecodeStep
    say(f"  case {wl.name}: N={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"D={wl.head_dim} B={wl.block_size} {wl.dtype} maxlen={wl.max_seq_len} "
        f"pt={partition_tokens} seed={wl.seed}")
    step = DecodeStep(wl, partition_tokens=partition_tokens)
    step.copy()
    step.write()
    if attention:
        step.attention()
    torch.cuda.synchronize()
    ost = run_step(wl, keep_values=False)
    # the two block managers agree on the step's host part
    assert np.array_equal(step.slot_mapping_h, ost.slot_mapping)
    assert np.array_equal(step.cow_pairs_h.reshape(-1, 2), ost.cow_pairs.reshape(-1, 2))
    assert np.array_equal(step.block_tables_h, ost.block_tables)
    return step, ost


def host_bits(t):
    from paged_attention_slot_amd.runtime import to_host_bits
    return to_host_bits(t)


def check_pools(step, ost):
    assert np.array_equal(host_bits(step.k_cache), ost.k_pool), "K pool differs"
    assert np.array_equal(host_bits(step.v_cache), ost.v_pool), "V pool differs"


def gpu_out(step):
    return to_f64(host_bits(step.out))


LENS = [1, 7, 16, 17, 33, 100, 255, 300]
SMALL = [
    # dtype, B, D, Hq, Hkv
    ("bf16", 16, 128, 16, 8),
    ("bf16", 16, 128, 32, 8),
    ("bf16", 32, 128, 64, 8),
    ("bf16", 8, 64, 8, 8),
    ("bf16", 64, 64, 12, 4),
    ("bf16", 16, 128, 16, 1),
    ("f32", 16, 64, 8, 2),
    ("f32", 32, 128, 4, 4),
    ("f32", 8, 128, 6, 2),
]


@pytest.mark.parametrize("dtype,B,D,Hq,Hkv", SMALL, ids=lambda v: str(v))
def test_small_write_and_attention(dtype, B, D, Hq, Hkv):
    wl = independent_workload(LENS, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                              dtype=dtype, seed=100 + B + D + Hq)
    step, ost = run_both(wl)
    check_pools(step, ost)
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    out = gpu_out(step)
    r = assert_gate(out, ref, dtype, wl.name)
    say("  gate", r)
    G = Hq // Hkv
    for i, L in enumerate(wl.seq_lens):
        if L == 1:  # a single position: the output is that position's value, exactly
            for h in range(Hq):
                assert np.array_equal(out[i, h], to_f64(wl.new_v[i, h // G]))


@pytest.mark.parametrize("name", ["qwen3-0.6b-layer", "shared-prefix-cow", "llama3.1-70b-longctx"])
def test_cacheable_and_streaming_loads_agree(name):
    """PKV_KV_SHARED only changes how K/V are loaded (cacheable instead of
    non-temporal), so both give bit-identical outputs, whichever the batch."""
    wl = config_workload(name)
    step, _ = run_both(wl, attention=False)
    a = host_bits(step.attention(out=torch.empty_like(step.q)))
    step.kv_shared = not step.kv_shared
    b = host_bits(step.attention(out=torch.empty_like(step.q)))
    torch.cuda.synchronize()
    say(f"  kv_shared (detected) = {not step.kv_shared}, split {step.split}")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("ppw", [None, "3"])
@pytest.mark.parametrize("pt", [0, 32, 96, 512])
def test_matrix_route_matches_oracle(pt, ppw, tuning):
    """The matrix-core route with fixed partitions (PKV_ATTN_MODE=3; the
    default for more than 16 query heads per KV head), 8 heads per group,
    with automatic or given partitions, and with runs of 3 partitions per
    workgroup (PKV_ATTN_PARTS_PER_WG): outputs against the oracle's split (or
    unsplit) attention."""
    tuning("PKV_ATTN_MODE", 3)
    tuning("PKV_ATTN_PARTS_PER_WG", int(ppw) if ppw else 0)
    wl = independent_workload([1, 15, 16, 17, 64, 200, 333, 1500], num_q_heads=64,
                              num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                              seed=17 + pt)
    step, ost = run_both(wl, partition_tokens=pt)
    say(f"  split {step.split} runs={ppw}")
    assert step.split["mode"] == "matrix"
    got = gpu_out(step)
    if pt:
        ref = oracle_split(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale, pt)
    else:
        ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                               wl.scale)
    say("  gate", assert_gate(got, ref, "bf16", f"matrix route pt={pt}"))


@pytest.mark.parametrize("pt", [32, 64, 96])
def test_matrix_route_equal_shares(pt, tuning):
    """More short partitions than the GPU holds at once on the matrix-core
    route: workgroups take runs of whole partitions and fold each run into one
    piece, so the workspace holds fewer rows than partitions.  Outputs against the oracle's split
    attention; then again with one history emptied, which must give zeros."""
    from paged_attention_slot_amd import ops
    tuning("PKV_ATTN_MODE", 3)
    tuning("PKV_ATTN_PARTS_PER_WG", 0)
    wl = independent_workload([1, 2, 31, 33, 500, 2047, 6000, 7500], num_q_heads=64,
                              num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                              seed=40 + pt)
    step, ost = run_both(wl, partition_tokens=pt)
    assert step.split["mode"] == "matrix"
    n_parts = -(-wl.max_seq_len // pt)
    whole = wl.num_seqs * wl.num_q_heads * n_parts * (128 + 2) * 4
    ws = ops.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.max_seq_len, step.k_cache, pt)
    say(f"  workspace {ws} bytes, {whole} for one piece per partition")
    assert 0 < ws < whole
    got = gpu_out(step)
    ref = oracle_split(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens, wl.scale,
                       pt)
    say("  gate", assert_gate(got, ref, "bf16", f"equal shares pt={pt}"))
    lens = step.seq_lens.clone()
    lens[5] = 0
    out = torch.full_like(step.q, 7.0)
    ops.attention_decode(step.q, step.k_cache, step.v_cache, step.block_tables, lens, wl.scale,
                         out=out, max_seq_len=wl.max_seq_len, partition_tokens=pt)
    torch.cuda.synchronize()
    o = to_f64(host_bits(out))
    assert not o[5].any()
    ref = oracle_split(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, lens.cpu().numpy(),
                       wl.scale, pt)
    assert_gate(o, ref, "bf16", f"equal shares, one empty history, pt={pt}")


@pytest.mark.parametrize("Hq,pt,shared,mode", [(16, None, False, 0), (16, None, True, 0),
                                               (32, 64, False, 1), (64, None, False, 3),
                                               (64, 32, False, 3), (64, None, False, 0),
                                               (64, 96, False, 0)],
                         ids=["balanced", "balanced-cacheable", "partitions", "matrix",
                              "matrix-shares", "matrix-balanced", "matrix-given-partitions"])
def test_split_phases_match_one_call(Hq, pt, shared, mode, tuning):
    """pkv_attention_decode_phase: the per-partition phase, then the merge
    phase in a call of its own (which reads what the first left in the
    workspace: pieces, and on the balanced splits each stream's first and last
    interval), gives the bits of one call with both phases; a second merge
    call gives them again."""
    tuning("PKV_ATTN_MODE", mode)
    tuning("PKV_ATTN_PARTS_PER_WG", 0)
    wl = independent_workload([1, 15, 16, 17, 64, 200, 333, 1500, 2047, 3000], num_q_heads=Hq,
                              num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                              seed=60 + Hq + (pt or 0))
    step, _ = run_both(wl, partition_tokens=pt, attention=False)
    step.kv_shared = shared
    say(f"  split {step.split} kv_shared={shared}")
    one = host_bits(step.attention(out=torch.empty_like(step.q)))
    out = torch.empty_like(step.q)
    step.attention(out=out, phases=1)
    step.attention(out=out, phases=2)
    first = host_bits(out)
    step.attention(out=out, phases=2)
    again = host_bits(out)
    torch.cuda.synchronize()
    assert np.array_equal(one, first), "phase 1 then phase 2 differs from one call"
    assert np.array_equal(one, again), "a second merge call differs"


SPLITS = [(pt, dtype, B) for pt in (16, 32, 64, 128, 256)
          for dtype, B in (("bf16", 16), ("f32", 16), ("bf16", 32)) if pt % B == 0]


@pytest.mark.parametrize("pt,dtype,B", SPLITS, ids=lambda v: str(v))
def test_split_kv_matches_oracle_and_unsplit(pt, dtype, B):
    wl = independent_workload([1, 15, 16, 17, 64, 200, 333, 513], num_q_heads=16,
                              num_kv_heads=4, head_dim=128, block_size=B, dtype=dtype, seed=7)
    step, ost = run_both(wl, partition_tokens=pt)
    split = gpu_out(step)
    ref = oracle_split(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens, wl.scale,
                       pt)
    assert_gate(split, ref, dtype, f"split {pt}")
    whole = to_f64(host_bits(step.attention(partition_tokens=10**6 // B * B)))
    torch.cuda.synchronize()
    assert_gate(split, whole, dtype, "split vs unsplit")


def test_physical_placement_gives_bit_identical_output():
    a = independent_workload([5, 40, 97, 160], num_q_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=16, dtype="bf16", seed=3)
    b = independent_workload([5, 40, 97, 160], num_q_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=16, dtype="bf16", seed=3)
    b.free_order = np.random.default_rng(1234).permutation(b.num_blocks).astype(np.int32)
    sa, oa = run_both(a)
    sb, ob = run_both(b)
    assert not np.array_equal(oa.block_tables, ob.block_tables)
    assert np.array_equal(host_bits(sa.out), host_bits(sb.out))


def test_zero_length_sequences_give_zeros():
    from paged_attention_slot_amd import ops
    wl = independent_workload([3, 50, 20], num_q_heads=8, num_kv_heads=2, head_dim=64,
                              block_size=16, dtype="bf16", seed=9)
    step, ost = run_both(wl, attention=False)
    lens = step.seq_lens.clone()
    lens[1] = 0
    for pt in (0, 16):
        out = torch.full_like(step.q, 7.0)
        ops.attention_decode(step.q, step.k_cache, step.v_cache, step.block_tables, lens,
                             wl.scale, out=out, max_seq_len=50, partition_tokens=pt)
        torch.cuda.synchronize()
        o = to_f64(host_bits(out))
        assert not o[1].any()
        ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables,
                               lens.cpu().numpy(), wl.scale)
        assert_gate(o, ref, "bf16", f"zero-length pt={pt}")


def test_copy_on_write_family_small():
    wl = shared_prefix_workload(prefix_tokens=64, suffix_lens=[3, 16, 7, 1, 12, 30, 9],
                                forking_parents=4, samples_per_fork=4, num_q_heads=16,
                                num_kv_heads=4, head_dim=128, block_size=16, dtype="bf16", seed=5)
    step, ost = run_both(wl)
    assert len(ost.cow_pairs) == 12
    check_pools(step, ost)
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    assert_gate(gpu_out(step), ref, "bf16", "cow family")


# -- full-size configurations, in the bench's launch configuration -----------

_ORACLE = {}


def oracle_of(name):
    """The oracle's pools, tables and attention of a configuration, computed
    once for the two forms of its step (kept for one configuration at a
    time)."""
    if name not in _ORACLE:
        _ORACLE.clear()
        wl = config_workload(name)
        ost = run_step(wl, keep_values=False)
        ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                               wl.scale)
        _ORACLE[name] = (wl, ost, ref)
    return _ORACLE[name]


CONFIGS = ["tiny", "qwen3-0.6b-layer", "llama3-8b-layer", "shared-prefix-cow",
           "llama3.1-70b-longctx"]


@pytest.mark.parametrize("fused", [False, True], ids=["write-then-attention", "append-folded"])
@pytest.mark.parametrize("name", CONFIGS)
def test_config_full(name, fused):
    """Every output element of every configuration against the oracle, pools
    bit-exact.  ``fused``: the step as the bench times it (copy, then
    pkv_attention_decode_append: the append inside the attention or its
    row-copy kernel), else copy -> write -> attention."""
    from paged_attention_slot_amd.runtime import DecodeStep
    wl, ost, ref = oracle_of(name)
    say(f"  case {name}: N={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"D={wl.head_dim} B={wl.block_size} {wl.dtype} maxlen={wl.max_seq_len} fused={fused}")
    step = DecodeStep(wl)
    assert np.array_equal(step.slot_mapping_h, ost.slot_mapping)
    assert np.array_equal(step.cow_pairs_h.reshape(-1, 2), ost.cow_pairs.reshape(-1, 2))
    assert np.array_equal(step.block_tables_h, ost.block_tables)
    say(f"  split {step.split} kv_shared={step.kv_shared} "
        f"folded={step.append_folded if fused else None}")
    step.step(fused=fused)
    torch.cuda.synchronize()
    check_pools(step, ost)
    out = gpu_out(step)
    assert np.isfinite(out).all()
    r = assert_gate(out, ref, wl.dtype, name)
    say("  gate", r)
    if name == "tiny":
        # the page's self-check bound, fp32 end to end
        assert r["max_abs"] < 1e-5
    del step
    torch.cuda.empty_cache()


def test_long_context_config_partitions_against_oracle_split():
    """The long-context configuration at its 512-token partitions against the
    oracle's split attention with the same partitions (the log-sum-exp merge
    of 256 pieces per history), every element."""
    wl, ost, _ = oracle_of("llama3.1-70b-longctx")
    step, _ = run_both(wl)
    ref = oracle_split(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens, wl.scale,
                       512)
    say("  gate", assert_gate(gpu_out(step), ref, "bf16", "long context, 512-token partitions"))


@pytest.mark.parametrize("zeros", [(), (0,), (4,), (9,), (0, 4, 9), tuple(range(10))],
                         ids=["none", "first", "middle", "last", "several", "all"])
def test_matrix_balanced_empty_histories_and_used_workspaces(zeros, tuning):
    """The matrix-core balanced split with its merge: empty histories anywhere
    in the batch (or all of it) give zero rows; a workspace of arbitrary bytes
    gives the bits of a zeroed one; the two phases in calls of their own give
    the same bits; a smaller batch right after, on the same workspace, gives
    the bits of its own call on a fresh one."""
    from paged_attention_slot_amd import ops
    tuning("PKV_ATTN_MODE", 4)
    lens_all = [1, 15, 16, 17, 64, 200, 333, 1500, 2047, 3000]
    wl = independent_workload(lens_all, num_q_heads=32, num_kv_heads=8, head_dim=128,
                              block_size=16, dtype="bf16", seed=91)
    step, ost = run_both(wl, attention=False)
    say(f"  split {step.split} zeros={zeros}")
    lens = step.seq_lens.clone()
    for z in zeros:
        lens[z] = 0
    N, Hq = wl.num_seqs, wl.num_q_heads
    need = ops.workspace_bytes(N, Hq, wl.max_seq_len, step.k_cache, 0)
    dev = step.q.device
    gen = torch.Generator(device="cpu").manual_seed(5)
    dirty_h = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=gen)

    def call(n, ws, phases=3):
        out = torch.full_like(step.q[:n], 7.0)
        for ph in ((1, 2) if phases == 12 else (3,)):
            ops.attention_decode(step.q[:n], step.k_cache, step.v_cache, step.block_tables[:n],
                                 lens[:n], wl.scale, out=out, max_seq_len=wl.max_seq_len,
                                 workspace=ws, phases=ph)
        torch.cuda.synchronize()
        return host_bits(out)

    clean = call(N, torch.zeros(need, dtype=torch.uint8, device=dev))
    dirty_ws = dirty_h.to(dev)
    dirty = call(N, dirty_ws)
    assert np.array_equal(clean, dirty), "a workspace of arbitrary bytes changes the result"
    split = call(N, dirty_ws, phases=12)
    assert np.array_equal(clean, split), "phase 1 then phase 2 differs from one call"
    o = to_f64(clean)
    for z in zeros:
        assert not o[z].any(), f"empty history {z} not zero"
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, lens.cpu().numpy(),
                           wl.scale)
    say("  gate", assert_gate(o, ref, "bf16", f"matrix-balanced zeros={zeros}"))
    n2 = 6
    again = call(n2, dirty_ws)
    fresh = call(n2, torch.zeros(ops.workspace_bytes(n2, Hq, wl.max_seq_len, step.k_cache, 0),
                                 dtype=torch.uint8, device=dev))
    assert np.array_equal(again, fresh), "a smaller batch on a used workspace differs"


# -- the two work distributions ------------------------------------------------

@pytest.fixture
def mode_env(tuning):
    def set_mode(mode):
        tuning("PKV_ATTN_MODE", mode)
    return set_mode


@pytest.mark.parametrize("mode", [1, 2], ids=["partitions", "balanced"])
@pytest.mark.parametrize("dtype,B,D,Hq,Hkv", [("bf16", 16, 128, 16, 8), ("bf16", 32, 128, 64, 8),
                                              ("bf16", 16, 128, 64, 4), ("bf16", 8, 64, 12, 1),
                                              ("f32", 16, 64, 8, 2)], ids=lambda v: str(v))
def test_modes_match_oracle(mode_env, mode, dtype, B, D, Hq, Hkv):
    mode_env(mode)
    lens = [1, 2, 15, 16, 17, 31, 100, 255, 256, 257, 600, 1000]
    wl = independent_workload(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                              dtype=dtype, seed=31 + Hq)
    step, ost = run_both(wl)
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    assert_gate(gpu_out(step), ref, dtype, f"mode {mode}")


@pytest.mark.parametrize("mode", [2, 3, 4], ids=["balanced", "matrix", "matrix-balanced"])
@pytest.mark.parametrize("scale", [-0.0884, 0.0, 0.75], ids=["negative", "zero", "sharp"])
def test_routes_with_unusual_scales(mode_env, mode, scale):
    """Softmax scales taken as they come ([KVM] §19.2.3 applies the caller's
    scale to q.k): negative (the weights favour the least similar keys), zero
    (uniform weights over the history) and large (a sharp softmax whose
    running reference moves often), on the vector balanced split and both
    matrix-core routes, every element against the oracle."""
    mode_env(mode)
    lens = [1, 17, 32, 33, 300, 1000, 2047]
    wl = independent_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                              dtype="bf16", seed=140 + mode, scale=scale)
    step, ost = run_both(wl)
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    say("  gate", assert_gate(gpu_out(step), ref, "bf16", f"mode {mode} scale {scale}"))


MBAL = [  # B, Hq, Hkv
    (16, 16, 8), (16, 32, 8), (32, 64, 8), (8, 32, 2), (16, 128, 8), (64, 24, 4), (32, 128, 16),
]


@pytest.mark.parametrize("B,Hq,Hkv", MBAL, ids=lambda v: str(v))
def test_matrix_balanced_route_matches_oracle(mode_env, B, Hq, Hkv):
    """The balanced split on the matrix cores (PKV_ATTN_MODE=4; the default
    for 2 to 16 heads per group at head_dim 128 with automatic partitions)
    on bf16 pools: ragged lengths from 1 to a few thousand (streams cut by
    many intervals, streams inside one), every element against the oracle;
    then the two phases in separate calls give the same bits."""
    mode_env(4)
    lens = [1, 2, 31, 32, 33, 100, 257, 600, 1000, 2500, 4100, 17]
    wl = independent_workload(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                              block_size=B, dtype="bf16", seed=90 + B + Hq)
    step, ost = run_both(wl)
    say(f"  split {step.split}")
    assert step.split["mode"] == "matrix-balanced"
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    one = host_bits(step.out)
    say("  gate", assert_gate(to_f64(one), ref, "bf16", "matrix-balanced"))
    out = torch.empty_like(step.q)
    step.attention(out=out, phases=1)
    step.attention(out=out, phases=2)
    torch.cuda.synchronize()
    assert np.array_equal(one, host_bits(out))


def test_balanced_stream_across_more_than_1024_shares(mode_env):
    """One long sequence and one KV head: every wave group holds a piece of the
    same stream, so the merge folds more than 1024 pieces."""
    mode_env(2)
    wl = independent_workload([40000], num_q_heads=4, num_kv_heads=1, head_dim=128,
                              block_size=16, dtype="bf16", seed=77)
    step, ost = run_both(wl)
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    assert_gate(gpu_out(step), ref, "bf16", "one stream, many shares")


def test_balanced_many_short_sequences(mode_env):
    """Far fewer tiles than wave groups (every share a single tile)."""
    mode_env(2)
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 40, size=300)
    wl = independent_workload(lens, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                              dtype="bf16", seed=12)
    step, ost = run_both(wl)
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                           wl.scale)
    assert_gate(gpu_out(step), ref, "bf16", "many short")
