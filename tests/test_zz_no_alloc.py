"""pkv_attention_decode_noalloc (the library's own device scratch as the
workspace, nothing allocated) through the C ABI, against pkv_attention_decode
with a caller's workspace: two calls in a row, the second with a smaller batch
(the scratch still holds the first call's pieces), give the bits of the
workspace entry point; both are also within the gate of the oracle.  Then
batches of eight heads per group on both matrix-core routes and an fp32
batch.  Every case prints its shape first."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.attention import attention_decode, to_f64  # noqa: E402
from oracle.replay import run_step  # noqa: E402
from tests.parity import assert_gate  # noqa: E402
from workloads import config_workload, independent_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()


def prepared(wl):
    from paged_attention_slot_amd.runtime import DecodeStep
    say(f"  case {wl.name}: N={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"D={wl.head_dim} B={wl.block_size} maxlen={wl.max_seq_len}")
    step = DecodeStep(wl)
    step.copy()
    step.write()
    ref_ws = step.attention(out=torch.empty_like(step.q))   # the workspace entry point
    torch.cuda.synchronize()
    return step, ref_ws


def noalloc(step):
    from paged_attention_slot_amd import ops
    out = torch.full_like(step.q, 7.0)
    return ops.attention_decode_noalloc(step.q, step.k_cache, step.v_cache, step.block_tables,
                                        step.seq_lens, step.wl.scale, out,
                                        max_seq_len=step.max_seq_len)


def bits(t):
    from paged_attention_slot_amd.runtime import to_host_bits
    return to_host_bits(t)


def test_noalloc_twice_matches_the_workspace_entry_point():
    big = config_workload("qwen3-0.6b-layer")
    small = independent_workload([1, 17, 300, 33, 2000, 5], num_q_heads=16, num_kv_heads=8,
                                 head_dim=128, block_size=16, dtype="bf16", seed=71,
                                 name="ragged-small")
    s1, r1 = prepared(big)
    s2, r2 = prepared(small)
    say(f"  routes {s1.split} / {s2.split}")
    o1 = noalloc(s1)   # two calls in a row on the one scratch,
    o2 = noalloc(s2)   # the second smaller
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(r1)), "first call differs from pkv_attention_decode"
    assert np.array_equal(bits(o2), bits(r2)), "second call differs from pkv_attention_decode"
    for wl, o in ((big, o1), (small, o2)):
        ost = run_step(wl, keep_values=False)
        ref = attention_decode(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens,
                               wl.scale)
        say("  gate", assert_gate(to_f64(bits(o)), ref, "bf16", wl.name))


@pytest.mark.parametrize("mode", [0, 3], ids=["default", "matrix-route"])
def test_noalloc_eight_heads_per_group_and_f32(mode, tuning):
    """Eight query heads per KV head on the default route (the balanced
    split on the matrix cores) and on the matrix-core route with fixed
    partitions (PKV_ATTN_MODE=3), then an fp32 batch."""
    tuning("PKV_ATTN_MODE", mode)
    cases = [independent_workload([1, 15, 200, 1500, 64], num_q_heads=64, num_kv_heads=8,
                                  head_dim=128, block_size=16, dtype="bf16", seed=72,
                                  name="eight-heads-per-group"),
             independent_workload([3, 40, 257], num_q_heads=8, num_kv_heads=2, head_dim=64,
                                  block_size=16, dtype="f32", seed=73, name="f32")]
    for wl in cases:
        step, ref_ws = prepared(wl)
        say(f"  route {step.split}")
        o = noalloc(step)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o).view(np.uint32) if wl.dtype == "f32" else bits(o),
                              bits(ref_ws).view(np.uint32) if wl.dtype == "f32" else bits(ref_ws))
