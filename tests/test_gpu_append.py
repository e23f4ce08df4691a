"""GPU parity of pkv_attention_decode_append (the step's KV append folded into
the decode attention) through the C ABI.

Against the oracle: the pools after the call bit-exact with the oracle's write
(full pools), the attention within the gate of the oracle's decode attention.
Against the library's own unfused step (pkv_write, then pkv_attention_decode
on a second copy of the pools): bit-identical outputs, since the new token
enters the same arithmetic with the same bits.  Cases: all five workload
configurations in the launch configuration the bench times (balanced split,
and the long-context configuration's fixed partitions), small families over
dtypes, block sizes 8-64, head dims and group sizes (two waves per KV head at
G = 8), explicit partitions, and hand-built edge cases (skipped slots,
sequences with an empty history, lengths beyond max_seq_len).  Every case
prints its shape first."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.attention import attention_decode as oracle_attention  # noqa: E402
from oracle.attention import to_f64  # noqa: E402
from oracle.replay import run_step  # noqa: E402
from tests.parity import assert_gate  # noqa: E402
from workloads import config_workload, independent_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()


def bits(t):
    from paged_attention_slot_amd.runtime import to_host_bits
    return to_host_bits(t)


def fused_vs_unfused(wl, partition_tokens=None):
    """Fused step on the runtime's pools (layer 0), unfused step on a copy
    (layer 1, identical tables); returns both outputs and the step."""
    from paged_attention_slot_amd.runtime import DecodeStep
    say(f"  case {wl.name}: N={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"D={wl.head_dim} B={wl.block_size} {wl.dtype} maxlen={wl.max_seq_len} "
        f"pt={partition_tokens} seed={wl.seed}")
    step = DecodeStep(wl, layers=2, partition_tokens=partition_tokens)
    step.copy(0)
    fused = step.attention_append(0, out=torch.empty_like(step.q))
    step.copy(1)
    step.write(1)
    plain = step.attention(1, out=torch.empty_like(step.q))
    torch.cuda.synchronize()
    return bits(fused), bits(plain), step


def check_against_oracle(wl, step, fused):
    ost = run_step(wl, keep_values=False)
    assert np.array_equal(bits(step.k_caches[0]), ost.k_pool), "K pool differs from the oracle's"
    assert np.array_equal(bits(step.v_caches[0]), ost.v_pool), "V pool differs from the oracle's"
    ref = oracle_attention(wl.q, ost.k_pool, ost.v_pool, ost.block_tables, ost.seq_lens, wl.scale)
    say("  gate", assert_gate(to_f64(fused), ref, wl.dtype, wl.name))


@pytest.mark.parametrize("name", ["tiny", "qwen3-0.6b-layer", "llama3-8b-layer",
                                  "shared-prefix-cow", "llama3.1-70b-longctx"])
def test_configs(name):
    wl = config_workload(name)
    fused, plain, step = fused_vs_unfused(wl)
    say(f"  split {step.split}")
    assert np.array_equal(fused, plain), "fused and unfused outputs differ"
    assert np.array_equal(bits(step.k_caches[0]), bits(step.k_caches[1]))
    assert np.array_equal(bits(step.v_caches[0]), bits(step.v_caches[1]))
    if name in ("tiny", "qwen3-0.6b-layer", "shared-prefix-cow"):
        check_against_oracle(wl, step, fused)


LENS = [1, 7, 8, 9, 16, 17, 33, 100, 255, 300]
SMALL = [
    # dtype, B, D, Hq, Hkv, partition_tokens (None: balanced)
    ("bf16", 16, 128, 16, 8, None),
    ("bf16", 8, 128, 64, 8, None),     # G = 8: two waves per KV head, blocks of 8
    ("bf16", 64, 64, 12, 4, None),
    ("bf16", 32, 128, 32, 4, 64),      # fixed partitions
    ("bf16", 8, 64, 16, 2, 16),
    ("f32", 16, 64, 8, 2, None),
    ("f32", 8, 128, 6, 2, 32),
]


@pytest.mark.parametrize("dtype,B,D,Hq,Hkv,pt", SMALL, ids=lambda v: str(v))
def test_small_families(dtype, B, D, Hq, Hkv, pt):
    wl = independent_workload(LENS, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                              dtype=dtype, seed=300 + B + D + Hq)
    fused, plain, step = fused_vs_unfused(wl, partition_tokens=pt)
    assert np.array_equal(fused, plain)
    check_against_oracle(wl, step, fused)


@pytest.mark.parametrize("Hq", [4, 16])
def test_edge_cases(Hq):
    """Hand-built call: sequence 1 has an empty history (nothing written,
    zeros out), sequence 2's slot is -1 (nothing written: its newest position
    is read from the pool, as after a skipped pkv_write), sequence 3 is longer
    than max_seq_len (no new position: nothing written, the attention covers
    max_seq_len positions of the pool).  Run with 2 and with 8 query heads per
    KV head (the append folded into the attention kernel, and the copy kernel
    launched first)."""
    from paged_attention_slot_amd import ops
    rng = np.random.default_rng(5)
    nb, B, Hkv, D = 12, 16, 2, 128
    say(f"  case edge: Hq={Hq} Hkv={Hkv}")
    dev = torch.device("cuda:0")

    def bf(shape):
        u = rng.normal(0, 1, shape).astype(np.float32).view(np.uint32)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)

    def t(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    kp, vp = bf((nb, B, Hkv, D)), bf((nb, B, Hkv, D))
    q, kn, vn = bf((4, Hq, D)), bf((4, Hkv, D)), bf((4, Hkv, D))
    tables = np.array([[3, 5, 7], [-1, -1, -1], [1, 2, -1], [8, 9, 10]], np.int32)
    lens = np.array([40, 0, 20, 48], np.int32)
    max_len = 40
    slots = np.array([7 * B + 7, 4 * B, -1, 10 * B + 15], np.int32)
    k_cache, v_cache = t(kp), t(vp)
    out = ops.attention_decode_append(t(q), t(kn), t(vn), torch.from_numpy(slots).to(dev),
                                      k_cache, v_cache, torch.from_numpy(tables).to(dev),
                                      torch.from_numpy(lens).to(dev), 1 / np.sqrt(D),
                                      max_seq_len=max_len)
    torch.cuda.synchronize()
    # the pool: only sequence 0's slot changed
    ek, ev = kp.copy(), vp.copy()
    ek.reshape(-1, Hkv, D)[slots[0]] = kn[0]
    ev.reshape(-1, Hkv, D)[slots[0]] = vn[0]
    assert np.array_equal(bits(k_cache), ek) and np.array_equal(bits(v_cache), ev)
    # the attention: the oracle over the expected pools, sequence 3 cut at
    # max_seq_len
    ref = oracle_attention(q, ek, ev, tables, np.minimum(lens, max_len), 1 / np.sqrt(D))
    got = to_f64(bits(out))
    assert_gate(got, ref, "bf16", "edge cases")
    assert not got[1].any()


def test_quantized_pools_are_refused():
    from paged_attention_slot_amd import ops
    dev = torch.device("cuda:0")
    kc = torch.zeros((4, 16, 1, 128), dtype=torch.float8_e4m3fn, device=dev)
    with pytest.raises(TypeError):
        ops.attention_decode_append(torch.zeros((1, 1, 128), dtype=torch.bfloat16, device=dev),
                                    kc, kc, torch.zeros(1, dtype=torch.int32, device=dev), kc, kc,
                                    torch.zeros((1, 1), dtype=torch.int32, device=dev),
                                    torch.ones(1, dtype=torch.int32, device=dev), 1.0)
