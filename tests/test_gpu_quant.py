"""GPU parity of the quantized-cache path (FP8 e4m3, per-token INT8) through the
C ABI against the quantized oracle (oracle/quant.py, oracle/replay.py).

Codes and INT8 scales: bit-exact full pools after the quantizing write and the
copy-on-write copies.  Attention: the gate of tests/parity.py against the fp64
attention over the dequantized pools.  The one-position cases pin the device's
e4m3 decoding to the format's value table exactly: an output over a single
position is that position's dequantized V row, which bf16 holds exactly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import quant  # noqa: E402
from oracle.replay import run_step_quant  # noqa: E402
from tests.parity import assert_gate  # noqa: E402
from workloads import config_workload, independent_workload, shared_prefix_workload  # noqa: E402

pytestmark = pytest.mark.gpu

KINDS = [quant.FP8, quant.INT8]


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()
    return torch.device("cuda:0")


def run_both(wl, kind, partition_tokens=None, k_scale=1.0, v_scale=1.0, attention=True):
    from paged_attention_slot_amd.runtime import DecodeStep
    say(f"  case {wl.name} {kind}: N={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"B={wl.block_size} maxlen={wl.max_seq_len} pt={partition_tokens} seed={wl.seed}")
    step = DecodeStep(wl, partition_tokens=partition_tokens, kv_dtype=kind, k_scale=k_scale,
                      v_scale=v_scale)
    step.copy()
    step.write()
    if attention:
        step.attention()
    torch.cuda.synchronize()
    ost = run_step_quant(wl, kind, k_scale, v_scale)
    assert np.array_equal(step.block_tables_h, ost.block_tables)
    return step, ost


def bits(t):
    from paged_attention_slot_amd.runtime import to_host_bits
    return to_host_bits(t)


def check_pools(step, ost):
    assert np.array_equal(bits(step.k_cache), ost.k_pool), "K codes differ"
    assert np.array_equal(bits(step.v_cache), ost.v_pool), "V codes differ"
    if ost.k_scales is not None:
        assert np.array_equal(bits(step.k_scale_pools[0]), ost.k_scales), "K scales differ"
        assert np.array_equal(bits(step.v_scale_pools[0]), ost.v_scales), "V scales differ"


def gpu_out(step):
    from oracle.attention import to_f64
    return to_f64(bits(step.out))


LENS = [1, 7, 16, 17, 33, 100, 255, 300]
SHAPES = [(16, 128, 16, 8), (16, 128, 32, 8), (32, 128, 64, 8), (8, 128, 8, 8),
          (16, 128, 16, 1), (64, 128, 12, 4)]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("B,D,Hq,Hkv", SHAPES, ids=lambda v: str(v))
def test_small_write_and_attention(kind, B, D, Hq, Hkv):
    wl = independent_workload(LENS, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                              dtype="bf16", seed=200 + B + Hq)
    step, ost = run_both(wl, kind)
    check_pools(step, ost)
    r = assert_gate(gpu_out(step), ost.attention(), "bf16", f"{kind} {wl.name}")
    say("  gate", r)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mode", [1, 2, 4], ids=["partitions", "balanced", "matrix-balanced"])
def test_modes_and_splits(kind, mode, tuning):
    tuning("PKV_ATTN_MODE", mode)
    wl = independent_workload([1, 2, 15, 16, 17, 31, 100, 256, 257, 600, 1000], num_q_heads=32,
                              num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", seed=41)
    step, ost = run_both(wl, kind, partition_tokens=64 if mode == 1 else 0)
    say(f"  split {step.split}")
    assert_gate(gpu_out(step), ost.attention(), "bf16", f"{kind} mode {mode}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mode", [2, 3, 4], ids=["balanced", "matrix", "matrix-balanced"])
@pytest.mark.parametrize("scale", [-0.0884, 0.75], ids=["negative", "sharp"])
def test_unusual_softmax_scales(kind, mode, scale, tuning):
    """A negative softmax scale and one large enough that the running
    references move often, over one-byte caches (the FP8 tensor scale and the
    INT8 per-slot key scales folded into the exponents) on the vector and both
    matrix-core routes."""
    tuning("PKV_ATTN_MODE", mode)
    wl = independent_workload([1, 17, 33, 300, 1000, 2047], num_q_heads=32, num_kv_heads=8,
                              head_dim=128, block_size=16, dtype="bf16", seed=47, scale=scale)
    step, ost = run_both(wl, kind, k_scale=0.5 if kind == "fp8_e4m3" else 1.0)
    say("  gate", assert_gate(gpu_out(step), ost.attention(), "bf16", f"{kind} mode {mode}"))


def test_fp8_scales_other_than_one():
    wl = independent_workload([5, 40, 129], num_q_heads=16, num_kv_heads=4, head_dim=128,
                              block_size=16, dtype="bf16", seed=43)
    step, ost = run_both(wl, quant.FP8, k_scale=0.25, v_scale=3.0)
    check_pools(step, ost)
    assert_gate(gpu_out(step), ost.attention(), "bf16", "fp8 scales")


@pytest.mark.parametrize("kind", KINDS)
def test_copy_on_write_family(kind):
    wl = shared_prefix_workload(prefix_tokens=64, suffix_lens=[3, 16, 7, 1, 12, 30, 9],
                                forking_parents=4, samples_per_fork=4, num_q_heads=16,
                                num_kv_heads=4, head_dim=128, block_size=16, dtype="bf16", seed=6)
    step, ost = run_both(wl, kind)
    assert len(ost.cow_pairs) == 12
    check_pools(step, ost)
    assert_gate(gpu_out(step), ost.attention(), "bf16", f"{kind} cow family")


def test_e4m3_decoding_matches_the_format_table_exactly():
    """Every finite code appears as a V value of a one-position sequence: the
    output must equal e4m3_values()[code] * v_scale exactly."""
    from paged_attention_slot_amd import ops
    dev = torch.device("cuda:0")
    vals = quant.e4m3_values()
    codes = np.array([c for c in range(256) if not np.isnan(vals[c])], dtype=np.uint8)  # 254
    H, D, B = 2, 128, 16
    N = 2                                   # 2 sequences x 2 heads x 128 = 512 >= 254 values
    nb = 4
    v_rows = np.resize(codes, (N, H, D)).astype(np.uint8)
    k_rows = np.full((N, H, D), 0x38, np.uint8)                          # 1.0
    kc = torch.zeros((nb, B, H, D), dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
    vc = torch.zeros_like(kc)
    slots = torch.tensor([0, B], dtype=torch.int32, device=dev)          # position 0 of blocks 0, 1
    ops.write(torch.from_numpy(k_rows).to(dev).view(torch.float8_e4m3fn),
              torch.from_numpy(v_rows).to(dev).view(torch.float8_e4m3fn), slots, kc, vc)
    q = torch.ones((N, 2 * H, D), dtype=torch.bfloat16, device=dev)
    tables = torch.tensor([[0, -1], [1, -1]], dtype=torch.int32, device=dev)
    lens = torch.tensor([1, 1], dtype=torch.int32, device=dev)
    for vs in (1.0, 0.5):
        out = ops.attention_decode_quant(q, kc, vc, tables, lens, 0.1, 1.0, vs)
        torch.cuda.synchronize()
        got = bits(out).astype(np.uint32) << 16
        got = got.view(np.float32).astype(np.float64)
        want = np.repeat(vals[v_rows] * vs, 2, axis=1)   # query heads 2g, 2g+1 read KV head g
        assert np.array_equal(got, want)


def test_int8_one_position_is_code_times_scale():
    """One position, at offset 0 of block 2: the output is that slot's V codes
    times its scale (powers of two, so bf16 holds the result exactly).  The
    other slots of the tile hold NaN scales: masked positions must not read
    them into the result."""
    from paged_attention_slot_amd import ops
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(9)
    H, D, B, nb = 2, 128, 8, 4
    slot = 2 * B
    v_row = rng.integers(-127, 128, (H, D)).astype(np.int8)
    kc = torch.zeros((nb, B, H, D), dtype=torch.int8, device=dev)
    vc = torch.zeros_like(kc)
    kc.view(-1, H, D)[slot] = 1
    vc.view(-1, H, D)[slot] = torch.from_numpy(v_row).to(dev)
    vs = (2.0 ** rng.integers(-8, -3, H)).astype(np.float32)
    ks = torch.ones((nb * B, H), dtype=torch.float32, device=dev)
    vsp = torch.full((nb * B, H), float("nan"), dtype=torch.float32, device=dev)  # unread slots
    vsp[slot] = torch.from_numpy(vs).to(dev)
    q = torch.ones((1, 2 * H, D), dtype=torch.bfloat16, device=dev)
    tables = torch.tensor([[2, 0]], dtype=torch.int32, device=dev)
    lens = torch.tensor([1], dtype=torch.int32, device=dev)
    out = ops.attention_decode_quant(q, kc, vc, tables, lens, 0.1, k_scales=ks, v_scales=vsp)
    torch.cuda.synchronize()
    got = (bits(out).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = np.repeat(v_row.astype(np.float64)[None] * vs[None, :, None], 2, axis=1)
    assert np.array_equal(got, want)


# -- full-size configuration, in the bench's launch configuration -------------

@pytest.mark.parametrize("kind", KINDS)
def test_qwen_layer_full(kind):
    wl = config_workload("qwen3-0.6b-layer")
    step, ost = run_both(wl, kind)
    check_pools(step, ost)
    r = assert_gate(gpu_out(step), ost.attention(), "bf16", f"{kind} qwen layer")
    say("  gate", r)
