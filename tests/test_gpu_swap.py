"""GPU parity of block swap (pkv_bm_swap_out/in + pkv_swap_out/in) through the
C ABI against the oracle.

Pause-and-resume traces (workloads.preemption_workload) run through the
runtime: the library's manager makes the pairs, the swap kernel moves the
blocks between the HBM pools and a pinned host pool, the residents' growth
overwrites the released blocks, and the resumed sequences decode.  Device
pools and host pools must equal the oracle's bit for bit; attention must pass
the gate of tests/parity.py.  Every case prints its shape and seed first."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import quant  # noqa: E402
from oracle.cache_ops import swap_blocks  # noqa: E402
from oracle.replay import run_step, run_step_quant  # noqa: E402
from tests.parity import assert_gate  # noqa: E402
from workloads import preemption_config_workload, preemption_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()


def bits(t):
    from paged_attention_slot_amd.runtime import to_host_bits
    return to_host_bits(t)


def run_trace(wl, kind=None, attention=True):
    from paged_attention_slot_amd.runtime import DecodeStep
    say(f"  case {wl.name} kv={kind or wl.dtype}: N={wl.num_seqs} Hq={wl.num_q_heads} "
        f"Hkv={wl.num_kv_heads} D={wl.head_dim} B={wl.block_size} blocks={wl.num_blocks} "
        f"host={wl.num_host_blocks} seed={wl.seed}")
    step = DecodeStep(wl, kv_dtype=kind)
    step.copy()
    step.write()
    if attention:
        step.attention()
    torch.cuda.synchronize()
    ost = run_step_quant(wl, kind) if kind else run_step(wl, keep_values=False)
    assert np.array_equal(step.block_tables_h, ost.block_tables)
    assert len(step.swap_events) == len(ost.swaps)
    for (k0, p0), (k1, p1) in zip(step.swap_events, ost.swaps):
        assert k0 == k1 and np.array_equal(p0, np.asarray(p1, np.int32).reshape(-1, 2))
    return step, ost


def check_pools(step, ost):
    assert np.array_equal(bits(step.k_cache), ost.k_pool), "device K differs"
    assert np.array_equal(bits(step.v_cache), ost.v_pool), "device V differs"
    assert np.array_equal(bits(step.host.k), ost.k_host), "host K differs"
    assert np.array_equal(bits(step.host.v), ost.v_host), "host V differs"
    if getattr(ost, "k_scales", None) is not None:
        assert np.array_equal(bits(step.k_scale_pools[0]), ost.k_scales)
        assert np.array_equal(bits(step.v_scale_pools[0]), ost.v_scales)
        assert np.array_equal(bits(step.host.k_scales), ost.k_scales_host)
        assert np.array_equal(bits(step.host.v_scales), ost.v_scales_host)


def out_f64(step):
    from oracle.attention import to_f64
    return to_f64(bits(step.out))


TRACES = {
    "latecomers": dict(lens_before=[20, 7, 33, 16, 9, 130, 64], swapped=[4, 5, 6],
                       grow=[13, 30, 5, 40, 0, 0, 0]),
    "fork-pair": dict(lens_before=[18, 11, 30], forks=[0], swapped=[0, 3], grow=[0, 21, 9, 0]),
    "fork-child": dict(lens_before=[18, 11], forks=[0], swapped=[2], grow=[6, 3, 0]),
    "all": dict(lens_before=[5, 12, 1, 8, 300], swapped=[0, 1, 2, 3, 4], grow=[0] * 5),
}
SHAPES = [  # Hq, Hkv, D, B, dtype
    (16, 8, 128, 16, "bf16"), (8, 2, 64, 16, "f32"), (32, 8, 128, 32, "bf16"),
    (16, 1, 128, 8, "bf16"), (12, 4, 64, 64, "bf16"), (8, 8, 128, 8, "f32"),
]


@pytest.mark.parametrize("trace", sorted(TRACES))
@pytest.mark.parametrize("Hq,Hkv,D,B,dt", SHAPES, ids=lambda v: str(v))
def test_preemption_traces(trace, Hq, Hkv, D, B, dt):
    wl = preemption_workload(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                             dtype=dt, seed=70 + B + D, name=f"preempt-{trace}",
                             **TRACES[trace])
    step, ost = run_trace(wl)
    check_pools(step, ost)
    assert_gate(out_f64(step), ost.attention(), dt, f"{trace} {wl.name}")


@pytest.mark.parametrize("kind", [quant.FP8, quant.INT8])
@pytest.mark.parametrize("trace", ["latecomers", "fork-pair"])
def test_preemption_traces_quantized(kind, trace):
    wl = preemption_workload(num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                             dtype="bf16", seed=91, name=f"preempt-{trace}", **TRACES[trace])
    step, ost = run_trace(wl, kind)
    check_pools(step, ost)
    assert_gate(out_f64(step), ost.attention(), "bf16", f"{kind} {trace}")


def direct_case(seed, nb, nh, shape, dtype):
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    from paged_attention_slot_amd import ops
    host = ops.HostPool(nh, torch.empty((1,) + shape, dtype=dtype, device=dev))
    if dtype == torch.int8:
        vals = lambda n: rng.integers(-127, 128, (n,) + shape).astype(np.int8)  # noqa: E731
    else:
        vals = lambda n: rng.integers(0, 2**16, (n,) + shape).astype(np.uint16)  # noqa: E731
    k = vals(nb)
    v = vals(nb)
    hk0, hv0 = vals(nh), vals(nh)
    tdev = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)  # noqa
    kc = tdev(k).to(dev).view(dtype)
    vc = tdev(v).to(dev).view(dtype)
    host.k.copy_(tdev(hk0).view(dtype))
    host.v.copy_(tdev(hv0).view(dtype))
    return rng, host, k, v, hk0, hv0, kc, vc


def test_direct_pairs_out_of_range_are_skipped():
    """Arbitrary pair lists, a repeated source, pairs naming blocks outside
    either pool (skipped), pairs in pinned host memory, empty lists."""
    from paged_attention_slot_amd import ops
    shape = (16, 2, 64)
    rng, host, k, v, hk0, hv0, kc, vc = direct_case(5, 40, 24, shape, torch.bfloat16)
    valid = [(3, 0), (17, 5), (3, 9), (39, 23), (0, 1)]
    bad = [(40, 2), (-1, 3), (5, 24), (6, -7)]
    pairs = np.asarray(valid + bad, np.int32)
    say(f"  swap_out {len(valid)} valid + {len(bad)} skipped pairs")
    ops.swap_out(torch.from_numpy(pairs).cuda(), kc, vc, host)
    torch.cuda.synchronize()
    hk, hv = hk0.copy(), hv0.copy()
    swap_blocks(valid, k, hk)
    swap_blocks(valid, v, hv)
    assert np.array_equal(bits(host.k), hk) and np.array_equal(bits(host.v), hv)
    # back into other device blocks, with the pairs in pinned host memory
    back = np.asarray([(23, 30), (5, 2), (0, 7)] + [(24, 0), (1, 40)], np.int32)
    pinned = torch.from_numpy(back).pin_memory()
    ops.swap_in(pinned, host, kc, vc)
    torch.cuda.synchronize()
    swap_blocks(back[:3], hk, k)
    swap_blocks(back[:3], hv, v)
    assert np.array_equal(bits(kc), k) and np.array_equal(bits(vc), v)
    ops.swap_in(torch.empty((0, 2), dtype=torch.int32, device="cuda"), host, kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), k)


@pytest.mark.parametrize("B,H,D", [(16, 8, 128), (64, 8, 128), (1, 1, 128), (8, 1, 64),
                                   (32, 2, 128)])
def test_direct_block_sizes(B, H, D):
    """Blocks of 256 B to 256 KiB: whole rounds of the kernel and a partial
    last round."""
    from paged_attention_slot_amd import ops
    shape = (B, H, D)
    rng, host, k, v, hk0, hv0, kc, vc = direct_case(B + H, 50, 50, shape, torch.bfloat16)
    pairs = np.stack([rng.permutation(50)[:37], rng.permutation(50)[:37]], 1).astype(np.int32)
    say(f"  B={B} H={H} D={D} block bytes={B * H * D * 2} pairs={len(pairs)}")
    ops.swap_out(torch.from_numpy(pairs).cuda(), kc, vc, host)
    torch.cuda.synchronize()
    swap_blocks(pairs, k, hk0)
    swap_blocks(pairs, v, hv0)
    assert np.array_equal(bits(host.k), hk0) and np.array_equal(bits(host.v), hv0)


def test_int8_scale_pools_move_with_their_blocks():
    from paged_attention_slot_amd import ops
    shape = (16, 4, 128)
    rng, host, k, v, hk0, hv0, kc, vc = direct_case(8, 20, 12, shape, torch.int8)
    ks = rng.random((20 * 16, 4)).astype(np.float32)
    vs = rng.random((20 * 16, 4)).astype(np.float32)
    kst, vst = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    pairs = np.asarray([(4, 11), (19, 0), (7, 6)], np.int32)
    say("  int8 pools with scales, 3 pairs")
    ops.swap_out(torch.from_numpy(pairs).cuda(), kc, vc, host, kst, vst)
    torch.cuda.synchronize()
    hks = np.zeros((12 * 16, 4), np.float32)
    hvs = np.zeros_like(hks)
    swap_blocks(pairs, ks.reshape(20, 16, 4), hks.reshape(12, 16, 4))
    swap_blocks(pairs, vs.reshape(20, 16, 4), hvs.reshape(12, 16, 4))
    swap_blocks(pairs, k, hk0)
    assert np.array_equal(bits(host.k), hk0)
    assert np.array_equal(bits(host.k_scales), hks) and np.array_equal(bits(host.v_scales), hvs)


def test_memory_kinds_are_checked_on_the_host():
    """Pageable host memory, or device memory given as the host pool, is
    refused before any launch."""
    from paged_attention_slot_amd import _lib, lib, ops
    from paged_attention_slot_amd._lib import PkvHostPool
    kc = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pairs = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    pageable = np.zeros(4 * 16 * 2 * 64 * 2 + 64, np.uint8)
    addr = (pageable.ctypes.data + 15) // 16 * 16
    g = ops.geom_of(kc)
    for hk, what in ((addr, "host k"), (kc.data_ptr(), "pinned host")):
        hp = PkvHostPool(4, ctypes.c_void_p(hk), ctypes.c_void_p(hk), None, None)
        st = lib().pkv_swap_out(ctypes.c_void_p(pairs.data_ptr()), 1, ctypes.c_void_p(kc.data_ptr()),
                                ctypes.c_void_p(vc.data_ptr()), None, ctypes.byref(hp),
                                ctypes.byref(g), None)
        assert st == _lib.PKV_ERR_INVALID_ARG
        assert what in lib().pkv_last_error().decode()
    host = ops.HostPool(4, kc)
    st = lib().pkv_swap_out(ctypes.c_void_p(addr), 1, ctypes.c_void_p(kc.data_ptr()),
                            ctypes.c_void_p(vc.data_ptr()), None, ctypes.byref(host.struct()),
                            ctypes.byref(g), None)
    assert st == _lib.PKV_ERR_INVALID_ARG          # pageable pairs
    torch.cuda.synchronize()


def test_qwen_layer_preemption_full():
    """The swap measurement's own trace (the qwen3-0.6b layer shape, the latest
    quarter of the sequences paused), in the launch configuration it times."""
    wl = preemption_config_workload("qwen3-0.6b-layer")
    step, ost = run_trace(wl)
    check_pools(step, ost)
    r = assert_gate(out_f64(step), ost.attention(), "bf16", "qwen preempt")
    say("  gate", r)
