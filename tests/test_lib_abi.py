"""The C-ABI library loads, exports every symbol ``include/pkv.h`` declares,
and rejects bad arguments on the host with the documented status codes
(no GPU: none of these calls reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

pkv = pytest.importorskip("paged_attention_slot_amd")
from paged_attention_slot_amd import _lib  # noqa: E402
from paged_attention_slot_amd._lib import PkvGeom  # noqa: E402

HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))


def test_library_loads():
    lib = pkv.lib()
    assert lib.pkv_version() >= 100


def test_every_declared_symbol_is_exported_and_bound():
    lib = pkv.lib()
    names = declared_symbols()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def g(nb=16, B=16, H=2, D=64, dt=0):
    return PkvGeom(nb, B, H, D, dt)


def last_error():
    return pkv.lib().pkv_last_error().decode()


def test_write_validation():
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)
    assert lib.pkv_write(x, x, x, 1, x, x, None, None) == _lib.PKV_ERR_INVALID_ARG
    assert "geometry" in last_error()
    assert lib.pkv_write(x, x, x, 1, x, x, ctypes.byref(g(B=12)), None) == _lib.PKV_ERR_INVALID_ARG
    assert "power of two" in last_error()
    assert lib.pkv_write(x, x, x, -1, x, x, ctypes.byref(g()), None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_write(x, x, x, 0, x, x, ctypes.byref(g()), None) == _lib.PKV_OK
    bad = ctypes.c_void_p(0x1004)
    assert lib.pkv_write(bad, x, x, 1, x, x, ctypes.byref(g()), None) == _lib.PKV_ERR_INVALID_ARG
    assert "misaligned" in last_error()
    assert lib.pkv_write(None, x, x, 1, x, x, ctypes.byref(g()), None) == _lib.PKV_ERR_INVALID_ARG
    big = g(nb=1 << 27, B=16)
    assert lib.pkv_write(x, x, x, 1, x, x, ctypes.byref(big), None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_write(x, x, x, 1, x, x, ctypes.byref(g(H=1, D=2, dt=1)), None) == \
        _lib.PKV_ERR_INVALID_ARG     # 4-byte rows are not a multiple of 16


def test_copy_validation():
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)
    assert lib.pkv_copy_blocks(x, 0, x, x, ctypes.byref(g()), None) == _lib.PKV_OK
    assert lib.pkv_copy_blocks(x, -2, x, x, ctypes.byref(g()), None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_copy_blocks(None, 3, x, x, ctypes.byref(g()), None) == _lib.PKV_ERR_INVALID_ARG


def test_attention_validation_and_workspace_size():
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)

    def call(geom, N=2, Hq=8, maxlen=100, pt=0, ws=None, wsb=0, scale=0.1, mb=7):
        return lib.pkv_attention_decode(x, x, x, x, mb, x, scale, x, N, Hq, maxlen, pt, ws, wsb,
                                        ctypes.byref(geom), None)

    assert call(g(D=96)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(g(B=4)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(g(), Hq=7) == _lib.PKV_ERR_INVALID_ARG
    assert call(g(), pt=24) == _lib.PKV_ERR_INVALID_ARG
    assert call(g(), scale=float("nan")) == _lib.PKV_ERR_INVALID_ARG
    assert call(g(), N=0) == _lib.PKV_OK
    # phases: 1, 2 or 3, optionally with PKV_KV_SHARED (4)
    for bad in (0, 4, 8, 11):
        assert lib.pkv_attention_decode_phase(bad, x, x, x, x, 7, x, 0.1, x, 2, 8, 100, 0, None,
                                              0, ctypes.byref(g()), None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_attention_decode_phase(7, x, x, x, x, 7, x, 0.1, x, 0, 8, 100, 0, None, 0,
                                          ctypes.byref(g()), None) == _lib.PKV_OK
    # a fixed split needs a workspace
    assert call(g(), maxlen=100, pt=32) == _lib.PKV_ERR_INVALID_ARG
    assert "workspace" in last_error()
    # fixed partitions: N * Hq * P * (D + 2) floats
    n = lib.pkv_attention_workspace_bytes(2, 8, 100, 32, ctypes.byref(g()))
    assert n == 2 * 8 * 4 * (64 + 2) * 4
    # the automatic (balanced) split: (N * H_kv + 8192 shares + 8192 chunks) * G
    # rows of D + 2 floats and the (N + 1) prefix sums rounded up to 256 bytes
    rows = (2 * 2 + 8192 + 8192) * 4
    assert lib.pkv_attention_workspace_bytes(2, 8, 100, 0, ctypes.byref(g())) == \
        rows * (64 + 2) * 4 + 256
    assert lib.pkv_attention_workspace_bytes(2, 8, 100, 24, ctypes.byref(g())) == \
        ctypes.c_size_t(-1).value


@pytest.mark.parametrize("maxlen,B,expect", [(100, 16, 112), (4096, 16, 256), (8192, 16, 512),
                                             (131072, 32, 512), (10, 64, 64), (300, 8, 256)])
def test_automatic_partition_beyond_balanced_limit(maxlen, B, expect):
    """Batches of more than 4096 sequences use fixed partitions; the automatic
    length is 256 up to 4096-long contexts, 512 beyond, no split if one
    partition suffices."""
    lib = pkv.lib()
    got = lib.pkv_attention_partition_tokens(5000, 8, maxlen, ctypes.byref(g(nb=8192, B=B)))
    assert got == expect
    assert got % 16 == 0 and got % B == 0


def test_automatic_plan_is_balanced_for_moderate_batches():
    lib = pkv.lib()
    assert lib.pkv_attention_partition_tokens(256, 32, 8192, ctypes.byref(g(nb=8192, H=8, D=128,
                                                                             dt=1))) == 0


def test_block_manager_errors():
    bm = pkv.BlockManager(2, 4)
    bm.add_seq(1)
    with pytest.raises(pkv.PkvError):
        bm.add_seq(1)
    with pytest.raises(pkv.PkvError):
        bm.fork(9, 10)
    with pytest.raises(pkv.NoFreeBlocks):
        bm.append_slots([1], 9)
    assert bm.num_tokens(1) == 0 and bm.num_free() == 2
    with pytest.raises(pkv.PkvError):
        bm.export([1, 2], 4)
    assert pkv.lib().pkv_bm_create(0, 4, None) is None
    bad = (ctypes.c_int32 * 3)(0, 0, 1)
    assert pkv.lib().pkv_bm_create(3, 4, bad) is None


def test_quantized_entry_points_validate_on_the_host():
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)
    fp8 = g(H=2, D=128, dt=_lib.PKV_FP8_E4M3)
    i8 = g(H=2, D=128, dt=_lib.PKV_INT8)
    bf = g(H=2, D=128, dt=_lib.PKV_BF16)
    sc = _lib.PkvKvScales(1.0, 1.0, None, None)
    # plain calls refuse INT8 pools (scales would be lost) and quantized attention
    assert lib.pkv_write(x, x, x, 1, x, x, ctypes.byref(i8), None) == _lib.PKV_ERR_INVALID_ARG
    assert "pkv_write_quant" in last_error()
    assert lib.pkv_copy_blocks(x, 1, x, x, ctypes.byref(i8), None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_attention_decode(x, x, x, x, 7, x, 0.1, x, 2, 8, 100, 0, x, 1 << 30,
                                    ctypes.byref(fp8), None) == _lib.PKV_ERR_INVALID_ARG
    assert "pkv_attention_decode_quant" in last_error()
    # the quantized calls refuse model-dtype pools, other head sizes, bad scales
    assert lib.pkv_write_quant(x, x, x, 1, x, x, ctypes.byref(sc), ctypes.byref(bf), None) == \
        _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_write_quant(x, x, x, 1, x, x, ctypes.byref(sc),
                               ctypes.byref(g(H=2, D=64, dt=_lib.PKV_FP8_E4M3)), None) == \
        _lib.PKV_ERR_UNSUPPORTED
    bad = _lib.PkvKvScales(0.0, 1.0, None, None)
    assert lib.pkv_write_quant(x, x, x, 1, x, x, ctypes.byref(bad), ctypes.byref(fp8), None) == \
        _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_write_quant(x, x, x, 1, x, x, ctypes.byref(sc), ctypes.byref(i8), None) == \
        _lib.PKV_ERR_INVALID_ARG               # INT8 needs scale pools
    assert lib.pkv_write_quant(x, x, x, 0, x, x, ctypes.byref(sc), ctypes.byref(fp8), None) == \
        _lib.PKV_OK
    assert lib.pkv_copy_blocks_quant(x, 1, x, x, ctypes.byref(sc), ctypes.byref(i8), None) == \
        _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_copy_blocks_quant(x, 0, x, x, None, ctypes.byref(fp8), None) == _lib.PKV_OK

    def attn(geom, scales):
        return lib.pkv_attention_decode_quant(3, x, x, x, scales, x, 7, x, 0.1, x, 2, 8, 100, 0,
                                              x, 1 << 30, ctypes.byref(geom), None)
    assert attn(bf, ctypes.byref(sc)) == _lib.PKV_ERR_INVALID_ARG
    assert attn(fp8, None) == _lib.PKV_ERR_INVALID_ARG
    assert attn(i8, ctypes.byref(sc)) == _lib.PKV_ERR_INVALID_ARG      # null scale pools
    # workspace sizing takes the quantized geometry like any other
    assert lib.pkv_attention_workspace_bytes(2, 8, 100, 0, ctypes.byref(fp8)) == \
        lib.pkv_attention_workspace_bytes(2, 8, 100, 0, ctypes.byref(bf))


def test_multi_token_entry_point_validates_on_the_host():
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)
    bf = g(H=2, D=128, dt=_lib.PKV_BF16)

    def call(geom, Hq=8, total=4, maxq=2, pt=0, ws=None, wsb=0):
        return lib.pkv_attention_multi(x, x, x, x, x, 7, x, 0.1, x, 2, Hq, total, maxq, 100, pt,
                                       ws, wsb, ctypes.byref(geom), None)
    assert call(g(H=2, D=128, dt=_lib.PKV_F32)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(g(H=2, D=96, dt=_lib.PKV_BF16)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(bf, Hq=7) == _lib.PKV_ERR_INVALID_ARG
    assert call(bf, pt=48) == _lib.PKV_ERR_INVALID_ARG       # not a multiple of 32
    assert call(bf, total=0) == _lib.PKV_OK
    # a split needs a workspace of the size the sizing call reports
    n = lib.pkv_attention_multi_workspace_bytes(2, 8, 4, 2, 100, 32, ctypes.byref(bf))
    assert n == 4 * 8 * 4 * (128 * 4 + 8) + 4 * 8 * 4          # rows * parts * (acc + ml) + np
    assert call(bf, pt=32) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_attention_multi_workspace_bytes(2, 8, 4, 2, 100, 0, ctypes.byref(bf)) == 0


def test_swap_entry_points_validate_on_the_host():
    from paged_attention_slot_amd._lib import PkvHostPool, PkvKvScales
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)
    hp = PkvHostPool(8, x, x, None, None)
    for fn, args in ((lib.pkv_swap_out, lambda n, h, geo: (x, n, x, x, None, h, geo, None)),
                     (lib.pkv_swap_in, lambda n, h, geo: (x, n, h, x, x, None, geo, None))):
        assert fn(*args(1, ctypes.byref(hp), None)) == _lib.PKV_ERR_INVALID_ARG
        assert "geometry" in last_error()
        assert fn(*args(-1, ctypes.byref(hp), ctypes.byref(g()))) == _lib.PKV_ERR_INVALID_ARG
        assert fn(*args(1, None, ctypes.byref(g()))) == _lib.PKV_ERR_INVALID_ARG
        assert "host pool" in last_error()
        for nh in (0, -3, 1 << 27):
            bad = PkvHostPool(nh, x, x, None, None)
            assert fn(*args(1, ctypes.byref(bad), ctypes.byref(g()))) == _lib.PKV_ERR_INVALID_ARG
            assert "host num_blocks" in last_error()
        assert fn(*args(0, ctypes.byref(hp), ctypes.byref(g()))) == _lib.PKV_OK
        nul = PkvHostPool(8, x, None, None, None)
        assert fn(*args(1, ctypes.byref(nul), ctypes.byref(g()))) == _lib.PKV_ERR_INVALID_ARG
        assert "null pool" in last_error()
        mis = PkvHostPool(8, x, ctypes.c_void_p(0x1008), None, None)
        assert fn(*args(1, ctypes.byref(mis), ctypes.byref(g()))) == _lib.PKV_ERR_INVALID_ARG
        assert "misaligned" in last_error()
        # INT8: scale blocks of 4 bytes are not supported; missing scales refused
        i8 = g(B=1, H=1, D=128, dt=_lib.PKV_INT8)
        assert fn(*args(1, ctypes.byref(hp), ctypes.byref(i8))) == _lib.PKV_ERR_UNSUPPORTED
        assert fn(*args(1, ctypes.byref(hp), ctypes.byref(g(dt=_lib.PKV_INT8)))) == \
            _lib.PKV_ERR_INVALID_ARG
    sc = PkvKvScales(1.0, 1.0, x, None)
    hp8 = PkvHostPool(8, x, x, x, x)
    assert lib.pkv_swap_out(x, 1, x, x, ctypes.byref(sc), ctypes.byref(hp8),
                            ctypes.byref(g(dt=_lib.PKV_INT8)), None) == _lib.PKV_ERR_INVALID_ARG
    assert "null pool" in last_error()


def test_block_manager_swap_errors():
    bm = pkv.BlockManager(8, 4, num_host_blocks=4)
    bm.add_seq(0)
    bm.append_slots([0], 9)                  # 3 blocks
    bm.add_seq(1)
    bm.append_slots([1], 9)
    with pytest.raises(pkv.NoFreeBlocks):
        bm.swap_out([0, 1])                  # 6 > 4 host blocks
    assert bm.num_free_host() == 4 and not bm.is_swapped(0)
    p = bm.swap_out([0])
    assert p.shape == (3, 2) and bm.is_swapped(0)
    for call in (lambda: bm.append_slots([0], 1), lambda: bm.export([0], 4),
                 lambda: bm.fork(0, 5), lambda: bm.swap_out([0]), lambda: bm.swap_in([1]),
                 lambda: bm.swap_out([1, 1])):
        with pytest.raises(pkv.PkvError):
            call()
    lib = pkv.lib()
    seqs = (ctypes.c_int64 * 1)(0)
    n = ctypes.c_int32(-1)
    # capacity too small: refused, state unchanged
    st = lib.pkv_bm_swap_in(bm._h, seqs, 1, None, 0, ctypes.byref(n))
    assert st == _lib.PKV_ERR_INVALID_ARG and "capacity" in last_error() and bm.is_swapped(0)
    assert lib.pkv_bm_add_host_pool(bm._h, 4, None) == _lib.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError):
        bm.distinct_blocks([42])
    bm.free_seq(0)
    assert bm.num_free_host() == 4
    bm.check()


def test_quantized_matrix_core_entry_points_validate_on_the_host():
    from paged_attention_slot_amd._lib import PkvKvScales
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)
    fp8 = g(nb=16, B=16, H=2, D=128, dt=_lib.PKV_FP8_E4M3)
    i8 = g(nb=16, B=16, H=2, D=128, dt=_lib.PKV_INT8)
    bf = g(nb=16, B=16, H=2, D=128, dt=_lib.PKV_BF16)
    good = PkvKvScales(1.0, 1.0, x, x)

    def multi(geo, sc=good):
        return lib.pkv_attention_multi_quant(x, x, x, x, None if sc is None else ctypes.byref(sc),
                                             x, 4, x, 0.1, x, 2, 4, 4, 2, 64, 0, x, 1 << 30,
                                             ctypes.byref(geo), None)

    def shared(geo, sc=good):
        return lib.pkv_attention_decode_shared_quant(
            x, x, x, None if sc is None else ctypes.byref(sc), x, 4, x, x, x, 1, 2, 32, 0, 0.1,
            x, 2, 4, 64, x, 1 << 30, ctypes.byref(geo), None)
    for fn in (multi, shared):
        assert fn(bf) == _lib.PKV_ERR_INVALID_ARG and "quantized" in last_error()
        assert fn(g(nb=16, B=16, H=2, D=64, dt=_lib.PKV_FP8_E4M3)) == _lib.PKV_ERR_UNSUPPORTED
        assert fn(fp8, None) == _lib.PKV_ERR_INVALID_ARG and "scales" in last_error()
        assert fn(fp8, PkvKvScales(0.0, 1.0, None, None)) == _lib.PKV_ERR_INVALID_ARG
        assert fn(fp8, PkvKvScales(1.0, float("inf"), None, None)) == _lib.PKV_ERR_INVALID_ARG
        assert fn(i8, PkvKvScales(1.0, 1.0, None, x)) == _lib.PKV_ERR_INVALID_ARG
        assert fn(i8, PkvKvScales(1.0, 1.0, ctypes.c_void_p(0x1002), x)) == _lib.PKV_ERR_INVALID_ARG
    # the bf16 entry points refuse one-byte pools, the workspace sizes accept them
    assert lib.pkv_attention_multi(x, x, x, x, x, 4, x, 0.1, x, 2, 4, 4, 2, 64, 0, x, 1 << 30,
                                   ctypes.byref(fp8), None) == _lib.PKV_ERR_UNSUPPORTED
    assert lib.pkv_attention_multi_workspace_bytes(2, 4, 4, 2, 64, 32, ctypes.byref(i8)) > 0
    assert lib.pkv_attention_shared_workspace_bytes(2, 4, 1, 2, 32, 0, 64, ctypes.byref(fp8)) > 0


def test_fused_append_entry_point_validates_on_the_host():
    lib = pkv.lib()
    x = ctypes.c_void_p(0x1000)
    bad = ctypes.c_void_p(0x1004)

    def call(geom, kn=x, vn=x, sl=x, N=2, phases=3):
        return lib.pkv_attention_decode_append(phases, x, kn, vn, sl, x, x, x, 7, x, 0.1, x, N, 8,
                                               100, 0, None, 0, ctypes.byref(geom), None)

    # one-byte pools are refused before anything else
    assert call(g(H=2, D=128, dt=_lib.PKV_FP8_E4M3)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(g(H=2, D=128, dt=_lib.PKV_INT8)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(g(), N=0) == _lib.PKV_OK
    assert call(g(), kn=None) == _lib.PKV_ERR_INVALID_ARG
    assert "new-token" in last_error()
    assert call(g(), sl=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(g(), vn=bad) == _lib.PKV_ERR_INVALID_ARG
    assert call(g(), phases=4) == _lib.PKV_ERR_INVALID_ARG
    assert call(g(D=96)) == _lib.PKV_ERR_UNSUPPORTED
    # the balanced split needs a workspace
    assert call(g()) == _lib.PKV_ERR_INVALID_ARG
    assert "workspace" in last_error()


def test_append_fold_query(tuning):
    """pkv_attention_decode_append_folded: the append rides in the attention
    kernel on the balanced split on the matrix cores, and on the vector routes
    for waves of up to two query heads, not on vector batches that share
    blocks or whose query groups span several waves (both keep cacheable
    loads), not on the matrix route with partitions; one-byte pools give -1
    (the fused append refuses them)."""
    tuning("PKV_ATTN_APPEND", 0)
    tuning("PKV_ATTN_MODE", 0)
    tuning("PKV_ATTN_HEADS_PER_WAVE", 0)
    lib = pkv.lib()

    def folded(N, Hq, H, D, dt, shared=0, pt=0, maxlen=4096):
        return lib.pkv_attention_decode_append_folded(
            N, Hq, maxlen, pt, shared, ctypes.byref(g(nb=8192, H=H, D=D, dt=dt)))

    assert folded(64, 16, 8, 128, _lib.PKV_BF16) == 1          # matrix-core balanced split
    assert folded(64, 16, 8, 128, _lib.PKV_BF16, shared=1) == 1
    assert folded(64, 32, 8, 128, _lib.PKV_BF16) == 1
    assert folded(64, 16, 8, 128, _lib.PKV_BF16, pt=256) == 1  # fixed partitions, 2 heads per wave
    assert folded(4, 64, 8, 128, _lib.PKV_BF16) == 1           # 8 heads per group: the same
    assert folded(4, 64, 8, 128, _lib.PKV_BF16, pt=512) == 0   # matrix route (partitions given)
    assert folded(64, 16, 8, 64, _lib.PKV_BF16, shared=1) == 0  # vector kernels, cacheable loads
    assert folded(64, 8, 8, 128, _lib.PKV_F32) == 1            # 1 head per wave
    assert folded(64, 16, 8, 128, _lib.PKV_F32) == 0           # group split over 2 waves
    assert folded(4, 256, 8, 128, _lib.PKV_BF16) == 0          # matrix route
    assert folded(4, 64, 8, 128, _lib.PKV_FP8_E4M3) == -1
    assert folded(4, 63, 8, 128, _lib.PKV_BF16) == -1
    tuning("PKV_ATTN_MODE", 1)                                 # vector kernels, partitions
    assert folded(64, 16, 8, 128, _lib.PKV_BF16, pt=256) == 1  # 2 heads per wave
    assert folded(64, 32, 8, 128, _lib.PKV_BF16, pt=256) == 0  # 4 heads per wave
    tuning("PKV_ATTN_APPEND", 2)
    assert folded(64, 32, 8, 128, _lib.PKV_BF16, pt=256) == 1
    tuning("PKV_ATTN_APPEND", 1)
    assert folded(64, 16, 8, 128, _lib.PKV_BF16, pt=256) == 0
    tuning("PKV_ATTN_MODE", 0)
    assert folded(64, 16, 8, 128, _lib.PKV_BF16) == 0


def test_decode_route_query(tuning):
    """pkv_attention_decode_route: 2 to 16 query heads per KV head at head_dim
    128 (bf16 or one-byte pools, automatic partitions) take the balanced
    split on the matrix cores; wider groups, or 8 or more heads with given
    partitions (a multiple of 32), the matrix-core route with fixed
    partitions; one head per group, fp32 pools, 64-wide heads, 16-token
    partitions and narrower groups with given partitions stay on the vector
    kernels; bad arguments give -1."""
    lib = pkv.lib()
    tuning("PKV_ATTN_MODE", 0)

    def route(N, Hq, H, D, dt, pt=0, maxlen=4096):
        return lib.pkv_attention_decode_route(N, Hq, maxlen, pt,
                                              ctypes.byref(g(nb=8192, H=H, D=D, dt=dt)))

    M, B, P = _lib.PKV_ROUTE_MATRIX, _lib.PKV_ROUTE_BALANCED, _lib.PKV_ROUTE_PARTITIONS
    MB = _lib.PKV_ROUTE_MATRIX_BALANCED
    assert route(4, 64, 8, 128, _lib.PKV_BF16) == MB
    assert route(4, 64, 8, 128, _lib.PKV_BF16, pt=512) == M      # partitions given
    assert route(4, 64, 8, 128, _lib.PKV_FP8_E4M3) == MB
    assert route(4, 64, 8, 128, _lib.PKV_INT8) == MB
    assert route(4, 128, 8, 128, _lib.PKV_BF16) == MB          # 16 heads per group
    assert route(4, 256, 8, 128, _lib.PKV_BF16) == M           # 32 heads per group
    assert route(4, 256, 8, 128, _lib.PKV_INT8, pt=512) == M
    assert route(4, 64, 8, 128, _lib.PKV_BF16, pt=16) == P
    assert route(64, 16, 8, 128, _lib.PKV_BF16) == MB
    assert route(64, 32, 8, 128, _lib.PKV_BF16) == MB
    assert route(64, 16, 8, 128, _lib.PKV_BF16, pt=256) == P
    assert route(4, 64, 8, 64, _lib.PKV_BF16) == B
    assert route(4, 64, 8, 128, _lib.PKV_F32) == B
    assert route(4, 63, 8, 128, _lib.PKV_BF16) == -1
    assert route(256, 32, 8, 128, _lib.PKV_FP8_E4M3) == MB
    assert route(64, 16, 8, 128, _lib.PKV_INT8) == MB
    assert route(64, 16, 8, 128, _lib.PKV_INT8, pt=256) == P
    assert route(64, 8, 8, 128, _lib.PKV_FP8_E4M3) == B     # one head per group
    assert route(64, 16, 8, 64, _lib.PKV_BF16) == B         # head_dim 64: vector kernels
    # the workspace of the matrix route (PKV_ATTN_MODE=3): N * Hq * runs rows
    # of D + 2 floats.  256 partitions of 512 over 32 (sequence, KV head)
    # histories are more than the GPU holds at once: 64 runs of 4 whole
    # partitions each (about 2048 workgroups in all)
    tuning("PKV_ATTN_MODE", 3)
    assert route(4, 64, 8, 128, _lib.PKV_BF16, pt=512) == M
    n = lib.pkv_attention_workspace_bytes(4, 64, 131072, 512,
                                          ctypes.byref(g(nb=8192, H=8, D=128, dt=1)))
    assert n == 4 * 64 * 64 * (128 + 2) * 4
    # few partitions fill the GPU as whole partitions: one piece each
    n = lib.pkv_attention_workspace_bytes(4, 64, 4096, 512,
                                          ctypes.byref(g(nb=8192, H=8, D=128, dt=1)))
    assert n == 4 * 64 * 8 * (128 + 2) * 4


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """pkv_attention_decode_noalloc refuses, on the host and before anything
    is enqueued, sizes whose workspace exceeds the library's scratch."""
    lib = pkv.lib()
    geo = PkvGeom(1 << 20, 16, 8, 128, _lib.PKV_BF16)
    need = lib.pkv_attention_workspace_bytes(4096, 32, 8192, 0, ctypes.byref(geo))
    assert need > _lib.PKV_NOALLOC_SCRATCH_BYTES
    st = lib.pkv_attention_decode_noalloc(None, None, None, None, 512, None, 0.1, None, 4096, 32,
                                          8192, 0, ctypes.byref(geo), None)
    assert st == _lib.PKV_ERR_INVALID_ARG
    assert "scratch" in last_error() and str(need) in last_error()
    q8 = PkvGeom(1 << 20, 16, 8, 128, _lib.PKV_FP8_E4M3)
    assert lib.pkv_attention_decode_noalloc(None, None, None, None, 1, None, 0.1, None, 1, 8, 16,
                                            0, ctypes.byref(q8), None) == _lib.PKV_ERR_INVALID_ARG


def test_tuning_knobs_read_once_and_set_through_the_abi(tuning):
    """Knobs start from the environment once per process; later environment
    changes do nothing, pkv_set_tuning does (and refuses unknown names and
    values out of range)."""
    lib = pkv.lib()
    geo = ctypes.byref(g(nb=8192, H=8, D=64, dt=_lib.PKV_BF16))
    tuning("PKV_ATTN_MODE", 0)
    assert lib.pkv_attention_decode_route(64, 16, 4096, 0, geo) == _lib.PKV_ROUTE_BALANCED
    os.environ["PKV_ATTN_MODE"] = "1"
    try:
        assert lib.pkv_attention_decode_route(64, 16, 4096, 0, geo) == _lib.PKV_ROUTE_BALANCED
    finally:
        del os.environ["PKV_ATTN_MODE"]
    tuning("PKV_ATTN_MODE", 1)
    assert lib.pkv_get_tuning(b"PKV_ATTN_MODE") == 1
    assert lib.pkv_attention_decode_route(64, 16, 4096, 0, geo) == _lib.PKV_ROUTE_PARTITIONS
    assert lib.pkv_set_tuning(b"PKV_ATTN_MODE", 5) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_set_tuning(b"PKV_ATTN_WAVES_PER_BLOCK", 3) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_set_tuning(b"PKV_NOT_A_KNOB", 1) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_get_tuning(b"PKV_NOT_A_KNOB") == -1
    assert lib.pkv_get_tuning(b"PKV_ATTN_MODE") == 1


def test_piece_tokens_query(tuning):
    """pkv_attention_piece_tokens: what one split-KV piece covers.  Fixed
    partitions on the vector kernels: one partition.  The matrix-core route
    with more partitions than the GPU holds at once: runs of whole
    partitions (the long-context shape: 64 pieces of 2,048 positions for
    512-token partitions); with few partitions, one partition each.  The
    balanced splits: 0."""
    lib = pkv.lib()

    def piece(N, Hq, maxlen, pt, H=8, D=128, B=16, dt=_lib.PKV_BF16, nb=8192):
        return lib.pkv_attention_piece_tokens(N, Hq, maxlen, pt,
                                              ctypes.byref(g(nb=nb, B=B, H=H, D=D, dt=dt)))

    tuning("PKV_ATTN_MODE", 0)
    assert piece(4, 64, 131072, 512, B=32, nb=18022) == 2048  # partitions given: matrix route
    assert piece(4, 64, 131072, 0, B=32, nb=18022) == 0       # matrix-core balanced split
    assert piece(64, 16, 4096, 0) == 0            # balanced split
    assert piece(4, 63, 4096, 0) == 0             # invalid: 63 heads over 8
    tuning("PKV_ATTN_MODE", 3)                    # the matrix-core route
    assert piece(4, 64, 131072, 512, B=32, nb=18022) == 2048
    assert piece(4, 64, 4096, 512) == 512
    tuning("PKV_ATTN_MODE", 1)                    # vector kernels, fixed partitions
    assert piece(64, 16, 4096, 256) == 256
