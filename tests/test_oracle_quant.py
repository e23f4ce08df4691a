"""Pins of the quantized-cache oracle (oracle/quant.py) against facts fixed
outside it: the e4m3 range and bit split the pages give ([PFX] "KV Cache 量化":
1 sign / 4 exponent / 3 mantissa bits, maximum 448), PyTorch's own float8_e4m3fn
casts (an independent library routine), the per-token INT8 formula's
consequences ([KVM §19.2.4]), and lossless cases where quantized attention must
equal the pinned plain attention."""
import numpy as np
import pytest

from oracle import quant
from oracle.attention import attention_decode
from oracle.cache_ops import copy_blocks

torch = pytest.importorskip("torch")


def test_e4m3_range_and_spacing_from_the_page():
    v = quant.e4m3_values()
    finite = v[~np.isnan(v)]
    assert finite.max() == 448.0 and finite.min() == -448.0        # page: largest 448
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9            # smallest normal / subnormal
    # 3 mantissa bits: 8 steps per binade, relative spacing 1/8 at the binade start
    pos = np.unique(finite[finite > 0])
    assert pos.size == 126
    binade = pos[(pos >= 1.0) & (pos < 2.0)]
    assert np.allclose(np.diff(binade), 1.0 / 8.0) and binade.size == 8


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = quant.e4m3_values()
    same_nan = np.isnan(ref) == np.isnan(ours)
    assert same_nan.all()
    assert np.array_equal(ref[~np.isnan(ref)], ours[~np.isnan(ours)])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 60, 20000),
                        rng.uniform(-448, 448, 20000), rng.normal(0, 1e-3, 5000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = quant.e4m3_encode(x)
    # torch keeps the sign of a negative zero result as well
    assert np.array_equal(ours, ref)


def test_e4m3_encode_round_trip_saturation_ties_sign():
    v = quant.e4m3_values()
    codes = np.array([c for c in range(256) if not np.isnan(v[c])], dtype=np.uint8)
    assert np.array_equal(quant.e4m3_encode(v[codes].astype(np.float32)), codes)
    assert quant.e4m3_encode(np.float32(1e6)) == 0x7E
    assert quant.e4m3_encode(np.float32(-1e6)) == 0xFE
    assert quant.e4m3_encode(np.float32(449.0)) == 0x7E
    # midpoint between 1.0 (0x38, even) and 1.125 (0x39): ties to even -> 0x38;
    # between 1.125 and 1.25 (0x3A, even) -> 0x3A
    assert quant.e4m3_encode(np.float32(1.0625)) == 0x38
    assert quant.e4m3_encode(np.float32(1.1875)) == 0x3A
    assert quant.e4m3_encode(np.float32(-2.0 ** -11)) == 0x80     # rounds to -0
    # nearest: every fp32 input lands on a code at least as close as its neighbours
    x = np.linspace(-450, 450, 100001).astype(np.float32)
    c = quant.e4m3_encode(x)
    err = np.abs(v[c] - np.clip(x.astype(np.float64), -448, 448))
    for d in (-1, 1):
        nb = c.astype(np.int64) + d
        ok = (nb & 0x7F) <= 0x7E
        nb = np.clip(nb, 0, 255)
        alt = np.abs(v[nb] - np.clip(x.astype(np.float64), -448, 448))
        same_sign = (nb >> 7) == (c.astype(np.int64) >> 7)
        assert np.all(err[ok & same_sign & ~np.isnan(alt)] <= alt[ok & same_sign & ~np.isnan(alt)])


def test_int8_per_token_formula_consequences():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 3, (500, 8, 128)).astype(np.float32)
    x[3, 2] = 0.0
    codes, scale = quant.int8_quantize_rows(x)
    assert codes.dtype == np.int8 and scale.shape == (500, 8)
    # the largest magnitude of each vector maps to +-127, nothing exceeds it
    amax_idx = np.abs(x).argmax(axis=-1)
    top = np.take_along_axis(codes, amax_idx[..., None], -1)[..., 0].astype(int)
    nz = scale > 0
    assert np.all(np.abs(top[nz]) == 127)
    assert np.all(np.abs(codes.astype(int)) <= 127)
    # dequantized values are within half a step of the input
    deq = codes.astype(np.float64) * scale[..., None]
    assert np.all(np.abs(deq - x) <= 0.5 * scale[..., None] * (1 + 1e-5) + 1e-30)
    # signs are kept, zero vectors give scale 0 and codes 0
    assert np.all(np.sign(codes[np.abs(x) > scale[..., None]]) == np.sign(x[np.abs(x) > scale[..., None]]))
    assert scale[3, 2] == 0 and not codes[3, 2].any()
    # scale = max|x| / 127 in fp32
    assert np.array_equal(scale, (np.abs(x).max(-1) / np.float32(127)).astype(np.float32))


def _exact_pools(kind, rng, nb, B, H, D):
    """Pools whose values every encoding represents exactly."""
    if kind == quant.FP8:
        v = quant.e4m3_values()
        ok = np.array([c for c in range(256) if not np.isnan(v[c]) and abs(v[c]) <= 4])
        k = rng.choice(ok, size=(nb, B, H, D)).astype(np.uint8)
        vv = rng.choice(ok, size=(nb, B, H, D)).astype(np.uint8)
        return k, vv, None, None
    k = rng.integers(-127, 128, size=(nb, B, H, D)).astype(np.int8)
    vv = rng.integers(-127, 128, size=(nb, B, H, D)).astype(np.int8)
    ks = (2.0 ** rng.integers(-8, -4, size=(nb * B, H))).astype(np.float32)
    vs = (2.0 ** rng.integers(-8, -4, size=(nb * B, H))).astype(np.float32)
    return k, vv, ks, vs


@pytest.mark.parametrize("kind", [quant.FP8, quant.INT8])
def test_quantized_attention_equals_plain_attention_when_lossless(kind):
    rng = np.random.default_rng(2)
    nb, B, H, D, N, Hq = 12, 4, 2, 16, 3, 4
    kc, vc, ks, vs = _exact_pools(kind, rng, nb, B, H, D)
    kd = quant.dequantize_pool(kc, kind, 1.0, ks)
    vd = quant.dequantize_pool(vc, kind, 1.0, vs)
    tables = np.stack([rng.permutation(nb)[:4] for _ in range(N)]).astype(np.int32)
    lens = np.array([16, 5, 9], dtype=np.int32)
    q = (rng.normal(0, 1, (N, Hq, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    a = quant.attention_decode_quant(q, kc, vc, tables, lens, 0.25, kind, k_scales=ks, v_scales=vs)
    b = attention_decode(q, kd, vd, tables, lens, 0.25)
    assert np.array_equal(a, b)
    # with per-tensor scales, FP8 attention scales K and V exactly
    if kind == quant.FP8:
        c = quant.attention_decode_quant(q, kc, vc, tables, lens, 0.25, kind, k_scale=2.0, v_scale=0.5)
        d = attention_decode(q, kd * 2.0, vd * 0.5, tables, lens, 0.25)
        assert np.allclose(c, d, rtol=0, atol=0)


def test_write_quant_int8_and_fp8_round_trip_of_representable_rows():
    rng = np.random.default_rng(3)
    nb, B, H, D, T = 6, 4, 2, 16, 5
    # bf16 rows that are exactly e4m3 values: FP8 with scale 1 stores them losslessly
    v = quant.e4m3_values()
    ok = np.array([c for c in range(256) if not np.isnan(v[c]) and abs(v[c]) <= 8])
    vals = v[rng.choice(ok, size=(T, H, D))].astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    kp = np.zeros((nb, B, H, D), np.uint8); vp = np.zeros_like(kp)
    slots = np.array([3, 17, -1, 0, 9])
    quant.write_quant(bits, bits, slots, kp, vp, quant.FP8)
    deq = quant.dequantize_pool(kp, quant.FP8).reshape(nb * B, H, D)
    live = slots >= 0
    assert np.array_equal(deq[slots[live]], vals[live].astype(np.float64))
    # INT8: codes and scales land at the slot; dequantized within half a step
    kp8 = np.zeros((nb, B, H, D), np.int8); vp8 = np.zeros_like(kp8)
    ks = np.zeros((nb * B, H), np.float32); vs = np.zeros_like(ks)
    quant.write_quant(bits, bits, slots, kp8, vp8, quant.INT8, k_scales=ks, v_scales=vs)
    d8 = quant.dequantize_pool(kp8, quant.INT8, scales=ks).reshape(nb * B, H, D)
    err = np.abs(d8[slots[live]] - vals[live])
    assert np.all(err <= 0.5 * ks[slots[live]][..., None] * (1 + 1e-5))
    assert not ks[2].any()          # untouched slot


def test_copy_blocks_quant_carries_scales():
    rng = np.random.default_rng(4)
    nb, B, H, D = 5, 4, 2, 8
    kp = rng.integers(-127, 128, size=(nb, B, H, D)).astype(np.int8); vp = kp.copy()
    ks = rng.random((nb * B, H)).astype(np.float32); vs = ks.copy()
    before = quant.dequantize_pool(kp, quant.INT8, scales=ks)
    quant.copy_blocks_quant([[1, 3], [0, 4]], kp, vp, quant.INT8, ks, vs)
    after = quant.dequantize_pool(kp, quant.INT8, scales=ks)
    assert np.array_equal(after[3], before[1]) and np.array_equal(after[4], before[0])
    # FP8 copy is the plain block copy
    k8 = rng.integers(0, 126, size=(nb, B, H, D)).astype(np.uint8); v8 = k8.copy()
    ref = k8.copy(); copy_blocks([[2, 0]], ref, ref.copy())
    quant.copy_blocks_quant([[2, 0]], k8, v8, quant.FP8)
    assert np.array_equal(k8, ref)
