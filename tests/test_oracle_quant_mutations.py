"""Planted mistakes in copies of the quantization oracle: each must fail at least
one independent pin (PyTorch's float8_e4m3fn casts, the page's 448 maximum and
3-bit mantissa, the INT8 formula's consequences).  The oracle is untouched."""
import numpy as np
import pytest

from oracle import quant

torch = pytest.importorskip("torch")


def values_mutant(bias=7, subnormal=True):
    vals = np.empty(256)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
        if e == 15 and m == 7:
            v = np.nan
        elif e == 0:
            v = (m / 8.0) * 2.0 ** (1 - bias) if subnormal else 0.0
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - bias)
        vals[code] = -v if s else v
    return vals


def encode_mutant(mode):
    pos = quant.e4m3_values()[:127]

    def enc(x):
        x = np.asarray(x, dtype=np.float32)
        a = np.abs(x.astype(np.float64))
        if mode != "no_saturation":
            a = np.minimum(a, 448.0)
        hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 126)
        lo = np.clip(hi - 1, 0, 126)
        d_lo, d_hi = np.abs(a - pos[lo]), np.abs(pos[hi] - a)
        if mode == "truncate":
            pick = pos[hi] == a
        elif mode == "ties_up":
            pick = d_hi <= d_lo
        else:
            pick = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
        mag = np.where(pick, hi, lo).astype(np.uint8)
        if mode == "no_saturation":
            mag = np.where(a > 448.0, np.uint8(0x7F), mag)
        sign = np.signbit(x) if mode != "drop_neg_zero" else (x < 0) & (mag > 0)
        return (mag | np.where(sign, np.uint8(0x80), np.uint8(0))).astype(np.uint8)
    return enc


def int8_mutant(mode):
    def q8(x):
        x = np.asarray(x, dtype=np.float32)
        div = np.float32(128.0 if mode == "div128" else 127.0)
        scale = (np.abs(x).max(-1) / div).astype(np.float32)
        safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
        r = (x / safe[..., None]).astype(np.float32)
        q = np.floor(r) if mode == "floor" else np.rint(r)
        if mode == "per_tensor":
            s = np.float32(np.abs(x).max() / 127.0)
            q = np.rint(x / s)
            scale = np.full(scale.shape, s, np.float32)
        return np.clip(q, -127, 127).astype(np.int8), scale
    return q8


def e4m3_pins_pass(values, encode):
    ref_vals = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    v = values()
    if not np.array_equal(np.isnan(v), np.isnan(ref_vals)):
        return False
    if not np.array_equal(v[~np.isnan(v)], ref_vals[~np.isnan(ref_vals)]):
        return False
    if np.nanmax(v) != 448.0:
        return False
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 30, 20000), rng.normal(0, 1e-3, 2000),
                        [1.0625, 1.1875, -2.0 ** -11]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if not np.array_equal(encode(x), ref):
        return False
    return int(encode(np.float32(1e6))) == 0x7E and int(encode(np.float32(-1e6))) == 0xFE


def int8_pins_pass(q8):
    rng = np.random.default_rng(6)
    x = rng.normal(0, 3, (200, 4, 64)).astype(np.float32)
    x[:, 0] *= 10.0
    codes, scale = q8(x)
    amax_idx = np.abs(x).argmax(-1)
    top = np.take_along_axis(codes, amax_idx[..., None], -1)[..., 0].astype(int)
    if not np.all(np.abs(top) == 127):
        return False
    deq = codes.astype(np.float64) * scale[..., None]
    return bool(np.all(np.abs(deq - x) <= 0.5 * scale[..., None] * (1 + 1e-5)))


def test_oracle_passes_its_pins():
    assert e4m3_pins_pass(quant.e4m3_values, quant.e4m3_encode)
    assert int8_pins_pass(quant.int8_quantize_rows)


@pytest.mark.parametrize("bias,subnormal", [(8, True), (7, False)])
def test_decode_mutants_fail(bias, subnormal):
    assert not e4m3_pins_pass(lambda: values_mutant(bias, subnormal), quant.e4m3_encode)


@pytest.mark.parametrize("mode", ["truncate", "ties_up", "no_saturation", "drop_neg_zero"])
def test_encode_mutants_fail(mode):
    assert not e4m3_pins_pass(quant.e4m3_values, encode_mutant(mode))


@pytest.mark.parametrize("mode", ["div128", "floor", "per_tensor"])
def test_int8_mutants_fail(mode):
    assert not int8_pins_pass(int8_mutant(mode))
