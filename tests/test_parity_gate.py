"""The attention gate used by the GPU parity tests, pinned on the CPU: its
bounds follow from the oracle value alone."""
import numpy as np

from tests.parity import attention_gate, half_ulp_bf16


def bf16_rne(x):
    """Round float32 values to bf16 (nearest, ties to even) and back."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_half_ulp_matches_bf16_spacing():
    for x in (0.3, 1.0, 1.5, 3.0, 100.0):
        e = np.floor(np.log2(x))
        assert half_ulp_bf16(np.array([x]))[0] == 2.0 ** (e - 8)


def test_fp32_results_within_the_bound_pass_once_rounded_to_bf16():
    """Any fp32 value within 2e-3 and 0.5 % of the oracle passes after
    rounding to bf16 (which adds at most 0.4 % relative), including across a
    binade edge (b just below 2, the result rounded up)."""
    rng = np.random.default_rng(3)
    b = np.concatenate([rng.normal(size=4000), [1.999, -1.999, 0.9995, 3.9985]])
    room = np.minimum(2e-3, 5e-3 * np.abs(b))
    d = rng.uniform(-1.0, 1.0, size=b.size) * room
    d[-4:] = [2e-3, -2e-3, 2e-3, 2e-3]
    a = bf16_rne(b + d * 0.999)
    r = attention_gate(a, b, "bf16")
    assert r["ok"], r


def test_a_wrong_output_does_not_widen_its_own_bound():
    """b = 1.996: an output of 2.004 (error 8e-3) lies past 2e-3 plus half a
    bf16 ulp at 1.998 (5.9e-3); taking the ulp at the output's own magnitude
    (7.8e-3 above 2) would have let it pass."""
    b = np.array([1.996])
    assert not attention_gate(np.array([2.004]), b, "bf16")["ok"]
    assert attention_gate(np.array([2.0]), b, "bf16")["ok"]
    assert not attention_gate(np.array([1.996 + 2.5e-3]), b, "f32")["ok"]
    assert attention_gate(np.array([1.996 + 1.5e-3]), b, "f32")["ok"]
