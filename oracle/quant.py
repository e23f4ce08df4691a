"""Oracle KV-cache quantization: FP8 e4m3 and per-token INT8.  Test
infrastructure (only tests/, the smoke check and the bench's CPU baseline use
it).

What the pages fix:
  [KVM §19.2.4] KV-cache quantization: the precision table (FP16/BF16 2 bytes,
      FP8 and INT8 1 byte, INT4 half a byte per element) and per-token INT8,
      where each token's vector is scaled by its own factor: the code is the
      value divided by the scale, rounded, and the scale is the vector's
      largest magnitude over 127; dequantizing multiplies the scale back.
  [PFX §"KV Cache 量化"] FP8 e4m3: 1 sign, 4 exponent and 3 mantissa bits,
      largest magnitude 448; a scale maps values into that range when writing
      and back when reading; the engine default is a per-tensor scale of 1.0.
  [ENG §7.5] a copy-on-write copy of a per-token-quantized cache is a plain
      bit copy of codes and scales.

Readings (where the pages leave a step open):
  * e4m3 is the OCP "fn" encoding the 448 maximum implies: exponent bias 7,
    subnormals at exponent field 0, no infinities, S.1111.111 is NaN.
  * FP8 encoding: x / scale in fp32, saturated to +-448, then the nearest e4m3
    value, ties to the even code (last mantissa bit 0).  The sign bit is kept,
    so a negative value that rounds to zero gives code 0x80.
  * INT8 "per token" means per (token, KV head): one scale per head vector of
    head_dim elements.  scale = max|x| / 127 and code = round(x / scale) are
    both computed in fp32 (the kernel's precision; a code is an integer decided
    by floating point, so both sides decide it the same way), round is
    round-half-to-even, codes are clamped to [-127, 127].  An all-zero vector
    has scale 0 and codes 0.
  * FP8 scales are per tensor (one for K, one for V); INT8 scales are stored in
    fp32 pools shaped [num_blocks * block_size, num_kv_heads], slot-major like
    the data pools.

Functions:
  e4m3_values          value of each of the 256 codes (float64, NaN for NaN codes)
  e4m3_encode          fp32 -> e4m3 codes (nearest, ties to even, saturating)
  int8_quantize_rows   per-vector INT8 codes and scales
  write_quant          quantizing slot write into FP8 / INT8 pools
  copy_blocks_quant    block copy of codes and (INT8) scale rows
  dequantize_pool      pool of codes -> float64 values
  attention_decode_quant  the plain attention definition over dequantized K/V
"""
from __future__ import annotations

import numpy as np

from oracle.attention import attention_decode
from oracle.cache_ops import copy_blocks, write

E4M3_MAX = 448.0
FP8 = "fp8_e4m3"
INT8 = "int8"


def e4m3_values() -> np.ndarray:
    """Value of every e4m3 code 0..255: sign s, exponent field e, mantissa m;
    e == 0 is subnormal (m/8 * 2^-6), otherwise (1 + m/8) * 2^(e-7); e == 15
    with m == 7 is NaN."""
    vals = np.empty(256)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
        if e == 15 and m == 7:
            v = np.nan
        elif e == 0:
            v = (m / 8.0) * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = -v if s else v
    return vals


_POS = e4m3_values()[:127]          # codes 0..126: 0 .. 448, strictly increasing


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each fp32 value (after saturation to +-448), ties
    to the even code.  NaN gives 0x7F."""
    x = np.asarray(x, dtype=np.float32)
    xd = x.astype(np.float64)
    a = np.minimum(np.abs(xd), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = np.abs(a - _POS[lo])
    d_hi = np.abs(_POS[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = mag | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0)).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def int8_quantize_rows(x):
    """Per-vector INT8 over the last axis: returns (codes int8, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint((x / safe[..., None]).astype(np.float32))
    q = np.where(scale[..., None] > 0, q, 0.0)
    return np.clip(q, -127, 127).astype(np.int8), scale


def _bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def write_quant(k_bf16, v_bf16, slot_mapping, k_pool, v_pool, kind, k_scale=1.0, v_scale=1.0,
                k_scales=None, v_scales=None) -> None:
    """Quantize bf16 token rows [T, H_kv, D] and scatter them into slot
    ``slot_mapping[i]`` (negative = skip) of the code pools; INT8 also stores
    each (token, head) scale at [slot, head] of ``k_scales`` / ``v_scales``.
    In place."""
    kf = _bf16_bits_to_f32(k_bf16)
    vf = _bf16_bits_to_f32(v_bf16)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if kind == FP8:
        kc = e4m3_encode(kf / np.float32(k_scale))
        vc = e4m3_encode(vf / np.float32(v_scale))
    elif kind == INT8:
        kc, ks = int8_quantize_rows(kf)
        vc, vs = int8_quantize_rows(vf)
        live = slots >= 0
        k_scales[slots[live]] = ks[live]
        v_scales[slots[live]] = vs[live]
    else:
        raise ValueError(kind)
    write(kc, vc, slots, k_pool, v_pool)


def copy_blocks_quant(pairs, k_pool, v_pool, kind, k_scales=None, v_scales=None) -> None:
    """Block copy of codes; INT8 copies the blocks' scale rows too ([ENG §7.5])."""
    copy_blocks(pairs, k_pool, v_pool)
    if kind == INT8:
        nb, B, H, _ = k_pool.shape
        ks = k_scales.reshape(nb, B, H)
        vs = v_scales.reshape(nb, B, H)
        for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
            ks[dst] = ks[src]
            vs[dst] = vs[src]


def dequantize_pool(pool, kind, scale=1.0, scales=None) -> np.ndarray:
    """Codes -> float64 values: e4m3 value times the tensor scale (FP8), or
    code times its (slot, head) scale (INT8)."""
    if kind == FP8:
        return e4m3_values()[np.asarray(pool, dtype=np.uint8)] * float(scale)
    if kind == INT8:
        nb, B, H, _ = pool.shape
        s = np.asarray(scales, dtype=np.float64).reshape(nb, B, H, 1)
        return np.asarray(pool, dtype=np.float64) * s
    raise ValueError(kind)


def attention_decode_quant(q_bf16, k_pool, v_pool, block_tables, seq_lens, scale, kind,
                           k_scale=1.0, v_scale=1.0, k_scales=None, v_scales=None, seqs=None):
    """Decode attention over a quantized cache: the plain definition of
    oracle.attention.attention_decode applied to the dequantized pools."""
    kd = dequantize_pool(k_pool, kind, k_scale, k_scales)
    vd = dequantize_pool(v_pool, kind, v_scale, v_scales)
    return attention_decode(q_bf16, kd, vd, block_tables, seq_lens, scale, seqs=seqs)


def attention_multi_quant(q_bf16, q_offsets, k_pool, v_pool, block_tables, seq_lens, scale, kind,
                          k_scale=1.0, v_scale=1.0, k_scales=None, v_scales=None):
    """Multi-token query attention over a quantized cache: the definition of
    oracle.attention.attention_multi applied to the dequantized pools."""
    from .attention import attention_multi
    kd = dequantize_pool(k_pool, kind, k_scale, k_scales)
    vd = dequantize_pool(v_pool, kind, v_scale, v_scales)
    return attention_multi(q_bf16, q_offsets, kd, vd, block_tables, seq_lens, scale)
