"""FP8 (E4M3) KV-cache encoding for the CPU oracle -- test infrastructure only.

The intelliparadigm article's §4.3 lists FP8 K/V storage among the cache
precisions (with a per-precision speed-up over FP16). It does not fix the
8-bit format or how values are scaled, so this module takes the plainest
reading:

* The format is OCP 8-bit floating point E4M3, the variant with no
  infinities. One sign bit, four exponent bits with bias 7, three mantissa
  bits. Exponent field 0 holds subnormals: value = mantissa * 2^-9.
  Otherwise value = 2^(E-7) * (1 + mantissa/8). The all-ones magnitude code
  (0x7F / 0xFF) is NaN, so the largest finite value is 0x7E = 448.
* Each cache tensor has one fp32 scale. A stored code c stands for
  ``decode(c) * scale``. Writing value x stores ``encode(fp32(x) / scale)``:
  the division is an IEEE fp32 division, and the encoding rounds to nearest
  even, clamps magnitudes above 448 to 448 and maps NaN to 0x7F.

Everything here is float64 / integer NumPy written from that definition.
The pins in ``tests/test_oracle_fp8.py`` check it against torch's
independent ``float8_e4m3fn`` conversion and the format's fixed points.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

__all__ = ["E4M3_MAX", "E4M3_NAN", "e4m3_decode", "e4m3_encode", "quantize_e4m3",
           "cache_write_fp8"]

E4M3_MAX = 448.0
E4M3_NAN = 0x7F
_BIAS = 7
_MIN_NORMAL_EXP = 1 - _BIAS          # 2^-6, the smallest normal binade
_SUBNORMAL_QUANTUM = 2.0 ** -9       # spacing of the subnormals (and of [2^-6, 2^-5))


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact float64 value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * _SUBNORMAL_QUANTUM,
                   np.ldexp(1.0 + m / 8.0, (e - _BIAS).astype(np.int64)))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """E4M3 code of each value: round to nearest even, saturate at 448, NaN -> 0x7F.

    ``x`` is taken as given (float32 or float64); the rounding is done in
    float64, where scaling by a power of two is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    for i, v in enumerate(flat_x.tolist()):
        if v != v:                                   # NaN
            flat_o[i] = E4M3_NAN
            continue
        sign = 0x80 if (v < 0 or (v == 0 and np.signbit(v))) else 0
        a = min(abs(v), E4M3_MAX)
        if a < 2.0 ** _MIN_NORMAL_EXP:
            # subnormal range: count quanta of 2^-9; 8 quanta is the smallest
            # normal, whose code (exponent 1, mantissa 0) is also 8
            q = int(np.rint(a / _SUBNORMAL_QUANTUM))
            code = q
        else:
            e = int(np.floor(np.log2(a)))
            # guard against log2 rounding at exact powers of two
            if 2.0 ** e > a:
                e -= 1
            elif 2.0 ** (e + 1) <= a:
                e += 1
            q = int(np.rint(a / 2.0 ** (e - 3)))    # 8..16 steps of the binade's quantum
            if q == 16:
                e, q = e + 1, 8
            code = ((e + _BIAS) << 3) | (q - 8)
        flat_o[i] = sign | min(code, 0x7E)
    return out


def quantize_e4m3(bits: np.ndarray, src_dtype: str, scale) -> np.ndarray:
    """Codes for 2-byte storage values: ``encode(fp32(x) / fp32(scale))``."""
    from .paged_attention import to_float64
    x32 = to_float64(bits, src_dtype).astype(np.float32)      # exact
    y = (x32 / np.float32(scale)).astype(np.float32)          # IEEE fp32 division
    return e4m3_encode(y)


def cache_write_fp8(key_cache: np.ndarray, value_cache: np.ndarray, k: np.ndarray,
                    v: np.ndarray, slots: np.ndarray, src_dtype: str, k_scale,
                    v_scale) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the uint8 caches with token i's quantized k/v stored at ``slots[i]``.

    The slot rule is the one of :func:`oracle.paged_attention.cache_write`;
    the stored row is ``quantize_e4m3`` of the token's ``[num_kv_heads,
    head_size]`` row with that tensor's scale. Negative slots are skipped.
    """
    kc = key_cache.copy()
    vc = value_cache.copy()
    bs = kc.shape[1]
    live = [int(x) for x in np.asarray(slots).tolist() if x >= 0]
    assert len(live) == len(set(live)), "cache_write_fp8: duplicate slots"
    for i, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0:
            continue
        kc[slot // bs, slot % bs] = quantize_e4m3(k[i], src_dtype, k_scale)
        vc[slot // bs, slot % bs] = quantize_e4m3(v[i], src_dtype, v_scale)
    return kc, vc
