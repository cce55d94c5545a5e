"""FP8 E4M3 cache format (test infrastructure only; see ``oracle/__init__``).

An FP8 KV cache halves the bytes per block ([p2] "PagedAttention: KV cache as
virtual memory", section "Deep dive" and the follow-up on raising the
concurrency ceiling).  The pages do not fix the FP8 flavour; the reading taken
is the OCP 8-bit "E4M3" format with no infinities, written here from its
definition rather than from any library:

* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
* exponent field 0 encodes subnormals ``m * 2**-9``;
* other fields encode ``(1 + m/8) * 2**(e - 7)``;
* exponent 15 with mantissa 7 (codes 0x7F, 0xFF) is NaN; there is no infinity,
  so the largest finite magnitude is ``1.75 * 2**8 = 448``.

Quantisation of a cache value ``x`` with per-tensor scale ``s``:
``code = encode(clamp(fp32(x) / fp32(s), -448, 448))`` where the division is one
correctly rounded float32 operation and ``encode`` rounds to the nearest
representable value, ties to the code with an even last bit (round to nearest
even).  Dequantisation is ``decode(code) * s``.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# magnitudes of codes 0x00..0x7E, strictly increasing with the code
_POS_VALUES = np.array([e4m3_decode(c) for c in range(0x7F)], dtype=np.float64)


def e4m3_encode(x: float) -> int:
    """Nearest finite E4M3 code to ``x`` (ties to even code), saturating at 448.

    The caller clamps first; values beyond 448 still saturate here, NaN maps to
    0x7F.
    """
    x = float(x)
    if x != x:
        return 0x7F
    sign = 0x80 if np.signbit(x) else 0x00
    a = min(abs(x), E4M3_MAX)
    # first code whose value is >= a
    hi = int(np.searchsorted(_POS_VALUES, a, side="left"))
    if hi < len(_POS_VALUES) and _POS_VALUES[hi] == a:
        return sign | hi
    lo = hi - 1
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    if d_lo < d_hi:
        c = lo
    elif d_hi < d_lo:
        c = hi
    else:
        c = lo if (lo & 1) == 0 else hi
    return sign | c


def e4m3_quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """Quantise a float16/float32 array with a per-tensor scale -> uint8 codes."""
    q = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float32)
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    flat = q.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    # exact table method, vectorised: same rule as e4m3_encode
    a = np.abs(flat.astype(np.float64))
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi_c = np.minimum(hi, len(_POS_VALUES) - 1)
    lo_c = np.maximum(hi - 1, 0)
    exact = _POS_VALUES[hi_c] == a
    d_lo = a - _POS_VALUES[lo_c]
    d_hi = _POS_VALUES[hi_c] - a
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((lo_c & 1) == 0))
    code = np.where(exact, hi_c, np.where(pick_lo, lo_c, hi_c)).astype(np.uint8)
    sign = np.where(np.signbit(flat), 0x80, 0).astype(np.uint8)
    out[:] = code | sign
    return out.reshape(np.shape(x))


_DECODE_TABLE = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """uint8 codes -> float64 values ``decode(code) * scale``."""
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] * float(np.float32(scale))
