"""FP8 KV pool, oracle side: OCP E4M3 ("fn": finite values and NaN only) decode and the store's
encoding. TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Inside SGLang", Step 6 (the KV dtype lever): with ``--kv-cache-dtype fp8_e4m3`` every cached
element takes one byte instead of two; attention must read the FP8 cache directly, without a
separate dequantisation pass, and needs a scale per tensor, which defaults to 1.0 when the
checkpoint has none. Here an element's value is ``scale * e4m3(byte)``.

The E4M3 encoding, from the format's definition: bit 7 is the sign, bits 6..3 the exponent
(bias 7), bits 2..0 the mantissa. Exponent 0 holds the subnormals m * 2^-9 (and the two zeros);
exponents 1..15 hold (1 + m/8) * 2^(e-7), except exponent 15 with mantissa 7, which is NaN.
There are no infinities; the largest finite magnitude is 448.

Reading of what the pages leave open, for the store (``kv_store_fp8``): the new bf16 element
is widened to float32, multiplied by the float32 reciprocal of the scale (1/scale computed in
float64 and rounded once to float32), clamped to [-448, 448] (a NaN in the pool would poison
every query that reads it), and rounded to the nearest E4M3 value, ties to the even mantissa.
The sign of a zero result is the sign of the product. Inputs must be finite.
"""

import numpy as np

from .formats import bf16_bits_to_f64

E4M3_MAX = 448.0


def e4m3_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact float64 value of each E4M3 byte (NaN for 0x7F and 0xFF)."""
    b = np.asarray(b)
    if b.dtype != np.uint8:
        raise TypeError(f"fp8 data must be uint8 bytes, got {b.dtype}")
    bi = b.astype(np.int64)
    sign = np.where(bi & 0x80, -1.0, 1.0)
    e = (bi >> 3) & 0xF
    m = (bi & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((bi & 0x7F) == 0x7F, np.nan, out)


def e4m3_round(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 byte of each finite value with |y| <= 448, ties to the even code.

    Written from the format: for |y| >= 2^-6 (the normal range) take the binary exponent e of
    |y| (|y| = s * 2^e, 1 <= s < 2), round the 3-bit mantissa (s - 1) * 8 to the nearest
    integer with ties to even, and carry into the exponent when it rounds up to 8; below 2^-6
    round |y| / 2^-9 the same way (the subnormal step; 8 lands on the smallest normal, code 8).
    All scalings are by powers of two, so nothing but the final rounding is inexact.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("E4M3 rounding takes finite values")
    a = np.abs(y)
    if np.any(a > E4M3_MAX):
        raise ValueError("values beyond 448 must be clamped before rounding")
    frac, exp = np.frexp(a)                      # a = frac * 2^exp, 0.5 <= frac < 1 (a > 0)
    e = exp.astype(np.int64) - 1                 # a = (2 frac) * 2^e, 1 <= 2 frac < 2
    m = np.rint((2.0 * frac - 1.0) * 8.0)        # 0 .. 8
    carry = m == 8.0
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0.0, m)
    normal = a >= 2.0 ** -6
    code_n = ((e + 7) << 3) | m.astype(np.int64)
    code_s = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = np.where(np.signbit(y), code | 0x80, code)
    return code.astype(np.uint8)


def reciprocal_f32(scale: float) -> np.float32:
    """1/scale in float64, rounded once to float32 (the store's multiplier)."""
    s = float(np.float32(scale))
    if not np.isfinite(s) or s <= 0:
        raise ValueError("an FP8 scale must be finite and positive")
    return np.float32(1.0 / s)


def quantize_bf16(bits: np.ndarray, scale: float) -> np.ndarray:
    """Bytes the store writes for bf16 elements ``bits`` under ``scale`` (see module doc)."""
    x = bf16_bits_to_f64(bits).astype(np.float32)       # exact
    if not np.all(np.isfinite(x)):
        raise ValueError("values stored into an FP8 pool must be finite")
    y = x * reciprocal_f32(scale)                       # float32 product, rounded once
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_round(y.astype(np.float64))


def kv_store_fp8(k_pool, v_pool, k_new, v_new, loc, k_scale=1.0, v_scale=1.0):
    """FP8 pools (uint8 ``[slots, kv_heads, head_dim]``) with row ``loc[i]`` replaced by the
    encoding of the i-th new bf16 row; other rows unchanged. As ``kv_store``: the locations
    must be distinct and inside the pool."""
    if loc is None:
        raise ValueError("kv_store needs the slot locations of the new rows")
    if k_pool.dtype != np.uint8 or v_pool.dtype != np.uint8:
        raise TypeError("FP8 pools hold uint8 bytes")
    if k_pool.shape != v_pool.shape or k_pool.ndim != 3:
        raise ValueError("pools must both be [slots, kv_heads, head_dim]")
    S, Hkv, D = k_pool.shape
    loc = np.asarray(loc)
    n = loc.shape[0]
    if k_new.shape != (n, Hkv, D) or v_new.shape != (n, Hkv, D):
        raise ValueError("new rows do not match the pool")
    if n and (loc.min() < 0 or loc.max() >= S):
        raise ValueError("a slot location lies outside the pool")
    if np.unique(loc).shape[0] != n:
        raise ValueError("slot locations must be distinct")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    k_out[loc] = quantize_bf16(k_new, k_scale)
    v_out[loc] = quantize_bf16(v_new, v_scale)
    return k_out, v_out
