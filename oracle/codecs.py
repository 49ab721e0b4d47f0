"""Exact decoders for the cache storage formats (test infrastructure only).

bf16: the upper 16 bits of an IEEE-754 binary32 value.
e4m3 ("fn" variant of the OCP 8-bit float): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is
NaN; there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.

Pins: every one of the 65536 bf16 patterns and 256 e4m3 codes is checked
against the library casts ``torch.bfloat16`` / ``torch.float8_e4m3fn`` and the
closed form above in ``tests/test_oracle_pins.py``.
"""
import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> float64 by the closed form."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, subnormal, normal)
    out = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, out)
    return out


def decode_kv_rows(rows: np.ndarray, kv_dtype: str, scale=None) -> np.ndarray:
    """Decode cache rows [..., D] to float64; for e4m3 multiply each row by its
    own per-token scale (one fp32 value per cached token)."""
    if kv_dtype == "bf16":
        return decode_bf16(rows)
    if kv_dtype == "fp32":
        return np.asarray(rows, dtype=np.float32).astype(np.float64)
    if kv_dtype == "fp8_e4m3":
        vals = decode_e4m3(rows)
        return vals * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    raise ValueError(kv_dtype)
