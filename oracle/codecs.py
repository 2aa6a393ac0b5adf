"""Stored values -> float64, exactly.  (Oracle; test infrastructure only.)

* fp32: widened to float64.
* bf16: the 16 stored bits are the top half of a float32.
* fp8: OCP E4M3FN -- sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN and there
  is no infinity, so the largest finite magnitude is 448.  The pages name the
  format only as "FP8 (1 B)" per value ("KV cache, PagedAttention and
  FlashAttention", Problem 3, worked answer); the bit layout is the OCP 8-bit
  floating point specification's.  A stored code is then multiplied by its
  fp32 scale for its (block, KV head), in float64.
"""
import numpy as np


def f32_to_f64(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp_field = (c >> 3) & 0xF
    man = c & 0x7
    normal = (1.0 + man / 8.0) * np.exp2(exp_field - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    mag = np.where(exp_field == 0, subnormal, normal)
    val = np.where(sign == 1, -mag, mag)
    return np.where((exp_field == 15) & (man == 7), np.nan, val)


def decode_storage(x: np.ndarray, kind: str) -> np.ndarray:
    """Decode an array stored as 'f32' | 'bf16' | 'fp8' to float64 (no scale)."""
    if kind == "f32":
        return f32_to_f64(x)
    if kind == "bf16":
        return bf16_bits_to_f64(x)
    if kind == "fp8":
        return e4m3fn_to_f64(x)
    raise ValueError(kind)
