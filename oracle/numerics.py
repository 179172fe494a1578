"""Storage codecs of the oracle (TEST INFRASTRUCTURE ONLY; see oracle/__init__).

Storage dtypes are named by strings and held in NumPy arrays of their bit
patterns:

* ``"f32"``  - IEEE binary32, held as ``np.float32``.
* ``"bf16"`` - bfloat16 bit patterns, held as ``np.uint16``.
* ``"fp8"``  - OCP 8-bit floating point E4M3 ("E4M3FN": bias 7, no
  infinities, one NaN pattern per sign, largest finite 448), held as
  ``np.uint8`` codes.

The pages only say that the FP8 KV cache stores values in 8 bits and turns them
back into 16-bit values as they are read ("How Easy Is It to Start Serving
LLMs?", "What each setting does to performance" and Phase 4 §1 key results);
they do not name the variant.  The reading taken here is OCP E4M3FN with one
fp32 scale per tensor: the stored code ``c`` stands for ``value(c) * scale``.

Everything is written from the format definitions, not from any library:

* decode: sign, exponent and mantissa fields are pulled apart and the value is
  formed as ``(-1)^s * 2^(e-7) * (1 + m/8)`` (normal) or
  ``(-1)^s * 2^-6 * (m/8)`` (subnormal, e = 0).
* encode: the nearest finite E4M3 value to ``x / scale`` (division in fp32,
  IEEE round-to-nearest-even), ties to the even code, magnitudes at or above
  448 saturate to 448, NaN becomes ``0x7F``.

Pins (tests/test_oracle_numerics.py): all 256 codes against the OCP table in
tests/golden/ and against ``torch.float8_e4m3fn``; exhaustive encode of all
65,536 bf16 patterns against torch's conversion where torch does not saturate;
hand-checked edges (ties, 448/464, the smallest subnormal, signed zero, NaN);
bf16 rounding against ``torch.bfloat16``.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bfloat16
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    The nearest bf16 to an fp32 value is found by adding half a bf16 ulp
    (0x7FFF plus the parity of the kept part, so that exact ties land on the
    even pattern) and truncating the low 16 bits.  NaN maps to the quiet NaN
    with the same sign.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint32)
    sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint32)
    out = np.where(np.isnan(f), sign | np.uint32(0x7FC0), rounded)
    return out.astype(np.uint16)


# --------------------------------------------------------------------------
# OCP FP8 E4M3FN
# --------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F
E4M3_MAX_CODE = 0x7E


def _e4m3_field_value(code: int) -> float:
    """Value of one code from its fields (fp64, exact)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (-6)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


_DECODE_TABLE = np.array([_e4m3_field_value(c) for c in range(256)], dtype=np.float64)


def e4m3_value_table() -> np.ndarray:
    """The 256 code values in fp64 (NaN for 0x7F and 0xFF)."""
    return _DECODE_TABLE.copy()


def e4m3_decode(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """E4M3FN codes -> fp64 values times the fp32 ``scale`` (exact in fp64)."""
    c = np.asarray(codes, dtype=np.uint8)
    return _DECODE_TABLE[c] * np.float64(np.float32(scale))


# Non-negative finite values in code order 0x00..0x7E (monotonic increasing).
_POS_VALUES = _DECODE_TABLE[: E4M3_MAX_CODE + 1]


def e4m3_encode(x: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """fp32 values -> E4M3FN codes of ``fl32(x / scale)``.

    Steps (each the plain definition):
      1. y = x / scale in fp32 (IEEE division, round to nearest even).
      2. NaN -> 0x7F.
      3. |y| >= 448 -> the largest finite magnitude (saturation).
      4. otherwise the nearest of the 127 non-negative finite values to |y|;
         on an exact tie the code with the even low bit wins.
      5. the sign bit of y is copied (so -0.0 -> 0x80).
    """
    xf = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        y = (xf / np.float32(scale)).astype(np.float32)
    a = np.abs(y).astype(np.float64)
    sign = np.signbit(y)

    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi_c = np.clip(hi, 0, E4M3_MAX_CODE)
    lo_c = np.clip(hi - 1, 0, E4M3_MAX_CODE)
    d_hi = np.abs(_POS_VALUES[hi_c] - a)
    d_lo = np.abs(a - _POS_VALUES[lo_c])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    code = np.where(pick_hi, hi_c, lo_c).astype(np.int64)
    code = np.where(a >= E4M3_MAX, E4M3_MAX_CODE, code)
    code = np.where(sign, code | 0x80, code)
    code = np.where(np.isnan(y), E4M3_NAN_CODE, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# generic storage decode
# --------------------------------------------------------------------------

STORAGE_NUMPY_DTYPE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def decode_storage(arr: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Storage array -> exact fp64 values (fp8 codes times their fp32 scale)."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "fp8":
        return e4m3_decode(arr, scale)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def encode_storage(values: np.ndarray, src_dtype: str, dst_dtype: str, scale: float = 1.0) -> np.ndarray:
    """Convert stored values of ``src_dtype`` into ``dst_dtype`` storage.

    Identity when the two dtypes match (bits are copied); fp32 -> bf16 rounds
    to nearest even; f32/bf16 -> fp8 divides by ``scale`` in fp32 and rounds
    to E4M3FN with saturation.  Other pairs are not part of the method.
    """
    if src_dtype == dst_dtype:
        return np.array(values, dtype=STORAGE_NUMPY_DTYPE[dst_dtype], copy=True)
    if src_dtype == "f32" and dst_dtype == "bf16":
        return f32_to_bf16_bits(values)
    if dst_dtype == "fp8" and src_dtype in ("f32", "bf16"):
        x32 = decode_storage(values, src_dtype).astype(np.float32)  # exact
        return e4m3_encode(x32, scale)
    raise ValueError(f"unsupported conversion {src_dtype} -> {dst_dtype}")
