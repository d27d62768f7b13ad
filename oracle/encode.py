"""KV storage encoders of the oracle: f32 copy, bf16, fp8 e4m3fn with a per-row scale,
and the pages' own unscaled fp8 e4m3fn.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it.

Sources (page "How serving works in Tlaloc"):
- section 2, the bf16 bullet: f32 values are rounded to bf16 (the same page,
  section 6 "Int8 weights", names round-half-even as its rounding rule);
- section 6 "Int8 weights", FP8 paragraph: e4m3fn codes, ``scale = max|x| / 448``,
  codes rounded to nearest even;
- section 6 "Int8 weights", FP8 KV cache paragraph: values clamped to +-448
  before the convert (e4m3fn has no infinity; 448 is its largest finite value).
  That paragraph's pool has no scale at all: a value is stored as itself, so one
  beyond +-448 saturates ("fp8u" below); the scaled form ("fp8") is the
  per-(token, head) scale of the fp8 decode workload.
- section 6 "Int8 weights", the int8 formula (scale = max|W| / 127 per output row, 1
  for an all-zero row; code = clamp(round_half_even(W / scale), -127, 127)).  The
  pages list int8 KV pools as not built; the reading here applies that formula to
  each stored (token, kv head) row ("int8" below), as the scaled fp8 pool does with
  448.
- section 6 "Int8 weights", the int8 formula: a scale of 1 for an all-zero row.

Everything here is written from the format definitions, not from a library
cast: the tests cross-check it against torch's CPU casts and against
brute-force nearest-value searches.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


# ------------------------------------------------------------------ bf16
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """f32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    bf16 keeps the top 16 bits of the f32 pattern.  Rounding adds half an ulp
    of the kept part (0x7FFF) plus the kept part's lowest bit, so an exact tie
    moves up only when that bit is 1 (odd).  NaN stays a quiet NaN with its sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = np.isnan(x)
    if np.any(nan):
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    return r.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> f64 values (exact widening)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


# ------------------------------------------------------------ fp8 e4m3fn
def _e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn code: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m/8 * 2^-6).  There are no infinities; the
    all-ones pattern S.1111.111 is NaN, so the largest finite value is
    1.75 * 2^8 = 448.
    """
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


FP8_E4M3FN = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)
# positive finite codes 0x00..0x7E are ordered by value
_POS = FP8_E4M3FN[:0x7F]


def fp8_value(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes -> f64 values."""
    return FP8_E4M3FN[np.asarray(codes, dtype=np.uint8)]


def fp8_code(x: np.ndarray) -> np.ndarray:
    """f32 values within [-448, 448] -> nearest e4m3fn code, ties to the even code.

    "Even" is the code whose lowest mantissa bit is 0.  The sign bit is the
    input's sign bit, so -0.0 and tiny negatives give 0x80.
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("fp8_code: non-finite input")
    mag = np.abs(x.astype(np.float64))
    if np.any(mag > FP8_MAX):
        raise ValueError("fp8_code: input beyond +-448 (clamp first)")
    hi = np.searchsorted(_POS, mag, side="left")  # first code with value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS[hi] - mag
    d_lo = mag - _POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    pick_hi |= _POS[lo] > mag  # hi == 0 case: mag == 0
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x)
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def fp8_quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row e4m3fn quantisation over the last axis.

    scale = f32(max|x| / 448) (an IEEE f32 divide; 1 for an all-zero row),
    code  = RNE_e4m3fn(clamp(f32(x / scale), -448, 448)).
    Returns (codes uint8 with x's shape, scales f32 with the last axis dropped).
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("fp8_quantize_rows: non-finite input")
    a = np.max(np.abs(x), axis=-1)
    scale = (a / np.float32(FP8_MAX)).astype(np.float32)
    scale = np.where(a == 0, np.float32(1.0), scale).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return fp8_code(y), scale


def int8_quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row int8 over the last axis: scale = f32(max|x| / 127) (IEEE f32 divide; 1
    for an all-zero row), code = clamp(round_half_even(f32(x / scale)), -127, 127)."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("int8_quantize_rows: non-finite input")
    a = np.max(np.abs(x), axis=-1)
    scale = (a / np.float32(127.0)).astype(np.float32)
    scale = np.where(a == 0, np.float32(1.0), scale).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    code = np.clip(np.rint(y), -127, 127).astype(np.int8)  # rint: round half to even
    return code, scale


def fp8_unscaled(x: np.ndarray) -> np.ndarray:
    """The pages' fp8 KV: code = RNE_e4m3fn(clamp(x, -448, 448)), no scale."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("fp8_unscaled: non-finite input")
    return fp8_code(np.clip(x, np.float32(-FP8_MAX), np.float32(FP8_MAX)))


# ------------------------------------------------------------- KV dtypes
def encode_kv(x: np.ndarray, kv_dtype: str) -> tuple[np.ndarray, np.ndarray | None]:
    """Encode f32 rows [..., D] for storage: (raw, scale or None)."""
    x = np.asarray(x, dtype=np.float32)
    if kv_dtype == "f32":
        return x.copy(), None
    if kv_dtype == "bf16":
        return bf16_bits(x), None
    if kv_dtype == "fp8":
        return fp8_quantize_rows(x)
    if kv_dtype == "fp8u":
        return fp8_unscaled(x), None
    if kv_dtype == "int8":
        return int8_quantize_rows(x)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def kv_values(raw: np.ndarray, scale: np.ndarray | None, kv_dtype: str) -> np.ndarray:
    """Stored rows widened exactly to f64 (fp8: code value times its f32 scale)."""
    if kv_dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return bf16_value(raw)
    if kv_dtype == "fp8":
        return fp8_value(raw) * np.asarray(scale, dtype=np.float64)[..., None]
    if kv_dtype == "fp8u":
        return fp8_value(raw)
    if kv_dtype == "int8":
        return np.asarray(raw, dtype=np.int8).astype(np.float64) * np.asarray(scale, dtype=np.float64)[..., None]
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


RAW_DTYPE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "fp8u": np.uint8, "int8": np.int8}
SCALED = ("fp8", "int8")  # dtypes stored with one f32 scale per (token, kv head)
