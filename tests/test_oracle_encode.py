"""Pins of the oracle's KV encoders against the format definitions and torch's CPU casts.

bf16: round to nearest, ties to even, checked by a nearest-value search over
both bf16 neighbours of every input (a different method from the oracle's
add-and-truncate), on every upper-half bit pattern crossed with the tie-critical
lower halves.  fp8 e4m3fn: the 256-code table against its closed form and
torch's decode; the encoder against a brute-force nearest search over all
finite codes and against torch's cast (round to nearest even, which does not
saturate, hence the inputs stay within +-448).
"""
import numpy as np
import pytest
import torch

from oracle import encode as E


# ------------------------------------------------------------------- bf16
def _bf16_nearest_by_search(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 of each finite f32 by comparing both neighbours (ties: even pattern)."""
    u = x.view(np.uint32).astype(np.uint64)
    t = (u & np.uint64(0xFFFF0000)) >> np.uint64(16)  # truncated toward zero
    n = t + np.uint64(1)                               # next magnitude up
    def val(bits):
        b = bits.astype(np.uint64)
        exp_all_ones = ((b >> np.uint64(7)) & np.uint64(0xFF)) == np.uint64(0xFF)
        f = (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        # the step past the largest finite bf16 lands on 2^128 for distance purposes
        sign = np.where((b >> np.uint64(15)) & np.uint64(1), -1.0, 1.0)
        return np.where(exp_all_ones, sign * 2.0 ** 128, f)
    xv = x.astype(np.float64)
    dt, dn = np.abs(xv - val(t)), np.abs(val(n) - xv)
    pick_n = (dn < dt) | ((dn == dt) & ((n & np.uint64(1)) == 0))
    return np.where(pick_n, n, t).astype(np.uint16)


def _strata():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFE, 0xFFFF],
                    dtype=np.uint32)
    rnd = np.random.default_rng(7).integers(0, 1 << 16, size=6, dtype=np.uint32)
    bits = (hi[:, None] | np.concatenate([lows, rnd])[None, :]).reshape(-1)
    return bits.view(np.float32)


def test_bf16_matches_nearest_search_on_all_upper_halves():
    x = _strata()
    fin = np.isfinite(x)
    got = E.bf16_bits(x[fin])
    want = _bf16_nearest_by_search(x[fin])
    assert np.array_equal(got, want)


def test_bf16_matches_torch_cast():
    x = _strata()
    fin = np.isfinite(x)
    t = torch.from_numpy(x[fin].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(E.bf16_bits(x[fin]), t)


def test_bf16_special_values():
    x = np.array([1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 3.4028235e38], dtype=np.float32)
    assert E.bf16_bits(x).tolist() == [0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x7F80]
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1 (even); 1 + 3*2^-8 -> 1 + 2^-6
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], dtype=np.float32)
    assert E.bf16_bits(x).tolist() == [0x3F80, 0x3F82]
    nan = E.bf16_bits(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all(E.bf16_value(nan) != E.bf16_value(nan))  # still NaN
    assert (int(nan[1]) >> 15) == 1


def test_bf16_value_is_exact_widening():
    bits = np.arange(1 << 16, dtype=np.uint16)
    v = E.bf16_value(bits)
    fin = np.isfinite(v)
    assert np.array_equal(E.bf16_bits(v[fin].astype(np.float32)), bits[fin])


# -------------------------------------------------------------- fp8 table
def test_fp8_table_closed_form_points():
    t = E.FP8_E4M3FN
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0                  # exponent field 7 = bias
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)       # positive codes ordered by value
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])


def test_fp8_table_matches_torch_decode():
    tt = torch.tensor(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    t = E.FP8_E4M3FN
    both_nan = np.isnan(tt) & np.isnan(t)
    assert np.all((tt == t) | both_nan)


# ------------------------------------------------------------ fp8 encoder
def _fp8_brute(x: np.ndarray) -> np.ndarray:
    """Argmin over every finite code; among equally near codes take the even one."""
    t = E.FP8_E4M3FN
    codes = np.array([c for c in range(256) if not np.isnan(t[c])])
    vals = t[codes]
    xv = x.astype(np.float64)
    d = np.abs(xv[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # prefer: same sign as x (for zero), then even code
    same_sign = (codes[None, :] >= 0x80) == np.signbit(x)[:, None]
    even = (codes[None, :] & 1) == 0
    score = cand * (4 + 2 * same_sign + even)
    return codes[np.argmax(score, axis=1)].astype(np.uint8)


def _fp8_midpoints():
    pos = E.FP8_E4M3FN[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(-np.inf))
    x = np.concatenate([pos.astype(np.float32), mid, up, dn, [np.float32(448.0)]])
    x = x[np.abs(x) <= 448]
    return np.concatenate([x, -x])


def test_fp8_code_matches_brute_force():
    rng = np.random.default_rng(11)
    x = np.concatenate([_fp8_midpoints(), rng.uniform(-448, 448, 50000).astype(np.float32),
                        (rng.standard_normal(50000) * 0.05).astype(np.float32)])
    assert np.array_equal(E.fp8_code(x), _fp8_brute(x))


def test_fp8_code_matches_torch_cast_on_1e7_values():
    rng = np.random.default_rng(12)
    x = np.concatenate([_fp8_midpoints(), rng.uniform(-448, 448, 5_000_000).astype(np.float32),
                        (rng.standard_normal(5_000_000) * 3).astype(np.float32)])
    x = np.clip(x, -448, 448)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(E.fp8_code(x), t)


def test_fp8_code_rejects_out_of_range():
    with pytest.raises(ValueError):
        E.fp8_code(np.array([449.0], dtype=np.float32))
    with pytest.raises(ValueError):
        E.fp8_code(np.array([np.nan], dtype=np.float32))


# ------------------------------------------------------- fp8 row quantiser
def test_fp8_rows_absmax_maps_to_448_and_codes_are_nearest():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((4000, 128)).astype(np.float32) * rng.uniform(1e-3, 1e3, (4000, 1)).astype(np.float32)
    codes, scale = E.fp8_quantize_rows(x)
    assert scale.dtype == np.float32
    i = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(len(x)), i]
    assert np.all((top == 0x7E) | (top == 0xFE))
    # every code is the brute-force nearest code of the f32 quotient x / scale
    y = np.clip((x / scale[:, None]).astype(np.float32), -448, 448)
    sub = slice(0, 300)
    assert np.array_equal(codes[sub].reshape(-1), _fp8_brute(y[sub].reshape(-1)))
    # scale is the f32 quotient absmax / 448: 448 * scale brackets absmax within one f32 ulp
    a = np.abs(x).max(axis=1).astype(np.float64)
    s = scale.astype(np.float64)
    assert np.all(np.abs(448.0 * s - a) <= np.spacing(a.astype(np.float32)).astype(np.float64) * 448 / 2 + 1e-300)
    # reconstruction error within half a code step
    rec = E.fp8_value(codes) * s[:, None]
    mag = (codes & 0x7F).astype(np.int64)
    up = E.fp8_value(np.minimum(mag + 1, 0x7E)) - E.fp8_value(mag)
    down = E.fp8_value(mag) - E.fp8_value(np.maximum(mag - 1, 0))
    step = np.maximum(up, down)
    assert np.all(np.abs(rec - x) <= 0.5 * step * s[:, None] * (1 + 1e-6) + 1e-300)


def test_fp8_rows_zero_row_has_scale_one():
    codes, scale = E.fp8_quantize_rows(np.zeros((3, 64), dtype=np.float32))
    assert np.all(scale == 1.0) and np.all((codes & 0x7F) == 0)


def test_fp8_rows_quarter_of_f32_bytes():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))
    x = np.ones((8, 128), dtype=np.float32)
    codes, _ = E.fp8_quantize_rows(x)
    assert codes.nbytes / x.nbytes == g["fp8_pool_quarter"]["ratio"]
    assert E.fp8_value(np.array([0x7E]))[0] == g["fp8_scale_rule"]["max_code_value"]


def test_fp8_unscaled_is_the_nearest_code_of_the_clamped_value():
    """Page section 6, FP8 KV cache paragraph: no scale, values clamped to +-448 and
    converted; checked by brute-force nearest search over the 254 finite codes (ties
    to the even code), including values far beyond 448 and below the smallest
    subnormal."""
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(20000) * rng.choice([1e-3, 1.0, 30.0, 1e3], 20000),
                        [448.0, 449.0, 464.0, 1e6, -1e6, 2.0 ** -10, -(2.0 ** -10), 0.0, -0.0]]).astype(np.float32)
    codes = E.fp8_unscaled(x)
    table = E.fp8_value(np.arange(256, dtype=np.uint8))
    finite = np.nonzero(np.isfinite(table))[0]
    for xi, ci in zip(x[:3000].tolist() + x[-9:].tolist(), codes[:3000].tolist() + codes[-9:].tolist()):
        y = min(max(xi, -448.0), 448.0)
        d = np.abs(table[finite] - y)
        best = finite[d == d.min()]
        if len(best) > 1:  # a tie: the even code (mantissa lsb 0), sign from y
            best = [b for b in best if (b & 1) == 0 and (b >> 7) == (1 if np.signbit(y) else 0)] or best
        assert E.fp8_value(np.array([ci], np.uint8))[0] == table[best[0]], (xi, ci, best)
    assert codes[-6] == 0x7E and codes[-5] == 0xFE  # 1e6 and -1e6 saturate to +-448
    raw, sc = E.encode_kv(x.reshape(-1, 1), "fp8u")
    assert sc is None and np.array_equal(E.kv_values(raw, None, "fp8u").reshape(-1), E.fp8_value(codes))


def test_int8_rows_follow_the_formula_by_plain_python():
    """int8 KV rows (the pages' int8 formula per (token, kv head) row): recomputed with
    Python floats and round() (ties to even), independent of numpy's rint; the absmax
    element maps to +-127 exactly; an all-zero row has scale 1 and codes 0."""
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((300, 64)) * rng.choice([1e-3, 1.0, 50.0], (300, 1))).astype(np.float32)
    x[5] = 0.0
    x[7, :4] = [2.5, -2.5, 1.0, 0.5]  # exact ties after the divide when absmax = 127 * 2^k
    x[7, 4:] = 0.0
    x[7, 10] = 127.0 / 64
    codes, scale = E.int8_quantize_rows(x)
    for r in range(x.shape[0]):
        a = max(abs(float(v)) for v in x[r])
        s = np.float32(1.0) if a == 0 else np.float32(np.float32(a) / np.float32(127.0))
        assert scale[r] == s
        for d in range(x.shape[1]):
            y = float(np.float32(x[r, d] / s))
            want = max(-127, min(127, round(y)))  # Python's round: half to even
            assert codes[r, d] == want, (r, d, x[r, d], y, codes[r, d], want)
        if a > 0:
            i = int(np.argmax(np.abs(x[r])))
            assert abs(int(codes[r, i])) == 127
    assert scale[5] == 1.0 and np.all(codes[5] == 0)
    raw, sc = E.encode_kv(x, "int8")
    assert raw.dtype == np.int8 and np.array_equal(raw, codes) and np.array_equal(sc, scale)
    v = E.kv_values(raw, sc, "int8")
    assert np.all(np.abs(v - x) <= scale[:, None].astype(np.float64) * 0.5 + 1e-12)
