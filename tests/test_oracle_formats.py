"""Pins of the oracle's number formats (bf16, e4m3fn, E8M0) against exact
rational arithmetic, brute force over codebooks and published format tables.

None of these re-types the oracle's formulas: rounding is checked by
searching all representable values with Python's exact Fractions.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "number_formats.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _val(v):
    return float(v) if not isinstance(v, str) else float(v)


# ------------------------------------------------------------------ published values
def test_e4m3_table_matches_ocp_values():
    table = F.e4m3_decode_table()
    for item in _golden()["e4m3"]:
        code = int(item["code"], 16)
        v = _val(item["value"])
        if math.isnan(v):
            assert math.isnan(table[code])
        else:
            assert table[code] == v, (item, table[code])


def test_e4m3_table_structure():
    table = F.e4m3_decode_table()
    finite = table[np.isfinite(table)]
    assert len(finite) == 254                      # 256 codes minus two NaNs
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    pos = np.sort(np.unique(np.abs(finite)))
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9
    assert len(pos) == 127                         # +-0 share a value


def test_e8m0_values():
    for item in _golden()["e8m0"]:
        b = int(item["byte"], 16)
        v = _val(item["value"])
        got = F.e8m0_value(np.array([b]))[0]
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v


def test_bf16_golden():
    g = _golden()
    for item in g["bf16"]:
        bits = int(item["bits"], 16)
        v = _val(item["value"])
        assert F.bf16_bits_to_f64(np.array([bits], dtype=np.uint16))[0] == v
    for item in g["bf16_rounding"]:
        f32 = np.array([int(item["fp32_bits"], 16)], dtype=np.uint32).view(np.float32)
        got = F.f64_to_bf16_bits(f32.astype(np.float64))[0]
        assert got == int(item["bf16_bits"], 16), item


# ------------------------------------------------------------------ bf16 RNE, brute force
def _bf16_neighbours_exact(x: float):
    """The two bf16 values bracketing x, found from fp32 bit patterns."""
    f = np.array([x], dtype=np.float32).view(np.uint32)[0]
    lo_bits = (int(f) >> 16)
    cand = []
    for b in (lo_bits - 1, lo_bits, lo_bits + 1, lo_bits + 2):
        b &= 0xFFFF
        v = F.bf16_bits_to_f64(np.array([b], dtype=np.uint16))[0]
        if np.isfinite(v):
            cand.append((b, v))
    return cand


def _bf16_rne_bruteforce(x: float) -> float:
    cand = _bf16_neighbours_exact(x)
    fx = Fraction(x)
    best = min(abs(Fraction(v) - fx) for _, v in cand)
    ties = [(b, v) for b, v in cand if abs(Fraction(v) - fx) == best]
    if len(ties) == 1:
        return ties[0][1]
    even = [v for b, v in ties if (b & 1) == 0]
    return even[0]


def test_bf16_rne_random_against_exact_rationals():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32).astype(np.float64)
    xs = xs[np.isfinite(xs) & (np.abs(xs) < 3.0e38)]
    # add exact ties and near-ties
    ties = (rng.integers(0, 2 ** 16, size=500).astype(np.uint32) << 16) | 0x8000
    xs = np.concatenate([xs, ties.view(np.float32).astype(np.float64)])
    xs = xs[np.isfinite(xs) & (np.abs(xs) < 3.0e38)]
    got = F.bf16_round(xs)
    for x, g in zip(xs, got):
        assert g == _bf16_rne_bruteforce(float(x)), x


def test_bf16_specials():
    r = F.f64_to_bf16_bits(np.array([np.nan, np.inf, -np.inf, 0.0, -0.0]))
    assert r[0] == 0x7FC0 and r[1] == 0x7F80 and r[2] == 0xFF80
    assert r[3] == 0x0000 and r[4] == 0x8000


def test_bf16_matches_torch_cast_for_fp32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f64_to_bf16_bits(x.astype(np.float64)), t)


# ------------------------------------------------------------------ e4m3 RNE, brute force
_CODES = np.array([c for c in range(256) if np.isfinite(F.e4m3_decode_table()[c])])
_VALS = F.e4m3_decode_table()[_CODES]


def _e4m3_bruteforce(x: float):
    """Nearest finite e4m3 value to x by exhaustive search, ties to the even
    mantissa (even code), saturating at +-448."""
    fx = Fraction(x)
    if abs(x) > 448:
        return math.copysign(448.0, x)
    d = [abs(Fraction(v) - fx) for v in _VALS]
    best = min(d)
    idx = [i for i, di in enumerate(d) if di == best]
    vals = {float(_VALS[i]) for i in idx}
    if len(vals) == 1:
        v = vals.pop()
    else:
        v = [float(_VALS[i]) for i in idx if _CODES[i] % 2 == 0][0]
    return v


def test_e4m3_rne_dense_sweep():
    rng = np.random.default_rng(13)
    xs = np.concatenate([
        rng.uniform(-448, 448, 3000),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000),           # subnormal range
        (np.arange(-900, 901) / 2.0),                         # many exact ties between codes
        _VALS + np.ldexp(1.0, -12), _VALS - np.ldexp(1.0, -12),
    ])
    # midpoints between consecutive finite values: exact ties
    pos = np.sort(np.unique(np.abs(_VALS)))
    mids = (pos[:-1] + pos[1:]) / 2
    xs = np.concatenate([xs, mids, -mids])
    got = F.e4m3_round(xs)
    for x, g in zip(xs, got):
        assert g == _e4m3_bruteforce(float(x)), x


def test_e4m3_encode_decode_roundtrip_all_codes():
    codes = F.f64_to_e4m3(_VALS)
    # +0 and -0 keep their sign bit
    assert np.array_equal(codes, _CODES.astype(np.uint8))
    assert F.f64_to_e4m3(np.array([np.nan]))[0] == 0x7F
    assert F.f64_to_e4m3(np.array([-1e-9]))[0] == 0x80     # rounds to -0
    assert F.f64_to_e4m3(np.array([1000.0]))[0] == 0x7E    # saturates


def test_e4m3_torch_cast_cross_check_in_range():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    rng = np.random.default_rng(14)
    x = rng.uniform(-440, 440, 20000).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.f64_to_e4m3(x.astype(np.float64)), t)


# ------------------------------------------------------------------ E8M0 scale rule
def _ceil_log2_fraction(q: Fraction) -> int:
    """ceil(log2(q)) for a positive rational, exactly."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e < q:
        e += 1
    while Fraction(2) ** (e - 1) >= q:
        e -= 1
    return e


def test_scale_exponent_against_exact_ceil_log2():
    rng = np.random.default_rng(15)
    amax = np.concatenate([
        np.abs(rng.standard_normal(3000)) * np.exp2(rng.integers(-120, 120, 3000)),
        448.0 * np.exp2(np.arange(-100, 100, dtype=np.float64)),          # exact boundaries
        np.nextafter(448.0 * np.exp2(np.arange(-100, 100, dtype=np.float64)), np.inf),
        np.nextafter(448.0 * np.exp2(np.arange(-100, 100, dtype=np.float64)), 0),
    ])
    amax = F.bf16_round(amax)
    amax = amax[amax > 0]
    E = F.mx_scale_exponent(amax)
    for a, e in zip(amax, E):
        want = _ceil_log2_fraction(Fraction(float(a)) / 448)
        want = max(-127, min(127, want))
        assert e == want, (a, e, want)


def test_scale_exponent_edge_cases():
    assert F.mx_scale_exponent(np.array([0.0]))[0] == -127
    assert F.e8m0_byte(F.mx_scale_exponent(np.array([np.inf])))[0] == 0xFF
    assert F.mx_scale_exponent(np.array([448.0]))[0] == 0          # exactly representable
    assert F.mx_scale_exponent(np.array([448.0 * 2 ** 5]))[0] == 5
    assert F.mx_scale_exponent(np.array([np.nextafter(448.0, 1e9)]))[0] == 1
    assert F.mx_scale_exponent(np.array([1e-45]))[0] == -127       # clamps


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mx_block_roundtrip_within_half_ulp(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(300):
        scale = np.exp2(rng.integers(-40, 40))
        v = F.bf16_round(rng.standard_t(3, size=32) * scale)
        codes, byte = F.mx_quantize_block(v)
        X = F.e8m0_value(np.array([byte]))[0]
        deq = F.e4m3_decode(codes) * X
        assert np.all(np.abs(v / X) <= 448)
        bound = 0.5 * F.e4m3_ulp(v / X) * X
        assert np.all(np.abs(deq - v) <= bound)


def test_mx_block_edge_cases():
    z = np.zeros(32)
    codes, byte = F.mx_quantize_block(z)
    assert byte == 0 and np.all(codes == 0)
    one = np.zeros(32)
    one[7] = -3.0
    codes, byte = F.mx_quantize_block(one)
    X = F.e8m0_value(np.array([byte]))[0]
    assert F.e4m3_decode(codes)[7] * X == -3.0 and np.all(np.delete(codes, 7) == 0)
    b = np.full(32, 448.0 * 4)
    codes, byte = F.mx_quantize_block(b)
    assert byte == 127 + 2 and np.all(codes == 0x7E)


# ------------------------------------------------------------------ e5m2 (gradient format)
_CODES5 = np.array([c for c in range(256) if np.isfinite(F.e5m2_decode_table()[c])])
_VALS5 = F.e5m2_decode_table()[_CODES5]


def test_e5m2_table_matches_ocp_values():
    table = F.e5m2_decode_table()
    for item in _golden()["e5m2"]:
        code = int(item["code"], 16)
        v = float(item["value"])
        if math.isnan(v):
            assert math.isnan(table[code])
        else:
            assert table[code] == v, (item, table[code])


def test_e5m2_table_structure():
    table = F.e5m2_decode_table()
    assert len(_VALS5) == 248                      # 256 minus 2 infinities and 6 NaNs
    pos = np.sort(np.unique(np.abs(_VALS5)))
    assert pos[-1] == 57344.0 and pos[1] == 2.0 ** -16
    assert np.isinf(table[0x7C]) and np.isinf(table[0xFC])


def _e5m2_bruteforce(x: float):
    fx = Fraction(x)
    if abs(x) > 57344:
        return math.copysign(57344.0, x)
    d = [abs(Fraction(v) - fx) for v in _VALS5]
    best = min(d)
    idx = [i for i, di in enumerate(d) if di == best]
    vals = {float(_VALS5[i]) for i in idx}
    if len(vals) == 1:
        return vals.pop()
    return [float(_VALS5[i]) for i in idx if _CODES5[i] % 2 == 0][0]


def test_e5m2_rne_dense_sweep():
    rng = np.random.default_rng(23)
    pos = np.sort(np.unique(np.abs(_VALS5)))
    mids = (pos[:-1] + pos[1:]) / 2
    xs = np.concatenate([rng.uniform(-57344, 57344, 1500), rng.uniform(-2.0 ** -12, 2.0 ** -12, 1500),
                         rng.uniform(-8, 8, 1500), mids, -mids,
                         _VALS5 + np.ldexp(np.abs(_VALS5), -6), _VALS5 - np.ldexp(np.abs(_VALS5), -6)])
    got = F.e5m2_round(xs)
    for x, g in zip(xs, got):
        assert g == _e5m2_bruteforce(float(x)), x


def test_e5m2_encode_decode_roundtrip_all_codes():
    assert np.array_equal(F.f64_to_e5m2(_VALS5), _CODES5.astype(np.uint8))
    assert F.f64_to_e5m2(np.array([1e9]))[0] == 0x7B        # saturates (finite)
    assert F.f64_to_e5m2(np.array([-1e-12]))[0] == 0x80     # rounds to -0


def test_e5m2_torch_cast_cross_check_in_range():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e5m2"):
        pytest.skip("torch has no float8_e5m2")
    rng = np.random.default_rng(24)
    x = np.concatenate([rng.uniform(-57000, 57000, 10000), rng.uniform(-1, 1, 10000),
                        rng.uniform(-1e-4, 1e-4, 5000)]).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(F.f64_to_e5m2(x.astype(np.float64)), t)


def test_e5m2_scale_exponent_against_exact_ceil_log2():
    rng = np.random.default_rng(25)
    b = 57344.0 * np.exp2(np.arange(-120, 100, dtype=np.float64))
    amax = np.concatenate([np.abs(rng.standard_normal(2000)) * np.exp2(rng.integers(-120, 120, 2000)),
                           b, np.nextafter(b, np.inf), np.nextafter(b, 0)])
    amax = F.bf16_round(amax)
    amax = amax[amax > 0]
    E = F.mx_scale_exponent(amax, "e5m2")
    for a, e in zip(amax, E):
        want = max(-127, min(127, _ceil_log2_fraction(Fraction(float(a)) / 57344)))
        assert e == want, (a, e, want)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mx_block_e5m2_roundtrip_within_half_ulp(seed):
    rng = np.random.default_rng(seed + 40)
    v = F.bf16_round(rng.standard_normal(32) * np.exp2(rng.integers(-30, 30)))
    codes, byte = F.mx_quantize_block(v, "e5m2")
    X = F.e8m0_value(byte)
    back = F.e5m2_decode(codes) * X
    assert np.max(np.abs(v)) / X <= 57344
    p = np.maximum(np.floor(np.log2(np.maximum(np.abs(v) / X, 2.0 ** -30))), -14)
    assert np.all(np.abs(back - v) <= 0.5 * np.exp2(p - 2) * X + 0.0)
