"""Number formats of the oracle: bf16, OCP e4m3fn and E8M0 block scales.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain CPU oracle that the
GPU library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
never does.  It shares no code with the HIP library.

Everything here works on float64 values and plain integer bit patterns, and
every rounding is done by exact power-of-two scaling followed by numpy's
round-half-to-even (``np.rint``), so each result can be checked by hand.

Formats, as the fusion-kernels pages use them ("Boosting MoE Training
Throughput with Advanced Fusion Kernels", section "Fusionando cuantización
MXFP8 y NVFP4": the activation output is BF16 and the quantised copy is
MXFP8 with 1x32 blocks and E8M0 scales):

* bf16: 1 sign, 8 exponent, 7 stored mantissa bits; same exponent range as
  fp32 (normals down to 2^-126, subnormals down to 2^-133).
* e4m3fn (OCP 8-bit float, "fn" = finite, no infinity): exponent bias 7,
  largest finite value 448 = 1.75 * 2^8, S.1111.111 is NaN, subnormals are
  m * 2^-9 for m = 1..7.
* e5m2 (OCP 8-bit float for gradients): exponent bias 15, largest finite
  value 57344 = 1.75 * 2^15, S.11111.00 is infinity and S.11111.xx (xx != 0)
  NaN, subnormals are m * 2^-16 for m = 1..3.  Used for the MXFP8 copies of
  gradients (the E5M2 option of the MXFP8 recipe); the block scale rule is
  the e4m3 one with 57344 in place of 448.
* E8M0: an unsigned biased exponent, value 2^(byte - 127); 0xFF is NaN.
"""
from __future__ import annotations

import numpy as np

BF16_MIN_NORMAL_EXP = -126
E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6
E5M2_MAX = 57344.0
E5M2_MIN_NORMAL_EXP = -14
E8M0_NAN = 0xFF


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """Exact floor(log2(a)) for finite a > 0 (frexp gives a = f*2^p, f in [0.5, 1))."""
    _, p = np.frexp(a)
    return p.astype(np.int64) - 1


# ----------------------------------------------------------------------------- bf16

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64 (exact: bf16 is a prefix of fp32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (RNE).

    The quantum of a bf16 number with floor(log2|x|) = p is 2^(max(p,-126)-7);
    dividing by it is exact, np.rint rounds half to even, and multiplying back
    is exact.  Magnitudes that round to 2^128 or beyond become infinities,
    NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    a = np.abs(x[fin])
    p = np.maximum(_floor_log2(a), BF16_MIN_NORMAL_EXP)
    q = np.ldexp(1.0, p - 7)
    r = np.rint(a / q) * q
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    out[fin] = np.copysign(r, x[fin])
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """Encode float64 to bf16 bit patterns with round-to-nearest-even.

    The rounded value is exactly representable in fp32, so its top 16 bits are
    the bf16 pattern.  NaN maps to the canonical quiet NaN 0x7FC0.
    """
    r = bf16_round(x)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(r), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


# ----------------------------------------------------------------------------- e4m3fn

def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 e4m3fn codes (float64; NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_TABLE = e4m3_decode_table()


def e4m3_decode(codes) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes).astype(np.int64)]


def e4m3_round(x) -> np.ndarray:
    """Round float64 to the nearest e4m3fn value, ties to even, saturating at +-448.

    The quantum for floor(log2|x|) = p is 2^(max(p,-6)-3) (3 stored mantissa
    bits, subnormal quantum 2^-9).  Magnitudes above 448 saturate to 448 (the
    scale rule below never produces them; saturation is the OCP "satfinite"
    choice).  The sign of the input is kept, also on a result of zero.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.zeros_like(a)
    nz = a > 0
    p = np.maximum(_floor_log2(a[nz]), E4M3_MIN_NORMAL_EXP)
    q = np.ldexp(1.0, p - 3)
    out[nz] = np.minimum(np.rint(a[nz] / q) * q, E4M3_MAX)
    return np.copysign(out, x)


def f64_to_e4m3(x) -> np.ndarray:
    """Encode float64 values to e4m3fn codes (uint8), RNE, saturating, sign kept.

    NaN inputs give the NaN code 0x7F (0xFF when the sign bit is set).
    """
    x = np.asarray(x, dtype=np.float64)
    r = e4m3_round(np.where(np.isnan(x), 0.0, x))
    a = np.abs(r)
    code = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    p = np.maximum(_floor_log2(a[nz]), E4M3_MIN_NORMAL_EXP)
    mant = np.rint(a[nz] / np.ldexp(1.0, p - 3)).astype(np.int64)  # 8..15 normal, 1..7 subnormal
    is_norm = mant >= 8
    code_nz = np.where(is_norm, ((p + 7) << 3) + (mant - 8), mant)
    code[nz] = code_nz
    code = code | np.where(np.signbit(r), 0x80, 0)
    code = np.where(np.isnan(x), np.where(np.signbit(x), 0xFF, 0x7F), code)
    return code.astype(np.uint8)


def e4m3_ulp(v) -> np.ndarray:
    """Spacing of e4m3fn numbers at |v| (|v| <= 448): 2^(max(floor(log2|v|),-6)-3)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    p = np.full(a.shape, E4M3_MIN_NORMAL_EXP, dtype=np.int64)
    nz = a > 0
    p[nz] = np.maximum(_floor_log2(a[nz]), E4M3_MIN_NORMAL_EXP)
    return np.ldexp(1.0, p - 3)


# ----------------------------------------------------------------------------- e5m2

def e5m2_decode_table() -> np.ndarray:
    """Value of each of the 256 e5m2 codes (float64; +-inf for S.11111.00, NaN for
    the other S.11111.xx codes)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 2) & 0x1F
        m = c & 0x3
        if e == 0x1F:
            vals[c] = s * np.inf if m == 0 else np.nan
        elif e == 0:
            vals[c] = s * (m / 4.0) * 2.0 ** -14
        else:
            vals[c] = s * (1.0 + m / 4.0) * 2.0 ** (e - 15)
    return vals


_E5M2_TABLE = e5m2_decode_table()


def e5m2_decode(codes) -> np.ndarray:
    return _E5M2_TABLE[np.asarray(codes).astype(np.int64)]


def e5m2_round(x) -> np.ndarray:
    """Round float64 to the nearest e5m2 value, ties to even, saturating at +-57344
    (2 stored mantissa bits: the quantum for floor(log2|x|) = p is
    2^(max(p,-14)-2), subnormal quantum 2^-16).  The sign is kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.zeros_like(a)
    nz = a > 0
    p = np.maximum(_floor_log2(a[nz]), E5M2_MIN_NORMAL_EXP)
    q = np.ldexp(1.0, p - 2)
    out[nz] = np.minimum(np.rint(a[nz] / q) * q, E5M2_MAX)
    return np.copysign(out, x)


def f64_to_e5m2(x) -> np.ndarray:
    """Encode float64 values to e5m2 codes (uint8), RNE, saturating, sign kept;
    NaN gives 0x7F (0xFF with the sign bit set)."""
    x = np.asarray(x, dtype=np.float64)
    r = e5m2_round(np.where(np.isnan(x), 0.0, x))
    a = np.abs(r)
    code = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    p = np.maximum(_floor_log2(a[nz]), E5M2_MIN_NORMAL_EXP)
    mant = np.rint(a[nz] / np.ldexp(1.0, p - 2)).astype(np.int64)   # 4..7 normal, 1..3 subnormal
    code[nz] = np.where(mant >= 4, ((p + 15) << 2) + (mant - 4), mant)
    code = code | np.where(np.signbit(r), 0x80, 0)
    code = np.where(np.isnan(x), np.where(np.signbit(x), 0xFF, 0x7F), code)
    return code.astype(np.uint8)


def e5m2_ulp(v) -> np.ndarray:
    """Spacing of e5m2 numbers at |v| (|v| <= 57344): 2^(max(floor(log2|v|),-14)-2)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    p = np.full(a.shape, E5M2_MIN_NORMAL_EXP, dtype=np.int64)
    nz = a > 0
    p[nz] = np.maximum(_floor_log2(a[nz]), E5M2_MIN_NORMAL_EXP)
    return np.ldexp(1.0, p - 2)


FP8_FORMATS = {"e4m3": (E4M3_MAX, 8), "e5m2": (E5M2_MAX, 15)}   # (largest value, its exponent)


# ----------------------------------------------------------------------------- E8M0 scale

def mx_scale_exponent(amax, fmt: str = "e4m3") -> np.ndarray:
    """Block scale exponent E for block maxima ``amax`` (float64, >= 0).

    E is the smallest integer with amax / 2^E <= vmax (448 for e4m3, 57344 for
    e5m2), i.e. ceil(log2(amax/vmax)), clamped to [-127, 127].  An all-zero
    block gets E = -127.  This "round the scale up" rule guarantees every
    scaled element is within the element format's finite range, so
    dequantize(quantize(v)) is within half an ulp times 2^E of v.  Non-finite
    amax is reported as E = 128 (byte 0xFF, NaN).
    """
    vmax, vexp = FP8_FORMATS[fmt]
    a = np.asarray(amax, dtype=np.float64)
    E = np.full(a.shape, -127, dtype=np.int64)
    fin = np.isfinite(a)
    pos = fin & (a > 0)
    ap = a[pos]
    e = _floor_log2(ap) - vexp       # vmax * 2^(floor(log2 a) - vexp) lies in [0.875, 1.75) * a
    # step up until amax <= vmax * 2^e, then down while the next lower power still fits
    for _ in range(3):
        e = np.where(ap > vmax * np.ldexp(1.0, e), e + 1, e)
    for _ in range(3):
        e = np.where(ap <= vmax * np.ldexp(1.0, e - 1), e - 1, e)
    E[pos] = np.clip(e, -127, 127)
    E[~fin] = 128
    return E


def e8m0_byte(E) -> np.ndarray:
    E = np.asarray(E, dtype=np.int64)
    return np.where(E >= 128, E8M0_NAN, E + 127).astype(np.uint8)


def e8m0_value(byte) -> np.ndarray:
    b = np.asarray(byte).astype(np.int64)
    return np.where(b == E8M0_NAN, np.nan, np.ldexp(1.0, b - 127))


def mx_quantize_block(v, fmt: str = "e4m3") -> tuple[np.ndarray, int]:
    """Quantise one block of values (float64, already bf16-rounded) to MXFP8.

    Returns (element codes, E8M0 byte).  Elements are v * 2^-E rounded RNE to
    e4m3fn (or e5m2); the multiply by a power of two is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    amax = np.max(np.abs(v)) if v.size else 0.0
    E = int(mx_scale_exponent(np.array([amax]), fmt)[0])
    if E == 128:
        return np.full(v.shape, 0x7F, dtype=np.uint8), E8M0_NAN
    enc = f64_to_e4m3 if fmt == "e4m3" else f64_to_e5m2
    return enc(np.ldexp(v, -E)), E + 127


def fp8_decode(codes, fmt: str = "e4m3") -> np.ndarray:
    return e4m3_decode(codes) if fmt == "e4m3" else e5m2_decode(codes)
