"""Number formats used by the method, in plain float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
imports this module.

Formats
-------
* bf16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits.  Values are
  carried as uint16 bit patterns.  ``bf16_round`` rounds a float64 straight to
  bf16 with round-to-nearest-even (one rounding, never via fp32).
* fp32: ``fl32`` is a single IEEE round-to-nearest-even to binary32.
* e4m3: the OCP 8-bit "E4M3FN" format that the speedrun pages call
  ``float8_e4m3`` (NanoGPT Speedrun (Track 1), "Changes vs Record #83" item 1
  and "Approach" item 5): 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
  infinities, NaN = S.1111.111, largest finite 448, smallest subnormal 2^-9.
  The encoder rounds to nearest even and saturates (|v| >= 448, infinities
  included, -> +-448), keeps the sign of zero, and maps NaN to 0x7F / 0xFF.
"""
import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------
def bf16_to_f64(bits):
    """Exact decode of uint16 bf16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round(x):
    """Round float64 values to bf16, round-to-nearest-even, one rounding.

    Returns uint16 bit patterns.  Overflow goes to +-inf (IEEE RNE), values
    below half the smallest subnormal go to signed zero, NaN -> 0x7FC0|sign.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.signbit(x)
    finite = np.isfinite(a)
    af = np.where(finite, a, 0.0)
    _, e2 = np.frexp(af)                 # af = f * 2**e2, f in [0.5, 1)
    # quantum of bf16 at this magnitude: 8 significant bits, exponent >= -126
    q_exp = np.maximum(e2 - 8, -133)
    q = np.ldexp(1.0, q_exp)
    r = np.rint(af / q) * q              # np.rint: ties to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(finite, r, a)
    out = np.where(sign, -r, r).astype(np.float32).view(np.uint32)
    out = (out >> 16).astype(np.uint16)
    nan = np.isnan(x)
    out = np.where(nan, np.where(sign, 0xFFC0, 0x7FC0), out).astype(np.uint16)
    return out


def bf16(x):
    """float64 -> bf16 (RNE) -> float64."""
    return bf16_to_f64(bf16_round(x))


# --------------------------------------------------------------------------
# fp32
# --------------------------------------------------------------------------
def fl32(x):
    """One IEEE round-to-nearest-even to binary32, returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# OCP e4m3 (E4M3FN)
# --------------------------------------------------------------------------
def _e4m3_table():
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * m * 2.0 ** -9          # subnormal: m/8 * 2^-6
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _e4m3_table()


def e4m3_decode(codes):
    """Exact decode of uint8 e4m3 codes to float64 (NaN for 0x7F / 0xFF)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v):
    """Encode float64 values to e4m3 codes: RNE, saturate to +-448.

    Steps, for a = |v|:
      * NaN                    -> 0x7F (sign kept in bit 7)
      * a >= 448 (inf too)     -> 0x7E (saturate to the largest finite)
      * a <  2^-6 (subnormal)  -> k = rint(a / 2^-9); the code is k itself,
                                  and k == 8 lands on the smallest normal 0x08
      * otherwise              -> e = floor(log2 a), m = rint(a / 2^(e-3)) in
                                  [8, 16]; m == 16 carries into e + 1;
                                  code = ((e + 7) << 3) | (m - 8)
    The sign bit is kept for every input, zero included (-0.0 -> 0x80).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    nan = np.isnan(v)
    a0 = np.where(nan, 0.0, a)
    sat = a0 >= E4M3_MAX
    a1 = np.where(sat, 1.0, a0)
    sub = a1 < 2.0 ** -6
    # subnormal branch
    k = np.rint(a1 / 2.0 ** -9)
    code_sub = k
    # normal branch
    _, e2 = np.frexp(np.where(sub, 1.0, a1))
    e = e2 - 1                                   # a1 = 1.x * 2^e
    m = np.rint(np.where(sub, 8.0, a1) / np.ldexp(1.0, e - 3))
    carry = m >= 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    code_norm = ((e + 7) << 3) | (m.astype(np.int64) - 8)
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)
