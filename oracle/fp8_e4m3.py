"""OCP FP8 E4M3 ("e4m3fn") decode and encode.  Oracle / test infrastructure.

InferX ("The kernels underneath", FP8 KV cache paragraph) stores K and V as
fp8 e4m3 with per-layer scales frozen at warm-up; the chunked-prefill workload
here quantises each KV head with an fp32 scale equal to absmax/448, which only
fits the OCP "fn" variant (largest finite magnitude 448, no infinities).

Format, from the OCP 8-bit floating point specification:

* bit 7 sign, bits 6..3 exponent E (bias 7), bits 2..0 mantissa M;
* E == 0:       value = (-1)^s * (M / 8) * 2^(1 - 7)   (subnormal, incl. +-0)
* 0 < E:        value = (-1)^s * (1 + M / 8) * 2^(E - 7)
* E == 15, M == 7 (0x7F, 0xFF): NaN.  There is no infinity.

Encoding reading (the pages name only "e4m3"; this is the plainest reading):

* y = float32(x) / float32(scale), one correctly rounded IEEE binary32 divide;
* |y| is rounded to the nearest finite E4M3 magnitude, ties to the code with an
  even mantissa (round-to-nearest-even);
* magnitudes above 448 saturate to 448 ("satfinite"), +-inf included;
* the sign of y is kept, so a negative value that rounds to zero gives 0x80;
* NaN encodes as 0x7F.
"""

import numpy as np

NAN_CODE = 0x7F
MAX_FINITE = 448.0


def decode_code(code):
    """Exact value of one E4M3 code (0..255) as a Python float."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError("E4M3 codes are bytes")
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - 7)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return sign * mag


DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes, indexed by code 0x00..0x7E.  The codes of a
# given sign are ordered like their magnitudes, so this array is increasing.
_POS_MAGNITUDES = DECODE_TABLE[:0x7F].copy()


def decode(codes):
    """uint8 array of E4M3 codes -> float64 array (exact)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x, scale=1.0):
    """Quantise ``x / scale`` to E4M3 codes (uint8), per the module docstring.

    ``x`` is converted to float32 first (bf16 and fp32 inputs are exact in
    float32); ``scale`` is a float32 scalar or an array broadcastable to x.
    """
    xf = np.asarray(x, dtype=np.float32)
    sf = np.asarray(scale, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (xf / sf).astype(np.float32)          # IEEE binary32 divide
    mag = np.abs(y.astype(np.float64))
    nan = np.isnan(y)
    mag_ok = np.where(nan, 0.0, mag)

    # Nearest neighbours in the magnitude table: lo <= |y| <= hi.
    hi = np.searchsorted(_POS_MAGNITUDES, mag_ok, side="left")
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = mag_ok - _POS_MAGNITUDES[lo]
    d_hi = _POS_MAGNITUDES[hi] - mag_ok
    # Choose the nearer one; on an exact tie choose the even code.
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    # |y| equal to a table entry: d_hi == 0 picks hi (the entry itself).
    code = np.where(_POS_MAGNITUDES[hi] == mag_ok, hi, code)
    # Saturate beyond the largest finite magnitude (searchsorted clipped hi).
    code = np.where(mag_ok > MAX_FINITE, 0x7E, code).astype(np.uint8)

    neg = np.signbit(y)
    code = np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(nan, np.uint8(NAN_CODE), code).astype(np.uint8)
    return code

