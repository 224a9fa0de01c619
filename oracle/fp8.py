"""MX-FP8 (OCP e4m3 elements with one power-of-two scale per 32 values) quantisation and the
expert FFN on quantised operands, in exact / fp64 arithmetic. TEST INFRASTRUCTURE ONLY (see
the package docstring).

Definitions followed:
  * FP8 training and serving of MoE layers spends much of its time in quantise /
    dequantise and data movement next to the GEMMs, which fused FP8 MoE designs remove
    ([EP-wiki] 关键观察, observation 3; FP8FlowMoE among the papers citing the concept).
  * E4M3 (OCP 8-bit floating point, "fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent field 0 encodes subnormals m/8 * 2^-6; the largest finite value is
    1.75 * 2^8 = 448 (code 0x7E); code 0x7F (and 0xFF) is NaN; there is no infinity.
  * MX block scaling (OCP Microscaling): a block of 32 values shares the scale 2^X with
    X = floor(log2(max |v|)) - 8 (8 = the largest exponent of an E4M3 normal), stored as
    an 8-bit biased exponent (E8M0, bias 127); each value is v / 2^X rounded to E4M3.

Readings where the definitions leave a choice:
  * Rounding to E4M3 is to nearest, ties to the even code (even mantissa); magnitudes
    above 448 saturate to 448 (as the MX conversion allows), never NaN.
  * The sign bit is the sign of v, also when v rounds to zero (-0 -> 0x80).
  * A block whose values are all zero gets X = -127 (scale byte 0); X is clamped to
    [-127, 127].
  * Blocks run along the reduction dimension: 32 consecutive columns of a row of x, of a
    gated-product row, of a weight row.

Pins (tests/test_oracle_fp8.py): the E4M3 value table against its closed form and
torch.float8_e4m3fn (in range), every code round-trips, every midpoint goes to the even
code, saturation, the scale exponent at powers of two, and the quantisation error bound.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

E4M3_MAX_CODE = 0x7E


def e4m3_value(code):
    """Exact value of a non-NaN E4M3 code (0x00..0x7E, 0x80..0xFE)."""
    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 7
    if (code & 0x7F) == 0x7F:
        raise ValueError("NaN code")
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


_POS = [e4m3_value(c) for c in range(E4M3_MAX_CODE + 1)]   # increasing with the code


def e4m3_encode(v):
    """Code of v (a float): nearest E4M3 value, ties to the even code, |v| > 448 -> 448."""
    neg = math.copysign(1.0, v) < 0
    a = abs(Fraction(v))
    if a >= _POS[-1]:
        code = E4M3_MAX_CODE
    else:
        # brute force: the nearest of the 127 non-negative values; on a tie the even code
        best = None
        for c, val in enumerate(_POS):
            d = abs(val - a)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        code = best[1]
    return code | (0x80 if neg else 0)


_POS64 = np.array([float(v) for v in _POS])     # exact in fp64


def e4m3_encode_array(V):
    """e4m3_encode over an array of fp64 values (each exact): the nearest table value found
    by a sorted search, a midpoint going to the even code. The table values and their
    midpoints are exact in fp64, so every comparison is exact."""
    V = np.asarray(V, dtype=np.float64)
    neg = np.signbit(V)
    a = np.abs(V)
    hi = np.searchsorted(_POS64, a, side="left").clip(1, E4M3_MAX_CODE)   # _POS64[hi-1] < a <= ...
    lo = hi - 1
    dlo = a - _POS64[lo]
    dhi = _POS64[hi] - a
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= _POS64[-1], E4M3_MAX_CODE, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def mx_scale_exponent(block):
    """X of one block: floor(log2(max |v|)) - 8 (exact), -127 for an all-zero block,
    clamped to [-127, 127]."""
    amax = max(abs(Fraction(float(v))) for v in block)
    if amax == 0:
        return -127
    # floor(log2(amax)) exactly from the rational value
    e = amax.numerator.bit_length() - amax.denominator.bit_length()
    if Fraction(2) ** e > amax:
        e -= 1
    return max(-127, min(127, e - 8))


def mx_quantize_rows(X, block=32):
    """codes [rows][cols] uint8 and scale bytes [rows][cols/block] uint8 (X + 127). The
    values must be exact in fp64 (for example fp32 or bf16 inputs, or fp64 results)."""
    X = np.asarray(X, dtype=np.float64)
    rows, cols = X.shape
    assert cols % block == 0
    B = X.reshape(rows, cols // block, block)
    amax = np.abs(B).max(axis=2)
    _, e = np.frexp(amax)                       # amax = m 2^e, m in [0.5, 1)
    x = np.where(amax == 0, -127, np.clip(e - 1 - 8, -127, 127))
    scaled = B / np.exp2(x)[:, :, None]         # a power-of-two scaling: exact
    codes = e4m3_encode_array(scaled).reshape(rows, cols)
    return codes, (x + 127).astype(np.uint8)


_LUT = np.array([float(e4m3_value(c)) if (c & 0x7F) != 0x7F else np.nan for c in range(256)])


def mx_dequantize(codes, scales, block=32):
    """fp64 values codes * 2^(scale - 127) (exact in fp64)."""
    codes = np.asarray(codes)
    scales = np.asarray(scales).astype(np.int64)
    vals = _LUT[codes]
    return vals * np.repeat(np.exp2(scales - 127.0), block, axis=1)


def swiglu_ffn_mx(xq, xs, w13q, w13s, w2q, w2s):
    """One expert's SwiGLU FFN on MX-FP8 operands, with the gated product quantised to
    MX-FP8 (blocks of 32 along its columns) before the down projection, all else fp64:
      a, b = deq(x) deq(W_g)^T, deq(x) deq(W_u)^T;  H = silu(a) * b;
      y = deq(q(H)) deq(W_d)^T.
    Returns (y, H, H codes, H scale bytes)."""
    x = mx_dequantize(xq, xs)
    w13 = mx_dequantize(w13q, w13s)
    w2 = mx_dequantize(w2q, w2s)
    inter = w13.shape[0] // 2
    a = x @ w13[:inter].T
    b = x @ w13[inter:].T
    H = a / (1.0 + np.exp(-a)) * b
    hq, hs = mx_quantize_rows(H)
    return mx_dequantize(hq, hs) @ w2.T, H, hq, hs
