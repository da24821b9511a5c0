"""Storage formats of the oracle: bfloat16 and float8 e4m3fn (TEST INFRASTRUCTURE).

Definitions followed (NumKong for Python page):

* "Scalar Types" table: ``bfloat16`` is 1+8+7 bits with Inf and NaN;
  ``float8_e4m3`` is 1+4+3 bits, range +-448, no Inf, NaN present.
* "ml_dtypes Interoperability" table: ``float8_e4m3`` is identical to
  ``ml_dtypes.float8_e4m3fn`` (exponent bias 7, the all-ones pattern
  ``S.1111.111`` is NaN, no infinities); the ``fnuz`` variants are rejected.
* "Buffer-First Casting": narrowing float conversion rounds to nearest,
  ties to even.

Rounding is done directly from float64 to the target grid (one rounding), with
``numpy.rint`` (round half to even) on the value scaled so that the target
ulp is 1.  e4m3 conversion saturates finite overflow at +-448 (the float8
kernels store ``x / scale`` with ``scale = absmax / 448``, so magnitudes never
exceed 448 by more than a rounding step).
"""

import numpy as np

BF16_MANT_BITS = 7
BF16_EMIN = -126                      # smallest normal is 2**-126
BF16_MAX = float.fromhex("0x1.fep127")  # (2 - 2**-7) * 2**127

E4M3_MANT_BITS = 3
E4M3_BIAS = 7
E4M3_EMIN = 1 - E4M3_BIAS             # smallest normal is 2**-6
E4M3_MAX = 448.0                      # 1.75 * 2**8
E4M3_NAN_CODE = 0x7F


def _round_to_grid(x, mant_bits, emin):
    """Round |x| (float64) to a binary grid with ``mant_bits`` stored mantissa
    bits and smallest normal 2**emin, ties to even.  Returns float64 |q|."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)                       # ax = m * 2**e, m in [0.5, 1)
    # the binade [2**(e-1), 2**e) has ulp 2**(e-1-mant_bits); below the
    # smallest normal the spacing stays that of the subnormals
    ulp_exp = np.maximum(e - 1 - mant_bits, emin - mant_bits)
    return np.ldexp(np.rint(np.ldexp(ax, -ulp_exp)), ulp_exp)


def bf16_round(x):
    """float64 -> nearest bfloat16 value (RNE, overflow to +-inf), as float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        q = _round_to_grid(np.where(np.isfinite(x), x, 0.0), BF16_MANT_BITS, BF16_EMIN)
        q = np.where(q > BF16_MAX, np.inf, q)
        q = np.copysign(q, x)
    q = np.where(np.isinf(x), x, q)
    return np.where(np.isnan(x), np.nan, q)


def bf16_bits(values):
    """bfloat16-representable float64 values -> uint16 bit patterns."""
    v = np.asarray(values, dtype=np.float64)
    bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), bits).astype(np.uint16)


def bf16_value(bits):
    """uint16 bfloat16 bit patterns -> float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_round(x):
    """float64 -> nearest float32 value (RNE), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def e4m3_round(x):
    """float64 -> nearest e4m3fn value, RNE, saturating at +-448, as float64."""
    x = np.asarray(x, dtype=np.float64)
    finite = np.where(np.isfinite(x), x, 0.0)
    q = _round_to_grid(finite, E4M3_MANT_BITS, E4M3_EMIN)
    q = np.minimum(q, E4M3_MAX)
    q = np.where(np.isinf(x), E4M3_MAX, q)
    q = np.copysign(q, x)
    return np.where(np.isnan(x), np.nan, q)


def e4m3_code(x):
    """float64 -> e4m3fn code byte (RNE, saturating; NaN -> 0x7F)."""
    x = np.asarray(x, dtype=np.float64)
    q = e4m3_round(x)
    aq = np.abs(np.where(np.isnan(q), 0.0, q))
    sign = np.signbit(q).astype(np.uint8) << 7
    _, e = np.frexp(aq)                        # aq = m * 2**e, m in [0.5, 1)
    unbiased = e - 1                           # aq in [2**unbiased, 2**(unbiased+1))
    normal = aq >= 2.0 ** E4M3_EMIN
    exp_field = np.where(normal, unbiased + E4M3_BIAS, 0)
    # normal: aq = (1 + M/8) * 2**unbiased ; subnormal: aq = M/8 * 2**EMIN
    mant_norm = np.ldexp(aq, -unbiased) * 8.0 - 8.0
    mant_sub = np.ldexp(aq, 3 - E4M3_EMIN)
    mant = np.where(normal, mant_norm, mant_sub)
    code = sign | (exp_field.astype(np.uint8) << 3) | np.rint(mant).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(E4M3_NAN_CODE) | sign, code).astype(np.uint8)


def e4m3_value(code):
    """e4m3fn code byte -> float64 value (NaN for S.1111.111)."""
    c = np.asarray(code).astype(np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    mant = c & 0x7
    normal = exp_field > 0
    mag = np.where(normal,
                   np.ldexp(1.0 + mant / 8.0, exp_field - E4M3_BIAS),
                   np.ldexp(mant / 8.0, E4M3_EMIN))
    val = sign * mag
    return np.where((exp_field == 0xF) & (mant == 0x7), np.nan, val)


def storage_round(x, dtype):
    """Round float64 values to what a ``dtype`` store holds ('f32' or 'bf16')."""
    if dtype == "f32":
        return f32_round(x)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(f"no plain rounding for {dtype!r}")


def fp8_scale(absmax):
    """Per-(token, head) e4m3 scale: the float32 value nearest absmax / 448."""
    return f32_round(np.asarray(absmax, dtype=np.float64) / E4M3_MAX)


def fp8_quantize(x, axis=-1):
    """Quantise rows of float64 ``x`` to e4m3 codes with one scale per row.

    scale = fl32(max|x| / 448); code = e4m3(x / scale); an all-zero row gets
    scale 0 and zero codes.  Returns (codes uint8, scale float64-of-f32).
    """
    x = np.asarray(x, dtype=np.float64)
    scale = fp8_scale(np.max(np.abs(x), axis=axis, keepdims=True))
    safe = np.where(scale > 0, scale, 1.0)
    codes = np.where(scale > 0, e4m3_code(x / safe), np.uint8(0)).astype(np.uint8)
    return codes, np.squeeze(scale, axis=axis)
