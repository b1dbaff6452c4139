"""bfloat16 helpers for the oracle (TEST INFRASTRUCTURE ONLY).

bfloat16 keeps the fp32 sign and 8-bit exponent and 7 explicit mantissa bits.
The weights the method updates are stored in bf16 ([LoGRA] Memory section: the
7B model's bf16 weights take about 14 GB), and the merge writes its result back
into them ([LoGRA] Sketch), so the oracle needs exact bf16 decoding and a
single round-to-nearest-even (RNE) from fp64.
"""
import numpy as np


def bits_to_f64(bits):
    """Decode bf16 bit patterns (uint16 array) to exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bits(x):
    """Round float64 values to bf16 once, ties to even, and return uint16 bits.

    The rounding is done directly from the fp64 value (no intermediate fp32),
    so there is exactly one rounding.  Subnormals keep the fp32 subnormal grid
    (spacing 2**-133); magnitudes that round past the largest finite bf16
    become infinity; NaN becomes the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    ax = np.abs(np.where(nan, 0.0, x))
    m, e = np.frexp(ax)                      # ax = m * 2**e, 0.5 <= m < 1
    # In the binade [2**(e-1), 2**e) a bf16 has 8 significant bits, so its
    # spacing is 2**(e-8); below the smallest normal (2**-126) it stays 2**-133.
    ulp_exp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(ax, -ulp_exp))      # exact scaling; rint = ties-to-even
    y = np.ldexp(q, ulp_exp)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)           # exact: y is on the bf16 grid
    mag = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    mag = np.where(y >= 2.0 ** 128, np.uint16(0x7F80), mag)
    sign = np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))
    out[...] = mag | sign
    out[nan] = np.uint16(0x7FC0)
    return out


def round_f64(x):
    """Value of the single RNE rounding of fp64 x to bf16, as float64."""
    return bits_to_f64(f64_to_bits(x))
