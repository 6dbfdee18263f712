"""Exact number-format codecs for the oracle (fp64 numpy).

Test infrastructure: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
path.

* OCP 8-bit floating point, format E4M3 ("e4m3fn"): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111, largest
  finite magnitude 448.  The DeepSeek-V3.2 write-up (intelliparadigm.com,
  section 2.2) only says the indexer runs in FP8; e4m3fn is the FP8 flavour
  of the target hardware.
* bfloat16: the upper 16 bits of an IEEE-754 binary32.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """e4m3fn code -> fp64, by the closed form of the format.

    normal (E > 0):  (-1)^S * 2^(E-7) * (1 + M/8)
    subnormal (E=0): (-1)^S * 2^(-6) * (M/8)
    E = 15, M = 7:   NaN
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64) / 8.0, -6),
                   np.ldexp(1.0 + m.astype(np.float64) / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(x) -> np.ndarray:
    """fp64 -> e4m3fn code, round to nearest with ties to an even mantissa,
    saturating to +-448 (no NaN is produced for finite input).

    The grid spacing for |x| in [2^e, 2^(e+1)) with e >= -6 is 2^(e-3); below
    2^-6 (subnormals) it is 2^-9.  |x|/spacing is exact in binary floating
    point, so np.rint (round half to even) gives the correctly rounded count
    of grid steps.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.signbit(x)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                # floor(log2 a), clamped to the subnormal range
    step = np.ldexp(1.0, (e - 3).astype(np.int64))
    v = np.rint(a / step) * step              # rounded magnitude (exact)
    v = np.minimum(v, E4M3_MAX)               # saturate
    # encode the exact magnitude v
    _, ev = np.frexp(np.where(v > 0, v, 1.0))
    ev = ev - 1
    normal = v >= 2.0 ** -6
    exp_field = np.where(normal, ev + 7, 0)
    man_field = np.where(normal, np.rint(np.ldexp(v, -ev.astype(np.int64)) * 8.0 - 8.0),
                         np.rint(v * 2.0 ** 9))
    code = (exp_field.astype(np.int64) << 3) | man_field.astype(np.int64)
    code = np.where(v == 0, 0, code)
    code = code | (sign.astype(np.int64) << 7)
    code = np.where(v == 0, 0, code)          # -0 encodes as +0 (a zero stays a zero)
    return code.astype(np.uint8)


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit pattern (uint16) -> fp64: shift into the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_decode(bits_or_values) -> np.ndarray:
    return np.asarray(bits_or_values, dtype=np.float32).astype(np.float64)


def f64_to_f32_rne(x) -> np.ndarray:
    """fp64 -> binary32 with IEEE round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
