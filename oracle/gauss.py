"""Gaussian projection matrix of the sortLSH hash.

Test infrastructure only (see the package docstring).

The hash finds large attention entries with Hamming-sorted LSH ([S]
"Approach"; [A] "Abstract": LSH identifies the large entries).  The pages
print no projection recipe; this library reads "LSH" as random-hyperplane
(sign) hashing with r Gaussian directions R[p] in R^d, one matrix per call,
shared by queries and keys (both must fall in the same buckets), by all
heads and by every node of the causal recursion.

The Gaussians are drawn by Box-Muller [BM] from Philox words.  So that the
HIP library can draw the very same fp32 matrix on the device, the
transcendental steps are *defined* here as fixed sequences of IEEE fp64
additions, multiplications and divisions (never fused), with frexp/ldexp
for exact scaling:

  * ln by the atanh series  ln f = 2(s + s^3/3 + ... + s^21/21),
    s = (f-1)/(f+1), after an exact reduction of u to f in (sqrt2/2, sqrt2];
  * sin/cos of 2*pi*u by exact reduction to an octant-centred angle
    a in [-pi/4, pi/4] and the Taylor series to a^19 (sin) / a^20 (cos);
  * sqrt by six Newton steps from a linear start.

Python floats are IEEE doubles and Python evaluates these expressions
exactly in the written order, one rounding per operation, so the results
are a deterministic function of the Philox words.  ``tests`` pin each of
them against libm (``math.log``, ``math.sin``, ``math.cos``, ``math.sqrt``)
to a few ulps.
"""

import math

import numpy as np

from .philox import philox_words

LN2 = 0.6931471805599453          # nearest double to ln 2
SQRT2 = 1.4142135623730951        # nearest double to sqrt 2
HALF_PI = 1.5707963267948966      # nearest double to pi / 2

# atanh-series coefficients 1/(2k+1), k = 0..10
_LOG_C = [1.0 / (2 * k + 1) for k in range(11)]
# Taylor coefficients (-1)^k/(2k+1)!, k = 0..9 and (-1)^k/(2k)!, k = 0..10
_SIN_C = [(-1.0) ** k / float(math.factorial(2 * k + 1)) for k in range(10)]
_COS_C = [(-1.0) ** k / float(math.factorial(2 * k)) for k in range(11)]


def neg2_log_u(x):
    """-2 ln(u) with u = (x + 1/2) / 2^32 for a 32-bit word x; u is never 0
    or 1.  u = y / 2^33 with y = 2x + 1 odd, so y = f 2^e exactly."""
    y = 2 * int(x) + 1
    e = y.bit_length() - 1
    f = math.ldexp(float(y), -e)             # [1, 2), exact
    if f > SQRT2:
        f = f * 0.5                          # exact
        e = e + 1
    s = (f - 1.0) / (f + 1.0)
    z = s * s
    acc = _LOG_C[10]
    for k in range(9, -1, -1):
        acc = acc * z + _LOG_C[k]
    ln_f = 2.0 * (s * acc)
    ln_u = ln_f + float(e - 33) * LN2
    return -2.0 * ln_u


def sincos_2pi(x):
    """(cos, sin) of 2 pi u, u = (x + 1/2) / 2^32.  4u = y / 2^31 with y odd:
    the quarter-turn count and the remainder are exact integers."""
    y = 2 * int(x) + 1
    q = y >> 31
    rem = y & ((1 << 31) - 1)
    if rem >= (1 << 30):
        rem = rem - (1 << 31)
        q = q + 1
    w = math.ldexp(float(rem), -31)          # [-1/2, 1/2), exact
    a = w * HALF_PI
    a2 = a * a
    sacc = _SIN_C[9]
    for k in range(8, -1, -1):
        sacc = sacc * a2 + _SIN_C[k]
    sin_a = a * sacc
    cacc = _COS_C[10]
    for k in range(9, -1, -1):
        cacc = cacc * a2 + _COS_C[k]
    cos_a = cacc
    q = q & 3
    if q == 0:
        return cos_a, sin_a
    if q == 1:
        return -sin_a, cos_a
    if q == 2:
        return -cos_a, -sin_a
    return sin_a, -cos_a


def sqrt_newton(v):
    """sqrt(v), v > 0 finite: v = f 2^e with e even and f in [1/4, 1),
    six Newton steps from 0.41731 + 0.59016 f, then exact rescaling."""
    f, e = math.frexp(v)
    if e & 1:
        f = f * 0.5
        e = e + 1
    y = 0.41731 + 0.59016 * f
    for _ in range(6):
        y = 0.5 * (y + f / y)
    return math.ldexp(y, e // 2)


def box_muller(wa, wb):
    """Two standard normals from two 32-bit words [BM]: radius from wa,
    angle from wb."""
    rho = sqrt_newton(neg2_log_u(wa))
    c, s = sincos_2pi(wb)
    return rho * c, rho * s


def projections(seed, d, r):
    """R in float32[r][d].  Element e = p*d + k uses Philox counter
    (e // 4, 0, 0, 0) under the seed; words (w0, w1) feed elements 4j, 4j+1
    and words (w2, w3) feed 4j+2, 4j+3 through ``box_muller``; each fp64
    normal is rounded to the nearest fp32 (ties to even)."""
    total = r * d
    words = philox_words(seed, ((total + 3) // 4) * 4)
    out = np.empty(((total + 3) // 4) * 4, dtype=np.float64)
    for pair in range(len(words) // 2):
        z0, z1 = box_muller(int(words[2 * pair]), int(words[2 * pair + 1]))
        out[2 * pair] = z0
        out[2 * pair + 1] = z1
    return out[:total].astype(np.float32).reshape(r, d)
