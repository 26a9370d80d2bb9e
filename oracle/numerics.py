"""Rounding helpers of the oracle (test infrastructure only).

The layer stores activations in bfloat16 at a few declared points (normalised input
to the experts, SwiGLU output, layer output).  bfloat16 is the upper half of an IEEE
binary32: 1 sign bit, 8 exponent bits, 7 stored fraction bits, so 8 significant bits
for normal numbers and the same exponent range as binary32.

``round_bf16`` rounds a float64 value straight to the nearest bfloat16 value, ties to
even, by scaling the value so that the 8 kept significant bits become the integer
part and calling ``np.rint`` (which rounds half to even).  It is written from the
format's definition, not from any conversion routine.
"""

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")  # largest finite bfloat16: (2 - 2**-7) * 2**127
_BF16_MIN_NORMAL_EXP = -125  # frexp exponent of 2**-126, the smallest normal


def round_bf16(a):
    """Nearest bfloat16 value of every element of ``a`` (float64 in, float64 out)."""
    a = np.asarray(a, dtype=np.float64)
    out = a.copy()
    sel = np.isfinite(a) & (a != 0.0)
    v = a[sel]
    _, e = np.frexp(v)  # v = m * 2**e with 0.5 <= |m| < 1
    # 8 significant bits => spacing 2**(e-8); below the normal range the spacing
    # stays at that of the smallest binade (bfloat16 subnormals).
    e = np.maximum(e, _BF16_MIN_NORMAL_EXP)
    q = np.rint(np.ldexp(v, 8 - e))  # exact scaling; rint = round half to even
    r = np.ldexp(q, e - 8)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    out[sel] = r
    return out


def round_f32(a):
    """Nearest binary32 value of every element (NumPy's cast rounds to nearest even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def rounder(act_dtype):
    """The storage rounding used for activations of a layer computed in ``act_dtype``
    ("f64" keeps every value exact, for the hand-worked pins)."""
    if act_dtype == "f64":
        return lambda a: np.asarray(a, dtype=np.float64)
    if act_dtype == "bf16":
        return round_bf16
    if act_dtype == "f32":
        return round_f32
    raise ValueError(f"unknown activation dtype {act_dtype!r}")
