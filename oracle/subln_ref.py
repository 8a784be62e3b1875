"""CPU oracle of the sub-layer norm in front of step A1 (SubLN + act-quant).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite may import it (see
the package docstring).

What the pages say.  "BitNet b1.58 2B4T Technical Report" (Chinese
translation, developer.volcengine.com), section 2: the model normalises with
subln to steady training, and no linear or normalisation layer has a bias.
The BitNet b1.58 2B4T explainer (zhichai.net), component table: subln takes
the place of a transformer's RMSNorm / LayerNorm.  "BitNet解读", section on
LLaMA-alike components: the model keeps RMSNorm.  None prints a formula.

Reading (stated, since no page fixes it): SubLN is an RMS norm with a
per-feature gain g and no bias, and its output is what step A1 quantises:
normalise first, then quantise, in this order and precision

    S      = sum_k x[t, k]^2, exact, rounded once to binary64
             (every x^2 of a binary32 x is exact in binary64; the sum is
             taken exactly, as gamma's, so no order of summation matters),
    ms     = RN32(RN64(S / K)),
    r      = RN32(1 / RN32(sqrt(RN32(ms + eps_n)))),
    x_hat  = RN32(RN32(x * g) * r),
    q, a   = step A1 of x_hat (its int8 codes and its absmax, exact).

eps_n = 1e-5 in binary32.  a is the token's dequantisation absmax that step
A3 takes in place of A1's absmax.  Inputs whose mean square is beyond the
binary32 range have no finite r and are outside the domain (ValueError).

``subln_plain`` writes the same norm in binary64 throughout, for a pin that
bounds how far the binary32 route may stray from it.
"""

import math

import numpy as np

from .bitlinear_ref import EPS_A, QB, _check_finite, quant_act, widen_bf16

#: epsilon under the root of the RMS norm (value: a reading; no page gives one).
EPS_N = 1e-5


def _as_f32(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = widen_bf16(x)
    return np.asarray(x, dtype=np.float32)


def sum_squares(x):
    """S[t] = sum_k x[t, k]^2 per token, exact, rounded once to binary64.

    math.fsum keeps exact partial sums and rounds once; each square of a
    binary32 value is exact in binary64 (at most 48 significant bits, no
    overflow or underflow), so the result does not depend on any order."""
    x = _as_f32(x).astype(np.float64)
    return np.array([math.fsum((row * row).tolist()) for row in x], dtype=np.float64)


def rms_factor(x, eps_n=EPS_N):
    """r = RN32(1 / RN32(sqrt(RN32(RN32(RN64(S / K)) + eps_n)))) per token,
    binary32; x as given, before the gain, as an RMS norm defines it."""
    x = _as_f32(x)
    k = x.shape[1]
    ms64 = sum_squares(x) / float(k)            # one binary64 division
    if np.any(ms64 > float(np.finfo(np.float32).max)):
        raise ValueError("mean of squares beyond the binary32 range")
    ms = ms64.astype(np.float32)                # one rounding to binary32
    v = ms + np.float32(eps_n)                  # binary32 addition
    root = np.sqrt(v)                           # binary32 square root (correctly rounded)
    return np.float32(1.0) / root               # binary32 division


def normalise(x, gain, eps_n=EPS_N):
    """x_hat = RN32(RN32(x * g) * r): the gain first, then the token's factor."""
    x = _as_f32(x)
    g = np.asarray(gain, dtype=np.float32)
    if x.ndim != 2 or g.shape != (x.shape[1],):
        raise ValueError("x must be [T, K] and gain [K]")
    _check_finite(x, "x")
    _check_finite(g, "gain")
    r = rms_factor(x, eps_n)
    u = x * g[None, :]                          # one binary32 product per element
    _check_finite(u, "x * gain")
    return u * r[:, None], r                    # one binary32 product per element


def subln_quant_act(x, gain, eps_n=EPS_N):
    """SubLN followed by step A1, as defined in the module docstring.

    ``x`` is float32[T, K] or bfloat16 bit patterns uint16[T, K]; ``gain`` is
    float32[K].  Returns (q int8[T, K], a float32[T], rowsum int32[T],
    r float32[T]): the codes of x_hat, its absmax (the scale handed to step
    A3), the sum of the codes, and the token's RMS factor."""
    xh, r = normalise(x, gain, eps_n)
    q, a, rowsum = quant_act(xh)
    return q, a, rowsum, r


def subln_plain(x, gain, eps_n=EPS_N):
    """The norm in binary64 throughout: x_hat = x * g / sqrt(mean x^2 + eps_n),
    then per-token absmax to [-127, 127] with round half to even.  Returns
    (q int8[T, K], absmax of x_hat float64[T])."""
    x = _as_f32(x).astype(np.float64)
    g = np.asarray(gain, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps_n)
    xh = x * g[None, :] * r[:, None]
    m = np.max(np.abs(xh), axis=1)
    s = QB / np.maximum(m, float(EPS_A))
    q = np.clip(np.rint(xh * s[:, None]), -QB, QB).astype(np.int8)
    return q, m
