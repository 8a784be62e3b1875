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
per-feature gain g and no bias, in front of the activation quantiser:

    x_hat[t, k] = x[t, k] * g[k] / sqrt(mean_k(x[t, k]^2) + eps_n),
    eps_n = 1e-5.

The per-token absmax quantiser of step A1 divides each token by its own
absmax, so a positive per-token factor r = 1 / sqrt(mean(x^2) + eps_n)
cancels out of the int8 codes: quantising x_hat gives the codes of x * g, and
the token's dequantisation absmax is r * max|x * g|.  The fused step is
therefore defined as

    u = x * g                 (one binary32 product per element),
    q, a = A1(u)              (exactly step A1: codes and absmax of u),
    scale = r * a             (the absmax of x_hat, passed on to step A3).

``subln_plain`` writes the norm out literally in binary64 (normalise, then
quantise) so that the pins can check the rewrite against it.
"""

import numpy as np

from .bitlinear_ref import EPS_A, QB, _check_finite, quant_act, widen_bf16

#: epsilon under the root of the RMS norm (value: a reading; no page gives one).
EPS_N = 1e-5


def _as_f32(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = widen_bf16(x)
    return np.asarray(x, dtype=np.float32)


def rms_factor(x, eps_n=EPS_N):
    """r = 1 / sqrt(mean_k x^2 + eps_n) per token, in binary64 (x as given,
    before the gain, as an RMS norm defines it)."""
    x = _as_f32(x).astype(np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps_n)


def subln_quant_act(x, gain, eps_n=EPS_N):
    """SubLN followed by step A1, in the form defined in the module docstring.

    ``x`` is float32[T, K] or bfloat16 bit patterns uint16[T, K]; ``gain`` is
    float32[K].  Returns (q int8[T, K], scale float64[T], rowsum int32[T],
    a float32[T]): the codes, the token's dequantisation absmax r * a, the sum
    of the codes, and a = max|x * g| (exact)."""
    x = _as_f32(x)
    g = np.asarray(gain, dtype=np.float32)
    if x.ndim != 2 or g.shape != (x.shape[1],):
        raise ValueError("x must be [T, K] and gain [K]")
    _check_finite(x, "x")
    _check_finite(g, "gain")
    u = x * g[None, :]                       # one binary32 product per element
    q, a, rowsum = quant_act(u)
    scale = rms_factor(x, eps_n) * a.astype(np.float64)
    return q, scale, rowsum, a


def subln_plain(x, gain, eps_n=EPS_N):
    """The norm written out literally in binary64: x_hat = x * g * r, then
    per-token absmax to [-127, 127] with round half to even.  Returns
    (q int8[T, K], absmax of x_hat float64[T])."""
    x = _as_f32(x).astype(np.float64)
    g = np.asarray(gain, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps_n)
    xh = x * g[None, :] * r[:, None]
    m = np.max(np.abs(xh), axis=1)
    s = QB / np.maximum(m, float(EPS_A))
    q = np.clip(np.rint(xh * s[:, None]), -QB, QB).astype(np.int8)
    return q, m
