"""CPU oracle of the binary-weight (W1A8) variant of the BitLinear forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite may import it (see
the package docstring).

What the pages say.  The BitNet b1.58 2B4T explainer (zhichai.net), section
2, and "BitNet解读" (on the meaning of the zero weight): the original 1-bit
BitNet has only the two weight values +1 and -1, with no zero, so every input
feature contributes to every output, positively or negatively.  No page gives
the rule that maps latent weights to the two values, their scale, or how they
are stored.

Reading (stated): the absmean scheme of eq. (1)-(3) of "BitNet解读" with the
two levels {-1, +1} in place of {-1, 0, +1}:

* gamma = mean |W| over the whole matrix (eq. (3), unchanged);
* t = the level nearest to W / (gamma + eps), i.e. +1 where W >= 0 and -1
  where W < 0; the tie at W = 0 (either sign of zero) goes to +1;
* steps A1 (activations) and A3 (rescale by gamma * max(absmax, eps) / 127)
  are those of the ternary forward, and the contraction is the same exact
  integer sum, now with t in {-1, +1}.

Storage (reading): one bit per weight, b = 1 for +1 and b = 0 for -1; within
a 32-weight group g of a row, weight k = 32g + 4j + i (j in 0..7, i in 0..3)
sits at bit 8i + j of a little-endian 32-bit word at row byte offset 4g; a row
takes K / 8 bytes, so K must be a multiple of 32.
"""

import numpy as np

from .bitlinear_ref import _check_finite, absmean_gamma, contract, quant_act, rescale


def binarize(w):
    """t = +1 where W >= 0 (both zeros included), -1 where W < 0 (int8)."""
    w = np.asarray(w, dtype=np.float32)
    _check_finite(w, "W")
    return np.where(w >= np.float32(0), 1, -1).astype(np.int8)


def pack_binary(t):
    """Pack t[N, K] in {-1, +1} to one bit per weight in the layout of the
    module docstring: uint8[N, K/8]."""
    t = np.asarray(t)
    if t.ndim != 2:
        raise ValueError("t must be 2-D")
    n_rows, k = t.shape
    if k % 32 != 0:
        raise ValueError("K must be a multiple of 32")
    if not np.all((t == -1) | (t == 1)):
        raise ValueError("t must be binary (+1 or -1)")
    bits = (t > 0).astype(np.uint32).reshape(n_rows, k // 32, 8, 4)   # [n, g, j, i]
    words = np.zeros((n_rows, k // 32), dtype=np.uint32)
    for j in range(8):
        for i in range(4):
            words |= bits[:, :, j, i] << np.uint32(8 * i + j)
    return words.astype("<u4").view(np.uint8).reshape(n_rows, k // 8)


def pack_weights_binary(w):
    """Step A0 of the binary variant: (packed uint8[N, K/8], gamma float32)."""
    return pack_binary(binarize(w)), absmean_gamma(w)


def forward_binary(w, x):
    """All steps of the binary variant: W[N, K], x[T, K] -> (y binary64,
    acc int32, packed, gamma)."""
    packed, gamma = pack_weights_binary(w)
    q, absmax, _ = quant_act(x)
    acc = contract(q, binarize(w))
    return rescale(acc, gamma, absmax), acc, packed, gamma
