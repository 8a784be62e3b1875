"""Plain, slow, CPU oracle of the BitLinear (W1.58A8) forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or call anything in this package.  The HIP library never calls it and shares
no code, constant table or helper with it.

Sources (the pages this follows, by title and section):

* "BitNet解读" (markgoyens.top), section on the weight quantisation
  function: eq. (3) defines the per-matrix scale gamma as the mean absolute
  value over all n*m entries; eq. (1) divides the weights by gamma plus a small
  epsilon; eq. (2) RoundClip rounds to the nearest integer and clips to
  [-1, 1].  The section on activation quantisation scales every token into
  [-Qb, Qb] with no zero point.  The section on computational efficiency says
  a ternary weight turns the product into add (+1), subtract (-1) or skip (0).
* "BitNet b1.58 2B4T Technical Report" (Chinese translation,
  developer.volcengine.com), section 2 (architecture): BitLinear replaces
  torch.nn.Linear, weights use absmean ternary quantisation, activations are
  8-bit with per-token absmax; no bias anywhere.  Section 5.1 (GPU inference):
  four ternary values are stored in one 8-bit integer.
* "BitNet b1.58 2B4T Technical Report | Summary" (greeksharifa.github.io),
  sections 2 and 5.1: the same facts in English.
* bitnet.cpp post (gitcode.csdn.net), section 1.1: the ternary weights come
  with a scale factor that restores the value range.

Readings taken where the pages are silent (no page prints these values, so
they are pinned by the readings themselves, not by a printed number):

* epsilon = 1e-5 in float32, added to gamma as eq. (1) prints it;
* Qb = 127, symmetric clip to [-127, 127];
* an all-zero token uses max(absmax, 1e-5) so it quantises to zeros;
* every round-to-integer is round-half-to-even;
* the decisions that produce integers (the weight division, the activation
  scale and product) are taken in IEEE binary32, the precision of the kernel;
* gamma is the exact sum of |W| rounded once to binary64, divided by n*m in
  binary64, rounded to binary32;
* the output is acc * gamma * max(absmax, 1e-5) / 127 in binary64 (the kernel
  returns binary32 within 1e-5 relative);
* the 2-bit code of a weight t is c = t + 1 in {0, 1, 2}; row n occupies K/4
  bytes at byte offset n*K/4; the weights k = 16g + 4j + i (j, i in 0..3) of
  group g form one little-endian 32-bit word at row byte offset 4g, with
  weight k in bits [8i + 2j, 8i + 2j + 2).

Every function works in numpy on the host; floating-point steps that decide an
integer are written with explicit numpy.float32 operands so that each step is
one IEEE binary32 operation, and nothing is fused or reordered.
"""

import itertools
import math

import numpy as np

#: eps of eq. (1), added to gamma before the division (value: a reading).
EPS_W = np.float32(1e-5)
#: floor on a token's absmax so that an all-zero token divides safely (reading).
EPS_A = np.float32(1e-5)
#: Qb of the activation quantiser, 8-bit symmetric (reading).
QB = 127


def _check_finite(a, what):
    if not np.all(np.isfinite(a)):
        raise ValueError(f"{what} must be finite")


# --------------------------------------------------------------------------
# Step A0: absmean ternarisation of the weights and 2-bit packing
# --------------------------------------------------------------------------

def absmean_gamma(w):
    """gamma = (1/(n*m)) * sum_ij |W_ij|, one scale for the whole matrix.

    Follows eq. (3) of "BitNet解读" (weight quantisation function).  The sum
    is exact (math.fsum keeps exact partials and rounds once to binary64), the
    mean is one binary64 division, and gamma is that mean rounded to binary32.
    The |W| of a binary32 value is exact, so no order of summation matters.
    """
    w = np.asarray(w, dtype=np.float32)
    _check_finite(w, "W")
    if w.size == 0:
        raise ValueError("W must not be empty")
    flat = w.reshape(-1)
    chunk = 1 << 20
    # A single fsum over every element (fed in chunks to bound memory).
    total = math.fsum(itertools.chain.from_iterable(
        np.abs(flat[i:i + chunk]).astype(np.float64).tolist()
        for i in range(0, flat.size, chunk)))
    mean = total / float(flat.size)
    return np.float32(mean)


def ternarize(w, gamma):
    """W~ = RoundClip(W / (gamma + eps), -1, 1), values in {-1, 0, +1}.

    Follows eq. (1) and eq. (2) of "BitNet解读" (weight quantisation
    function).  gamma + eps is one binary32 addition, W / (gamma + eps) one
    binary32 division per weight, and RoundClip rounds half to even then
    clips to [-1, 1].
    """
    w = np.asarray(w, dtype=np.float32)
    _check_finite(w, "W")
    d = np.float32(gamma) + EPS_W
    u = w / d
    return np.clip(np.rint(u), -1, 1).astype(np.int8)


def pack_ternary(t):
    """Pack a ternary matrix t[N, K] to 2-bit codes, four weights per byte.

    Four ternary values share one 8-bit integer ("BitNet b1.58 2B4T Technical
    Report", section 5.1, GPU inference).  The code and bit order are the
    reading stated in the module docstring: code c = t + 1; within a 16-weight
    group g of a row, weight k = 16g + 4j + i sits at bits [8i + 2j, 8i + 2j + 2)
    of a little-endian 32-bit word at row byte offset 4g.
    """
    t = np.asarray(t)
    if t.ndim != 2:
        raise ValueError("t must be 2-D")
    n_rows, k = t.shape
    if k % 16 != 0:
        raise ValueError("K must be a multiple of 16")
    if not np.all((t >= -1) & (t <= 1)):
        raise ValueError("t must be ternary")
    codes = (t.astype(np.int64) + 1).astype(np.uint32)
    codes = codes.reshape(n_rows, k // 16, 4, 4)          # [n, g, j, i]
    words = np.zeros((n_rows, k // 16), dtype=np.uint32)
    for j in range(4):
        for i in range(4):
            words |= codes[:, :, j, i] << np.uint32(8 * i + 2 * j)
    return words.astype("<u4").view(np.uint8).reshape(n_rows, k // 4)


def pack_weights(w):
    """Whole step A0: returns (packed uint8[N, K/4], gamma float32)."""
    gamma = absmean_gamma(w)
    return pack_ternary(ternarize(w, gamma)), gamma


# --------------------------------------------------------------------------
# Step A1: per-token absmax quantisation of the activations to int8
# --------------------------------------------------------------------------

def widen_bf16(bits):
    """bfloat16 bit patterns (uint16) -> float32, exactly (bits << 16)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quant_act(x):
    """Per-token absmax int8 quantisation; returns (q, absmax, rowsum).

    Follows "BitNet解读" (activation quantisation: every token is scaled into
    [-Qb, Qb], no zero point) and "BitNet b1.58 2B4T Technical Report",
    section 2 (8-bit activations, absmax taken per token).  Per token t:
    a = max_k |x|, m = max(a, eps), s = 127 / m (one binary32 division),
    v = x * s (one binary32 product), q = clip(round_half_even(v), -127, 127).
    ``absmax`` is a itself (exact); ``rowsum`` is sum_k q, in int32.
    ``x`` is float32[T, K], or bfloat16 bit patterns as uint16[T, K].
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = widen_bf16(x)
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    _check_finite(x, "x")
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    m = np.maximum(a, EPS_A)
    s = np.float32(QB) / m
    v = x * s[:, None]
    q = np.clip(np.rint(v), -QB, QB).astype(np.int8)
    rowsum = q.astype(np.int64).sum(axis=1).astype(np.int32)
    return q, a.astype(np.float32), rowsum


# --------------------------------------------------------------------------
# Step A2: ternary x int8 contraction into int32
# --------------------------------------------------------------------------

def contract(q, t):
    """acc[t, n] = sum_k t[n, k] * q[t, k], exact, returned as int32.

    With a ternary weight every product is +q, -q or 0 ("BitNet解读",
    computational efficiency), so the result is an exact integer.  The matmul
    runs in binary64, which is exact here: every product and partial sum is an
    integer of magnitude at most 127*K < 2**53.
    """
    q = np.asarray(q)
    t = np.asarray(t)
    if q.shape[1] != t.shape[1]:
        raise ValueError("K mismatch")
    if 127 * q.shape[1] >= 2 ** 31:
        raise ValueError("K too large for an int32 accumulator")
    acc = q.astype(np.float64) @ t.astype(np.float64).T
    return acc.astype(np.int64).astype(np.int32)


# --------------------------------------------------------------------------
# Step A3: rescale by gamma times the activation scale
# --------------------------------------------------------------------------

def rescale(acc, gamma, absmax):
    """y[t, n] = acc[t, n] * gamma * max(absmax[t], eps) / 127, in binary64.

    The scale factor that restores the range of the ternary weights
    (bitnet.cpp post, section 1.1) is gamma; the activation side undoes the
    127 / absmax scaling of step A1.
    """
    acc = np.asarray(acc, dtype=np.int64)
    m = np.maximum(np.asarray(absmax, dtype=np.float32), EPS_A).astype(np.float64)
    return acc.astype(np.float64) * np.float64(np.float32(gamma)) * m[:, None] / 127.0


def forward(w, x):
    """All four steps: latent weights W[N, K] and activations x[T, K] -> y."""
    packed, gamma = pack_weights(w)
    t = ternarize(w, gamma)
    q, absmax, _ = quant_act(x)
    acc = contract(q, t)
    return rescale(acc, gamma, absmax), acc, packed, gamma
