"""CPU oracle of the gated ReLU^2 step after the gate and up projections.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite may import it (see
the package docstring).

What the pages say.  "BitNet b1.58 2B4T Technical Report" (Chinese
translation), section 2, and its English summary, section 2: the
feed-forward sublayer uses squared ReLU (ReLU^2) as its activation, chosen
for sparsity and compute.  The layer's projections are read as q, k, v, o,
gate, up and down (the pages list no projection set; see the layer reading of
the decode workload).

Reading (stated): the activation that feeds the down projection is
h = ReLU(g)^2 * u, with g and u the outputs of the gate and up BitLinear
layers on the same input, stored as bfloat16 (the activation dtype of the
workloads).  g and u are step A3's values as this oracle defines them (the
binary64 rescale of ``bitlinear_ref.rescale``), rounded once to binary32;
because h is rounded to bfloat16 and must be the same bits on every side, the
binary32 order of what follows is part of the definition:

    g = RN32(A3(acc_gate)),  u = RN32(A3(acc_up))
    r = max(g, 0)
    h = bf16_rne(RN32(RN32(r * r) * u))

``gated_relu2_plain`` evaluates ReLU(g)^2 * u in binary64 from the binary64
outputs of step A3, for a pin that bounds how far the binary32 route may
stray from it.
"""

import numpy as np

from .bitlinear_ref import EPS_A, QB, _check_finite, rescale


def a3_f32(acc, gamma, absmax):
    """Step A3 rounded to binary32: RN32 of the binary64 rescale."""
    return rescale(acc, gamma, absmax).astype(np.float32)


def bf16_rne(x):
    """Round binary32 values to bfloat16, nearest with ties to even; returns
    the uint16 bit patterns (finite inputs; a value beyond the bfloat16 range
    rounds to infinity)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    return ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def gated_relu2(acc_gate, acc_up, gamma_gate, gamma_up, absmax):
    """h = bf16_rne(RN32(RN32(max(g, 0)^2) * u)) as uint16 bfloat16 bits [T, N]."""
    g = a3_f32(acc_gate, gamma_gate, absmax)
    u = a3_f32(acc_up, gamma_up, absmax)
    _check_finite(g, "gate output")
    _check_finite(u, "up output")
    r = np.maximum(g, np.float32(0))
    h = (r * r) * u                     # two binary32 products, in this order
    return bf16_rne(h)


def gated_relu2_plain(acc_gate, acc_up, gamma_gate, gamma_up, absmax):
    """ReLU(g)^2 * u in binary64 from binary64 outputs of step A3."""
    m = np.maximum(np.asarray(absmax, np.float32), EPS_A).astype(np.float64)
    g = np.asarray(acc_gate, np.float64) * float(gamma_gate) * m[:, None] / QB
    u = np.asarray(acc_up, np.float64) * float(gamma_up) * m[:, None] / QB
    r = np.maximum(g, 0.0)
    return r * r * u
