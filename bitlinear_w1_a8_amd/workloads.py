"""Seeded synthetic inputs and the named workloads.

This module only draws random numbers and describes shapes; it holds none of
the BitLinear arithmetic, so the HIP path and the CPU oracle can both take
their inputs from it.  Every array comes from numpy's PCG64 generator
(``numpy.random.default_rng(seed)``), with
``seed = 1000 * workload + 10 * matrix_index + (0 for W, 1 for x)``.

Shapes follow the 2B-class model (hidden 2560, FFN 6912, key/value width
640) and the 70B-class model (hidden 8192, FFN 28672) of the BitNet b1.58
line of work; no trained weight, dataset or prompt is used.
"""

from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x):
    """Round float32 values to bfloat16 (round-half-to-even); uint16 bits.

    Inputs are finite, so the NaN branch of the conversion is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def latent_weights(n, k, sigma, seed):
    """Latent weights W[n, k] ~ N(0, sigma) in float32."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def activations_normal(t, k, seed, outlier_frac=0.0, outlier_mult=8.0):
    """x[t, k] ~ N(0, 1) float32; a Bernoulli(outlier_frac) mask drawn from
    the same generator multiplies the selected entries by outlier_mult."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((t, k), dtype=np.float32)
    if outlier_frac > 0.0:
        mask = rng.random((t, k)) < outlier_frac
        x[mask] *= np.float32(outlier_mult)
    return x


def activations_student_t(t, k, nu, seed):
    """Heavy-tailed x[t, k] ~ Student-t(nu), drawn in float64, stored float32."""
    rng = np.random.default_rng(seed)
    return rng.standard_t(nu, size=(t, k)).astype(np.float32)


def seed_of(workload, matrix_index, is_x):
    return 1000 * workload + 10 * matrix_index + (1 if is_x else 0)


@dataclass
class Matrix:
    name: str
    k: int          # input features
    n: int          # output features


@dataclass
class Workload:
    index: int
    name: str
    matrices: list
    tokens: list            # token counts T run on every matrix
    sigma: float            # std of the latent weights
    x_dtype: str            # "f32" or "bf16"
    x_dist: str             # "normal", "normal_outliers" or "student_t4"
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def weights(self, mi):
        m = self.matrices[mi]
        return latent_weights(m.n, m.k, self.sigma, seed_of(self.index, mi, False))

    def activations(self, mi, t):
        """float32 activations for matrix mi at T = t (before any bf16 cast).

        The seed also folds in T so that each token count draws its own x.
        """
        m = self.matrices[mi]
        seed = seed_of(self.index, mi, True) + 100000 * t
        if self.x_dist == "normal":
            return activations_normal(t, m.k, seed)
        if self.x_dist == "normal_outliers":
            return activations_normal(t, m.k, seed, 0.01, 8.0)
        if self.x_dist == "student_t4":
            return activations_student_t(t, m.k, 4, seed)
        raise ValueError(self.x_dist)


# The 2B-class decoder layer in the order its projections run: q, k, v, o,
# gate, up, down.  Only four distinct shapes occur.
LAYER_2B = [
    Matrix("q", 2560, 2560),
    Matrix("k", 2560, 640),
    Matrix("v", 2560, 640),
    Matrix("o", 2560, 2560),
    Matrix("gate", 2560, 6912),
    Matrix("up", 2560, 6912),
    Matrix("down", 6912, 2560),
]

WORKLOADS = {
    1: Workload(1, "toy_t4_k256_n512", [Matrix("toy", 256, 512)], [4],
                0.02, "f32", "normal_outliers",
                "single forward, fp32 activations with 1% outliers x8"),
    2: Workload(2, "decode_2b_t1_layer", LAYER_2B, [1], 0.02, "bf16", "normal",
                "2B-class decode, all seven projections of a layer back to back"),
    3: Workload(3, "batched_decode_2b", [Matrix("up", 2560, 6912),
                                          Matrix("down", 6912, 2560)],
                [8, 32, 64], 0.02, "bf16", "student_t4",
                "GEMV-to-GEMM crossover, heavy-tailed activations"),
    4: Workload(4, "prefill_2b_t2048", [Matrix("up", 2560, 6912),
                                         Matrix("down", 6912, 2560)],
                [2048], 0.02, "bf16", "normal",
                "prefill, act-quant plus GEMM"),
    5: Workload(5, "llm70b_shapes", [Matrix("up", 8192, 28672),
                                      Matrix("down", 28672, 8192)],
                [1, 256], 0.01, "bf16", "normal",
                "70B-class shapes at decode and T=256"),
}
