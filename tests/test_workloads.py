"""The seeded input generators (CPU): reproducible, with the stated shapes,
dtypes and distributions."""

import numpy as np

from bitlinear_w1_a8_amd import workloads as wl


def test_seeds_reproducible():
    a = wl.latent_weights(64, 256, 0.02, 1000)
    b = wl.latent_weights(64, 256, 0.02, 1000)
    assert a.dtype == np.float32 and np.array_equal(a, b)
    assert not np.array_equal(a, wl.latent_weights(64, 256, 0.02, 1001))


def test_distributions():
    w = wl.latent_weights(512, 1024, 0.02, 7)
    assert abs(float(w.std()) - 0.02) < 2e-4 and abs(float(w.mean())) < 2e-4
    x = wl.activations_normal(64, 4096, 8, 0.01, 8.0)
    assert abs(float(np.mean(np.abs(x) > 8.0)) - 0.01 * 0.4237) < 0.002  # P(|8z| > 8)
    s = wl.activations_student_t(64, 4096, 4, 9)
    assert float(np.max(np.abs(s))) > 10.0


def test_bf16_rounding():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-40], np.float32)
    b = wl.bf16_bits(x)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0003]  # ties go to even
    y = np.array([1.0 + 2 ** -7 + 2 ** -20], np.float32)
    assert wl.bf16_bits(y).tolist() == [0x3F81]


def test_workload_table():
    assert [m.k for m in wl.WORKLOADS[2].matrices] == [2560] * 6 + [6912]
    assert wl.WORKLOADS[3].tokens == [8, 32, 64]
    assert wl.WORKLOADS[5].matrices[1].k == 28672
    for w in wl.WORKLOADS.values():
        for m in w.matrices:
            assert m.k % 16 == 0


def test_bf16_matches_torch():
    import torch
    x = wl.activations_student_t(8, 1024, 4, 3) * np.float32(1e-3)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.bf16_bits(x), ref)
