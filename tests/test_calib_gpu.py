"""The measurement helpers do the work they claim (needs a HIP device).

The read helper must touch every byte: the XOR of its per-wave results has
to equal the XOR of the buffer's 32-bit words computed on the host.  The
matrix-core loop must run every MFMA: each wave's result is the closed form
4 * iters * 32 * byte^2 (mod 2^32).
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl(built_lib):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from bitlinear_w1_a8_amd import binding
    binding.load()
    return binding


# sizes: one vector; less than a chunk; chunks plus a ragged tail; whole
# grid-stride rounds (1024 blocks x 256 lanes x 8 loads of 16 bytes) plus a
# tail; 64 MiB; 56 MiB + 48 bytes
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48, (1024 * 256 * 16 * 8) * 3 + 4112,
                                    64 << 20, (56 << 20) + 48])
def test_calib_read_touches_every_word(bl, nbytes, layout):
    rng = np.random.default_rng(nbytes + layout)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = bl.calib_read(buf, layout)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("iters,byte", [(1, 1), (8, 3), (64, -128), (5, 127)])
def test_calib_mfma_closed_form(bl, iters, byte):
    sink = bl.calib_mfma(iters, byte)
    torch.cuda.synchronize()
    want = np.array([(4 * iters * 32 * byte * byte) % (1 << 32)], dtype=np.uint64)
    want = want.astype(np.uint32).view(np.int32)[0]
    got = sink[:4096].cpu().numpy()
    assert np.all(got == want), (got[:4], want)


def test_calib_empty_runs(bl):
    for _ in range(8):
        bl.calib_empty()
    torch.cuda.synchronize()
