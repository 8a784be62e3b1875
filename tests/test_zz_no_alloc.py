"""bitlinear_pack_weights_noalloc against bitlinear_pack_weights (needs an MI355X).

The no-workspace entry point keeps gamma's exponent buckets in the library's
own device array.  It is called here through the C ABI (ctypes, raw device
pointers) twice in a row, the second time on a smaller matrix, so a bucket
left over from the first call would change the second gamma; each result must
equal the workspace entry point's bit for bit, and both must equal the oracle.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from bitlinear_w1_a8_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib(built_lib):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from bitlinear_w1_a8_amd import binding
    return binding.load()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _outputs(n, k):
    return (torch.empty((n, k // 4), dtype=torch.uint8, device="cuda"),
            torch.empty(1, dtype=torch.float32, device="cuda"))


def _pack_workspace(lib, w):
    n, k = w.shape
    packed, gamma = _outputs(n, k)
    wsb = int(lib.bitlinear_pack_workspace_bytes(n, k))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    rc = lib.bitlinear_pack_weights(w.data_ptr(), n, k, packed.data_ptr(), gamma.data_ptr(),
                                    ws.data_ptr(), wsb, _stream())
    assert rc == 0, lib.bitlinear_last_error()
    return packed, gamma


def _pack_noalloc(lib, w):
    n, k = w.shape
    packed, gamma = _outputs(n, k)
    rc = lib.bitlinear_pack_weights_noalloc(w.data_ptr(), n, k, packed.data_ptr(),
                                            gamma.data_ptr(), _stream())
    assert rc == 0, lib.bitlinear_last_error()
    return packed, gamma


# (N, K, sigma, seed): the larger matrix first, then a smaller one whose
# gamma would absorb any bucket the first call left behind.
CALLS = [(2560, 6912, 0.02, 71), (512, 256, 0.5, 72)]


def test_noalloc_pack_equals_workspace_pack_twice(lib):
    print(f"noalloc pack: calls {CALLS}", flush=True)
    results = []
    for n, k, sigma, seed in CALLS:
        w_host = wl.latent_weights(n, k, sigma, seed)
        w = torch.from_numpy(w_host).cuda()
        p_na, g_na = _pack_noalloc(lib, w)
        p_ws, g_ws = _pack_workspace(lib, w)
        torch.cuda.synchronize()
        results.append((n, k, w_host, p_na.cpu().numpy(), g_na.cpu().numpy(),
                        p_ws.cpu().numpy(), g_ws.cpu().numpy()))
    for n, k, w_host, p_na, g_na, p_ws, g_ws in results:
        assert g_na.view(np.uint32)[0] == g_ws.view(np.uint32)[0], (n, k, g_na[0], g_ws[0])
        assert np.array_equal(p_na, p_ws), f"{n}x{k}: packed bytes differ"
        packed_ref, gamma_ref = oracle.pack_weights(w_host)
        assert g_na.view(np.uint32)[0] == np.float32(gamma_ref).view(np.uint32), (n, k)
        assert np.array_equal(p_na, packed_ref), f"{n}x{k}: packed bytes differ from the oracle"


def test_noalloc_pack_allocates_nothing(lib):
    """With its outputs already allocated the call takes no device memory."""
    n, k = 640, 2560
    w = torch.from_numpy(wl.latent_weights(n, k, 0.02, 73)).cuda()
    packed, gamma = _outputs(n, k)
    # a first call loads the library's code object (and its device array)
    rc = lib.bitlinear_pack_weights_noalloc(w.data_ptr(), n, k, packed.data_ptr(),
                                            gamma.data_ptr(), _stream())
    assert rc == 0, lib.bitlinear_last_error()
    torch.cuda.synchronize()
    before = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        rc = lib.bitlinear_pack_weights_noalloc(w.data_ptr(), n, k, packed.data_ptr(),
                                                gamma.data_ptr(), _stream())
        assert rc == 0, lib.bitlinear_last_error()
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == before
    p_ws, g_ws = _pack_workspace(lib, w)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), p_ws.cpu().numpy())
    assert gamma.cpu().numpy().view(np.uint32)[0] == g_ws.cpu().numpy().view(np.uint32)[0]
