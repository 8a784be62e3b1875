"""The Python binding refuses mis-shaped tensors before it calls the library
(needs a HIP device to hold the tensors).

The library trusts the extents it is given: a caller buffer shorter than
[T, N] or a gamma / absmax / gain vector of the wrong length would be read or
written past its end.  Every case below swaps in a library object that fails
the test if any entry point is reached, so a check that is missing shows up
as a test failure on the host and never as a kernel launch.
"""

import pytest
import torch

pytestmark = pytest.mark.gpu

T, N, K = 3, 48, 256


class _NoLaunch:
    def __getattr__(self, name):
        raise AssertionError(f"{name} was called with mis-shaped arguments")


@pytest.fixture()
def bl(built_lib, monkeypatch):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from bitlinear_w1_a8_amd import binding
    monkeypatch.setattr(binding, "load", lambda: _NoLaunch())
    return binding


def _good():
    d = "cuda"
    return dict(packed=torch.zeros((N, K // 4), dtype=torch.uint8, device=d),
                gamma=torch.ones(1, dtype=torch.float32, device=d),
                xq=torch.zeros((T, K), dtype=torch.int8, device=d),
                absmax=torch.ones(T, dtype=torch.float32, device=d))


def _f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


FORWARD_BAD = {
    "packed_short_rows": dict(packed=torch.zeros((N - 1, K // 4), dtype=torch.uint8)),
    "packed_short_k": dict(packed=torch.zeros((N, K // 4 - 4), dtype=torch.uint8)),
    "gamma_empty": dict(gamma=torch.ones(0, dtype=torch.float32)),
    "absmax_short": dict(absmax=torch.ones(T - 1, dtype=torch.float32)),
    "xq_1d": dict(xq=torch.zeros(T * K, dtype=torch.int8)),
}


@pytest.mark.parametrize("case", sorted(FORWARD_BAD))
def test_forward_rejects_mis_shaped_inputs(bl, case):
    args = _good()
    args.update({k: v.cuda() for k, v in FORWARD_BAD[case].items()})
    with pytest.raises(ValueError):
        bl.forward(args["packed"], args["gamma"], args["xq"], args["absmax"], N)


@pytest.mark.parametrize("out_shape", [(T, N - 1), (T - 1, N), (T * N,), (N, T)])
def test_forward_rejects_mis_shaped_out(bl, out_shape):
    a = _good()
    with pytest.raises(ValueError):
        bl.forward(a["packed"], a["gamma"], a["xq"], a["absmax"], N, out=_f32(*out_shape))
    with pytest.raises(ValueError):
        bl.forward(a["packed"], a["gamma"], a["xq"], a["absmax"], N, want_acc=True,
                   acc_out=_i32(*out_shape))


def test_forward_rejects_wrong_out_dtype_and_layout(bl):
    a = _good()
    with pytest.raises(TypeError):
        bl.forward(a["packed"], a["gamma"], a["xq"], a["absmax"], N,
                   out=torch.zeros((T, N), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(TypeError):
        bl.forward(a["packed"], a["gamma"], a["xq"], a["absmax"], N, acc_out=_f32(T, N))
    with pytest.raises(ValueError):
        bl.forward(a["packed"], a["gamma"], a["xq"], a["absmax"], N, out=_f32(N, T).t())


def test_grouped_rejects_mixed_token_counts_and_widths(bl):
    a = _good()
    x = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        bl.linear_grouped([x, x[:T - 1]], [(a["packed"], a["gamma"])] * 2)
    with pytest.raises(ValueError):
        bl.linear_grouped([x], [(a["packed"][:, :K // 8].contiguous(), a["gamma"])])
    with pytest.raises(ValueError):
        bl.linear_grouped([x], [(a["packed"], _f32(2))])
    with pytest.raises(ValueError):
        bl.linear_grouped([x] * 9, [(a["packed"], a["gamma"])] * 9)


def test_subln_rejects_wrong_gain_length(bl):
    x = _f32(T, K)
    with pytest.raises(ValueError):
        bl.subln_quant_act(x, _f32(K - 1))
    with pytest.raises(ValueError):
        bl.subln_quant_act(x, _f32(1))


def test_gated_rejects_mis_shaped_scales(bl):
    x = _f32(T, K)
    gu = torch.zeros((2 * N, K // 4), dtype=torch.uint8, device="cuda")
    one = _f32(1)
    with pytest.raises(ValueError):
        bl.gated_relu2(x, gu, _f32(0), one)
    with pytest.raises(ValueError):
        bl.gated_relu2(x, gu, one, _f32(2))
    with pytest.raises(ValueError):
        bl.gated_relu2(x, gu[:, :K // 8].contiguous(), one, one)


def test_interleave_rejects_mismatched_pair(bl):
    a = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        bl.interleave_rows(a, a[:N - 1])
    with pytest.raises(ValueError):
        bl.interleave_rows(a.flatten(), a.flatten())


def test_binary_forward_rejects_mis_shaped_inputs(bl):
    packed = torch.zeros((N, K // 8), dtype=torch.uint8, device="cuda")
    xq = torch.zeros((T, K), dtype=torch.int8, device="cuda")
    one, am = _f32(1), _f32(T)
    with pytest.raises(ValueError):
        bl.forward_binary(packed, one, xq, _f32(T - 1))
    with pytest.raises(ValueError):
        bl.forward_binary(packed, _f32(0), xq, am)
    with pytest.raises(ValueError):
        bl.forward_binary(packed[:, :K // 16].contiguous(), one, xq, am)


def test_good_shapes_reach_the_library(bl):
    """The checks pass correctly shaped tensors through: the stub library is
    reached, which proves the cases above were stopped by the checks alone."""
    a = _good()
    with pytest.raises(AssertionError, match="called with mis-shaped"):
        bl.forward(a["packed"], a["gamma"], a["xq"], a["absmax"], N, want_acc=True,
                   out=_f32(T, N), acc_out=_i32(T, N))
