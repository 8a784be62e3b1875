"""BitLinear (W1.58A8) forward for AMD Instinct MI355X (gfx950).

The compute lives in libbitlinear.so (hand-written HIP kernels behind the C
ABI of include/bitlinear.h); ``binding`` marshals torch tensors to it.  The
names below load the library on first use and fail loudly if it is missing.
"""

_EXPORTS = ("pack_weights", "quant_act", "subln_quant_act", "forward", "bitlinear", "linear_grouped",
            "interleave_rows", "gated_relu2", "pack_weights_binary", "forward_binary",
            "gemv_max_tokens",
            "BitLinearError", "load", "last_error")


def __getattr__(name):
    if name in _EXPORTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
