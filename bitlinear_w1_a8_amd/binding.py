"""ctypes binding of libbitlinear.so (include/bitlinear.h), same names.

Argument marshalling only: tensors are allocated with torch on the caller's
device, their data pointers and the current HIP stream are passed to the C
ABI, and a non-OK status raises BitLinearError with the library's message.
Every step of the forward runs in the library's HIP kernels; there is no
other code path.  If the library is not built, loading raises ImportError.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitlinear.so")

BL_F32, BL_BF16 = 0, 1
ALGOS = {"auto": 0, "gemv": 1, "gemm": 2, "lut": 3, "dot4": 4}

_lib = None

_c_i64, _c_sz, _c_vp, _c_int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int

# name -> (restype, argtypes), as declared in include/bitlinear.h
SIGNATURES = {
    "bitlinear_abi_version": (_c_int, []),
    "bitlinear_last_error": (ctypes.c_char_p, []),
    "bitlinear_gemv_max_tokens": (_c_i64, []),
    "bitlinear_pack_workspace_bytes": (_c_sz, [_c_i64, _c_i64]),
    "bitlinear_pack_weights": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "bitlinear_quant_act": (_c_int, [_c_vp, _c_int, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp]),
    "bitlinear_subln_quant_act": (_c_int, [_c_vp, _c_int, _c_vp, ctypes.c_float, _c_i64, _c_i64,
                                           _c_vp, _c_vp, _c_vp, _c_vp]),
    "bitlinear_forward": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                                   _c_vp, _c_vp, _c_vp]),
    "bitlinear_forward_algo": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                                        _c_vp, _c_vp, _c_int, _c_vp]),
}


class BlLinear(ctypes.Structure):
    """struct bl_linear of include/bitlinear.h."""
    _fields_ = [("x", _c_vp), ("packed", _c_vp), ("gamma", _c_vp), ("N", _c_i64),
                ("K", _c_i64), ("y", _c_vp), ("xq", _c_vp), ("absmax", _c_vp), ("acc", _c_vp)]


SIGNATURES["bitlinear_pack_weights_binary"] = (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp,
                                                        _c_sz, _c_vp])
SIGNATURES["bitlinear_forward_binary"] = (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                                                   _c_vp, _c_vp, _c_int, _c_vp])
SIGNATURES["bitlinear_interleave_rows"] = (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp])
SIGNATURES["bitlinear_gated_relu2"] = (_c_int, [_c_vp, _c_int, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64,
                                                _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp])
SIGNATURES["bitlinear_linear_grouped"] = (_c_int, [ctypes.POINTER(BlLinear), _c_int, _c_i64,
                                                   _c_int, _c_vp])
SIGNATURES["bitlinear_pack_weights_noalloc"] = (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp])
SIGNATURES["bitlinear_calib_sink_len"] = (_c_i64, [])
SIGNATURES["bitlinear_calib_empty"] = (_c_int, [_c_vp])
SIGNATURES["bitlinear_calib_read"] = (_c_int, [_c_vp, _c_i64, _c_int, _c_vp, _c_vp])
SIGNATURES["bitlinear_calib_mfma"] = (_c_int, [_c_i64, _c_int, _c_vp, _c_vp])


class BitLinearError(RuntimeError):
    """A non-OK status from libbitlinear; ``status`` holds the code."""

    def __init__(self, status, message):
        super().__init__(f"libbitlinear status {status}: {message}")
        self.status = status


def load():
    """Load libbitlinear.so once and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m bitlinear_w1_a8_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_error():
    return load().bitlinear_last_error().decode()


def _check(status):
    if status != 0:
        raise BitLinearError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_shape(t, name, shape):
    """The library reads and writes exactly these extents: a tensor of another
    shape would be read or written past its end."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(name, *ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"{name}: all tensors must be on one device, got {sorted(map(str, devs))}")


def gemv_max_tokens():
    return int(load().bitlinear_gemv_max_tokens())


def pack_weights(w):
    """Step A0 on the GPU: float32 W[N, K] -> (packed uint8[N, K/4], gamma float32[1])."""
    lib = load()
    _need_cuda(w, "w", torch.float32)
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    gamma = torch.empty(1, dtype=torch.float32, device=w.device)
    wsb = int(lib.bitlinear_pack_workspace_bytes(n, k))
    ws = torch.empty(wsb, dtype=torch.uint8, device=w.device)
    _check(lib.bitlinear_pack_weights(_ptr(w), n, k, _ptr(packed), _ptr(gamma), _ptr(ws), wsb,
                                      _stream(w.device)))
    return packed, gamma


def pack_weights_noalloc(w, packed=None, gamma=None):
    """Step A0 through the library's own device buckets (no workspace): the
    same results as pack_weights.  ``packed`` and ``gamma`` may be passed in
    (preallocated outputs); otherwise they are allocated here."""
    lib = load()
    _need_cuda(w, "w", torch.float32)
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    if packed is None:
        packed = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=w.device)
    _need_cuda(packed, "packed", torch.uint8)
    _need_cuda(gamma, "gamma", torch.float32)
    _need_shape(packed, "packed", (n, k // 4))
    _need_shape(gamma, "gamma", (1,))
    _same_device("pack_weights_noalloc", w, packed, gamma)
    _check(lib.bitlinear_pack_weights_noalloc(_ptr(w), n, k, _ptr(packed), _ptr(gamma),
                                              _stream(w.device)))
    return packed, gamma


def quant_act(x, with_rowsum=True):
    """Step A1 on the GPU: x[T, K] (float32 or bfloat16) -> (xq int8, absmax f32[T], rowsum i32[T] or None)."""
    lib = load()
    _need_cuda(x, "x")
    if x.dtype == torch.float32:
        dt = BL_F32
    elif x.dtype == torch.bfloat16:
        dt = BL_BF16
    else:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 2:
        raise ValueError("x must be [T, K]")
    t, k = x.shape
    xq = torch.empty((t, k), dtype=torch.int8, device=x.device)
    absmax = torch.empty(t, dtype=torch.float32, device=x.device)
    rowsum = torch.empty(t, dtype=torch.int32, device=x.device) if with_rowsum else None
    _check(lib.bitlinear_quant_act(_ptr(x), dt, t, k, _ptr(xq), _ptr(absmax), _ptr(rowsum),
                                   _stream(x.device)))
    return xq, absmax, rowsum


def subln_quant_act(x, gain, eps_n=1e-5, with_rowsum=True):
    """Sub-layer norm (RMS with per-feature gain) fused with step A1 on the GPU:
    x[T, K] (float32 or bfloat16), gain float32[K] -> (xq int8, scale f32[T],
    rowsum i32[T] or None); scale takes the place of absmax in forward()."""
    lib = load()
    _need_cuda(x, "x")
    _need_cuda(gain, "gain", torch.float32)
    if x.dtype == torch.float32:
        dt = BL_F32
    elif x.dtype == torch.bfloat16:
        dt = BL_BF16
    else:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 2:
        raise ValueError("x must be [T, K]")
    t, k = x.shape
    _need_shape(gain, "gain", (k,))
    _same_device("subln_quant_act", x, gain)
    xq = torch.empty((t, k), dtype=torch.int8, device=x.device)
    scale = torch.empty(t, dtype=torch.float32, device=x.device)
    rowsum = torch.empty(t, dtype=torch.int32, device=x.device) if with_rowsum else None
    _check(lib.bitlinear_subln_quant_act(_ptr(x), dt, _ptr(gain), float(eps_n), t, k, _ptr(xq),
                                         _ptr(scale), _ptr(rowsum), _stream(x.device)))
    return xq, scale, rowsum


def forward(packed, gamma, xq, absmax, n, algo="auto", want_acc=False, out=None, acc_out=None,
            rowsum=None):
    """Steps A2 + A3 on the GPU: -> y float32[T, N] (and acc int32[T, N] if want_acc).

    ``rowsum`` (int32[T], the row sums quant_act returns) lets the kernels
    take each token's sum of q instead of deriving it."""
    lib = load()
    _need_cuda(packed, "packed", torch.uint8)
    _need_cuda(gamma, "gamma", torch.float32)
    _need_cuda(xq, "xq", torch.int8)
    _need_cuda(absmax, "absmax", torch.float32)
    if xq.dim() != 2:
        raise ValueError("xq must be [T, K]")
    t, k = xq.shape
    _need_shape(packed, "packed", (n, k // 4))
    _need_shape(gamma, "gamma", (1,))
    _need_shape(absmax, "absmax", (t,))
    if rowsum is not None:
        _need_cuda(rowsum, "rowsum", torch.int32)
        _need_shape(rowsum, "rowsum", (t,))
    if out is not None:
        _need_cuda(out, "out", torch.float32)
        _need_shape(out, "out", (t, n))
    y = out if out is not None else torch.empty((t, n), dtype=torch.float32, device=xq.device)
    acc = acc_out
    if acc is not None:
        _need_cuda(acc, "acc_out", torch.int32)
        _need_shape(acc, "acc_out", (t, n))
    if want_acc and acc is None:
        acc = torch.empty((t, n), dtype=torch.int32, device=xq.device)
    _same_device("forward", packed, gamma, xq, absmax, y, acc, rowsum)
    _check(lib.bitlinear_forward_algo(_ptr(packed), _ptr(gamma), _ptr(xq), _ptr(absmax),
                                      _ptr(rowsum), t, n, k, _ptr(y), _ptr(acc), ALGOS[algo],
                                      _stream(xq.device)))
    return (y, acc) if want_acc else y


def bitlinear(x, packed, gamma, n, algo="auto"):
    """Quantise x and run the forward: y = BitLinear(x) with pre-packed weights."""
    xq, absmax, rowsum = quant_act(x)
    return forward(packed, gamma, xq, absmax, n, algo=algo, rowsum=rowsum)


def linear_grouped(xs, weights, want_acc=False):
    """Steps A1-A3 for several independent problems in one call.

    xs: list of activations [T, K_i] (one dtype, float32 or bfloat16, same T);
    weights: list of (packed, gamma) from pack_weights.  Returns a list of
    (y, xq, absmax, acc-or-None) per problem.
    """
    lib = load()
    if not xs or len(xs) != len(weights):
        raise ValueError("need one (packed, gamma) per activation tensor")
    dt = {torch.float32: BL_F32, torch.bfloat16: BL_BF16}.get(xs[0].dtype)
    if dt is None:
        raise TypeError(f"x must be float32 or bfloat16, got {xs[0].dtype}")
    if len(xs) > 8:
        raise ValueError("at most 8 problems per call")
    t = xs[0].shape[0]
    outs, descs = [], (BlLinear * len(xs))()
    for i, (x, (packed, gamma)) in enumerate(zip(xs, weights)):
        _need_cuda(x, "x", xs[0].dtype)
        _need_cuda(packed, "packed", torch.uint8)
        _need_cuda(gamma, "gamma", torch.float32)
        if x.dim() != 2 or x.shape[0] != t:
            raise ValueError(f"problem {i}: x must be [T, K] with the same T as the others")
        k = x.shape[1]
        n = packed.shape[0]
        _need_shape(packed, f"problem {i}: packed", (n, k // 4))
        _need_shape(gamma, f"problem {i}: gamma", (1,))
        _same_device("linear_grouped", xs[0], x, packed, gamma)
        y = torch.empty((t, n), dtype=torch.float32, device=x.device)
        xq = torch.empty((t, k), dtype=torch.int8, device=x.device)
        absmax = torch.empty(t, dtype=torch.float32, device=x.device)
        acc = torch.empty((t, n), dtype=torch.int32, device=x.device) if want_acc else None
        descs[i] = BlLinear(x.data_ptr(), packed.data_ptr(), gamma.data_ptr(), n, k,
                            y.data_ptr(), xq.data_ptr(), absmax.data_ptr(),
                            acc.data_ptr() if acc is not None else None)
        outs.append((y, xq, absmax, acc))
    _check(lib.bitlinear_linear_grouped(descs, len(xs), t, dt, _stream(xs[0].device)))
    return outs


def interleave_rows(packed_a, packed_b):
    """Row interleave of two packed [N, K/4] matrices -> [2N, K/4] (row 2i
    from a, 2i + 1 from b), the weight layout of gated_relu2."""
    lib = load()
    _need_cuda(packed_a, "packed_a", torch.uint8)
    _need_cuda(packed_b, "packed_b", torch.uint8)
    if packed_a.dim() != 2 or packed_a.shape != packed_b.shape:
        raise ValueError("the two packed matrices must be [N, K/4] of the same shape")
    _same_device("interleave_rows", packed_a, packed_b)
    n, k4 = packed_a.shape
    out = torch.empty((2 * n, k4), dtype=torch.uint8, device=packed_a.device)
    _check(lib.bitlinear_interleave_rows(_ptr(packed_a), _ptr(packed_b), n, 4 * k4, _ptr(out),
                                         _stream(packed_a.device)))
    return out


def gated_relu2(x, packed_gu, gamma_gate, gamma_up, want_acc=False):
    """Gate and up projections of x [T, K] (float32 or bfloat16) with the
    squared-ReLU gate, written as bfloat16: returns (h bfloat16 [T, N], xq,
    absmax, acc int32 [T, 2N] or None); packed_gu from interleave_rows."""
    lib = load()
    _need_cuda(x, "x")
    _need_cuda(packed_gu, "packed_gu", torch.uint8)
    _need_cuda(gamma_gate, "gamma_gate", torch.float32)
    _need_cuda(gamma_up, "gamma_up", torch.float32)
    dt = {torch.float32: BL_F32, torch.bfloat16: BL_BF16}.get(x.dtype)
    if dt is None:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 2 or packed_gu.dim() != 2:
        raise ValueError("x must be [T, K] and packed_gu [2N, K/4]")
    t, k = x.shape
    n2 = packed_gu.shape[0]
    if n2 % 2 or packed_gu.shape[1] * 4 != k:
        raise ValueError("packed_gu must be [2N, K/4]")
    _need_shape(gamma_gate, "gamma_gate", (1,))
    _need_shape(gamma_up, "gamma_up", (1,))
    _same_device("gated_relu2", x, packed_gu, gamma_gate, gamma_up)
    n = n2 // 2
    h = torch.empty((t, n), dtype=torch.bfloat16, device=x.device)
    xq = torch.empty((t, k), dtype=torch.int8, device=x.device)
    absmax = torch.empty(t, dtype=torch.float32, device=x.device)
    acc = torch.empty((t, n2), dtype=torch.int32, device=x.device) if want_acc else None
    _check(lib.bitlinear_gated_relu2(_ptr(x), dt, _ptr(packed_gu), _ptr(gamma_gate),
                                     _ptr(gamma_up), t, n, k, _ptr(h), _ptr(xq), _ptr(absmax),
                                     _ptr(acc), _stream(x.device)))
    return h, xq, absmax, acc


def pack_weights_binary(w):
    """Step A0 for binary weights on the GPU: float32 [N, K] -> (packed uint8
    [N, K/8], gamma float32[1]); K a multiple of 256, at most 32768."""
    lib = load()
    _need_cuda(w, "w", torch.float32)
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    packed = torch.empty((n, k // 8), dtype=torch.uint8, device=w.device)
    gamma = torch.empty(1, dtype=torch.float32, device=w.device)
    ws_bytes = lib.bitlinear_pack_workspace_bytes(n, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=w.device)
    _check(lib.bitlinear_pack_weights_binary(_ptr(w), n, k, _ptr(packed), _ptr(gamma), _ptr(ws),
                                             ws_bytes, _stream(w.device)))
    return packed, gamma


def forward_binary(packed, gamma, xq, absmax, algo="auto", want_acc=False):
    """Steps A2 + A3 on binary weights: -> y float32[T, N] (and acc int32)."""
    lib = load()
    _need_cuda(packed, "packed", torch.uint8)
    _need_cuda(gamma, "gamma", torch.float32)
    _need_cuda(xq, "xq", torch.int8)
    _need_cuda(absmax, "absmax", torch.float32)
    if xq.dim() != 2 or packed.dim() != 2:
        raise ValueError("xq must be [T, K] and packed [N, K/8]")
    t, k = xq.shape
    n = packed.shape[0]
    if packed.shape[1] * 8 != k:
        raise ValueError("packed must be [N, K/8]")
    _need_shape(gamma, "gamma", (1,))
    _need_shape(absmax, "absmax", (t,))
    _same_device("forward_binary", packed, gamma, xq, absmax)
    y = torch.empty((t, n), dtype=torch.float32, device=xq.device)
    acc = torch.empty((t, n), dtype=torch.int32, device=xq.device) if want_acc else None
    _check(lib.bitlinear_forward_binary(_ptr(packed), _ptr(gamma), _ptr(xq), _ptr(absmax), t, n, k,
                                        _ptr(y), _ptr(acc), ALGOS[algo], _stream(xq.device)))
    return (y, acc) if want_acc else y


def calib_empty(device=None):
    """One empty kernel on the current stream of `device` (the launch floor)."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    _check(load().bitlinear_calib_empty(_stream(dev)))


#: layouts of calib_read (bl_read_layout)
READ_CHUNKS, READ_STRIDE = 0, 1


def calib_read(buf, layout=READ_CHUNKS, sink=None):
    """Read the whole of `buf` (a contiguous CUDA tensor, 16-byte aligned, size a
    multiple of 16 bytes) at full width in `layout` (READ_CHUNKS: contiguous
    32 KiB chunks per block; READ_STRIDE: a grid-stride loop); returns the int32
    sink whose 4096 entries (one per wave) XOR to the XOR of the buffer's 32-bit
    words."""
    lib = load()
    _need_cuda(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(lib.bitlinear_calib_sink_len(), dtype=torch.int32, device=buf.device)
    _need_cuda(sink, "sink", torch.int32)
    _need_shape(sink, "sink", (lib.bitlinear_calib_sink_len(),))
    _check(lib.bitlinear_calib_read(_ptr(buf), nbytes, int(layout), _ptr(sink),
                                    _stream(buf.device)))
    return sink


def calib_mfma(iters, byte=1, device=None, sink=None):
    """4096 waves x iters rounds of four v_mfma_i32_32x32x32_i8 (4 * iters *
    4096 * 32768 int8 multiply-adds); returns the int32 sink, each of whose
    first 4096 entries is 4 * iters * 32 * byte^2 (mod 2^32)."""
    lib = load()
    dev = torch.device("cuda") if device is None else torch.device(device)
    if sink is None:
        sink = torch.empty(lib.bitlinear_calib_sink_len(), dtype=torch.int32, device=dev)
    _need_cuda(sink, "sink", torch.int32)
    _need_shape(sink, "sink", (lib.bitlinear_calib_sink_len(),))
    _check(lib.bitlinear_calib_mfma(int(iters), int(byte), _ptr(sink), _stream(sink.device)))
    return sink
