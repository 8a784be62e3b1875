"""The C ABI without a GPU: the library loads, exports every function that
include/bitlinear.h declares, and rejects bad arguments with the documented
status before making any HIP call (so these run on a CPU-only host).

Every call below fails at least one host-side check; none reaches a launch.
"""

import ctypes
import os
import re
import threading

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "bitlinear.h")

BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_WORKSPACE, BL_ERR_HIP, BL_ERR_ARG = range(8)

# fake device addresses: never dereferenced, every call using them fails a check
A16 = 0x7F0000000000
A_ODD = 0x7F0000000001


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib(built_lib):
    from bitlinear_w1_a8_amd import binding
    return binding.load()


def test_header_symbols_exported(lib):
    names = header_functions()
    assert len(names) == 19
    for name in names:
        assert hasattr(lib, name), name


def test_binding_covers_header():
    from bitlinear_w1_a8_amd import binding
    assert sorted(binding.SIGNATURES) == header_functions()


def test_constants(lib):
    assert lib.bitlinear_abi_version() == 3
    assert lib.bitlinear_gemv_max_tokens() == 64
    assert lib.bitlinear_pack_workspace_bytes(2560, 2560) == 2048
    assert lib.bitlinear_pack_workspace_bytes(28672, 8192) == 2048


def _err(lib):
    return lib.bitlinear_last_error().decode()


def test_pack_errors(lib):
    f = lib.bitlinear_pack_weights
    assert f(None, 16, 64, A16, A16, A16, 4096, None) == BL_ERR_NULL
    assert "NULL" in _err(lib)
    assert f(A16, 16, 40, A16, A16, A16, 4096, None) == BL_ERR_SHAPE
    assert "K=40" in _err(lib)
    assert f(A16, 16, 0, A16, A16, A16, 4096, None) == BL_ERR_SHAPE
    assert f(A16, 16, 131072 + 16, A16, A16, A16, 4096, None) == BL_ERR_SHAPE
    assert f(A16, 0, 64, A16, A16, A16, 4096, None) == BL_ERR_SHAPE
    assert f(A16, (1 << 26) + 1, 64, A16, A16, A16, 4096, None) == BL_ERR_SHAPE
    assert f(A_ODD, 16, 64, A16, A16, A16, 4096, None) == BL_ERR_ALIGN
    assert f(A16, 16, 64, A16 + 8, A16, A16, 4096, None) == BL_ERR_ALIGN
    assert f(A16, 16, 64, A16, A16, A16 + 4, 4096, None) == BL_ERR_ALIGN
    assert f(A16, 16, 64, A16, A16, A16, 2047, None) == BL_ERR_WORKSPACE
    assert "2048" in _err(lib)


def test_pack_noalloc_errors(lib):
    f = lib.bitlinear_pack_weights_noalloc
    assert f(None, 16, 64, A16, A16, None) == BL_ERR_NULL
    assert f(A16, 16, 64, None, A16, None) == BL_ERR_NULL
    assert f(A16, 16, 64, A16, None, None) == BL_ERR_NULL
    assert f(A16, 16, 40, A16, A16, None) == BL_ERR_SHAPE
    assert f(A16, 0, 64, A16, A16, None) == BL_ERR_SHAPE
    # the fixed buckets sum at most 2^38 weights exactly
    assert f(A16, 1 << 26, 8192, A16, A16, None) == BL_ERR_SHAPE
    assert "2^38" in _err(lib)
    assert f(A_ODD, 16, 64, A16, A16, None) == BL_ERR_ALIGN
    assert f(A16, 16, 64, A16 + 8, A16, None) == BL_ERR_ALIGN
    assert f(A16, 16, 64, A16, A16 + 2, None) == BL_ERR_ALIGN


def test_quant_errors(lib):
    f = lib.bitlinear_quant_act
    assert f(A16, 1, 4, 64, None, A16, None, None) == BL_ERR_NULL
    assert f(A16, 1, 4, 64, A16, None, None, None) == BL_ERR_NULL
    assert f(A16, 2, 4, 64, A16, A16, None, None) == BL_ERR_DTYPE
    assert f(A16, -1, 4, 64, A16, A16, None, None) == BL_ERR_DTYPE
    assert f(A16, 1, 4, 63, A16, A16, None, None) == BL_ERR_SHAPE
    assert f(A16, 1, 0, 64, A16, A16, None, None) == BL_ERR_SHAPE
    assert f(A16, 1, (1 << 24) + 1, 64, A16, A16, None, None) == BL_ERR_SHAPE
    assert f(A16 + 8, 1, 4, 64, A16, A16, None, None) == BL_ERR_ALIGN
    assert f(A16, 1, 4, 64, A16 + 1, A16, None, None) == BL_ERR_ALIGN
    assert f(A16, 1, 4, 64, A16, A16 + 2, None, None) == BL_ERR_ALIGN
    assert f(A16, 1, 4, 64, A16, A16, A16 + 2, None) == BL_ERR_ALIGN


def test_forward_errors(lib):
    f = lib.bitlinear_forward_algo
    good = (A16, A16, A16, A16, None)          # packed, gamma, xq, absmax, rowsum
    assert f(None, A16, A16, A16, None, 1, 16, 64, A16, None, 0, None) == BL_ERR_NULL
    assert f(*good, 1, 16, 64, None, None, 0, None) == BL_ERR_NULL
    assert f(*good, 1, 16, 48 + 1, A16, None, 0, None) == BL_ERR_SHAPE
    assert f(*good, 0, 16, 64, A16, None, 0, None) == BL_ERR_SHAPE
    assert f(*good, 1, 0, 64, A16, None, 0, None) == BL_ERR_SHAPE
    assert f(*good, 1 << 20, 1 << 20, 64, A16, None, 0, None) == BL_ERR_SHAPE
    assert f(A16 + 4, A16, A16, A16, None, 1, 16, 64, A16, None, 0, None) == BL_ERR_ALIGN
    assert f(A16, A16, A16 + 8, A16, None, 1, 16, 64, A16, None, 0, None) == BL_ERR_ALIGN
    assert f(*good, 1, 16, 64, A16 + 2, None, 0, None) == BL_ERR_ALIGN
    assert f(*good, 1, 16, 64, A16, A16 + 1, 0, None) == BL_ERR_ALIGN
    # rowsum: NULL is accepted (the kernels derive the sums), a given one must be aligned
    assert f(A16, A16, A16, A16, A16 + 2, 1, 16, 64, A16, None, 0, None) == BL_ERR_ALIGN
    assert "alignment" in _err(lib)
    assert f(A16, A16, A16, A16, A16, 1, 16, 64, A16, None, 5, None) == BL_ERR_ARG
    assert f(*good, 1, 16, 64, A16, None, 5, None) == BL_ERR_ARG
    assert f(*good, 1, 16, 64, A16, None, -1, None) == BL_ERR_ARG
    assert lib.bitlinear_forward(None, A16, A16, A16, None, 1, 16, 64, A16, None, None) == BL_ERR_NULL
    assert lib.bitlinear_forward(A16, A16, A16, A16, A16 + 1, 1, 16, 64, A16, None, None) == BL_ERR_ALIGN


def test_header_returns_bl_status():
    # every entry point that reports a status is declared to return bl_status
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decls = dict((n, r) for r, n in re.findall(r"\b(\w+)\s+(bitlinear_\w+)\s*\(", text))
    values = {"bitlinear_abi_version": "int", "bitlinear_last_error": "char",
              "bitlinear_gemv_max_tokens": "int64_t", "bitlinear_pack_workspace_bytes": "size_t",
              "bitlinear_calib_sink_len": "int64_t"}
    for name, ret in decls.items():
        assert ret == values.get(name, "bl_status"), (name, ret)


def test_subln_quant_act_errors(lib):
    f = lib.bitlinear_subln_quant_act
    ok = (A16, 1, A16, 1e-5, 4, 64, A16, A16, None, None)
    assert f(None, *ok[1:]) == BL_ERR_NULL
    assert f(ok[0], ok[1], None, *ok[3:]) == BL_ERR_NULL
    assert f(*ok[:7], None, None, None) == BL_ERR_NULL
    assert f(ok[0], 5, *ok[2:]) == BL_ERR_DTYPE
    for bad in (0.0, -1e-5, float("inf"), float("nan")):
        assert f(*ok[:3], bad, *ok[4:]) == BL_ERR_ARG
    assert f(*ok[:4], 4, 72, *ok[6:]) == BL_ERR_SHAPE       # K % 16
    assert f(*ok[:4], 0, 64, *ok[6:]) == BL_ERR_SHAPE
    assert f(ok[0], ok[1], A16 + 4, *ok[3:]) == BL_ERR_ALIGN  # gain read 16 bytes at a time
    assert f(*ok[:7], A16 + 2, None, None) == BL_ERR_ALIGN
    assert "eps_n" in (f(*ok[:3], 0.0, *ok[4:]) and _err(lib))


def test_last_error_is_per_thread(lib):
    assert lib.bitlinear_quant_act(None, 1, 4, 64, A16, A16, None, None) == BL_ERR_NULL
    seen = {}

    def other():
        seen["before"] = _err(lib)
        lib.bitlinear_quant_act(A16, 7, 4, 64, A16, A16, None, None)
        seen["after"] = _err(lib)

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["before"] == ""
    assert "x_dtype 7" in seen["after"]
    assert "NULL" in _err(lib)


def test_binding_raises(built_lib):
    from bitlinear_w1_a8_amd import binding
    with pytest.raises(binding.BitLinearError) as ei:
        binding._check(BL_ERR_SHAPE)
    assert ei.value.status == BL_ERR_SHAPE


def test_linear_grouped_errors(lib):
    from bitlinear_w1_a8_amd.binding import BlLinear
    f = lib.bitlinear_linear_grouped
    good = BlLinear(A16, A16, A16, 32, 256, A16, A16, A16, None)
    arr = (BlLinear * 9)(*([good] * 9))
    assert f(None, 1, 1, 1, None) == BL_ERR_NULL
    assert f(arr, 0, 1, 1, None) == BL_ERR_ARG
    assert f(arr, 9, 1, 1, None) == BL_ERR_ARG
    assert f(arr, 2, 1, 3, None) == BL_ERR_DTYPE
    assert f(arr, 2, 0, 1, None) == BL_ERR_SHAPE
    bad = (BlLinear * 2)(good, BlLinear(A16, A16, A16, 32, 256, A16, None, A16, None))
    assert f(bad, 2, 1, 1, None) == BL_ERR_NULL
    assert "problem 1" in _err(lib)
    bad = (BlLinear * 2)(good, BlLinear(A16, A16, A16, 32, 250, A16, A16, A16, None))
    assert f(bad, 2, 1, 1, None) == BL_ERR_SHAPE
    bad = (BlLinear * 2)(good, BlLinear(A16 + 2, A16, A16, 32, 256, A16, A16, A16, None))
    assert f(bad, 2, 1, 1, None) == BL_ERR_ALIGN
    bad = (BlLinear * 1)(BlLinear(A16, A16, A16, 0, 256, A16, A16, A16, None))
    assert f(bad, 1, 1, 1, None) == BL_ERR_SHAPE


def test_interleave_rows_errors(lib):
    f = lib.bitlinear_interleave_rows
    assert f(None, A16, 4, 64, A16, None) == BL_ERR_NULL
    assert f(A16, A16, 4, 64, None, None) == BL_ERR_NULL
    assert f(A16, A16, 0, 64, A16, None) == BL_ERR_SHAPE
    assert f(A16, A16, (1 << 25) + 1, 64, A16, None) == BL_ERR_SHAPE
    assert f(A16, A16, 4, 40, A16, None) == BL_ERR_SHAPE
    assert f(A16, A16 + 2, 4, 64, A16, None) == BL_ERR_ALIGN


def test_gated_relu2_errors(lib):
    f = lib.bitlinear_gated_relu2
    ok = [A16, 1, A16, A16, A16, 4, 100, 256, A16, A16, A16, None, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    for i in (0, 2, 3, 4, 8, 9, 10):
        assert call(**{f"a{i}": None}) == BL_ERR_NULL
    assert call(a1=2) == BL_ERR_DTYPE
    assert call(a5=0) == BL_ERR_SHAPE
    assert call(a6=0) == BL_ERR_SHAPE
    assert call(a6=(1 << 25) + 1) == BL_ERR_SHAPE
    assert call(a7=264) == BL_ERR_SHAPE            # K % 16
    assert call(a2=A16 + 4) == BL_ERR_ALIGN        # packed rows read 16 bytes at a time
    assert call(a8=A16 + 1) == BL_ERR_ALIGN        # bfloat16 output
    assert call(a11=A16 + 2) == BL_ERR_ALIGN
    assert "bitlinear_gated_relu2" in (call(a5=0) and _err(lib))


def test_binary_errors(lib):
    f = lib.bitlinear_pack_weights_binary
    assert f(None, 4, 256, A16, A16, A16, 4096, None) == BL_ERR_NULL
    assert f(A16, 4, 128, A16, A16, A16, 4096, None) == BL_ERR_SHAPE      # K % 256
    assert f(A16, 4, 32768 + 256, A16, A16, A16, 4096, None) == BL_ERR_SHAPE
    assert f(A16, 0, 256, A16, A16, A16, 4096, None) == BL_ERR_SHAPE
    assert f(A16 + 4, 4, 256, A16, A16, A16, 4096, None) == BL_ERR_ALIGN
    assert f(A16, 4, 256, A16, A16, A16, 8, None) == BL_ERR_WORKSPACE
    g = lib.bitlinear_forward_binary
    ok = (A16, A16, A16, A16, 2, 64, 512, A16, None, 0, None)
    assert g(None, *ok[1:]) == BL_ERR_NULL
    assert g(*ok[:7], None, None, 0, None) == BL_ERR_NULL
    assert g(*ok[:6], 768 + 32, *ok[7:]) == BL_ERR_SHAPE
    assert g(*ok[:4], 0, *ok[5:]) == BL_ERR_SHAPE
    assert g(*ok[:5], 0, *ok[6:]) == BL_ERR_SHAPE
    assert g(A16 + 8, *ok[1:]) == BL_ERR_ALIGN
    assert g(*ok[:9], 3, None) == BL_ERR_ARG                        # no table-lookup kernel
    assert g(*ok[:9], 4, None) == BL_ERR_ARG                        # nor a v_dot4 one
    assert g(*ok[:9], 9, None) == BL_ERR_ARG
    assert "binary" in (g(*ok[:9], 3, None) and _err(lib))


def test_calib_errors(lib):
    """The measurement helpers check their arguments like every other call."""
    assert lib.bitlinear_calib_sink_len() == 4096
    r = lib.bitlinear_calib_read
    for lay in (0, 1):
        assert r(None, 1024, lay, A16, None) == BL_ERR_NULL
        assert r(A16, 1024, lay, None, None) == BL_ERR_NULL
        assert r(A16, 0, lay, A16, None) == BL_ERR_SHAPE
        assert r(A16, 1000, lay, A16, None) == BL_ERR_SHAPE         # not a multiple of 16
        assert r(A16, (1 << 40) + 16, lay, A16, None) == BL_ERR_SHAPE
        assert r(A16 + 8, 1024, lay, A16, None) == BL_ERR_ALIGN
        assert r(A16, 1024, lay, A_ODD, None) == BL_ERR_ALIGN
    assert r(A16, 1024, 2, A16, None) == BL_ERR_ARG
    assert r(A16, 1024, -1, A16, None) == BL_ERR_ARG
    assert "layout" in (r(A16, 1024, 2, A16, None) and _err(lib))
    m = lib.bitlinear_calib_mfma
    assert m(16, 1, None, None) == BL_ERR_NULL
    assert m(0, 1, A16, None) == BL_ERR_ARG
    assert m((1 << 20) + 1, 1, A16, None) == BL_ERR_ARG
    assert m(16, 128, A16, None) == BL_ERR_ARG
    assert m(16, -129, A16, None) == BL_ERR_ARG
    assert m(16, 1, A_ODD, None) == BL_ERR_ALIGN
    assert "iters" in (m(0, 1, A16, None) and _err(lib))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No CPU fallback: without the built library every entry point raises."""
    from bitlinear_w1_a8_amd import binding
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libbitlinear.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(ImportError):
        binding.load()
    with pytest.raises(ImportError):
        binding.gemv_max_tokens()


def test_product_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "bitlinear_w1_a8_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f
