"""Parity of the HIP path with the CPU oracle (needs an MI355X).

Every test feeds the same seeded inputs to both sides and compares element
by element: packed bytes, gamma bits, int8 activations, absmax bits, row sums
and int32 sums must be equal; float32 outputs must be within 1e-5 relative of
the oracle's binary64 values, and exactly +0 wherever the sum is 0.  Test ids
name the shapes, so a failing or faulting case is named by `pytest -v`.
"""

import numpy as np
import pytest
import torch

import oracle
from bitlinear_w1_a8_amd import workloads as wl

pytestmark = pytest.mark.gpu

Y_RTOL = 1e-5


@pytest.fixture(scope="module")
def bl(built_lib):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from bitlinear_w1_a8_amd import binding
    binding.load()
    return binding


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ------------------------------------------------------------------ checks

def check_pack(bl, w):
    packed_ref, gamma_ref = oracle.pack_weights(w)
    packed, gamma = bl.pack_weights(dev(w))
    g = host(gamma)
    assert g.view(np.uint32)[0] == np.float32(gamma_ref).view(np.uint32), (g[0], gamma_ref)
    p = host(packed)
    bad = int(np.count_nonzero(p != packed_ref))
    assert bad == 0, f"{bad} of {p.size} packed bytes differ"
    return packed, gamma, packed_ref, gamma_ref


def check_quant(bl, x, dtype):
    if dtype == "bf16":
        bits = wl.bf16_bits(x)
        q_ref, a_ref, rs_ref = oracle.quant_act(bits)
        xin = dev_bf16(bits)
    else:
        q_ref, a_ref, rs_ref = oracle.quant_act(x)
        xin = dev(x)
    xq, absmax, rowsum = bl.quant_act(xin)
    q = host(xq)
    bad = int(np.count_nonzero(q != q_ref))
    assert bad == 0, f"{bad} of {q.size} int8 activations differ"
    assert np.array_equal(host(absmax).view(np.uint32), a_ref.view(np.uint32))
    assert np.array_equal(host(rowsum), rs_ref)
    return xq, absmax, q_ref, a_ref, rowsum


def check_y(y, acc_ref, gamma, absmax_ref):
    y_ref = oracle.rescale(acc_ref, gamma, absmax_ref)
    zero = acc_ref == 0
    assert np.all(y[zero] == 0.0) and not np.any(np.signbit(y[zero]))
    nz = ~zero
    if np.any(nz):
        rel = np.abs(y[nz].astype(np.float64) - y_ref[nz]) / np.abs(y_ref[nz])
        assert float(rel.max()) <= Y_RTOL, f"max relative error {rel.max():.3g}"


def check_forward(bl, packed_dev, gamma_dev, xq_dev, absmax_dev, t_ref, q_ref, gamma_ref,
                  absmax_ref, algo, rowsum_dev=None):
    """The forward without row sums (each kernel derives them), and for the
    matrix-core kernels also with the tokens' row sums given: the int32 sums
    must equal the oracle's and y must be the same bits both ways."""
    n = t_ref.shape[0]
    y, acc = bl.forward(packed_dev, gamma_dev, xq_dev, absmax_dev, n, algo=algo, want_acc=True)
    acc_ref = oracle.contract(q_ref, t_ref)
    a = host(acc)
    bad = int(np.count_nonzero(a != acc_ref))
    assert bad == 0, f"{bad} of {a.size} int32 sums differ ({algo})"
    yh = host(y)
    check_y(yh, acc_ref, gamma_ref, absmax_ref)
    if algo in ("auto", "gemv", "gemm"):
        if rowsum_dev is None:
            rowsum_dev = dev(q_ref.astype(np.int64).sum(axis=1).astype(np.int32))
        y2, acc2 = bl.forward(packed_dev, gamma_dev, xq_dev, absmax_dev, n, algo=algo,
                              want_acc=True, rowsum=rowsum_dev)
        bad = int(np.count_nonzero(host(acc2) != acc_ref))
        assert bad == 0, f"{bad} of {a.size} int32 sums differ ({algo}, rowsum given)"
        assert np.array_equal(host(y2).view(np.uint32), yh.view(np.uint32))
    return a


# ------------------------------------------------------------------ step A0

PACK_SHAPES = [(1, 16), (2, 32), (3, 48), (16, 64), (17, 272), (33, 96), (512, 256),
               (640, 2560), (2560, 2560), (6912, 2560), (2560, 6912)]


@pytest.mark.parametrize("n,k", PACK_SHAPES, ids=[f"N{n}_K{k}" for n, k in PACK_SHAPES])
def test_pack_random(bl, n, k):
    check_pack(bl, wl.latent_weights(n, k, 0.02, 7000 + n + k))


def _tie_matrix():
    """Weights with W/(gamma+eps) exactly +-0.5 (round to 0) and +-0.5 ulp
    around it, at a fixed point of gamma."""
    base = np.full((16, 64), 0.5, np.float32)
    d = np.float32(0.5)
    for _ in range(6):
        w = base.copy()
        half = np.float32(0.5) * d
        w[0, :8] = [half, -half, np.nextafter(half, np.float32(1)), -np.nextafter(half, np.float32(1)),
                    np.nextafter(half, np.float32(0)), half, half, -half]
        w[1, :4] = [np.float32(1.5) * d, np.float32(-1.5) * d, np.float32(2.5) * d, 0.0]
        g = oracle.absmean_gamma(w)
        d_new = np.float32(g) + np.float32(1e-5)
        if d_new == d:
            break
        d = d_new
    u = w[0, :2] / (np.float32(oracle.absmean_gamma(w)) + np.float32(1e-5))
    assert np.all(np.abs(u) == 0.5)
    return w


def _awkward_matrix():
    rng = np.random.default_rng(77)
    mant = rng.random((64, 96)) + 0.5
    expo = rng.integers(-140, 60, size=(64, 96))
    w = (mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    w *= np.where(rng.random((64, 96)) < 0.5, -1, 1).astype(np.float32)
    w[rng.random((64, 96)) < 0.1] = 0.0
    return w


def _huge_matrix():
    """Exponents from 2^-100 to 2^120: some above where the histogram pass
    sums in fixed point, the rest spread over more than its window."""
    rng = np.random.default_rng(78)
    mant = rng.random((64, 128)) + 0.5
    expo = rng.integers(-100, 121, size=(64, 128))
    w = (mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    return w * np.where(rng.random((64, 128)) < 0.5, -1, 1).astype(np.float32)


def _late_large_matrix():
    """Small weights first, then a few far larger ones late in the scan: the
    sums taken so far move into the buckets and the reference rises."""
    w = wl.latent_weights(128, 512, 0.02, 79)
    w[100, 7] = np.float32(1e20)
    w[127, 511] = np.float32(-3e36)
    w[120, 300] = np.float32(7.5e-3)
    return w


SPECIAL = {
    "all_zero": lambda: np.zeros((32, 64), np.float32),
    "huge_exponents": _huge_matrix,
    "late_large": _late_large_matrix,
    "constant": lambda: np.full((8, 128), np.float32(-0.0123), np.float32),
    "ties": _tie_matrix,
    "awkward_exponents": _awkward_matrix,
    "one_row_zero": lambda: np.where(np.arange(64)[:, None] == 5, 0.0,
                                     wl.latent_weights(64, 256, 0.02, 5)).astype(np.float32),
}


@pytest.mark.parametrize("name", sorted(SPECIAL))
def test_pack_special(bl, name):
    _, _, packed_ref, _ = check_pack(bl, SPECIAL[name]())
    if name == "all_zero":
        assert np.all(packed_ref == 0x55)


# ------------------------------------------------------------------ step A1

QUANT_SHAPES = [(1, 16), (4, 256), (7, 48), (3, 2560), (2, 6912), (1, 28672), (65, 8192),
                (300, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("t,k", QUANT_SHAPES, ids=[f"T{t}_K{k}" for t, k in QUANT_SHAPES])
def test_quant_random(bl, t, k, dtype):
    x = wl.activations_student_t(t, k, 4, 9000 + t + k)
    check_quant(bl, x, dtype)


def test_quant_wide_f32(bl):
    # more 16-byte vectors than one pass holds in registers: re-read path
    x = wl.activations_normal(2, 65536, 31, 0.01, 8.0)
    check_quant(bl, x, "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_special_rows(bl, dtype):
    rng = np.random.default_rng(41)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    x[0] = 0.0                                            # all-zero token
    x[1, :8] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -126.5, 126.5]  # exact ties
    x[1, 8:] = 0.25
    x[2] *= np.float32(1e-30)                             # tiny values
    x[3] *= np.float32(1e30)                              # huge values
    x[4, :] = np.float32(-3.0)                            # constant negative row
    x[5, :] = np.float32(1e-39)                           # subnormal row
    x[6, 3] = np.float32(1e4)                             # one outlier
    check_quant(bl, x, dtype)


# ------------------------------------------------------------------ steps A2 + A3

FWD_SHAPES = [(1, 1, 16), (1, 16, 64), (2, 17, 48), (3, 5, 16), (4, 512, 256), (16, 33, 320),
              (17, 100, 256), (33, 64, 128), (64, 200, 1024), (65, 130, 192), (130, 257, 272),
              (1, 2560, 2560), (8, 640, 2560), (1, 100, 6912), (5, 37, 28672),
              # decode kernel edges: ragged N, T = 16 at the staging limit,
              # many waves per block, one chunk per wave
              (3, 37, 512), (16, 50, 2048), (2, 17, 8192), (1, 3, 256), (1, 1000, 28672),
              # prefill kernel on ragged T and N: 48 tiles of 64 x 128 with K
              # in 6 parts (the last one short); 112 tiles, which take
              # 128 x 512 tiles with K in parts; the 128 x 256 tiles; the
              # 128 x 512 tiles
              (200, 1500, 28672), (200, 3500, 16384), (1100, 3800, 512), (1500, 8100, 256),
              # table-lookup kernel: 4-wave blocks with word loads and a short last chunk
              (40, 900, 3088),
              # decode kernel, several int8 tokens, 257 row tiles: two per block
              (9, 4100, 1024),
              # one int8 token over 512 tiles and more: ragged last tiles,
              # a short last wave (K = 2304: 9 chunks), one chunk per row,
              # 4 and 7 chunks per wave, K = 32768
              (1, 8200, 2304), (1, 12288, 1024), (1, 20480, 512), (1, 16384, 256),
              (1, 30000, 1024), (1, 9000, 16384), (1, 8192, 32768),
              (1, 24576, 512), (1, 20480, 8448), (1, 12288, 16640),
              # the longest rows the boundary takes (K = 131072: the largest
              # sums, 127 K, are still exact in binary32)
              (2, 40, 131072), (70, 300, 131072),
              # up to 64 tokens over fewer than 40 tiles of 64 x 128: K split
              # into parts, the last one short (18 and 54 steps of 128)
              (33, 200, 2304), (64, 2560, 6912), (61, 4900, 1152),
              # decode kernel, rows not a multiple of 256 k (a short last
              # chunk of one to three 64-k quads): the 3B-class rows (3200,
              # 8640), one partial chunk only, T = 16, two row tiles per
              # block (several tokens; one token over 513 tiles)
              (1, 3200, 3200), (1, 3200, 8640), (4, 300, 64), (3, 100, 128),
              (16, 40, 448), (9, 4100, 576), (1, 8200, 704),
              # K % 128 == 64 with K in parts (the half step in the last
              # part): 64 x 128 tiles at up to 64 tokens and over few tiles
              # of long rows
              (33, 200, 2368), (64, 2560, 8640), (128, 3200, 8640), (200, 1500, 16448),
              # up to four int8 tokens over long rows: the decode kernel
              # stages up to 128 KiB of activations (a short last chunk too)
              (2, 300, 28672), (4, 1000, 28672), (3, 64, 24640),
              # two to four int8 tokens over 512 tiles and more: the
              # persistent kernel with one LDS row per token (ragged last
              # tiles, one chunk per row)
              (2, 8200, 2304), (3, 12288, 1024), (4, 9000, 8192), (4, 30000, 256),
              # ... and at the largest tile count it takes (64 tiles per block)
              (4, 524288, 256),
              # 64 x 128 tiles on eight waves of 32 x 32 (unsplit; ragged T and N)
              (200, 4000, 8192), (77, 1000, 1024)]


def _forward_inputs(t, n, k, seed, zero_rows=True):
    rng = np.random.default_rng(seed)
    tern = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    if zero_rows and n > 2:
        tern[n // 2] = 0
    x = wl.activations_student_t(t, k, 4, seed + 1)
    if t > 2:
        x[t // 2] = 0.0
    q, absmax, _ = oracle.quant_act(x)
    gamma = np.float32(0.0173)
    return tern, q, absmax, gamma


@pytest.mark.parametrize("algo", ["gemv", "gemm", "lut", "dot4"])
@pytest.mark.parametrize("t,n,k", FWD_SHAPES, ids=[f"T{t}_N{n}_K{k}" for t, n, k in FWD_SHAPES])
def test_forward_shapes(bl, t, n, k, algo):
    tern, q, absmax, gamma = _forward_inputs(t, n, k, 100 * t + n + k)
    check_forward(bl, dev(oracle.pack_ternary(tern)), dev(np.array([gamma])), dev(q), dev(absmax),
                  tern, q, gamma, absmax, algo)


# prefill-sized problems on the 128 x 512 tiles: ragged T and N (partial
# tiles in both directions), K steps 1, 4 and 5 (a whole three-stage cycle,
# one and two steps past it)
WIDE_SHAPES = [(2085, 6976, 512), (2048, 6500, 640), (2304, 6400, 128),
               # 272 tiles of 128 x 512 (a second round under a quarter full):
               # 64 x 256 tiles instead
               (2048, 8300, 384),
               # 64 x 320 tiles (256 of them, the last ones ragged in T and N)
               (2000, 2500, 1024),
               # K % 128 == 64, a half last K step on every tile shape: the
               # 3B-class down projection (64 x 256), 128 x 512 (ragged),
               # 128 x 256, 64 x 320, 64 x 128 (four stages)
               (2048, 3200, 8640), (2085, 6976, 704), (2048, 3500, 320), (2000, 2500, 1088),
               (256, 3000, 8640)]


@pytest.mark.parametrize("algo", ["gemm", "auto"])
@pytest.mark.parametrize("t,n,k", WIDE_SHAPES, ids=[f"T{t}_N{n}_K{k}" for t, n, k in WIDE_SHAPES])
def test_forward_wide_tiles_ragged(bl, t, n, k, algo):
    tern, q, absmax, gamma = _forward_inputs(t, n, k, 7 * t + n + k)
    check_forward(bl, dev(oracle.pack_ternary(tern)), dev(np.array([gamma])), dev(q), dev(absmax),
                  tern, q, gamma, absmax, algo)


def test_forward_extremes(bl):
    """All q = +-127 against all-ones rows: the largest sums the contraction makes."""
    t, n, k = 3, 48, 4096
    tern = np.ones((n, k), np.int8)
    tern[1::2] = -1
    tern[5] = 0
    q = np.full((t, k), 127, np.int8)
    q[1] = -127
    q[2, ::2] = -127
    absmax = np.array([5.0, 0.25, 1e-7], np.float32)
    gamma = np.float32(3.0)
    for algo in ("gemv", "gemm", "lut", "dot4"):
        a = check_forward(bl, dev(oracle.pack_ternary(tern)), dev(np.array([gamma])), dev(q),
                          dev(absmax), tern, q, gamma, absmax, algo)
        assert a[0, 0] == 127 * k


def test_forward_deterministic_and_kernels_agree(bl):
    t, n, k = 32, 1000, 2560
    tern, q, absmax, gamma = _forward_inputs(t, n, k, 55)
    args = (dev(oracle.pack_ternary(tern)), dev(np.array([gamma])), dev(q), dev(absmax), n)
    runs = [bl.forward(*args, algo=a, want_acc=True) for a in ("gemv", "gemv", "gemm", "gemm")]
    ys = [host(y) for y, _ in runs]
    accs = [host(a) for _, a in runs]
    for i in range(1, 4):
        assert np.array_equal(accs[i], accs[0])
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    assert np.array_equal(ys[2].view(np.uint32), ys[3].view(np.uint32))


def test_forward_on_side_stream(bl):
    t, n, k = 4, 300, 512
    tern, q, absmax, gamma = _forward_inputs(t, n, k, 66)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        args = (dev(oracle.pack_ternary(tern)), dev(np.array([gamma])), dev(q), dev(absmax))
        y, acc = bl.forward(*args, n, want_acc=True)
    s.synchronize()
    assert np.array_equal(acc.cpu().numpy(), oracle.contract(q, tern))


def test_bitlinear_end_to_end(bl):
    w = wl.latent_weights(96, 320, 0.02, 3)
    x = wl.activations_normal(5, 320, 4)
    packed, gamma = bl.pack_weights(dev(w))
    y = host(bl.bitlinear(dev(x), packed, gamma, 96))
    y_ref, acc_ref, _, gamma_ref = oracle.forward(w, x)
    _, a_ref, _ = oracle.quant_act(x)
    check_y(y, acc_ref, gamma_ref, a_ref)


# ------------------------------------------------------------------ the five workloads, full size

def _workload_cases():
    cases = []
    for idx, w in sorted(wl.WORKLOADS.items()):
        for mi, m in enumerate(w.matrices):
            cases.append(pytest.param(idx, mi, id=f"w{idx}_{w.name}_{m.name}_K{m.k}_N{m.n}"))
    return cases


@pytest.mark.parametrize("widx,mi", _workload_cases())
def test_workload_full_size(bl, widx, mi):
    w = wl.WORKLOADS[widx]
    m = w.matrices[mi]
    weights = w.weights(mi)
    packed, gamma, packed_ref, gamma_ref = check_pack(bl, weights)
    tern = oracle.ternarize(weights, gamma_ref)
    del weights
    for t in w.tokens:
        x = w.activations(mi, t)
        xq, absmax, q_ref, a_ref, rowsum = check_quant(bl, x, w.x_dtype)
        algos = ["auto"] + (["gemv", "gemm", "lut", "dot4"] if widx == 3 else []) + (
            ["lut", "dot4"] if widx == 2 else [])
        for algo in algos:
            check_forward(bl, packed, gamma, xq, absmax, tern, q_ref, gamma_ref, a_ref, algo,
                          rowsum_dev=rowsum)
    if widx in (2, 5):
        # the ternary zero fraction of Gaussian weights, about 31%
        assert abs(float(np.mean(tern == 0)) - 0.3101) < 0.005


# ------------------------------------------------------------------ SubLN + A1

SUBLN_CASES = [(1, 2560, "bf16"), (4, 6912, "bf16"), (3, 256, "f32"), (2048, 2560, "bf16"),
               (5, 28672, "bf16"), (7, 48, "f32"), (1, 131072, "bf16"), (65, 4096, "f32")]


def _subln_inputs(t, k, dtype, seed):
    rng = np.random.default_rng(seed)
    x = wl.activations_student_t(t, k, 4, seed + 1)
    if t > 2:
        x[1] = 0.0                                       # an all-zero token
    g = (1.0 + 0.5 * rng.standard_normal(k)).astype(np.float32)   # some gains negative
    if dtype == "bf16":
        bits = wl.bf16_bits(x)
        return bits, dev_bf16(bits), g
    return x, dev(x), g


def check_subln(bl, xref, xin, g):
    """Codes, the scale (absmax of x_hat) and row sums, all bit for bit."""
    q_ref, a_ref, rs_ref, _ = oracle.subln_quant_act(xref, g)
    xq, scale, rowsum = bl.subln_quant_act(xin, dev(g))
    q = host(xq)
    bad = int(np.count_nonzero(q != q_ref))
    assert bad == 0, f"{bad} of {q.size} int8 activations differ"
    assert np.array_equal(host(rowsum), rs_ref)
    sc = host(scale)
    bad = np.flatnonzero(sc.view(np.uint32) != a_ref.view(np.uint32))
    assert bad.size == 0, f"scale differs on tokens {bad[:8]}: {sc[bad[:4]]} vs {a_ref[bad[:4]]}"
    return xq, scale, q_ref, a_ref


@pytest.mark.parametrize("t,k,dtype", SUBLN_CASES, ids=[f"T{t}_K{k}_{d}" for t, k, d in SUBLN_CASES])
def test_subln_quant(bl, t, k, dtype):
    xref, xin, g = _subln_inputs(t, k, dtype, 900 + t + k)
    check_subln(bl, xref, xin, g)


def _subln_special_rows(k, seed):
    """Rows that take every branch of the exact sum of squares: nonzero
    elements more than 31 binades below the row's largest (the per-exponent
    buckets), a row of subnormals (the sum shifted down), zeros, a constant
    row, one huge entry among ones, the worked example's values tiled, and
    the window's edge: every binade from 0 to 31 below the largest (fixed
    point, both bf16 accumulators) and the same with one element 32 below
    (buckets)."""
    rng = np.random.default_rng(seed)
    x = np.zeros((10, k), np.float32)
    x[0] = rng.standard_normal(k) * 10.0 ** rng.uniform(-30, 17, k)
    x[1] = rng.standard_normal(k) * np.float32(1e-39)
    x[2] = 0.0
    x[3] = -0.375
    x[4] = 1.0
    x[4, k // 3] = np.float32(2.0 ** 60)
    x[5] = rng.standard_normal(k)
    x[5, ::37] *= np.float32(1e-13)
    x[6] = np.tile(np.float32([-1.0, -1.0, 4.0, 2.0]), k // 4)
    x[7] = rng.standard_normal(k) * np.float32(1e-30)
    x[7, 5] = np.float32(3e-3)
    x[8] = np.float32(-1.5) * np.exp2(-(np.arange(k) % 32)).astype(np.float32)
    x[9] = x[8]
    x[9, k // 2] = np.float32(2.0 ** -32)
    g = (1.0 + 0.5 * rng.standard_normal(k)).astype(np.float32)
    g[:4] = [1.0, 0.5, 0.25, 0.5]
    return x, g


@pytest.mark.parametrize("k,dtype", [(4096, "f32"), (4096, "bf16"), (64, "f32"), (131072, "f32")],
                         ids=["K4096_f32", "K4096_bf16", "K64_f32", "K131072_f32"])
def test_subln_special(bl, k, dtype):
    x, g = _subln_special_rows(k, 970 + k)
    if dtype == "bf16":
        bits = wl.bf16_bits(x)
        check_subln(bl, bits, dev_bf16(bits), g)
    else:
        check_subln(bl, x, dev(x), g)


def test_subln_worked_example(bl):
    # E6: normalising first gives the code -63 where quantising x * g would
    # give the tie 63.5 -> -64 (K padded to 16 with the same four values)
    x = np.tile(np.float32([-1.0, -1.0, 4.0, 2.0]), 4)[None, :]
    g = np.tile(np.float32([1.0, 0.5, 0.25, 0.5]), 4)
    xq, scale, q_ref, _ = check_subln(bl, x, dev(x), g)
    assert host(xq)[0, :4].tolist() == [-127, -63, 127, 127]


def test_subln_then_forward(bl):
    t, n, k = 4, 2560, 2560
    w = wl.latent_weights(n, k, 0.02, 951)
    packed, gamma, _, gamma_ref = check_pack(bl, w)
    tern = oracle.ternarize(w, gamma_ref)
    xref, xin, g = _subln_inputs(t, k, "bf16", 952)
    xq, scale, q_ref, a_ref = check_subln(bl, xref, xin, g)
    y, acc = bl.forward(packed, gamma, xq, scale, n, want_acc=True)
    acc_ref = oracle.contract(q_ref, tern)
    assert np.array_equal(host(acc), acc_ref)
    check_y(host(y), acc_ref, gamma_ref, a_ref)


# ------------------------------------------------------------------ grouped A1-A3

GROUPS = {
    "layer_qkv_t1_bf16": (1, "bf16", [(2560, 2560), (2560, 640), (2560, 640)]),
    "layer_gateup_t1_bf16": (1, "bf16", [(2560, 6912), (2560, 6912)]),
    "layer_down_t1_bf16": (1, "bf16", [(6912, 2560)]),
    # unequal problems cut into row pieces of the narrowest one's block count
    # (ragged last pieces, int32 sums and y written through the row stride)
    "t1_bf16_cut_ragged": (1, "bf16", [(2560, 100), (2560, 37)]),
    "t3_f32_cut": (3, "f32", [(1024, 300), (1024, 64), (512, 70)]),
    "t4_f32_ragged": (4, "f32", [(256, 37), (512, 100), (768, 1)]),
    "t3_bf16_mixed_k": (3, "bf16", [(2048, 50), (256, 17)]),
    "t2_k28672": (2, "bf16", [(28672, 64)]),
    "eight_problems": (2, "bf16", [(256 * (i + 1), 16 * (i + 1) + 3) for i in range(8)]),
    "fallback_t8": (8, "bf16", [(2560, 200), (512, 33)]),
    "fallback_k_not_256": (2, "f32", [(48, 20), (256, 16)]),
    # T above the decode range: act-quant, then the tiled MFMA kernel
    "fallback_t300_gemm": (300, "bf16", [(512, 700), (1024, 300)]),
    # one token, K = 16384: 8 waves of 8 chunks each in the fused kernel
    "t1_bf16_eight_chunks_per_wave": (1, "bf16", [(16384, 300)]),
    # many row blocks: fused at one token (8.4M staged elements, under 16M)
    "t1_bf16_many_blocks": (1, "bf16", [(8192, 8200), (8192, 8200)]),
    # one problem over many tiles: the persistent kernel quantises once per
    # block (bf16 and f32, ragged rows, 2, 4 and 7 chunks per wave; 2 or 3
    # tiles per block, 3 to 5, 3 or 4)
    "t1_bf16_persistent": (1, "bf16", [(8192, 8200)]),
    "t1_f32_persistent_ragged": (1, "f32", [(2304, 9000)]),
    "t1_bf16_persistent_k28672": (1, "bf16", [(28672, 8192)]),
    "t1_bf16_persistent_k16384": (1, "bf16", [(16384, 9000)]),
    "t1_f32_persistent_many_tiles": (1, "f32", [(1024, 30000)]),
    "t1_bf16_persistent_k12288": (1, "bf16", [(12288, 20480)]),
    # one token, K = 28672: fused, the raw row held in registers (14 waves of 8 chunks)
    "t1_k28672_fused": (1, "bf16", [(28672, 100)]),
    # one token whose int8 row does not fit the LDS limit: act-quant runs separately
    "t1_k33024_unfused": (1, "bf16", [(33024, 100)]),
    # two tokens over the two-token work limit (4M): act-quant runs separately
    "t2_bf16_many_blocks": (2, "bf16", [(8192, 8200)]),
    # several tokens, at least 256 row tiles of short rows: two tiles per
    # block in the fused kernel (ragged last block, a cut narrow problem)
    "t3_bf16_two_tiles_ragged": (3, "bf16", [(2560, 4100), (2560, 37)]),
    "t4_f32_two_tiles": (4, "f32", [(1024, 4096)]),
    # one token, rows not a multiple of 256 k: the fused kernel on a short
    # last chunk (the 3B-class layer shapes; mixed K in one launch)
    "t1_bf16_3b_qkv": (1, "bf16", [(3200, 3200), (3200, 3200), (3200, 3200)]),
    "t1_bf16_3b_gateup": (1, "bf16", [(3200, 8640), (3200, 8640)]),
    "t1_f32_3b_down": (1, "f32", [(8640, 3200)]),
    "t1_bf16_short_chunks_mixed": (1, "bf16", [(320, 100), (2560, 37), (64, 20), (448, 300)]),
    # two to four tokens, rows not a multiple of 256 k: the staged raw rows
    # quantised with zeros past K (two row tiles per block in the second)
    "t3_bf16_3b_qkv": (3, "bf16", [(3200, 3200), (3200, 3200), (3200, 3200)]),
    "t4_f32_short_chunks_many_tiles": (4, "f32", [(576, 4100), (320, 37)]),
    "t2_bf16_3b_down": (2, "bf16", [(8640, 3200)]),
}


@pytest.mark.parametrize("name", sorted(GROUPS))
def test_linear_grouped(bl, name):
    t, dtype, shapes = GROUPS[name]
    xs, ws, refs = [], [], []
    for i, (k, n) in enumerate(shapes):
        w = wl.latent_weights(n, k, 0.02, 500 + 7 * i + k)
        x = wl.activations_student_t(t, k, 4, 600 + 7 * i + k)
        if t > 2:
            x[1] = 0.0                                  # an all-zero token
        packed, gamma, _, gamma_ref = check_pack(bl, w)
        tern = oracle.ternarize(w, gamma_ref)
        if dtype == "bf16":
            bits = wl.bf16_bits(x)
            xs.append(dev_bf16(bits))
            q_ref, a_ref, _ = oracle.quant_act(bits)
        else:
            xs.append(dev(x))
            q_ref, a_ref, _ = oracle.quant_act(x)
        ws.append((packed, gamma))
        refs.append((tern, q_ref, a_ref, gamma_ref))
    outs = bl.linear_grouped(xs, ws, want_acc=True)
    for (y, xq, absmax, acc), (tern, q_ref, a_ref, gamma_ref) in zip(outs, refs):
        assert np.array_equal(host(xq), q_ref)
        assert np.array_equal(host(absmax).view(np.uint32), a_ref.view(np.uint32))
        acc_ref = oracle.contract(q_ref, tern)
        a = host(acc)
        assert int(np.count_nonzero(a != acc_ref)) == 0
        check_y(host(y), acc_ref, gamma_ref, a_ref)


# ------------------------------------------------------------------ gated ReLU^2 into bfloat16

def test_interleave_rows(bl):
    rng = np.random.default_rng(991)
    for n, k in [(1, 16), (5, 48), (300, 2560)]:
        a = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
        b = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
        want = np.empty((2 * n, k // 4), np.uint8)
        want[0::2] = a
        want[1::2] = b
        assert np.array_equal(host(bl.interleave_rows(dev(a), dev(b))), want)


# (T, N outputs, K, dtype): fused decode (T <= 4, K % 256 == 0), the int8
# decode kernel (T <= 16), the 64-token decode kernel (K % 256 != 0, or
# 16 < T <= 128), T above 128 with K % 128 != 0, the tiled MFMA kernel
# (every tile shape), and a decode shape over the fused-work limit
GATED_CASES = [(1, 6912, 2560, "bf16"), (3, 100, 512, "f32"), (4, 37, 256, "bf16"),
               (9, 300, 1024, "bf16"), (16, 50, 2048, "f32"), (40, 77, 1008, "bf16"),
               (70, 64, 320, "f32"), (130, 300, 1040, "bf16"), (300, 500, 2560, "bf16"),
               (1024, 6144, 512, "bf16"), (2, 8200, 8192, "bf16"), (1, 28672, 8192, "bf16"),
               # gated MFMA kernel on 64 x 256 and 128 x 256 tiles
               (1100, 1900, 512, "bf16"), (256, 14336, 1024, "bf16"),
               # two row tiles per block with several tokens: the int8 decode
               # kernel (T = 8, 864 tiles), the fused one (T = 3, 2 * 2100
               # rows), the 64-token kernel (T = 32)
               (8, 6912, 2560, "bf16"), (3, 2100, 1024, "f32"), (32, 2100, 512, "bf16"),
               # rows not a multiple of 256 k: fused at one token, and int8
               # after a separate act-quant at five
               (1, 8640, 3200, "bf16"), (1, 100, 448, "f32"), (5, 300, 320, "bf16"),
               (3, 200, 576, "bf16")]


def _gated_inputs(bl, t, n, k, dtype, seed):
    wg = wl.latent_weights(n, k, 0.02, seed)
    wu = wl.latent_weights(n, k, 0.03, seed + 1)
    pg, gg, _, gg_ref = check_pack(bl, wg)
    pu, gu, _, gu_ref = check_pack(bl, wu)
    tg = oracle.ternarize(wg, gg_ref)
    tu = oracle.ternarize(wu, gu_ref)
    x = wl.activations_student_t(t, k, 4, seed + 2)
    if t > 2:
        x[1] = 0.0                                  # an all-zero token
    if dtype == "bf16":
        bits = wl.bf16_bits(x)
        xin, xref = dev_bf16(bits), bits
    else:
        xin, xref = dev(x), x
    return bl.interleave_rows(pg, pu), gg, gu, xin, xref, tg, tu, gg_ref, gu_ref


def _check_gated(h, xq, absmax, acc, xref, tg, tu, gg_ref, gu_ref, rows=None):
    q_ref, a_ref, _ = oracle.quant_act(xref)
    if rows is not None:
        q_ref, a_ref = q_ref[rows], a_ref[rows]
        h, xq, absmax, acc = h[rows], xq[rows], absmax[rows], acc[rows]
    assert np.array_equal(xq, q_ref)
    assert np.array_equal(absmax.view(np.uint32), a_ref.view(np.uint32))
    ag = oracle.contract(q_ref, tg)
    au = oracle.contract(q_ref, tu)
    assert np.array_equal(acc[:, 0::2], ag) and np.array_equal(acc[:, 1::2], au)
    h_ref = oracle.gated_relu2(ag, au, gg_ref, gu_ref, a_ref)
    bad = int(np.count_nonzero(h != h_ref))
    assert bad == 0, f"{bad} of {h.size} bfloat16 outputs differ"


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("t,n,k,dtype", GATED_CASES,
                         ids=[f"T{t}_N{n}_K{k}_{d}" for t, n, k, d in GATED_CASES])
def test_gated_relu2(bl, t, n, k, dtype):
    pgu, gg, gu, xin, xref, tg, tu, gg_ref, gu_ref = _gated_inputs(bl, t, n, k, dtype, 7000 + t + k)
    h, xq, absmax, acc = bl.gated_relu2(xin, pgu, gg, gu, want_acc=True)
    _check_gated(_bits(h), host(xq), host(absmax), host(acc), xref, tg, tu, gg_ref, gu_ref)
    # without the optional sums: the same bits
    h2, _, _, _ = bl.gated_relu2(xin, pgu, gg, gu)
    assert np.array_equal(_bits(h2), _bits(h))


def test_gated_relu2_prefill_full_size(bl):
    """The 2B gate/up projections at T = 2048 (128 x 512 tiles), every token
    (the zero token among them) checked."""
    t, n, k = 2048, 6912, 2560
    pgu, gg, gu, xin, xref, tg, tu, gg_ref, gu_ref = _gated_inputs(bl, t, n, k, "bf16", 7100)
    h, xq, absmax, acc = bl.gated_relu2(xin, pgu, gg, gu, want_acc=True)
    _check_gated(_bits(h), host(xq), host(absmax), host(acc), xref, tg, tu, gg_ref, gu_ref)


def test_gated_relu2_then_down(bl):
    """The FFN of one decode step: gate/up with the gated epilogue, then the
    down projection on the bfloat16 h with act-quant fused (grouped call)."""
    t, n, k = 1, 6912, 2560
    pgu, gg, gu, xin, xref, tg, tu, gg_ref, gu_ref = _gated_inputs(bl, t, n, k, "bf16", 7200)
    h, _, _, _ = bl.gated_relu2(xin, pgu, gg, gu)
    wd = wl.latent_weights(k, n, 0.02, 7203)
    pd, gd, _, gd_ref = check_pack(bl, wd)
    (y, xq, absmax, acc), = bl.linear_grouped([h], [(pd, gd)], want_acc=True)
    q_ref, a_ref, _ = oracle.quant_act(xref)
    h_ref = oracle.gated_relu2(oracle.contract(q_ref, tg), oracle.contract(q_ref, tu),
                               gg_ref, gu_ref, a_ref)
    qd, ad, _ = oracle.quant_act(h_ref)
    assert np.array_equal(host(xq), qd)
    acc_ref = oracle.contract(qd, oracle.ternarize(wd, gd_ref))
    assert np.array_equal(host(acc), acc_ref)
    check_y(host(y), acc_ref, gd_ref, ad)


# ------------------------------------------------------------------ binary weights (W1A8)

BIN_PACK_SHAPES = [(1, 256), (17, 512), (300, 2560), (2560, 6912), (64, 32768)]


@pytest.mark.parametrize("n,k", BIN_PACK_SHAPES, ids=[f"N{n}_K{k}" for n, k in BIN_PACK_SHAPES])
def test_pack_binary(bl, n, k):
    w = wl.latent_weights(n, k, 0.02, 3000 + n + k)
    w[0, :8] = [0.0, -0.0, 1e-45, -1e-45, 0.0, -0.0, 3.0, -3.0]
    packed_ref, gamma_ref = oracle.pack_weights_binary(w)
    packed, gamma = bl.pack_weights_binary(dev(w))
    assert host(gamma).view(np.uint32)[0] == np.float32(gamma_ref).view(np.uint32)
    p = host(packed)
    bad = int(np.count_nonzero(p != packed_ref))
    assert bad == 0, f"{bad} of {p.size} packed bytes differ"


# (T, N, K, algo): the decode kernel (whole and half 512-k chunks, one chunk
# per wave, eight chunks per wave, K = 32768 at one token per launch, forced
# for T > 16 in token groups) and the tiled MFMA kernel (both tile widths,
# ragged T and N)
BIN_FWD = [(1, 2560, 2560, "auto"), (1, 6912, 2560, "auto"), (1, 2560, 6912, "auto"),
           (4, 37, 768, "auto"), (16, 50, 2048, "auto"), (3, 100, 256, "auto"),
           (1, 8192, 28672, "auto"), (1, 64, 32768, "auto"), (2, 300, 28672, "gemv"),
           (40, 77, 1024, "gemv"), (40, 77, 1024, "auto"), (300, 500, 2560, "auto"),
           (1100, 3800, 512, "auto"), (17, 1000, 6912, "gemm"), (5, 33, 256, "gemm"),
           # one-bit MFMA kernel on 128 x 256 and 128 x 512 tiles
           (256, 28672, 1024, "gemm"), (2048, 6912, 256, "gemm")]


@pytest.mark.parametrize("t,n,k,algo", BIN_FWD, ids=[f"T{t}_N{n}_K{k}_{a}" for t, n, k, a in BIN_FWD])
def test_forward_binary(bl, t, n, k, algo):
    w = wl.latent_weights(n, k, 0.02, 3100 + t + n + k)
    x = wl.activations_student_t(t, k, 4, 3200 + t + k)
    if t > 2:
        x[1] = 0.0                                       # an all-zero token
    packed, gamma = bl.pack_weights_binary(dev(w))
    q_ref, a_ref, _ = oracle.quant_act(x)
    y, acc = bl.forward_binary(packed, gamma, dev(q_ref), dev(a_ref), algo=algo, want_acc=True)
    _, gamma_ref = oracle.pack_weights_binary(w)
    acc_ref = oracle.contract(q_ref, oracle.binarize(w))
    a = host(acc)
    bad = int(np.count_nonzero(a != acc_ref))
    assert bad == 0, f"{bad} of {a.size} int32 sums differ"
    check_y(host(y), acc_ref, gamma_ref, a_ref)


def test_forward_binary_extremes(bl):
    """All q = +-127 against all-+1 / all--1 / alternating rows, and an all-zero
    matrix (every weight +1, gamma = 0): the largest sums and exact zeros."""
    t, n, k = 3, 48, 4096
    w = np.ones((n, k), np.float32)
    w[1::2] = -1.0
    w[5, ::2] = -1.0
    q = np.full((t, k), 127, np.int8)
    q[1] = -127
    q[2, ::2] = -127
    absmax = np.array([5.0, 0.25, 1e-7], np.float32)
    packed, gamma = bl.pack_weights_binary(dev(w))
    for algo in ("gemv", "gemm"):
        y, acc = bl.forward_binary(packed, gamma, dev(q), dev(absmax), algo=algo, want_acc=True)
        acc_ref = oracle.contract(q, oracle.binarize(w))
        a = host(acc)
        assert np.array_equal(a, acc_ref) and a[0, 0] == 127 * k
        check_y(host(y), acc_ref, oracle.pack_weights_binary(w)[1], absmax)
    wz = np.zeros((n, k), np.float32)
    packed, gamma = bl.pack_weights_binary(dev(wz))
    assert np.all(host(packed) == 0xFF) and host(gamma)[0] == 0.0
    y = host(bl.forward_binary(packed, gamma, dev(q), dev(absmax)))
    assert np.all(y == 0.0)           # -0 where the sum is negative, as acc * +0 gives


# ------------------------------------------------------------------ HIP graph capture

def test_graph_replays_match_eager(bl):
    """The entry points a decode or prefill loop would capture, replayed from
    a HIP graph several times with unrelated eager work in between: every
    replay equals the eager result bit for bit (no memset nodes are recorded;
    the K-split path clears with a kernel)."""
    k, n = 2560, 640
    ws = []
    for i in range(3):
        w = wl.latent_weights(n, k, 0.02, 8000 + i)
        ws.append(bl.pack_weights(dev(w)))
    x1 = dev_bf16(wl.bf16_bits(wl.activations_normal(1, k, 8010)))
    pg, gg = ws[0]
    pu, gu = ws[1]
    pgu = bl.interleave_rows(pg, pu)
    wbig = wl.latent_weights(1500, 28672, 0.02, 8011)
    pbig, gbig = bl.pack_weights(dev(wbig))
    xq_big, am_big, _ = bl.quant_act(dev(wl.activations_normal(200, 28672, 8012)))
    pb, gb = bl.pack_weights_binary(dev(wl.latent_weights(n, k, 0.02, 8013)))
    xq1, am1, _ = bl.quant_act(x1)

    def calls():
        outs = [o[0] for o in bl.linear_grouped([x1, x1, x1], ws)]
        outs.append(bl.gated_relu2(x1, pgu, gg, gu)[0])
        outs.append(bl.forward(pbig, gbig, xq_big, am_big, 1500, algo="gemm"))  # K split
        outs.append(bl.forward_binary(pb, gb, xq1, am1))
        return outs

    eager = [host(o).copy() for o in [t.view(torch.int16) if t.dtype == torch.bfloat16 else t
                                      for t in calls()]]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        calls()                                          # warm up on the capture stream
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        static = calls()
    for rep in range(4):
        for t in static:
            t.fill_(7)                                   # stale values must be overwritten
        junk = torch.randn(4096, device="cuda").sum()    # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = [host(t.view(torch.int16) if t.dtype == torch.bfloat16 else t) for t in static]
        for i, (a, b) in enumerate(zip(got, eager)):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {rep}, output {i}"
        del junk


# ------------------------------------------------------------------ seeded random sweep
#
# Shapes drawn from a fixed seed (the ids name each one): every entry point,
# every kernel choice, on sizes no hand-picked list above holds.  The same
# element-by-element bar as the cases above.

def _draw(seed, count, fn):
    rng = np.random.default_rng(seed)
    return [fn(rng) for _ in range(count)]


_T_CHOICES = [1, 1, 1, 2, 3, 4, 5, 8, 13, 16, 17, 31, 64, 65, 100, 257]

SWEEP_FWD = _draw(9101, 20, lambda r: (int(r.choice(_T_CHOICES)), int(r.integers(1, 1200)),
                                       16 * int(r.integers(1, 385))))


@pytest.mark.parametrize("t,n,k", SWEEP_FWD, ids=[f"T{t}_N{n}_K{k}" for t, n, k in SWEEP_FWD])
def test_sweep_forward(bl, t, n, k):
    tern, q, absmax, gamma = _forward_inputs(t, n, k, 9200 + t + n + k)
    args = (dev(oracle.pack_ternary(tern)), dev(np.array([gamma])), dev(q), dev(absmax))
    for algo in ("auto", "gemv", "gemm", "lut", "dot4"):
        check_forward(bl, *args, tern, q, gamma, absmax, algo)


def _group(r):
    t = int(r.choice([1, 1, 2, 3, 4, 5, 9, 70]))
    count = int(r.integers(1, 9))
    dtype = "bf16" if r.random() < 0.7 else "f32"
    shapes = []
    for _ in range(count):
        k = 256 * int(r.integers(1, 25)) if r.random() < 0.8 else 16 * int(r.integers(1, 200))
        shapes.append((k, int(r.integers(1, 900))))
    return t, dtype, shapes


SWEEP_GROUPS = _draw(9102, 10, _group)


@pytest.mark.parametrize("t,dtype,shapes", SWEEP_GROUPS,
                         ids=[f"T{t}_{d}_" + "_".join(f"{k}x{n}" for k, n in s)
                              for t, d, s in SWEEP_GROUPS])
def test_sweep_grouped(bl, t, dtype, shapes):
    xs, ws, refs = [], [], []
    for i, (k, n) in enumerate(shapes):
        tern, _, _, gamma = _forward_inputs(1, n, k, 9300 + 7 * i + k + n, zero_rows=True)
        x = wl.activations_student_t(t, k, 4, 9400 + 7 * i + k)
        if t > 2:
            x[t - 1] = 0.0                                   # an all-zero token
        if dtype == "bf16":
            bits = wl.bf16_bits(x)
            xs.append(dev_bf16(bits))
            q_ref, a_ref, _ = oracle.quant_act(bits)
        else:
            xs.append(dev(x))
            q_ref, a_ref, _ = oracle.quant_act(x)
        ws.append((dev(oracle.pack_ternary(tern)), dev(np.array([gamma]))))
        refs.append((tern, q_ref, a_ref, gamma))
    outs = bl.linear_grouped(xs, ws, want_acc=True)
    for (y, xq, absmax, acc), (tern, q_ref, a_ref, gamma) in zip(outs, refs):
        assert np.array_equal(host(xq), q_ref)
        assert np.array_equal(host(absmax).view(np.uint32), a_ref.view(np.uint32))
        acc_ref = oracle.contract(q_ref, tern)
        assert int(np.count_nonzero(host(acc) != acc_ref)) == 0
        check_y(host(y), acc_ref, gamma, a_ref)


SWEEP_GATED = _draw(9103, 8, lambda r: (int(r.choice([1, 1, 2, 3, 4, 7, 16, 33, 150])),
                                        int(r.integers(1, 700)),
                                        (256 if r.random() < 0.7 else 16) * int(r.integers(1, 17)),
                                        "bf16" if r.random() < 0.6 else "f32"))


@pytest.mark.parametrize("t,n,k,dtype", SWEEP_GATED,
                         ids=[f"T{t}_N{n}_K{k}_{d}" for t, n, k, d in SWEEP_GATED])
def test_sweep_gated(bl, t, n, k, dtype):
    pgu, gg, gu, xin, xref, tg, tu, gg_ref, gu_ref = _gated_inputs(bl, t, n, k, dtype, 9500 + t + n + k)
    h, xq, absmax, acc = bl.gated_relu2(xin, pgu, gg, gu, want_acc=True)
    _check_gated(_bits(h), host(xq), host(absmax), host(acc), xref, tg, tu, gg_ref, gu_ref)


SWEEP_BIN = _draw(9104, 8, lambda r: (int(r.choice(_T_CHOICES)), int(r.integers(1, 1200)),
                                      256 * int(r.integers(1, 33)),
                                      str(r.choice(["auto", "gemv", "gemm"]))))


@pytest.mark.parametrize("t,n,k,algo", SWEEP_BIN, ids=[f"T{t}_N{n}_K{k}_{a}" for t, n, k, a in SWEEP_BIN])
def test_sweep_binary(bl, t, n, k, algo):
    w = wl.latent_weights(n, k, 0.02, 9600 + t + n + k)
    x = wl.activations_student_t(t, k, 4, 9700 + t + k)
    packed_ref, gamma_ref = oracle.pack_weights_binary(w)
    packed, gamma = bl.pack_weights_binary(dev(w))
    assert np.array_equal(host(packed), packed_ref)
    assert host(gamma).view(np.uint32)[0] == np.float32(gamma_ref).view(np.uint32)
    q_ref, a_ref, _ = oracle.quant_act(x)
    y, acc = bl.forward_binary(packed, gamma, dev(q_ref), dev(a_ref), algo=algo, want_acc=True)
    acc_ref = oracle.contract(q_ref, oracle.binarize(w))
    assert int(np.count_nonzero(host(acc) != acc_ref)) == 0
    check_y(host(y), acc_ref, gamma_ref, a_ref)


SWEEP_SUBLN = _draw(9105, 6, lambda r: (int(r.choice([1, 2, 5, 64, 300])), 16 * int(r.integers(1, 1025)),
                                        "bf16" if r.random() < 0.6 else "f32"))


@pytest.mark.parametrize("t,k,dtype", SWEEP_SUBLN, ids=[f"T{t}_K{k}_{d}" for t, k, d in SWEEP_SUBLN])
def test_sweep_subln(bl, t, k, dtype):
    xref, xin, g = _subln_inputs(t, k, dtype, 9800 + t + k)
    check_subln(bl, xref, xin, g)
