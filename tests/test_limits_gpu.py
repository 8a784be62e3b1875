"""Kernels at the largest sizes the C ABI accepts (needs a HIP device).

N = 2^26 output rows at one token (the decode kernels) and T = 2^24 tokens
(act-quant and the tiled kernel, T * K up to 2^32): offsets there no longer
fit 32 bits.  Every output is checked.  Sampled rows / tokens hold random
values and are compared with the oracle; all the others hold constant rows
whose results have a closed form:
  - a weight row of one ternary value v gives sum_k v * q_k = v * sum(q);
  - a token row of one int8 value c gives sum_k t_k * c = c * sum(t);
  - a raw activation row of one value x quantises to sign(x) * 127 with
    absmax |x| (x * RN(127 / |x|) lies within an ulp of +-127).
"""

import numpy as np
import pytest
import torch

import oracle
from bitlinear_w1_a8_amd import workloads as wl

pytestmark = pytest.mark.gpu

N_MAX = 1 << 26
T_MAX = 1 << 24
SAMPLES = 1024


@pytest.fixture(scope="module")
def bl(built_lib):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from bitlinear_w1_a8_amd import binding
    binding.load()
    return binding


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def sample_idx(rng, n):
    idx = rng.choice(n, size=SAMPLES - 2, replace=False)
    return np.unique(np.concatenate([idx, [0, n - 1]])).astype(np.int64)


def check_y(y, acc_ref, gamma, absmax):
    """y against the oracle's binary64 rescale of the exact sums (1e-5 relative; +0 where acc = 0)."""
    y_ref = oracle.rescale(acc_ref, gamma, absmax)
    zero = acc_ref == 0
    assert np.all(y[zero] == 0.0) and not np.any(np.signbit(y[zero]))
    nz = ~zero
    if np.any(nz):
        rel = np.abs(y[nz].astype(np.float64) - y_ref[nz]) / np.abs(y_ref[nz])
        assert float(rel.max()) <= 1e-5, f"max relative error {rel.max():.3g}"


@pytest.mark.parametrize("k", [16, 256])
def test_max_rows_one_token(bl, k):
    """N = 2^26 rows, T = 1: rows of a constant code (row % 3 -> t = -1, 0, +1)
    and sampled random ternary rows."""
    rng = np.random.default_rng(4100 + k)
    n = N_MAX
    idx = sample_idx(rng, n)
    t_s = rng.integers(-1, 2, size=(idx.size, k)).astype(np.int8)
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    # a row of code c everywhere: every 2-bit field of every byte is c
    const_byte = torch.tensor([0x00, 0x55, 0xAA], dtype=torch.uint8, device="cuda")
    rows = torch.arange(n, device="cuda", dtype=torch.int64)
    packed[:] = const_byte[rows % 3][:, None]
    del rows
    packed[torch.from_numpy(idx).cuda()] = torch.from_numpy(oracle.pack_ternary(t_s)).cuda()
    gamma_ref = np.float32(0.0123)
    gamma = torch.tensor([gamma_ref], device="cuda")
    q = rng.integers(-127, 128, size=(1, k)).astype(np.int8)
    q[0, 0] = 127
    a_ref = np.array([1.75], np.float32)
    xq, absmax = torch.from_numpy(q).cuda(), torch.from_numpy(a_ref).cuda()
    print(f"max rows: N={n} K={k}", flush=True)
    y, acc = bl.forward(packed, gamma, xq, absmax, n, want_acc=True)
    a = host(acc)[0]
    yh = host(y)[0]
    del packed, y, acc
    torch.cuda.empty_cache()
    # every row of a constant code: (c - 1) * sum(q)
    sq = int(q.astype(np.int64).sum())
    want = ((np.arange(n, dtype=np.int64) % 3) - 1) * sq
    want[idx] = oracle.contract(q, t_s)[0]
    bad = np.flatnonzero(a != want)
    assert bad.size == 0, f"{bad.size} int32 sums differ, first rows {bad[:4]}"
    check_y(yh[idx][None, :], want[idx][None, :].astype(np.int32), gamma_ref, a_ref)
    # the constant rows' outputs: three values, each from the oracle
    for c in range(3):
        acc_c = np.array([[(c - 1) * sq]], np.int32)
        y_c = yh[c::3]
        keep = np.ones(y_c.size, bool)
        keep[(idx[idx % 3 == c] - c) // 3] = False
        vals = np.unique(y_c[keep])
        assert vals.size == 1, vals[:4]
        check_y(vals[None, :1], acc_c, gamma_ref, a_ref)


def _max_tokens_inputs(rng, t, k):
    """xq[T, K]: token r holds the constant c_r = (r % 255) - 127, sampled
    tokens random int8; absmax from a seeded table."""
    idx = sample_idx(rng, t)
    q_s = rng.integers(-127, 128, size=(idx.size, k)).astype(np.int8)
    r = torch.arange(t, device="cuda", dtype=torch.int64)
    c = ((r % 255) - 127).to(torch.int8)
    xq = c[:, None].expand(t, k).contiguous()
    xq[torch.from_numpy(idx).cuda()] = torch.from_numpy(q_s).cuda()
    a_tab = (0.5 + rng.random(97)).astype(np.float32)
    absmax = torch.from_numpy(a_tab).cuda()[r % 97].contiguous()
    del r, c
    return idx, q_s, xq, absmax, a_tab


@pytest.mark.parametrize("k", [16, 256])
def test_max_tokens_tiled(bl, k):
    """T = 2^24 tokens (T * K = 2^32 at K = 256) through the automatic choice
    (the tiled kernel), N = 16 random ternary rows."""
    rng = np.random.default_rng(4200 + k)
    t, n = T_MAX, 16
    t_ref = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    packed = torch.from_numpy(oracle.pack_ternary(t_ref)).cuda()
    gamma_ref = np.float32(0.0371)
    gamma = torch.tensor([gamma_ref], device="cuda")
    idx, q_s, xq, absmax, a_tab = _max_tokens_inputs(rng, t, k)
    print(f"max tokens: T={t} K={k} N={n}", flush=True)
    y, acc = bl.forward(packed, gamma, xq, absmax, n, want_acc=True)
    a = host(acc)
    yh = host(y)
    del xq, y, acc
    torch.cuda.empty_cache()
    # every token of a constant c: c * (row sums of t)
    tsum = t_ref.astype(np.int64).sum(axis=1)
    cvec = (np.arange(t, dtype=np.int64) % 255) - 127
    want = cvec[:, None] * tsum[None, :]
    want[idx] = oracle.contract(q_s, t_ref)
    bad = int(np.count_nonzero(a != want))
    assert bad == 0, f"{bad} int32 sums differ"
    absmax_all = a_tab[np.arange(t) % 97]
    check_y(yh[idx], want[idx].astype(np.int32), gamma_ref, absmax_all[idx])
    # the constant tokens: 255 x 97 distinct (c, absmax) pairs, one from each
    first = np.arange(255 * 97)
    first = first[~np.isin(first, idx)]
    check_y(yh[first], want[first].astype(np.int32), gamma_ref, absmax_all[first])
    # and every other token repeats the output of its (c, absmax) pair
    key = (np.arange(t) % (255 * 97))
    rep = yh[key]
    keep = np.ones(t, bool)
    keep[idx] = False
    keep[np.isin(key, idx)] = False         # their representative is a sampled token
    assert np.array_equal(yh[keep].view(np.uint32), rep[keep].view(np.uint32))


@pytest.mark.parametrize("k", [16, 256])
def test_max_tokens_act_quant(bl, k):
    """Step A1 over T = 2^24 bf16 rows: row r a constant x_r, sampled rows random."""
    rng = np.random.default_rng(4300 + k)
    t = T_MAX
    idx = sample_idx(rng, t)
    bits_s = wl.bf16_bits(rng.standard_normal((idx.size, k)).astype(np.float32))
    vals = np.array([-3.5, -0.25, 0.0078125, 1.0, 0.0029296875, -15360.0, 6.0], np.float32)
    vbits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((vbits.astype(np.uint32) << 16).view(np.float32), vals)   # exact in bf16
    r = torch.arange(t, device="cuda", dtype=torch.int64)
    row_bits = torch.from_numpy(vbits.view(np.int16)).cuda()[r % vals.size]
    x = row_bits[:, None].expand(t, k).contiguous()
    x[torch.from_numpy(idx).cuda()] = torch.from_numpy(bits_s.view(np.int16)).cuda()
    del r, row_bits
    print(f"max tokens act-quant: T={t} K={k}", flush=True)
    xq, absmax, rowsum = bl.quant_act(x.view(torch.bfloat16))
    del x
    torch.cuda.empty_cache()
    q_ref, a_ref, rs_ref = oracle.quant_act(bits_s)
    assert np.array_equal(host(xq[torch.from_numpy(idx).cuda()]), q_ref)
    am = host(absmax)
    rs = host(rowsum)
    assert np.array_equal(am[idx].view(np.uint32), a_ref.view(np.uint32))
    assert np.array_equal(rs[idx], rs_ref)
    # constant rows: codes sign(x) * 127, absmax |x|, row sum +-127 * K
    keep = torch.ones(t, dtype=torch.bool, device="cuda")
    keep[torch.from_numpy(idx).cuda()] = False
    sel = torch.arange(t, device="cuda")[keep]
    v = torch.from_numpy(np.sign(vals).astype(np.int8) * np.int8(127)).cuda()[sel % vals.size]
    assert bool(torch.all(xq[sel] == v[:, None]).item())
    want_a = np.abs(vals)[np.arange(t) % vals.size]
    keep_h = np.ones(t, bool)
    keep_h[idx] = False
    assert np.array_equal(am[keep_h].view(np.uint32), want_a[keep_h].view(np.uint32))
    want_rs = (np.sign(vals).astype(np.int64) * 127 * k)[np.arange(t) % vals.size]
    assert np.array_equal(rs[keep_h], want_rs[keep_h])


@pytest.mark.parametrize("n", [1 << 19, (1 << 19) + 16, N_MAX],
                         ids=["persistent_64_tiles_per_block", "one_tile_past", "N_max"])
def test_max_rows_fused_bf16(bl, n):
    """One bf16 token with step A1 fused (the grouped call): the persistent
    kernel up to 64 tiles per block (2^19 rows on 256 CUs), the per-tile
    kernel past that, up to N = 2^26; rows of constant codes and sampled
    random rows as above."""
    rng = np.random.default_rng(4400 + n % 997)
    k = 256
    idx = sample_idx(rng, n)
    t_s = rng.integers(-1, 2, size=(idx.size, k)).astype(np.int8)
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    const_byte = torch.tensor([0x00, 0x55, 0xAA], dtype=torch.uint8, device="cuda")
    rows = torch.arange(n, device="cuda", dtype=torch.int64)
    packed[:] = const_byte[rows % 3][:, None]
    del rows
    packed[torch.from_numpy(idx).cuda()] = torch.from_numpy(oracle.pack_ternary(t_s)).cuda()
    gamma_ref = np.float32(0.0123)
    gamma = torch.tensor([gamma_ref], device="cuda")
    bits = wl.bf16_bits(rng.standard_normal((1, k)).astype(np.float32))
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    print(f"fused bf16 one token: N={n} K={k}", flush=True)
    (y, xq, absmax, acc), = bl.linear_grouped([x], [(packed, gamma)], want_acc=True)
    q_ref, a_ref, _ = oracle.quant_act(bits)
    assert np.array_equal(host(xq), q_ref)
    assert np.array_equal(host(absmax).view(np.uint32), a_ref.view(np.uint32))
    a = host(acc)[0]
    yh = host(y)[0]
    del packed, y, acc
    torch.cuda.empty_cache()
    sq = int(q_ref.astype(np.int64).sum())
    want = ((np.arange(n, dtype=np.int64) % 3) - 1) * sq
    want[idx] = oracle.contract(q_ref, t_s)[0]
    bad = np.flatnonzero(a != want)
    assert bad.size == 0, f"{bad.size} int32 sums differ, first rows {bad[:4]}"
    check_y(yh[None, :], want[None, :].astype(np.int32), gamma_ref, a_ref)


def test_max_rows_binary(bl):
    """Binary weights, N = 2^26 rows at one token (K = 256): rows of all -1
    (byte 0x00) and all +1 (0xFF) alternate, sampled random rows."""
    from oracle import binary_ref
    rng = np.random.default_rng(4500)
    n, k = N_MAX, 256
    idx = sample_idx(rng, n)
    t_s = np.where(rng.random((idx.size, k)) < 0.5, -1, 1).astype(np.int8)
    packed = torch.empty((n, k // 8), dtype=torch.uint8, device="cuda")
    const_byte = torch.tensor([0x00, 0xFF], dtype=torch.uint8, device="cuda")
    rows = torch.arange(n, device="cuda", dtype=torch.int64)
    packed[:] = const_byte[rows % 2][:, None]
    del rows
    packed[torch.from_numpy(idx).cuda()] = torch.from_numpy(binary_ref.pack_binary(t_s)).cuda()
    gamma_ref = np.float32(0.0217)
    gamma = torch.tensor([gamma_ref], device="cuda")
    q = rng.integers(-127, 128, size=(1, k)).astype(np.int8)
    a_ref = np.array([2.5], np.float32)
    print(f"max rows binary: N={n} K={k}", flush=True)
    y, acc = bl.forward_binary(packed, gamma, torch.from_numpy(q).cuda(),
                               torch.from_numpy(a_ref).cuda(), want_acc=True)
    a = host(acc)[0]
    yh = host(y)[0]
    del packed, y, acc
    torch.cuda.empty_cache()
    sq = int(q.astype(np.int64).sum())
    want = (2 * (np.arange(n, dtype=np.int64) % 2) - 1) * sq
    want[idx] = oracle.contract(q, t_s)[0]
    bad = np.flatnonzero(a != want)
    assert bad.size == 0, f"{bad.size} int32 sums differ, first rows {bad[:4]}"
    check_y(yh[None, :], want[None, :].astype(np.int32), gamma_ref, a_ref)


def test_max_tokens_subln(bl):
    """SubLN + A1 over T = 2^24 bf16 rows (K = 16, gain 1): row r a constant
    x_r, whose codes are sign(x) * 127 and whose scale the oracle gives from
    one such row; sampled random rows against the oracle."""
    from oracle import subln_ref
    rng = np.random.default_rng(4600)
    t, k = T_MAX, 16
    idx = sample_idx(rng, t)
    bits_s = wl.bf16_bits(rng.standard_normal((idx.size, k)).astype(np.float32))
    vals = np.array([-3.5, -0.25, 0.0078125, 1.0, 0.0029296875, -15360.0, 6.0], np.float32)
    vbits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    gain = np.ones(k, np.float32)
    r = torch.arange(t, device="cuda", dtype=torch.int64)
    row_bits = torch.from_numpy(vbits.view(np.int16)).cuda()[r % vals.size]
    x = row_bits[:, None].expand(t, k).contiguous()
    x[torch.from_numpy(idx).cuda()] = torch.from_numpy(bits_s.view(np.int16)).cuda()
    del r, row_bits
    print(f"max tokens subln: T={t} K={k}", flush=True)
    xq, scale, rowsum = bl.subln_quant_act(x.view(torch.bfloat16), torch.from_numpy(gain).cuda())
    del x
    torch.cuda.empty_cache()
    q_ref, s_ref, rs_ref, _ = subln_ref.subln_quant_act(bits_s, gain)
    assert np.array_equal(host(xq[torch.from_numpy(idx).cuda()]), q_ref)
    sc, rs = host(scale), host(rowsum)
    assert np.array_equal(sc[idx].view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(rs[idx], rs_ref)
    const_rows = np.repeat(vbits[:, None], k, axis=1)
    qc, sc_c, rs_c, _ = subln_ref.subln_quant_act(const_rows, gain)
    keep = np.ones(t, bool)
    keep[idx] = False
    j = np.arange(t) % vals.size
    assert np.array_equal(sc[keep].view(np.uint32), sc_c[j[keep]].view(np.uint32))
    assert np.array_equal(rs[keep], rs_c[j[keep]])
    keep_d = torch.from_numpy(keep).cuda()
    sel = torch.arange(t, device="cuda")[keep_d]
    want_q = torch.from_numpy(qc).cuda()[sel % vals.size]
    assert bool(torch.all(xq[sel] == want_q).item())


def test_max_outputs_gated(bl):
    """Gated ReLU^2 with the largest output count, N = 2^25 (2^26 interleaved
    gate / up rows) at one bf16 token, K = 256: row r of a constant code
    (r % 3), so output i takes one of three (gate, up) sum pairs; sampled
    outputs with random gate and up rows; every h checked against the
    oracle's gated epilogue."""
    rng = np.random.default_rng(4700)
    n, k = N_MAX // 2, 256
    idx = sample_idx(rng, n)
    tg = rng.integers(-1, 2, size=(idx.size, k)).astype(np.int8)
    tu = rng.integers(-1, 2, size=(idx.size, k)).astype(np.int8)
    packed = torch.empty((2 * n, k // 4), dtype=torch.uint8, device="cuda")
    const_byte = torch.tensor([0x00, 0x55, 0xAA], dtype=torch.uint8, device="cuda")
    rows = torch.arange(2 * n, device="cuda", dtype=torch.int64)
    packed[:] = const_byte[rows % 3][:, None]
    del rows
    di = torch.from_numpy(idx).cuda()
    packed[2 * di] = torch.from_numpy(oracle.pack_ternary(tg)).cuda()
    packed[2 * di + 1] = torch.from_numpy(oracle.pack_ternary(tu)).cuda()
    gg_ref, gu_ref = np.float32(0.0123), np.float32(0.0311)
    bits = wl.bf16_bits(rng.standard_normal((1, k)).astype(np.float32))
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    print(f"max outputs gated: N={n} K={k}", flush=True)
    h, xq, absmax, acc = bl.gated_relu2(x, packed, torch.tensor([gg_ref], device="cuda"),
                                        torch.tensor([gu_ref], device="cuda"), want_acc=True)
    q_ref, a_ref, _ = oracle.quant_act(bits)
    assert np.array_equal(host(xq), q_ref)
    assert np.array_equal(host(absmax).view(np.uint32), a_ref.view(np.uint32))
    hb = host(h.view(torch.int16)).view(np.uint16)[0]
    a = host(acc)[0]
    del packed, h, acc
    torch.cuda.empty_cache()
    sq = int(q_ref.astype(np.int64).sum())
    want = ((np.arange(2 * n, dtype=np.int64) % 3) - 1) * sq
    want[2 * idx] = oracle.contract(q_ref, tg)[0]
    want[2 * idx + 1] = oracle.contract(q_ref, tu)[0]
    bad = np.flatnonzero(a != want)
    assert bad.size == 0, f"{bad.size} int32 sums differ, first rows {bad[:4]}"
    h_ref = oracle.gated_relu2(want[0::2][None, :].astype(np.int32),
                               want[1::2][None, :].astype(np.int32), gg_ref, gu_ref, a_ref)
    bad = np.flatnonzero(hb != np.asarray(h_ref).reshape(-1).view(np.uint16))
    assert bad.size == 0, f"{bad.size} bf16 outputs differ, first {bad[:4]}"
