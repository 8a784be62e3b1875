"""The oracle against facts that do not come from itself (CPU only).

``test_pin`` runs every pin of tests/pins.py on the oracle.  ``test_mutant``
plants one plausible mistake at a time into a copy of the oracle (a dropped
epsilon, another rounding rule, a swapped bit order, a per-row instead of a
per-matrix scale, a transposed or truncated contraction, ...) and checks that
at least one pin fails, so each pin set is shown to be able to see it.
"""

import math
import types

import numpy as np
import pytest

import oracle
from tests import pins


def _ns(**overrides):
    d = {k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("__")}
    d.update(overrides)
    return types.SimpleNamespace(**d)


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


# ------------------------------------------------------------------ mutants

def _per_row_gamma(w):
    w = np.asarray(w, np.float32)
    return np.float32(np.mean(np.abs(w), axis=1, dtype=np.float64)[0])


def _f32_sum_gamma(w):
    w = np.asarray(w, np.float32)
    s = np.float32(0)
    for v in np.abs(w).ravel():
        s = np.float32(s + v)
    return np.float32(s / np.float32(w.size))


def _f64_sequential_gamma(w):
    w = np.asarray(w, np.float32)
    s = 0.0
    for v in np.abs(w).ravel().tolist():
        s += v
    return np.float32(s / w.size)


def _tern_no_eps(w, gamma):
    u = np.asarray(w, np.float32) / np.float32(gamma)
    return np.clip(np.rint(u), -1, 1).astype(np.int8)


def _half_away(v):
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def _tern_half_away(w, gamma):
    u = np.asarray(w, np.float32) / (np.float32(gamma) + np.float32(1e-5))
    return np.clip(_half_away(u), -1, 1).astype(np.int8)


def _tern_eps_as_max(w, gamma):
    u = np.asarray(w, np.float32) / np.maximum(np.float32(gamma), np.float32(1e-5))
    return np.clip(np.rint(u), -1, 1).astype(np.int8)


def _tern_threshold_gamma(w, gamma):
    # the prose paraphrase "above the mean -> +1" instead of eq. (1)-(2)
    w = np.asarray(w, np.float32)
    return ((w > gamma).astype(np.int8) - (w < -gamma).astype(np.int8))


def _pack_swapped(t):
    n, k = t.shape
    c = (t.astype(np.int64) + 1).astype(np.uint32).reshape(n, k // 16, 4, 4)
    words = np.zeros((n, k // 16), np.uint32)
    for j in range(4):
        for i in range(4):
            words |= c[:, :, j, i] << np.uint32(2 * i + 8 * j)
    return words.astype("<u4").view(np.uint8).reshape(n, k // 4)


def _pack_twos_complement(t):
    n, k = t.shape
    c = (t.astype(np.int64) & 3).astype(np.uint32).reshape(n, k // 16, 4, 4)
    words = np.zeros((n, k // 16), np.uint32)
    for j in range(4):
        for i in range(4):
            words |= c[:, :, j, i] << np.uint32(8 * i + 2 * j)
    return words.astype("<u4").view(np.uint8).reshape(n, k // 4)


def _make_quant(rounder=np.rint, qb=127, order="scale_first", eps=True, per_token=True):
    def quant(x):
        x = np.asarray(x)
        if x.dtype == np.uint16:
            x = oracle.widen_bf16(x)
        x = np.asarray(x, np.float32)
        a = np.max(np.abs(x), axis=1) if per_token else np.full(x.shape[0], np.max(np.abs(x)), np.float32)
        m = np.maximum(a, np.float32(1e-5)) if eps else a
        if order == "scale_first":
            v = x * (np.float32(qb) / m)[:, None]
        else:
            v = (x * np.float32(qb)) / m[:, None]
        with np.errstate(invalid="ignore"):
            q = np.clip(rounder(v), -127, 127)
        if not np.all(np.isfinite(q)):
            raise FloatingPointError("non-finite q")
        q = q.astype(np.int8)
        return q, a.astype(np.float32), q.astype(np.int64).sum(axis=1).astype(np.int32)
    return quant


def _contract_neg(q, t):
    return -oracle.contract(q, t)


def _contract_drop_last(q, t):
    return oracle.contract(q[:, :-1], t[:, :-1])


def _contract_transposed_t(q, t):
    tt = np.asarray(t)
    if tt.shape[0] == tt.shape[1]:
        tt = tt.T
    return oracle.contract(q, tt)


def _contract_f32(q, t):
    acc = np.asarray(q, np.float32) @ np.asarray(t, np.float32).T
    return acc.astype(np.int32)


def _rescale_gamma_eps(acc, gamma, absmax):
    return oracle.rescale(acc, np.float32(gamma) + np.float32(1e-5), absmax)


def _rescale_128(acc, gamma, absmax):
    return oracle.rescale(acc, gamma, absmax) * (127.0 / 128.0)


def _rescale_no_floor(acc, gamma, absmax):
    m = np.asarray(absmax, np.float32).astype(np.float64)
    return np.asarray(acc, np.float64) * np.float64(gamma) * m[:, None] / 127.0


def _subln(x, gain, eps_n=oracle.EPS_N, *, use_gain=True, rms_of="x", eps=True, sum_mode="exact",
           r_mode="steps", order="gain_first", codes_of_u=False, scale_of_u=False, mean_abs=False):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = oracle.widen_bf16(x)
    x = np.asarray(x, np.float32)
    g = np.asarray(gain, np.float32)
    k = x.shape[1]
    u = x * g[None, :] if use_gain else x
    src = (u if rms_of == "u" else x).astype(np.float64)
    sq = np.abs(src) if mean_abs else src * src
    if sum_mode == "exact":
        s = np.array([math.fsum(row.tolist()) for row in sq])
    elif sum_mode == "seq":
        s = np.zeros(x.shape[0])
        for j in range(k):
            s = s + sq[:, j]
    elif sum_mode == "np":
        s = np.sum(sq, axis=1)
    else:                                    # a binary32 running sum
        s32 = np.zeros(x.shape[0], np.float32)
        for j in range(k):
            s32 = s32 + sq[:, j].astype(np.float32)
        s = s32.astype(np.float64)
    ms64 = s / k
    e = np.float32(eps_n) if eps else np.float32(0.0)
    with np.errstate(all="ignore"):
        if r_mode == "f64":
            r64 = 1.0 / (ms64 + float(e)) if mean_abs else 1.0 / np.sqrt(ms64 + float(e))
            r = r64.astype(np.float32)
        elif r_mode == "one_rounding":
            v = ms64.astype(np.float32) + e
            r = (1.0 / np.sqrt(v.astype(np.float64))).astype(np.float32)
        else:
            v = ms64.astype(np.float32) + e
            r = np.float32(1.0) / (v if mean_abs else np.sqrt(v))
    if codes_of_u:
        # quantise x * g and hand on r * max|x * g| as the scale
        q, a, rowsum = oracle.quant_act(u)
        return q, (a.astype(np.float64) * r.astype(np.float64)).astype(np.float32), rowsum, r
    if r_mode == "f64":
        xh = (u.astype(np.float64) * r64[:, None]).astype(np.float32)
    elif order == "gain_first":
        xh = u * r[:, None]
    else:
        xh = (x * r[:, None]) * g[None, :]
    q, a, rowsum = oracle.quant_act(xh)
    if scale_of_u:
        a = np.max(np.abs(u), axis=1).astype(np.float32)
    return q, a, rowsum, r


def _subln_mutant(**kw):
    return lambda x, gain, eps_n=oracle.EPS_N: _subln(x, gain, eps_n, **kw)


def _bf16_trunc(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _bf16_half_away(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint16)


def _gated(acc_gate, acc_up, gamma_gate, gamma_up, absmax, *, relu=True, square=True, relu_up=False,
           order="rr_u", scale32=False, rounder=None, swap=False):
    if swap:
        acc_gate, acc_up, gamma_gate, gamma_up = acc_up, acc_gate, gamma_up, gamma_gate
    if scale32:
        # a binary32 scale RN32(RN32(gamma * m) / 127) applied to the sum
        m = np.maximum(np.asarray(absmax, np.float32), oracle.EPS_A)
        sg = (np.float32(gamma_gate) * m) / np.float32(127)
        su = (np.float32(gamma_up) * m) / np.float32(127)
        g = np.asarray(acc_gate).astype(np.float32) * sg[:, None]
        u = np.asarray(acc_up).astype(np.float32) * su[:, None]
    else:
        g = oracle.a3_f32(acc_gate, gamma_gate, absmax)
        u = oracle.a3_f32(acc_up, gamma_up, absmax)
    r = np.maximum(g, np.float32(0)) if relu else g
    if relu_up:
        u = np.maximum(u, np.float32(0))
    if not square:
        h = r * u
    elif order == "rr_u":
        h = (r * r) * u
    else:
        h = r * (r * u)
    return (rounder or oracle.bf16_rne)(h)


def _gated_mutant(**kw):
    return lambda ag, au, gg, gu, a: _gated(ag, au, gg, gu, a, **kw)


def _binarize_zero_to_minus(w):
    w = np.asarray(w, np.float32)
    return np.where(w > 0, 1, -1).astype(np.int8)


def _binarize_centered(w):
    # the original binary BitNet's Sign(W - mean W): not what the pages give
    w = np.asarray(w, np.float32)
    c = w - np.float32(np.mean(w, dtype=np.float64))
    return np.where(c >= 0, 1, -1).astype(np.int8)


def _pack_binary_with(bitpos=lambda j, i: 8 * i + j, one_is_plus=True):
    def pack(t):
        t = np.asarray(t)
        n, k = t.shape
        if k % 32 != 0:
            raise ValueError("K")
        if not np.all((t == -1) | (t == 1)):
            raise ValueError("binary")
        bits = ((t > 0) if one_is_plus else (t < 0)).astype(np.uint32).reshape(n, k // 32, 8, 4)
        words = np.zeros((n, k // 32), np.uint32)
        for j in range(8):
            for i in range(4):
                words |= bits[:, :, j, i] << np.uint32(bitpos(j, i))
        return words.astype("<u4").view(np.uint8).reshape(n, k // 8)
    return pack


def _pack_weights_binary_with(binarize):
    return lambda w: (oracle.pack_binary(binarize(w)), oracle.absmean_gamma(w))


MUTANTS = {
    "binary_zero_to_minus": dict(binarize=_binarize_zero_to_minus),
    "binary_centered_sign": dict(binarize=_binarize_centered,
                                 pack_weights_binary=_pack_weights_binary_with(_binarize_centered)),
    "binary_bit_order_swapped": dict(pack_binary=_pack_binary_with(bitpos=lambda j, i: 4 * j + i)),
    "binary_bit_means_minus": dict(pack_binary=_pack_binary_with(one_is_plus=False)),
    "gated_no_relu": dict(gated_relu2=_gated_mutant(relu=False)),
    "gated_not_squared": dict(gated_relu2=_gated_mutant(square=False)),
    "gated_relu_on_up_too": dict(gated_relu2=_gated_mutant(relu_up=True)),
    "gated_other_product_order": dict(gated_relu2=_gated_mutant(order="r_ru")),
    "gated_binary32_scale": dict(gated_relu2=_gated_mutant(scale32=True)),
    "gated_bf16_truncate": dict(gated_relu2=_gated_mutant(rounder=_bf16_trunc)),
    "gated_bf16_half_away": dict(gated_relu2=_gated_mutant(rounder=_bf16_half_away)),
    "gated_gate_up_swapped": dict(gated_relu2=_gated_mutant(swap=True)),
    "bf16_truncate": dict(bf16_rne=_bf16_trunc),
    "bf16_half_away": dict(bf16_rne=_bf16_half_away),
    "subln_codes_of_x_times_g": dict(subln_quant_act=_subln_mutant(codes_of_u=True)),
    "subln_no_gain": dict(subln_quant_act=_subln_mutant(use_gain=False)),
    "subln_rms_of_x_times_g": dict(subln_quant_act=_subln_mutant(rms_of="u")),
    "subln_no_eps": dict(subln_quant_act=_subln_mutant(eps=False)),
    "subln_sum_running_binary64": dict(subln_quant_act=_subln_mutant(sum_mode="seq")),
    "subln_sum_numpy_pairwise": dict(subln_quant_act=_subln_mutant(sum_mode="np")),
    "subln_sum_binary32": dict(subln_quant_act=_subln_mutant(sum_mode="f32")),
    "subln_r_in_binary64": dict(subln_quant_act=_subln_mutant(r_mode="f64")),
    "subln_r_one_rounding": dict(subln_quant_act=_subln_mutant(r_mode="one_rounding")),
    "subln_norm_before_gain": dict(subln_quant_act=_subln_mutant(order="norm_first")),
    "subln_scale_is_max_x_times_g": dict(subln_quant_act=_subln_mutant(scale_of_u=True)),
    "subln_mean_abs_not_rms": dict(subln_quant_act=_subln_mutant(mean_abs=True)),
    "gamma_per_row": dict(absmean_gamma=_per_row_gamma),
    "gamma_f32_running_sum": dict(absmean_gamma=_f32_sum_gamma),
    "gamma_f64_running_sum": dict(absmean_gamma=_f64_sequential_gamma),
    "ternarize_no_eps": dict(ternarize=_tern_no_eps),
    "ternarize_half_away": dict(ternarize=_tern_half_away),
    "ternarize_eps_as_max": dict(ternarize=_tern_eps_as_max),
    "ternarize_threshold_gamma": dict(ternarize=_tern_threshold_gamma),
    "pack_swapped_bits": dict(pack_ternary=_pack_swapped),
    "pack_twos_complement": dict(pack_ternary=_pack_twos_complement),
    "quant_half_away": dict(quant_act=_make_quant(rounder=_half_away)),
    "quant_qb128": dict(quant_act=_make_quant(qb=128)),
    "quant_product_first": dict(quant_act=_make_quant(order="product_first")),
    "quant_no_eps": dict(quant_act=_make_quant(eps=False)),
    "quant_per_tensor": dict(quant_act=_make_quant(per_token=False)),
    "contract_negated": dict(contract=_contract_neg),
    "contract_drop_last_k": dict(contract=_contract_drop_last),
    "contract_transposed": dict(contract=_contract_transposed_t),
    "contract_f32": dict(contract=_contract_f32),
    "rescale_gamma_plus_eps": dict(rescale=_rescale_gamma_eps),
    "rescale_by_128": dict(rescale=_rescale_128),
    "rescale_no_floor": dict(rescale=_rescale_no_floor),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    o = _ns(**MUTANTS[name])
    failed = []
    for pin in pins.PINS:
        try:
            pin(o)
        except Exception:  # an assertion, or the mutant raising on a pin's input
            failed.append(pin.__name__)
    assert failed, f"no pin detects the planted mistake {name}"
