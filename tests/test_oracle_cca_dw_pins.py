"""Pins for the CCA oracle's depthwise intermediate (dw_mode 2, the default).

ZayaCCA ("vllm.model_executor.models.zaya", the layer's depthwise Conv1d ahead
of the grouped Conv1d) materialises the depthwise output in the model dtype.
The plainest reading: the exact value of bias + taps, rounded once to bf16
(nearest, ties to even). These pins check the oracle against that reading by
means that share nothing with it:

* exact rational arithmetic (``fractions.Fraction``) and a nearest-even choice
  among enumerated bf16 neighbours, on random inputs whose exponents spread
  wide and on planted cases: catastrophic cancellation, sums sitting exactly on
  a bf16 midpoint or a tiny amount off it (where only the exact value decides),
  and sums too wide for a double (the oracle's binary128 path);
* the library convolution ``torch.nn.functional.conv1d`` in float64 followed
  by the library's bf16 cast, on positions where the float64 result is
  representable in fp32 (the library casts float64 to bf16 through fp32, which
  is a second rounding elsewhere, so those positions go through an exact fp32
  step first).

The grouped stage is made transparent: identity weights at the newest tap, zero
grouped bias, and q = -k so that both residuals vanish; the q/k part of the
output row is then the depthwise value itself.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synthetic import bf16_to_f32, cca_case


def _bits(v: float) -> int:
    """bf16 bit pattern of a value that bf16 represents exactly."""
    u = np.array([v], np.float32).view(np.uint32)[0]
    assert u & 0xFFFF == 0, v
    return int(u >> 16)


def _val(bits) -> Fraction:
    return Fraction(float(bf16_to_f32(np.array([bits], np.uint16))[0]))


def _nearest_bf16(v: Fraction) -> int:
    """Nearest bf16 to the exact value v, ties to even, by enumerating the
    finite bf16 values around it (exact comparisons)."""
    if v == 0:
        return 0
    f = float(v)
    u = int(np.array([f], np.float32).view(np.uint32)[0] >> 16)
    best = None
    for cand in range(max(0, (u & 0x7FFF) - 2), min(0x7F7F, (u & 0x7FFF) + 2) + 1):
        c = cand | (u & 0x8000)
        d = abs(_val(c) - v)
        key = (d, c & 1)                     # smaller distance, then even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _transparent_case(seed, T_lens, t0, *, hd=8, nq=2, nkv=1):
    case = cca_case("dwpin", seed, nq=nq, nkv=nkv, hd=hd, t0=t0, t1=2, num_decodes=1,
                    prefill_lens=T_lens, num_slots=8, w_std=0.3)
    case.w_gr[:] = 0
    case.b_gr[:] = 0
    one = _bits(1.0)
    for o in range(case.C):
        case.w_gr[o, o % hd, 1] = one
    return case


def _set_q_minus_k(case):
    G = case.nq // case.nkv
    hd = case.hd
    for h in range(case.nq):
        kk = case.k[:, (h // G) * hd:(h // G + 1) * hd]
        case.q[:, h * hd:(h + 1) * hd] = kk ^ 0x8000          # exact negation


def _ext_rows(case, s, L, slot, h):
    """ext[c][u] (bf16 bits) for one request: history then raw [q | k]."""
    raw = np.concatenate([case.q[s:s + L], case.k[s:s + L]], axis=1).T     # (C, L)
    hist = case.conv_state[slot] if h else np.zeros_like(case.conv_state[slot])
    return np.concatenate([hist, raw], axis=1)


def _reqs(case):
    r = [(i, 1, case.decode_slots[i], 1) for i in range(case.num_decodes)]
    r += [(case.num_decodes + case.qsl_p[i], case.qsl_p[i + 1] - case.qsl_p[i],
           case.prefill_slots[i], case.prefill_h[i]) for i in range(case.num_prefills)]
    return r


def _random_wide_bf16(rng, shape, lo, hi):
    """bf16 values with random sign, mantissa and exponent in [lo, hi]."""
    e = rng.integers(lo, hi + 1, shape)
    m = rng.integers(0, 128, shape)
    s = rng.integers(0, 2, shape)
    return ((s << 15) | ((e + 127) << 7) | m).astype(np.uint16)


def _plant(case, s, t0, *, double_exact_only=False):
    """Planted sums on channel columns of the k group, at the request starting
    at row s (its rows s.. are raw inputs; taps read rows s+u-(t0-1)+a).
    double_exact_only: only the sums a double holds exactly."""
    C, hd = case.C, case.hd
    kc = C - hd                               # first channel of the k group
    cases = []
    # catastrophic cancellation: 256 + (1+2^-7)*2^-16 - 256 = 2^-16 + 2^-23
    cases.append((256.0, [1 + 2 ** -7, -1.0], [2.0 ** -16, 256.0]))
    # exactly a bf16 midpoint (ties to even)
    cases.append((1.0, [2.0 ** -4, 2.0 ** -35], [2.0 ** -4, 0.0]))
    # within a double's reach but not a float's, just off that midpoint: a
    # detour through fp32 would land on the midpoint and round to even
    cases.append((1.0, [2.0 ** -4, 2.0 ** -15], [2.0 ** -4, 2.0 ** -15]))
    cases.append((1.0, [2.0 ** -4, 2.0 ** -15], [2.0 ** -4, -(2.0 ** -15)]))
    if not double_exact_only:
        # a representable value (odd mantissa) plus a hair beyond a double
        cases.append((1 + 2 ** -7, [2.0 ** -35, 2.0 ** -35], [2.0 ** -35, 0.0]))
        # a hair above / below that midpoint, far below a double's precision
        # (the oracle's binary128 path)
        cases.append((1.0, [2.0 ** -4, 2.0 ** -35], [2.0 ** -4, 2.0 ** -35]))
        cases.append((1.0, [2.0 ** -4, 2.0 ** -35], [2.0 ** -4, -(2.0 ** -35)]))
        # a term far below the others that still decides a midpoint
        cases.append((2.0 ** 60, [2.0 ** 52, 2.0 ** -20], [1.0, 2.0 ** -20]))
    for j, (b, w, x) in enumerate(cases):
        c = kc + j
        col = c - (C - case.nkv * hd)
        # the channel's other inputs are 1.0, so its other sums stay within
        # binary128's reach next to the planted bias
        case.k[:, col] = _bits(1.0)
        case.conv_state[:, c, :] = _bits(1.0)
        case.b_dw[c] = _bits(b)
        # the planted pair is the newest two taps (older taps weigh zero); they
        # read rows s+1 (older) and s+2 (newer): the output at request row 2
        case.w_dw[c, :] = 0
        case.w_dw[c, t0 - 2] = _bits(w[0])
        case.w_dw[c, t0 - 1] = _bits(w[1])
        case.k[s + 1, col] = _bits(x[0])
        case.k[s + 2, col] = _bits(x[1])
    return kc, len(cases)


@pytest.mark.parametrize("t0", [2, 3, 4])
def test_cca_dw_exact_value_rounded_once(t0):
    rng = np.random.default_rng(1100 + t0)
    case = _transparent_case(1200 + t0, [7, 1, 5], t0)
    # terms spread over up to ~84 binades: most sums do not fit a double and
    # take the oracle's binary128 path
    for name in ("k", "conv_state"):
        arr = getattr(case, name)
        arr[...] = _random_wide_bf16(rng, arr.shape, -20, 20)
    case.w_dw[...] = _random_wide_bf16(rng, case.w_dw.shape, -20, 8)
    case.b_dw[...] = _random_wide_bf16(rng, case.b_dw.shape, -20, 8)
    s0 = case.num_decodes                     # first prefill request's first row
    # with t0 = 2 the planted pair sits at positions 1, 2 of the request; for
    # wider windows the extra (oldest) taps carry zero weights
    kc, nplant = _plant(case, s0, t0)
    case.prefill_h[0] = 0
    _set_q_minus_k(case)
    out, _, _, _ = oracle.cca(case, out_dtype="f64")
    n, C = case.n, case.C
    planted_seen = 0
    for s, L, slot, h in _reqs(case):
        ext = _ext_rows(case, s, L, slot, h)
        for t in range(L):
            u = n + t
            for c in range(C):
                v = _val(case.b_dw[c])
                for a in range(t0):
                    v += _val(case.w_dw[c, a]) * _val(ext[c, u - (t0 - 1) + a])
                exp = float(bf16_to_f32(np.array([_nearest_bf16(v)], np.uint16))[0])
                assert out[s + t, c] == exp, (s, t, c, v, out[s + t, c], exp)
                if s == s0 and t == 2 and kc <= c < kc + nplant:
                    planted_seen += 1
    assert planted_seen == nplant


def test_planted_sums_are_ones_an_fp32_chain_gets_wrong():
    # The planted cancellation case is one where rounding an fp32 intermediate
    # changes the answer: the pin above would catch an oracle that did that.
    b, w, x = 256.0, [1 + 2 ** -7, -1.0], [2.0 ** -16, 256.0]
    exact = Fraction(b) + Fraction(w[0]) * Fraction(x[0]) + Fraction(w[1]) * Fraction(x[1])
    s1 = np.float32(Fraction(b) + Fraction(w[0]) * Fraction(x[0]))     # rounded to fp32
    chain = Fraction(float(s1)) + Fraction(w[1]) * Fraction(x[1])
    assert exact == Fraction(2) ** -16 + Fraction(2) ** -23
    assert _nearest_bf16(exact) != _nearest_bf16(chain)
    # and the double-width case: a double holds neither sum exactly
    big = Fraction(2) ** 60 + Fraction(2) ** 52 + Fraction(2) ** -40
    assert Fraction(float(big)) != big


def test_cca_dw_matches_library_conv_then_bf16_cast():
    # Exponents drawn from narrow ranges: every float64 sum here is exact (its
    # terms span under 40 bits), so the library's float64 conv is the exact value.
    rng = np.random.default_rng(77)
    case = _transparent_case(1300, [9, 4], 2)
    case.k[...] = _random_wide_bf16(rng, case.k.shape, -3, 3)
    case.conv_state[...] = _random_wide_bf16(rng, case.conv_state.shape, -3, 3)
    case.w_dw[...] = _random_wide_bf16(rng, case.w_dw.shape, -3, 0)
    case.b_dw[...] = _random_wide_bf16(rng, case.b_dw.shape, -3, 0)
    kc, _ = _plant(case, case.num_decodes, 2, double_exact_only=True)
    _set_q_minus_k(case)
    out, _, _, _ = oracle.cca(case, out_dtype="f64")
    n, C = case.n, case.C
    wd = torch.from_numpy(bf16_to_f32(case.w_dw).astype(np.float64)[:, None, :])
    bd = torch.from_numpy(bf16_to_f32(case.b_dw).astype(np.float64))
    checked = 0
    for s, L, slot, h in _reqs(case):
        ext = torch.from_numpy(bf16_to_f32(_ext_rows(case, s, L, slot, h)).astype(np.float64))
        dw = F.conv1d(ext[None], wd, bd, groups=C)[0]          # (C, n + L - 1), float64
        dw = dw[:, n - 1:]                                      # positions n .. n+L-1
        f32 = dw.to(torch.float32)
        exact32 = f32.to(torch.float64) == dw                   # no rounding on the way to fp32
        ref = f32.to(torch.bfloat16).to(torch.float64).T.numpy()
        got = out[s:s + L, :C]
        m = exact32.T.numpy()
        np.testing.assert_array_equal(got[m], ref[m])
        checked += int(m.sum())
        if s == case.num_decodes:
            assert m[2, kc], "the planted cancellation sum is representable in fp32"
    assert checked > 0.5 * sum(L for _, L, _, _ in _reqs(case)) * C


def test_chain_diff_diagnostic_counts_the_planted_case():
    case = _transparent_case(1400, [6], 2)
    case.k[...] = _bits(0.5)
    case.w_dw[...] = _bits(0.25)
    case.b_dw[...] = _bits(0.125)
    _plant(case, case.num_decodes, 2)
    _set_q_minus_k(case)
    cnt = []
    oracle.cca(case, out_dtype="f64", chain_diff=cnt)
    # the cancellation sum and the midpoint-plus-hair sums round differently
    # through an fp32 chain; everything else is exact in fp32
    assert cnt[0] >= 2
