"""Pins for the CCA oracle's rounding allowance (``oracle.cca(..., allow=[])``).

The layer materialises its depthwise output in bf16 ("vllm.model_executor.
models.zaya", ZayaCCA: the depthwise Conv1d ahead of the grouped Conv1d); the
oracle takes the exact value rounded once. A kernel that sums bias + taps in
fp32 first (in any order) and then rounds may land on the other bf16 neighbour
when the exact value lies close to a rounding boundary. The allowance is the
oracle's bound on how far that can move each conv output: the sum over its
depthwise inputs of |W2| times the spread of the bf16 roundings of the values
within the fp32 summation bound of the exact sum. These pins check it by means
that share nothing with its code:

* brute force over fp32 summation orders (every order of the terms, every
  partial sum rounded to fp32 with exact rational arithmetic), each result
  rounded to bf16: none may leave the allowance, and on planted sums near a
  midpoint some do move;
* the oracle's own fp32 chain mode (dw_mode 1, another summation order) through
  the whole grouped stage with random grouped weights: every output moves by
  at most its allowance, outputs with a zero allowance do not move at all, and
  some do move;
* closed cases: zero allowance where every sum is exact in fp32 and far from a
  boundary, one bf16 spacing times |W2| at an exact midpoint, and one spacing
  for a sum one fp32 rounding off a midpoint (which an fp32 order lands on).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synthetic import bf16_to_f32
from tests.test_oracle_cca_dw_pins import (_bits, _ext_rows, _nearest_bf16, _plant,
                                           _random_wide_bf16, _reqs, _set_q_minus_k,
                                           _transparent_case, _val)


def _nearest_f32(v: Fraction) -> Fraction:
    """Nearest fp32 to the exact value v, ties to even (exact comparisons among
    the fp32 neighbours of the double nearest to v)."""
    if v == 0:
        return Fraction(0)
    f = np.float32(float(v))
    cands = [f]
    for d in (np.float32(np.inf), np.float32(-np.inf)):
        g = f
        for _ in range(2):
            g = np.nextafter(g, d)
            cands.append(g)
    best = None
    for c in cands:
        bits = int(np.array([c], np.float32).view(np.uint32)[0])
        key = (abs(Fraction(float(c)) - v), bits & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return Fraction(float(best[1]))


def _bf16_value(v: Fraction) -> float:
    return float(bf16_to_f32(np.array([_nearest_bf16(v)], np.uint16))[0])


def _fp32_orders(bias: Fraction, w, x):
    """Every fp32 evaluation of bias + sum w[a] x[a] that adds the terms one at
    a time in some order, rounding every partial sum to fp32 (the products of
    two bf16 values are exact in fp32, so fusing them changes nothing)."""
    terms = [bias] + [wa * xa for wa, xa in zip(w, x)]
    seen = set()
    for perm in itertools.permutations(terms):
        acc = None
        for t in perm:
            acc = _nearest_f32(t if acc is None else acc + t)
        seen.add(acc)
    return seen


@pytest.mark.parametrize("t0", [2, 3])
def test_allowance_covers_every_fp32_order(t0):
    rng = np.random.default_rng(2100 + t0)
    case = _transparent_case(2200 + t0, [6, 1, 4], t0)
    for name in ("k", "conv_state"):
        arr = getattr(case, name)
        arr[...] = _random_wide_bf16(rng, arr.shape, -6, 6)
    case.w_dw[...] = _random_wide_bf16(rng, case.w_dw.shape, -6, 2)
    case.b_dw[...] = _random_wide_bf16(rng, case.b_dw.shape, -6, 2)
    kc, nplant = _plant(case, case.num_decodes, t0, double_exact_only=True)
    case.prefill_h[0] = 0
    _set_q_minus_k(case)
    al = []
    out, _, _, _ = oracle.cca(case, out_dtype="f64", allow=al)
    allow = al[0]
    n, C = case.n, case.C
    moved = 0
    for s, L, slot, h in _reqs(case):
        ext = _ext_rows(case, s, L, slot, h)
        for t in range(L):
            u = n + t
            for c in range(C):
                b = _val(case.b_dw[c])
                w = [_val(case.w_dw[c, a]) for a in range(t0)]
                x = [_val(ext[c, u - (t0 - 1) + a]) for a in range(t0)]
                for r in _fp32_orders(b, w, x):
                    alt = _bf16_value(r)
                    d = abs(alt - out[s + t, c])
                    assert d <= allow[s + t, c], (s, t, c, alt, out[s + t, c], allow[s + t, c])
                    moved += d > 0
    assert moved > 0, "no fp32 order moved a planted sum: the pin has no teeth"


def test_allowance_bounds_the_fp32_chain_mode_through_the_grouped_stage():
    # wide exponents make sums that cancel and sit near rounding boundaries;
    # random grouped weights spread each depthwise value over 2 * hd outputs
    rng = np.random.default_rng(2301)
    from synthetic import cca_case
    case = cca_case("allowpin", 2302, nq=4, nkv=2, hd=16, t0=3, t1=2, num_decodes=5,
                    prefill_lens=[40, 1, 70], num_slots=16)
    for name in ("q", "k", "conv_state"):
        arr = getattr(case, name)
        arr[...] = _random_wide_bf16(rng, arr.shape, -12, 12)
    case.w_dw[...] = _random_wide_bf16(rng, case.w_dw.shape, -12, 4)
    case.b_dw[...] = _random_wide_bf16(rng, case.b_dw.shape, -12, 4)
    # and the planted sums (cancellation, midpoints and a hair off them) in the
    # k group's first channels at the first prefill request's third row
    _plant(case, case.num_decodes, case.t0, double_exact_only=True)
    al, nd = [], []
    exact, _, _, ab = oracle.cca(case, out_dtype="f64", absum=True, allow=al, chain_diff=nd)
    chain, _, _, _ = oracle.cca(case, out_dtype="f64", dw_mode=1)
    allow = al[0]
    C = case.C
    d = np.abs(chain[:, :C] - exact[:, :C])
    # the grouped sums are taken in double in the same order on both sides:
    # only the depthwise values differ (plus the double sums' own rounding)
    slack = 2.0 ** -45 * ab[:, :C]
    assert (d <= allow[:, :C] + slack).all()
    assert (d[allow[:, :C] == 0] == 0).all()
    assert nd[0] > 0 and (d > 0).sum() > 0
    assert (allow[:, C:] == 0).all()


def test_allowance_zero_far_from_boundaries_and_one_spacing_at_a_midpoint():
    case = _transparent_case(2400, [6], 2)
    # every sum is 0.375 + 0.25 (x0 + x1) with x0, x1 in {-0.5, 0, 0.5}
    # (q = -k makes the residuals vanish): 0.125 to 0.625, exact in fp32 and
    # far from any rounding boundary (a sum that cancels to zero would not be:
    # near zero the bf16 spacing is finer than the fp32 bound, and the
    # allowance there is that bound times |W2|)
    case.k[...] = _bits(0.5)
    case.conv_state[...] = _bits(0.5)
    case.w_dw[...] = _bits(0.25)
    case.b_dw[...] = _bits(0.375)
    _set_q_minus_k(case)
    al = []
    oracle.cca(case, out_dtype="f64", allow=al)
    assert (al[0] == 0).all()
    # one channel planted on the midpoint 1 + 2^-8 between 1 and 1 + 2^-7
    # (bias 1, newest tap 2^-4 * 2^-4, older tap zero): the fp32 sum is exact
    # there too, but the bound admits both neighbours, one bf16 spacing apart
    c = case.C - 1
    col = c - (case.C - case.nkv * case.hd)
    s = case.num_decodes
    case.b_dw[c] = _bits(1.0)
    case.w_dw[c, :] = [_bits(0.0), _bits(2.0 ** -4)]
    case.k[s + 3, col] = _bits(2.0 ** -4)
    _set_q_minus_k(case)
    # its grouped weight (newest tap) halved: the allowance scales with |W2|
    case.w_gr[c, c % case.hd, 1] = _bits(-0.5)
    al = []
    out, _, _, _ = oracle.cca(case, out_dtype="f64", allow=al)
    assert out[s + 3, c] == -0.5                      # 1 + 2^-8 ties to even: 1
    assert al[0][s + 3, c] == 0.5 * 2.0 ** -7
    others = np.ones_like(al[0], bool)
    others[s + 3, c] = False
    # the planted column's other rows: 1 + 2^-4 * 0.5, exact and far
    assert (al[0][others] == 0).all()


def test_allowance_reaches_a_sum_one_fp32_rounding_off_a_midpoint():
    # 1 + 2^-4 * 2^-4 + (1.625 * 2^-13) * 2^-12 = 1 + 2^-8 + 0.8125 * 2^-24: just
    # above the midpoint between 1 and 1 + 2^-7, by less than half an fp32 ulp
    # at 1, so adding the small product last lands an fp32 sum on the midpoint
    # (ties to even: 1) while the exact value rounds up. The allowance must
    # admit that; a bound under 0.8125 * 2^-24 (a quarter of the fp32 bound
    # or less) would not.
    case = _transparent_case(2500, [6], 2)
    case.k[...] = _bits(0.5)
    case.conv_state[...] = _bits(0.5)
    case.w_dw[...] = _bits(0.25)
    case.b_dw[...] = _bits(0.375)
    c = case.C - 2
    col = c - (case.C - case.nkv * case.hd)
    s = case.num_decodes
    case.b_dw[c] = _bits(1.0)
    case.w_dw[c, :] = [_bits(1.625 * 2.0 ** -13), _bits(2.0 ** -4)]
    case.k[s + 2, col] = _bits(2.0 ** -12)
    case.k[s + 3, col] = _bits(2.0 ** -4)
    _set_q_minus_k(case)
    al = []
    out, _, _, _ = oracle.cca(case, out_dtype="f64", allow=al)
    assert out[s + 3, c] == 1.0 + 2.0 ** -7
    assert al[0][s + 3, c] == 2.0 ** -7
    orders = _fp32_orders(Fraction(1), [_val(case.w_dw[c, 0]), _val(case.w_dw[c, 1])],
                          [Fraction(2) ** -12, Fraction(2) ** -4])
    assert 1.0 in {_bf16_value(r) for r in orders}
    # every other output of the channel sits far from a boundary
    others = np.ones(al[0].shape[0], bool)
    others[s + 3] = False
    assert (al[0][others, c] == 0).all()
