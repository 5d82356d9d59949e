"""Pins for the oracle's speculative (rolling-buffer) update and for the
non-speculative steps on a buffer widened for rollback.

The rolling buffer is the GDN page's `_spec_forward` conv: a state row of
S = H + num_spec entries; a request with q draft tokens and `a` tokens accepted
from its previous step reads the H entries starting at a-1 as its history, and
its buffer becomes the entries from a on, cut to S - q, followed by the q new
tokens. Pins used:

* meaning: with q = num_spec + 1 (the shape the buffer is sized for), every
  step's outputs equal the library convolution of the request's accepted token
  sequence (prefill tokens, then the accepted prefix of each earlier step's
  drafts) followed by the step's drafts. A slip in the history offset, the kept
  range or the append order changes which tokens the next step sees and fails
  this for some acceptance pattern;
* reduction: S = H, q = 1, a = 1 is the plain one-token decode (pinned
  elsewhere against the library convolution), bit for bit in outputs and pool;
* padding slots see a zero history and leave the pool alone;
* accepted counts outside [1, min(q, S - H + 1)] act as the nearest bound;
* a wide buffer under the non-speculative steps: identical to the narrow case
  on the first H columns, the other columns untouched (GDN page,
  `_spec_aware_nonspec`: only the first width-1 columns hold the window).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic
from synthetic import bf16_to_f32, conv_case


def f64(a, dtype):
    if a is None:
        return None
    return bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else np.asarray(a, np.float64)


def _lib_conv(seq, w, b, d, act):
    """Zero-padded causal conv of a (L, C) float64 sequence via conv1d."""
    K = w.shape[1]
    H = (K - 1) * d
    ext = np.concatenate([np.zeros((seq.shape[1], H)), seq.T], axis=1)[None]
    y = F.conv1d(torch.from_numpy(ext), torch.from_numpy(w[:, None, :]),
                 torch.from_numpy(b), dilation=d, groups=w.shape[0])[0].T
    return (F.silu(y) if act == "silu" else y).numpy()


def _spec_step(src, x, slots, acc, pool, q):
    """A batch of spec requests (q rows each) over `pool` (updated in place)."""
    c = replace(src, x=x, num_decodes=len(slots), q=q,
                decode_slots=np.asarray(slots, np.int32), decode_h=None,
                qsl_p=np.zeros(1, np.int32), prefill_slots=np.zeros(0, np.int32),
                prefill_h=np.zeros(0, np.uint8), pool=pool, ckpt_grid=0,
                cu_ckpt=None, ckpt_slots=None)
    return oracle.conv_spec(c, acc, out_dtype="f64", pool=pool)


@pytest.mark.parametrize("K,d,num_spec", [(4, 1, 1), (4, 1, 3), (4, 3, 3), (2, 1, 4),
                                          (3, 2, 2)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_spec_outputs_are_conv_of_accepted_sequence(K, d, num_spec, dtype):
    q = num_spec + 1
    B, L0, steps = 3, 6, 7
    src = conv_case("spec_pin", 1000 + K * 10 + d + num_spec, C=5, K=K, d=d, dtype=dtype,
                    act="silu", w_std=0.5, bias_std=0.3, num_slots=4,
                    prefill_lens=[L0] * B, prefill_h_all=0, num_spec=num_spec)
    w, b = f64(src.w, dtype), f64(src.bias, dtype)
    pool = src.pool.copy()
    # prefill from zero history puts the window in the first H columns
    _, pool, _ = oracle.conv(src, pool=pool)
    seqs = [f64(src.x[r * L0:(r + 1) * L0], dtype) for r in range(B)]
    slots = src.prefill_slots
    rng = np.random.default_rng(K * 100 + d)
    prev = None
    for s in range(steps):
        x = synthetic._normal(rng, (B * q, src.C), 1.0, dtype)
        if s == 0:
            acc = np.ones(B, np.int32)       # first step after prefill
        else:
            acc = rng.integers(1, q + 1, B).astype(np.int32)
            acc[s % B] = q if s % 2 else 1   # both extremes every step
            for r in range(B):
                seqs[r] = np.concatenate([seqs[r], prev[r * q:r * q + acc[r]]])
        out, pool, _ = _spec_step(src, x, slots, acc, pool, q)
        xs = f64(x, dtype)
        for r in range(B):
            full = np.concatenate([seqs[r], xs[r * q:(r + 1) * q]])
            ref = _lib_conv(full, w, b, d, "silu")[-q:]
            np.testing.assert_allclose(out[r * q:(r + 1) * q], ref, rtol=1e-12, atol=1e-13,
                                       err_msg=f"step {s} request {r} a={acc[r]}")
        prev = xs


def test_spec_reduces_to_decode():
    case = conv_case("spec_red", 1101, C=6, K=4, d=1, dtype="bf16", act="silu",
                     w_std=0.5, bias_std=0.3, num_slots=8, num_decodes=5, q=1)
    ref_out, ref_pool, _ = oracle.conv(case)
    out, pool, _ = oracle.conv_spec(case, np.ones(5, np.int32))
    np.testing.assert_array_equal(out, ref_out)
    np.testing.assert_array_equal(pool, ref_pool)


def test_spec_padding_slots_and_clamping():
    K, d, n = 4, 2, 3
    q, H = n + 1, (K - 1) * d
    case = conv_case("spec_pad", 1201, C=4, K=K, d=d, dtype="f32", act="none",
                     w_std=0.5, bias_std=0.3, num_slots=10, num_decodes=6, q=q,
                     num_spec=n)
    case.decode_slots[1] = -1
    case.decode_slots[4] = 10                      # out of range: padding
    acc = np.array([0, 2, -7, 99, 3, 1], np.int32)
    out, pool, _ = oracle.conv_spec(case, acc, out_dtype="f64")
    x, w, b = f64(case.x, "f32"), f64(case.w, "f32"), f64(case.bias, "f32")
    for r in (1, 4):
        np.testing.assert_allclose(out[r * q:(r + 1) * q], _lib_conv(x[r * q:(r + 1) * q], w, b, d,
                                                                     "none"), rtol=1e-12, atol=1e-13)
    touched = {int(s) for s in case.decode_slots if 0 <= s < 10}
    for s in range(10):
        if s not in touched:
            np.testing.assert_array_equal(pool[s], case.pool[s])
    amax = min(q, n + 1)
    clamped = np.clip(acc, 1, amax).astype(np.int32)
    out2, pool2, _ = oracle.conv_spec(case, clamped, out_dtype="f64")
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(pool, pool2)


def test_spec_buffer_roll_when_q_is_short():
    # q < num_spec + 1: the buffer keeps S - q entries from a on, then the drafts
    K, d, n, q = 4, 1, 4, 2
    case = conv_case("spec_short", 1301, C=3, K=K, d=d, dtype="bf16", act="none",
                     w_std=0.5, bias_std=0.3, num_slots=6, num_decodes=4, q=q,
                     num_spec=n)
    S, H = case.S, 3
    acc = np.array([1, 2, 1, 2], np.int32)
    out, pool, _ = oracle.conv_spec(case, acc, out_dtype="f64")
    x, w, b = f64(case.x, "bf16"), f64(case.w, "bf16"), f64(case.bias, "bf16")
    for r, slot in enumerate(case.decode_slots):
        a = int(acc[r])
        old = case.pool[slot]
        xr = case.x[r * q:(r + 1) * q].T
        np.testing.assert_array_equal(pool[slot][:, :S - q], old[:, a:a + S - q])
        np.testing.assert_array_equal(pool[slot][:, S - q:], xr)
        hist = f64(old[:, a - 1:a - 1 + H], "bf16")
        ext = np.concatenate([hist, x[r * q:(r + 1) * q].T], axis=1)[None]
        y = F.conv1d(torch.from_numpy(ext), torch.from_numpy(w[:, None, :]),
                     torch.from_numpy(b), groups=3)[0].T.numpy()
        np.testing.assert_allclose(out[r * q:(r + 1) * q], y, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("d", [1, 3])
def test_wide_buffer_nonspec_steps_use_first_columns(d):
    n = 3
    wide = conv_case("wide", 1401 + d, C=5, K=4, d=d, dtype="bf16", act="silu",
                     w_std=0.4, bias_std=0.2, num_slots=24, num_decodes=3, q=2,
                     prefill_lens=[1, 4, 17, 30], prefill_h_p=0.5, ckpt_grid=8 * d,
                     num_spec=n)
    H = 3 * d
    narrow = replace(wide, S=H, pool=np.ascontiguousarray(wide.pool[:, :, :H]))
    o1, p1, _ = oracle.conv(wide)
    o2, p2, _ = oracle.conv(narrow)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1[:, :, :H], p2)
    np.testing.assert_array_equal(p1[:, :, H:], wide.pool[:, :, H:])


# ---------------------------------------------------------------------------
# per-request draft counts (GDN page, _spec_forward's per-sequence loop over
# spec_query_start_loc: q_i = 0 is skipped)
# ---------------------------------------------------------------------------
def _varlen_step(src, x, slots, acc, pool, qsl):
    c = replace(src, x=x, num_decodes=len(slots), q=1,
                decode_slots=np.asarray(slots, np.int32), decode_h=None,
                qsl_p=np.zeros(1, np.int32), prefill_slots=np.zeros(0, np.int32),
                prefill_h=np.zeros(0, np.uint8), pool=pool, ckpt_grid=0,
                cu_ckpt=None, ckpt_slots=None)
    return oracle.conv_spec_varlen(c, acc, qsl, out_dtype="f64", pool=pool)


@pytest.mark.parametrize("K,d,num_spec", [(4, 1, 3), (4, 2, 2), (2, 1, 4)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_spec_varlen_outputs_are_conv_of_accepted_sequence(K, d, num_spec, dtype):
    """Each step, each request drafts either nothing or the q = num_spec + 1
    tokens the buffer is sized for. A drafting request's outputs are the
    library convolution of its accepted sequence followed by its drafts; a
    request that drafts nothing keeps its buffer, and its pending acceptance
    applies at its next drafting step."""
    q = num_spec + 1
    B, L0, steps = 4, 7, 8
    src = conv_case("spec_vl_pin", 2000 + K * 10 + d + num_spec, C=5, K=K, d=d, dtype=dtype,
                    act="silu", w_std=0.5, bias_std=0.3, num_slots=6,
                    prefill_lens=[L0] * B, prefill_h_all=0, num_spec=num_spec)
    w, b = f64(src.w, dtype), f64(src.bias, dtype)
    pool = src.pool.copy()
    _, pool, _ = oracle.conv(src, pool=pool)
    seqs = [f64(src.x[r * L0:(r + 1) * L0], dtype) for r in range(B)]
    slots = src.prefill_slots
    rng = np.random.default_rng(K * 1000 + d * 10 + num_spec)
    pending = [None] * B            # drafts of each request's last drafting step
    acc_next = np.ones(B, np.int32)  # accepted count its next drafting step uses
    for s in range(steps):
        qs = rng.integers(0, 2, B) * q
        qs[s % B] = 0
        qs[(s + 1) % B] = q
        qsl = np.zeros(B + 1, np.int32)
        qsl[1:] = np.cumsum(qs)
        x = synthetic._normal(rng, (int(qsl[-1]), src.C), 1.0, dtype)
        acc = acc_next.copy()
        for r in range(B):
            if qs[r] and pending[r] is not None:
                seqs[r] = np.concatenate([seqs[r], pending[r][:acc[r]]])
        before = pool.copy()
        out, pool, _ = _varlen_step(src, x, slots, acc, pool, qsl)
        xs = f64(x, dtype)
        for r in range(B):
            rows = slice(int(qsl[r]), int(qsl[r + 1]))
            if qs[r] == 0:
                np.testing.assert_array_equal(pool[slots[r]], before[slots[r]])
                continue
            full = np.concatenate([seqs[r], xs[rows]])
            ref = _lib_conv(full, w, b, d, "silu")[-q:]
            np.testing.assert_allclose(out[rows], ref, rtol=1e-12, atol=1e-13,
                                       err_msg=f"step {s} request {r} a={acc[r]}")
            pending[r] = xs[rows]
            acc_next[r] = rng.integers(1, q + 1)


def test_spec_varlen_slices_per_request():
    """Mixed draft counts in one batch, each against the page's slices: history
    = entries [a-1, a-1+H), new row = entries [a, a+S-q) then the q drafts
    (a clamped to [1, min(q, S-H+1)]); q = 0 and q > S leave the slot and the
    request's output rows untouched."""
    K, d, n = 4, 1, 3
    H, S = 3, 6
    qs = np.array([0, 1, 2, 3, 4, 5, 6, 7, 0, 4, 1], np.int64)
    B = qs.shape[0]
    case, qsl = synthetic.spec_varlen_case("spec_vl_sl", 2301, C=4, K=K, d=d, dtype="bf16",
                                           act="none", w_std=0.5, bias_std=0.3, num_slots=16,
                                           B=B, num_spec=n, q_lens=qs)
    case.decode_slots[9] = -1
    acc = np.array([1, 3, 4, 3, 0, 9, 2, 1, 3, 4, -2], np.int32)
    out, pool, _ = oracle.conv_spec_varlen(case, acc, qsl, out_dtype="f64")
    x, w, b = f64(case.x, "bf16"), f64(case.w, "bf16"), f64(case.bias, "bf16")
    for r in range(B):
        q, slot = int(qs[r]), int(case.decode_slots[r])
        rows = slice(int(qsl[r]), int(qsl[r + 1]))
        valid = 0 <= slot < 16
        if q == 0 or q > S:
            np.testing.assert_array_equal(out[rows], 0.0)
            if valid:
                np.testing.assert_array_equal(pool[slot], case.pool[slot])
            continue
        a = int(np.clip(acc[r], 1, min(q, S - H + 1)))
        old = case.pool[slot] if valid else np.zeros((4, S), case.pool.dtype)
        hist = f64(old[:, a - 1:a - 1 + H], "bf16")
        ext = np.concatenate([hist, x[rows].T], axis=1)[None]
        y = F.conv1d(torch.from_numpy(ext), torch.from_numpy(w[:, None, :]),
                     torch.from_numpy(b), groups=4)[0].T.numpy()
        np.testing.assert_allclose(out[rows], y, rtol=1e-12, atol=1e-13, err_msg=f"request {r}")
        if valid:
            np.testing.assert_array_equal(pool[slot][:, :S - q], old[:, a:a + S - q])
            np.testing.assert_array_equal(pool[slot][:, S - q:], case.x[rows].T)
    touched = {int(case.decode_slots[r]) for r in range(B) if 0 < qs[r] <= S}
    for s in range(16):
        if s not in touched:
            np.testing.assert_array_equal(pool[s], case.pool[s])


@pytest.mark.parametrize("layout", ["ds", "sd"])
def test_spec_varlen_equal_lengths_is_the_uniform_call(layout):
    case = conv_case("spec_vl_eq", 2401, C=6, K=4, d=2, dtype="bf16", act="silu",
                     w_std=0.5, bias_std=0.3, num_slots=12, num_decodes=7, q=3, num_spec=2)
    if layout == "sd":
        case = synthetic.as_sd(case)
    acc = synthetic.num_accepted(7, 7, 3, lo=0, hi=5)
    qsl = np.arange(8, dtype=np.int32) * 3
    o1, p1, _ = oracle.conv_spec(case, acc)
    o2, p2, _ = oracle.conv_spec_varlen(case, acc, qsl)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1, p2)
