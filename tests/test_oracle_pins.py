"""Pins for the CPU oracle: checks it against facts fixed by the pages and by
mathematics, never against itself or the GPU path.

Pins used (page titles as in the oracle's header):
* zero initial state == textbook zero-padded causal convolution (the PLE
  layer's Conv1d with padding=(K-1)*d and dilation d; the CCA profile-run
  path pads the raw input with the history length), checked against the
  library convolution ``torch.nn.functional.conv1d`` in float64;
* with history == the GDN page's per-sequence conv over ``cat([prior, x])``,
  again via ``conv1d``;
* state write-back == last H entries of ``[history, x]`` (ZayaCCA
  ``_mix_with_state``: the new history is the last n inputs);
* chunked prefill + decode == one-shot (state carry), bit for bit;
* checkpoint window at offset p == one-shot state after the first p tokens;
* decode (one token) closed form as a dot product;
* brute force over tiny shapes with a time-indexed formulation;
* bf16 rounding: nearest representable, ties to even, by enumeration of
  neighbours.
A planted mistake in the oracle (dropped bias, reversed taps, wrong dilation
offset, history read at the wrong end, transposed grouped weight, residual
pairing by the wrong head) fails at least one of these.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synthetic import bf16_to_f32, cca_case, conv_case


def f64(a, dtype):
    if a is None:
        return None
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def bf16_val(bits: int) -> float:
    return float(bf16_to_f32(np.array([bits], np.uint16))[0])


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------
def test_double_to_bf16_is_nearest_ties_even():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 127, 3000)))
    # exact ties between neighbouring bf16 values, both parities, and just off them
    for bits in [0x3F80, 0x3F81, 0x4049, 0x0001, 0x0080, 0x7F7E, 0xBF80, 0xC123]:
        a, b = bf16_val(bits), bf16_val(bits + 1)
        m = (a + b) / 2
        vals += [m, np.nextafter(m, np.inf), np.nextafter(m, -np.inf)]
    vals += [1.0, -1.5, 3.0e38, -3.0e38, 1e-45, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135]
    for v in vals:
        v = float(v)
        r = oracle.double_to_bf16(v)
        mag = r & 0x7FFF
        assert (r >> 15) == (1 if math.copysign(1.0, v) < 0 else 0), (v, hex(r))
        err = abs(abs(v) - bf16_val(mag))
        for nb in (mag - 1, mag + 1):
            if 0 <= nb <= 0x7F7F:
                e2 = abs(abs(v) - bf16_val(nb))
                assert err <= e2, (v, hex(r), hex(nb))
                if err == e2:
                    assert (mag & 1) == 0, ("tie not to even", v, hex(r))
    assert oracle.double_to_bf16(0.0) == 0x0000
    assert oracle.double_to_bf16(-0.0) == 0x8000
    assert oracle.double_to_bf16(1e39) == 0x7F80
    assert oracle.double_to_bf16(-1e39) == 0xFF80


def test_double_to_bf16_matches_library_on_fp32_values():
    # for values exactly representable in fp32, fp32->bf16 of the library is a
    # single rounding too
    rng = np.random.default_rng(8)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.double_to_bf16(float(x)) for x in v], np.uint16)
    assert np.array_equal(lib, ours)


# --------------------------------------------------------------------------
# depthwise conv vs library convolution
# --------------------------------------------------------------------------
def _torch_conv_request(x_r, hist, w, b, d, act):
    """conv1d over cat([history, x]) with no padding: one output per token."""
    ext = np.concatenate([hist, x_r.T], axis=1)[None]          # (1, C, H+L)
    y = F.conv1d(torch.from_numpy(ext), torch.from_numpy(w[:, None, :]),
                 None if b is None else torch.from_numpy(b), dilation=d,
                 groups=w.shape[0])[0].T
    if act == "silu":
        y = F.silu(y)
    return y.numpy()


@pytest.mark.parametrize("K,d", [(1, 1), (2, 1), (3, 2), (4, 1), (4, 3), (5, 2)])
@pytest.mark.parametrize("act", ["none", "silu"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_state_equals_padded_conv(K, d, act, dtype):
    case = conv_case("pin", 11 + K * 7 + d, C=6, K=K, d=d, dtype=dtype, act=act,
                     w_std=0.5, bias_std=0.3, num_slots=5,
                     prefill_lens=[1, 7, 19, 2], prefill_h_all=0)
    out, _, _ = oracle.conv(case, out_dtype="f64")
    x, w, b = f64(case.x, dtype), f64(case.w, dtype), f64(case.bias, dtype)
    H = (K - 1) * d
    for r in range(case.num_prefills):
        s, e = case.qsl_p[r], case.qsl_p[r + 1]
        # the PLE layer's module: Conv1d(C, C, K, groups=C, padding=H, dilation=d)
        conv = torch.nn.Conv1d(case.C, case.C, K, groups=case.C, padding=H,
                               dilation=d, bias=True, dtype=torch.float64)
        with torch.no_grad():
            conv.weight.copy_(torch.from_numpy(w[:, None, :]))
            conv.bias.copy_(torch.from_numpy(b))
            y = conv(torch.from_numpy(x[s:e].T[None]))[0, :, : e - s].T
            if act == "silu":
                y = F.silu(y)
        np.testing.assert_allclose(out[s:e], y.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("K,d", [(2, 1), (4, 1), (4, 3), (3, 4)])
def test_with_history_equals_library_conv_over_prior_and_x(K, d):
    case = conv_case("pin", 100 + K + d, C=5, K=K, d=d, dtype="bf16", act="silu",
                     w_std=0.5, bias_std=0.3, num_slots=9, num_decodes=3, q=2,
                     prefill_lens=[1, 2, 5, 13], prefill_h_p=0.5)
    case.prefill_h[:2] = [1, 0]
    out, _, _ = oracle.conv(case, out_dtype="f64")
    x, w, b = f64(case.x, "bf16"), f64(case.w, "bf16"), f64(case.bias, "bf16")
    pool = f64(case.pool, "bf16")
    reqs = [(i * case.q, case.q, case.decode_slots[i], 1) for i in range(case.num_decodes)]
    base = case.num_decode_tokens
    reqs += [(base + case.qsl_p[r], case.qsl_p[r + 1] - case.qsl_p[r],
              case.prefill_slots[r], case.prefill_h[r]) for r in range(case.num_prefills)]
    for s, L, slot, h in reqs:
        hist = pool[slot] * h
        y = _torch_conv_request(x[s:s + L], hist, w, b, d, "silu")
        np.testing.assert_allclose(out[s:s + L], y, rtol=1e-12, atol=1e-13)


def test_decode_closed_form():
    case = conv_case("pin", 5, C=7, K=4, d=1, dtype="f32", act="none", w_std=0.5,
                     bias_std=0.2, num_slots=6, num_decodes=4, q=1)
    out, pool_after, _ = oracle.conv(case, out_dtype="f64")
    x, w, b = f64(case.x, "f32"), f64(case.w, "f32"), f64(case.bias, "f32")
    pool = f64(case.pool, "f32")
    for i, slot in enumerate(case.decode_slots):
        for c in range(case.C):
            window = np.append(pool[slot, c], x[i, c])      # oldest ... newest
            assert out[i, c] == pytest.approx(np.dot(w[c], window) + b[c], rel=1e-13, abs=1e-14)
            # new state: the window without its oldest entry
            np.testing.assert_array_equal(f64(pool_after[slot, c], "f32"), window[1:])


# --------------------------------------------------------------------------
# state write-back, canaries, padding slots, zero-length requests
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d", [1, 3])
def test_state_writeback_is_last_inputs(d):
    case = conv_case("pin", 21 + d, C=4, K=4, d=d, dtype="bf16", act="silu",
                     w_std=0.3, bias_std=0.1, num_slots=16, num_decodes=2, q=3,
                     prefill_lens=[1, 2, 8, 9, 10, 31], prefill_h_p=0.5)
    H = 3 * d
    _, pool_after, _ = oracle.conv(case)
    reqs = [(i * case.q, case.q, case.decode_slots[i], 1) for i in range(case.num_decodes)]
    base = case.num_decode_tokens
    reqs += [(base + case.qsl_p[r], case.qsl_p[r + 1] - case.qsl_p[r],
              case.prefill_slots[r], case.prefill_h[r]) for r in range(case.num_prefills)]
    touched = set()
    for s, L, slot, h in reqs:
        hist = case.pool[slot] if h else np.zeros_like(case.pool[slot])
        ext = np.concatenate([hist, case.x[s:s + L].T], axis=1)
        np.testing.assert_array_equal(pool_after[slot], ext[:, -H:])
        touched.add(int(slot))
    for sl in range(case.num_slots):
        if sl not in touched:
            np.testing.assert_array_equal(pool_after[sl], case.pool[sl])


def test_padding_slot_and_zero_length():
    case = conv_case("pin", 31, C=3, K=3, d=2, dtype="f32", act="none",
                     w_std=0.3, bias_std=0.1, num_slots=6,
                     prefill_lens=[5, 0, 4], prefill_h_all=1)
    case.prefill_slots[0] = -1           # padding row: no read, no write
    out, pool_after, _ = oracle.conv(case, out_dtype="f64")
    # slot of the zero-length request is untouched; only slot of request 2 changes
    changed = [s for s in range(6) if not np.array_equal(pool_after[s], case.pool[s])]
    assert changed == [int(case.prefill_slots[2])]
    x, w, b = f64(case.x, "f32"), f64(case.w, "f32"), f64(case.bias, "f32")
    y = _torch_conv_request(x[0:5], np.zeros((3, 4)), w, b, 2, "none")
    np.testing.assert_allclose(out[0:5], y, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# state carry: chunked == one-shot, checkpoints == one-shot prefix state
# --------------------------------------------------------------------------
def _single(case_src, lo, hi, h, pool):
    """A one-request view of rows [lo, hi) of case_src as a prefill."""
    from dataclasses import replace
    c = replace(case_src, x=case_src.x[lo:hi].copy(), num_decodes=0,
                decode_slots=np.zeros(0, np.int32),
                qsl_p=np.array([0, hi - lo], np.int32),
                prefill_slots=np.array([0], np.int32),
                prefill_h=np.array([h], np.uint8), pool=pool, ckpt_grid=0,
                cu_ckpt=None, ckpt_slots=None)
    return c


@pytest.mark.parametrize("d,dtype", [(1, "bf16"), (3, "bf16"), (2, "f32")])
def test_chunked_equals_one_shot(d, dtype):
    L = 53
    src = conv_case("pin", 41 + d, C=9, K=4, d=d, dtype=dtype, act="silu",
                    w_std=0.3, bias_std=0.1, num_slots=1, prefill_lens=[L],
                    prefill_h_all=1)
    one_out, one_pool, _ = oracle.conv(_single(src, 0, L, 1, src.pool.copy()))
    for cuts in ([1], [2, 3], [5, 20, 21, 22], [40, 50, 51, 52], [3, 6, 9, 12]):
        pool = src.pool.copy()
        edges = [0] + cuts + [L]
        outs = []
        for i in range(len(edges) - 1):
            o, pool, _ = oracle.conv(_single(src, edges[i], edges[i + 1], 1, pool), pool=pool)
            outs.append(o)
        np.testing.assert_array_equal(np.concatenate(outs), one_out)
        np.testing.assert_array_equal(pool, one_pool)


def test_checkpoints_equal_prefix_states():
    g = 8
    case = conv_case("pin", 51, C=5, K=4, d=2, dtype="bf16", act="none",
                     w_std=0.3, bias_std=None, num_slots=40, num_decodes=2,
                     prefill_lens=[7, 8, 9, 16, 30, 33], prefill_h_p=0.5,
                     ckpt_grid=g)
    _, pool_after, _ = oracle.conv(case)
    base = case.num_decode_tokens
    for r in range(case.num_prefills):
        s = base + case.qsl_p[r]
        L = case.qsl_p[r + 1] - case.qsl_p[r]
        cnt = case.cu_ckpt[r + 1] - case.cu_ckpt[r]
        assert cnt == L // g
        for m in range(1, cnt + 1):
            pool = case.pool[[case.prefill_slots[r]]].copy()
            _, pref_pool, _ = oracle.conv(_single(case, s, s + m * g, case.prefill_h[r], pool),
                                          pool=pool)
            dst = case.ckpt_slots[case.cu_ckpt[r] + m - 1]
            np.testing.assert_array_equal(pool_after[dst], pref_pool[0])


# --------------------------------------------------------------------------
# tiny brute force, time-indexed formulation
# --------------------------------------------------------------------------
def test_tiny_brute_force():
    rng = np.random.default_rng(99)
    for C, K, d, L, h, pad in itertools.product([1, 3], [1, 2, 3, 4], [1, 2, 3],
                                                range(0, 8), [0, 1], [0, 1]):
        H = (K - 1) * d
        x = rng.standard_normal((L, C)).astype(np.float32)
        w = rng.standard_normal((C, K)).astype(np.float32)
        b = rng.standard_normal(C).astype(np.float32)
        pool = rng.standard_normal((2, C, H)).astype(np.float32)
        from synthetic import ConvCase
        case = ConvCase(name="bf", C=C, K=K, d=d, S=H, dtype="f32", act="none",
                        x=x, w=w, bias=b, pool=pool.copy(),
                        qsl_p=np.array([0, L], np.int32),
                        prefill_slots=np.array([-1 if pad else 1], np.int32),
                        prefill_h=np.array([h], np.uint8))
        out, pa, _ = oracle.conv(case, out_dtype="f64")
        for c in range(C):
            # sequence indexed by time; history entry j holds time j - H
            seq = {}
            for j in range(H):
                seq[j - H] = float(pool[1, c, j]) if (h and not pad) else 0.0
            for t in range(L):
                seq[t] = float(x[t, c])
            for t in range(L):
                acc = float(b[c])
                for k in range(K):
                    lag = (K - 1 - k) * d
                    acc += float(w[c, k]) * seq[t - lag]
                assert out[t, c] == pytest.approx(acc, rel=1e-12, abs=1e-12)
            if not pad and L > 0:
                exp_state = [seq[L - H + j] for j in range(H)]
                np.testing.assert_array_equal(pa[1, c].astype(np.float64), exp_state)
            else:
                np.testing.assert_array_equal(pa[1, c], pool[1, c])


# --------------------------------------------------------------------------
# CCA
# --------------------------------------------------------------------------
def _cca_f64(case):
    names = ["q", "k", "v_cur", "v_del", "w_dw", "b_dw", "w_gr", "b_gr",
             "delayed_init", "conv_state", "delayed_state"]
    return {n: f64(getattr(case, n), case.dtype) for n in names}


def _torch_cca_request(a, case, s, L, slot, h):
    """ZayaCCA conv stack on cat([history, raw]) plus residual mix, via the
    library convolutions and tensor ops, in float64."""
    nq, nkv, hd = case.nq, case.nkv, case.hd
    G = nq // nkv
    C = case.C
    raw = np.concatenate([a["q"][s:s + L], a["k"][s:s + L]], axis=1)   # (L, C)
    hist = a["conv_state"][slot] * h                                   # (C, n)
    ext = torch.from_numpy(np.concatenate([hist, raw.T], axis=1)[None])
    dw = F.conv1d(ext, torch.from_numpy(a["w_dw"][:, None, :]),
                  torch.from_numpy(a["b_dw"]), groups=C)
    yg = F.conv1d(dw, torch.from_numpy(a["w_gr"]), torch.from_numpy(a["b_gr"]),
                  groups=nq + nkv)[0].T                                  # (L, C)
    heads = (L, -1, hd)
    qv = torch.from_numpy(a["q"][s:s + L]).view(heads)
    kv = torch.from_numpy(a["k"][s:s + L]).view(heads)
    qres = 0.5 * (qv + kv.repeat_interleave(G, dim=1))
    kres = qres.view(L, -1, G, hd).mean(dim=2)
    query = yg[:, : nq * hd].reshape(heads) + qres
    key = yg[:, nq * hd:].reshape(heads) + kres
    first = a["delayed_state"][slot] if h else a["delayed_init"]
    dprev = np.concatenate([first[None], a["v_del"][s:s + L - 1]], axis=0)
    value = torch.from_numpy(np.concatenate([a["v_cur"][s:s + L], dprev], axis=1))
    return torch.cat([query, key, value.view(heads)], dim=1).flatten(1).numpy()


def _cca_reqs(case):
    reqs = [(i, 1, case.decode_slots[i], 1) for i in range(case.num_decodes)]
    reqs += [(case.num_decodes + case.qsl_p[r], case.qsl_p[r + 1] - case.qsl_p[r],
              case.prefill_slots[r], case.prefill_h[r]) for r in range(case.num_prefills)]
    return reqs


@pytest.mark.parametrize("shape", [(4, 2, 8, 2, 2), (2, 2, 4, 3, 2), (6, 2, 4, 2, 3)])
def test_cca_matches_library_convs(shape):
    nq, nkv, hd, t0, t1 = shape
    case = cca_case("pin", 61 + sum(shape), nq=nq, nkv=nkv, hd=hd, t0=t0, t1=t1,
                    num_decodes=3, prefill_lens=[1, 2, 3, 9], num_slots=12,
                    w_std=0.3)
    case.prefill_h[:4] = [0, 1, 1, 0]
    a = _cca_f64(case)
    out, cs, ds, _ = oracle.cca(case, out_dtype="f64", dw_mode=0,
                                io_override=("f64", a))
    for s, L, slot, h in _cca_reqs(case):
        exp = _torch_cca_request(a, case, s, L, slot, h)
        np.testing.assert_allclose(out[s:s + L], exp, rtol=1e-12, atol=1e-13)
        # history write-back and delayed value
        raw = np.concatenate([a["q"][s:s + L], a["k"][s:s + L]], axis=1)
        ext = np.concatenate([a["conv_state"][slot] * h, raw.T], axis=1)
        np.testing.assert_array_equal(cs[slot], ext[:, -case.n:])
        np.testing.assert_array_equal(ds[slot], a["v_del"][s + L - 1])


def test_cca_dw_rounded_once_from_fp32_chain():
    # dw_mode 1: the depthwise value is an fp32 fused multiply-add chain (bias
    # first) materialised in bf16; for bf16 operands each product is exact in
    # fp32, so fp32 adds in numpy give the same chain.
    case = cca_case("pin", 71, nq=2, nkv=1, hd=4, t0=2, t1=2, num_decodes=2,
                    prefill_lens=[3, 5], num_slots=8, w_std=0.5)
    out, _, _, _ = oracle.cca(case, out_dtype="f64", dw_mode=1)
    a = _cca_f64(case)
    b = {k: v.astype(np.float32) for k, v in a.items()}
    C, hd, n = case.C, case.hd, case.n
    for s, L, slot, h in _cca_reqs(case):
        raw = np.concatenate([b["q"][s:s + L], b["k"][s:s + L]], axis=1).T
        ext = np.concatenate([b["conv_state"][slot] * h, raw], axis=1)   # (C, n+L) f32
        dw = np.zeros((C, n + L), np.float32)
        for u in range(1, n + L):
            acc = b["b_dw"].copy()
            acc = acc + b["w_dw"][:, 0] * ext[:, u - 1]
            acc = acc + b["w_dw"][:, 1] * ext[:, u]
            dw[:, u] = torch.from_numpy(acc).to(torch.bfloat16).float().numpy()
        dw = dw.astype(np.float64)
        for t in range(L):
            u = n + t
            for o in range(C):
                g = o // hd
                y = a["b_gr"][o] + sum(a["w_gr"][o, j, bb] * dw[g * hd + j, u - 1 + bb]
                                       for j in range(hd) for bb in range(2))
                if o < case.nq * hd:
                    e, hh = o % hd, o // hd
                    y += 0.5 * (a["q"][s + t, o] + a["k"][s + t, (hh // 2) * hd + e])
                else:
                    e = o % hd
                    y += np.mean([0.5 * (a["q"][s + t, i * hd + e] + a["k"][s + t, e])
                                  for i in range(2)])
                assert out[s + t, o] == pytest.approx(y, rel=1e-12, abs=1e-13)


def test_cca_identity_grouped_reduces_to_depthwise():
    # W2 = identity at the newest tap and zero bias: the grouped stage passes
    # the depthwise output through, so the q/k part equals the depthwise
    # oracle over the same channels (history = last t0-1 raw inputs) + residual.
    case = cca_case("pin", 81, nq=4, nkv=2, hd=4, t0=3, t1=2, num_decodes=2,
                    prefill_lens=[1, 4, 6], num_slots=8, w_std=0.4)
    case.w_gr[:] = 0
    case.b_gr[:] = 0
    one = 0x3F80
    for o in range(case.C):
        case.w_gr[o, o % case.hd, case.t1 - 1] = one
    out, _, _, _ = oracle.cca(case, out_dtype="f64", dw_mode=0)
    from synthetic import ConvCase
    raw = np.concatenate([case.q, case.k], axis=1)
    H = case.t0 - 1
    dcase = ConvCase(name="dw", C=case.C, K=case.t0, d=1, S=H, dtype="bf16",
                     act="none", x=raw, w=case.w_dw, bias=case.b_dw,
                     pool=np.ascontiguousarray(case.conv_state[:, :, -H:]),
                     num_decodes=case.num_decodes, q=1, decode_slots=case.decode_slots,
                     qsl_p=case.qsl_p, prefill_slots=case.prefill_slots,
                     prefill_h=case.prefill_h)
    dout, _, _ = oracle.conv(dcase, out_dtype="f64")
    a = _cca_f64(case)
    G = case.nq // case.nkv
    hd = case.hd
    qh = a["q"].reshape(case.T, case.nq, hd)
    kh = a["k"].reshape(case.T, case.nkv, hd)
    qres = 0.5 * (qh + np.repeat(kh, G, axis=1))
    kres = qres.reshape(case.T, case.nkv, G, hd).mean(axis=2)
    exp = dout + np.concatenate([qres.reshape(case.T, -1), kres.reshape(case.T, -1)], axis=1)
    np.testing.assert_allclose(out[:, : case.C], exp, rtol=1e-12, atol=1e-13)


def test_cca_chunked_equals_one_shot():
    from dataclasses import replace
    L = 23
    src = cca_case("pin", 91, nq=4, nkv=2, hd=4, t0=2, t1=2, num_decodes=0,
                   prefill_lens=[L], num_slots=1, w_std=0.3)
    src.prefill_h[:] = 1
    one, cs1, ds1, _ = oracle.cca(src)

    def part(lo, hi, cs, ds, as_decode):
        sl = slice(lo, hi)
        kw = dict(q=src.q[sl], k=src.k[sl], v_cur=src.v_cur[sl], v_del=src.v_del[sl],
                  conv_state=cs, delayed_state=ds)
        if as_decode:
            return replace(src, num_decodes=hi - lo,
                           decode_slots=np.zeros(hi - lo, np.int32),
                           qsl_p=np.zeros(1, np.int32), prefill_slots=np.zeros(0, np.int32),
                           prefill_h=np.zeros(0, np.uint8), **kw)
        return replace(src, qsl_p=np.array([0, hi - lo], np.int32),
                       prefill_h=np.array([1], np.uint8), **kw)

    for cuts in ([1], [2, 11], [20, 21, 22]):
        cs, ds = src.conv_state.copy(), src.delayed_state.copy()
        edges = [0] + cuts + [L]
        outs = []
        for i in range(len(edges) - 1):
            lo, hi = edges[i], edges[i + 1]
            c = part(lo, hi, cs, ds, as_decode=(hi - lo == 1))
            o, cs, ds, _ = oracle.cca(c)
            outs.append(o)
        np.testing.assert_array_equal(np.concatenate(outs), one)
        np.testing.assert_array_equal(cs, cs1)
        np.testing.assert_array_equal(ds, ds1)


def test_gather_scatter_are_row_copies():
    rng = np.random.default_rng(3)
    pool = rng.integers(0, 65535, size=(10, 6, 3), dtype=np.uint16)
    idx = np.array([7, -1, 2, 9], np.int32)
    dense = np.full((4, 6, 3), 0xBEEF, np.uint16)
    oracle.state_gather(pool, idx, dense)
    np.testing.assert_array_equal(dense[[0, 2, 3]], pool[[7, 2, 9]])
    np.testing.assert_array_equal(dense[1], 0)
    newd = rng.integers(0, 65535, size=(4, 6, 3), dtype=np.uint16)
    p2 = pool.copy()
    oracle.state_scatter(newd, idx, p2)
    exp = pool.copy()
    exp[[7, 2, 9]] = newd[[0, 2, 3]]
    np.testing.assert_array_equal(p2, exp)
