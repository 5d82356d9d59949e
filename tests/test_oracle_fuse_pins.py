"""Pins for the oracle's residual fusion and logical-to-physical row mapping
(PLE page, `_short_conv`: "optionally fusing both residual additions", and
the dispatch's `token_indices`, which let the kernels address the spec and
non-spec rows of a mixed batch in place).

* mapping: scattering a case's rows to random physical rows of larger tensors
  (with rows no call references) and passing the map gives the same outputs
  at the mapped rows, the same pool and checkpoints, and leaves every other
  physical row untouched; for the varlen/decode call and the speculative call;
* fusion: with a residual R and outer residual O the stored value is the
  plain (pinned) conv output plus R plus O at the same physical row; a zero
  residual without O reduces to the plain conv; the sequence-parallel branch
  (conv into a zero buffer, then add the gated output and hidden states)
  equals the fused non-parallel call.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synthetic
from synthetic import bf16_to_f32, conv_case


def f64(a, dtype):
    return bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else np.asarray(a, np.float64)


def _scatter(case, extra, seed):
    """Physical tensors with `extra` unreferenced rows and a random row map."""
    rng = np.random.default_rng(seed)
    n = case.T + extra
    perm = rng.permutation(n)[:case.T].astype(np.int32)
    xp = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)   # junk in unused rows
    xp[perm] = case.x
    return xp, perm


def _mixed(dtype, d, seed):
    return conv_case("fuse", seed, C=6, K=4, d=d, dtype=dtype, act="silu", w_std=0.4,
                     bias_std=0.2, num_slots=40, num_decodes=5, q=2,
                     prefill_lens=[1, 3, 9, 17, 33], prefill_h_p=0.5, ckpt_grid=8 * d)


@pytest.mark.parametrize("dtype,d", [("bf16", 1), ("bf16", 3), ("f32", 2)])
def test_token_indices_match_plain_layout(dtype, d):
    case = _mixed(dtype, d, 2000 + d)
    ref, ref_pool, ref_ab = oracle.conv(case, out_dtype="f64", absum=True)
    xp, perm = _scatter(case, 11, 2100 + d)
    out, pool, ab = oracle.conv(case, out_dtype="f64", absum=True, x=xp, token_indices=perm)
    np.testing.assert_array_equal(out[perm], ref)
    np.testing.assert_array_equal(pool, ref_pool)
    np.testing.assert_array_equal(ab, ref_ab)
    unused = np.setdiff1d(np.arange(xp.shape[0]), perm)
    assert unused.size == 11 and not out[unused].any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_residual_fusion_is_plain_conv_plus_residuals(dtype):
    case = _mixed(dtype, 1, 2200)
    ref, ref_pool, _ = oracle.conv(case, out_dtype="f64")
    rng = np.random.default_rng(2201)
    xp, perm = _scatter(case, 7, 2202)
    R = synthetic._normal(rng, xp.shape, 1.0, dtype)
    O = synthetic._normal(rng, xp.shape, 1.0, dtype)
    out, pool, _ = oracle.conv(case, out_dtype="f64", x=xp, token_indices=perm, resid=R, outer=O)
    np.testing.assert_array_equal(pool, ref_pool)
    expect = (ref + f64(R, dtype)[perm]) + f64(O, dtype)[perm]
    np.testing.assert_array_equal(out[perm], expect)
    # a zero residual without the outer one is the plain conv
    z, _, _ = oracle.conv(case, out_dtype="f64", resid=np.zeros_like(case.x))
    np.testing.assert_array_equal(z, ref)
    # sequence-parallel branch: conv into zeros, then add gated output and hidden states
    G = synthetic._normal(rng, case.x.shape, 1.0, dtype)
    Hs = synthetic._normal(rng, case.x.shape, 1.0, dtype)
    sp = (oracle.conv(case, out_dtype="f64", resid=np.zeros_like(case.x))[0] + f64(G, dtype)) + f64(Hs, dtype)
    fused = oracle.conv(case, out_dtype="f64", resid=G, outer=Hs)[0]
    np.testing.assert_array_equal(fused, sp)


def test_fused_absum_counts_residual_terms():
    case = _mixed("f32", 1, 2300)
    _, _, ab = oracle.conv(case, out_dtype="f64", absum=True)
    R = np.full_like(case.x, -2.0)
    O = np.full_like(case.x, 0.5)
    _, _, ab2 = oracle.conv(case, out_dtype="f64", absum=True, resid=R, outer=O)
    np.testing.assert_array_equal(ab2, ab + 2.5)


def test_spec_token_indices_and_residuals():
    case = conv_case("fuse_spec", 2400, C=5, K=4, d=2, dtype="bf16", act="silu", w_std=0.4,
                     bias_std=0.2, num_slots=12, num_decodes=6, q=3, num_spec=2)
    acc = synthetic.num_accepted(2401, 6, 3)
    ref, ref_pool, _ = oracle.conv_spec(case, acc, out_dtype="f64")
    xp, perm = _scatter(replace(case, x=case.x[:case.num_decode_tokens]), 9, 2402)
    rng = np.random.default_rng(2403)
    R = synthetic._normal(rng, xp.shape, 1.0, "bf16")
    O = synthetic._normal(rng, xp.shape, 1.0, "bf16")
    out, pool, _ = oracle.conv_spec(case, acc, out_dtype="f64", x=xp, token_indices=perm,
                                    resid=R, outer=O)
    np.testing.assert_array_equal(pool, ref_pool)
    np.testing.assert_array_equal(out[perm], (ref + f64(R, "bf16")[perm]) + f64(O, "bf16")[perm])
    unused = np.setdiff1d(np.arange(xp.shape[0]), perm)
    assert not out[unused].any()
