"""GPU parity of the fused calls (PLE residual accumulation, outer residual,
logical-to-physical row map) against the CPU oracle.

Bar: state bit-exact; outputs at mapped rows within 2 bf16 ulp (bf16) or 1e-5
relative (fp32) of the oracle's float64 value, or within 2^-20 of the sum of
|terms| (which now includes |residual| and |outer residual|); physical rows
no call references are left exactly as they were."""
import numpy as np
import pytest

import oracle
import synthetic
from synthetic import conv_case
from tests._gpu import check_close, run_fused_case

pytestmark = pytest.mark.gpu

FLOOR = 2.0 ** -20


def scatter(case, extra, seed, rows=None):
    rng = np.random.default_rng(seed)
    T = case.T if rows is None else rows
    n = T + extra
    perm = rng.permutation(n)[:T].astype(np.int32)
    xp = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    xp[perm] = case.x[:T]
    R = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    O = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    return xp, perm, R, O


def fused_parity(case, xp, perm, R, O, *, accumulate=True, outer=True, num_accepted=None,
                 pool=None):
    print(f"[gpu] fused {case.name} T={case.T} C={case.C} K={case.K} d={case.d} "
          f"S={case.S} {case.dtype} acc={accumulate} outer={outer} "
          f"spec={num_accepted is not None}", flush=True)
    resid = R if accumulate else None
    oo = O if outer else None
    out, gpool = run_fused_case(case, xp, perm, resid=resid, outer=oo, pool=pool,
                                num_accepted=num_accepted)
    if num_accepted is not None:
        ref, rpool, ab = oracle.conv_spec(case, num_accepted, out_dtype="f64", absum=True,
                                          x=xp, token_indices=perm, resid=resid, outer=oo,
                                          pool=None if pool is None else pool.copy())
    else:
        ref, rpool, ab = oracle.conv(case, out_dtype="f64", absum=True, x=xp,
                                     token_indices=perm, resid=resid, outer=oo,
                                     pool=None if pool is None else pool.copy())
    np.testing.assert_array_equal(gpool, rpool, err_msg="state pool not bit-exact")
    frac = check_close(out[perm], ref[perm], ab, case.dtype, FLOOR, what="fused out")
    unused = np.setdiff1d(np.arange(xp.shape[0]), perm)
    init = R if accumulate else np.zeros_like(R)
    np.testing.assert_array_equal(out[unused], init[unused], err_msg="unreferenced rows changed")
    print(f"[gpu] fused {case.name}: ok (floor-only share {frac:.2e})", flush=True)


def test_ple_mixed_batch_fused():
    # the PLE shape: width 4, dilation 3, no bias or activation, decodes then
    # varlen prefills with checkpoints, gated output += conv + hidden states
    case = synthetic.ple_mixed_batch(C=2048, num_decodes=40, Bp=6, min_len=20, max_len=700,
                             grid=64, num_slots=256)
    xp, perm, R, O = scatter(case, 37, 4001)
    fused_parity(case, xp, perm, R, O)


@pytest.mark.parametrize("dtype,K,d,act,acc,outer", [
    ("bf16", 4, 1, "silu", True, False),
    ("bf16", 4, 1, "silu", False, True),
    ("bf16", 4, 2, "none", False, False),    # row map only
    ("bf16", 2, 1, "silu", True, True),
    ("bf16", 3, 1, "silu", True, True),      # odd width: one-channel kernel
    ("f32", 4, 1, "none", True, True),       # fp32: one-channel kernel
])
def test_fused_variants(dtype, K, d, act, acc, outer):
    case = conv_case("fused_var", 4100 + K * 7 + d, C=1536, K=K, d=d, dtype=dtype, act=act,
                     w_std=0.4, bias_std=0.2, num_slots=64, num_decodes=9, q=2,
                     prefill_lens=[1, 5, 16, 33, 70], prefill_h_p=0.5, ckpt_grid=16 * d)
    xp, perm, R, O = scatter(case, 13, 4200 + K)
    fused_parity(case, xp, perm, R, O, accumulate=acc, outer=outer)


@pytest.mark.parametrize("q", [1, 4])
def test_fused_decode_shapes(q):
    case = conv_case("fused_dec", 4300 + q, C=4096, K=4, d=1, dtype="bf16", act="silu",
                     w_std=0.3, bias_std=0.1, num_slots=300, num_decodes=130, q=q)
    xp, perm, R, O = scatter(case, 50, 4310 + q)
    fused_parity(case, xp, perm, R, O)


def test_fused_unaligned_channels():
    case = conv_case("fused_unal", 4401, C=1004, K=4, d=3, dtype="bf16", act="none",
                     w_std=0.3, bias_std=None, num_slots=30, num_decodes=5,
                     prefill_lens=[3, 40], prefill_h_all=1)
    xp, perm, R, O = scatter(case, 7, 4402)
    fused_parity(case, xp, perm, R, O)


@pytest.mark.parametrize("K,d,n,dtype", [(4, 1, 3, "bf16"), (4, 3, 3, "bf16"), (5, 1, 2, "bf16"),
                                         (4, 1, 2, "f32")])
def test_fused_speculative(K, d, n, dtype):
    q = n + 1
    case = conv_case("fused_spec", 4500 + K + d + n, C=2048, K=K, d=d, dtype=dtype, act="silu",
                     w_std=0.4, bias_std=0.2, num_slots=80, num_decodes=33, q=q, num_spec=n)
    xp, perm, R, O = scatter(case, 21, 4510 + K, rows=case.num_decode_tokens)
    fused_parity(case, xp, perm, R, O, num_accepted=synthetic.num_accepted(4520, 33, q))


def test_fused_wide_buffer_update():
    case = conv_case("fused_wide", 4601, C=2048, K=4, d=1, dtype="bf16", act="silu",
                     w_std=0.4, bias_std=0.2, num_slots=90, num_decodes=41, q=2,
                     prefill_lens=[3, 50], prefill_h_p=0.5, num_spec=3)
    xp, perm, R, O = scatter(case, 9, 4602)
    fused_parity(case, xp, perm, R, O)
