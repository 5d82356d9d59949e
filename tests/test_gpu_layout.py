"""GPU parity of every depthwise call on an SD state pool ((num_slots, S, C):
the conv-state cache viewed transposed, `is_conv_state_dim_first` false) against
the CPU oracle on the same SD pool.

Bar: as for the DS pool — state bit-exact; outputs within 2 bf16 ulp (bf16) or
1e-5 relative (fp32) of the oracle, or within 2^-20 of the sum of |terms|."""
import numpy as np
import pytest

import oracle
import synthetic
from synthetic import as_sd, conv_case
from tests._gpu import check_close, run_conv_case, run_fused_case, run_spec_case

pytestmark = pytest.mark.gpu

FLOOR = 2.0 ** -20


def parity_sd(case, **kw):
    print(f"[gpu] sd {case.name} T={case.T} C={case.C} K={case.K} d={case.d} S={case.S} "
          f"{case.dtype} act={case.act} kw={kw}", flush=True)
    out, pool = run_conv_case(case, **kw)
    ref, ref_pool, ab = oracle.conv(case, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, ref_pool, err_msg="SD state pool not bit-exact")
    check_close(out, ref, ab, case.dtype, FLOOR)


@pytest.mark.parametrize("K,d,dtype,act,num_spec", [
    (4, 1, "bf16", "silu", 0),     # pair kernels
    (4, 3, "bf16", "none", 0),     # dilated (PLE shape)
    (2, 1, "bf16", "silu", 0),
    (4, 1, "f32", "silu", 0),      # fp32 register-window kernel
    (3, 1, "bf16", "silu", 0),
    (4, 2, "bf16", "silu", 3),     # wide rows (S = H + 3) on the fast kernels
    (5, 2, "bf16", "silu", 1),     # one-channel kernel
])
def test_sd_mixed_batch(K, d, dtype, act, num_spec):
    case = conv_case("sd_mixed", 6000 + K * 10 + d + num_spec, C=2560, K=K, d=d, dtype=dtype,
                     act=act, w_std=0.4, bias_std=0.2, num_slots=128, num_decodes=23, q=1,
                     prefill_lens=[1, 3, 8, 17, 40, 131], prefill_h_p=0.5, ckpt_grid=16 * d,
                     num_spec=num_spec)
    parity_sd(as_sd(case))


@pytest.mark.parametrize("q", [2, 4, 3])
def test_sd_update_lengths(q):
    case = conv_case("sd_upd", 6100 + q, C=4096, K=4, d=1, dtype="bf16", act="silu",
                     w_std=0.3, bias_std=0.1, num_slots=300, num_decodes=70, q=q)
    case.decode_h = (np.arange(70) % 5 != 2).astype(np.uint8)
    case.decode_slots[7] = -1
    parity_sd(as_sd(case))


def test_sd_unaligned_and_strided():
    case = conv_case("sd_unal", 6201, C=1003, K=4, d=3, dtype="bf16", act="none",
                     w_std=0.3, bias_std=None, num_slots=30, num_decodes=5,
                     prefill_lens=[2, 41], prefill_h_all=1, ckpt_grid=9)
    parity_sd(as_sd(case))
    case2 = conv_case("sd_strided", 6202, C=2048, K=4, d=1, dtype="bf16", act="silu",
                      w_std=0.3, bias_std=0.1, num_slots=40, num_decodes=9,
                      prefill_lens=[5, 60], prefill_h_all=1)
    parity_sd(as_sd(case2), x_pad=16)


@pytest.mark.parametrize("K,d,n,dtype", [(4, 1, 3, "bf16"), (4, 3, 3, "bf16"), (4, 1, 2, "f32"),
                                         (5, 1, 2, "bf16")])
def test_sd_speculative(K, d, n, dtype):
    q = n + 1
    case = as_sd(conv_case("sd_spec", 6300 + K + d + n, C=2048, K=K, d=d, dtype=dtype,
                           act="silu", w_std=0.4, bias_std=0.2, num_slots=80, num_decodes=33,
                           q=q, num_spec=n))
    acc = synthetic.num_accepted(6350 + n, 33, q, lo=0, hi=q + 2)
    print(f"[gpu] sd spec K={K} d={d} n={n} {dtype}", flush=True)
    out, pool = run_spec_case(case, acc)
    ref, ref_pool, ab = oracle.conv_spec(case, acc, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, ref_pool)
    check_close(out, ref, ab, dtype, FLOOR)


def test_sd_fused_ple_batch():
    case = as_sd(synthetic.ple_mixed_batch(C=2048, num_decodes=40, Bp=6, min_len=20, max_len=500,
                                   grid=64, num_slots=256))
    rng = np.random.default_rng(6401)
    n = case.T + 19
    perm = rng.permutation(n)[:case.T].astype(np.int32)
    xp = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    xp[perm] = case.x
    R = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    O = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    print("[gpu] sd fused PLE batch", flush=True)
    out, pool = run_fused_case(case, xp, perm, resid=R, outer=O)
    ref, ref_pool, ab = oracle.conv(case, out_dtype="f64", absum=True, x=xp, token_indices=perm,
                                    resid=R, outer=O)
    np.testing.assert_array_equal(pool, ref_pool)
    check_close(out[perm], ref[perm], ab, case.dtype, FLOOR)
