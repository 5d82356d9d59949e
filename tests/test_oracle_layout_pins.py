"""Pins for the oracle's SD state layout ((num_slots, S, C): the conv-state
cache viewed transposed when it is not dim-first; GDN and PLE pages,
`is_conv_state_dim_first`). The DS layout ((num_slots, C, S)) is pinned
elsewhere against library convolutions; here every call on an SD pool must
give the same outputs, and the same pool up to the transposition, as the
call on the DS pool holding the same values."""
import numpy as np
import pytest

import oracle
import synthetic
from synthetic import as_sd, conv_case


def sd_to_ds(pool):
    return np.ascontiguousarray(pool.transpose(0, 2, 1))


@pytest.mark.parametrize("d,num_spec,dtype", [(1, 0, "bf16"), (3, 0, "bf16"), (2, 3, "f32"),
                                              (1, 2, "bf16")])
def test_sd_equals_ds_transposed(d, num_spec, dtype):
    case = conv_case("sd", 5000 + d + num_spec, C=7, K=4, d=d, dtype=dtype, act="silu",
                     w_std=0.4, bias_std=0.2, num_slots=48, num_decodes=6, q=2,
                     prefill_lens=[1, 2, 9, 20, 41], prefill_h_p=0.5, ckpt_grid=8 * d,
                     num_spec=num_spec)
    out_ds, pool_ds, ab_ds = oracle.conv(case, out_dtype="f64", absum=True)
    sd = as_sd(case)
    assert sd.pool.shape == (48, case.S, 7)
    out_sd, pool_sd, ab_sd = oracle.conv(sd, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(out_sd, out_ds)
    np.testing.assert_array_equal(ab_sd, ab_ds)
    np.testing.assert_array_equal(sd_to_ds(pool_sd), pool_ds)


@pytest.mark.parametrize("K,d,n", [(4, 1, 3), (4, 2, 2), (3, 1, 4)])
def test_sd_speculative_equals_ds(K, d, n):
    case = conv_case("sd_spec", 5100 + K + d + n, C=5, K=K, d=d, dtype="bf16", act="silu",
                     w_std=0.4, bias_std=0.2, num_slots=20, num_decodes=9, q=n + 1, num_spec=n)
    acc = synthetic.num_accepted(5150 + n, 9, n + 1, lo=0, hi=n + 3)
    out_ds, pool_ds, _ = oracle.conv_spec(case, acc, out_dtype="f64")
    out_sd, pool_sd, _ = oracle.conv_spec(as_sd(case), acc, out_dtype="f64")
    np.testing.assert_array_equal(out_sd, out_ds)
    np.testing.assert_array_equal(sd_to_ds(pool_sd), pool_ds)
