"""GPU parity of the speculative update with a draft count per request
(sc_conv_update_spec_varlen; GDN page, _spec_forward's per-sequence loop over
spec_query_start_loc) against the CPU oracle.

Bar: state bit-exact always; outputs within 2 bf16 ulp (bf16) or 1e-5 relative
(fp32) of the oracle's float64 result, or within 2^-20 of the sum of |terms|.
Requests with no drafts leave their rows and slot untouched; so do requests
that break the max_query_len bound. With every count equal, the call matches
the uniform speculative call bit for bit."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synthetic
from tests._gpu import check_close, dev, host, run_spec_case

pytestmark = pytest.mark.gpu

FLOOR = 2.0 ** -20


def run_varlen(case, acc, qsl, max_q, *, pool=None, x=None, token_indices=None, resid=None,
               outer=None, x_pad=0):
    """Runs the varlen speculative call; out starts as `resid` (accumulate) or
    zeros. Returns (out, pool_after) as NumPy arrays."""
    import torch
    import stateful_causal_short_amd as scs
    x = case.x if x is None else x
    T, C = x.shape
    if x_pad:
        xs = np.zeros((T, C + x_pad), x.dtype)
        xs[:, :C] = x
        xd = dev(xs)[:, :C]
        o0 = np.zeros((T, C + x_pad), x.dtype)
        if resid is not None:
            o0[:, :C] = resid
        od = dev(o0)[:, :C]
    else:
        xd = dev(x)
        od = dev(resid if resid is not None else np.zeros((T, C), x.dtype))
    pd = dev(case.pool if pool is None else pool)
    scs.sc_conv_update_spec_varlen(
        xd, od, dev(case.w), None if case.bias is None else dev(case.bias), pd,
        dev(np.asarray(case.decode_slots, np.int32)), dev(np.asarray(acc, np.int32)),
        dev(np.asarray(qsl, np.int32)), max_query_len=max_q, dilation=case.d,
        activation=case.act, state_layout=case.layout,
        token_indices=None if token_indices is None else dev(np.asarray(token_indices, np.int32)),
        accumulate=resid is not None, outer_residual=None if outer is None else dev(outer))
    torch.cuda.synchronize()
    return host(od.contiguous()), host(pd)


def varlen_parity(case, acc, qsl, max_q=None, **kw):
    qs = np.diff(qsl)
    max_q = int(qs.max()) if max_q is None else max_q
    print(f"[gpu] spec varlen {case.name} B={case.num_decodes} T={int(qsl[-1])} C={case.C} "
          f"K={case.K} d={case.d} S={case.S} {case.dtype} act={case.act} max_q={max_q} "
          f"layout={case.layout} kw={sorted(kw)}", flush=True)
    out, pool = run_varlen(case, acc, qsl, max_q, **kw)
    ref, ref_pool, absum = oracle.conv_spec_varlen(case, acc, qsl, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, ref_pool, err_msg="state pool not bit-exact")
    frac = check_close(out, ref, absum, case.dtype, FLOOR)
    print(f"[gpu] spec varlen {case.name}: ok (floor-only share {frac:.2e})", flush=True)
    return out, pool


@pytest.mark.parametrize("layout", ["ds", "sd"])
def test_spec_varlen_128_requests_8192_channels(layout):
    case, qsl = synthetic.spec_varlen_128req()
    if layout == "sd":
        case = synthetic.as_sd(case)
    acc = np.minimum(synthetic.num_accepted(91, case.num_decodes, 4), np.maximum(np.diff(qsl), 1))
    varlen_parity(case, acc, qsl)


@pytest.mark.parametrize("K,d,n,dtype,act,C,q_max", [
    (4, 1, 3, "bf16", "silu", 2560, 4),
    (4, 3, 3, "bf16", "none", 2560, 4),     # the PLE dilated shape
    (4, 2, 2, "f32", "silu", 2560, 3),
    (3, 1, 2, "bf16", "silu", 2560, 3),     # odd width: fp32 chain on bf16 data
    (2, 1, 4, "bf16", "silu", 2560, 5),
    (4, 1, 12, "bf16", "silu", 2560, 13),   # counts beyond the register path: one-channel kernel
    (5, 1, 2, "bf16", "silu", 2560, 3),     # width outside the vector shapes
    (4, 1, 3, "bf16", "silu", 1003, 4),     # unaligned channel count
    (4, 1, 14, "bf16", "none", 2048, 6),    # S = 17 beyond the LDS staging limit
])
def test_spec_varlen_shapes(K, d, n, dtype, act, C, q_max):
    case, qsl = synthetic.spec_varlen_case("spec_vl", 5100 + K * 31 + d * 7 + n, C=C, K=K, d=d,
                                           dtype=dtype, act=act, w_std=0.4, bias_std=0.2,
                                           num_slots=64, B=41, num_spec=n, q_max=q_max)
    acc = synthetic.num_accepted(K + n, 41, q_max, lo=0, hi=q_max + 2)
    varlen_parity(case, acc, qsl)


def test_spec_varlen_padding_strides_and_zero_counts():
    qs = [0, 3, 0, 0, 4, 1, 2, 0, 4, 4, 1]
    case, qsl = synthetic.spec_varlen_case("spec_vl_pad", 5301, C=1536, K=4, d=1, dtype="bf16",
                                           act="silu", w_std=0.4, bias_std=0.2, num_slots=16,
                                           B=len(qs), num_spec=3, q_lens=qs)
    case.decode_slots[4] = -1
    case.decode_slots[8] = 16                  # out of range: padding row
    acc = np.array([1, 3, 2, 0, 9, 1, 2, 4, 3, -1, 1], np.int32)
    varlen_parity(case, acc, qsl)
    varlen_parity(case, acc, qsl, x_pad=40)    # strided token rows
    varlen_parity(case, acc, qsl, max_q=6)     # a looser bound, still <= S


def test_spec_varlen_requests_beyond_the_bound_are_skipped():
    qs = np.array([2, 4, 1, 3, 4, 2], np.int64)
    case, qsl = synthetic.spec_varlen_case("spec_vl_bound", 5401, C=2048, K=4, d=1,
                                           dtype="bf16", act="silu", w_std=0.4, bias_std=0.2,
                                           num_slots=12, B=6, num_spec=3, q_lens=qs)
    acc = np.array([1, 2, 1, 3, 4, 2], np.int32)
    out, pool = run_varlen(case, acc, qsl, 3)      # requests 1 and 4 draft 4 > 3
    ref, ref_pool, ab = oracle.conv_spec_varlen(case, acc, qsl, out_dtype="f64", absum=True)
    for r in range(6):
        rows = slice(int(qsl[r]), int(qsl[r + 1]))
        slot = int(case.decode_slots[r])
        if qs[r] > 3:
            np.testing.assert_array_equal(out[rows], 0)
            np.testing.assert_array_equal(pool[slot], case.pool[slot])
        else:
            np.testing.assert_array_equal(pool[slot], ref_pool[slot])
            check_close(out[rows], ref[rows], ab[rows], "bf16", FLOOR, what=f"request {r}")


def test_spec_varlen_equal_counts_match_uniform_call():
    case = synthetic.conv_case("spec_vl_eq", 5501, C=4096, K=4, d=1, dtype="bf16", act="silu",
                               w_std=0.4, bias_std=0.2, num_slots=64, num_decodes=40, q=4,
                               num_spec=3)
    acc = synthetic.num_accepted(55, 40, 4)
    qsl = np.arange(41, dtype=np.int32) * 4
    o1, p1 = run_spec_case(case, acc)
    o2, p2 = run_varlen(case, acc, qsl, 4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1, p2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_spec_varlen_chain_matches_oracle_chain(dtype):
    """Steps with per-request counts in {0 .. num_spec + 1} and random
    acceptance, GPU and oracle side by side; every step bit-exact in state."""
    n, B, steps = 3, 30, 6
    case, _ = synthetic.spec_varlen_case("spec_vl_chain", 5601, C=1536, K=4, d=1, dtype=dtype,
                                         act="silu", w_std=0.4, bias_std=0.2, num_slots=48,
                                         B=B, num_spec=n)
    g_pool = case.pool.copy()
    r_pool = case.pool.copy()
    rng = np.random.default_rng(5602)
    for s in range(steps):
        qs = rng.integers(0, n + 2, B)
        qsl = np.zeros(B + 1, np.int32)
        qsl[1:] = np.cumsum(qs)
        x = synthetic._normal(rng, (int(qsl[-1]), case.C), 1.0, dtype)
        acc = rng.integers(1, n + 2, B).astype(np.int32)
        step = replace(case, x=x)
        g_out, g_pool = run_varlen(step, acc, qsl, n + 1, pool=g_pool)
        r_out, r_pool, ab = oracle.conv_spec_varlen(step, acc, qsl, out_dtype="f64",
                                                    absum=True, pool=r_pool.copy())
        np.testing.assert_array_equal(g_pool, r_pool, err_msg=f"step {s}")
        check_close(g_out, r_out, ab, dtype, FLOOR, what=f"step {s}")


@pytest.mark.parametrize("layout", ["ds", "sd"])
def test_spec_varlen_fused_residuals_and_row_map(layout):
    qs = [3, 0, 4, 1, 4, 2, 0, 4, 3, 1, 2, 4]
    case, qsl = synthetic.spec_varlen_case("spec_vl_fuse", 5701, C=2048, K=4, d=3, dtype="bf16",
                                           act="none", w_std=0.05, bias_std=None, num_slots=24,
                                           B=len(qs), num_spec=3, q_lens=qs)
    if layout == "sd":
        case = synthetic.as_sd(case)
    T = int(qsl[-1])
    rng = np.random.default_rng(5702)
    n = T + 9
    perm = rng.permutation(n)[:T].astype(np.int32)
    xp = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    xp[perm] = case.x
    R = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    O = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
    acc = synthetic.num_accepted(57, len(qs), 4)
    print(f"[gpu] spec varlen fused {layout} T={T} C={case.C}", flush=True)
    out, pool = run_varlen(case, acc, qsl, 4, x=xp, token_indices=perm, resid=R, outer=O)
    ref, rpool, ab = oracle.conv_spec_varlen(case, acc, qsl, out_dtype="f64", absum=True, x=xp,
                                             token_indices=perm, resid=R, outer=O)
    np.testing.assert_array_equal(pool, rpool, err_msg="state pool not bit-exact")
    check_close(out[perm], ref[perm], ab, case.dtype, FLOOR, what="fused out")
    unused = np.setdiff1d(np.arange(n), perm)
    np.testing.assert_array_equal(out[unused], R[unused], err_msg="unreferenced rows changed")


def test_spec_varlen_zero_work_and_errors():
    import torch
    import stateful_causal_short_amd as scs
    case, qsl = synthetic.spec_varlen_case("spec_vl_err", 5801, C=64, K=4, d=1, dtype="bf16",
                                           act="silu", w_std=0.4, bias_std=0.2, num_slots=8,
                                           B=3, num_spec=3, q_lens=[0, 0, 0])
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    w = dev(case.w)
    pool = dev(case.pool)
    slots = dev(np.asarray(case.decode_slots, np.int32))
    acc = dev(np.ones(3, np.int32))
    q = dev(np.asarray(qsl, np.int32))
    scs.sc_conv_update_spec_varlen(x, torch.zeros_like(x), w, None, pool, slots, acc, q,
                                   max_query_len=4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(pool), case.pool)
    x1 = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(scs.ScError, match="SC_ERR_INVALID_ARG"):
        scs.sc_conv_update_spec_varlen(x1, torch.zeros_like(x1), w, None, pool, slots, acc, q,
                                       max_query_len=7)     # 7 drafts do not fit S = 6
