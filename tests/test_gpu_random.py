"""Seeded random parity sweep of the depthwise calls against the CPU oracle:
mixed decode + varlen prefill batches (lengths including 0), random width,
dilation, channel count (aligned or not), dtype, activation and bias, both state
layouts, buffers widened for speculative rollback, padding slots, checkpoints,
strided rows, and fused residuals with a row map. Every case stays inside the
calls' documented preconditions.

Bar: state bit-exact; outputs within 2 bf16 ulp (bf16) or 1e-5 relative (fp32)
of the oracle's float64 value, or within 2^-20 of the sum of |terms|."""
import numpy as np
import pytest

import oracle
import synthetic
from synthetic import conv_case
from tests._gpu import check_close, run_conv_case, run_fused_case

pytestmark = pytest.mark.gpu

FLOOR = 2.0 ** -20


def random_case(seed):
    rng = np.random.default_rng(seed)
    K = int(rng.choice([1, 2, 3, 4, 4, 4, 5]))
    d = int(rng.choice([1, 1, 2, 3]))
    H = (K - 1) * d
    C = int(rng.choice([8, 24, 256, 1000, 2056, 4096]))
    dtype = str(rng.choice(["bf16", "f32"]))
    act = str(rng.choice(["silu", "none"]))
    bias = None if rng.random() < 0.3 else 0.2
    nd = int(rng.choice([0, 1, 7]))
    q = int(rng.choice([1, 1, 2, 3, 4]))
    lens = [int(v) for v in rng.integers(0, 71, size=int(rng.choice([0, 1, 5])))]
    if nd == 0 and not lens:
        lens = [int(rng.integers(1, 40))]
    grid = 0 if (H == 0 or rng.random() < 0.5) else int(H * rng.choice([1, 2, 3]))
    num_spec = int(rng.choice([0, 0, 2]))
    need = nd + len(lens) + (sum(n // grid for n in lens) if grid else 0)
    case = conv_case("random", seed, C=C, K=K, d=d, dtype=dtype, act=act, w_std=0.4,
                     bias_std=bias, num_slots=need + 6, num_decodes=nd, q=q, prefill_lens=lens,
                     prefill_h_p=0.5, ckpt_grid=grid, num_spec=num_spec)
    if nd and rng.random() < 0.5:
        case.decode_h = (rng.random(nd) < 0.7).astype(np.uint8)
    if len(lens) > 1 and rng.random() < 0.4:
        case.prefill_slots[int(rng.integers(0, len(lens)))] = -1      # a padding row
    if rng.random() < 0.4:
        case = synthetic.as_sd(case)
    return case, rng


@pytest.mark.parametrize("seed", range(120))
def test_random_depthwise_batches(seed):
    case, rng = random_case(0x7A0000 + seed)
    mode = str(rng.choice(["plain", "plain", "strided", "fused"]))
    print(f"[gpu] random seed={seed} mode={mode} T={case.T} C={case.C} K={case.K} d={case.d} "
          f"S={case.S} {case.dtype} act={case.act} bias={case.bias is not None} "
          f"decodes={case.num_decodes}x{case.q} lens={list(np.diff(case.qsl_p))} "
          f"grid={case.ckpt_grid} layout={case.layout}", flush=True)
    if mode == "fused":
        n = case.T + 5
        perm = rng.permutation(n)[:case.T].astype(np.int32)
        xp = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
        xp[perm] = case.x
        R = synthetic._normal(rng, (n, case.C), 1.0, case.dtype)
        O = synthetic._normal(rng, (n, case.C), 1.0, case.dtype) if rng.random() < 0.5 else None
        out, pool = run_fused_case(case, xp, perm, resid=R, outer=O)
        ref, rpool, ab = oracle.conv(case, out_dtype="f64", absum=True, x=xp,
                                     token_indices=perm, resid=R, outer=O)
        np.testing.assert_array_equal(pool, rpool, err_msg="state pool not bit-exact")
        check_close(out[perm], ref[perm], ab, case.dtype, FLOOR, what="fused out")
        unused = np.setdiff1d(np.arange(n), perm)
        np.testing.assert_array_equal(out[unused], R[unused])
        return
    out, pool = run_conv_case(case, x_pad=16 if mode == "strided" else 0)
    ref, rpool, ab = oracle.conv(case, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, rpool, err_msg="state pool not bit-exact")
    check_close(out, ref, ab, case.dtype, FLOOR)


# ---------------------------------------------------------------------------
# speculative update: uniform draft count and one count per request
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(64))
def test_random_speculative_batches(seed):
    from tests._gpu import run_spec_case
    from tests.test_gpu_spec_varlen import run_varlen
    rng = np.random.default_rng(0x7B0000 + seed)
    K = int(rng.choice([2, 3, 4, 4, 5]))
    d = int(rng.choice([1, 1, 2, 3]))
    n = int(rng.integers(1, 6))
    S = (K - 1) * d + n
    C = int(rng.choice([8, 24, 256, 1000, 2056]))
    dtype = str(rng.choice(["bf16", "f32"]))
    act = str(rng.choice(["silu", "none"]))
    B = int(rng.integers(1, 20))
    varlen = bool(rng.random() < 0.5)
    sd = bool(rng.random() < 0.4)
    print(f"[gpu] random spec seed={seed} K={K} d={d} S={S} C={C} {dtype} act={act} B={B} "
          f"varlen={varlen} sd={sd}", flush=True)
    if varlen:
        max_q = int(rng.integers(1, S + 1))
        case, qsl = synthetic.spec_varlen_case("rspec", 0x7B0000 + seed, C=C, K=K, d=d,
                                               dtype=dtype, act=act, w_std=0.4, bias_std=0.2,
                                               num_slots=B + 5, B=B, num_spec=n, q_max=max_q)
    else:
        q = int(rng.integers(1, S + 1))
        case = conv_case("rspec", 0x7B0000 + seed, C=C, K=K, d=d, dtype=dtype, act=act,
                         w_std=0.4, bias_std=0.2, num_slots=B + 5, num_decodes=B, q=q,
                         num_spec=n)
    if B > 2 and rng.random() < 0.5:
        case.decode_slots[int(rng.integers(0, B))] = -1
    if sd:
        case = synthetic.as_sd(case)
    acc = rng.integers(-1, S + 3, size=B).astype(np.int32)   # includes out-of-range counts
    fused = bool(rng.random() < 0.35)
    T = int(qsl[-1]) if varlen else B * case.q
    fz, perm = {}, None
    if fused:
        n_phys = T + 3
        perm = rng.permutation(n_phys)[:T].astype(np.int32)
        xp = synthetic._normal(rng, (n_phys, C), 1.0, dtype)
        xp[perm] = case.x[:T]
        R = synthetic._normal(rng, (n_phys, C), 1.0, dtype)
        O = synthetic._normal(rng, (n_phys, C), 1.0, dtype) if rng.random() < 0.5 else None
        fz = dict(x=xp, token_indices=perm, resid=R, outer=O)
    print(f"[gpu]   fused={fused}", flush=True)
    if varlen:
        max_q = max(int(np.diff(qsl).max()), 1)
        out, pool = run_varlen(case, acc, qsl, max_q, **fz)
        ref, rpool, ab = oracle.conv_spec_varlen(case, acc, qsl, out_dtype="f64", absum=True,
                                                 **fz)
    elif fused:
        out, pool = run_fused_case(case, fz["x"], perm, resid=fz["resid"], outer=fz["outer"],
                                   num_accepted=acc)
        ref, rpool, ab = oracle.conv_spec(case, acc, out_dtype="f64", absum=True, **fz)
    else:
        out, pool = run_spec_case(case, acc)
        ref, rpool, ab = oracle.conv_spec(case, acc, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, rpool, err_msg="state pool not bit-exact")
    if fused:
        # rows of skipped requests keep their residual in both (the oracle starts its
        # output from zeros and adds the residual only where it computes)
        live = np.zeros(T, bool)
        if varlen:
            for r in range(B):
                q_r = int(qsl[r + 1] - qsl[r])
                if 0 < q_r <= S:
                    live[int(qsl[r]):int(qsl[r + 1])] = True
        else:
            live[:] = True
        check_close(out[perm[live]], ref[perm[live]], ab[live], case.dtype, FLOOR, what="fused out")
        untouched = np.setdiff1d(np.arange(out.shape[0]), perm[live])
        np.testing.assert_array_equal(out[untouched], fz["resid"][untouched])
    else:
        check_close(out, ref, ab, case.dtype, FLOOR)


# ---------------------------------------------------------------------------
# CCA: head counts, head size and both kernel widths (MFMA and one-thread paths)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(40))
def test_random_cca_batches(seed):
    from tests._gpu import cca_floor_rel, run_cca_case
    rng = np.random.default_rng(0x7C0000 + seed)
    nq, nkv = [(4, 2), (2, 2), (8, 2), (16, 4), (4, 1)][int(rng.integers(0, 5))]
    hd = int(rng.choice([16, 32, 128, 128]))
    t0 = int(rng.choice([1, 2, 2, 3]))
    t1 = int(rng.choice([1, 2, 2, 3]))
    nd = int(rng.choice([0, 3, 40]))
    lens = [int(v) for v in rng.integers(0, 90, size=int(rng.choice([0, 2, 6])))]
    if nd == 0 and sum(lens) == 0:
        lens = [int(rng.integers(1, 60))]
    case = synthetic.cca_case("rcca", 0x7C0000 + seed, nq=nq, nkv=nkv, hd=hd, t0=t0, t1=t1,
                              num_decodes=nd, prefill_lens=lens,
                              num_slots=nd + len(lens) + 4)
    no_init = bool(rng.random() < 0.3)
    print(f"[gpu] random cca seed={seed} nq={nq} nkv={nkv} hd={hd} t0={t0} t1={t1} "
          f"decodes={nd} lens={lens} no_delayed_init={no_init}", flush=True)
    out, cs, ds = run_cca_case(case, no_delayed_init=no_init)
    from dataclasses import replace
    ocase = replace(case, delayed_init=np.zeros_like(case.delayed_init)) if no_init else case
    nd_chain, al = [], []
    ref, rcs, rds, ab = oracle.cca(ocase, out_dtype="f64", absum=True, chain_diff=nd_chain,
                                   allow=al)
    np.testing.assert_array_equal(cs, rcs, err_msg="conv state not bit-exact")
    np.testing.assert_array_equal(ds, rds, err_msg="delayed state not bit-exact")
    C = case.C
    np.testing.assert_array_equal(synthetic.bf16_to_f32(out[:, C:]).astype(np.float64),
                                  ref[:, C:], err_msg="value half not bit-exact")
    check_close(out[:, :C], ref[:, :C], ab[:, :C], "bf16", cca_floor_rel(case), what="q/k",
                allow=al[0][:, :C])
    print(f"[gpu] random cca seed={seed}: ok (depthwise values an fp32 chain rounds "
          f"elsewhere: {nd_chain[0]})", flush=True)


@pytest.mark.parametrize("seed", range(8))
def test_random_large_depthwise_batches(seed):
    """Wide rows and long requests: 8192 channels, up to 3000 tokens a request,
    the vector kernels' shapes (width 4 or 2, dilation 1-3), either layout."""
    rng = np.random.default_rng(0x7D0000 + seed)
    K, d = [(4, 1), (4, 2), (4, 3), (2, 1)][int(rng.integers(0, 4))]
    H = (K - 1) * d
    lens = [int(v) for v in rng.integers(0, 3001, size=int(rng.integers(1, 7)))]
    nd = int(rng.choice([0, 64]))
    q = int(rng.choice([1, 2, 4]))
    grid = 0 if rng.random() < 0.5 else int(max(H, 1) * rng.choice([64, 128]))
    need = nd + len(lens) + (sum(n // grid for n in lens) if grid else 0)
    case = conv_case("rlarge", 0x7D0000 + seed, C=8192, K=K, d=d, dtype="bf16",
                     act=str(rng.choice(["silu", "none"])), w_std=0.25, bias_std=0.1,
                     num_slots=need + 4, num_decodes=nd, q=q, prefill_lens=lens,
                     prefill_h_p=0.5, ckpt_grid=grid)
    if rng.random() < 0.5:
        case = synthetic.as_sd(case)
    print(f"[gpu] random large seed={seed} T={case.T} K={K} d={d} decodes={nd}x{q} "
          f"lens={lens} grid={grid} layout={case.layout}", flush=True)
    out, pool = run_conv_case(case)
    ref, rpool, ab = oracle.conv(case, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, rpool, err_msg="state pool not bit-exact")
    check_close(out, ref, ab, case.dtype, FLOOR)
