"""GPU parity of the speculative rolling-buffer update (sc_conv_update_spec)
and of the non-speculative calls on a buffer widened for rollback, against the
CPU oracle.

Bar: state bit-exact always; outputs within 2 bf16 ulp (bf16) or 1e-5 relative
(fp32) of the oracle's float64 result, or within 2^-20 of the sum of |terms|.
A fully accepted chain of speculative steps must reproduce the one-shot GPU
prefill outputs bit for bit (same tap arithmetic on both paths)."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synthetic
from synthetic import conv_case
from tests._gpu import check_close, dev, host, run_conv_case, run_spec_case

pytestmark = pytest.mark.gpu

FLOOR = 2.0 ** -20


def spec_parity(case, acc, **kw):
    print(f"[gpu] spec {case.name} B={case.num_decodes} q={case.q} C={case.C} K={case.K} "
          f"d={case.d} S={case.S} {case.dtype} act={case.act} kw={kw}", flush=True)
    out, pool = run_spec_case(case, acc, **kw)
    ref, ref_pool, absum = oracle.conv_spec(case, acc, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, ref_pool, err_msg="state pool not bit-exact")
    frac = check_close(out, ref, absum, case.dtype, FLOOR)
    print(f"[gpu] spec {case.name}: ok (floor-only share {frac:.2e})", flush=True)
    return out, pool


def test_spec_128req_q4_shape():
    case = synthetic.spec_128req_q4()
    spec_parity(case, synthetic.num_accepted(77, case.num_decodes, case.q))


def test_spec_ple_dilated_shape():
    case = conv_case("ple_spec", 3101, C=8192, K=4, d=3, dtype="bf16", act="none",
                     w_std=0.05, bias_std=None, num_slots=512, num_decodes=96, q=4,
                     num_spec=3)
    spec_parity(case, synthetic.num_accepted(78, 96, 4))


@pytest.mark.parametrize("K,d,n,q,dtype,act", [
    (4, 1, 3, 4, "bf16", "silu"),
    (4, 2, 2, 3, "bf16", "none"),
    (4, 3, 4, 5, "bf16", "silu"),
    (3, 1, 2, 3, "bf16", "silu"),      # odd width: fp32 chain on bf16 data
    (2, 1, 4, 5, "f32", "silu"),
    (4, 1, 3, 4, "f32", "none"),
    (4, 1, 7, 8, "bf16", "silu"),      # q at the register path's maximum
    (4, 1, 12, 13, "bf16", "silu"),    # q beyond it: one-channel kernel
    (4, 1, 14, 5, "bf16", "none"),     # S = 17 beyond the LDS staging limit
    (4, 1, 4, 2, "bf16", "silu"),      # q shorter than num_spec + 1
    (5, 1, 2, 3, "bf16", "silu"),      # width outside the vector shapes
    (4, 4, 2, 3, "f32", "none"),
    (1, 1, 2, 2, "bf16", "none"),      # no history at all
])
def test_spec_shapes(K, d, n, q, dtype, act):
    case = conv_case("spec_shape", 3200 + K * 31 + d * 7 + n + q, C=2048 + 512, K=K, d=d,
                     dtype=dtype, act=act, w_std=0.4, bias_std=0.2, num_slots=48,
                     num_decodes=37, q=q, num_spec=n)
    spec_parity(case, synthetic.num_accepted(K + q, 37, q))


def test_spec_padding_clamping_and_ragged_channels():
    case = conv_case("spec_pad", 3301, C=1000, K=4, d=1, dtype="bf16", act="silu",
                     w_std=0.4, bias_std=0.2, num_slots=12, num_decodes=9, q=4,
                     num_spec=3)
    case.decode_slots[2] = -1
    case.decode_slots[5] = 12                  # out of range: padding row
    acc = np.array([0, -4, 4, 99, 1, 2, 3, 7, 1], np.int32)
    spec_parity(case, acc)
    spec_parity(case, acc, x_pad=24)           # strided token rows


def test_spec_unaligned_channels_use_one_channel_kernel():
    case = conv_case("spec_unaligned", 3302, C=1003, K=4, d=2, dtype="bf16", act="silu",
                     w_std=0.4, bias_std=0.2, num_slots=12, num_decodes=7, q=3,
                     num_spec=2)
    spec_parity(case, synthetic.num_accepted(5, 7, 3, lo=0, hi=5))


@pytest.mark.parametrize("K,d,n,dtype", [(4, 1, 3, "bf16"), (4, 3, 3, "bf16"),
                                         (4, 1, 2, "f32"), (3, 1, 3, "bf16")])
def test_spec_chain_matches_oracle_chain(K, d, n, dtype):
    """Prefill into a wide buffer, then speculative steps with random
    acceptance, GPU and oracle side by side; every step bit-exact in state."""
    import torch
    import stateful_causal_short_amd as scs
    q, B, steps = n + 1, 24, 6
    src = conv_case("spec_chain", 3400 + K + d + n, C=1536, K=K, d=d, dtype=dtype,
                    act="silu", w_std=0.4, bias_std=0.2, num_slots=40,
                    prefill_lens=list(range(3, 3 + B)), prefill_h_p=0.5, num_spec=n)
    g_out, g_pool = run_conv_case(src)
    r_out, r_pool, ab = oracle.conv(src, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(g_pool, r_pool)
    check_close(g_out, r_out, ab, dtype, FLOOR, what="prefill")
    rng = np.random.default_rng(K * 10 + n)
    slots = src.prefill_slots
    for s in range(steps):
        x = synthetic._normal(rng, (B * q, src.C), 1.0, dtype)
        acc = np.ones(B, np.int32) if s == 0 else rng.integers(1, q + 1, B).astype(np.int32)
        step = replace(src, x=x, num_decodes=B, q=q, decode_slots=slots, decode_h=None,
                       qsl_p=np.zeros(1, np.int32), prefill_slots=np.zeros(0, np.int32),
                       prefill_h=np.zeros(0, np.uint8), pool=r_pool, ckpt_grid=0,
                       cu_ckpt=None, ckpt_slots=None)
        g_out, g_pool = run_spec_case(step, acc, pool=g_pool)
        r_out, r_pool, ab = oracle.conv_spec(step, acc, out_dtype="f64", absum=True,
                                             pool=r_pool.copy())
        np.testing.assert_array_equal(g_pool, r_pool, err_msg=f"step {s}")
        check_close(g_out, r_out, ab, dtype, FLOOR, what=f"step {s}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("K,d,dtype", [(4, 1, "bf16"), (4, 3, "bf16"), (4, 1, "f32"),
                                       (3, 1, "bf16")])
def test_spec_all_accepted_chain_equals_one_shot_prefill(K, d, dtype):
    """Every draft accepted: the step outputs are the one-shot prefill's rows,
    bit for bit (one-shot on a narrow buffer, fast prefill path)."""
    n, L0, steps, B = 3, 7, 5, 6
    q = n + 1
    L = L0 + steps * q
    narrow = conv_case("spec_oneshot", 3500 + K + d, C=2048, K=K, d=d, dtype=dtype,
                       act="silu", w_std=0.4, bias_std=0.2, num_slots=B,
                       prefill_lens=[L] * B, prefill_h_all=0)
    one_out, _ = run_conv_case(narrow)
    H = (K - 1) * d
    wide_pool = np.zeros((B, narrow.C, H + n), narrow.pool.dtype)
    xs = narrow.x.reshape(B, L, narrow.C)
    pre = replace(narrow, x=np.ascontiguousarray(xs[:, :L0].reshape(B * L0, -1)),
                  qsl_p=np.arange(B + 1, dtype=np.int32) * L0, S=H + n)
    _, pool = run_conv_case(pre, pool=wide_pool)
    for s in range(steps):
        x = np.ascontiguousarray(xs[:, L0 + s * q:L0 + (s + 1) * q].reshape(B * q, -1))
        step = replace(narrow, x=x, num_decodes=B, q=q, decode_slots=narrow.prefill_slots,
                       qsl_p=np.zeros(1, np.int32), prefill_slots=np.zeros(0, np.int32),
                       prefill_h=np.zeros(0, np.uint8), S=H + n)
        acc = np.full(B, 1 if s == 0 else q, np.int32)
        out, pool = run_spec_case(step, acc, pool=pool)
        ref = one_out.reshape(B, L, -1)[:, L0 + s * q:L0 + (s + 1) * q].reshape(B * q, -1)
        np.testing.assert_array_equal(out, ref, err_msg=f"step {s}")


@pytest.mark.parametrize("q,d,dtype", [(1, 1, "bf16"), (2, 3, "bf16"), (4, 1, "f32"),
                                       (3, 2, "bf16")])
def test_wide_buffer_nonspec_calls(q, d, dtype):
    """Decode / update and varlen prefill (with checkpoints) on a buffer of
    H + 3 entries: window in the first H, the rest untouched."""
    case = conv_case("wide", 3600 + q + d, C=2560, K=4, d=d, dtype=dtype, act="silu",
                     w_std=0.4, bias_std=0.2, num_slots=160, num_decodes=33, q=q,
                     prefill_lens=[1, 2, 9, 40, 130, 77], prefill_h_p=0.5,
                     ckpt_grid=16 * d, num_spec=3)
    case.decode_h = (np.arange(33) % 4 != 1).astype(np.uint8)
    case.decode_slots[3] = -1
    print(f"[gpu] wide q={q} d={d} {dtype} S={case.S}", flush=True)
    out, pool = run_conv_case(case)
    ref, ref_pool, absum = oracle.conv(case, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, ref_pool, err_msg="state pool not bit-exact")
    check_close(out, ref, absum, dtype, FLOOR)


@pytest.mark.parametrize("n", [0, 1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("C", [1000, 2056])
def test_ds_register_path_every_buffer_length(n, C):
    """Width 4, no dilation, bf16, DS pool, S = 3 + n: the entries are
    transposed in registers. Speculative calls (counts out of range included,
    a padding slot) and plain calls on the same widened buffer, with channel
    counts that leave a workgroup's last lanes empty."""
    S = 3 + n
    rng = np.random.default_rng(3800 + 17 * n + C)
    for q in sorted({1, min(n + 1, S), S}):
        act = "silu" if (q + n) % 2 else "none"
        case = conv_case("spec_ds", 3800 + 31 * n + q + C, C=C, K=4, d=1, dtype="bf16",
                         act=act, w_std=0.4, bias_std=0.2, num_slots=64, num_decodes=29,
                         q=q, num_spec=n)
        case.decode_slots[5] = -1
        acc = rng.integers(-1, S + 3, size=29).astype(np.int32)
        spec_parity(case, acc)
        wide = conv_case("wide_ds", 3900 + 31 * n + q + C, C=C, K=4, d=1, dtype="bf16",
                         act=act, w_std=0.4, bias_std=0.2, num_slots=64, num_decodes=29,
                         q=q, num_spec=n)
        wide.decode_h = (np.arange(29) % 3 != 1).astype(np.uint8)
        wide.decode_slots[7] = -1
        out, pool = run_conv_case(wide)
        ref, ref_pool, absum = oracle.conv(wide, out_dtype="f64", absum=True)
        np.testing.assert_array_equal(pool, ref_pool, err_msg=f"wide q={q}: pool not bit-exact")
        check_close(out, ref, absum, "bf16", FLOOR)


def test_spec_zero_work_and_errors():
    import torch
    import stateful_causal_short_amd as scs
    C = 64
    x = torch.zeros((0, C), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((C, 4), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((4, C, 6), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(0, dtype=torch.int32, device="cuda")
    scs.sc_conv_update_spec(x, x.clone(), w, None, pool, idx, idx.clone(), q=4)
    xx = torch.zeros((8, C), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(scs.ScError):   # q = 8 drafts do not fit S = 6
        scs.sc_conv_update_spec(xx, xx.clone(), w, None, pool,
                                torch.zeros(1, dtype=torch.int32, device="cuda"),
                                torch.ones(1, dtype=torch.int32, device="cuda"), q=8)
    torch.cuda.synchronize()
    assert host(pool).sum() == 0
