"""GPU parity of the depthwise stateful conv (sc_conv_prefill_varlen,
sc_conv_update) and of the state row copies, against the CPU oracle.

Bar: state bit-exact always; outputs within 2 bf16 ulp (bf16) or 1e-5 relative
(fp32) of the oracle's float64 result, or within 2^-20 of the sum of |terms|
(the fp32 accumulation bound for <= 9 terms, only reached where the sum
cancels)."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synthetic
from synthetic import conv_case
from tests._gpu import check_close, dev, host, run_conv_case

pytestmark = pytest.mark.gpu

FLOOR = 2.0 ** -20


def parity(case, **kw):
    """Every output row and the whole state pool against the oracle."""
    print(f"[gpu] {case.name} T={case.T} C={case.C} K={case.K} d={case.d} "
          f"{case.dtype} act={case.act} kw={kw}", flush=True)
    out, pool = run_conv_case(case, **kw)
    ref, ref_pool, absum = oracle.conv(case, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(pool, ref_pool, err_msg="state pool not bit-exact")
    frac = check_close(out, ref, absum, case.dtype, FLOOR)
    print(f"[gpu] {case.name}: ok (floor-only share {frac:.2e})", flush=True)
    return out, pool


# ----------------------------------------------------------------------------
# the five workload shapes (CCA is in test_gpu_cca.py)
# ----------------------------------------------------------------------------
def test_single_sequence_64ch_f32():
    parity(synthetic.single_seq_64ch())


def test_varlen_prefill_small_ragged():
    parity(synthetic.varlen_prefill_8seq(C=512, B=8, max_len=300))


def test_varlen_prefill_8seq_full():
    parity(synthetic.varlen_prefill_8seq())


def test_decode_512req_full():
    parity(synthetic.decode_512req())


def test_update_128req_q4_full():
    parity(synthetic.update_128req_q4())


def test_ple_mixed_small_with_checkpoints():
    parity(synthetic.ple_mixed_batch(C=512, num_decodes=16, Bp=6, min_len=5, max_len=700,
                             grid=64, num_slots=128))


def test_ple_mixed_full():
    parity(synthetic.ple_mixed_batch())


# ----------------------------------------------------------------------------
# edge cases
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("d", [1, 3])
def test_chunk_edges_and_short_requests(d):
    # around multiples of the one-pass chunk lengths (12 for H <= 4, 16 for H = 9)
    lens = [1, 2, 3, 8, 9, 10, 11, 12, 13, 15, 16, 17, 23, 24, 25, 31, 32, 33, 35, 36, 37,
            47, 48, 49, 63, 64, 65, 127, 128, 129, 200]
    case = conv_case("edges", 500 + d, C=256, K=4, d=d, dtype="bf16", act="silu",
                     w_std=0.25, bias_std=0.1, num_slots=128, prefill_lens=lens,
                     prefill_h_p=0.5, ckpt_grid=max(16, 3 * d))
    parity(case)


@pytest.mark.parametrize("B", [63, 64, 65, 129, 256, 1000, 4095, 4096, 4097, 16129])
@pytest.mark.parametrize("dtype,d", [("bf16", 1), ("bf16", 3), ("f32", 1)])
def test_many_prefills_request_lookup(B, dtype, d):
    # batches of B short prefills (zero-length ones included): the chunk ->
    # request lookup takes one round of loads below 64 requests, two for
    # 64 <= B <= 4096 and counts every entry above; the bf16 prefill kernel
    # and the fp32 one resolve it
    rng = np.random.default_rng(7000 + B)
    lens = rng.choice([0, 1, 2, 3, 7, 8, 9, 12, 13, 16, 17, 25], size=B)
    case = conv_case(f"many{B}", 7100 + B + d, C=256, K=4, d=d, dtype=dtype, act="silu",
                     w_std=0.25, bias_std=0.1, num_slots=B + 8, num_decodes=3,
                     prefill_lens=lens, prefill_h_p=0.5)
    parity(case)


def test_padding_and_out_of_range_slots():
    case = conv_case("pad", 601, C=256, K=4, d=1, dtype="bf16", act="silu", w_std=0.25,
                     bias_std=0.1, num_slots=16, num_decodes=4,
                     prefill_lens=[5, 70, 2], prefill_h_all=1)
    case.decode_slots[1] = -1
    case.decode_slots[2] = 16          # out of range: a padding row too
    case.prefill_slots[1] = -3
    parity(case)


def test_zero_length_requests_and_empty_batch():
    case = conv_case("zero", 602, C=512, K=4, d=1, dtype="bf16", act="none", w_std=0.25,
                     bias_std=None, num_slots=16, prefill_lens=[0, 7, 0, 0, 66, 0],
                     prefill_h_p=0.5)
    parity(case)
    import torch
    import stateful_causal_short_amd as scs
    x = dev(case.x)
    out = torch.zeros_like(x)
    pool = dev(case.pool)
    scs.sc_conv_prefill_varlen(x[:0], out[:0], dev(case.w), None, pool,
                               dev(np.zeros(1, np.int32)), dev(np.zeros(0, np.int32)),
                               dev(np.zeros(0, np.uint8)), activation="none")
    torch.cuda.synchronize()
    assert np.array_equal(host(pool), case.pool)


def test_strided_rows_and_2d_slot_indices():
    case = conv_case("strided", 603, C=512, K=4, d=3, dtype="bf16", act="none",
                     w_std=0.05, bias_std=None, num_slots=64, num_decodes=8,
                     prefill_lens=[100, 3, 250], prefill_h_p=0.5, ckpt_grid=32)
    parity(case, x_pad=24, slot_2d=3)


@pytest.mark.parametrize("C,K,d,dtype,act", [
    (100, 4, 1, "bf16", "silu"),     # C not a multiple of the vector width
    (256, 5, 2, "bf16", "silu"),     # width 5: generic kernel
    (256, 1, 1, "f32", "none"),      # width 1: no history
    (96, 3, 4, "f32", "silu"),       # generic dilation, fp32
    (64, 8, 9, "bf16", "none"),      # H = 63 < chunk
    (64, 8, 12, "f32", "none"),      # H = 84 > default chunk
])
def test_generic_kernel_shapes(C, K, d, dtype, act):
    case = conv_case("generic", 700 + C + K + d, C=C, K=K, d=d, dtype=dtype, act=act,
                     w_std=0.3, bias_std=0.1, num_slots=32, num_decodes=3, q=2,
                     prefill_lens=[1, 40, 150, 300], prefill_h_p=0.5,
                     ckpt_grid=max(64, (K - 1) * d))
    parity(case)


@pytest.mark.parametrize("dtype,d", [("f32", 1), ("f32", 3), ("bf16", 2)])
def test_fast_kernel_other_dtypes_and_dilations(dtype, d):
    case = conv_case("fast", 800 + d, C=1024, K=4, d=d, dtype=dtype, act="silu",
                     w_std=0.25, bias_std=0.1, num_slots=64, num_decodes=5, q=1,
                     prefill_lens=[1, 33, 64, 65, 300, 1000], prefill_h_p=0.5,
                     ckpt_grid=64)
    parity(case)


@pytest.mark.parametrize("q", [1, 2, 3, 4, 5, 70])
@pytest.mark.parametrize("d", [1, 3])
def test_update_lengths_and_flags(q, d):
    case = conv_case("update", 900 + q + d, C=512, K=4, d=d, dtype="bf16", act="silu",
                     w_std=0.25, bias_std=0.1, num_slots=64, num_decodes=20, q=q)
    case.decode_h = (np.arange(20) % 3 != 0).astype(np.uint8)
    parity(case)


def test_unaligned_rows_take_the_generic_path():
    # x and out start one element into their buffers: not 16-byte aligned
    import torch
    import stateful_causal_short_amd as scs
    case = conv_case("unaligned", 950, C=256, K=4, d=1, dtype="bf16", act="silu",
                     w_std=0.25, bias_std=0.1, num_slots=8,
                     prefill_lens=[9, 80], prefill_h_p=0.5)
    xs = np.zeros(case.T * case.C + 1, np.uint16)
    xs[1:] = case.x.reshape(-1)
    xd = dev(xs)[1:].view(case.T, case.C)
    od = torch.zeros(case.T * case.C + 1, dtype=torch.bfloat16, device="cuda")[1:].view(case.T, case.C)
    pool = dev(case.pool)
    scs.sc_conv_prefill_varlen(xd, od, dev(case.w), dev(case.bias), pool, dev(case.qsl_p),
                               dev(case.prefill_slots), dev(case.prefill_h),
                               activation="silu")
    torch.cuda.synchronize()
    ref, ref_pool, absum = oracle.conv(case, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(host(pool), ref_pool)
    check_close(host(od.contiguous()), ref, absum, "bf16", FLOOR)


def test_rounding_ties_to_even():
    # weights, bias and inputs chosen so every fp32 sum is exact: any output
    # difference would be a rounding-mode difference (bf16 ties to even).
    rng = np.random.default_rng(77)
    C, T = 512, 300
    x = synthetic.bf16_bits((rng.integers(128, 256, (T, C)) / 128.0) *
                            rng.choice([-1, 1], (T, C)) * np.exp2(rng.integers(-2, 3, (T, C))))
    w = synthetic.bf16_bits(rng.choice([-2, -1, -0.5, 0.5, 1, 2], (C, 4)))
    b = synthetic.bf16_bits(rng.choice([-1, 1], C) * np.exp2(rng.integers(-2, 3, C)))
    pool = synthetic.bf16_bits(rng.choice([-1.5, 1.25], (4, C, 3)))
    case = synthetic.ConvCase(name="ties", C=C, K=4, d=1, S=3, dtype="bf16", act="none",
                              x=x, w=w, bias=b, pool=pool,
                              qsl_p=np.array([0, 100, 300], np.int32),
                              prefill_slots=np.array([0, 2], np.int32),
                              prefill_h=np.array([1, 0], np.uint8))
    out, gpool = run_conv_case(case)
    ref, rpool, _ = oracle.conv(case)
    np.testing.assert_array_equal(gpool, rpool)
    np.testing.assert_array_equal(out, ref)


def test_gpu_chunked_equals_gpu_one_shot():
    # state carry on the GPU: prefill in pieces, then decodes == one shot
    L = 600
    src = conv_case("carry", 960, C=1024, K=4, d=3, dtype="bf16", act="silu", w_std=0.25,
                    bias_std=0.1, num_slots=2, prefill_lens=[L], prefill_h_all=1)

    def one(lo, hi, pool, as_decode):
        if as_decode:
            c = replace(src, x=src.x[lo:hi].copy(), num_decodes=hi - lo, q=1,
                        decode_slots=np.ones(hi - lo, np.int32),
                        qsl_p=np.zeros(1, np.int32), prefill_slots=np.zeros(0, np.int32),
                        prefill_h=np.zeros(0, np.uint8))
        else:
            c = replace(src, x=src.x[lo:hi].copy(), qsl_p=np.array([0, hi - lo], np.int32),
                        prefill_slots=np.array([1], np.int32),
                        prefill_h=np.array([1], np.uint8))
        return run_conv_case(c, pool=pool)

    whole = replace(src, prefill_slots=np.array([1], np.int32))
    o_all, p_all = run_conv_case(whole)
    pool = src.pool.copy()
    outs = []
    for lo, hi, dec in [(0, 1, False), (1, 70, False), (70, 71, True), (71, 500, False),
                        (500, 501, True), (501, 600, False)]:
        o, pool = one(lo, hi, pool, dec)
        outs.append(o)
    np.testing.assert_array_equal(np.concatenate(outs), o_all)
    np.testing.assert_array_equal(pool, p_all)


@pytest.mark.parametrize("row_bytes,dtype", [(3 * 8192 * 2, np.uint16), (6, np.uint16),
                                             (12, np.float32),
                                             # 5000 16-byte pieces: 5 workgroups a row,
                                             # a ragged last pass
                                             (16 * 5000, np.uint16),
                                             # 70001 pieces: 64 workgroups a row (the
                                             # cap), two passes, ragged
                                             (16 * 70001, np.uint16)])
def test_state_gather_scatter(row_bytes, dtype):
    import torch
    import stateful_causal_short_amd as scs
    rng = np.random.default_rng(row_bytes)
    per = row_bytes // np.dtype(dtype).itemsize
    if dtype == np.uint16:
        pool = rng.integers(0, 0x7F00, (50, per)).astype(np.uint16)   # finite bf16 bits
    else:
        pool = rng.standard_normal((50, per)).astype(np.float32)
    idx = rng.permutation(50)[:20].astype(np.int32)
    idx[3] = -1
    idx[7] = 50
    dense0 = np.full((20, per), 7, dtype)
    exp_dense = oracle.state_gather(pool, idx, dense0.copy())
    pd = dev(pool)
    dd = dev(dense0)
    scs.sc_state_gather(pd, dev(idx), dd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(dd), exp_dense)
    newd = (pool[:20] + 1).astype(dtype)
    exp_pool = oracle.state_scatter(newd, idx, pool.copy())
    scs.sc_state_scatter(dev(newd), dev(idx), pd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(pd), exp_pool)


def test_validate_metadata():
    import torch
    import stateful_causal_short_amd as scs
    case = synthetic.varlen_prefill_8seq()
    qsl = dev(case.qsl_p)
    slots = dev(np.asarray(case.prefill_slots, np.int32))
    T, S = int(case.qsl_p[-1]), case.num_slots
    print(f"[gpu] validate metadata B={case.num_prefills} T={T}", flush=True)
    assert scs.sc_validate_metadata(qsl, slots, num_tokens=T, num_slots=S)
    assert not scs.sc_validate_metadata(qsl, slots, num_tokens=T + 1, num_slots=S)
    bad = case.qsl_p.copy()
    bad[4] = bad[3] - 1                        # goes backwards
    assert not scs.sc_validate_metadata(dev(bad), None, num_tokens=T, num_slots=S)
    dup = np.asarray(case.prefill_slots, np.int32).copy()
    dup[5] = dup[1]
    assert not scs.sc_validate_metadata(None, dev(dup), num_tokens=T, num_slots=S)
    pad = np.asarray(case.prefill_slots, np.int32).copy()
    pad[2] = pad[6] = -1                       # repeated padding rows are fine
    assert scs.sc_validate_metadata(None, dev(pad), num_tokens=T, num_slots=S)
    big = np.asarray(case.prefill_slots, np.int32).copy()
    big[0] = S
    assert not scs.sc_validate_metadata(None, dev(big), num_tokens=T, num_slots=S)
    two_d = dev(np.stack([np.asarray(case.prefill_slots, np.int32), np.arange(8, dtype=np.int32)], 1))
    assert scs.sc_validate_metadata(None, two_d, num_tokens=T, num_slots=S)
    torch.cuda.synchronize()


def test_offsets_beyond_2gib_match_small_offsets():
    """Token rows and state slots more than 2 GiB into their tensors: a 320k-token
    varlen batch (x is 2.6 GB) gives bit for bit the outputs and states of each
    request run alone from row 0, and a decode on a 2.5 GB pool matches the same
    slots copied into a small pool (the small cases are pinned to the oracle
    elsewhere; this checks the 64-bit addressing)."""
    import torch
    import stateful_causal_short_amd as scs
    C, K = 4096, 4
    rng = np.random.default_rng(0xB16)
    block = dev(synthetic._normal(rng, (4096, C), 1.0, "bf16"))
    w = dev(synthetic._normal(rng, (C, K), 0.25, "bf16"))
    b = dev(synthetic._normal(rng, (C,), 0.1, "bf16"))
    lens = [150_001, 119_997, 50_011]
    T = sum(lens)
    print(f"[gpu] large offsets: prefill T={T} C={C} ({T * C * 2 / 2**30:.2f} GiB of x)", flush=True)
    x = block.repeat((T + 4095) // 4096, 1)[:T].contiguous()
    x[::7777] *= -0.5                                  # break the period a little
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = np.array([5, 0, 3], np.int32)
    h = np.array([1, 0, 1], np.uint8)
    pool0 = dev(synthetic._normal(rng, (8, C, 3), 1.0, "bf16"))
    out = torch.empty_like(x)
    pool = pool0.clone()
    scs.sc_conv_prefill_varlen(x, out, w, b, pool, dev(qsl), dev(slots), dev(h), activation="silu")
    torch.cuda.synchronize()
    for r in range(3):
        xr = x[int(qsl[r]):int(qsl[r + 1])].contiguous()
        o1 = torch.empty_like(xr)
        p1 = pool0.clone()
        scs.sc_conv_prefill_varlen(xr, o1, w, b, p1, dev(np.array([0, lens[r]], np.int32)),
                                   dev(slots[r:r + 1]), dev(h[r:r + 1]), activation="silu")
        torch.cuda.synchronize()
        assert torch.equal(o1, out[int(qsl[r]):int(qsl[r + 1])]), f"request {r} outputs"
        assert torch.equal(p1[int(slots[r])], pool[int(slots[r])]), f"request {r} state"
        del xr, o1, p1
    del x, out
    torch.cuda.empty_cache()

    n_slots, B = 100_000, 64
    print(f"[gpu] large offsets: decode B={B} on {n_slots} slots "
          f"({n_slots * C * 3 * 2 / 2**30:.2f} GiB pool)", flush=True)
    big = torch.empty((n_slots, C, 3), dtype=torch.bfloat16, device="cuda")
    big.copy_(block[:3].t().reshape(1, C, 3).expand(n_slots, C, 3))
    sl = np.sort(rng.choice(np.arange(n_slots - 5000, n_slots), B, replace=False)).astype(np.int32)
    assert int(sl[0]) * C * 3 * 2 > 2**31
    big[torch.from_numpy(sl).long().cuda()] = dev(synthetic._normal(rng, (B, C, 3), 1.0, "bf16"))
    xd = dev(synthetic._normal(rng, (B, C), 1.0, "bf16"))
    small = big[torch.from_numpy(sl).long().cuda()].clone()
    od1, od2 = torch.empty_like(xd), torch.empty_like(xd)
    scs.sc_conv_update(xd, od1, w, b, big, dev(sl), None, q=1, activation="silu")
    scs.sc_conv_update(xd, od2, w, b, small, dev(np.arange(B, dtype=np.int32)), None, q=1,
                       activation="silu")
    torch.cuda.synchronize()
    assert torch.equal(od1, od2)
    assert torch.equal(big[torch.from_numpy(sl).long().cuda()], small)


@pytest.mark.parametrize("C,lens,dtype", [
    (32768, [5, 70, 130, 1], "bf16"),     # 16 channel blocks per chunk
    (64, [100_000, 3], "bf16"),           # one long request, 8 live lanes per workgroup
    (24_576, [40, 12, 13, 300], "f32"),   # wide rows in fp32
])
def test_wide_rows_and_long_requests(C, lens, dtype):
    case = conv_case("wide_long", 1100 + C % 997 + len(lens), C=C, K=4, d=1, dtype=dtype,
                     act="silu", w_std=0.25, bias_std=0.1,
                     num_slots=8 + len(lens) + sum(n // 64 for n in lens), num_decodes=4, q=1,
                     prefill_lens=lens, prefill_h_p=0.5, ckpt_grid=64)
    parity(case)


def test_checkpoint_grid_with_no_checkpoint_reached():
    # every request is shorter than the grid: the destination array is empty
    # (a NULL data pointer), which exports nothing
    case = conv_case("ckpt_none", 1201, C=512, K=4, d=3, dtype="bf16", act="none",
                     w_std=0.1, bias_std=None, num_slots=16, num_decodes=2, q=1,
                     prefill_lens=[5, 30, 17], prefill_h_p=0.5, ckpt_grid=64)
    assert int(case.cu_ckpt[-1]) == 0 and case.ckpt_slots.size == 0
    parity(case)


@pytest.mark.parametrize("layout", ["ds", "sd"])
def test_launch_size_rules_do_not_change_results(layout):
    """The launcher picks the prefill chunk length and the decode requests per
    workgroup from the launch size. One large call (12-token chunks; 4 or 8
    requests per workgroup) and the same requests split into small calls
    (8-token chunks; 1 request per workgroup) must agree bit for bit."""
    import torch
    import stateful_causal_short_amd as scs
    C = 8192
    lens = [1900, 2100, 1700, 2300, 1500, 2000]                 # 11,500 tokens: above 2^26
    case = conv_case("rules", 1301, C=C, K=4, d=1, dtype="bf16", act="silu", w_std=0.25,
                     bias_std=0.1, num_slots=1200, num_decodes=1024, q=1, prefill_lens=lens,
                     prefill_h_p=0.5)
    if layout == "sd":
        case = synthetic.as_sd(case)
    print(f"[gpu] launch-size rules {layout}: T={case.T}", flush=True)
    big_out, big_pool = run_conv_case(case)
    nd = case.num_decodes
    x, w, b = dev(case.x), dev(case.w), dev(case.bias)
    out = torch.zeros_like(x)
    pool = dev(case.pool)
    kw = dict(dilation=1, activation="silu", state_layout=layout)
    for i in range(0, nd, 64):                                  # 64-request decode calls
        scs.sc_conv_update(x[i:i + 64], out[i:i + 64], w, b, pool,
                           dev(case.decode_slots[i:i + 64]), None, q=1, **kw)
    starts = nd + case.qsl_p[:-1]
    for r, L in enumerate(lens):                                # one prefill call per request
        s0 = int(starts[r])
        scs.sc_conv_prefill_varlen(x[s0:s0 + L], out[s0:s0 + L], w, b, pool,
                                   dev(np.array([0, L], np.int32)),
                                   dev(case.prefill_slots[r:r + 1]),
                                   dev(np.asarray(case.prefill_h[r:r + 1], np.uint8)), **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), big_out)
    np.testing.assert_array_equal(host(pool), big_pool)


@pytest.mark.parametrize("batch", [256, 512, 1024])
@pytest.mark.parametrize("off", [1, 2, 3])
def test_has_state_flags_at_every_byte_offset(batch, off):
    """The update and prefill kernels read a request's has-state flag as the
    aligned 32-bit word that holds it: flags passed as a view that starts 1-3
    bytes into its buffer, at batch sizes that put 2, 4 and 8 requests in a
    decode workgroup, pick out the right byte."""
    import torch
    import stateful_causal_short_amd as scs
    case = conv_case("flags", 1300 + batch + off, C=8192, K=4, d=1, dtype="bf16", act="silu",
                     w_std=0.25, bias_std=0.1, num_slots=batch + 16, num_decodes=batch, q=1,
                     prefill_lens=[5, 40, 3, 17, 64], prefill_h_p=0.5)
    rng = np.random.default_rng(off)
    case.decode_h = (rng.random(batch) < 0.6).astype(np.uint8)
    print(f"[gpu] flags batch={batch} off={off}", flush=True)
    dbuf = np.full(batch + 8, 0xAB, np.uint8)
    dbuf[off:off + batch] = case.decode_h
    pbuf = np.full(case.num_prefills + 8, 0xCD, np.uint8)
    pbuf[off:off + case.num_prefills] = case.prefill_h
    xd, od = dev(case.x), torch.zeros(case.T, case.C, dtype=torch.bfloat16, device="cuda")
    pd, wd, bd = dev(case.pool), dev(case.w), dev(case.bias)
    nd = case.num_decode_tokens
    scs.sc_conv_update(xd[:nd], od[:nd], wd, bd, pd, dev(np.asarray(case.decode_slots, np.int32)),
                       dev(dbuf)[off:off + batch], q=1, activation="silu")
    scs.sc_conv_prefill_varlen(xd[nd:], od[nd:], wd, bd, pd, dev(case.qsl_p),
                               dev(np.asarray(case.prefill_slots, np.int32)),
                               dev(pbuf)[off:off + case.num_prefills], activation="silu")
    torch.cuda.synchronize()
    ref, ref_pool, absum = oracle.conv(case, out_dtype="f64", absum=True)
    np.testing.assert_array_equal(host(pd), ref_pool, err_msg="state pool not bit-exact")
    check_close(host(od), ref, absum, "bf16", FLOOR)
