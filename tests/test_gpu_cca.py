"""GPU parity of the CCA q/k conv (sc_cca_qk_conv) against the CPU oracle.

Bar: conv and delayed states bit-exact; value half of the output (v_cur copy
and delayed shift) bit-exact; q/k outputs within 2 bf16 ulp of the oracle's
float64 result, or within the fp32 accumulation bound n * 2^-24 of the sum of
|terms| (n = bias + hd*t1 products + residual terms). Every output row is
checked. The oracle takes the depthwise intermediate as the layer's first
Conv1d materialises it: the exact value rounded once to bf16. The kernel sums
it in fp32 from the bias (taps in pairs on the two-term dot product on the
MFMA path, a fused multiply-add chain in tap order otherwise), which can land
on the other side of a bf16 midpoint; the oracle counts, as a diagnostic, the
depthwise values where an fp32 fused multiply-add chain rounds to a different
bf16 value, and each test prints that count. Where the kernel's value differs,
the grouped stage moves the output by at most |W2| times one bf16 spacing of
the depthwise value, inside the output tolerance."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synthetic
from tests._gpu import cca_floor_rel, check_close, run_cca_case

pytestmark = pytest.mark.gpu


def parity(case, **kw):
    print(f"[gpu] cca {case.name} T={case.T} nq={case.nq} nkv={case.nkv} hd={case.hd} "
          f"t0={case.t0} t1={case.t1} kw={kw}", flush=True)
    out, cs, ds = run_cca_case(case, **kw)
    ocase = case
    if kw.get("no_delayed_init"):
        ocase = replace(case, delayed_init=np.zeros_like(case.delayed_init))
    nd, al = [], []
    ref, rcs, rds, absum = oracle.cca(ocase, out_dtype="f64", absum=True, chain_diff=nd,
                                      allow=al)
    np.testing.assert_array_equal(cs, rcs, err_msg="conv state not bit-exact")
    np.testing.assert_array_equal(ds, rds, err_msg="delayed state not bit-exact")
    C = case.C
    # value half: exact copies
    np.testing.assert_array_equal(synthetic.bf16_to_f32(out[:, C:]).astype(np.float64),
                                  ref[:, C:], err_msg="value half not bit-exact")
    frac = check_close(out[:, :C], ref[:, :C], absum[:, :C], "bf16", cca_floor_rel(case),
                       what="q/k", allow=al[0][:, :C])
    print(f"[gpu] cca {case.name}: ok (floor-only share {frac:.2e}; depthwise values an "
          f"fp32 chain rounds elsewhere: {nd[0]} of {case.T * case.C})", flush=True)


def test_cca_mixed_32k_full():
    parity(synthetic.cca_mixed_32k())


def test_cca_small_tile_edges():
    case = synthetic.cca_case("cca_edges", 501, num_decodes=70,
                              prefill_lens=[1, 2, 3, 62, 63, 64, 65, 130, 7], num_slots=128)
    case.prefill_h[:] = [0, 1, 1, 0, 1, 0, 1, 1, 0]
    parity(case)


@pytest.mark.parametrize("nq,nkv,t0", [(4, 4, 2), (8, 1, 2), (4, 2, 1), (4, 2, 3), (2, 1, 4)])
def test_mfma_shapes(nq, nkv, t0):
    case = synthetic.cca_case("cca_shape", 600 + nq * 10 + nkv + t0, nq=nq, nkv=nkv, hd=128,
                              t0=t0, t1=2, num_decodes=9,
                              prefill_lens=[1, 5, 70, 33], num_slots=64)
    parity(case)


@pytest.mark.parametrize("hd,t0,t1", [(64, 2, 2), (32, 2, 3), (16, 3, 1)])
def test_generic_shapes(hd, t0, t1):
    case = synthetic.cca_case("cca_generic", 700 + hd + t0 + t1, nq=4, nkv=2, hd=hd,
                              t0=t0, t1=t1, num_decodes=5, prefill_lens=[1, 2, 9, 20],
                              num_slots=32)
    parity(case)


@pytest.mark.parametrize("nq,nkv", [(16, 4), (8, 1)])
def test_many_short_and_empty_prefills(nq, nkv):
    """Hundreds of requests of 0 to 2 tokens: a tile crosses more than 64
    request boundaries (a run of 90 empty requests), and with more tiles than
    a 256-CU grid has workgroups per head group (2 per CU / (nq + nkv)), a
    workgroup's next tile lies hundreds of requests after its previous one."""
    rng = np.random.default_rng(950 + nq)
    lens = np.concatenate([[3, 1], np.zeros(90, np.int64), rng.integers(0, 3, 900),
                           [100, 40, 0, 0, 65], rng.integers(0, 2, 70), [1000]])
    case = synthetic.cca_case("cca_many", 951 + nq, nq=nq, nkv=nkv, hd=128, num_decodes=37,
                              prefill_lens=lens, num_slots=1200)
    assert (case.T + 31) // 32 > 2 * 256 // (nq + nkv)
    parity(case)


def kv_helper_split(T, nq, nkv, cus=256, t0=2):
    """The launcher's tile split on a device with `cus` compute units: S main
    workgroups per head group (as many as fit resident), and for each kv-head
    group `hp` helpers taking its tiles from `jk * S` on (hp = 0: no helpers)."""
    ntiles = (T + 31) // 32
    per_cu = 2 if (t0 <= 2 and nq // nkv <= 4) else 1
    NG = nq + nkv
    S = min(max(cus * per_cu // NG, 1), ntiles)
    hp = (cus * per_cu - S * NG) // nkv
    if hp > 0 and S >= 8:
        jk = -(-ntiles // (S + hp))
        if jk * S < ntiles:
            return S, hp, jk
    return S, 0, 0


@pytest.mark.parametrize("nq,nkv,t0,decodes,lens", [
    (16, 4, 2, 100, [1200, 3, 2000, 1697]),       # 157 tiles: helpers take 150-156
    (4, 2, 2, 40, [2450, 3000]),                  # 172 tiles: one helper takes 170-171
    (8, 1, 2, 64, [9000, 7, 10929]),              # 625 tiles: four helpers take 560-624
    (16, 4, 3, 30, [4000, 1, 5669]),              # one workgroup per CU: S = 12, 4 helpers
])
def test_kv_head_helpers(nq, nkv, t0, decodes, lens):
    """Batches whose tile count makes the launcher split the kv-head groups'
    tiles between their main workgroups and helpers (with a ragged share among
    the helpers), checked on every row."""
    T = decodes + sum(lens)
    S, hp, jk = kv_helper_split(T, nq, nkv, t0=t0)
    assert hp > 0 and jk * S < (T + 31) // 32
    case = synthetic.cca_case("cca_kvhelp", 960 + nq + 7 * (t0 - 2), nq=nq, nkv=nkv, hd=128, t0=t0,
                              num_decodes=decodes, prefill_lens=lens,
                              num_slots=decodes + len(lens) + 8)
    case.prefill_h[:] = 1
    parity(case)


@pytest.mark.parametrize("T,path", [(65_000, "mfma"), (66_000, "one-thread")])
def test_row_offsets_near_and_past_2gib(T, path):
    """q, k, v_cur and v_del as column slices of one projection output with
    32 KiB rows. At 65,000 tokens its last rows lie just under 2 GiB into the
    buffer, where the MFMA kernel's 32-bit offsets end. At 66,000 they lie
    past it, and the launcher takes the one-thread kernel (64-bit offsets).
    Outputs are checked against the oracle on sampled rows (every request's
    first and last rows, the last 64 rows of the batch, 600 random rows), and
    the states in full."""
    X = 16384
    lens = [30_000, 17, T - 40 - 30_017]
    case = synthetic.cca_case("cca_2gib", 970 + T % 7, num_decodes=40, prefill_lens=lens,
                              num_slots=64)
    case.prefill_h[:] = [1, 0, 1]
    last_byte = ((T - 1) * X + case.q.shape[1] + case.k.shape[1] + 2 * case.v_cur.shape[1]) * 2
    assert (last_byte < 2 ** 31) == (path == "mfma")
    print(f"[gpu] cca offsets: T={T} rows of {X * 2} bytes, last byte {last_byte:,} ({path})",
          flush=True)
    rng = np.random.default_rng(T)
    rows = set(range(T - 64, T)) | set(int(v) for v in rng.integers(0, T, 600))
    starts = [0] + list(np.cumsum([1] * case.num_decodes + lens))
    for s0 in starts[:-1]:
        rows |= {s0, s0 + 1, s0 + 2}
    for s1 in starts[1:]:
        rows |= {s1 - 1, s1 - 2}
    mask = np.zeros(T, bool)
    mask[[r for r in rows if 0 <= r < T]] = True
    out, cs, ds = run_cca_case(case, fused=True, fused_width=X)
    al = []
    ref, rcs, rds, absum = oracle.cca(case, out_dtype="f64", absum=True, row_mask=mask, allow=al)
    np.testing.assert_array_equal(cs, rcs, err_msg="conv state not bit-exact")
    np.testing.assert_array_equal(ds, rds, err_msg="delayed state not bit-exact")
    C = case.C
    np.testing.assert_array_equal(synthetic.bf16_to_f32(out[mask, C:]).astype(np.float64),
                                  ref[mask, C:], err_msg="value half not bit-exact")
    check_close(out[:, :C], ref[:, :C], absum[:, :C], "bf16", cca_floor_rel(case),
                what="q/k", mask=mask, allow=al[0][:, :C])
    print(f"[gpu] cca offsets T={T}: ok on {int(mask.sum())} rows", flush=True)


def test_padding_slots_fused_rows_and_no_delayed_init():
    case = synthetic.cca_case("cca_pad", 801, num_decodes=6, prefill_lens=[4, 80, 1],
                              num_slots=16)
    case.decode_slots[2] = -1
    case.decode_slots[4] = 16               # out of range: padding row
    case.prefill_slots[1] = -5
    case.prefill_h[:] = 1
    parity(case, fused=True, no_delayed_init=True)


@pytest.mark.parametrize("no_init", [False, True])
def test_empty_state_pool(no_init):
    # zero slots: every request is a padding row, so histories are zeros and the
    # first token of each request takes delayed_init (or zeros) as its delayed
    # value; nothing is written to the (empty) pools
    case = synthetic.cca_case("cca_nopool", 803 + int(no_init), num_decodes=5,
                              prefill_lens=[3, 40, 1, 70], num_slots=16)
    n = case.t0 + case.t1 - 2
    vd = case.nkv * case.hd // 2
    case = replace(case, conv_state=np.zeros((0, case.C, n), case.conv_state.dtype),
                   delayed_state=np.zeros((0, vd), case.delayed_state.dtype))
    parity(case, no_delayed_init=no_init)


def test_gpu_cca_chunked_equals_one_shot():
    L = 150
    src = synthetic.cca_case("cca_carry", 901, num_decodes=0, prefill_lens=[L], num_slots=2)
    src.prefill_h[:] = 1
    src.prefill_slots[:] = 1
    one, cs1, ds1 = run_cca_case(src)
    cs, ds = src.conv_state.copy(), src.delayed_state.copy()
    outs = []
    for lo, hi, dec in [(0, 1, False), (1, 70, False), (70, 71, True), (71, 149, False),
                        (149, 150, True)]:
        sl = slice(lo, hi)
        kw = dict(q=src.q[sl], k=src.k[sl], v_cur=src.v_cur[sl], v_del=src.v_del[sl])
        if dec:
            c = replace(src, num_decodes=hi - lo, decode_slots=np.ones(hi - lo, np.int32),
                        qsl_p=np.zeros(1, np.int32), prefill_slots=np.zeros(0, np.int32),
                        prefill_h=np.zeros(0, np.uint8), **kw)
        else:
            c = replace(src, qsl_p=np.array([0, hi - lo], np.int32), **kw)
        o, cs, ds = run_cca_case(c, conv_state=cs, delayed_state=ds)
        outs.append(o)
    np.testing.assert_array_equal(np.concatenate(outs), one)
    np.testing.assert_array_equal(cs, cs1)
    np.testing.assert_array_equal(ds, ds1)
