"""The library's launches under HIP graph capture: every replay of a captured
decode + prefill (with checkpoints), speculative update or CCA call must equal
the eager result bit for bit.
Between replays the program does its own eager work (restoring the pool,
clearing the output) and synchronises."""
import numpy as np
import pytest

import synthetic
from tests._gpu import dev, host

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    import stateful_causal_short_amd as scs
    case = synthetic.ple_mixed_batch(C=2048, num_decodes=32, Bp=5, min_len=20, max_len=900,
                             grid=128, num_slots=256)
    print(f"[gpu] graph replay T={case.T} C={case.C}", flush=True)
    nd = case.num_decode_tokens
    x = dev(case.x)
    out = torch.zeros_like(x)
    pool0 = dev(case.pool)
    pool = pool0.clone()
    w = dev(case.w)
    dsl, qsl, psl = dev(case.decode_slots), dev(case.qsl_p), dev(case.prefill_slots)
    ph = dev(np.asarray(case.prefill_h, np.uint8))
    ck = (case.ckpt_grid, dev(case.cu_ckpt), dev(case.ckpt_slots))

    def step():
        scs.sc_conv_update(x[:nd], out[:nd], w, None, pool, dsl, None, q=1,
                           dilation=case.d, activation=case.act)
        scs.sc_conv_prefill_varlen(x[nd:], out[nd:], w, None, pool, qsl, psl, ph,
                                   dilation=case.d, activation=case.act, ckpt=ck)

    step()
    torch.cuda.synchronize()
    eager_out, eager_pool = host(out), host(pool)

    g = torch.cuda.CUDAGraph()
    pool.copy_(pool0)
    out.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        pool.copy_(pool0)           # eager work between replays
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), eager_out, err_msg=f"replay {rep} out")
        np.testing.assert_array_equal(host(pool), eager_pool, err_msg=f"replay {rep} pool")


def test_graph_replays_match_eager_speculative():
    """The speculative calls (uniform draft count, then a draft count per
    request) under capture, replayed several times against the eager result."""
    import torch
    import stateful_causal_short_amd as scs
    case, qsl = synthetic.spec_varlen_case("graph_spec", 6101, C=2048, K=4, d=1, dtype="bf16",
                                           act="silu", w_std=0.4, bias_std=0.2, num_slots=96,
                                           B=40, num_spec=3)
    print(f"[gpu] graph replay speculative B={case.num_decodes} T={int(qsl[-1])}", flush=True)
    B = case.num_decodes
    x = dev(case.x)
    out = torch.zeros_like(x)
    xu = dev(synthetic._normal(np.random.default_rng(6102), (B * 4, case.C), 1.0, "bf16"))
    outu = torch.zeros_like(xu)
    pool0 = dev(case.pool)
    pool = pool0.clone()
    w, b = dev(case.w), dev(case.bias)
    slots = dev(np.asarray(case.decode_slots, np.int32))
    acc = dev(synthetic.num_accepted(6103, B, 4, lo=0, hi=5))
    q = dev(qsl)

    def step():
        scs.sc_conv_update_spec(xu, outu, w, b, pool, slots, acc, q=4)
        scs.sc_conv_update_spec_varlen(x, out, w, b, pool, slots, acc, q, max_query_len=4)

    step()
    torch.cuda.synchronize()
    eager = (host(outu), host(out), host(pool))
    g = torch.cuda.CUDAGraph()
    pool.copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        pool.copy_(pool0)
        out.zero_()
        outu.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((host(outu), host(out), host(pool)), eager,
                                   ("uniform out", "varlen out", "pool")):
            np.testing.assert_array_equal(got, want, err_msg=f"replay {rep} {what}")


def test_graph_replays_match_eager_cca():
    """The CCA call (main kernel, then the state update) under capture: a
    batch of decodes and prefills large enough for the kv-head helpers,
    replayed several times against the eager result, pools restored and the
    output cleared by eager work between replays."""
    import torch
    import stateful_causal_short_amd as scs
    case = synthetic.cca_case("graph_cca", 6201, num_decodes=96,
                              prefill_lens=[2500, 1, 3100, 700, 1800], num_slots=128)
    print(f"[gpu] graph replay cca T={case.T}", flush=True)
    q, k, vc, vd = dev(case.q), dev(case.k), dev(case.v_cur), dev(case.v_del)
    out = torch.zeros((case.T, case.out_width), dtype=torch.bfloat16, device="cuda")
    cs0, ds0 = dev(case.conv_state), dev(case.delayed_state)
    cs, ds = cs0.clone(), ds0.clone()
    params = [dev(case.w_dw), dev(case.b_dw), dev(case.w_gr), dev(case.b_gr), dev(case.delayed_init)]
    dsl, qsl, psl = dev(case.decode_slots), dev(case.qsl_p), dev(case.prefill_slots)
    ph = dev(np.asarray(case.prefill_h, np.uint8))

    def step():
        scs.sc_cca_qk_conv(q, k, vc, vd, out, *params, cs, ds, dsl, qsl, psl, ph,
                           num_q_heads=case.nq, num_kv_heads=case.nkv, head_dim=case.hd,
                           t0=case.t0, t1=case.t1)

    step()
    torch.cuda.synchronize()
    eager = (host(out), host(cs), host(ds))
    g = torch.cuda.CUDAGraph()
    cs.copy_(cs0)
    ds.copy_(ds0)
    out.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        cs.copy_(cs0)
        ds.copy_(ds0)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((host(out), host(cs), host(ds)), eager,
                                   ("out", "conv state", "delayed state")):
            np.testing.assert_array_equal(got, want, err_msg=f"replay {rep} {what}")
