"""The library's launches under HIP graph capture: every replay of a captured
decode + prefill (with checkpoints) must equal the eager result bit for bit.
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
    case = synthetic.config4(C=2048, num_decodes=32, Bp=5, min_len=20, max_len=900,
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
