#!/usr/bin/env python3
"""Benchmark of the stateful causal short conv on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the hot path over one batch already resident in HBM.
The default workload is the varlen prefill batch (8 sequences, lengths
U{1..2048}, 8192 channels, width 4, bf16, bias + SiLU, 64-slot state pool):
state gather, conv, bias, SiLU and state write-back in one kernel; `value` is
its tokens/s. The same JSON line carries secondary objects for the method's
other workloads, each timed the same way in the same process: "decode" (512
requests x 1 token), "update_q4" (128 requests x 4 tokens), "spec" (128
requests x 4 speculative tokens on a 6-entry rolling buffer), "ple_mixed"
(dilated PLE batch: 256 decodes + 16 prefills with checkpoints; each kernel
and their sum) and "cca" (the 32k-token CCA q/k conv, main kernel + state
update), plus "copy_ceiling" (the practical HBM ceiling of a plain copy) and,
for every timed batch, "parity": one step on pristine inputs checked against
the oracle outside the timed region (state bit-exact, every output within
tolerance, and how many passed only through the accumulation floor).

Timing: W untimed eager steps, then K steps timed twice, bracketed by device
synchronisation and HIP events on the launch stream: as eager back-to-back
launches and as one replay of the K steps captured in a HIP graph (no host
launch cost inside the timed region); the faster is reported, both are kept.
For a batch with two kernels, each kernel's average comes from K launches of
that kernel alone, timed the same way. Identical buffer sets (x, out, state
pool) are rotated so that each step's inputs were last touched >= 1 GiB of
traffic earlier and come from HBM, not the 256 MB Infinity Cache. Prints one
JSON line on stdout; progress on stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s and achieved HBM GB/s (% of peak), varlen prefill + decode conv"
PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
ROTATE_BYTES = 1 << 30      # rotate buffer sets until >= 1 GiB is cycled


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def rotation_sets(touched_bytes, alloc_bytes, cap_bytes=24 << 30):
    """Buffer sets to rotate so that a step's data was last touched >= 1 GiB
    of traffic earlier (L2 and the 256 MB Infinity Cache hold none of it):
    ceil(1 GiB / bytes one step touches), at least 2, within a memory cap."""
    n = max(2, -(-ROTATE_BYTES // max(1, touched_bytes)))
    return int(max(2, min(n, cap_bytes // max(1, alloc_bytes))))


def cpu_threads():
    """(threads, affinity_cores, cgroup_quota): the CPU baseline runs on every
    core in the affinity mask, unless a cgroup CPU quota grants fewer cores'
    worth of time (then on that many)."""
    import math
    n = len(os.sched_getaffinity(0))
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
        if q != "max":
            quota = max(1, math.ceil(int(q) / int(per)))
    except (OSError, ValueError):
        pass
    return (min(n, quota) if quota else n), n, quota


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def conv_workload(name):
    import synthetic
    return {
        "varlen_prefill": synthetic.varlen_prefill_8seq,
        "single": synthetic.single_seq_64ch,
        "decode": synthetic.decode_512req,
        "update_q4": synthetic.update_128req_q4,
        "spec": synthetic.spec_128req_q4,
        "ple_mixed": synthetic.ple_mixed_batch,
        "ple_fused": synthetic.ple_mixed_batch,
    }[name]()


def conv_alg_bytes(case):
    """Algorithmic HBM bytes of one pass: every input element read once,
    every output and state element written once (state read only for
    requests with initial state), weights and bias read once; checkpoint
    windows written once."""
    es = case.elsize
    C, H = case.C, case.H
    b = case.T * C * es * 2                     # x read + out write
    hs = [1] * case.num_decodes if case.decode_h is None else list(case.decode_h)
    hs += list(case.prefill_h)
    slots = list(case.decode_slots) + list(case.prefill_slots)
    for h, s in zip(hs, slots):
        if 0 <= s < case.num_slots:
            b += (int(h) + 1) * C * H * es      # state read (if any) + write
    b += C * case.K * es + (C * es if case.bias is not None else 0)
    if case.ckpt_grid:
        b += int(case.cu_ckpt[-1]) * C * H * es
    return b


def spec_alg_bytes(case):
    """Speculative update: x read + out write, every state row read and
    written in full (S entries: the roll moves all of them), weights, bias and
    the accepted counts read once."""
    es, C = case.elsize, case.C
    b = case.num_decode_tokens * C * es * 2
    valid = sum(1 for s in case.decode_slots if 0 <= s < case.num_slots)
    b += valid * 2 * C * case.S * es
    b += C * case.K * es + (C * es if case.bias is not None else 0) + 4 * case.num_decodes
    return b


def conv_kernel_bytes(case):
    """Per-kernel split for mixed batches: (decode_update_bytes, prefill_bytes)."""
    from dataclasses import replace
    import numpy as np
    es, C, H = case.elsize, case.C, case.H
    w = C * case.K * es + (C * es if case.bias is not None else 0)
    dec = 0
    if case.num_decodes:
        hs = [1] * case.num_decodes if case.decode_h is None else list(case.decode_h)
        dec = case.num_decode_tokens * C * es * 2 + w
        dec += sum((int(h) + 1) * C * H * es for h in hs)
    pre = conv_alg_bytes(case) - dec + (w if case.num_decodes else 0)
    return dec, pre


def fused_extra_bytes(case):
    """PLE residual fusion: the residual (out) is read before it is written,
    and the outer residual is read, once per output element."""
    return 2 * case.T * case.C * case.elsize


class ConvRunner:
    def __init__(self, case, nsets, num_accepted=None, fused=False):
        import numpy as np
        import torch
        from tests._gpu import dev
        self.case = case
        nd = case.num_decode_tokens
        self.nd = nd
        base = dict(w=dev(case.w), b=None if case.bias is None else dev(case.bias),
                    dslots=dev(case.decode_slots), qsl=dev(case.qsl_p),
                    pslots=dev(case.prefill_slots),
                    ph=dev(np.asarray(case.prefill_h, np.uint8)),
                    dh=None if case.decode_h is None else dev(np.asarray(case.decode_h, np.uint8)),
                    ck=None)
        if case.ckpt_grid:
            base["ck"] = (case.ckpt_grid, dev(case.cu_ckpt), dev(case.ckpt_slots))
        self.acc = None if num_accepted is None else dev(num_accepted)
        self.base = base
        x0, p0 = dev(case.x), dev(case.pool)
        self.fused = fused
        self.sets = []
        for i in range(nsets):
            x = x0 if i == 0 else x0.clone()
            out = torch.randn_like(x) if fused else torch.empty_like(x)
            pool = p0 if i == 0 else p0.clone()
            outer = torch.randn_like(x) if fused else None
            self.sets.append((x, out, pool, outer))
        dk = "spec_update" if self.acc is not None else "decode_update"
        self.kernels = ([dk] if case.num_decodes else []) + \
                       (["prefill"] if case.num_prefills else [])

    def step(self, i, only=None):
        """One pass over the batch (decode rows, then prefill rows, as the PLE
        layer dispatches them); `only` restricts it to one kernel for timing."""
        import stateful_causal_short_amd as scs
        c, b = self.case, self.base
        x, out, pool, outer = self.sets[i % len(self.sets)]
        fz = dict(accumulate=True, outer_residual=outer) if self.fused else {}
        lay = dict(state_layout=c.layout)
        if c.num_decodes and self.acc is not None and only in (None, "spec_update"):
            scs.sc_conv_update_spec(x[:self.nd], out[:self.nd], b["w"], b["b"], pool,
                                    b["dslots"], self.acc, q=c.q, dilation=c.d,
                                    activation=c.act, **lay)
        elif c.num_decodes and only in (None, "decode_update"):
            fd = dict(fz, outer_residual=outer[:self.nd]) if self.fused else {}
            scs.sc_conv_update(x[:self.nd], out[:self.nd], b["w"], b["b"], pool,
                               b["dslots"], b["dh"], q=c.q, dilation=c.d, activation=c.act,
                               **fd, **lay)
        if c.num_prefills and only in (None, "prefill"):
            fp = dict(fz, outer_residual=outer[self.nd:]) if self.fused else {}
            scs.sc_conv_prefill_varlen(x[self.nd:], out[self.nd:], b["w"], b["b"], pool,
                                       b["qsl"], b["pslots"], b["ph"], dilation=c.d,
                                       activation=c.act, ckpt=b["ck"], **fp, **lay)


def cca_alg_bytes(case):
    """Algorithmic HBM bytes of one CCA pass (main kernel + state update):
    q, k, v_cur, v_del read once, the output row written once, each request's
    conv history and delayed value read (when continued) and written once,
    weights and biases read once. Returns (main_bytes, state_update_bytes)."""
    es, T, C, n = 2, case.T, case.C, case.n
    vd = case.nkv * case.hd // 2
    main = T * (C + 2 * vd) * es + T * case.out_width * es
    main += (C * case.t0 + C + C * case.hd * case.t1 + C + vd) * es
    hs = [1] * case.num_decodes + [int(h) for h in case.prefill_h]
    slots = list(case.decode_slots) + list(case.prefill_slots)
    live = [h for h, s in zip(hs, slots) if 0 <= s < case.num_slots]
    main += sum(live) * (C * n + vd) * es            # history read for continued requests
    upd = len(live) * (C * n + vd) * es              # new history and delayed value
    return main, upd


class CcaRunner:
    def __init__(self, case, nsets):
        import numpy as np
        import torch
        from tests._gpu import dev
        self.case = case
        c = case
        self.w = [dev(c.w_dw), dev(c.b_dw), dev(c.w_gr), dev(c.b_gr), dev(c.delayed_init)]
        self.meta = [dev(c.decode_slots), dev(c.qsl_p), dev(c.prefill_slots),
                     dev(np.asarray(c.prefill_h, np.uint8))]
        base = [dev(c.q), dev(c.k), dev(c.v_cur), dev(c.v_del), dev(c.conv_state),
                dev(c.delayed_state)]
        self.sets = []
        for i in range(nsets):
            q, k, vc, vdl, cs, ds = base if i == 0 else [t.clone() for t in base]
            out = torch.empty((c.T, c.out_width), dtype=torch.bfloat16, device="cuda")
            self.sets.append((q, k, vc, vdl, out, cs, ds))
        self.kernels = ["cca_main+state"]

    def step(self, i, only=None):
        import stateful_causal_short_amd as scs
        c = self.case
        q, k, vc, vdl, out, cs, ds = self.sets[i % len(self.sets)]
        scs.sc_cca_qk_conv(q, k, vc, vdl, out, *self.w, cs, ds, *self.meta,
                           num_q_heads=c.nq, num_kv_heads=c.nkv, head_dim=c.hd,
                           t0=c.t0, t1=c.t1)


def cpu_baseline_conv(case, budget_s=10.0, num_accepted=None, fused=False):
    """The oracle, as it stands, on the same batch; repeated until ~budget_s."""
    import oracle
    threads, aff, quota = cpu_threads()
    fz = dict(resid=case.x, outer=case.x) if fused else {}
    runs, t0 = 0, time.perf_counter()
    while True:
        if num_accepted is None:
            oracle.conv(case, nthreads=threads, **fz)
        else:
            oracle.conv_spec(case, num_accepted, nthreads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 1000:
            break
    res = {"value": case.T * runs / el, "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"the full batch ({case.T} tokens) run {runs}x through the fp64 "
                     f"oracle, {el:.1f} s wall on {threads} threads",
           "affinity_cores": aff, "cgroup_cpu_quota": quota}
    # one thread, one run of the batch (bounded: at most ~2x the budget)
    if threads > 1 and el / runs * threads <= 2 * budget_s:
        t1 = time.perf_counter()
        if num_accepted is None:
            oracle.conv(case, nthreads=1, **fz)
        else:
            oracle.conv_spec(case, num_accepted, nthreads=1)
        res["one_thread_value"] = case.T / (time.perf_counter() - t1)
    res["cpu_model"] = cpu_model()
    return res


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


DW_SOURCES = ("conv.hip", "conv_device.hpp", "common.hpp", "kernels.hpp")
CCA_SOURCES = ("cca.hip", "cca.hpp", "common.hpp")


def source_sha(files=DW_SOURCES):
    """Digest of the sources a kernel family is built from (depthwise by default)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "stateful_causal_short_amd", "csrc")
    for f in files:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key, files=DW_SOURCES):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel sources (else null)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_sha") != source_sha(files):
        return None
    return e.get("bytes_per_launch")


def time_launches(fn_steps, steps):
    """Average GPU time per launch (ms) of `steps` back-to-back launches made by
    fn_steps(), measured two ways with HIP events on the launch stream: eager
    launches, and one replay of the launches captured in a HIP graph (no host
    launch cost). Graph replay adds a few us between nodes on large kernels.
    Either way the average includes the gaps between back-to-back launches (an
    event pair around each launch would add the events' own cost, which is
    larger). Returns (eager_ms, graph_ms)."""
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # a GPU spin ahead of the region lets the host queue all launches before
    # the first runs, so small kernels are not timed at the host's launch rate
    torch.cuda._sleep(5_000_000)
    s.record()
    fn_steps()
    e.record()
    torch.cuda.synchronize()
    eager = s.elapsed_time(e) / steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn_steps()
    g.replay()                        # untimed first replay
    torch.cuda.synchronize()
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    graph = s.elapsed_time(e) / steps
    return eager, graph


def spec_varlen_alg_bytes(case, qsl):
    """Speculative update with a draft count per request: x read + out written
    for every draft row; each request with drafts reads and writes its whole
    state row (S entries: the roll moves all of them); weights, bias, accepted
    counts and offsets read once."""
    es, C = case.elsize, case.C
    qs = [int(qsl[r + 1] - qsl[r]) for r in range(case.num_decodes)]
    b = int(qsl[-1]) * C * es * 2
    b += sum(2 * C * case.S * es for r, q in enumerate(qs)
             if q > 0 and 0 <= case.decode_slots[r] < case.num_slots)
    b += C * case.K * es + (C * es if case.bias is not None else 0)
    b += 4 * case.num_decodes + 4 * (case.num_decodes + 1)
    return b


def spec_varlen_bench(args):
    """Speculative update with per-request draft counts (128 requests, counts
    uniform in {0..4}, 8192 channels, width 4, rolling buffer of 6 entries,
    bf16, bias + SiLU). One step = one sc_conv_update_spec_varlen call."""
    import numpy as np
    import torch
    import synthetic
    import stateful_causal_short_amd as scs
    from tests._gpu import dev
    case, qsl = synthetic.spec_varlen_128req()
    if args.state_layout == "sd":
        case = synthetic.as_sd(case)
    B, T = case.num_decodes, int(qsl[-1])
    acc = np.minimum(synthetic.num_accepted(synthetic.SEED_BASE + 0x38, B, 4),
                     np.maximum(np.diff(qsl), 1)).astype(np.int32)
    alg = spec_varlen_alg_bytes(case, qsl)
    max_q = int(np.diff(qsl).max())
    nsets = rotation_sets(alg, T * case.C * case.elsize * 2 + case.pool.nbytes)
    log(f"spec varlen B={B} T={T} C={case.C} S={case.S} layout={case.layout}; "
        f"alg bytes/step={alg}; {nsets} rotating buffer sets")
    w = dev(case.w)
    b = dev(case.bias)
    slots = dev(np.asarray(case.decode_slots, np.int32))
    accd = dev(acc)
    qd = dev(qsl)
    x0, p0 = dev(case.x), dev(case.pool)
    sets = [(x0 if i == 0 else x0.clone(), torch.empty_like(x0), p0 if i == 0 else p0.clone())
            for i in range(nsets)]

    def step(i):
        x, out, pool = sets[i % nsets]
        scs.sc_conv_update_spec_varlen(x, out, w, b, pool, slots, accd, qd, max_query_len=max_q,
                                       dilation=case.d, activation=case.act,
                                       state_layout=case.layout)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    eager, graph = time_launches(lambda: [step(args.warmup + i) for i in range(args.steps)],
                                 args.steps)
    ms = min(eager, graph)
    gbps = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak), speculative conv update",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": case.name, "requests": B, "tokens": T, "max_query_len": max_q,
                   "channels": case.C, "width": case.K, "dilation": case.d,
                   "activation": case.act, "state_slots": case.num_slots, "state_len": case.S,
                   "state_layout": case.layout},
        "hbm_gbps": gbps, "pct_peak": 100.0 * gbps / PEAK_GBPS,
        "kernel_us": {"spec_update": ms * 1e3},
        "timing": {"step": {"eager_us": eager * 1e3, "graph_us": graph * 1e3}},
        "roofline": {"kernel": "spec_update", "bound": "hbm", "achieved": gbps,
                     "peak": PEAK_GBPS, "unit": "GB/s", "frac": gbps / PEAK_GBPS,
                     "traffic": None, "alg_bytes_per_launch": alg},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        import oracle
        threads, _, _ = cpu_threads()
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.conv_spec_varlen(case, acc, qsl, nthreads=threads)
            runs += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or runs >= 1000:
                break
        result["cpu_baseline"] = {
            "value": T * runs / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the full batch ({T} tokens) run {runs}x through the fp64 oracle, "
                      f"{el:.1f} s wall on {threads} threads", "cpu_model": cpu_model()}
    print(json.dumps(result), flush=True)


def cca_bench(args):
    """CCA q/k conv on the 32k-token mixed batch (512 decodes + 64 prefills,
    16 q heads, 4 kv heads, head_dim 128, kernels 2 and 2). One step = one
    sc_cca_qk_conv call: the fused main kernel, then the state update, timed
    as the default line's CCA object is (measure_cca)."""
    case, run, m = measure_cca(args, parity=not args.no_parity)
    ms = m["step_us"] * 1e-3
    result = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak), CCA q/k conv",
        "value": case.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": case.name, "decodes": case.num_decodes,
                   "prefills": case.num_prefills, "tokens": case.T, "q_heads": case.nq,
                   "kv_heads": case.nkv, "head_dim": case.hd, "t0": case.t0, "t1": case.t1},
        "hbm_gbps": m["roofline"]["achieved"],
        "pct_peak": 100.0 * m["roofline"]["frac"],
        "grouped_conv_tflops": m["grouped_conv_tflops"],
        "timing": m["timing"],
        "rotating_sets": m["rotating_sets"],
        "roofline": m["roofline"],
        "parity": m.get("parity"),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline_cca(case)
    print(json.dumps(result), flush=True)


def cpu_baseline_cca(case, budget_s=10.0):
    """The CCA oracle, as it stands, on the same batch; repeated until ~budget_s."""
    import oracle
    threads, _, _ = cpu_threads()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.cca(case, nthreads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 20:
            break
    return {"value": case.T * runs / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full batch ({case.T} tokens) run {runs}x through the fp64 "
                      f"oracle, {el:.1f} s wall on {threads} threads",
            "cpu_model": cpu_model()}


def copy_calibration(args):
    """Plain copy of known size through the library's row-copy kernel
    (sc_state_gather with identity indices): 1 GiB read + 1 GiB written per
    launch. Gives the practical HBM ceiling and the scale of the FETCH_SIZE /
    WRITE_SIZE counters."""
    import torch
    import stateful_causal_short_amd as scs
    row = 48 * 1024
    rows = (1 << 30) // row
    nsets = 2
    src = [torch.empty(rows, row, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    dst = [torch.empty_like(src[0]) for _ in range(nsets)]
    for t in src:
        t.fill_(1)
    idx = torch.arange(rows, dtype=torch.int32, device="cuda")
    for i in range(args.warmup):
        scs.sc_state_gather(src[i % nsets], idx, dst[i % nsets])
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(args.steps):
        scs.sc_state_gather(src[i % nsets], idx, dst[i % nsets])
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    nbytes = rows * row
    print(json.dumps({"workload": "copy_calibration", "kernel": "row_copy",
                      "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
                      "us_per_launch": ms * 1e3,
                      "GBps": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


def traffic_from(d):
    """Rewrite the entries of profiles/traffic.json whose rocprofv3 --pmc runs
    (one counter each) are under directory d: pmc_<workload>_<COUNTER>/
    run_counter_collection.csv for COUNTER in FETCH_SIZE, WRITE_SIZE and
    workload varlen_prefill (the prefill kernel: the non-copy kernel with the
    most bytes) and/or cca (the CCA kernels together), plus the row-copy
    calibration pmc_copy_*. Each counter is scaled by the factor that maps the
    same counter of the row copy to its known bytes. CPU only; prints a summary."""
    import csv
    import statistics

    def per_kernel(workload, counter):
        path = os.path.join(d, f"pmc_{workload}_{counter}", "run_counter_collection.csv")
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    copy_bytes = ((1 << 30) // (48 * 1024)) * 48 * 1024     # copy_calibration's launch
    factors = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = per_kernel("copy", counter)
        ck = [k for k in cp if "row_copy" in k]
        if len(ck) != 1:
            raise SystemExit(f"copy run: expected one row_copy kernel, found {ck}")
        med = statistics.median(cp[ck[0]])
        factors[counter] = copy_bytes / 1024.0 / med
        print(f"{counter}: copy median {med:,.1f} KiB ({len(cp[ck[0]])} dispatches) -> factor "
              f"{factors[counter]:.5f}")

    def have(workload):
        return all(os.path.exists(os.path.join(d, f"pmc_{workload}_{c}", "run_counter_collection.csv"))
                   for c in ("FETCH_SIZE", "WRITE_SIZE"))

    entries = {}
    # depthwise workloads: the one library kernel of the run (largest counters)
    for workload, kern in (("varlen_prefill", "prefill"), ("decode", "decode_update")):
        if not have(workload):
            continue
        kib, names = {}, {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            pv = per_kernel(workload, counter)
            cand = {k: statistics.median(v) for k, v in pv.items() if k.startswith("void sc::")}
            names[counter] = max(cand, key=cand.get)
            kib[counter] = cand[names[counter]]
        if names["FETCH_SIZE"] != names["WRITE_SIZE"]:
            raise SystemExit(f"different dominant kernels: {names}")
        dec_b, pre_b = conv_kernel_bytes(conv_workload(workload))
        alg = pre_b if kern == "prefill" else dec_b
        entries[f"{workload}:{kern}"] = (kib, names["FETCH_SIZE"], alg, source_sha())
    if have("cca"):
        import synthetic
        kib, kern = {}, []
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            pv = per_kernel("cca", counter)
            ks = sorted(k for k in pv if "cca_" in k)
            kern = ks
            kib[counter] = sum(statistics.median(pv[k]) for k in ks)
        main_b, upd_b = cca_alg_bytes(synthetic.cca_mixed_32k())
        entries["cca:cca_main+state"] = (kib, " + ".join(kern), main_b + upd_b,
                                         source_sha(CCA_SOURCES))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path) as f:
        t = json.load(f)
    for key, (kib, kernel, alg, sha) in entries.items():
        total = int(round(1024 * sum(kib[c] * factors[c] for c in kib)))
        for c in kib:
            print(f"{key}: {c} median {kib[c]:,.2f} KiB -> {kib[c] * factors[c]:,.0f} KiB")
        print(f"{key}: total {total:,} bytes per launch vs {alg:,} algorithmic: ratio "
              f"{total / alg:.4f}; kernels {kernel}; source digest {sha}")
        t[key] = {"bytes_per_launch": total, "alg_bytes_per_launch": alg,
                  "fetch_kib": kib["FETCH_SIZE"], "write_kib": kib["WRITE_SIZE"],
                  "fetch_factor": factors["FETCH_SIZE"], "write_factor": factors["WRITE_SIZE"],
                  "kernel": kernel, "source_sha": sha}
    with open(path, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")


# ---------------------------------------------------------------------------
# parity of a timed batch (outside the timed region)
# ---------------------------------------------------------------------------
def spec_parity(case, run, acc):
    """conv_parity for the speculative update: the oracle's rolling buffer
    with the same accepted counts."""
    import numpy as np
    import torch
    import oracle
    from tests._gpu import check_close, dev, host
    x, out, pool, _ = run.sets[0]
    pool.copy_(dev(case.pool))
    out.zero_()
    run.step(0)
    torch.cuda.synchronize()
    got, gpool = host(out), host(pool)
    ref, rpool, ab = oracle.conv_spec(case, acc, out_dtype="f64", absum=True)
    res = {"reference": "oracle", "rows_checked": int(case.T), "elements": int(ref.size),
           "state_bit_exact": bool(np.array_equal(gpool, rpool))}
    try:
        share = check_close(got, ref, ab, case.dtype, 2.0 ** -20)
        res["outputs_within_tolerance"] = True
        res["floor_passes"] = int(round(share * ref.size))
    except AssertionError as e:
        res["outputs_within_tolerance"] = False
        res["floor_passes"] = None
        res["error"] = str(e)[:300]
    res["pass"] = res["state_bit_exact"] and res["outputs_within_tolerance"]
    return res


def conv_parity(case, run):
    """Restores buffer set 0 to the batch's pristine state, runs one step and
    checks it against the oracle on the same inputs: state pool bit-exact, every
    output element within the tolerance (2 bf16 ulp or 1e-5 relative, or the fp32
    accumulation floor 2^-20 of the sum of |terms|). floor_passes counts the
    elements that passed through the floor alone."""
    import numpy as np
    import torch
    import oracle
    from tests._gpu import check_close, dev, host
    x, out, pool, _ = run.sets[0]
    pool.copy_(dev(case.pool))
    out.zero_()
    run.step(0)
    torch.cuda.synchronize()
    got, gpool = host(out), host(pool)
    ref, rpool, ab = oracle.conv(case, out_dtype="f64", absum=True)
    res = {"reference": "oracle", "rows_checked": int(case.T), "elements": int(ref.size),
           "state_bit_exact": bool(np.array_equal(gpool, rpool))}
    try:
        share = check_close(got, ref, ab, case.dtype, 2.0 ** -20)
        res["outputs_within_tolerance"] = True
        res["floor_passes"] = int(round(share * ref.size))
    except AssertionError as e:
        res["outputs_within_tolerance"] = False
        res["floor_passes"] = None
        res["error"] = str(e)[:300]
    res["pass"] = res["state_bit_exact"] and res["outputs_within_tolerance"]
    return res


def cca_parity(case, run):
    """As conv_parity for the CCA call: both state pools and the value half
    bit-exact, the q/k half within 2 bf16 ulp or the fp32 accumulation floor."""
    import numpy as np
    import torch
    import oracle
    import synthetic
    from tests._gpu import cca_floor_rel, check_close, dev, host
    q, k, vc, vdl, out, cs, ds = run.sets[0]
    cs.copy_(dev(case.conv_state))
    ds.copy_(dev(case.delayed_state))
    out.zero_()
    run.step(0)
    torch.cuda.synchronize()
    got, gcs, gds = host(out), host(cs), host(ds)
    nd, al = [], []
    ref, rcs, rds, ab = oracle.cca(case, out_dtype="f64", absum=True, chain_diff=nd, allow=al)
    C = case.C
    res = {"reference": "oracle", "rows_checked": int(case.T), "elements": int(ref.size),
           "state_bit_exact": bool(np.array_equal(gcs, rcs) and np.array_equal(gds, rds)),
           "value_half_bit_exact": bool(np.array_equal(
               synthetic.bf16_to_f32(got[:, C:]).astype(np.float64), ref[:, C:])),
           "depthwise_values_an_fp32_chain_rounds_elsewhere": nd[0]}
    try:
        share = check_close(got[:, :C], ref[:, :C], ab[:, :C], "bf16", cca_floor_rel(case),
                            allow=al[0][:, :C])
        res["outputs_within_tolerance"] = True
        res["floor_passes"] = int(round(share * ref[:, :C].size))
    except AssertionError as e:
        res["outputs_within_tolerance"] = False
        res["floor_passes"] = None
        res["error"] = str(e)[:300]
    res["pass"] = (res["state_bit_exact"] and res["value_half_bit_exact"]
                   and res["outputs_within_tolerance"])
    return res


def roofline(kernel, alg_bytes, us, traffic=None):
    gbps = alg_bytes / (us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": gbps, "peak": PEAK_GBPS,
            "unit": "GB/s", "frac": gbps / PEAK_GBPS, "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes}


# ---------------------------------------------------------------------------
# one depthwise workload: step time, per-kernel times, rooflines, parity
# ---------------------------------------------------------------------------
def measure_conv(args, workload, *, parity=True, quiet=False):
    import torch
    import synthetic
    case = conv_workload(workload)
    if args.state_layout == "sd":
        case = synthetic.as_sd(case)
    acc = None
    if workload == "spec":
        acc = synthetic.num_accepted(synthetic.SEED_BASE + 0x36, case.num_decodes, case.q)
        alg = dec_b = spec_alg_bytes(case)
        pre_b = 0
    else:
        alg = conv_alg_bytes(case)
        dec_b, pre_b = conv_kernel_bytes(case)
    fused = workload == "ple_fused"
    if fused:
        # every output element also reads its residual and outer residual
        alg += fused_extra_bytes(case)
        dec_b += 2 * case.num_decode_tokens * case.C * case.elsize
        pre_b += 2 * (case.T - case.num_decode_tokens) * case.C * case.elsize
    alloc = case.T * case.C * case.elsize * (4 if fused else 2) + case.pool.nbytes
    nsets = rotation_sets(alg, alloc)
    log(f"{case.name}: T={case.T} C={case.C} K={case.K} d={case.d} {case.dtype} "
        f"act={case.act}; alg bytes/step={alg}; {nsets} rotating buffer sets")
    run = ConvRunner(case, nsets, acc, fused=fused)
    for i in range(args.warmup):
        run.step(i)
    torch.cuda.synchronize()
    timing = {}

    def timed(name, fn_steps):
        eager, graph = time_launches(fn_steps, args.steps)
        timing[name] = {"eager_us": eager * 1e3, "graph_us": graph * 1e3}
        return min(eager, graph)

    ms_step = timed("step", lambda: [run.step(args.warmup + i) for i in range(args.steps)])
    # per-kernel averages: with one kernel per step, the timed region itself;
    # otherwise K launches of each kernel alone, timed the same way
    if len(run.kernels) == 1:
        kms = {run.kernels[0]: ms_step}
    else:
        kms = {k: timed(k, lambda k=k: [run.step(i, only=k) for i in range(args.steps)])
               for k in run.kernels}
    log(f"{case.name}: {ms_step * 1e3:.2f} us/step; per kernel "
        + ", ".join(f"{k}={v * 1e3:.2f} us" for k, v in kms.items()))
    kb = {"prefill": pre_b, "decode_update": dec_b, "spec_update": dec_b}
    key = {"varlen_prefill": "varlen_prefill", "decode": "decode"}.get(workload)
    roofs = {k: roofline(k, kb[k], v * 1e3,
                         traffic_for(f"{key}:{k}") if key and args.state_layout == "ds" else None)
             for k, v in kms.items()}
    res = {"workload": case.name, "tokens": case.T, "decodes": case.num_decodes,
           "decode_q": case.q, "prefills": case.num_prefills, "channels": case.C,
           "width": case.K, "dilation": case.d, "activation": case.act,
           "state_slots": case.num_slots, "state_len": case.S, "state_layout": case.layout,
           "checkpoint_grid": case.ckpt_grid, "fused_residuals": fused,
           "rotating_sets": nsets, "step_us": ms_step * 1e3,
           "kernel_us": {k: v * 1e3 for k, v in kms.items()}, "timing": timing,
           "tokens_per_s": case.T / (ms_step * 1e-3),
           "alg_bytes_per_step": alg, "hbm_gbps": alg / (ms_step * 1e-3) / 1e9,
           "roofline": roofs}
    if len(kms) > 1:
        tot = sum(kms.values())
        res["kernels_sum_us"] = tot * 1e3
        res["roofline_sum"] = roofline("+".join(kms), sum(kb[k] for k in kms), tot * 1e3)
    if parity and not fused:
        log(f"{case.name}: parity against the oracle ...")
        res["parity"] = conv_parity(case, run) if acc is None else spec_parity(case, run, acc)
        log(f"{case.name}: parity {'pass' if res['parity']['pass'] else 'FAIL'}")
    return case, run, res, acc, fused


def measure_cca(args, *, parity=True):
    import torch
    import synthetic
    case = synthetic.cca_mixed_32k()
    main_b, upd_b = cca_alg_bytes(case)
    nsets = rotation_sets(main_b + upd_b, main_b + upd_b)
    log(f"CCA T={case.T} C={case.C}; alg bytes/step main={main_b} state={upd_b}; "
        f"{nsets} rotating buffer sets")
    run = CcaRunner(case, nsets)
    for i in range(args.warmup):
        run.step(i)
    torch.cuda.synchronize()
    eager, graph = time_launches(lambda: [run.step(args.warmup + i) for i in range(args.steps)],
                                 args.steps)
    ms = min(eager, graph)
    flops = 2.0 * case.T * case.C * case.hd * case.t1
    log(f"CCA: {ms * 1e3:.2f} us/step ({(main_b + upd_b) / (ms * 1e-3) / 1e9:.0f} GB/s)")
    res = {"workload": case.name, "tokens": case.T, "decodes": case.num_decodes,
           "prefills": case.num_prefills, "q_heads": case.nq, "kv_heads": case.nkv,
           "head_dim": case.hd, "t0": case.t0, "t1": case.t1, "rotating_sets": nsets,
           "step_us": ms * 1e3, "timing": {"eager_us": eager * 1e3, "graph_us": graph * 1e3},
           "tokens_per_s": case.T / (ms * 1e-3),
           "grouped_conv_tflops": flops / (ms * 1e-3) / 1e12,
           "roofline": roofline("cca_main+state_update", main_b + upd_b, ms * 1e3,
                                traffic_for("cca:cca_main+state", CCA_SOURCES))}
    if parity:
        log("CCA: parity against the oracle ...")
        res["parity"] = cca_parity(case, run)
        log(f"CCA: parity {'pass' if res['parity']['pass'] else 'FAIL'}")
    return case, run, res


def copy_ceiling(args):
    """The practical HBM ceiling: the library's row copy (sc_state_gather with
    identity indices) moving 1 GiB in and 1 GiB out per launch, two buffer
    sets alternated, 10 launches after 2 warmup launches."""
    import torch
    import stateful_causal_short_amd as scs
    row = 48 * 1024
    rows = (1 << 30) // row
    src = [torch.ones(rows, row, dtype=torch.uint8, device="cuda") for _ in range(2)]
    dst = [torch.empty_like(src[0]) for _ in range(2)]
    idx = torch.arange(rows, dtype=torch.int32, device="cuda")
    for i in range(2):
        scs.sc_state_gather(src[i % 2], idx, dst[i % 2])
    torch.cuda.synchronize()
    steps = 10
    eager, _ = time_launches(
        lambda: [scs.sc_state_gather(src[i % 2], idx, dst[i % 2]) for i in range(steps)], steps)
    nbytes = 2 * rows * row
    gbps = nbytes / (eager * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"copy ceiling: {gbps:.0f} GB/s")
    return {"kernel": "row_copy", "bytes_per_launch": nbytes, "us_per_launch": eager * 1e3,
            "achieved": gbps, "unit": "GB/s", "frac_of_peak": gbps / PEAK_GBPS}


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="varlen_prefill",
                    choices=["varlen_prefill", "single", "decode", "update_q4", "spec",
                             "spec_varlen", "ple_mixed", "ple_fused", "cca", "copy"])
    ap.add_argument("--state-layout", default="ds", choices=["ds", "sd"],
                    help="state pool layout: (slots, C, S) or (slots, S, C)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="varlen_prefill: only the headline workload (no decode, update, "
                         "PLE, CCA or copy-ceiling objects)")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle check of the timed batches")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="rewrite profiles/traffic.json from rocprofv3 --pmc runs under DIR "
                         "and exit (CPU only)")
    args = ap.parse_args()
    if args.traffic_from:
        return traffic_from(args.traffic_from)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no multi-GPU leg); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import stateful_causal_short_amd as scs
    scs.lib()
    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}; workload {args.workload}")

    if args.workload == "cca":
        return cca_bench(args)
    if args.workload == "copy":
        return copy_calibration(args)
    if args.workload == "spec_varlen":
        return spec_varlen_bench(args)

    case, run, m, acc, fused = measure_conv(args, args.workload, parity=not args.no_parity)
    ms_step = m["step_us"] * 1e-3
    # dominant kernel: the prefill kernel when present
    dom = "prefill" if "prefill" in m["roofline"] else run.kernels[0]
    result = {
        "metric": METRIC,
        "value": case.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {
            "workload": case.name, "decodes": case.num_decodes, "decode_q": case.q,
            "prefills": case.num_prefills, "tokens": case.T, "channels": case.C,
            "width": case.K, "dilation": case.d, "activation": case.act,
            "state_slots": case.num_slots, "checkpoint_grid": case.ckpt_grid,
            "state_len": case.S, "state_layout": case.layout, "fused_residuals": fused,
        },
        "hbm_gbps": m["hbm_gbps"],
        "pct_peak": 100.0 * m["hbm_gbps"] / PEAK_GBPS,
        "kernel_us": m["kernel_us"],
        "timing": m["timing"],
        "rotating_sets": m["rotating_sets"],
        "roofline": m["roofline"][dom],
        "parity": m.get("parity"),
        "cpu_baseline": None,
    }
    if "roofline_sum" in m:
        result["roofline_sum"] = m["roofline_sum"]
    if args.workload == "varlen_prefill" and not args.no_secondary:
        # The metric names the decode conv too, and the other workloads of the
        # method ride along as secondary objects (each timed the same way, in
        # the same process; `value` stays the varlen prefill's).
        for name, wl in (("decode", "decode"), ("update_q4", "update_q4"),
                         ("spec", "spec"), ("ple_mixed", "ple_mixed")):
            _, r2, res2, _, _ = measure_conv(args, wl, parity=not args.no_parity)
            result[name] = res2
            del r2
            torch.cuda.empty_cache()
        _, r3, result["cca"] = measure_cca(args, parity=not args.no_parity)
        del r3
        torch.cuda.empty_cache()
        result["copy_ceiling"] = copy_ceiling(args)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline_conv(case, num_accepted=acc, fused=fused)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
