"""Test-side helpers: move synthetic cases to the GPU and run them through the
C ABI (via the thin binding), and the output tolerance of the parity tests."""
from __future__ import annotations

import numpy as np

from synthetic import bf16_to_f32


def dev(a: np.ndarray, dtype: str = None):
    """NumPy array -> cuda tensor. uint16 arrays are bf16 bit patterns unless
    dtype says otherwise."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16 and dtype != "u16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def host(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def run_conv_case(case, *, pool=None, x_pad: int = 0, slot_2d: int = 0, stream=None):
    """Runs a ConvCase on the GPU: decode rows through sc_conv_update, then
    prefill rows through sc_conv_prefill_varlen (as the PLE layer's dispatch
    does). Returns (out, pool_after) as NumPy arrays.

    x_pad > 0 stores x and out with row stride C + x_pad (strided rows);
    slot_2d > 0 passes slots as column 0 of a (B, slot_2d) int32 tensor."""
    import torch
    import stateful_causal_short_amd as scs
    T, C = case.T, case.C
    if x_pad:
        xs = np.zeros((T, C + x_pad), case.x.dtype)
        xs[:, :C] = case.x
        xd = dev(xs)[:, :C]
        od = dev(np.zeros((T, C + x_pad), case.x.dtype))[:, :C]
    else:
        xd = dev(case.x)
        od = dev(np.zeros((T, C), case.x.dtype))
    pd = dev(case.pool if pool is None else pool)
    wd = dev(case.w)
    bd = None if case.bias is None else dev(case.bias)

    def slots(a):
        a = np.asarray(a, np.int32)
        if slot_2d:
            m = np.full((a.shape[0], slot_2d), -7, np.int32)
            m[:, 0] = a
            return dev(m)
        return dev(a)

    nd = case.num_decode_tokens
    if case.num_decodes:
        dh = None if case.decode_h is None else dev(np.asarray(case.decode_h, np.uint8))
        scs.sc_conv_update(xd[:nd], od[:nd], wd, bd, pd, slots(case.decode_slots), dh,
                           q=case.q, dilation=case.d, activation=case.act,
                           state_layout=case.layout, stream=stream)
    if case.num_prefills:
        ck = None
        if case.ckpt_grid:
            ck = (case.ckpt_grid, dev(case.cu_ckpt), dev(case.ckpt_slots))
        scs.sc_conv_prefill_varlen(xd[nd:], od[nd:], wd, bd, pd, dev(case.qsl_p),
                                   slots(case.prefill_slots),
                                   dev(np.asarray(case.prefill_h, np.uint8)),
                                   dilation=case.d, activation=case.act, ckpt=ck,
                                   state_layout=case.layout, stream=stream)
    torch.cuda.synchronize()
    return host(od.contiguous()), host(pd)


def run_spec_case(case, num_accepted, *, pool=None, x_pad: int = 0, stream=None):
    """Runs a ConvCase's decode requests (q rows each) as speculative requests
    through sc_conv_update_spec with the given accepted counts. Returns
    (out, pool_after) as NumPy arrays."""
    import torch
    import stateful_causal_short_amd as scs
    T, C = case.num_decode_tokens, case.C
    if x_pad:
        xs = np.zeros((T, C + x_pad), case.x.dtype)
        xs[:, :C] = case.x[:T]
        xd = dev(xs)[:, :C]
        od = dev(np.zeros((T, C + x_pad), case.x.dtype))[:, :C]
    else:
        xd = dev(case.x[:T])
        od = dev(np.zeros((T, C), case.x.dtype))
    pd = dev(case.pool if pool is None else pool)
    scs.sc_conv_update_spec(xd, od, dev(case.w), None if case.bias is None else dev(case.bias),
                            pd, dev(np.asarray(case.decode_slots, np.int32)),
                            dev(np.asarray(num_accepted, np.int32)), q=case.q,
                            dilation=case.d, activation=case.act, state_layout=case.layout,
                            stream=stream)
    torch.cuda.synchronize()
    return host(od.contiguous()), host(pd)


def ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def check_close(gpu: np.ndarray, ref64: np.ndarray, absum: np.ndarray, dtype: str,
                floor_rel: float, *, what: str = "out", mask=None, slab_rows: int = 2048,
                allow: np.ndarray = None):
    """Output tolerance: |gpu - ref| <= 2 bf16 ulp(ref) (bf16) or 1e-5 |ref|
    (fp32), or <= floor_rel * (sum of |terms|) — the fp32 accumulation bound,
    which only matters where the sum cancels — plus `allow` where given (the
    oracle's bound on how far an intermediate rounded after an fp32 sum of any
    order can move the output). Every element is checked, in slabs of rows so
    that the temporaries stay small at full size. Returns the share of
    elements that passed through the floor alone."""
    if allow is None:
        allow = np.zeros_like(absum)
    if mask is not None:
        gpu, ref64, absum, allow = gpu[mask], ref64[mask], absum[mask], allow[mask]
    n_bad, first, n_floor = 0, None, 0
    rows = gpu.shape[0] if gpu.ndim else 1
    for r0 in range(0, max(rows, 1), slab_rows):
        sl = slice(r0, r0 + slab_rows)
        g = as_f64(gpu[sl], dtype)
        ref = ref64[sl]
        diff = np.abs(g - ref)
        tol = 2.0 * ulp_bf16(ref) if dtype == "bf16" else 1e-5 * np.abs(ref)
        floor = floor_rel * absum[sl]
        ok = diff <= np.maximum(tol, floor) + allow[sl]
        if not ok.all():
            bad = np.argwhere(~ok)
            n_bad += len(bad)
            if first is None:
                i = tuple(bad[0])
                first = (tuple([i[0] + r0, *i[1:]]), g[i], ref[i], tol[i], floor[i])
        n_floor += int(((diff > tol) & (diff <= floor)).sum())
    if n_bad:
        i, gv, rv, tv, fv = first
        raise AssertionError(
            f"{what}: {n_bad} of {gpu.size} outside tolerance; first at {i}: "
            f"gpu={gv!r} ref={rv!r} tol={tv!r} floor={fv!r}")
    return float(n_floor) / max(1, gpu.size)


def run_cca_case(case, *, conv_state=None, delayed_state=None, fused=False,
                 no_delayed_init=False, fused_width=None):
    """Runs a CcaCase through sc_cca_qk_conv. Returns (out, conv_state_after,
    delayed_state_after) as NumPy arrays. fused=True passes q, k, v_cur and
    v_del as column slices of one (T, X) projection output (strided rows);
    X = fused_width when given (else their widths + 8)."""
    import torch
    import stateful_causal_short_amd as scs
    T = case.T
    if fused:
        parts = [case.q, case.k, case.v_cur, case.v_del]
        widths = [p.shape[1] for p in parts]
        X = sum(widths) + 8 if fused_width is None else fused_width
        assert X >= sum(widths)
        big = np.zeros((T, X), np.uint16)
        off, views = 0, []
        for p_, wdt in zip(parts, widths):
            big[:, off:off + wdt] = p_
            off += wdt
        bd = dev(big)
        off, views = 0, []
        for wdt in widths:
            views.append(bd[:, off:off + wdt])
            off += wdt
        qd, kd, vcd, vdd = views
    else:
        qd, kd, vcd, vdd = dev(case.q), dev(case.k), dev(case.v_cur), dev(case.v_del)
    out = torch.zeros((T, case.out_width), dtype=torch.bfloat16, device="cuda")
    cs = dev(case.conv_state if conv_state is None else conv_state)
    ds = dev(case.delayed_state if delayed_state is None else delayed_state)
    dsl = dev(case.decode_slots) if case.num_decodes else None
    qsl = dev(case.qsl_p) if case.num_prefills else None
    psl = dev(case.prefill_slots) if case.num_prefills else None
    ph = dev(np.asarray(case.prefill_h, np.uint8)) if case.num_prefills else None
    scs.sc_cca_qk_conv(qd, kd, vcd, vdd, out, dev(case.w_dw), dev(case.b_dw),
                       dev(case.w_gr), dev(case.b_gr),
                       None if no_delayed_init else dev(case.delayed_init), cs, ds,
                       dsl, qsl, psl, ph, num_q_heads=case.nq, num_kv_heads=case.nkv,
                       head_dim=case.hd, t0=case.t0, t1=case.t1)
    torch.cuda.synchronize()
    return host(out), host(cs), host(ds)


def cca_floor_rel(case) -> float:
    """fp32 accumulation bound for one CCA output: bias + hd*t1 products +
    residual terms (2 per query head, 2G per key head), gamma_n = n * 2^-24."""
    G = case.nq // case.nkv
    return (case.hd * case.t1 + 2 * G + 4) * 2.0 ** -24


def run_fused_case(case, xp, perm, *, resid=None, outer=None, pool=None, num_accepted=None):
    """Runs a ConvCase through the fused calls on physical tensors: x rows at
    xp[perm[j]] for logical row j, out initialised with `resid` (accumulate)
    or zeros, `outer` added. Decode rows go through sc_conv_update (or
    sc_conv_update_spec when num_accepted is given), prefill rows through
    sc_conv_prefill_varlen, each with its slice of the row map. Returns
    (out, pool_after) as NumPy arrays (physical rows)."""
    import torch
    import stateful_causal_short_amd as scs
    xd = dev(xp)
    od = dev(resid if resid is not None else np.zeros_like(xp))
    ou = None if outer is None else dev(outer)
    pd = dev(case.pool if pool is None else pool)
    wd = dev(case.w)
    bd = None if case.bias is None else dev(case.bias)
    tok = dev(np.asarray(perm, np.int32))
    nd = case.num_decode_tokens
    kw = dict(accumulate=resid is not None, outer_residual=ou, dilation=case.d,
              activation=case.act, state_layout=case.layout)
    if case.num_decodes:
        if num_accepted is not None:
            scs.sc_conv_update_spec(xd, od, wd, bd, pd, dev(np.asarray(case.decode_slots, np.int32)),
                                    dev(np.asarray(num_accepted, np.int32)), q=case.q,
                                    token_indices=tok[:nd], **kw)
        else:
            dh = None if case.decode_h is None else dev(np.asarray(case.decode_h, np.uint8))
            scs.sc_conv_update(xd, od, wd, bd, pd, dev(np.asarray(case.decode_slots, np.int32)), dh,
                               q=case.q, token_indices=tok[:nd], **kw)
    if case.num_prefills:
        ck = None
        if case.ckpt_grid:
            ck = (case.ckpt_grid, dev(case.cu_ckpt), dev(case.ckpt_slots))
        scs.sc_conv_prefill_varlen(xd, od, wd, bd, pd, dev(case.qsl_p),
                                   dev(np.asarray(case.prefill_slots, np.int32)),
                                   dev(np.asarray(case.prefill_h, np.uint8)), ckpt=ck,
                                   token_indices=tok[nd:], **kw)
    torch.cuda.synchronize()
    return host(od), host(pd)
