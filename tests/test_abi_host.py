"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/statefulconv.h declares, and rejects bad arguments on the host
with the documented status before any launch (fake device pointers are never
dereferenced on these paths)."""
import ctypes
import os
import re

import pytest

import stateful_causal_short_amd as scs
from stateful_causal_short_amd import sc_cca_desc, sc_ckpt_desc, sc_conv_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "statefulconv.h")

OK, NULL, INVALID, DTYPE, CAPACITY, UNSUPPORTED = 0, -1, -2, -3, -4, -5
P = ctypes.c_void_p(0x10000)   # a fake device pointer: never dereferenced here
P2 = ctypes.c_void_p(0x20000)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sc_status|const char\*|int32_t)\s+(sc_\w+)\s*\(",
                                 text, re.M)))


def test_library_exports_every_declared_function():
    lib = scs.lib()
    names = declared_functions()
    assert set(names) == set(scs.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.sc_abi_version() == 3
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert lib.sc_status_string(s)


def desc(**kw):
    d = dict(channels=64, width=4, dilation=1, state_len=3, dtype=1, activation=1,
             x_row_stride=64, out_row_stride=64, state_indices_stride=1)
    d.update(kw)
    return sc_conv_desc(**d)


def prefill(d, *, x=P, out=P2, w=P, bias=None, pool=P, num_slots=4, qsl=P, slots=P,
            h=P, batch=2, T=10, ckpt=None, fuse=None):
    return scs.lib().sc_conv_prefill_varlen(
        None if d is None else ctypes.byref(d), x, out, w, bias, pool, num_slots, qsl,
        slots, h, batch, T, None if ckpt is None else ctypes.byref(ckpt),
        None if fuse is None else ctypes.byref(fuse), None)


def update(d, *, x=P, out=P2, w=P, pool=P, num_slots=4, slots=P, h=None, batch=2, q=1,
           fuse=None):
    return scs.lib().sc_conv_update(None if d is None else ctypes.byref(d), x, out, w,
                                    None, pool, num_slots, slots, h, batch, q,
                                    None if fuse is None else ctypes.byref(fuse), None)


def spec(d, *, x=P, out=P2, w=P, pool=P, num_slots=4, slots=P, acc=P, batch=2, q=2,
         fuse=None):
    return scs.lib().sc_conv_update_spec(None if d is None else ctypes.byref(d), x, out, w,
                                         None, pool, num_slots, slots, acc, batch, q,
                                         None if fuse is None else ctypes.byref(fuse), None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), DTYPE),
    (dict(channels=0), INVALID),
    (dict(width=0), INVALID),
    (dict(width=9, state_len=8), UNSUPPORTED),
    (dict(dilation=0), INVALID),
    (dict(activation=3), INVALID),
    (dict(x_row_stride=63), INVALID),
    (dict(out_row_stride=10), INVALID),
    (dict(state_indices_stride=0), INVALID),
    (dict(state_len=2), CAPACITY),                 # (4-1)*1 = 3 needed
    (dict(dilation=3, state_len=8), CAPACITY),     # 9 needed
    (dict(state_len=(1 << 20) + 1), INVALID),
    (dict(state_layout=2), INVALID),
])
def test_descriptor_validation(kw, status):
    assert prefill(desc(**kw)) == status
    assert update(desc(**kw)) == status
    assert spec(desc(**kw)) == status


def test_wide_state_rows_are_accepted():
    # a buffer sized for speculative rollback (S = H + num_spec): zero-work calls succeed
    d = desc(state_len=7)
    assert prefill(d, batch=0) == OK
    assert update(d, batch=0) == OK
    assert spec(d, batch=0) == OK


def test_spec_rules():
    d = desc(state_len=6)
    assert spec(None) == NULL
    assert spec(d, acc=None) == NULL
    assert spec(d, slots=None) == NULL
    assert spec(d, pool=None) == NULL
    assert spec(d, out=P) == INVALID            # out aliases x
    assert spec(d, q=7) == INVALID              # 7 drafts do not fit 6 entries
    assert spec(d, q=7, batch=0) == INVALID     # checked before the zero-work exit
    assert spec(d, q=-1) == INVALID
    assert spec(d, batch=-1) == INVALID
    assert spec(d, x=None, out=None, w=None, slots=None, acc=None, pool=None, batch=0) == OK
    assert spec(d, q=0) == OK


def spec_varlen(d, *, x=P, out=P2, w=P, pool=P, num_slots=4, slots=P, acc=P, qsl=P, batch=2,
                T=6, maxq=3, fuse=None):
    return scs.lib().sc_conv_update_spec_varlen(
        None if d is None else ctypes.byref(d), x, out, w, None, pool, num_slots, slots, acc,
        qsl, batch, T, maxq, None if fuse is None else ctypes.byref(fuse), None)


def test_spec_varlen_rules():
    d = desc(state_len=6)
    assert spec_varlen(None) == NULL
    assert spec_varlen(d, qsl=None) == NULL
    assert spec_varlen(d, acc=None) == NULL
    assert spec_varlen(d, slots=None) == NULL
    assert spec_varlen(d, pool=None) == NULL
    assert spec_varlen(d, out=P) == INVALID            # out aliases x
    assert spec_varlen(d, maxq=7) == INVALID           # 7 drafts do not fit 6 entries
    assert spec_varlen(d, maxq=7, batch=0) == INVALID  # checked before the zero-work exit
    assert spec_varlen(d, maxq=-1) == INVALID
    assert spec_varlen(d, batch=-1) == INVALID
    assert spec_varlen(d, T=-1) == INVALID
    assert spec_varlen(d, T=1 << 31) == UNSUPPORTED
    assert spec_varlen(desc(state_len=2)) == CAPACITY
    none = dict(x=None, out=None, w=None, slots=None, acc=None, qsl=None, pool=None)
    assert spec_varlen(d, batch=0, **none) == OK
    assert spec_varlen(d, T=0, **none) == OK
    assert spec_varlen(d, maxq=0, **none) == OK


def test_null_arguments():
    d = desc()
    assert prefill(None) == NULL
    assert prefill(d, x=None) == NULL
    assert prefill(d, out=None) == NULL
    assert prefill(d, w=None) == NULL
    assert prefill(d, qsl=None) == NULL
    assert prefill(d, slots=None) == NULL
    assert prefill(d, h=None) == NULL            # required for prefill
    assert prefill(d, pool=None) == NULL
    assert update(None) == NULL
    assert update(d, x=None, out=None, w=None, slots=None, pool=None, batch=0) == OK
    assert update(d, slots=None) == NULL
    assert update(d, pool=None) == NULL


def test_size_and_alias_rules():
    d = desc()
    assert prefill(d, batch=-1) == INVALID
    assert prefill(d, T=-5) == INVALID
    assert prefill(d, num_slots=-1) == INVALID
    assert prefill(d, out=P) == INVALID           # out aliases x
    assert update(d, q=-1) == INVALID
    assert update(d, out=P) == INVALID
    # zero work: success without a launch
    assert prefill(d, batch=0) == OK
    assert prefill(d, T=0) == OK
    assert update(d, batch=0) == OK
    assert update(d, q=0) == OK


def test_checkpoint_rules():
    d = desc(dilation=3, state_len=9)
    assert prefill(d, ckpt=sc_ckpt_desc(grid=8, cu_ckpt=P, ckpt_slots=P), batch=0) == INVALID
    assert prefill(d, ckpt=sc_ckpt_desc(grid=-1, cu_ckpt=P, ckpt_slots=P), batch=0) == INVALID
    assert prefill(d, ckpt=sc_ckpt_desc(grid=16, cu_ckpt=None, ckpt_slots=P)) == NULL
    # (ckpt_slots NULL is an empty destination array: accepted, nothing exported;
    # covered on the GPU)
    # zero work needs no pointers at all (empty tensors carry NULL pointers)
    assert prefill(d, x=None, out=None, w=None, qsl=None, slots=None, h=None, pool=None,
                   ckpt=sc_ckpt_desc(grid=16, cu_ckpt=None, ckpt_slots=None), T=0) == OK
    assert prefill(d, ckpt=sc_ckpt_desc(grid=16, cu_ckpt=P, ckpt_slots=P), batch=0) == OK
    assert prefill(d, ckpt=sc_ckpt_desc(grid=0, cu_ckpt=None, ckpt_slots=None), batch=0) == OK


def test_state_copy_validation():
    L = scs.lib()
    assert L.sc_state_gather(P, 4, 96, P, 1, 3, None, None) == NULL
    assert L.sc_state_gather(P, 4, 0, P, 1, 3, P2, None) == INVALID
    assert L.sc_state_gather(P, 4, 96, P, 0, 3, P2, None) == INVALID
    assert L.sc_state_gather(P, 4, 96, P, 1, 0, P2, None) == OK
    assert L.sc_state_scatter(P, 96, None, 1, 3, P2, 4, None) == NULL
    assert L.sc_state_scatter(P, 96, P, 1, -1, P2, 4, None) == INVALID
    assert L.sc_state_scatter(P, 96, P, 1, 0, P2, 4, None) == OK


def cca_desc(**kw):
    d = dict(num_q_heads=16, num_kv_heads=4, head_dim=128, t0=2, t1=2, dtype=1,
             q_row_stride=2048, k_row_stride=512, v_cur_row_stride=256,
             v_del_row_stride=256, out_row_stride=3072, decode_slot_stride=1,
             prefill_slot_stride=1)
    d.update(kw)
    return sc_cca_desc(**d)


def cca(d, *, nd=2, npf=1, T=5, di=P, cs=P, ds=P, dslots=P, qsl=P, h=P):
    return scs.lib().sc_cca_qk_conv(ctypes.byref(d), P, P, P, P, P2, P, P, P, P, di, cs,
                                    ds, 8, nd, dslots, npf, qsl, P, h, T, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), DTYPE),
    (dict(num_kv_heads=3), INVALID),
    (dict(head_dim=127), INVALID),
    (dict(t0=0), INVALID),
    (dict(q_row_stride=100), INVALID),
    (dict(out_row_stride=3071), INVALID),
    (dict(decode_slot_stride=0), INVALID),
])
def test_cca_validation(kw, status):
    assert cca(cca_desc(**kw)) == status


def test_cca_null_and_empty():
    d = cca_desc()
    assert cca(d, dslots=None) == NULL
    assert cca(d, qsl=None) == NULL
    assert cca(d, h=None) == NULL
    assert cca(d, cs=None) == NULL
    assert cca(d, T=1) == INVALID                 # fewer rows than decodes
    assert cca(d, nd=0, npf=0, T=0) == OK
    assert cca(d, nd=0, npf=1, T=0, dslots=None) == OK


def test_fuse_descriptor_rules():
    from stateful_causal_short_amd import sc_conv_fuse
    d = desc()
    for call in (prefill, update, spec):
        dd = desc(state_len=6) if call is spec else d
        assert call(dd, fuse=sc_conv_fuse(accumulate=2), batch=0) == INVALID
        assert call(dd, fuse=sc_conv_fuse(token_indices=P, num_physical_rows=0), batch=0) == INVALID
        assert call(dd, fuse=sc_conv_fuse(outer_residual=P, outer_row_stride=63), batch=0) == INVALID
        assert call(dd, fuse=sc_conv_fuse(accumulate=1, outer_residual=P, outer_row_stride=64),
                    batch=0) == OK
        # the outer residual must not be the output
        assert call(dd, fuse=sc_conv_fuse(outer_residual=P2, outer_row_stride=64)) == INVALID


def test_validate_metadata_host_rules():
    lib = scs.lib()
    assert lib.sc_validate_metadata(None, None, 1, 0, 0, 0, None) == OK     # nothing to check
    assert lib.sc_validate_metadata(None, None, 1, 3, 10, 4, None) == OK    # both skipped
    assert lib.sc_validate_metadata(None, None, 1, -1, 0, 0, None) == INVALID
    assert lib.sc_validate_metadata(None, None, 0, 1, 0, 0, None) == INVALID
    assert lib.sc_validate_metadata(None, None, 1, 1, -5, 0, None) == INVALID
    # a stride whose index span overflows is rejected before any copy (the
    # pointer is never dereferenced)
    assert lib.sc_validate_metadata(None, ctypes.c_void_p(256), 1 << 62, 3, 0, 4, None) == INVALID
    assert scs.lib().sc_status_string(-6) == b"HIP runtime error (launch or copy)"


def test_binding_accepts_empty_row_tensors():
    import numpy as np
    import torch
    for shape in ((0, 8), (0, 1), (0, 4096)):
        t = torch.from_numpy(np.zeros(shape, np.float32))
        assert scs._rows(t, "x") == shape[1]
    with pytest.raises(ValueError):
        scs._rows(torch.zeros(3, 4).t(), "x")       # channel stride 3


def test_binding_rejects_host_tensors():
    """Every tensor argument is a device address for a kernel: the binding
    refuses a host tensor before anything reaches the library."""
    import torch
    C = 64
    x = torch.zeros(4, C, dtype=torch.bfloat16)
    w = torch.zeros(C, 4, dtype=torch.bfloat16)
    pool = torch.zeros(8, C, 3, dtype=torch.bfloat16)
    idx = torch.arange(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="on the GPU"):
        scs.sc_conv_update(x, torch.zeros_like(x), w, None, pool, idx, q=1)
    qsl = torch.tensor([0, 4], dtype=torch.int32)
    h = torch.ones(1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="on the GPU"):
        scs.sc_conv_prefill_varlen(x, torch.zeros_like(x), w, None, pool, qsl, idx[:1], h)
    with pytest.raises(ValueError, match="on the GPU"):
        scs.sc_state_gather(pool, idx, torch.zeros(4, C, 3, dtype=torch.bfloat16))


def test_binding_checks_dtypes_and_batch_coverage():
    """Float tensors share x's dtype (a bf16 pool read as fp32 would run past
    its end) and per-request arrays cover the batch; both are refused before
    any device address is taken, so meta tensors (no storage) suffice."""
    import torch
    C = 64
    m = dict(device="meta")
    x = torch.empty(8, C, dtype=torch.bfloat16, **m)
    w = torch.empty(C, 4, dtype=torch.bfloat16, **m)
    pool = torch.empty(16, C, 3, dtype=torch.bfloat16, **m)
    idx = torch.empty(8, dtype=torch.int32, **m)
    for kw, what in ((dict(out=torch.empty(8, C, dtype=torch.float32, **m)), "out"),
                     (dict(weight=w.float()), "weight"),
                     (dict(state_pool=pool.float()), "state_pool"),
                     (dict(bias=torch.empty(C, dtype=torch.float32, **m)), "bias"),
                     (dict(bias=torch.empty(C - 1, dtype=torch.bfloat16, **m)), "bias"),
                     (dict(out=torch.empty(7, C, dtype=torch.bfloat16, **m)), "out"),
                     (dict(state_indices=idx[:7]), "state_indices")):
        a = dict(x=x, out=torch.empty_like(x), weight=w, bias=None, state_pool=pool,
                 state_indices=idx)
        a.update(kw)
        with pytest.raises(ValueError, match=what):
            scs.sc_conv_update(a["x"], a["out"], a["weight"], a["bias"], a["state_pool"],
                               a["state_indices"], q=1)
    with pytest.raises(ValueError, match="num_accepted_tokens"):
        scs.sc_conv_update_spec(x, torch.empty_like(x), w, None, pool, idx[:2],
                                torch.empty(1, dtype=torch.int32, **m), q=4)
    qsl = torch.empty(4, dtype=torch.int32, **m)
    with pytest.raises(ValueError, match="has_initial_state"):
        scs.sc_conv_prefill_varlen(x, torch.empty_like(x), w, None, pool, qsl, idx,
                                   torch.empty(2, dtype=torch.uint8, **m))


def test_binding_checks_state_copy_rows():
    """Gather and scatter copy whole slot rows: the pool and the dense buffer
    must agree on the row size and the dense buffer must hold a row per index."""
    import torch
    m = dict(device="meta", dtype=torch.bfloat16)
    pool = torch.empty(16, 64, 3, **m)
    idx = torch.empty(4, dtype=torch.int32, device="meta")
    with pytest.raises(ValueError, match="bytes"):
        scs.sc_state_gather(pool, idx, torch.empty(4, 64, 2, **m))
    with pytest.raises(ValueError, match="bytes"):
        scs.sc_state_scatter(torch.empty(4, 64, 3, dtype=torch.float32, device="meta"), idx, pool)
    with pytest.raises(ValueError, match="dense"):
        scs.sc_state_gather(pool, idx, torch.empty(3, 64, 3, **m))


def test_binding_checks_cca_shapes():
    """The CCA kernels address every tensor from the head counts and q's row
    count: a tensor of the wrong shape is refused before any device address is
    taken (meta tensors, no storage)."""
    import torch
    nq, nkv, hd, t0, t1, T, S = 4, 2, 16, 2, 2, 10, 6
    C, vd, W, n = (nq + nkv) * hd, nkv * hd // 2, (nq + 2 * nkv) * hd, t0 + t1 - 2
    m = dict(device="meta", dtype=torch.bfloat16)
    good = dict(q=torch.empty(T, nq * hd, **m), k=torch.empty(T, nkv * hd, **m),
                v_cur=torch.empty(T, vd, **m), v_del=torch.empty(T, vd, **m),
                out=torch.empty(T, W, **m), w_dw=torch.empty(C, t0, **m),
                b_dw=torch.empty(C, **m), w_gr=torch.empty(C, hd, t1, **m),
                b_gr=torch.empty(C, **m), delayed_init=torch.empty(vd, **m),
                conv_state=torch.empty(S, C, n, **m), delayed_state=torch.empty(S, vd, **m))
    bad = [("q", torch.empty(T, nq * hd + 8, **m)), ("k", torch.empty(T - 1, nkv * hd, **m)),
           ("v_cur", torch.empty(T, vd - 8, **m)), ("v_del", torch.empty(T + 1, vd, **m)),
           ("out", torch.empty(T, W - 8, **m)), ("out", torch.empty(T - 1, W, **m)),
           ("w_dw", torch.empty(C, t0 + 1, **m)), ("b_dw", torch.empty(C - 1, **m)),
           ("w_gr", torch.empty(C, hd, t1 + 1, **m)), ("b_gr", torch.empty(C + 8, **m)),
           ("delayed_init", torch.empty(vd + 1, **m)),
           ("conv_state", torch.empty(S, C, n + 1, **m)),
           ("conv_state", torch.empty(S, C - 16, n, **m)),
           ("delayed_state", torch.empty(S - 1, vd, **m)),
           ("delayed_state", torch.empty(S, vd * 2, **m))]
    idx = torch.empty(2, dtype=torch.int32, device="meta")
    for name, t in bad:
        a = dict(good)
        a[name] = t
        with pytest.raises(ValueError, match=name):
            scs.sc_cca_qk_conv(a["q"], a["k"], a["v_cur"], a["v_del"], a["out"], a["w_dw"],
                               a["b_dw"], a["w_gr"], a["b_gr"], a["delayed_init"],
                               a["conv_state"], a["delayed_state"], idx, None, None, None,
                               num_q_heads=nq, num_kv_heads=nkv, head_dim=hd, t0=t0, t1=t1)
    with pytest.raises(ValueError, match="head"):
        scs.sc_cca_qk_conv(*good.values(), idx, None, None, None, num_q_heads=3,
                           num_kv_heads=2, head_dim=hd, t0=t0, t1=t1)
    # the good shapes pass the shape check and stop at the first device address
    with pytest.raises(ValueError, match="on the GPU"):
        scs.sc_cca_qk_conv(*good.values(), idx, None, None, None, num_q_heads=nq,
                           num_kv_heads=nkv, head_dim=hd, t0=t0, t1=t1)


def test_library_shares_torchs_hip_runtime():
    """Loading the library before torch must not put a second HIP runtime in
    the process: the binding imports torch first, so the library binds to
    torch's runtime and device pointers and streams mean the same to both."""
    import subprocess
    import sys
    code = ("import stateful_causal_short_amd as scs; scs.lib(); import torch; "
            "maps = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "1"
