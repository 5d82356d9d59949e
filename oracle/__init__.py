"""Python front of the CPU oracle (``oracle/oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``. The product package never imports
it. Arguments are NumPy arrays from :mod:`synthetic`; nothing here touches a GPU.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .build import LIB_PATH, build_oracle

F32, BF16, F64 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "f64": F64}
_NP = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build_oracle()
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.oracle_conv.restype = I32
        L.oracle_conv.argtypes = [I32, I32, I32, I32, I32, I32, P, I64, P, I64, P,
                                  P, P, P, I32, I32, I32, I32, I32, P, I64, P, I32, P, P,
                                  I64, P, I32, P, P, P, P, P, I64, P, I64, I32]
        L.oracle_conv_spec.restype = I32
        L.oracle_conv_spec.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, P, I64, P, I64,
                                       P, P, P, P, I32, I32, I32, P, I64, P, P, P, P, I64,
                                       P, I64, I32]
        L.oracle_conv_spec_varlen.restype = I32
        L.oracle_conv_spec_varlen.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, P, I64,
                                              P, I64, P, P, P, P, I32, I32, P, P, I64, P, P,
                                              P, P, I64, P, I64, I32]
        L.oracle_cca.restype = I32
        L.oracle_cca.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32,
                                 P, I64, P, I64, P, I64, P, I64, P, I64, P,
                                 P, P, P, P, P, P, P, I32, I32, P, I64, I32, P, P,
                                 I64, P, P, P, P, I32]
        L.oracle_state_gather.restype = I32
        L.oracle_state_gather.argtypes = [I32, I64, P, I32, P, I64, I32, P]
        L.oracle_state_scatter.restype = I32
        L.oracle_state_scatter.argtypes = [I32, I64, P, P, I64, I32, P, I32]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def double_to_bf16(v: float) -> int:
    return int(lib().oracle_double_to_bf16(float(v)))


def _layout(case) -> int:
    return 1 if getattr(case, "layout", "ds") == "sd" else 0


def _state_len(case, pool) -> int:
    """S of a (num_slots, C, S) pool, or of a (num_slots, S, C) one in SD layout."""
    return pool.shape[1] if _layout(case) else pool.shape[2]


def _fuse_args(x, token_indices, resid, outer):
    ti = _c(token_indices, np.int32)
    rs = _c(resid)
    ou = _c(outer)
    return (_p(ti), _p(rs), 0 if rs is None else rs.shape[1],
            _p(ou), 0 if ou is None else ou.shape[1])


def conv(case, *, out_dtype: Optional[str] = None, absum: bool = False,
         row_mask: Optional[np.ndarray] = None, nthreads: Optional[int] = None,
         pool: Optional[np.ndarray] = None, x: Optional[np.ndarray] = None,
         token_indices: Optional[np.ndarray] = None, resid: Optional[np.ndarray] = None,
         outer: Optional[np.ndarray] = None):
    """Run the depthwise oracle on a :class:`synthetic.ConvCase`.

    Returns ``(out, pool_after, absum_or_None)``; the case's arrays are not
    modified (the pool is copied unless ``pool`` is passed, which is then
    updated in place and returned). ``x`` overrides the case's rows (a
    physical batch tensor addressed through ``token_indices``); ``resid`` and
    ``outer`` (physical rows) are added to the result; ``out`` has x's rows.
    """
    odt = out_dtype or case.dtype
    T, C = case.T, case.C
    x = _c(case.x if x is None else x)
    out = np.zeros((x.shape[0], C), _NP[odt])
    ab = np.zeros((T, C), np.float64) if absum else None
    pool = np.array(case.pool, copy=True) if pool is None else pool
    assert pool.flags.c_contiguous
    w = _c(case.w)
    bias = _c(case.bias)
    dsl = _c(case.decode_slots, np.int32)
    dh = _c(case.decode_h, np.uint8)
    qsl = _c(case.qsl_p, np.int32)
    psl = _c(case.prefill_slots, np.int32)
    ph = _c(case.prefill_h, np.uint8)
    cu = _c(case.cu_ckpt, np.int32)
    cks = _c(case.ckpt_slots, np.int32)
    rm = _c(row_mask, np.uint8)
    rc = lib().oracle_conv(
        C, case.K, case.d, 1 if case.act == "silu" else 0, _DT[case.dtype],
        _DT[odt], _p(x), C, _p(out), C, _p(ab), _p(w), _p(bias), _p(pool),
        pool.shape[0], _state_len(case, pool), _layout(case), case.num_decodes, case.q,
        _p(dsl), 1, _p(dh),
        case.num_prefills, _p(qsl), _p(psl), 1, _p(ph), case.ckpt_grid,
        _p(cu), _p(cks), _p(rm), *_fuse_args(x, token_indices, resid, outer),
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_conv failed: {rc}")
    return out, pool, ab


def conv_spec(case, num_accepted, *, out_dtype: Optional[str] = None, absum: bool = False,
              row_mask: Optional[np.ndarray] = None, nthreads: Optional[int] = None,
              pool: Optional[np.ndarray] = None, x: Optional[np.ndarray] = None,
              token_indices: Optional[np.ndarray] = None, resid: Optional[np.ndarray] = None,
              outer: Optional[np.ndarray] = None):
    """Speculative update (rolling buffer) on a ConvCase whose decodes are the
    spec requests (q tokens each) and whose pool is (num_slots, C, S), S >= H.
    Returns (out, pool_after, absum_or_None); fusion arguments as in conv()."""
    odt = out_dtype or case.dtype
    T, C = case.num_decode_tokens, case.C
    x = _c(case.x[:T] if x is None else x)
    out = np.zeros((x.shape[0], C), _NP[odt])
    ab = np.zeros((T, C), np.float64) if absum else None
    pool = np.array(case.pool, copy=True) if pool is None else pool
    S = _state_len(case, pool)
    dsl = _c(case.decode_slots, np.int32)
    acc = _c(num_accepted, np.int32)
    rm = _c(row_mask, np.uint8)
    rc = lib().oracle_conv_spec(
        C, case.K, case.d, S, _layout(case), 1 if case.act == "silu" else 0, _DT[case.dtype],
        _DT[odt],
        _p(x), C, _p(out), C, _p(ab), _p(_c(case.w)), _p(_c(case.bias)), _p(pool),
        pool.shape[0], case.num_decodes, case.q, _p(dsl), 1, _p(acc), _p(rm),
        *_fuse_args(x, token_indices, resid, outer), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_conv_spec failed: {rc}")
    return out, pool, ab


def conv_spec_varlen(case, num_accepted, qsl, *, out_dtype: Optional[str] = None,
                     absum: bool = False, row_mask: Optional[np.ndarray] = None,
                     nthreads: Optional[int] = None, pool: Optional[np.ndarray] = None,
                     x: Optional[np.ndarray] = None, token_indices: Optional[np.ndarray] = None,
                     resid: Optional[np.ndarray] = None, outer: Optional[np.ndarray] = None):
    """Speculative update with a draft count per request: request r owns rows
    [qsl[r], qsl[r+1]) of x; its slot is case.decode_slots[r] (batch =
    case.num_decodes). Rows of skipped requests (0 or more than S drafts) keep
    the zeros `out` starts with. Returns (out, pool_after, absum_or_None)."""
    odt = out_dtype or case.dtype
    qsl = _c(qsl, np.int32)
    B = case.num_decodes
    T = int(qsl[B])
    C = case.C
    x = _c(case.x[:T] if x is None else x)
    out = np.zeros((x.shape[0], C), _NP[odt])
    ab = np.zeros((T, C), np.float64) if absum else None
    pool = np.array(case.pool, copy=True) if pool is None else pool
    S = _state_len(case, pool)
    dsl = _c(case.decode_slots, np.int32)
    acc = _c(num_accepted, np.int32)
    rm = _c(row_mask, np.uint8)
    rc = lib().oracle_conv_spec_varlen(
        C, case.K, case.d, S, _layout(case), 1 if case.act == "silu" else 0, _DT[case.dtype],
        _DT[odt], _p(x), C, _p(out), C, _p(ab), _p(_c(case.w)), _p(_c(case.bias)), _p(pool),
        pool.shape[0], B, _p(qsl), _p(dsl), 1, _p(acc), _p(rm),
        *_fuse_args(x, token_indices, resid, outer), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_conv_spec_varlen failed: {rc}")
    return out, pool, ab


def cca(case, *, out_dtype: Optional[str] = None, dw_mode: int = 2,
        absum: bool = False, row_mask: Optional[np.ndarray] = None,
        nthreads: Optional[int] = None, io_override=None, chain_diff: Optional[list] = None,
        allow: Optional[list] = None):
    """Run the CCA oracle on a :class:`synthetic.CcaCase`.

    Returns ``(out, conv_state_after, delayed_state_after, absum_or_None)``.
    ``dw_mode``: 2 (default) the depthwise intermediate is its exact value
    rounded once to the io dtype; 0 the unrounded double sum (float64 pins);
    1 an fp32 fma chain rounded afterwards (diagnostic only).
    ``io_override`` = (dtype_name, dict of arrays) lets pins feed float64 copies.
    ``chain_diff``: a list that receives the number of depthwise values an fp32
    fma chain would round differently from the exact value (dw_mode 2, bf16).
    ``allow``: a list that receives a (T, W) float64 array (dw_mode 2): for each
    conv output, the most it moves when its depthwise inputs are summed in fp32
    in any order before their rounding (zero where no input lies within the
    fp32 summation bound of a rounding boundary; zero for value columns).
    """
    io = case.dtype
    arrs = dict(q=case.q, k=case.k, v_cur=case.v_cur, v_del=case.v_del,
                w_dw=case.w_dw, b_dw=case.b_dw, w_gr=case.w_gr, b_gr=case.b_gr,
                delayed_init=case.delayed_init, conv_state=case.conv_state,
                delayed_state=case.delayed_state)
    if io_override is not None:
        io, over = io_override
        arrs.update(over)
    odt = out_dtype or io
    a = {k: (None if v is None else np.array(v, copy=True, order="C"))
         for k, v in arrs.items()}
    T, Wd = case.T, case.out_width
    out = np.zeros((T, Wd), _NP[odt])
    ab = np.zeros((T, Wd), np.float64) if absum else None
    dsl = _c(case.decode_slots, np.int32)
    qsl = _c(case.qsl_p, np.int32)
    psl = _c(case.prefill_slots, np.int32)
    ph = _c(case.prefill_h, np.uint8)
    rm = _c(row_mask, np.uint8)
    nd = np.zeros(1, np.int64) if chain_diff is not None else None
    al = np.zeros((T, Wd), np.float64) if allow is not None else None
    rc = lib().oracle_cca(
        case.nq, case.nkv, case.hd, case.t0, case.t1, _DT[io], _DT[odt], dw_mode,
        _p(a["q"]), a["q"].shape[1], _p(a["k"]), a["k"].shape[1],
        _p(a["v_cur"]), a["v_cur"].shape[1], _p(a["v_del"]), a["v_del"].shape[1],
        _p(out), Wd, _p(ab), _p(a["w_dw"]), _p(a["b_dw"]), _p(a["w_gr"]),
        _p(a["b_gr"]), _p(a["delayed_init"]), _p(a["conv_state"]),
        _p(a["delayed_state"]), case.num_slots, case.num_decodes, _p(dsl), 1,
        case.num_prefills, _p(qsl), _p(psl), 1, _p(ph), _p(rm), _p(nd), _p(al),
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_cca failed: {rc}")
    if chain_diff is not None:
        chain_diff.append(int(nd[0]))
    if allow is not None:
        allow.append(al)
    return out, a["conv_state"], a["delayed_state"], ab


def state_gather(pool: np.ndarray, idx: np.ndarray, dense: np.ndarray) -> np.ndarray:
    pool = np.ascontiguousarray(pool)
    idx = _c(idx, np.int32)
    row = int(np.prod(pool.shape[1:]))
    rc = lib().oracle_state_gather(pool.itemsize, row, _p(pool), pool.shape[0],
                                   _p(idx), 1, idx.shape[0], _p(dense))
    assert rc == 0
    return dense


def state_scatter(dense: np.ndarray, idx: np.ndarray, pool: np.ndarray) -> np.ndarray:
    dense = np.ascontiguousarray(dense)
    idx = _c(idx, np.int32)
    row = int(np.prod(pool.shape[1:]))
    rc = lib().oracle_state_scatter(pool.itemsize, row, _p(dense), _p(idx), 1,
                                    idx.shape[0], _p(pool), pool.shape[0])
    assert rc == 0
    return pool
