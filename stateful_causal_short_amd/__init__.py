"""MI355X (gfx950) stateful causal short convolution.

Thin Python binding of ``libstatefulconv.so`` (C ABI in
``include/statefulconv.h``). Every function here only marshals arguments —
device pointers, sizes, strides, the current HIP stream — and calls the
library; every step of the computation runs in the library's HIP kernels.
PyTorch provides device memory and streams. There is no CPU fallback: if the
library is missing, import-time loading fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libstatefulconv.so")

SC_OK = 0
SC_ABI_VERSION = 3   # the struct layouts and signatures below
STATUS = {0: "SC_OK", -1: "SC_ERR_NULL_ARG", -2: "SC_ERR_INVALID_ARG",
          -3: "SC_ERR_DTYPE", -4: "SC_ERR_STATE_CAPACITY",
          -5: "SC_ERR_UNSUPPORTED", -6: "SC_ERR_HIP"}
SC_DTYPE_F32, SC_DTYPE_BF16 = 0, 1
SC_ACT_NONE, SC_ACT_SILU = 0, 1
SC_STATE_DS, SC_STATE_SD = 0, 1

EXPORTS = ("sc_conv_prefill_varlen", "sc_conv_update", "sc_conv_update_spec",
           "sc_conv_update_spec_varlen", "sc_validate_metadata", "sc_state_gather",
           "sc_state_scatter", "sc_cca_qk_conv", "sc_status_string",
           "sc_abi_version")


class ScError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().sc_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")


class sc_conv_desc(ctypes.Structure):
    _fields_ = [("channels", ctypes.c_int32), ("width", ctypes.c_int32),
                ("dilation", ctypes.c_int32), ("state_len", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("x_row_stride", ctypes.c_int64), ("out_row_stride", ctypes.c_int64),
                ("state_indices_stride", ctypes.c_int64), ("state_layout", ctypes.c_int32)]


class sc_ckpt_desc(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("cu_ckpt", ctypes.c_void_p),
                ("ckpt_slots", ctypes.c_void_p)]


class sc_conv_fuse(ctypes.Structure):
    _fields_ = [("token_indices", ctypes.c_void_p), ("num_physical_rows", ctypes.c_int64),
                ("accumulate", ctypes.c_int32), ("outer_residual", ctypes.c_void_p),
                ("outer_row_stride", ctypes.c_int64)]


class sc_cca_desc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("t0", ctypes.c_int32),
                ("t1", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q_row_stride", ctypes.c_int64), ("k_row_stride", ctypes.c_int64),
                ("v_cur_row_stride", ctypes.c_int64), ("v_del_row_stride", ctypes.c_int64),
                ("out_row_stride", ctypes.c_int64), ("decode_slot_stride", ctypes.c_int64),
                ("prefill_slot_stride", ctypes.c_int64)]


_lib = None


def lib():
    """Load libstatefulconv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch first: it carries its own HIP runtime, and the library must
        # bind to that one (loaded first, the library would pull in the
        # system runtime and the process would hold two, whose device
        # pointers and streams the other does not know)
        _torch()
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        D = ctypes.POINTER(sc_conv_desc)
        L.sc_conv_prefill_varlen.restype = I32
        F = ctypes.POINTER(sc_conv_fuse)
        L.sc_conv_prefill_varlen.argtypes = [D, P, P, P, P, P, I32, P, P, P, I32, I64,
                                             ctypes.POINTER(sc_ckpt_desc), F, P]
        L.sc_conv_update.restype = I32
        L.sc_conv_update.argtypes = [D, P, P, P, P, P, I32, P, P, I32, I32, F, P]
        L.sc_conv_update_spec.restype = I32
        L.sc_conv_update_spec.argtypes = [D, P, P, P, P, P, I32, P, P, I32, I32, F, P]
        L.sc_conv_update_spec_varlen.restype = I32
        L.sc_conv_update_spec_varlen.argtypes = [D, P, P, P, P, P, I32, P, P, P, I32, I64, I32,
                                                 F, P]
        L.sc_validate_metadata.restype = I32
        L.sc_validate_metadata.argtypes = [P, P, I64, I32, I64, I32, P]
        L.sc_state_gather.restype = I32
        L.sc_state_gather.argtypes = [P, I32, I64, P, I64, I32, P, P]
        L.sc_state_scatter.restype = I32
        L.sc_state_scatter.argtypes = [P, I64, P, I64, I32, P, I32, P]
        L.sc_cca_qk_conv.restype = I32
        L.sc_cca_qk_conv.argtypes = [ctypes.POINTER(sc_cca_desc), P, P, P, P, P, P, P,
                                     P, P, P, P, P, I32, I32, P, I32, P, P, P, I64, P]
        L.sc_status_string.restype = ctypes.c_char_p
        L.sc_status_string.argtypes = [I32]
        L.sc_abi_version.restype = I32
        L.sc_abi_version.argtypes = []
        if L.sc_abi_version() != SC_ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.sc_abi_version()}, the binding "
                               f"expects {SC_ABI_VERSION}: rebuild the library")
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
_torch_mod = None
_dtype_codes = None


def _torch():
    global _torch_mod
    if _torch_mod is None:
        import torch
        _torch_mod = torch
    return _torch_mod


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None passes through). Every tensor argument
    is read or written by a kernel, so a host tensor is rejected here rather
    than handed to the GPU as an address."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a tensor on the GPU, got one on {t.device}")
    return t.data_ptr()


def _stream(stream, like=None) -> Optional[int]:
    """Raw HIP stream: the given one, else torch's current stream on the device
    of tensor `like` (or the current device)."""
    torch = _torch()
    if like is not None and not like.is_cuda:
        raise ValueError(f"expected a tensor on the GPU, got one on {like.device}")
    cur = torch.cuda.current_device()
    if like is not None and like.get_device() != cur:
        # the library launches on the current device
        raise ValueError(f"tensors are on cuda:{like.get_device()} but the current device is "
                         f"cuda:{cur}; call under torch.cuda.device({like.get_device()})")
    if stream is not None:
        return stream.cuda_stream
    return torch._C._cuda_getCurrentRawStream(cur)


def _dtype_code(t) -> int:
    global _dtype_codes
    if _dtype_codes is None:
        torch = _torch()
        _dtype_codes = {torch.bfloat16: SC_DTYPE_BF16, torch.float32: SC_DTYPE_F32}
    return _dtype_codes.get(t.dtype, -1)


def _rows(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D tensor")
    if t.numel() == 0:
        return t.shape[1]        # no rows to address (zero-work calls are no-ops)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: expected a 2-D tensor with unit channel stride")
    # with at most one row the row stride is never used
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _index_stride(t, name) -> int:
    """Row stride of int32 slot indices: 1-D, or 2-D whose column 0 holds the slot."""
    torch = _torch()
    if t.dtype != torch.int32:
        raise ValueError(f"{name}: expected int32")
    if t.dim() not in (1, 2):
        raise ValueError(f"{name}: expected a 1-D or 2-D tensor")
    # with at most one row the stride is never used (empty tensors may report 0)
    return t.stride(0) if t.shape[0] > 1 else 1


def _index(t, name) -> Tuple[int, int]:
    return _ptr(t), _index_stride(t, name)


def _flags(t, name):
    torch = _torch()
    if t is None:
        return None
    if t.dtype not in (torch.bool, torch.uint8) or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous bool/uint8 tensor")
    return _ptr(t)


def _check(fn: str, status: int):
    if status != SC_OK:
        raise ScError(fn, status)


def _fuse(x, out, token_indices, accumulate, outer_residual):
    """The optional residual-fusion / row-map descriptor (None = plain call)."""
    if token_indices is None and not accumulate and outer_residual is None:
        return None
    torch = _torch()
    if token_indices is not None and (token_indices.dtype != torch.int32 or
                                      not token_indices.is_contiguous()):
        raise ValueError("token_indices: expected a contiguous int32 tensor")
    if outer_residual is not None and (outer_residual.shape[0] != out.shape[0] or
                                       outer_residual.dtype != x.dtype):
        raise ValueError("outer_residual: expected as many rows as out, in x's dtype")
    if token_indices is not None and out.shape[0] != x.shape[0]:
        raise ValueError("with token_indices, x and out are the full batch tensors")
    return ctypes.byref(sc_conv_fuse(
        token_indices=_ptr(token_indices), num_physical_rows=x.shape[0],
        accumulate=1 if accumulate else 0, outer_residual=_ptr(outer_residual),
        outer_row_stride=0 if outer_residual is None else _rows(outer_residual, "outer_residual")))


def _covers(batch, **tensors):
    """Per-request arrays (slots, flags, counts) must hold at least `batch`
    entries: the kernels read entry r for every request r."""
    for name, t in tensors.items():
        if t is not None and t.shape[0] < batch:
            raise ValueError(f"{name}: {t.shape[0]} entries for {batch} requests")


def _conv_desc(x, out, weight, state_pool, dilation, activation, state_indices,
               state_layout="ds", bias=None):
    C = x.shape[1]
    K = weight.shape[-1]
    act = {"silu": SC_ACT_SILU, "none": SC_ACT_NONE, None: SC_ACT_NONE}[activation]
    # one dtype for every float tensor: the library reads them all as x's
    for name, t in (("out", out), ("weight", weight), ("bias", bias),
                    ("state_pool", state_pool)):
        if t is not None and t.dtype != x.dtype:
            raise ValueError(f"{name}: dtype {t.dtype} differs from x's {x.dtype}")
    if out.dim() != 2 or out.shape[1] != C or out.shape[0] < x.shape[0]:
        raise ValueError("out: expected at least as many (rows, C) as x")
    if weight.numel() != C * K or not weight.is_contiguous():
        raise ValueError("weight: expected a contiguous (C, K) or (C, 1, K) tensor")
    if bias is not None and (bias.numel() != C or not bias.is_contiguous()):
        raise ValueError("bias: expected a contiguous tensor of C entries")
    sd = {"ds": False, "sd": True}[state_layout]
    if not state_pool.is_contiguous() or state_pool.dim() != 3 or \
            state_pool.shape[2 if sd else 1] != C:
        raise ValueError("state_pool: expected a contiguous (num_slots, C, S) tensor, or "
                         "(num_slots, S, C) with state_layout='sd'")
    sst = _index_stride(state_indices, "state_indices")
    return sc_conv_desc(channels=C, width=K, dilation=dilation,
                        state_len=state_pool.shape[1 if sd else 2], dtype=_dtype_code(x),
                        activation=act, x_row_stride=_rows(x, "x"),
                        out_row_stride=_rows(out, "out"), state_indices_stride=sst,
                        state_layout=SC_STATE_SD if sd else SC_STATE_DS)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def sc_conv_prefill_varlen(x, out, weight, bias, state_pool, query_start_loc,
                           state_indices, has_initial_state, *, dilation: int = 1,
                           activation: Optional[str] = "silu", ckpt=None, token_indices=None,
                           accumulate: bool = False, outer_residual=None,
                           state_layout: str = "ds", stream=None):
    """Varlen prefill conv; updates ``state_pool`` in place.

    x, out: (num_tokens, C); weight (C, K); bias (C) or None; state_pool
    (num_slots, C, S), S >= (K-1)*dilation (window in the first (K-1)*dilation
    entries of each row); query_start_loc int32 (B+1);
    state_indices int32 (B) or (B, n) using column 0; has_initial_state
    bool/uint8 (B); ckpt = None or (grid, cu_ckpt int32 (B+1), ckpt_slots int32).
    token_indices (int32, one per logical row) maps the call's rows to rows of
    x / out / outer_residual; accumulate adds the result to out's contents;
    outer_residual is added too.
    """
    desc = _conv_desc(x, out, weight, state_pool, dilation, activation, state_indices,
                      state_layout, bias)
    _covers(query_start_loc.shape[0] - 1, state_indices=state_indices,
            has_initial_state=has_initial_state)
    cd = None
    if ckpt is not None:
        grid, cu, slots = ckpt
        if grid:
            _covers(query_start_loc.shape[0], cu_ckpt=cu)
        cd = ctypes.byref(sc_ckpt_desc(grid=grid, cu_ckpt=_ptr(cu), ckpt_slots=_ptr(slots)))
    st = lib().sc_conv_prefill_varlen(
        ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(weight), _ptr(bias),
        _ptr(state_pool), state_pool.shape[0], _ptr(query_start_loc),
        _index(state_indices, "state_indices")[0],
        _flags(has_initial_state, "has_initial_state"),
        query_start_loc.shape[0] - 1,
        x.shape[0] if token_indices is None else token_indices.shape[0], cd,
        _fuse(x, out, token_indices, accumulate, outer_residual), _stream(stream, x))
    _check("sc_conv_prefill_varlen", st)


def sc_conv_update(x, out, weight, bias, state_pool, state_indices,
                   has_initial_state=None, *, q: int = 1, dilation: int = 1,
                   activation: Optional[str] = "silu", token_indices=None,
                   accumulate: bool = False, outer_residual=None, state_layout: str = "ds",
                   stream=None):
    """Decode / multi-token update: x (B*q, C) rows, request r owns rows
    [r*q, (r+1)*q) (logical rows, mapped by token_indices when given);
    updates ``state_pool`` in place."""
    rows = x.shape[0] if token_indices is None else token_indices.shape[0]
    if rows % max(q, 1):
        raise ValueError("rows must be a multiple of q")
    desc = _conv_desc(x, out, weight, state_pool, dilation, activation, state_indices,
                      state_layout, bias)
    B = rows // q if q else 0
    _covers(B, state_indices=state_indices, has_initial_state=has_initial_state)
    st = lib().sc_conv_update(
        ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(weight), _ptr(bias),
        _ptr(state_pool), state_pool.shape[0], _index(state_indices, "state_indices")[0],
        _flags(has_initial_state, "has_initial_state"), B, q,
        _fuse(x, out, token_indices, accumulate, outer_residual), _stream(stream, x))
    _check("sc_conv_update", st)


def sc_conv_update_spec(x, out, weight, bias, state_pool, state_indices, num_accepted_tokens,
                        *, q: int, dilation: int = 1, activation: Optional[str] = "silu",
                        token_indices=None, accumulate: bool = False, outer_residual=None,
                        state_layout: str = "ds", stream=None):
    """Speculative update on a rolling buffer: x (B*q, C) rows, request r owns
    rows [r*q, (r+1)*q); state_pool (num_slots, C, S) with S >= (K-1)*dilation;
    num_accepted_tokens int32 (B). Updates ``state_pool`` in place."""
    rows = x.shape[0] if token_indices is None else token_indices.shape[0]
    if q < 1 or rows % q:
        raise ValueError("rows must be a positive multiple of q")
    torch = _torch()
    if num_accepted_tokens.dtype != torch.int32 or not num_accepted_tokens.is_contiguous():
        raise ValueError("num_accepted_tokens: expected a contiguous int32 tensor")
    desc = _conv_desc(x, out, weight, state_pool, dilation, activation, state_indices,
                      state_layout, bias)
    _covers(rows // q, state_indices=state_indices, num_accepted_tokens=num_accepted_tokens)
    st = lib().sc_conv_update_spec(
        ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(weight), _ptr(bias),
        _ptr(state_pool), state_pool.shape[0], _index(state_indices, "state_indices")[0],
        _ptr(num_accepted_tokens), rows // q, q,
        _fuse(x, out, token_indices, accumulate, outer_residual), _stream(stream, x))
    _check("sc_conv_update_spec", st)


def sc_conv_update_spec_varlen(x, out, weight, bias, state_pool, state_indices,
                               num_accepted_tokens, query_start_loc, *, max_query_len: int,
                               dilation: int = 1, activation: Optional[str] = "silu",
                               token_indices=None, accumulate: bool = False,
                               outer_residual=None, state_layout: str = "ds", stream=None):
    """Speculative update with a draft count per request: request r owns rows
    [query_start_loc[r], query_start_loc[r+1]) of x (int32, batch+1 entries);
    max_query_len bounds every count (<= S). Updates ``state_pool`` in place."""
    torch = _torch()
    for name, t in (("num_accepted_tokens", num_accepted_tokens),
                    ("query_start_loc", query_start_loc)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous int32 tensor")
    batch = query_start_loc.shape[0] - 1
    if batch < 0:
        raise ValueError("query_start_loc: expected batch + 1 entries")
    rows = x.shape[0] if token_indices is None else token_indices.shape[0]
    desc = _conv_desc(x, out, weight, state_pool, dilation, activation, state_indices,
                      state_layout, bias)
    _covers(batch, state_indices=state_indices, num_accepted_tokens=num_accepted_tokens)
    st = lib().sc_conv_update_spec_varlen(
        ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(weight), _ptr(bias),
        _ptr(state_pool), state_pool.shape[0], _index(state_indices, "state_indices")[0],
        _ptr(num_accepted_tokens), _ptr(query_start_loc), batch, rows, max_query_len,
        _fuse(x, out, token_indices, accumulate, outer_residual), _stream(stream, x))
    _check("sc_conv_update_spec_varlen", st)


def sc_validate_metadata(query_start_loc=None, state_indices=None, *, num_tokens: int = 0,
                         num_slots: int = 0, batch: Optional[int] = None, stream=None) -> bool:
    """Host check of the device-side preconditions (syncs the stream): True if
    query_start_loc runs non-decreasing from 0 to num_tokens and the
    non-negative state indices are distinct and below num_slots."""
    torch = _torch()
    if batch is None:
        batch = (query_start_loc.shape[0] - 1) if query_start_loc is not None else \
            (state_indices.shape[0] if state_indices is not None else 0)
    if query_start_loc is not None and (query_start_loc.dtype != torch.int32 or
                                        not query_start_loc.is_contiguous()):
        raise ValueError("query_start_loc: expected a contiguous int32 tensor")
    p, s = _index(state_indices, "state_indices") if state_indices is not None else (None, 1)
    like = query_start_loc if query_start_loc is not None else state_indices
    st = lib().sc_validate_metadata(_ptr(query_start_loc), p, s, batch, num_tokens, num_slots,
                                    None if like is None else _stream(stream, like))
    if st == -2:
        return False
    _check("sc_validate_metadata", st)
    return True


def _copy_rows(state_pool, idx, dense) -> int:
    """Bytes per slot row; the pool and the dense buffer must agree on it, be
    contiguous, and the dense buffer must hold a row per index."""
    for name, t in (("state_pool", state_pool), ("dense", dense)):
        if not t.is_contiguous() or t.dim() < 1:
            raise ValueError(f"{name}: expected a contiguous tensor of rows")
    row_of = lambda t: (t.numel() // t.shape[0] if t.shape[0] else
                        math.prod(t.shape[1:])) * t.element_size()
    if row_of(state_pool) != row_of(dense):
        raise ValueError(f"state_pool rows hold {row_of(state_pool)} bytes, dense rows "
                         f"{row_of(dense)}")
    _covers(idx.shape[0], dense=dense)
    return max(row_of(dense), 1)


def sc_state_gather(state_pool, idx, dense, *, stream=None):
    """dense[i] = state_pool[idx[i]] (zeros for an index outside the pool)."""
    row = _copy_rows(state_pool, idx, dense)
    p, s = _index(idx, "idx")
    st = lib().sc_state_gather(_ptr(state_pool), state_pool.shape[0], row, p, s,
                               idx.shape[0], _ptr(dense), _stream(stream, dense))
    _check("sc_state_gather", st)


def sc_state_scatter(dense, idx, state_pool, *, stream=None):
    """state_pool[idx[i]] = dense[i] (indices outside the pool skipped)."""
    row = _copy_rows(state_pool, idx, dense)
    p, s = _index(idx, "idx")
    st = lib().sc_state_scatter(_ptr(dense), row, p, s, idx.shape[0], _ptr(state_pool),
                                state_pool.shape[0], _stream(stream, dense))
    _check("sc_state_scatter", st)


def _cca_shapes(q, k, v_cur, v_del, out, w_dw, b_dw, w_gr, b_gr, delayed_init, conv_state,
                delayed_state, nq, nkv, hd, t0, t1):
    """The CCA kernels address every tensor from the head counts and the token
    count (q's rows): each tensor must hold what they reach."""
    if nq < 1 or nkv < 1 or hd < 2 or nq % nkv or hd % 2 or t0 < 1 or t1 < 1:
        raise ValueError("expected num_q_heads a multiple of num_kv_heads, an even "
                         "head_dim and kernel widths >= 1")
    C, vd, W, n = (nq + nkv) * hd, nkv * hd // 2, (nq + 2 * nkv) * hd, t0 + t1 - 2
    T = q.shape[0] if q.dim() == 2 else -1
    for name, t, cols in (("q", q, nq * hd), ("k", k, nkv * hd), ("v_cur", v_cur, vd),
                          ("v_del", v_del, vd), ("out", out, W)):
        if t.dim() != 2 or t.shape[1] != cols or t.shape[0] != T:
            raise ValueError(f"{name}: expected ({T}, {cols}), got {tuple(t.shape)}")
    for name, t, numel in (("w_dw", w_dw, C * t0), ("b_dw", b_dw, C),
                           ("w_gr", w_gr, C * hd * t1), ("b_gr", b_gr, C),
                           ("delayed_init", delayed_init, vd)):
        if t is not None and t.numel() != numel:
            raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    slots = conv_state.shape[0] if conv_state.dim() else 0
    if conv_state.dim() != 3 or tuple(conv_state.shape[1:]) != (C, n):
        raise ValueError(f"conv_state: expected (num_slots, {C}, {n}), got "
                         f"{tuple(conv_state.shape)}")
    if delayed_state.dim() != 2 or tuple(delayed_state.shape) != (slots, vd):
        raise ValueError(f"delayed_state: expected ({slots}, {vd}), got "
                         f"{tuple(delayed_state.shape)}")


def sc_cca_qk_conv(q, k, v_cur, v_del, out, w_dw, b_dw, w_gr, b_gr, delayed_init,
                   conv_state, delayed_state, decode_slots, prefill_qsl, prefill_slots,
                   prefill_has_initial_state, *, num_q_heads: int, num_kv_heads: int,
                   head_dim: int, t0: int, t1: int, stream=None):
    """CCA q/k conv with per-request state; updates both state pools in place.

    Rows: len(decode_slots) one-token decodes, then prefills (prefill_qsl
    rebased to 0). Pass decode_slots / prefill tensors as None when absent."""
    _cca_shapes(q, k, v_cur, v_del, out, w_dw, b_dw, w_gr, b_gr, delayed_init, conv_state,
                delayed_state, num_q_heads, num_kv_heads, head_dim, t0, t1)
    nd = 0 if decode_slots is None else decode_slots.shape[0]
    npf = 0 if prefill_qsl is None else prefill_qsl.shape[0] - 1
    dp, ds = _index(decode_slots, "decode_slots") if nd else (None, 1)
    pp, ps = _index(prefill_slots, "prefill_slots") if npf else (None, 1)
    desc = sc_cca_desc(num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                       head_dim=head_dim, t0=t0, t1=t1, dtype=_dtype_code(q),
                       q_row_stride=_rows(q, "q"), k_row_stride=_rows(k, "k"),
                       v_cur_row_stride=_rows(v_cur, "v_cur"),
                       v_del_row_stride=_rows(v_del, "v_del"),
                       out_row_stride=_rows(out, "out"), decode_slot_stride=ds,
                       prefill_slot_stride=ps)
    for name, t in (("w_dw", w_dw), ("b_dw", b_dw), ("w_gr", w_gr), ("b_gr", b_gr),
                    ("conv_state", conv_state), ("delayed_state", delayed_state)):
        if not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous tensor")
    # one dtype for every float tensor: the library reads them all as q's
    for name, t in (("k", k), ("v_cur", v_cur), ("v_del", v_del), ("out", out),
                    ("w_dw", w_dw), ("b_dw", b_dw), ("w_gr", w_gr), ("b_gr", b_gr),
                    ("delayed_init", delayed_init), ("conv_state", conv_state),
                    ("delayed_state", delayed_state)):
        if t is not None and t.dtype != q.dtype:
            raise ValueError(f"{name}: dtype {t.dtype} differs from q's {q.dtype}")
    if npf:
        _covers(npf, prefill_slots=prefill_slots,
                prefill_has_initial_state=prefill_has_initial_state)
    st = lib().sc_cca_qk_conv(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v_cur), _ptr(v_del), _ptr(out),
        _ptr(w_dw), _ptr(b_dw), _ptr(w_gr), _ptr(b_gr), _ptr(delayed_init),
        _ptr(conv_state), _ptr(delayed_state), conv_state.shape[0], nd, dp, npf,
        _ptr(prefill_qsl), pp, _flags(prefill_has_initial_state, "prefill_has_initial_state"),
        q.shape[0], _stream(stream, q))
    _check("sc_cca_qk_conv", st)


__all__ = ["lib", "ScError", "LIB_PATH", "EXPORTS", "sc_conv_desc", "sc_ckpt_desc",
           "sc_cca_desc", "sc_conv_fuse", "sc_conv_prefill_varlen", "sc_conv_update",
           "sc_conv_update_spec", "sc_conv_update_spec_varlen", "sc_validate_metadata",
           "sc_state_gather", "sc_state_scatter", "sc_cca_qk_conv"]
