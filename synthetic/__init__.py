"""Seeded synthetic inputs for the stateful causal short convolution.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no convolution, no state carry, no rounding of results).
Both the CPU oracle (through the tests) and the GPU path (through the tests,
the smoke check and the benchmark) take their inputs from here, so the two
sides see identical bytes.

Every array is a NumPy array. bf16 tensors are carried as ``uint16`` bit
patterns (NumPy has no bfloat16); fp32 tensors as ``float32``.

Workloads follow the shapes of the pages' layers:

* depthwise conv cases (GDN mixed-qkv conv, dilated PLE short conv): token
  rows ``(T, C)`` with decode rows first and prefill rows after them, a
  ``(num_slots, C, S)`` state pool, per-request slots and has-initial-state
  flags, optional prefill checkpoints every ``grid`` tokens;
* CCA cases (ZAYA compressed convolutional attention): raw q/k projections,
  current and delayed v projections, depthwise + grouped conv weights, and the
  two-part state (raw q/k history, previous delayed value).

"N(0, s)" below means a normal with standard deviation ``s``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_BASE = 0x5C0DE000

__all__ = [
    "SEED_BASE", "ConvCase", "CcaCase", "bf16_bits", "bf16_to_f32",
    "conv_case", "cca_case", "single_seq_64ch", "varlen_prefill_8seq", "decode_512req", "update_128req_q4",
    "ple_mixed_batch", "cca_mixed_32k", "storage_dtype",
]


# --------------------------------------------------------------------------
# encoding helpers (input generation only)
# --------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode real values as bf16 bit patterns (via fp32, nearest-even).

    Used only to produce bf16 *inputs*: any bf16 value is a valid input, so the
    two-step rounding here is immaterial.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns to float32 (exact)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def storage_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16}[dtype]


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    v = rng.standard_normal(size=shape) * std
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "bf16":
        return bf16_bits(v)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# depthwise cases
# --------------------------------------------------------------------------
@dataclass
class ConvCase:
    """One batch for the depthwise conv path.

    Token rows: ``num_decodes * q`` decode rows first (request ``i`` owns rows
    ``[i*q, (i+1)*q)``), then the prefill rows, whose offsets ``qsl_p`` are
    relative to the first prefill row.
    """
    name: str
    C: int
    K: int
    d: int
    S: int
    dtype: str                     # "f32" | "bf16": x, out, weight, bias, pool
    act: str                       # "none" | "silu"
    x: np.ndarray                  # (T, C)
    w: np.ndarray                  # (C, K)
    bias: Optional[np.ndarray]     # (C,) or None
    pool: np.ndarray               # (num_slots, C, S), or (num_slots, S, C) when layout == "sd"
    num_decodes: int = 0
    q: int = 1                     # tokens per decode request
    decode_slots: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    decode_h: Optional[np.ndarray] = None   # None = every decode continues its state
    qsl_p: np.ndarray = field(default_factory=lambda: np.zeros(1, np.int32))
    prefill_slots: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    prefill_h: np.ndarray = field(default_factory=lambda: np.zeros(0, np.uint8))
    ckpt_grid: int = 0
    cu_ckpt: Optional[np.ndarray] = None    # (B_p + 1,) exclusive prefix
    ckpt_slots: Optional[np.ndarray] = None
    layout: str = "ds"                      # state pool layout: "ds" (slot, C, S) | "sd" (slot, S, C)

    @property
    def H(self) -> int:
        return (self.K - 1) * self.d

    @property
    def num_prefills(self) -> int:
        return int(self.qsl_p.shape[0]) - 1

    @property
    def num_decode_tokens(self) -> int:
        return self.num_decodes * self.q

    @property
    def num_prefill_tokens(self) -> int:
        return int(self.qsl_p[-1])

    @property
    def T(self) -> int:
        return self.num_decode_tokens + self.num_prefill_tokens

    @property
    def num_slots(self) -> int:
        return int(self.pool.shape[0])

    @property
    def elsize(self) -> int:
        return 4 if self.dtype == "f32" else 2


def conv_case(name: str, seed: int, *, C: int, K: int, d: int, dtype: str,
              act: str, w_std: float, bias_std: Optional[float],
              num_slots: int, num_decodes: int = 0, q: int = 1,
              prefill_lens=(), prefill_h_p: float = 0.5,
              prefill_h_all: Optional[int] = None, ckpt_grid: int = 0,
              x_std: float = 1.0, state_std: float = 1.0,
              decode_h: Optional[np.ndarray] = None, num_spec: int = 0) -> ConvCase:
    """Build a depthwise case; slots are a random permutation of the pool.

    Slot assignment from one permutation: decodes first, then prefills, then
    checkpoint destinations, so every slot in one call is distinct and the
    untouched slots act as canaries. ``num_spec`` > 0 widens each state row to
    S = H + num_spec (a buffer sized for speculative rollback).
    """
    rng = np.random.default_rng(seed)
    H = (K - 1) * d
    prefill_lens = np.asarray(prefill_lens, dtype=np.int64)
    Bp = int(prefill_lens.shape[0])
    qsl_p = np.zeros(Bp + 1, np.int32)
    qsl_p[1:] = np.cumsum(prefill_lens)
    T = num_decodes * q + int(qsl_p[-1])
    x = _normal(rng, (T, C), x_std, dtype)
    w = _normal(rng, (C, K), w_std, dtype)
    bias = None if bias_std is None else _normal(rng, (C,), bias_std, dtype)
    S = H + num_spec
    pool = _normal(rng, (num_slots, C, S), state_std, dtype)
    if prefill_h_all is not None:
        prefill_h = np.full(Bp, prefill_h_all, np.uint8)
    else:
        prefill_h = (rng.random(Bp) < prefill_h_p).astype(np.uint8)
    if ckpt_grid:
        nck = prefill_lens // ckpt_grid
        cu_ckpt = np.zeros(Bp + 1, np.int32)
        cu_ckpt[1:] = np.cumsum(nck)
        n_ck = int(cu_ckpt[-1])
    else:
        cu_ckpt, n_ck = None, 0
    need = num_decodes + Bp + n_ck
    if need > num_slots:
        raise ValueError(f"{name}: {need} slots needed, pool has {num_slots}")
    perm = rng.permutation(num_slots).astype(np.int32)
    decode_slots = perm[:num_decodes].copy()
    prefill_slots = perm[num_decodes:num_decodes + Bp].copy()
    ckpt_slots = perm[num_decodes + Bp:need].copy() if ckpt_grid else None
    return ConvCase(name=name, C=C, K=K, d=d, S=S, dtype=dtype, act=act, x=x,
                    w=w, bias=bias, pool=pool, num_decodes=num_decodes, q=q,
                    decode_slots=decode_slots, decode_h=decode_h, qsl_p=qsl_p,
                    prefill_slots=prefill_slots, prefill_h=prefill_h,
                    ckpt_grid=ckpt_grid, cu_ckpt=cu_ckpt, ckpt_slots=ckpt_slots)


def single_seq_64ch(seed: int = SEED_BASE + 1) -> ConvCase:
    """Single sequence, 64 channels, width 4, fp32, no activation, zero state."""
    return conv_case("single_seq_64ch_f32", seed, C=64, K=4, d=1, dtype="f32",
                     act="none", w_std=0.25, bias_std=0.1, num_slots=1,
                     prefill_lens=[256], prefill_h_all=0)


def varlen_prefill_8seq(seed: int = SEED_BASE + 2, *, C: int = 8192, B: int = 8,
            max_len: int = 2048, num_slots: int = 64) -> ConvCase:
    """Varlen prefill: B sequences, lengths U{1..max_len}, bf16, bias, SiLU."""
    rng = np.random.default_rng(seed ^ 0xA5A5)
    lens = rng.integers(1, max_len + 1, size=B)
    return conv_case("varlen_prefill_8seq_8192ch", seed, C=C, K=4, d=1, dtype="bf16",
                     act="silu", w_std=0.25, bias_std=0.1, num_slots=num_slots,
                     prefill_lens=lens, prefill_h_p=0.5)


def decode_512req(seed: int = SEED_BASE + 3, *, C: int = 8192, B: int = 512,
             num_slots: int = 1024) -> ConvCase:
    """Decode: B requests x 1 token, state continued, bf16, bias, SiLU."""
    return conv_case("decode_512req_8192ch", seed, C=C, K=4, d=1, dtype="bf16",
                     act="silu", w_std=0.25, bias_std=0.1, num_slots=num_slots,
                     num_decodes=B, q=1)


def update_128req_q4(seed: int = SEED_BASE + 0x33, *, C: int = 8192, B: int = 128,
             q: int = 4, num_slots: int = 1024) -> ConvCase:
    """Multi-token update: B requests x q tokens, all consumed."""
    return conv_case("update_128req_q4_8192ch", seed, C=C, K=4, d=1, dtype="bf16",
                     act="silu", w_std=0.25, bias_std=0.1, num_slots=num_slots,
                     num_decodes=B, q=q)


def spec_128req_q4(seed: int = SEED_BASE + 0x35, *, C: int = 8192, B: int = 128,
                  num_spec: int = 3, num_slots: int = 1024) -> ConvCase:
    """Speculative update: B requests x (num_spec + 1) tokens on a rolling
    buffer of (K-1) + num_spec entries (accepted counts from num_accepted)."""
    return conv_case("spec_128req_q4_8192ch", seed, C=C, K=4, d=1, dtype="bf16",
                     act="silu", w_std=0.25, bias_std=0.1, num_slots=num_slots,
                     num_decodes=B, q=num_spec + 1, num_spec=num_spec)


def spec_varlen_case(name: str, seed: int, *, C: int, K: int, d: int, dtype: str, act: str,
                     w_std: float, bias_std: Optional[float], num_slots: int, B: int,
                     num_spec: int, q_lens=None, q_max: Optional[int] = None):
    """Speculative requests with a draft count each (rolling buffer of
    S = H + num_spec entries). Draft counts are `q_lens`, else uniform in
    {0 .. q_max} (default num_spec + 1). Returns (case, qsl): request r owns
    rows [qsl[r], qsl[r+1]) of case.x and slot case.decode_slots[r]
    (case.num_decodes = B; case.q is not used)."""
    rng = np.random.default_rng(seed ^ 0x5EC)
    if q_lens is None:
        hi = num_spec + 1 if q_max is None else q_max
        q_lens = rng.integers(0, hi + 1, size=B)
    q_lens = np.asarray(q_lens, np.int64)
    assert q_lens.shape[0] == B
    qsl = np.zeros(B + 1, np.int32)
    qsl[1:] = np.cumsum(q_lens)
    T = int(qsl[-1])
    # T rows as "prefill" lengths give x its shape; the requests are then
    # re-labelled as speculative ones (all continuing their buffer)
    base = conv_case(name, seed, C=C, K=K, d=d, dtype=dtype, act=act, w_std=w_std,
                     bias_std=bias_std, num_slots=num_slots, num_decodes=B, q=1,
                     num_spec=num_spec)
    x = _normal(rng, (T, C), 1.0, dtype)
    from dataclasses import replace
    return replace(base, x=x), qsl


def spec_varlen_128req(seed: int = SEED_BASE + 0x37, *, C: int = 8192, B: int = 128,
                         num_spec: int = 3, num_slots: int = 1024):
    """Speculative update with per-request draft counts uniform in
    {0 .. num_spec + 1} (the GDN page's per-sequence loop), otherwise as
    spec_128req_q4. Returns (case, qsl)."""
    return spec_varlen_case("spec_varlen_128req_8192ch", seed, C=C, K=4, d=1, dtype="bf16", act="silu",
                            w_std=0.25, bias_std=0.1, num_slots=num_slots, B=B,
                            num_spec=num_spec)


def ple_mixed_batch(seed: int = SEED_BASE + 4, *, C: int = 8192, num_decodes: int = 256,
            Bp: int = 16, min_len: int = 128, max_len: int = 4096,
            grid: int = 512, num_slots: int = 1024) -> ConvCase:
    """Dilated PLE-style mixed batch: decodes then varlen prefills with
    checkpoints every ``grid`` tokens; width 4, dilation 3, no bias/act."""
    rng = np.random.default_rng(seed ^ 0xA5A5)
    lens = rng.integers(min_len, max_len + 1, size=Bp)
    return conv_case("ple_mixed_8192ch_d3", seed, C=C, K=4, d=3,
                     dtype="bf16", act="none", w_std=0.05, bias_std=None,
                     num_slots=num_slots, num_decodes=num_decodes, q=1,
                     prefill_lens=lens, prefill_h_p=0.5, ckpt_grid=grid)


# --------------------------------------------------------------------------
# CCA cases
# --------------------------------------------------------------------------
@dataclass
class CcaCase:
    name: str
    nq: int
    nkv: int
    hd: int
    t0: int
    t1: int
    q: np.ndarray          # (T, nq*hd)      bf16 bits
    k: np.ndarray          # (T, nkv*hd)
    v_cur: np.ndarray      # (T, nkv*hd//2)
    v_del: np.ndarray      # (T, nkv*hd//2)
    w_dw: np.ndarray       # (C, t0)
    b_dw: np.ndarray       # (C,)
    w_gr: np.ndarray       # (C, hd, t1)
    b_gr: np.ndarray       # (C,)
    delayed_init: np.ndarray   # (nkv*hd//2,)
    conv_state: np.ndarray     # (slots, C, n)
    delayed_state: np.ndarray  # (slots, nkv*hd//2)
    num_decodes: int
    decode_slots: np.ndarray
    qsl_p: np.ndarray
    prefill_slots: np.ndarray
    prefill_h: np.ndarray
    dtype: str = "bf16"

    @property
    def C(self) -> int:
        return (self.nq + self.nkv) * self.hd

    @property
    def n(self) -> int:
        return self.t0 + self.t1 - 2

    @property
    def T(self) -> int:
        return self.num_decodes + int(self.qsl_p[-1])

    @property
    def num_prefills(self) -> int:
        return int(self.qsl_p.shape[0]) - 1

    @property
    def num_slots(self) -> int:
        return int(self.conv_state.shape[0])

    @property
    def out_width(self) -> int:
        return (self.nq + 2 * self.nkv) * self.hd


def cca_case(name: str, seed: int, *, nq: int = 16, nkv: int = 4, hd: int = 128,
             t0: int = 2, t1: int = 2, num_decodes: int = 512,
             prefill_lens=None, num_prefills: int = 64,
             num_prefill_tokens: int = 32256, num_slots: int = 1024,
             w_std: float = 0.02, prefill_h_p: float = 0.5,
             dtype: str = "bf16") -> CcaCase:
    """CCA batch: ``num_decodes`` one-token requests, then prefills whose
    lengths are a random composition of ``num_prefill_tokens`` (distinct
    sorted cut points), unless ``prefill_lens`` is given."""
    rng = np.random.default_rng(seed)
    if prefill_lens is None:
        if num_prefills:
            cuts = np.sort(rng.choice(np.arange(1, num_prefill_tokens),
                                      num_prefills - 1, replace=False))
            edges = np.concatenate([[0], cuts, [num_prefill_tokens]])
            prefill_lens = np.diff(edges)
        else:
            prefill_lens = np.zeros(0, np.int64)
    prefill_lens = np.asarray(prefill_lens, np.int64)
    Bp = int(prefill_lens.shape[0])
    qsl_p = np.zeros(Bp + 1, np.int32)
    qsl_p[1:] = np.cumsum(prefill_lens)
    T = num_decodes + int(qsl_p[-1])
    C = (nq + nkv) * hd
    vd = nkv * hd // 2
    n = t0 + t1 - 2
    case = CcaCase(
        name=name, nq=nq, nkv=nkv, hd=hd, t0=t0, t1=t1,
        q=_normal(rng, (T, nq * hd), 1.0, dtype),
        k=_normal(rng, (T, nkv * hd), 1.0, dtype),
        v_cur=_normal(rng, (T, vd), 1.0, dtype),
        v_del=_normal(rng, (T, vd), 1.0, dtype),
        w_dw=_normal(rng, (C, t0), w_std, dtype),
        b_dw=_normal(rng, (C,), w_std, dtype),
        w_gr=_normal(rng, (C, hd, t1), w_std, dtype),
        b_gr=_normal(rng, (C,), w_std, dtype),
        delayed_init=_normal(rng, (vd,), w_std, dtype),
        conv_state=_normal(rng, (num_slots, C, n), 1.0, dtype),
        delayed_state=_normal(rng, (num_slots, vd), 1.0, dtype),
        num_decodes=num_decodes, decode_slots=np.zeros(0, np.int32),
        qsl_p=qsl_p, prefill_slots=np.zeros(0, np.int32),
        prefill_h=(rng.random(Bp) < prefill_h_p).astype(np.uint8), dtype=dtype)
    if num_decodes + Bp > num_slots:
        raise ValueError(f"{name}: pool too small")
    perm = rng.permutation(num_slots).astype(np.int32)
    case.decode_slots = perm[:num_decodes].copy()
    case.prefill_slots = perm[num_decodes:num_decodes + Bp].copy()
    return case


def cca_mixed_32k(seed: int = SEED_BASE + 5, **kw) -> CcaCase:
    """CCA q/k conv: 16 q heads, 4 kv heads, head_dim 128, kernels 2 and 2,
    512 decodes + 64 prefills, 32768 tokens in all."""
    return cca_case("cca_mixed_32k_tokens", seed, **kw)


def num_accepted(seed: int, batch: int, q: int, lo: int = 1, hi: Optional[int] = None) -> np.ndarray:
    """Accepted-token counts of the previous speculative step, uniform in
    [lo, hi] (hi defaults to q). Values outside the meaningful range can be
    asked for on purpose (lo=0, hi > q) to exercise clamping."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, (q if hi is None else hi) + 1, size=batch).astype(np.int32)


def as_sd(case: ConvCase) -> ConvCase:
    """The same case with its state pool stored (num_slots, S, C)."""
    from dataclasses import replace
    assert case.layout == "ds"
    return replace(case, pool=np.ascontiguousarray(case.pool.transpose(0, 2, 1)), layout="sd")
