// CCA q/k convolution for gfx950 ("vllm.model_executor.models.zaya", ZayaCCA:
// the conv_qk_depthwise / conv_qk_grouped modules, `project` and
// `_mix_with_state`).
//
// Per token row t of request r (position p in the request) and raw channel c
// of qk = [q | k] (C = (nq+nkv)*hd), ext is the request's raw input extended by
// its saved history of n = t0+t1-2 inputs (zeros without state):
//   dw(c, u)  = bf16( fp32 chain: b1[c], then w1[c,a] * ext(u-(t0-1)+a), a < t0 )
//   yg(o, t)  = b2[o] + sum_{j<hd, b<t1} W2[o, j, b] * dw(grp(o)*hd + j, p-(t1-1)+b)
//   out row   = [yg_q + 0.5(q + k of the head's kv group) | yg_k + mean of the
//                group's q residuals | v_cur | previous token's v_del]
// and afterwards each slot holds the last n raw inputs and the last v_del row.
//
// Two launches: the main kernel only reads the state pools; cca_state_update
// (ordered after it on the stream) writes them, so no workgroup can overwrite a
// history another workgroup still has to read, and main-kernel tiles may mix
// decode and prefill rows freely. On the MFMA path the state update also writes
// the delayed-value columns of each request's first row (from the saved value
// it then replaces), which keeps that rare case out of the main kernel's loop.
//
// The main kernel for hd = 128, t1 = 2 (the ZAYA shape) is cca_persist_main
// below (persistent, weight-stationary, grouped conv on MFMA); other shapes
// take the one-thread-per-output cca_generic_main.
#include <algorithm>

#include "common.hpp"
#include "cca.hpp"

namespace sc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kQslCache = 1024;   // prefill boundaries cached in LDS (else searched in HBM)
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// two fp32 -> one word of two bf16 (lo, hi), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  f32x2 p = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}
__device__ __forceinline__ uint32_t f2bf(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}
// acc + w.lo * x.lo + w.hi * x.hi on bf16 pairs (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_pair(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x),
                                         acc, false);
}
// element e (0..7) of vectors a (low half) and b (high half) as one bf16 pair
__device__ __forceinline__ uint32_t cca_pair(const u32x4& a, const u32x4& b, int e) {
  return __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
}

// Row -> (request position, slot, has-state). Decodes first (one row each,
// always continuing), then prefills by prefill_qsl (rebased to 0).
struct RowInfo {
  int p;        // position in the request, -1 = no row
  int32_t slot;
  bool h;       // reads saved history (valid slot and has-state)
  bool valid;   // slot inside the pool
};

__device__ __forceinline__ int upper_search(const int32_t* qsl, int B, int x) {
  // largest r in [0, B) with qsl[r] <= x
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ RowInfo row_info(const CcaArgs& a, int64_t t, const int32_t* qsl_lds) {
  RowInfo ri{-1, -1, false, false};
  if (t < 0 || t >= a.num_tokens) return ri;
  if (t < a.num_decodes) {
    ri.p = 0;
    ri.slot = a.decode_slots[t * a.dslot_stride];
    ri.valid = ri.slot >= 0 && ri.slot < a.num_slots;
    ri.h = ri.valid;
    return ri;
  }
  if (a.num_prefills <= 0) return ri;
  const int x = (int)(t - a.num_decodes);
  const int r = qsl_lds ? upper_search(qsl_lds, a.num_prefills, x)
                        : upper_search(a.prefill_qsl, a.num_prefills, x);
  const int s0 = a.prefill_qsl[r], s1 = a.prefill_qsl[r + 1];
  if (x < s0 || x >= s1) return ri;
  ri.p = x - s0;
  ri.slot = a.prefill_slots[(int64_t)r * a.pslot_stride];
  ri.valid = ri.slot >= 0 && ri.slot < a.num_slots;
  ri.h = ri.valid && a.prefill_h[r] != 0;
  return ri;
}

// raw qk channel c of token row t
__device__ __forceinline__ uint32_t raw_el(const CcaArgs& a, int64_t t, int c) {
  const int qd = a.nq * a.hd;
  const uint16_t* src = c < qd ? (const uint16_t*)a.q + t * a.q_rs + c
                               : (const uint16_t*)a.k + t * a.k_rs + (c - qd);
  return *src;
}

// Logical workgroup index: workgroups are dealt to the 8 XCDs round-robin;
// this gives each XCD a contiguous run of logical blocks, so the head groups
// of one token chunk (which re-read each other's raw rows for the residuals)
// share an L2.
__device__ __forceinline__ int logical_block_cca(const CcaArgs& a) {
  const int b = (int)blockIdx.x;
  const int lb = (b % 8) * a.per_xcd + b / 8;
  return lb < a.n_logical ? lb : -1;
}

// Raw buffer access (range-checked by the hardware): an offset at or beyond
// `bytes` reads zeros and drops stores, so masked rows cost no branch.
// Offsets are 32-bit; every resource below spans at most one token chunk.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOff = 0x80000000u;   // an offset outside every resource
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)b, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 bld16_stream(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ void bst16_stream(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
}

}  // namespace

// ---------------------------------------------------------------------------
// generic main kernel: one thread per (row, output column), any shape
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void cca_generic_main(CcaArgs a) {
  const int W = (a.nq + 2 * a.nkv) * a.hd;
  const int C = (a.nq + a.nkv) * a.hd;
  const int vd = a.nkv * a.hd / 2, qd = a.nq * a.hd, G = a.nq / a.nkv;
  const int n = a.t0 + a.t1 - 2;
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t t = idx / W;
  const int col = (int)(idx - t * W);
  if (t >= a.num_tokens) return;
  const RowInfo ri = row_info(a, t, nullptr);
  if (ri.p < 0) return;
  const uint16_t* cs = (const uint16_t*)a.conv_state;
  float y;
  if (col < C) {
    const int grp = col / a.hd;
    // ext(c, pos) for pos relative to the request
    auto ext = [&](int c, int pos) -> float {
      if (pos >= 0) return bf2f(raw_el(a, t - ri.p + pos, c));
      if (!ri.h) return 0.f;
      return bf2f(cs[((int64_t)ri.slot * C + c) * n + (n + pos)]);
    };
    float acc = bf2f(((const uint16_t*)a.b_gr)[col]);
    for (int j = 0; j < a.hd; ++j) {
      const int c = grp * a.hd + j;
      for (int b = 0; b < a.t1; ++b) {
        const int pos = ri.p - (a.t1 - 1) + b;
        float d = bf2f(((const uint16_t*)a.b_dw)[c]);
        for (int s = 0; s < a.t0; ++s)
          d = __builtin_fmaf(bf2f(((const uint16_t*)a.w_dw)[(int64_t)c * a.t0 + s]),
                             ext(c, pos - (a.t0 - 1) + s), d);
        d = bf2f(f2bf(d));   // the depthwise output is materialised in bf16
        acc = __builtin_fmaf(bf2f(((const uint16_t*)a.w_gr)[((int64_t)col * a.hd + j) * a.t1 + b]),
                             d, acc);
      }
    }
    float res;
    if (col < qd) {
      const int h = col / a.hd, e = col - h * a.hd;
      res = 0.5f * (bf2f(raw_el(a, t, col)) + bf2f(raw_el(a, t, qd + (h / G) * a.hd + e)));
    } else {
      const int kg = (col - qd) / a.hd, e = col - qd - kg * a.hd;
      const float kv = bf2f(raw_el(a, t, qd + kg * a.hd + e));
      float s = 0.f;
      for (int i = 0; i < G; ++i) s += bf2f(raw_el(a, t, (kg * G + i) * a.hd + e));
      res = 0.5f * (s / (float)G + kv);
    }
    y = acc + res;
    ((uint16_t*)a.out)[t * a.out_rs + col] = (uint16_t)f2bf(y);
    return;
  }
  uint16_t v;
  if (col < C + vd) {
    v = ((const uint16_t*)a.v_cur)[t * a.vc_rs + (col - C)];
  } else {
    const int e = col - C - vd;
    if (ri.p >= 1) v = ((const uint16_t*)a.v_del)[(t - 1) * a.vd_rs + e];
    else if (ri.h) v = ((const uint16_t*)a.delayed_state)[(int64_t)ri.slot * vd + e];
    else v = a.delayed_init ? ((const uint16_t*)a.delayed_init)[e] : (uint16_t)0;
  }
  ((uint16_t*)a.out)[t * a.out_rs + col] = v;
}

// ---------------------------------------------------------------------------
// state update (after the main kernel): new history = last n raw inputs of
// [history, tokens]; delayed state = the request's last v_del row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void cca_state_update(CcaArgs a) {
  const int C = (a.nq + a.nkv) * a.hd;
  const int vd = a.nkv * a.hd / 2;
  const int n = a.t0 + a.t1 - 2;
  const int req = blockIdx.x;
  int64_t start;
  int L;
  int32_t slot;
  bool h;
  if (req < a.num_decodes) {
    start = req;
    L = 1;
    slot = a.decode_slots[(int64_t)req * a.dslot_stride];
    h = true;
  } else {
    const int r = req - a.num_decodes;
    start = a.num_decodes + a.prefill_qsl[r];
    L = a.prefill_qsl[r + 1] - a.prefill_qsl[r];
    slot = a.prefill_slots[(int64_t)r * a.pslot_stride];
    h = a.prefill_h[r] != 0;
  }
  if (slot < 0 || slot >= a.num_slots || L <= 0) return;
  if (start + L > a.num_tokens) return;
  uint16_t* cs = (uint16_t*)a.conv_state + (int64_t)slot * C * n;
  for (int c = threadIdx.x; c < C; c += kBlock) {
    uint16_t nv[8];
    for (int jj = 0; jj < n && jj < 8; ++jj) {
      const int pos = L - n + jj;
      uint16_t v = 0;
      if (pos >= 0) v = (uint16_t)raw_el(a, start + pos, c);
      else if (h) v = cs[(int64_t)c * n + (n + pos)];
      nv[jj] = v;
    }
    for (int jj = 0; jj < n && jj < 8; ++jj) cs[(int64_t)c * n + jj] = nv[jj];
  }
  uint16_t* ds = (uint16_t*)a.delayed_state + (int64_t)slot * vd;
  const uint16_t* last = (const uint16_t*)a.v_del + (start + L - 1) * a.vd_rs;
  for (int e = threadIdx.x; e < vd; e += kBlock) ds[e] = last[e];
}

// ---------------------------------------------------------------------------
// vectorised state update (after cca_persist_main): 8 channels (16 bytes) per
// lane, history length N. It first writes the delayed-value columns of each
// request's first output row, which take the saved delayed value (continuing
// request with a valid slot), else delayed_init, else zeros: the main kernel
// writes the shifted v_del row there for every row and leaves this case here,
// where the old delayed value is read before it is replaced.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(kBlock) void cca_state_update_vec(CcaArgs a) {
  const int C = (a.nq + a.nkv) * a.hd, qd = a.nq * a.hd;
  const int vd = a.nkv * a.hd / 2;
  const int req = blockIdx.x;
  int64_t start;
  int L;
  int32_t slot;
  bool h;
  if (req < a.num_decodes) {
    start = req;
    L = 1;
    slot = a.decode_slots[(int64_t)req * a.dslot_stride];
    h = true;
  } else {
    const int r = req - a.num_decodes;
    start = a.num_decodes + a.prefill_qsl[r];
    L = a.prefill_qsl[r + 1] - a.prefill_qsl[r];
    slot = a.prefill_slots[(int64_t)r * a.pslot_stride];
    h = a.prefill_h[r] != 0;
  }
  if (L <= 0 || start + L > a.num_tokens) return;
  const bool valid = slot >= 0 && slot < a.num_slots;
  const int ncv = C / 8, nvv = vd / 8;
  for (int e8 = threadIdx.x * 8; e8 < vd; e8 += kBlock * 8) {
    u32x4 old = {0, 0, 0, 0};
    if (valid && h) old = ld16((const uint16_t*)a.delayed_state + (int64_t)slot * vd + e8);
    else if (a.delayed_init) old = ld16((const uint16_t*)a.delayed_init + e8);
    st16((uint16_t*)a.out + start * a.out_rs + C + vd + e8, old);
  }
  __syncthreads();   // every old delayed value read before any is replaced
  if (!valid) return;
  for (int v = threadIdx.x; v < ncv + nvv; v += kBlock) {
    if (v >= ncv) {
      const int e8 = (v - ncv) * 8;
      st16((uint16_t*)a.delayed_state + (int64_t)slot * vd + e8,
           ld16((const uint16_t*)a.v_del + (start + L - 1) * a.vd_rs + e8));
      continue;
    }
    const int c0 = v * 8;
    const uint16_t* src = c0 < qd ? (const uint16_t*)a.q + c0 : (const uint16_t*)a.k + (c0 - qd);
    const int64_t srs = c0 < qd ? a.q_rs : a.k_rs;
    uint16_t* sp = (uint16_t*)a.conv_state + ((int64_t)slot * C + c0) * N;
    u32x4 old[N], xr[N], nv[N];
#pragma unroll
    for (int jj = 0; jj < N; ++jj) {
      old[jj] = (h && L < N) ? ld16(sp + jj * 8) : u32x4{0, 0, 0, 0};
      const int pos = L - N + jj;
      xr[jj] = pos >= 0 ? ld16(src + (start + pos) * srs) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int jj = 0; jj < N; ++jj)
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        uint32_t val = BF16::get(xr[jj], ch);
#pragma unroll
        for (int m = 1; m < N; ++m)      // L = m < N: entry jj < N - m keeps old[m + jj]
          if (m + jj < N && m == L) {
            const int el = ch * N + m + jj;
            val = BF16::get(old[el / 8], el % 8);
          }
        const int el = ch * N + jj;
        BF16::set(nv[el / 8], el % 8, val);
      }
#pragma unroll
    for (int jj = 0; jj < N; ++jj) st16(sp + jj * 8, nv[jj]);
  }
}

// ---------------------------------------------------------------------------
// MFMA main kernel (hd = 128, t1 = 2, t0 = T0 <= 4): persistent and
// weight-stationary. The grid holds S workgroups per head group (NG = nq +
// nkv groups), plus helpers for the kv-head groups in the slots left over;
// main workgroup (head group grp, lane k0) walks the 32-row tiles k0, k0 + S,
// k0 + 2S, ..., so every tile is visited by the NG workgroups of one S-slice
// at about the same time, and each workgroup loads the 128 x 256 grouped
// weight of its head group once. Each of the 8 waves
// keeps the slice of 16 output channels it multiplies in registers.
//
// Per tile: (A) the depthwise output of each row at its own position goes to
// LDS row `act`; its value one position earlier is the previous LDS row when
// both rows belong to one request, is computed into a side row `prv` when the
// row starts a request (its window is then all history), and for the tile's
// first row from the rows before the tile. The residual (plus grouped bias) is
// computed alongside in fp32. (B) the grouped conv is the GEMM
// out^T (128 x 32) = W2 (128 x 256) . act^T (256 x 32) with K ordered
// k = b*128 + j (tap b, input channel j) on v_mfma_f32_16x16x32_bf16; the
// epilogue adds the residual and stages bf16 rows, stored as 256-byte row
// segments. The raw rows (and value columns) of the tile two ahead are in
// flight meanwhile (one ahead for the k head, which also reads the bundle's
// q rows). All row traffic uses range-checked buffer instructions: masked
// rows read zeros and drop stores without a branch.
// ---------------------------------------------------------------------------
constexpr int kCcaThreads = 512;   // 8 waves: 16 output channels each
constexpr int kCcaMT = 32;         // token rows per tile
constexpr int kCcaRowTiles = kCcaThreads / kCcaMT;   // tiles whose row info is resolved at once

template <int T0>
struct CcaSmem {
  static constexpr int HD = 128, MT = kCcaMT;
  // bf16 rows of the depthwise tiles, padded by 32 bytes: the MFMA B reads
  // (16 rows x 4 16-byte pieces per instruction) then meet no bank conflict
  static constexpr int AROW = HD + 16;
  static constexpr int RROW = HD + 4;   // fp32 residual rows (padded)
  static constexpr int T0P = (T0 + 1) & ~1;   // taps per channel in LDS: whole pairs
  uint16_t act[(MT + 1) * AROW];        // depthwise rows: row i+1 = token i, row 0 = token -1
  uint16_t prv[MT * AROW];              // depthwise one position back, for request starts
  uint16_t ost[MT * HD];                // staged bf16 output rows, unpadded, pieces swizzled (cca_ost)
  float res[MT * RROW];                 // residual + grouped bias, fp32, half-major (cca_hslot)
  uint16_t w1[HD * T0P];                // depthwise weights: (cca_hslot(c), c % 4, tap), taps padded to even
  float b1[HD];                         // depthwise biases, fp32, (cca_hslot(c), c % 4)
  float b2[HD];                         // grouped biases, fp32, same order
  int32_t qsl_s[kQslCache];
  int row_p[kCcaRowTiles][MT];          // position in the request (-1: no row), per tile of a batch
  int row_hs[kCcaRowTiles][MT];         // saved-history slot of a row at position < T0, else -1
};

// Phase A gives a lane 8 channels v*8 .. v*8+7 of a row and computes them as
// two halves of 4. Its LDS parameters and residual rows are stored by block
// (half, v), so that the 16 lanes of a row touch one contiguous run per half.
__device__ __forceinline__ constexpr int cca_hslot(int c) { return ((c >> 2) & 1) * 16 + (c >> 3); }

// Element offset of (row r, column e) in the output staging rows: 128-element
// rows, the 16-byte piece e / 8 stored at piece (e / 8) ^ (r % 16). The
// epilogue writes 8 bytes per lane down 16 rows and the store reads whole
// rows; with this swizzle neither meets more than a two-way bank conflict.
__device__ __forceinline__ int cca_ost(int r, int e) {
  return r * 128 + ((((e >> 3) ^ r) & 15) << 3) + (e & 7);
}

// Waves per SIMD the main kernel is compiled for: 4 (two resident 8-wave
// workgroups per CU, so one's phase A overlaps the other's MFMA and stores)
// for depthwise widths up to 2 and at most 4 q heads per kv head; wider
// windows and larger groups need more than 128 registers and run one
// workgroup per CU.
__host__ __device__ constexpr int cca_waves_per_simd(int t0, int gmax) {
  return (t0 <= 2 && gmax <= 4) ? 4 : 2;
}

// Row info of token row t: position in its request (-1: no row) and source
// (prefill request index, or -2 - t for decode row t). `cur` is the thread's
// prefill request index from its previous (earlier) row: the search gallops
// forward from it, then bisects.
template <typename QP>
__device__ __forceinline__ void cca_row(const CcaArgs& a, int64_t t, QP qsl, int& cur, int& p,
                                        int& src) {
  p = -1;
  src = -1;
  if (t < a.num_tokens) {
    if (t < a.num_decodes) {
      p = 0;
      src = -2 - (int)t;
    } else if (a.num_prefills > 0) {
      const int B = a.num_prefills;
      const int x = (int)(t - a.num_decodes);
      int r = cur, step = 1;
      while (r + step < B && qsl[r + step] <= x) {
        r += step;
        step <<= 1;
      }
      int lo = r, hi = min(r + step, B) - 1;      // largest index with qsl <= x
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= x) lo = mid;
        else hi = mid - 1;
      }
      cur = lo;
      const int s0 = qsl[lo], s1 = qsl[lo + 1];
      if (x >= s0 && x < s1) {
        p = x - s0;
        src = lo;
      }
    }
  }
}

// Slot and has-state flag of a row's request (global reads: request starts only).
__device__ __forceinline__ void cca_row_state(const CcaArgs& a, int src, int32_t& slot, bool& h) {
  slot = -1;
  h = false;
  if (src <= -2) {
    slot = a.decode_slots[(int64_t)(-2 - src) * a.dslot_stride];
    h = slot >= 0 && slot < a.num_slots;
  } else if (src >= 0) {
    slot = a.prefill_slots[(int64_t)src * a.pslot_stride];
    h = slot >= 0 && slot < a.num_slots && a.prefill_h[src] != 0;
  }
}

template <int T0, int GMAX, bool ISK>
__device__ __forceinline__ void cca_persist_body(const CcaArgs& a, CcaSmem<T0>& sm, int grp, int k0,
                                                 int S, int my_tiles) {
  using SM = CcaSmem<T0>;
  constexpr int HD = 128;
  constexpr int MT = kCcaMT;
  constexpr int N = T0;                // history length n = t0 + t1 - 2 with t1 = 2
  constexpr int AROW = SM::AROW;
  constexpr int RROW = SM::RROW;
  constexpr int NR = T0 + 1;           // raw rows per lane: i-T0 .. i
  constexpr bool isk = ISK;
  // tiles of loads in flight ahead of the one computed: the k head also
  // holds the bundle's q rows per tile, so it keeps one tile in flight
  constexpr int AHEAD = 1;

  const int NG = a.nq + a.nkv, G = a.nq / a.nkv;
  const float inv_g = 1.0f / (float)G;           // exact when G is a power of two
  const int C = NG * HD, vd = a.nkv * HD / 2, nvv = vd / 8;
  const int g = isk ? grp - a.nq : grp / G;       // kv head of the bundle
  const int cbase = grp * HD;                      // raw / output channel base
  const int tid = (int)threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool wave0 = __builtin_amdgcn_readfirstlane(wv) == 0;
  const int v = tid & 15, i = tid >> 4;            // depthwise: channel vector, tile row
  const bool use_lds_qsl = a.num_prefills > 0 && a.num_prefills + 1 <= kQslCache;
  // Value columns (v_cur copied, v_del shifted one token) are dealt over the
  // nq q-head groups only (the k head's workgroups carry the bundle's q rows
  // instead). A row's value columns are 2*nvv/8 lines of 128 bytes (8
  // vectors; nvv = 8 nkv, so the first nkv lines are v_cur's, the rest
  // v_del's); line l goes to q group l % nq, so each line is read and written
  // whole by 8 consecutive lanes of one workgroup (16-byte pieces from
  // different workgroups would each cost a partial-line transfer). A group
  // holds at most two lines; line j of the group is item (row vr, vector vk)
  // of the 256 threads 256 j .. 256 j + 255, so each wave copies one kind of
  // line or none (vkind: 0 none, 1 v_cur, 2 v_del, uniform per wave) and
  // issues only the instructions it needs.
  const int vlines = 2 * nvv / 8;
  const int nl = (isk || grp >= vlines) ? 0 : (vlines - grp + a.nq - 1) / a.nq;
  const int vj = tid / (MT * 8), vr = (tid / 8) % MT, vk = tid & 7;
  const bool vitem = vj < nl;
  const int vvv = (grp + vj * a.nq) * 8 + vk;   // this thread's value vector
  const int vkind = __builtin_amdgcn_readfirstlane(vitem ? (vvv < nvv ? 1 : 2) : 0);
  const int64_t qrs = a.q_rs * 2, krs = a.k_rs * 2, ors = a.out_rs * 2;   // bytes
  const int64_t vcb = a.vc_rs * 2, vdb = a.vd_rs * 2;
  const int64_t srs = isk ? krs : qrs;
  const int scol = ((isk ? g : grp) * HD + v * 8) * 2;    // byte column of the raw input

  // ---- setup: prefill boundaries and parameters (loaded here, stored to LDS
  // once the first tile's loads are out: loads retire in issue order, so a
  // store after each would serialise their round trips), weights to registers ----
  static_assert(kQslCache % kCcaThreads == 0 && HD * SM::T0P <= kCcaThreads, "setup items");
  constexpr int QPT = kQslCache / kCcaThreads;   // boundaries per thread
  int32_t qv[QPT];
#pragma unroll
  for (int m = 0; m < QPT; ++m) {
    const int k = tid + m * kCcaThreads;
    qv[m] = use_lds_qsl && k <= a.num_prefills ? a.prefill_qsl[k] : 0;
  }
  const int w1c = tid / SM::T0P, w1t = tid - w1c * SM::T0P;   // this thread's (channel, tap)
  const uint16_t w1v = tid < HD * SM::T0P && w1t < T0
                           ? ((const uint16_t*)a.w_dw)[(int64_t)(cbase + w1c) * T0 + w1t]
                           : (uint16_t)0;
  // (every thread loads a bias pair, threads from HD on a duplicate: a load
  // under a branch would be waited for where the branch ends)
  const uint16_t b1raw = ((const uint16_t*)a.b_dw)[cbase + (tid & (HD - 1))];
  const uint16_t b2raw = ((const uint16_t*)a.b_gr)[cbase + (tid & (HD - 1))];
  // grouped weights of this wave's 16 output channels, K ordered b*128 + j:
  // one 32-byte run of a (C, hd, t1) row holds taps 0 and 1 of 8 channels
  bf16x8 wf[8];
  {
    const uint16_t* wrow = (const uint16_t*)a.w_gr + (int64_t)(cbase + wv * 16 + (lane & 15)) * (2 * HD);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int j = kk * 32 + 8 * (lane >> 4);
      const u32x4 lo = ld16(wrow + 2 * j), hi = ld16(wrow + 2 * j + 8);
      u32x4 t0v, t1v;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        t0v[w] = __builtin_amdgcn_perm(lo[2 * w + 1], lo[2 * w], 0x05040100u);
        t1v[w] = __builtin_amdgcn_perm(lo[2 * w + 1], lo[2 * w], 0x07060302u);
        t0v[w + 2] = __builtin_amdgcn_perm(hi[2 * w + 1], hi[2 * w], 0x05040100u);
        t1v[w + 2] = __builtin_amdgcn_perm(hi[2 * w + 1], hi[2 * w], 0x07060302u);
      }
      wf[kk] = __builtin_bit_cast(bf16x8, t0v);
      wf[kk + 4] = __builtin_bit_cast(bf16x8, t1v);
    }
  }

  // whole-tensor buffer resources (the launcher keeps every tensor under
  // 2 GiB, so all offsets are 32-bit); a row before the batch wraps to an
  // offset outside the resource and reads zeros
  const uint32_t T = (uint32_t)a.num_tokens;
  const rsrc_t qbuf = make_rsrc(a.q, (int64_t)T * qrs);
  const rsrc_t kbuf = make_rsrc(a.k, (int64_t)T * krs);
  const rsrc_t obuf = make_rsrc(a.out, (int64_t)T * ors);
  const rsrc_t vcbuf = make_rsrc(a.v_cur, (int64_t)T * vcb);
  const rsrc_t vdbuf = make_rsrc(a.v_del, (int64_t)T * vdb);
  const rsrc_t sbuf = isk ? kbuf : qbuf;
  const rsrc_t vbuf = vkind == 1 ? vcbuf : vdbuf;                 // this wave's value tensor
  const uint32_t vrs32 = (uint32_t)(vkind == 1 ? vcb : vdb);
  const uint32_t srs32 = (uint32_t)srs, krs32 = (uint32_t)krs, qrs32 = (uint32_t)qrs;
  const uint32_t ors32 = (uint32_t)ors;
  // per-lane parts of the offsets (row i of the tile; raw slot s is row i-T0+s)
  const uint32_t x_lane = (uint32_t)(i - T0) * srs32 + (uint32_t)scol;
  const uint32_t k_lane = (uint32_t)i * krs32 + (uint32_t)((g * HD + v * 8) * 2);
  const uint32_t q_lane = (uint32_t)i * qrs32 + (uint32_t)((g * G * HD + v * 8) * 2);
  // value item offset: v_cur row t, or v_del row t-1 (row -1 wraps out of
  // the resource and reads zeros)
  const uint32_t v_lane = vkind == 1 ? (uint32_t)vr * (uint32_t)vcb + (uint32_t)(vvv * 16)
                                     : (uint32_t)(vr - 1) * (uint32_t)vdb + (uint32_t)((vvv - nvv) * 16);
  const uint32_t o_lane = (uint32_t)i * ors32 + (uint32_t)((cbase + v * 8) * 2);
  const uint32_t ov_lane = (uint32_t)vr * ors32 + (uint32_t)((C + vvv * 8) * 2);

  auto tile_ta = [&](int u) -> uint32_t { return (uint32_t)(k0 + u * S) * MT; };

  // one tile's loads: raw rows i-T0 .. i of this lane's channel vector (rows
  // of another request are loaded too and never used), the residual rows, and
  // this thread's value item (v_cur row t, or v_del row t-1 for the shift;
  // one load instruction from the wave's value tensor, skipped by waves
  // without items: loads into one register from two instructions would make
  // the compiler wait for every load in flight)
  struct Pref {
    u32x4 x[NR], r[isk ? GMAX : 1], val;
  };
  // (value loads first: the value store at the next tile's start then waits
  // for them alone, not for the rows behind them)
  auto issue = [&](int u, Pref& f) {
    const uint32_t ta = tile_ta(u);
    if constexpr (!isk) {
      if (vkind != 0) f.val = bld16_stream(vbuf, v_lane + ta * vrs32);
    }
    // raw row i - T0 feeds only the side row before the tile's first row, so
    // only wave 0 (rows 0-3) loads it
    if (wave0) f.x[0] = bld16(sbuf, x_lane + ta * srs32);
    else f.x[0] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 1; s < NR; ++s) f.x[s] = bld16(sbuf, x_lane + (ta + s) * srs32);
    if constexpr (!isk) {
      f.r[0] = bld16(kbuf, k_lane + ta * krs32);
    } else {
#pragma unroll
      for (int qi = 0; qi < GMAX; ++qi)
        f.r[qi] = bld16(qbuf, qi < G ? q_lane + ta * qrs32 + (uint32_t)(qi * HD * 2) : kOff);
    }
  };

  int rcur = 0;
  const gptr<int32_t> qsl_g = (gptr<int32_t>)a.prefill_qsl;
  // row info of tiles u0 .. u0 + kCcaRowTiles - 1: one row per thread, so the
  // searches of a whole batch run side by side once per kCcaRowTiles tiles
  // (with the history slot of rows near a request's start: their depthwise
  // windows reach into the saved history, and phase A then needs only the
  // history load itself)
  auto rows_batch = [&](int u0) {
    const int j = tid / MT, ii = tid - j * MT;
    int p = -1, src = -1, hs = -1;
    if (u0 + j < my_tiles) {
      const int64_t t = (int64_t)tile_ta(u0 + j) + ii;
      if (use_lds_qsl) cca_row(a, t, sm.qsl_s, rcur, p, src);
      else cca_row(a, t, qsl_g, rcur, p, src);
      if (p >= 0 && p < T0) {
        int32_t slot;
        bool h;
        cca_row_state(a, src, slot, h);
        hs = h ? slot : -1;
      }
    }
    sm.row_p[j][ii] = p;
    sm.row_hs[j][ii] = hs;
  };
  auto tile = [&](int u, Pref& f) {
    const uint32_t ta = tile_ta(u);
    // (every read of the previous batch's row info precedes the previous
    // tile's second barrier)
    if (u % kCcaRowTiles == 0) {
      rows_batch(u);
      __syncthreads();
    }
    const int* rp = sm.row_p[u % kCcaRowTiles];
    const int* rhs = sm.row_hs[u % kCcaRowTiles];
    // value item of this tile, stored first (only the tile's own loads and the
    // previous tile's stores are in flight here, so its wait is short); at a
    // request's first token the state update kernel rewrites it with the saved
    // delayed value
    if constexpr (!isk) {
      if (vkind != 0) bst16_stream(obuf, rp[vr] >= 0 ? ov_lane + ta * ors32 : kOff, f.val);
    }
    // ---- (A) depthwise rows, the request-start and tile-start side rows, residual ----
    // The lane's 8 channels are done in two halves of 4, one after the other,
    // which halves the fp32 working set of this phase.
    {
      const int p = rp[i];
      uint2 dwh[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int c4 = 4 * hf;                        // first channel of the half
        const int hs = hf * 16 + v;                   // the half's parameter / residual block
        // depthwise weights of the half as words of two taps (word ch * T0P / 2
        // + tap / 2), biases in fp32
        constexpr int WPC = SM::T0P / 2;              // weight words per channel
        uint32_t wd[4 * WPC];
#pragma unroll
        for (int k = 0; k < 4 * WPC; k += 2) {
          const uint2 w2 = *(const uint2*)(sm.w1 + hs * 4 * SM::T0P + 2 * k);
          wd[k] = w2.x;
          wd[k + 1] = w2.y;
        }
        const f32x4 b1v = *(const f32x4*)(sm.b1 + hs * 4);
        const f32x4 b2v = *(const f32x4*)(sm.b2 + hs * 4);
        auto xe = [&](int s, int ch) -> float { return bf2f(BF16::get(f.x[s], c4 + ch)); };
        // Taps are taken in pairs on v_dot2c_f32_bf16 (products summed in fp32,
        // then added to the running sum, which starts at the bias), an odd last
        // tap by fma. xw(t) is the bf16 pair (tap t, tap t + 1) of one channel,
        // xl() the last tap's input.
        auto taps = [&](int ch, float acc, auto xw, auto xl) -> float {
#pragma unroll
          for (int t = 0; t + 1 < T0; t += 2) acc = dot2_pair(wd[ch * WPC + t / 2], xw(t), acc);
          if constexpr ((T0 & 1) != 0)
            acc = __builtin_fmaf(bf2f(wd[ch * WPC + T0 / 2] & 0xFFFFu), xl(), acc);
          return acc;
        };
        // depthwise of this row's request at position pos for the half; tap
        // `tap` reads raw slot base + tap when its ext position is >= 0, else
        // the request's history (zeros without state)
        auto dw = [&](int pos, int base) -> uint2 {
          float d[4];
          if (pos >= T0 - 1) {
#pragma unroll
            for (int ch = 0; ch < 4; ++ch)
              d[ch] = taps(ch, b1v[ch],
                           [&](int t) { return cca_pair(f.x[base + t], f.x[base + t + 1], c4 + ch); },
                           [&]() { return xe(base + T0 - 1, ch); });
          } else {
            // near a request's start: the saved history (global reads, rare)
            const int32_t hslot = rhs[i];
            const bool hn = hslot >= 0;
            const uint16_t* hp = (const uint16_t*)a.conv_state +
                                 ((int64_t)(hn ? hslot : 0) * C + cbase + v * 8) * N;
            u32x4 hist[N];
#pragma unroll
            for (int q = 0; q < N; ++q) hist[q] = hn ? ld16(hp + q * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
              // bf16 bits of each tap's input: the raw row, or history entry
              // N - q for ext position -q (zeros without state)
              uint32_t xv[T0];
#pragma unroll
              for (int tap = 0; tap < T0; ++tap) {
                const int ep = pos - (T0 - 1) + tap;
                uint32_t x = BF16::get(f.x[base + tap], c4 + ch);
                if (ep < 0) {
                  x = 0u;
#pragma unroll
                  for (int q = 1; q <= N; ++q) {
                    const int el = (c4 + ch) * N + N - q;
                    if (ep == -q) x = BF16::get(hist[el / 8], el % 8);
                  }
                }
                xv[tap] = x;
              }
              d[ch] = taps(ch, b1v[ch], [&](int t) { return xv[t] | (xv[t + 1] << 16); },
                           [&]() { return bf2f(xv[T0 - 1]); });
            }
          }
          return uint2{pk_bf16(d[0], d[1]), pk_bf16(d[2], d[3])};
        };
        // residual + grouped bias, fp32
        float y[4];
        if constexpr (!isk) {
          // b2 + 0.5 x + 0.5 k: both halves on one v_dot2c (exact products)
#pragma unroll
          for (int ch = 0; ch < 4; ++ch)
            y[ch] = dot2_pair(0x3F003F00u, cca_pair(f.x[T0], f.r[0], c4 + ch), b2v[ch]);
        } else {
          // the mean over the bundle's q heads, summed in head order (the
          // rows of heads G .. GMAX-1 were read as zeros)
#pragma unroll
          for (int ch = 0; ch < 4; ++ch) {
            float s = 0.f;
#pragma unroll
            for (int qi = 0; qi < GMAX; ++qi) s += bf2f(BF16::get(f.r[qi], c4 + ch));
            y[ch] = b2v[ch] + 0.5f * __builtin_fmaf(s, inv_g, xe(T0, ch));
          }
        }
        uint2 cur_dw = {0u, 0u};
        if (p >= 0) {
          cur_dw = dw(p, 1);
          if (p == 0) *(uint2*)(sm.prv + i * AROW + v * 8 + c4) = dw(-1, 0);
        }
        dwh[hf] = cur_dw;
        *(float4*)(sm.res + i * RROW + hs * 4) = float4{y[0], y[1], y[2], y[3]};
        // the tile's first row continues a request: its previous position
        if (i == 0 && p >= 1) *(uint2*)(sm.act + v * 8 + c4) = dw(p - 1, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      *(u32x4*)(sm.act + (i + 1) * AROW + v * 8) = u32x4{dwh[0].x, dwh[0].y, dwh[1].x, dwh[1].y};
    }
    // store offset of this tile (its row info is rewritten by a later batch)
    const uint32_t ooff = rp[i] >= 0 ? o_lane + ta * ors32 : kOff;
    __syncthreads();
    // the next tile's loads, issued after the barrier: the eight waves'
    // load instructions queue for the CU's vector memory unit one behind
    // another, and each wave then goes on to its MFMAs instead of waiting at
    // the barrier for the last wave's loads to be accepted
    if (u + AHEAD < my_tiles) issue(u + AHEAD, f);

    // ---- (B) grouped conv on MFMA: this wave's 16 channels x 32 tokens ----
    f32x4 acc[2];
    {
      const uint16_t* bp[2][2];
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const int n = th * 16 + (lane & 15);
        bp[th][0] = (rp[n] >= 1 ? sm.act + n * AROW : sm.prv + n * AROW) + 8 * (lane >> 4);
        bp[th][1] = sm.act + (n + 1) * AROW + 8 * (lane >> 4);
        acc[th] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // B fragments in batches of 4 LDS reads (2 K steps), each batch read
      // ahead of its MFMAs
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        u32x4 bv[2][2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int th = 0; th < 2; ++th)
            bv[th][k2] = *(const u32x4*)(bp[th][kb >> 1] + ((kb & 1) * 2 + k2) * 32);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int th = 0; th < 2; ++th)
            acc[th] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[kb * 2 + k2],
                                                              __builtin_bit_cast(bf16x8, bv[th][k2]),
                                                              acc[th], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    }
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      const int n = th * 16 + (lane & 15);
      const int cl = wv * 16 + 4 * (lane >> 4);
      const float4 rr = *(const float4*)(sm.res + n * RROW + cca_hslot(cl) * 4);
      uint2 o;
      o.x = pk_bf16(acc[th][0] + rr.x, acc[th][1] + rr.y);
      o.y = pk_bf16(acc[th][2] + rr.z, acc[th][3] + rr.w);
      *(uint2*)(sm.ost + cca_ost(n, cl)) = o;
    }
    __syncthreads();
    // full 256-byte row segments of the group's output columns
    bst16_stream(obuf, ooff, *(const u32x4*)(sm.ost + cca_ost(i, v * 8)));
  };

  auto store_params = [&]() {
#pragma unroll
    for (int m = 0; m < QPT; ++m) {
      const int k = tid + m * kCcaThreads;
      if (use_lds_qsl && k <= a.num_prefills) sm.qsl_s[k] = qv[m];
    }
    if (tid < HD * SM::T0P) sm.w1[(cca_hslot(w1c) * 4 + (w1c & 3)) * SM::T0P + w1t] = w1v;
    if (tid < HD) {
      sm.b1[cca_hslot(tid) * 4 + (tid & 3)] = bf2f(b1raw);
      sm.b2[cca_hslot(tid) * 4 + (tid & 3)] = bf2f(b2raw);
    }
  };
  if constexpr (AHEAD == 1) {
    Pref fa;
    issue(0, fa);
    store_params();
    __syncthreads();   // qsl and parameters visible
    for (int u = 0; u < my_tiles; ++u) tile(u, fa);
  } else {
    Pref fa, fb;
    issue(0, fa);
    if (my_tiles > 1) issue(1, fb);
    store_params();
    __syncthreads();   // qsl and parameters visible
    for (int u = 0; u < my_tiles; u += 2) {
      tile(u, fa);
      if (u + 1 < my_tiles) tile(u + 1, fb);
    }
  }
}

template <int T0, int GMAX>
__global__ __launch_bounds__(kCcaThreads, cca_waves_per_simd(T0, GMAX)) void cca_persist_main(CcaArgs a) {
  __shared__ __attribute__((aligned(16))) CcaSmem<T0> sm;
  const int lb = logical_block_cca(a);
  if (lb < 0) return;
  const int NG = a.nq + a.nkv;
  const int64_t ntiles = (a.num_tokens + kCcaMT - 1) / kCcaMT;
  int grp, k0, S, my_tiles;
  if (lb < a.n_main) {
    // main workgroup: tiles k0, k0 + S, ... (a kv-head group's stop at
    // kv_main_tiles when it has helpers)
    grp = lb % NG;
    k0 = lb / NG;
    S = a.n_main / NG;
    if (k0 >= ntiles) return;
    my_tiles = (int)((ntiles - 1 - k0) / S + 1);
    if (grp >= a.nq && a.kv_help > 0) my_tiles = min(my_tiles, a.kv_main_tiles);
  } else {
    // helper of a kv-head group: the tiles from kv_main_tiles * S on, dealt
    // over the group's kv_help helpers
    const int h = lb - a.n_main;
    grp = a.nq + h / a.kv_help;
    k0 = a.kv_main_tiles * (a.n_main / NG) + h % a.kv_help;
    S = a.kv_help;
    if (k0 >= ntiles) return;
    my_tiles = (int)((ntiles - 1 - k0) / S + 1);
  }
  if (grp >= a.nq) cca_persist_body<T0, GMAX, true>(a, sm, grp, k0, S, my_tiles);
  else cca_persist_body<T0, GMAX, false>(a, sm, grp, k0, S, my_tiles);
}

// ---------------------------------------------------------------------------
hipError_t launch_cca(const CcaArgs& a, hipStream_t stream) {
  const int64_t W = (int64_t)(a.nq + 2 * a.nkv) * a.hd;
  const int vd = a.nkv * a.hd / 2;
  const uintptr_t al = (uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v_cur | (uintptr_t)a.v_del |
                       (uintptr_t)a.out | (uintptr_t)a.w_dw | (uintptr_t)a.b_dw | (uintptr_t)a.w_gr |
                       (uintptr_t)a.b_gr | (uintptr_t)a.conv_state | (uintptr_t)a.delayed_state |
                       (uintptr_t)(a.delayed_init ? a.delayed_init : a.q);
  const bool strides16 = (a.q_rs * 2) % 16 == 0 && (a.k_rs * 2) % 16 == 0 &&
                         (a.vc_rs * 2) % 16 == 0 && (a.vd_rs * 2) % 16 == 0 &&
                         (a.out_rs * 2) % 16 == 0;
  // the MFMA kernel addresses every token tensor with 32-bit offsets
  const int64_t max_rs = std::max(std::max(a.q_rs, a.k_rs), std::max(std::max(a.vc_rs, a.vd_rs), a.out_rs));
  const bool fits32 = a.num_tokens * max_rs * 2 <= 0x7FFFFFFFLL;
  const bool mfma = a.hd == 128 && a.t1 == 2 && a.t0 >= 1 && a.t0 <= 4 && (al & 15) == 0 &&
                    strides16 && vd % 8 == 0 && a.nq / a.nkv <= 8 && fits32;
  if (mfma) {
    // persistent grid: a multiple of the head-group count, as many workgroups
    // as fit on the device at once, never more than there are tiles to share
    const int NG = a.nq + a.nkv;
    const bool g8 = a.nq / a.nkv > 4;
    const int per_cu = cca_waves_per_simd(a.t0, g8 ? 8 : 4) / 2;   // resident 8-wave workgroups per CU
    const int64_t ntiles = (a.num_tokens + kCcaMT - 1) / kCcaMT;
    int64_t S = (int64_t)device_cus() * per_cu / NG;
    if (S < 1) S = 1;
    if (S > ntiles) S = ntiles;
    CcaArgs b = a;
    b.n_main = (int)(S * NG);
    b.kv_help = 0;
    b.kv_main_tiles = 0;
    // The slots left over (resident slots minus S * NG) go to the kv-head
    // groups, whose tiles cost more (G residual rows per lane): kv_help
    // helpers per kv group take the tail of its tiles, and the group's main
    // workgroups stop after kv_main_tiles, the smallest count the helpers
    // can match. The main walk keeps one stride S for all groups, so the
    // partners of a tile still read it at about the same time.
    {
      const int64_t spare = (int64_t)device_cus() * per_cu - S * NG;
      const int64_t hp = spare / a.nkv;
      if (hp > 0 && S >= 8) {
        const int64_t jk = (ntiles + S + hp - 1) / (S + hp);
        if (jk * S < ntiles) {
          b.kv_help = (int)hp;
          b.kv_main_tiles = (int)jk;
        }
      }
    }
    b.n_logical = b.n_main + b.kv_help * a.nkv;
    b.per_xcd = (b.n_logical + 7) / 8;
    dim3 grid((unsigned)(b.per_xcd * 8));
    const dim3 block(kCcaThreads);
    switch (a.t0 * 2 + (g8 ? 1 : 0)) {
      case 2: hipLaunchKernelGGL((cca_persist_main<1, 4>), grid, block, 0, stream, b); break;
      case 3: hipLaunchKernelGGL((cca_persist_main<1, 8>), grid, block, 0, stream, b); break;
      case 4: hipLaunchKernelGGL((cca_persist_main<2, 4>), grid, block, 0, stream, b); break;
      case 5: hipLaunchKernelGGL((cca_persist_main<2, 8>), grid, block, 0, stream, b); break;
      case 6: hipLaunchKernelGGL((cca_persist_main<3, 4>), grid, block, 0, stream, b); break;
      case 7: hipLaunchKernelGGL((cca_persist_main<3, 8>), grid, block, 0, stream, b); break;
      case 8: hipLaunchKernelGGL((cca_persist_main<4, 4>), grid, block, 0, stream, b); break;
      default: hipLaunchKernelGGL((cca_persist_main<4, 8>), grid, block, 0, stream, b); break;
    }
  } else {
    if (a.t0 + a.t1 - 2 > 8) return hipErrorNotSupported;
    const int64_t total = a.num_tokens * W;
    const int64_t blocks = (total + kBlock - 1) / kBlock;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cca_generic_main, dim3((unsigned)blocks), dim3(kBlock), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int reqs = a.num_decodes + a.num_prefills;
  // (the MFMA path's state update also completes the request-start value
  // columns, so it runs even without a pool)
  if (reqs > 0 && (a.num_slots > 0 || mfma)) {
    const int n = a.t0 + a.t1 - 2;
    if (mfma && n >= 1 && n <= 4) {
      switch (n) {
        case 1: hipLaunchKernelGGL((cca_state_update_vec<1>), dim3((unsigned)reqs), dim3(kBlock), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((cca_state_update_vec<2>), dim3((unsigned)reqs), dim3(kBlock), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((cca_state_update_vec<3>), dim3((unsigned)reqs), dim3(kBlock), 0, stream, a); break;
        default: hipLaunchKernelGGL((cca_state_update_vec<4>), dim3((unsigned)reqs), dim3(kBlock), 0, stream, a); break;
      }
    } else {
      hipLaunchKernelGGL(cca_state_update, dim3((unsigned)reqs), dim3(kBlock), 0, stream, a);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace sc
