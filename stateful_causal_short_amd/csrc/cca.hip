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
// decode and prefill rows freely.
//
// Main kernel for hd = 128, t1 = 2 (the ZAYA shape): a workgroup owns MT token
// rows of one kv bundle (the G q heads of kv head g plus k head g), so both
// residuals stay inside the workgroup. For each of the bundle's G+1 head
// groups it materialises the depthwise outputs in LDS as bf16 (prev, cur)
// pairs, i.e. K ordered k = 2j + b, which makes each grouped-weight fragment a
// contiguous 16-byte slice of the (C, hd, t1) weight; then the grouped conv is
// the GEMM out^T (128 x MT) = W2_g (128 x 256) . act^T (256 x MT) on
// v_mfma_f32_32x32x16_bf16 (each wave 32 output channels), and the epilogue adds
// bias and residual and stores bf16.
#include "common.hpp"
#include "cca.hpp"

namespace sc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kQslCache = 1024;   // prefill boundaries cached in LDS (else searched in HBM)

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// two fp32 -> one word of two bf16 (lo, hi), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  f32x2 p = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}
__device__ __forceinline__ uint32_t f2bf(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
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
// vectorised state update: 8 channels (16 bytes) per lane, history length N
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
  if (slot < 0 || slot >= a.num_slots || L <= 0 || start + L > a.num_tokens) return;
  const int ncv = C / 8, nvv = vd / 8;
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
// MFMA main kernel (hd = 128, t1 = 2, t0 = T0 <= 4): MT rows per workgroup,
// 8 waves per 64 rows (4 channel blocks x MT/32 token tiles)
// ---------------------------------------------------------------------------
template <int MT>
constexpr int cca_threads() { return 256 * (MT / 32); }

template <int T0, int MT>
__global__ __launch_bounds__(cca_threads<MT>(), SC_CCA_MIN_WAVES) void cca_mfma_main(CcaArgs a) {
  constexpr int HD = 128;
  constexpr int NV = HD / 8;           // 16-byte vectors per head row
  constexpr int N = T0;                // history length n = t0 + t1 - 2 with t1 = 2
  constexpr int AROW = 2 * HD + 8;     // LDS row of (prev, cur) pairs, padded (bf16)
  constexpr int OROW = HD + 8;         // LDS row of staged outputs (bf16)
  constexpr int RROW = NV + 1;         // LDS raw row in 16-byte vectors, padded
  constexpr int NTH = cca_threads<MT>();
  constexpr int RPT = MT * NV / NTH;   // depthwise rows per lane (= 2)
  constexpr int NR = RPT + T0;         // raw rows per lane: its rows plus the halo
  constexpr int KS = 2 * HD / 16;      // MFMA K steps
  static_assert(MT % 32 == 0 && MT <= 128 && RPT * NTH == MT * NV, "tile rows");
  static_assert(MT * OROW <= MT * AROW, "output staging fits in the pair buffer");

  __shared__ __attribute__((aligned(16))) uint16_t act[MT * AROW];
  __shared__ u32x4 rawc[MT * RROW];    // current rows of the q head being processed
  __shared__ u32x4 rawk[MT * RROW];    // current rows of the bundle's k head
  __shared__ int32_t qsl_s[kQslCache];
  __shared__ int row_p[MT];
  __shared__ int32_t row_slot[MT];
  __shared__ uint8_t row_h[MT];

  const int nkv = a.nkv, G = a.nq / a.nkv;
  const int C = (a.nq + a.nkv) * HD;
  const int qd = a.nq * HD, vd = a.nkv * HD / 2;
  const int tile = (int)blockIdx.x / nkv, g = (int)blockIdx.x - tile * nkv;
  const int64_t t0 = (int64_t)tile * MT;
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cw = wave & 3, nt = wave >> 2;          // GEMM: channel block, token tile
  const int v = tid % NV, i0 = (tid / NV) * RPT;    // depthwise: channel vector, first row
  const bool use_lds_qsl = a.num_prefills > 0 && a.num_prefills + 1 <= kQslCache;

  if (use_lds_qsl)
    for (int i = tid; i <= a.num_prefills; i += NTH) qsl_s[i] = a.prefill_qsl[i];
  __syncthreads();
  if (tid < MT) {
    const RowInfo ri = row_info(a, t0 + tid, use_lds_qsl ? qsl_s : nullptr);
    row_p[tid] = ri.p;
    row_slot[tid] = ri.slot;
    row_h[tid] = ri.h ? 1 : 0;
  }
  __syncthreads();

  int rp[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) rp[r] = row_p[i0 + r];

  // depthwise inputs of one head group: raw rows i0-T0 .. i0+RPT-1 (halo rows
  // only when the first row's request reaches back to them), weights, bias
  u32x4 xr[NR], wv[T0], bv;
  auto issue_dw = [&](int gi) {
    const bool isk = gi == G;
    const int cbase = isk ? (a.nq + g) * HD : (g * G + gi) * HD;
    const uint16_t* src = isk ? (const uint16_t*)a.k + g * HD
                              : (const uint16_t*)a.q + (int64_t)(g * G + gi) * HD;
    const int64_t srs = isk ? a.k_rs : a.q_rs;
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const int i = i0 - T0 + s;
      const bool need = s >= T0 ? rp[s - T0] >= 0 : rp[0] >= T0 - s;
      xr[s] = need ? ld16(src + (t0 + i) * srs + v * 8) : u32x4{0, 0, 0, 0};
    }
    const uint16_t* wp = (const uint16_t*)a.w_dw + (int64_t)(cbase + v * 8) * T0;
#pragma unroll
    for (int s = 0; s < T0; ++s) wv[s] = ld16(wp + s * 8);
    bv = ld16((const uint16_t*)a.b_dw + cbase + v * 8);
  };
  issue_dw(0);

  // the bundle's k head rows (residual of every group)
  for (int it = tid; it < MT * NV; it += NTH) {
    const int i = it / NV, vv = it - i * NV;
    u32x4 val = {0, 0, 0, 0};
    if (row_p[i] >= 0) val = ld16((const uint16_t*)a.k + (t0 + i) * a.k_rs + g * HD + vv * 8);
    rawk[i * RROW + vv] = val;
  }

  f32x16 qsum;
#pragma unroll
  for (int r = 0; r < 16; ++r) qsum[r] = 0.f;

  for (int gi = 0; gi <= G; ++gi) {
    const bool isk = gi == G;
    const int cbase = isk ? (a.nq + g) * HD : (g * G + gi) * HD;
#if !SC_CCA_XPREF
    if (gi > 0) issue_dw(gi);
#endif
    const uint16_t* wrow = (const uint16_t*)a.w_gr +
                           ((int64_t)(cbase + cw * 32 + (lane & 31)) * (2 * HD)) + 8 * (lane >> 5);
    // history of rows that reach back before their request's first token
    u32x4 hist[RPT][N];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const bool need = rp[r] >= 0 && rp[r] < T0 && row_h[i0 + r];
      const uint16_t* hp = (const uint16_t*)a.conv_state +
                           ((int64_t)(need ? row_slot[i0 + r] : 0) * C + cbase + v * 8) * N;
#pragma unroll
      for (int vv = 0; vv < N; ++vv) hist[r][vv] = need ? ld16(hp + vv * 8) : u32x4{0, 0, 0, 0};
    }

    __syncthreads();   // previous group's output staging has been stored
    // ---- depthwise: (prev, cur) bf16 pairs for 8 channels of RPT rows ----
    {
      float wf32[T0][8], bs[8];
#pragma unroll
      for (int s = 0; s < T0; ++s) {
        float f[8];
        BF16::unpack(wv[s], f);
        // wv[s] holds w_dw[(c0+ch)*T0 + tap] in element order ch*T0 + tap
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int flat = s * 8 + e, ch = flat / T0, tap = flat % T0;
          wf32[tap][ch] = f[e];
        }
      }
      BF16::unpack(bv, bs);
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int p = rp[r];
        uint32_t pairs[8];
        float e[T0 + 1][8];
#pragma unroll
        for (int s = 0; s <= T0; ++s) BF16::unpack(xr[r + s], e[s]);
        if (p < T0) {
          // the window reaches back before the request: history (or zeros)
#pragma unroll
          for (int s = 0; s < T0; ++s) {
            const int pos = p - T0 + s;          // ext position of tap s
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) {
              float hv = 0.f;
#pragma unroll
              for (int q = 1; q <= N; ++q) {
                const int el = ch * N + N - q;
                if (pos == -q) hv = bf2f(BF16::get(hist[r][el / 8], el % 8));
              }
              if (pos < 0) e[s][ch] = hv;
            }
          }
        }
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          float dp = bs[ch], dc = bs[ch];
#pragma unroll
          for (int s = 0; s < T0; ++s) {
            dp = __builtin_fmaf(wf32[s][ch], e[s][ch], dp);
            dc = __builtin_fmaf(wf32[s][ch], e[s + 1][ch], dc);
          }
          pairs[ch] = p >= 0 ? pk_bf16(dp, dc) : 0u;
        }
        u32x4* ap = (u32x4*)(act + (i0 + r) * AROW + v * 16);
        ap[0] = u32x4{pairs[0], pairs[1], pairs[2], pairs[3]};
        ap[1] = u32x4{pairs[4], pairs[5], pairs[6], pairs[7]};
        if (!isk) rawc[(i0 + r) * RROW + v] = p >= 0 ? xr[r + T0] : u32x4{0, 0, 0, 0};
      }
    }
#if SC_CCA_XPREF
    if (gi < G) issue_dw(gi + 1);      // next group's inputs in flight during the GEMM
#endif
    __syncthreads();

    // ---- grouped conv on MFMA: out^T tile = W2 (32 ch x 256) . act^T (256 x 32 tok) ----
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll SC_CCA_KUNROLL
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, ld16(wrow + ks * 16));
      const u32x4 bvv = *(const u32x4*)(act + (nt * 32 + (lane & 31)) * AROW + ks * 16 + 8 * (lane >> 5));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8, bvv), acc, 0, 0, 0);
    }

    // ---- epilogue: bias + residual, bf16 staged in LDS (act is reused) ----
    __syncthreads();   // every wave is done reading act (GEMM) before it is reused
    uint16_t* ost = act;
    {
      const int i = nt * 32 + (lane & 31);
#pragma unroll
      for (int run = 0; run < 4; ++run) {
        const int cl = cw * 32 + 8 * run + 4 * (lane >> 5);     // channel within the head
        const uint2 bb = *(const uint2*)((const uint16_t*)a.b_gr + cbase + cl);
        const float b2[4] = {bf2f(bb.x & 0xFFFFu), bf2f(bb.x >> 16), bf2f(bb.y & 0xFFFFu), bf2f(bb.y >> 16)};
        const int vsel = cl >> 3, half = (cl >> 2) & 1;
        const u32x4 kv4 = rawk[i * RROW + vsel];
        const uint32_t k01 = kv4[2 * half], k23 = kv4[2 * half + 1];
        const float kf[4] = {bf2f(k01 & 0xFFFFu), bf2f(k01 >> 16), bf2f(k23 & 0xFFFFu), bf2f(k23 >> 16)};
        float y[4];
        if (!isk) {
          const u32x4 qv4 = rawc[i * RROW + vsel];
          const uint32_t q01 = qv4[2 * half], q23 = qv4[2 * half + 1];
          const float qf[4] = {bf2f(q01 & 0xFFFFu), bf2f(q01 >> 16), bf2f(q23 & 0xFFFFu), bf2f(q23 >> 16)};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            qsum[4 * run + s] += qf[s];
            y[s] = acc[4 * run + s] + b2[s] + 0.5f * (qf[s] + kf[s]);
          }
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            y[s] = acc[4 * run + s] + b2[s] + 0.5f * (qsum[4 * run + s] / (float)G + kf[s]);
        }
        uint2 o;
        o.x = pk_bf16(y[0], y[1]);
        o.y = pk_bf16(y[2], y[3]);
        *(uint2*)(ost + i * OROW + cl) = o;
      }
    }
    __syncthreads();
    // full 256-byte row segments of the group's output columns
    const int ocol = isk ? qd + g * HD : (g * G + gi) * HD;
    for (int it = tid; it < MT * NV; it += NTH) {
      const int ii = it / NV, vv = it - ii * NV;
      if (row_p[ii] >= 0)
        st16_stream((uint16_t*)a.out + (t0 + ii) * a.out_rs + ocol + vv * 8,
                    *(const u32x4*)(ost + ii * OROW + vv * 8));
    }
  }

  // ---- value part: v_cur copied, v_del shifted by one token (this bundle's
  // share of the 16-byte vectors) ----
  const int nvv = vd / 8;   // vectors per value half
  for (int it = tid; it < MT * 2 * nvv; it += NTH) {
    const int i = it / (2 * nvv), vv = it - i * (2 * nvv);
    if (vv % nkv != g) continue;
    const int p = row_p[i];
    if (p < 0) continue;
    const int64_t t = t0 + i;
    u32x4 val;
    if (vv < nvv) {
      val = ld16((const uint16_t*)a.v_cur + t * a.vc_rs + vv * 8);
    } else {
      const int e8 = (vv - nvv) * 8;
      if (p >= 1) val = ld16((const uint16_t*)a.v_del + (t - 1) * a.vd_rs + e8);
      else if (row_h[i]) val = ld16((const uint16_t*)a.delayed_state + (int64_t)row_slot[i] * vd + e8);
      else if (a.delayed_init) val = ld16((const uint16_t*)a.delayed_init + e8);
      else val = u32x4{0, 0, 0, 0};
    }
    st16_stream((uint16_t*)a.out + t * a.out_rs + C + vv * 8, val);
  }
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
  const bool mfma = a.hd == 128 && a.t1 == 2 && a.t0 >= 1 && a.t0 <= 4 && (al & 15) == 0 &&
                    strides16 && vd % 8 == 0 && !SC_CCA_GENERIC;
  if (mfma) {
    constexpr int MT = SC_CCA_TILE;
    const int64_t tiles = (a.num_tokens + MT - 1) / MT;
    const int64_t blocks = tiles * a.nkv;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks);
    const dim3 block(cca_threads<MT>());
    switch (a.t0) {
      case 1: hipLaunchKernelGGL((cca_mfma_main<1, MT>), grid, block, 0, stream, a); break;
      case 2: hipLaunchKernelGGL((cca_mfma_main<2, MT>), grid, block, 0, stream, a); break;
      case 3: hipLaunchKernelGGL((cca_mfma_main<3, MT>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((cca_mfma_main<4, MT>), grid, block, 0, stream, a); break;
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
  if (reqs > 0 && a.num_slots > 0) {
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
