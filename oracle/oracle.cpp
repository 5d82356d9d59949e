// Oracle for the stateful causal short convolution.
//
// TEST INFRASTRUCTURE ONLY. This file is a plain, slow CPU implementation of
// what the GPU path computes, written from the defining pages. Only the test
// suite, the smoke check and the benchmark's CPU-baseline leg load it; the
// product library never links, loads or calls it, and it shares no code,
// header, table or helper with the GPU sources.
//
// Sources (cited by page title and section):
//  * "vllm.model_executor.models.zaya", class ZayaCCA: the layer's two Conv1d
//    modules (depthwise, then grouped), `project` (residual mix, value layout)
//    and `_mix_with_state` (request resolution, history gather with the
//    has-state mask, delayed value shift, history write-back).
//  * "vllm.model_executor.layers.mamba.ops.cpu.gdn_attention": decode and
//    varlen prefill conv calls (`_spec_aware_nonspec`), bias + SiLU, the
//    (num_slots, dim, state_len) state view (`_conv_buffer_view`), the
//    per-sequence conv over [prior, x] in `_spec_forward`.
//  * "vllm.models.qwen4_exp.nvidia.ple_layer", Qwen4ExpPLELayer: dilated
//    conv (state length (kernel-1)*dilation, Conv1d with padding and
//    dilation), prefill checkpoints (the comment in the layer's constructor:
//    the window that ends at a checkpoint holds the raw inputs just before it;
//    offsets are multiples of the grid, `get_kv_cache_spec`).
//
// Arithmetic: every convolution output is accumulated in double, bias first,
// then taps in order, and rounded once to the output type (round to nearest,
// ties to even). The CCA depthwise intermediate, which the layer's first
// Conv1d materialises in the model dtype before the grouped conv, is the exact
// value of bias + taps rounded once to that dtype (dw_mode 2, the default of
// the Python front); dw_mode 1 (an fp32 fused multiply-add chain, rounded
// afterwards) is kept as a diagnostic only, to count where such a chain would
// round differently.
//
// Parity pins: every function here is pinned by the CPU tests (zero-state vs.
// a library convolution, a dense Toeplitz formulation, chunked == one-shot
// state carry, checkpoint == one-shot prefix state, tiny brute force, CCA vs.
// library depthwise+grouped convolutions and its special cases). The
// speculative update is pinned by the library convolution of each request's
// accepted token sequence across chains of steps, by its reduction to the
// one-token decode, and by its padding and clamping rules; the per-request
// draft counts by the same accepted-sequence chains with requests that skip
// steps, by the page's slices per request in mixed batches, and by reduction
// to the uniform call; the wide-buffer non-speculative steps by their
// reduction to the narrow buffer.
#include <cmath>
#include <cstdint>
#include <algorithm>
#include <atomic>
#include <cstring>
#include <thread>
#include <vector>

namespace {

enum Dtype { F32 = 0, BF16 = 1, F64 = 2 };

double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// One round-to-nearest-even from double to bfloat16 (8 significant bits,
// exponent range of fp32). The value is scaled by a power of two so that the
// bf16 spacing becomes 1, rounded with nearbyint (ties to even under the
// default rounding mode), and scaled back; all steps but the rounding are exact.
uint16_t double_to_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  double a = std::fabs(v);
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  if (a == 0.0) return sign;
  if (std::isinf(a)) return sign | 0x7F80;
  int e;
  std::frexp(a, &e);            // a in [2^(e-1), 2^e)
  int pe = e - 8;               // spacing of 8-bit significands there
  if (pe < -133) pe = -133;     // subnormal spacing
  double q = std::ldexp(1.0, pe);
  double r = std::nearbyint(a / q) * q;
  if (r >= std::ldexp(1.0, 128)) return sign | 0x7F80;   // overflow -> inf
  float f = (float)r;           // exact: r has <= 8 significant bits
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

// Error-free sum of two doubles (Knuth's TwoSum, round to nearest): s + e
// equals a + b exactly. Needs strict IEEE evaluation (no contraction).
template <class T>
T two_sum(T a, T b, T* e) {
  const T s = a + b;
  const T bb = s - a;
  *e = (a - (s - bb)) + (b - bb);
  return s;
}

// Round a binary128 value once to bfloat16 (nearest, ties to even). hi is the
// nearest double and lo the (sign-exact) remainder; the nearest bf16 of v is
// that of hi unless hi sits exactly on a bf16 midpoint, where lo decides.
uint16_t quad_to_bf16(__float128 v) {
  const double hi = (double)v;
  const double lo = (double)(v - (__float128)hi);
  const uint16_t r = double_to_bf16(hi);
  if (lo == 0.0 || std::isinf(hi) || hi == 0.0) return r;
  int e;
  std::frexp(std::fabs(hi), &e);
  const double half = std::ldexp(1.0, e - 9);          // half a bf16 spacing at hi
  const double m = std::fabs(hi) / half;
  if (m != std::floor(m) || std::fmod(m, 2.0) == 0.0) return r;   // not a midpoint
  // midpoint: round away from hi in the direction of lo
  const double below = (std::floor(m) - 1.0) * half, above = (std::floor(m) + 1.0) * half;
  const double mag = ((lo > 0.0) == (hi > 0.0)) ? above : below;
  return double_to_bf16(hi > 0.0 ? mag : -mag);
}

float quad_to_f32(__float128 v) {
  const double hi = (double)v;
  const double lo = (double)(v - (__float128)hi);
  const float r = (float)hi;
  if (lo == 0.0 || (double)r == hi) return r;      // no rounding decided by lo
  // hi is a float midpoint only if it has exactly 25 significant bits
  const double other = (double)std::nextafter(r, (hi > (double)r) ? INFINITY : -INFINITY);
  if (hi - (double)r != other - hi) return r;         // not a midpoint
  return ((lo > 0.0) == (other > (double)r)) ? (float)other : r;
}

// Exact value of bias + sum_a w[a] * x[a] (n <= 8 taps, products of io values),
// rounded once to io dtype `dt` (for F64 the double sum itself). Each product
// of two bf16 or fp32 values is exact in double; the running sum is certified
// exact with TwoSum, and when a step loses bits the whole sum is redone in
// binary128 with the same certificate. Returns false if even that is inexact
// (terms spanning more than ~90 binades), which no pinned or random input does.
bool exact_dw(int dt, double bias, const double* w, const double* x, int n, double* out) {
  if (dt == F64) {
    double s = bias;
    for (int a = 0; a < n; ++a) s += w[a] * x[a];
    *out = s;
    return true;
  }
  bool exact = true;
  double s = bias, e;
  for (int a = 0; a < n && exact; ++a) {
    s = two_sum(s, w[a] * x[a], &e);
    exact = e == 0.0;
  }
  if (exact) {
    *out = dt == BF16 ? bf16_to_double(double_to_bf16(s)) : (double)(float)s;
    return true;
  }
  __float128 q = bias, qe;
  for (int a = 0; a < n; ++a) {
    q = two_sum(q, (__float128)w[a] * (__float128)x[a], &qe);
    if (qe != 0) return false;
  }
  *out = dt == BF16 ? bf16_to_double(quad_to_bf16(q)) : (double)quad_to_f32(q);
  return true;
}

// Spread of the roundings to io dtype `dt` of the values within e of s: the
// largest distance from r (the rounding of the exact value) to the rounding of
// any value in [s - e, s + e]. Rounding to nearest is monotone, so those
// roundings lie between the roundings of s - e and s + e. Zero unless a
// rounding boundary lies within e of s.
double round_spread(int dt, double s, double e, double r) {
  if (dt == F64) return 0.0;
  auto rnd = [&](double v) {
    return dt == BF16 ? bf16_to_double(double_to_bf16(v)) : (double)(float)v;
  };
  return std::fmax(rnd(s + e) - r, r - rnd(s - e));
}

double ld(const void* p, int dt, int64_t i) {
  switch (dt) {
    case F32: return (double)((const float*)p)[i];
    case BF16: return bf16_to_double(((const uint16_t*)p)[i]);
    default: return ((const double*)p)[i];
  }
}

// Stores one value; for a value that is already representable in `dt` (a state
// copy) this is an exact copy.
void st(void* p, int dt, int64_t i, double v) {
  switch (dt) {
    case F32: ((float*)p)[i] = (float)v; break;   // C conversion: nearest-even
    case BF16: ((uint16_t*)p)[i] = double_to_bf16(v); break;
    default: ((double*)p)[i] = v; break;
  }
}

bool dtype_ok(int dt) { return dt == F32 || dt == BF16 || dt == F64; }

// A resolved request: token rows [start, start+len), its state slot, and
// whether it continues from saved history.
struct Req {
  int64_t start, len;
  int32_t slot;
  int has_state;
};

// Request resolution ("_mix_with_state" builds slots/starts/lens/has-state
// with decodes first, then prefills from query_start_loc; the GDN and PLE
// pages split the batch the same way: decode rows first, prefill rows after).
// Decode requests own q rows each (q = 1 for plain decode; the GDN page's
// multi-token update views x as (B, q, dim)).
std::vector<Req> resolve(int32_t num_decodes, int32_t q, const int32_t* dslots,
                         int64_t dstride, const uint8_t* dh, int32_t num_prefills,
                         const int32_t* qsl_p, const int32_t* pslots,
                         int64_t pstride, const uint8_t* ph) {
  std::vector<Req> rs;
  for (int32_t i = 0; i < num_decodes; ++i)
    rs.push_back({(int64_t)i * q, (int64_t)q, dslots[i * dstride],
                  dh ? (int)(dh[i] != 0) : 1});
  int64_t base = (int64_t)num_decodes * q;
  for (int32_t r = 0; r < num_prefills; ++r)
    rs.push_back({base + qsl_p[r], (int64_t)qsl_p[r + 1] - qsl_p[r],
                  pslots[r * pstride], ph ? (int)(ph[r] != 0) : 1});
  return rs;
}

template <class F>
void parallel_for(int n, int nthreads, F f) {
  if (nthreads <= 1 || n <= 1) {
    f(0, n);
    return;
  }
  if (nthreads > n) nthreads = n;
  std::vector<std::thread> th;
  for (int i = 0; i < nthreads; ++i) {
    int a = (int)((int64_t)n * i / nthreads), b = (int)((int64_t)n * (i + 1) / nthreads);
    th.emplace_back([=] { f(a, b); });
  }
  for (auto& t : th) t.join();
}

// Row mapping and residual fusion shared by the depthwise entry points (PLE
// page, `_short_conv`: the conv result is accumulated into `residual`, and
// `outer_residual` is added in the same pass; `token_indices` maps the call's
// logical rows to rows of the full batch tensors, for batches that mix
// speculative and non-speculative requests).
struct Fuse {
  const int32_t* idx;    // logical row -> physical row of x / out / resid / outer (nullable)
  const void* resid;     // residual added to the result (io dtype, nullable)
  int64_t resid_rs;
  const void* outer;     // outer residual added to the result (io dtype, nullable)
  int64_t outer_rs;
  int64_t row(int64_t logical) const { return idx ? (int64_t)idx[logical] : logical; }
};

// The value stored for one output: act(z) plus the residuals, in double; the
// residual magnitudes join the sum of |terms|.
double fuse_value(const Fuse& f, int io, int64_t prow, int c, double y, double* A) {
  if (f.resid) {
    const double r = ld(f.resid, io, prow * f.resid_rs + c);
    y += r;
    *A += std::fabs(r);
  }
  if (f.outer) {
    const double o = ld(f.outer, io, prow * f.outer_rs + c);
    y += o;
    *A += std::fabs(o);
  }
  return y;
}

// Index of state entry u (oldest first) of channel c in slot `slot`: the pool
// is (num_slots, C, S) ("DS", channel-major; GDN `_conv_buffer_view`) or
// (num_slots, S, C) ("SD", the cache viewed transposed when the conv state is
// not dim-first; GDN and PLE pages, `is_conv_state_dim_first`).
int64_t sidx(int sd, int64_t slot, int64_t C, int64_t S, int64_t c, int64_t u) {
  return sd ? (slot * S + u) * C + c : (slot * C + c) * S + u;
}

struct ConvArgs {
  int32_t C, K, d, act, io, odt;
  const void* x;
  int64_t x_rs;
  void* out;
  int64_t out_rs;
  double* absum;
  const void* w;
  const void* bias;
  void* pool;
  int32_t num_slots;
  int32_t S;                 // state row length (>= H); the window is columns [0, H)
  int32_t sd;                // 1: pool is (num_slots, S, C)
  int32_t ckpt_grid;
  const int32_t* cu_ckpt;
  const int32_t* ckpt_slots;
  int32_t first_prefill;     // index in the request list of prefill 0
  const uint8_t* row_mask;
  Fuse fz;
};

// Depthwise causal conv of one channel range over every request.
//
// For request r and channel c, ext is the request's tokens extended on the left
// by its saved history (H = (K-1)*d raw inputs, oldest first), or by zeros when
// it has no initial state. Output t is the cross-correlation
//   z = b_c + sum_k w[c,k] * ext[H + t - (K-1-k)*d],
// (w[c,K-1] multiplies the current token), then SiLU or identity. The new
// history is the last H entries of ext; a checkpoint at offset p (a multiple of
// the grid, p <= len) receives ext[p .. p+H), the inputs just before p.
void conv_channels(const ConvArgs& a, const std::vector<Req>& reqs, int c0, int c1) {
  const int H = (a.K - 1) * a.d;
  std::vector<double> ext;
  for (size_t ri = 0; ri < reqs.size(); ++ri) {
    const Req& r = reqs[ri];
    if (r.len <= 0) continue;   // a zero-length request has no rows; slot untouched
    const bool valid = r.slot >= 0 && r.slot < a.num_slots;
    for (int c = c0; c < c1; ++c) {
      ext.assign((size_t)(H + r.len), 0.0);
      for (int u = 0; u < H; ++u)
        ext[u] = (r.has_state && valid)
                     ? ld(a.pool, a.io, sidx(a.sd, r.slot, a.C, a.S, c, u))
                     : 0.0;
      for (int64_t t = 0; t < r.len; ++t)
        ext[H + t] = ld(a.x, a.io, a.fz.row(r.start + t) * a.x_rs + c);
      const double b = a.bias ? ld(a.bias, a.io, c) : 0.0;
      for (int64_t t = 0; t < r.len; ++t) {
        const int64_t row = r.start + t;
        if (a.row_mask && !a.row_mask[row]) continue;
        double z = b, A = std::fabs(b);
        for (int k = 0; k < a.K; ++k) {
          double term = ld(a.w, a.io, (int64_t)c * a.K + k) *
                        ext[H + t - (int64_t)(a.K - 1 - k) * a.d];
          z += term;
          A += std::fabs(term);
        }
        const int64_t prow = a.fz.row(row);
        double y = a.act ? z / (1.0 + std::exp(-z)) : z;
        y = fuse_value(a.fz, a.io, prow, c, y, &A);
        st(a.out, a.odt, prow * a.out_rs + c, y);
        if (a.absum) a.absum[row * a.C + c] = A;
      }
      if (valid)
        for (int j = 0; j < H; ++j)
          st(a.pool, a.io, sidx(a.sd, r.slot, a.C, a.S, c, j), ext[r.len + j]);
      if (a.ckpt_grid > 0 && (int)ri >= a.first_prefill && a.cu_ckpt) {
        const int pr = (int)ri - a.first_prefill;
        const int32_t cnt = a.cu_ckpt[pr + 1] - a.cu_ckpt[pr];
        for (int32_t m = 1; m <= cnt; ++m) {
          const int64_t p = (int64_t)m * a.ckpt_grid;
          if (p > r.len) break;
          const int32_t dst = a.ckpt_slots[a.cu_ckpt[pr] + m - 1];
          if (dst < 0 || dst >= a.num_slots) continue;
          for (int j = 0; j < H; ++j)
            st(a.pool, a.io, sidx(a.sd, dst, a.C, a.S, c, j), ext[p + j]);
        }
      }
    }
  }
}

// Shared by the uniform and the per-request-length calls: request r owns rows
// [start(r), start(r) + len(r)). A request with len 0 is skipped (the GDN
// page's loop: `if q_i == 0: continue`); one with len > S cannot be rolled
// (the kept range S - len would be negative) and is skipped as well.
template <class Start, class Len>
void spec_requests(int32_t C, int32_t K, int32_t d, int32_t S, int32_t state_layout, int32_t act,
                   int32_t io_dtype, int32_t out_dtype, const void* x, int64_t x_rs, void* out,
                   int64_t out_rs, double* absum, const void* w, const void* bias, void* pool,
                   int32_t num_slots, int32_t B, Start start_of, Len len_of, const int32_t* slots,
                   int64_t slot_stride, const int32_t* num_accepted, const uint8_t* row_mask,
                   const Fuse& fz, int32_t nthreads) {
  const int H = (K - 1) * d;
  auto body = [&](int c0, int c1) {
    std::vector<double> ext, buf((size_t)S);
    for (int r = 0; r < B; ++r) {
      const int q = len_of(r);
      if (q <= 0 || q > S) continue;
      ext.assign((size_t)(H + q), 0.0);
      const int32_t slot = slots[r * slot_stride];
      const bool valid = slot >= 0 && slot < num_slots;
      const int a = std::min(std::max(num_accepted[r], 1), std::min(q, S - H + 1));
      const int64_t start = start_of(r);
      for (int c = c0; c < c1; ++c) {
        for (int j = 0; j < S; ++j)
          buf[j] = valid ? ld(pool, io_dtype, sidx(state_layout, slot, C, S, c, j)) : 0.0;
        for (int u = 0; u < H; ++u) ext[u] = buf[a - 1 + u];
        for (int t = 0; t < q; ++t) ext[H + t] = ld(x, io_dtype, fz.row(start + t) * x_rs + c);
        const double b = bias ? ld(bias, io_dtype, c) : 0.0;
        for (int t = 0; t < q; ++t) {
          const int64_t row = start + t;
          if (row_mask && !row_mask[row]) continue;
          double z = b, A = std::fabs(b);
          for (int k = 0; k < K; ++k) {
            double term = ld(w, io_dtype, (int64_t)c * K + k) * ext[H + t - (int64_t)(K - 1 - k) * d];
            z += term;
            A += std::fabs(term);
          }
          const int64_t prow = fz.row(row);
          const double y = fuse_value(fz, io_dtype, prow, c, act ? z / (1.0 + std::exp(-z)) : z, &A);
          st(out, out_dtype, prow * out_rs + c, y);
          if (absum) absum[row * C + c] = A;
        }
        if (valid) {
          for (int j = 0; j < S - q; ++j)
            st(pool, io_dtype, sidx(state_layout, slot, C, S, c, j), buf[a + j]);
          for (int t = 0; t < q; ++t)
            st(pool, io_dtype, sidx(state_layout, slot, C, S, c, (S - q) + t), ext[H + t]);
        }
      }
    }
  };
  parallel_for(C, nthreads, body);
}

}  // namespace

extern "C" {

int oracle_abi_version(void) { return 1; }

// Exposed for the rounding pins.
uint16_t oracle_double_to_bf16(double v) { return double_to_bf16(v); }

// Depthwise stateful causal conv over one batch (decode rows, then prefills).
// x, w, bias and pool share io_dtype; out is written in out_dtype (F64 allowed
// so that pins compare unrounded sums). pool is (num_slots, C, S), or
// (num_slots, S, C) with state_layout = 1, with
// S = state_len >= H = (K-1)*d (0 means H). When S > H (a buffer sized for
// speculative rollback) the non-speculative steps keep their window in the
// first H columns and leave the rest alone, as the GDN page's wide-buffer path
// does (`_spec_aware_nonspec`: the live window is the leading width-1 entries
// of each row).
// absum (nullable, (T, C) doubles, by logical row) receives |b| + sum_k |w*x|
// (+ |resid| + |outer|) per output.
// row_mask (nullable, T bytes, by logical row): rows with mask 0 are not written.
// token_indices (nullable): logical row -> physical row of x, out, resid and
// outer. resid / outer (nullable): added to the result (see Fuse).
int oracle_conv(int32_t C, int32_t K, int32_t d, int32_t act, int32_t io_dtype,
                int32_t out_dtype, const void* x, int64_t x_rs, void* out,
                int64_t out_rs, double* absum, const void* w, const void* bias,
                void* pool, int32_t num_slots, int32_t state_len, int32_t state_layout,
                int32_t num_decodes, int32_t q,
                const int32_t* decode_slots, int64_t decode_slot_stride,
                const uint8_t* decode_h, int32_t num_prefills,
                const int32_t* qsl_p, const int32_t* prefill_slots,
                int64_t prefill_slot_stride, const uint8_t* prefill_h,
                int32_t ckpt_grid, const int32_t* cu_ckpt,
                const int32_t* ckpt_slots, const uint8_t* row_mask,
                const int32_t* token_indices, const void* resid, int64_t resid_rs,
                const void* outer, int64_t outer_rs, int32_t nthreads) {
  if (C <= 0 || K <= 0 || d <= 0 || q < 0 || num_decodes < 0 || num_prefills < 0)
    return -2;
  const int32_t S = state_len > 0 ? state_len : (K - 1) * d;
  if (S < (K - 1) * d) return -2;
  if (!dtype_ok(io_dtype) || !dtype_ok(out_dtype)) return -3;
  std::vector<Req> reqs =
      resolve(num_decodes, q, decode_slots, decode_slot_stride, decode_h,
              num_prefills, qsl_p, prefill_slots, prefill_slot_stride, prefill_h);
  ConvArgs a{C, K, d, act, io_dtype, out_dtype, x, x_rs, out, out_rs, absum, w,
             bias, pool, num_slots, S, state_layout ? 1 : 0, ckpt_grid, cu_ckpt, ckpt_slots, num_decodes,
             row_mask, Fuse{token_indices, resid, resid_rs, outer, outer_rs}};
  parallel_for(C, nthreads, [&](int c0, int c1) { conv_channels(a, reqs, c0, c1); });
  return 0;
}

// Speculative multi-token update with a rolling state buffer (GDN page,
// _spec_forward: after the step the row loses its accepted prefix at the front
// and gains the new drafts at the back, so its length stays state_len).
// pool is (num_slots, C, S), S >= H = (K-1)*d. Request r owns rows
// [r*q, (r+1)*q) and has `a = num_accepted[r]` accepted tokens from the
// previous step, clamped to [1, min(q, S-H+1)] (the range in which the
// page's slices are well formed). Then
//   ext      = [pool[s][c][a-1 : a-1+H], x_r]     (the window ending at the last accepted input)
//   outputs  = the depthwise definition over ext
//   pool[s]  = [pool[s][c][a : a+S-q], x_r]      (length S; q <= S required)
// A slot outside the pool is a padding row: zero window, no write.
int oracle_conv_spec(int32_t C, int32_t K, int32_t d, int32_t S, int32_t state_layout, int32_t act,
                     int32_t io_dtype, int32_t out_dtype, const void* x, int64_t x_rs,
                     void* out, int64_t out_rs, double* absum, const void* w,
                     const void* bias, void* pool, int32_t num_slots, int32_t B,
                     int32_t q, const int32_t* slots, int64_t slot_stride,
                     const int32_t* num_accepted, const uint8_t* row_mask,
                     const int32_t* token_indices, const void* resid, int64_t resid_rs,
                     const void* outer, int64_t outer_rs, int32_t nthreads) {
  const int H = (K - 1) * d;
  if (C <= 0 || K <= 0 || d <= 0 || B < 0 || q < 1 || S < H || q > S) return -2;
  if (!dtype_ok(io_dtype) || !dtype_ok(out_dtype)) return -3;
  spec_requests(C, K, d, S, state_layout, act, io_dtype, out_dtype, x, x_rs, out, out_rs, absum,
                w, bias, pool, num_slots, B, [&](int r) { return (int64_t)r * q; },
                [&](int) { return q; }, slots, slot_stride, num_accepted, row_mask,
                Fuse{token_indices, resid, resid_rs, outer, outer_rs}, nthreads);
  return 0;
}

// The same update with a draft count per request (GDN page, _spec_forward's
// per-sequence loop over spec_query_start_loc): request r owns rows
// [qsl[r], qsl[r+1]) and q_r = qsl[r+1] - qsl[r]; the rule above applies with
// q = q_r. q_r = 0: the request is skipped (nothing read or written);
// q_r > S: skipped too (its buffer cannot take the drafts).
int oracle_conv_spec_varlen(int32_t C, int32_t K, int32_t d, int32_t S, int32_t state_layout,
                            int32_t act, int32_t io_dtype, int32_t out_dtype, const void* x,
                            int64_t x_rs, void* out, int64_t out_rs, double* absum,
                            const void* w, const void* bias, void* pool, int32_t num_slots,
                            int32_t B, const int32_t* qsl, const int32_t* slots,
                            int64_t slot_stride, const int32_t* num_accepted,
                            const uint8_t* row_mask, const int32_t* token_indices,
                            const void* resid, int64_t resid_rs, const void* outer,
                            int64_t outer_rs, int32_t nthreads) {
  const int H = (K - 1) * d;
  if (C <= 0 || K <= 0 || d <= 0 || B < 0 || S < H || !qsl) return -2;
  if (!dtype_ok(io_dtype) || !dtype_ok(out_dtype)) return -3;
  for (int r = 0; r < B; ++r)
    if (qsl[r + 1] < qsl[r] || qsl[r] < 0) return -2;
  spec_requests(C, K, d, S, state_layout, act, io_dtype, out_dtype, x, x_rs, out, out_rs, absum,
                w, bias, pool, num_slots, B, [&](int r) { return (int64_t)qsl[r]; },
                [&](int r) { return qsl[r + 1] - qsl[r]; }, slots, slot_stride, num_accepted,
                row_mask, Fuse{token_indices, resid, resid_rs, outer, outer_rs}, nthreads);
  return 0;
}

// CCA q/k conv with delayed value (ZayaCCA.project + _mix_with_state).
//
// Channels: raw qk = [q (nq*hd), k (nkv*hd)], C = (nq+nkv)*hd; history
// n = t0 + t1 - 2 raw inputs per channel. Per request and channel, ext is the
// raw input extended by the history (zeros without initial state).
//   dw(c,u)  = b1_c + sum_{a<t0} w1[c,a] * ext[c][u-(t0-1)+a]
//              (dw_mode 2: the exact value rounded once to the io dtype;
//               dw_mode 1, diagnostic: an fp32 fmaf chain, bias first, then
//               rounded to the io dtype; dw_mode 0: the double sum, not rounded)
//   yg(o,t)  = b2_o + sum_{j<hd} sum_{b<t1} W2[o,j,b] * dw(g*hd+j, n+t-(t1-1)+b),
//              g = o / hd  (grouped conv weight (C, hd, t1))
//   qres[h]  = 0.5 * (q[h] + k[h / G]),  G = nq / nkv      (per head, per dim)
//   kres[g]  = mean_{i<G} qres[g*G + i]
//   out row  = [yg_q + qres | yg_k + kres | v_cur | dprev]
//   dprev(t) = v_del[row-1] for t >= 1 in the request, else the saved delayed
//              value (has state) or delayed_init (NULL = zeros).
// State: conv_state[slot][c][j] = ext[c][len + j] (j < n);
//        delayed_state[slot] = v_del[last row of the request].
// dw_chain_diff (nullable; dw_mode 2, bf16): receives the number of depthwise
// values that an fp32 fmaf chain (bias first, taps in order) would round to a
// different bf16 value than the exact one (a diagnostic, not a result).
// dw_allow (nullable, (T, W) doubles, dw_mode 2): for each conv output, the
// most it can move when its depthwise inputs are summed in fp32 in any order
// before the rounding to the io dtype: sum over its inputs of |W2| times the
// rounding spread of that input, where the spread is taken over the values
// within the fp32 summation bound gamma_{t0+1} (|b1| + sum |w1 x|) of the exact
// sum (a tolerance term for the checker, not a result; zero for value columns).
// Returns -4 if a depthwise sum is not exact even in binary128.
int oracle_cca(int32_t nq, int32_t nkv, int32_t hd, int32_t t0, int32_t t1,
               int32_t io_dtype, int32_t out_dtype, int32_t dw_mode,
               const void* qp, int64_t q_rs, const void* kp, int64_t k_rs,
               const void* vcur, int64_t vc_rs, const void* vdel, int64_t vd_rs,
               void* out, int64_t out_rs, double* absum, const void* w_dw,
               const void* b_dw, const void* w_gr, const void* b_gr,
               const void* delayed_init, void* conv_state, void* delayed_state,
               int32_t num_slots, int32_t num_decodes, const int32_t* decode_slots,
               int64_t dstride, int32_t num_prefills, const int32_t* qsl_p,
               const int32_t* prefill_slots, int64_t pstride,
               const uint8_t* prefill_h, const uint8_t* row_mask,
               int64_t* dw_chain_diff, double* dw_allow, int32_t nthreads) {
  if (nq <= 0 || nkv <= 0 || hd <= 0 || t0 <= 0 || t1 <= 0 || nq % nkv) return -2;
  if (dw_mode < 0 || dw_mode > 2 || (dw_mode == 2 && t0 > 8)) return -2;
  if (!dtype_ok(io_dtype) || !dtype_ok(out_dtype)) return -3;
  std::atomic<bool> inexact_any{false};
  std::atomic<int64_t> chain_diff{0};
  const int C = (nq + nkv) * hd, n = t0 + t1 - 2, G = nq / nkv;
  const int qdim = nq * hd, vd = nkv * hd / 2, W = (nq + 2 * nkv) * hd;
  const int ngroups = nq + nkv;
  std::vector<Req> reqs = resolve(num_decodes, 1, decode_slots, dstride, nullptr,
                                  num_prefills, qsl_p, prefill_slots, pstride,
                                  prefill_h);

  auto raw = [&](int64_t row, int c) -> double {
    return c < qdim ? ld(qp, io_dtype, row * q_rs + c)
                    : ld(kp, io_dtype, row * k_rs + (c - qdim));
  };

  // Conv part, one group (hd dw channels in, hd conv channels out) at a time.
  // fp32 summation bound of bias + t0 products, any order (each product and
  // each of the t0 additions rounded at most once), plus the double sum's own
  // rounding
  const double u32 = std::ldexp(1.0, -24);
  const double gam = (t0 + 1) * u32 / (1.0 - (t0 + 1) * u32) + (t0 + 1) * std::ldexp(1.0, -52);
  const bool want_allow = dw_allow && dw_mode == 2;
  auto groups = [&](int g0, int g1) {
    std::vector<double> ext, dw, spr;
    bool inexact = false;
    int64_t ndiff = 0;
    for (const Req& r : reqs) {
      if (r.len <= 0) continue;
      const bool valid = r.slot >= 0 && r.slot < num_slots;
      const int64_t E = n + r.len;
      for (int g = g0; g < g1; ++g) {
        // ext and dw for the group's input channels, indexed [j][u]
        ext.assign((size_t)hd * E, 0.0);
        dw.assign((size_t)hd * E, 0.0);
        if (want_allow) spr.assign((size_t)hd * E, 0.0);
        for (int j = 0; j < hd; ++j) {
          const int c = g * hd + j;
          double* e = &ext[(size_t)j * E];
          for (int u = 0; u < n; ++u)
            e[u] = (r.has_state && valid)
                       ? ld(conv_state, io_dtype, ((int64_t)r.slot * C + c) * n + u)
                       : 0.0;
          for (int64_t t = 0; t < r.len; ++t) e[n + t] = raw(r.start + t, c);
          for (int64_t u = t0 - 1; u < E; ++u) {
            double v;
            if (dw_mode == 2) {
              // the Conv1d output materialised in the io dtype: exact value,
              // one rounding
              double wa[8], xa[8];
              for (int a = 0; a < t0; ++a) {
                wa[a] = ld(w_dw, io_dtype, (int64_t)c * t0 + a);
                xa[a] = e[u - (t0 - 1) + a];
              }
              if (!exact_dw(io_dtype, ld(b_dw, io_dtype, c), wa, xa, t0, &v)) inexact = true;
              if (want_allow) {
                double sd = ld(b_dw, io_dtype, c), A1 = std::fabs(sd);
                for (int a = 0; a < t0; ++a) {
                  sd += wa[a] * xa[a];
                  A1 += std::fabs(wa[a] * xa[a]);
                }
                spr[(size_t)j * E + u] = round_spread(io_dtype, sd, gam * A1, v);
              }
              if (dw_chain_diff && io_dtype == BF16) {
                // diagnostic: would an fp32 fmaf chain (bias first) round elsewhere?
                float acc = (float)ld(b_dw, io_dtype, c);
                for (int a = 0; a < t0; ++a) acc = std::fmaf((float)wa[a], (float)xa[a], acc);
                if (bf16_to_double(double_to_bf16(acc)) != v) ++ndiff;
              }
            } else if (dw_mode == 1) {
              float acc = (float)ld(b_dw, io_dtype, c);
              for (int a = 0; a < t0; ++a)
                acc = std::fmaf((float)ld(w_dw, io_dtype, (int64_t)c * t0 + a),
                                (float)e[u - (t0 - 1) + a], acc);
              // materialised in the io dtype (round from the fp32 value)
              if (io_dtype == BF16) v = bf16_to_double(double_to_bf16(acc));
              else v = (double)acc;
            } else {
              v = ld(b_dw, io_dtype, c);
              for (int a = 0; a < t0; ++a)
                v += ld(w_dw, io_dtype, (int64_t)c * t0 + a) * e[u - (t0 - 1) + a];
            }
            dw[(size_t)j * E + u] = v;
          }
        }
        for (int64_t t = 0; t < r.len; ++t) {
          const int64_t row = r.start + t, u = n + t;
          if (row_mask && !row_mask[row]) continue;
          for (int oo = 0; oo < hd; ++oo) {
            const int o = g * hd + oo;
            double y = ld(b_gr, io_dtype, o), A = std::fabs(y), allow = 0.0;
            for (int j = 0; j < hd; ++j)
              for (int b = 0; b < t1; ++b) {
                const double w2 = ld(w_gr, io_dtype, ((int64_t)o * hd + j) * t1 + b);
                double term = w2 * dw[(size_t)j * E + u - (t1 - 1) + b];
                y += term;
                A += std::fabs(term);
                if (want_allow) allow += std::fabs(w2) * spr[(size_t)j * E + u - (t1 - 1) + b];
              }
            double res;
            if (o < qdim) {   // query head h = g, paired key head h / G
              const int e = oo, h = g;
              const double qv = raw(row, h * hd + e), kv = raw(row, qdim + (h / G) * hd + e);
              res = 0.5 * (qv + kv);
              A += 0.5 * (std::fabs(qv) + std::fabs(kv));
            } else {          // key head kg: mean of its G query residuals
              const int kg = g - nq, e = oo;
              const double kv = raw(row, qdim + kg * hd + e);
              double s = 0.0;
              for (int i = 0; i < G; ++i) {
                const double qv = raw(row, (kg * G + i) * hd + e);
                s += 0.5 * (qv + kv);
                A += 0.5 * (std::fabs(qv) + std::fabs(kv)) / G;
              }
              res = s / G;
            }
            st(out, out_dtype, row * out_rs + o, y + res);
            if (absum) absum[row * W + o] = A;
            if (dw_allow) dw_allow[row * W + o] = allow;
          }
        }
        if (valid)
          for (int j = 0; j < hd; ++j)
            for (int jj = 0; jj < n; ++jj)
              st(conv_state, io_dtype, ((int64_t)r.slot * C + g * hd + j) * n + jj,
                 ext[(size_t)j * E + r.len + jj]);
      }
    }
    if (inexact) inexact_any = true;
    if (dw_chain_diff && ndiff) chain_diff += ndiff;
  };
  parallel_for(ngroups, nthreads, groups);
  if (inexact_any) return -4;   // a depthwise sum that binary128 cannot hold exactly
  if (dw_chain_diff) *dw_chain_diff = chain_diff;

  // Value part: current value copied, delayed value shifted by one token.
  for (const Req& r : reqs) {
    if (r.len <= 0) continue;
    const bool valid = r.slot >= 0 && r.slot < num_slots;
    for (int64_t t = 0; t < r.len; ++t) {
      const int64_t row = r.start + t;
      if (row_mask && !row_mask[row]) continue;
      for (int e = 0; e < vd; ++e) {
        st(out, out_dtype, row * out_rs + C + e, ld(vcur, io_dtype, row * vc_rs + e));
        double dp;
        if (t >= 1) dp = ld(vdel, io_dtype, (row - 1) * vd_rs + e);
        else if (r.has_state && valid) dp = ld(delayed_state, io_dtype, (int64_t)r.slot * vd + e);
        else dp = delayed_init ? ld(delayed_init, io_dtype, e) : 0.0;
        st(out, out_dtype, row * out_rs + C + vd + e, dp);
        if (absum) {
          absum[row * W + C + e] = 0.0;
          absum[row * W + C + vd + e] = 0.0;
        }
        if (dw_allow) {
          dw_allow[row * W + C + e] = 0.0;
          dw_allow[row * W + C + vd + e] = 0.0;
        }
      }
    }
    if (valid)
      for (int e = 0; e < vd; ++e)
        st(delayed_state, io_dtype, (int64_t)r.slot * vd + e,
           ld(vdel, io_dtype, (r.start + r.len - 1) * vd_rs + e));
  }
  return 0;
}

// Plain copies between a dense (n, row_elems) buffer and pool rows idx[i].
// Gather of an index outside [0, num_slots) yields a zero row (a padding row
// has no history: _mix_with_state masks history by has-state); scatter skips it.
int oracle_state_gather(int32_t elsize, int64_t row_elems, const void* pool,
                        int32_t num_slots, const int32_t* idx, int64_t idx_stride,
                        int32_t n, void* dense) {
  const int64_t rb = row_elems * elsize;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = idx[i * idx_stride];
    if (s < 0 || s >= num_slots)
      std::memset((char*)dense + i * rb, 0, (size_t)rb);
    else
      std::memcpy((char*)dense + i * rb, (const char*)pool + s * rb, (size_t)rb);
  }
  return 0;
}

int oracle_state_scatter(int32_t elsize, int64_t row_elems, const void* dense,
                         const int32_t* idx, int64_t idx_stride, int32_t n,
                         void* pool, int32_t num_slots) {
  const int64_t rb = row_elems * elsize;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = idx[i * idx_stride];
    if (s < 0 || s >= num_slots) continue;
    std::memcpy((char*)pool + s * rb, (const char*)dense + i * rb, (size_t)rb);
  }
  return 0;
}

}  // extern "C"
