// Device helpers shared by the depthwise kernels (conv.hip, spec.hip):
// workgroup -> request/chunk resolution, register-window element access,
// weight loading, the fp32 tap chain and the bf16 tap-pair dot product.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace sc {

// ---------------------------------------------------------------------------
// request / chunk resolution
// ---------------------------------------------------------------------------

// Logical workgroup index from the hardware one. Workgroups are dealt to the
// 8 XCDs round-robin; this gives each XCD a contiguous run of logical blocks,
// so consecutive chunks of the same channels (whose halos overlap) share an L2.
__device__ __forceinline__ int logical_block(int n_logical, int per_xcd) {
  const int b = (int)blockIdx.x;
  const int lb = (b % kXcds) * per_xcd + b / kXcds;
  return lb < n_logical ? lb : -1;
}

// Chunk ids of request r are [base(r), base(r+1)) with
// base(r) = floor(qsl[r] / chunk) + r, an upper bound on the chunks the request
// needs that is monotone in r and computable per request. So the request owning
// chunk id `id` is #{i in [1, B] : base(i) <= id}, counted wave-parallel. The
// predicate base(i) <= id holds for i up to the answer and fails after it, so
// up to B = 4096 two rounds of loads find it: 64 evenly spaced samples (every
// step-th index, step = ceil(B / 64)) locate the segment between two samples
// that holds the boundary, then the step - 1 indices inside it are counted.
// Larger batches count every index in rounds of 64.
// Must be called by full waves (uses ballot).
__device__ __forceinline__ int find_request(const int32_t* qsl, int B, int id, int chunk) {
  const int lane = (int)(threadIdx.x & 63);
  if (B > 4096) {
    int cnt = 0;
    for (int i0 = 1; i0 <= B; i0 += 64) {
      const int i = i0 + lane;
      bool p = false;
      if (i <= B) p = (qsl[i] / chunk + i) <= id;
      cnt += __popcll(__ballot(p));
    }
    return cnt;
  }
  const int step = (B + 63) >> 6;                  // 1 .. 64
  const int i1 = (lane + 1) * step;                // samples step, 2 step, ... (those <= B)
  bool p1 = false;
  if (i1 <= B) p1 = (qsl[i1] / chunk + i1) <= id;
  const int c1 = __popcll(__ballot(p1));           // the answer is in [c1 step, (c1 + 1) step)
  const int i2 = c1 * step + 1 + lane;
  bool p2 = false;
  if (lane < step - 1 && i2 <= B) p2 = (qsl[i2] / chunk + i2) <= id;
  return c1 * step + __popcll(__ballot(p2));
}

// Request lookup that also returns qsl[r] and qsl[r+1]. With B < 64 every
// needed entry is loaded once by one lane (lane l holds qsl[l]) and read back
// with readlane; larger batches use find_request plus two loads.
// Must be called by full waves.
__device__ __forceinline__ int find_request_bounds(const int32_t* qsl, int B, int id, int chunk,
                                                   int& s0, int& s1) {
  if (B < 64) {
    const int lane = (int)(threadIdx.x & 63);
    const int v = lane <= B ? qsl[lane] : 0x7FFFFFFF;
    const bool p = lane >= 1 && lane <= B && (v / chunk + lane) <= id;
    const int r = __popcll(__ballot(p));
    s0 = __builtin_amdgcn_readlane(v, r);
    s1 = __builtin_amdgcn_readlane(v, min(r + 1, 63));
    return r;
  }
  const int r = find_request(qsl, B, id, chunk);
  if (r < B) {
    s0 = qsl[r];
    s1 = qsl[r + 1];
  }
  return r;
}

// Has-state flag of request r when r is the same for the whole workgroup:
// the aligned 32-bit word holding the flag byte is read with a scalar load
// (gfx9 has no scalar byte load; a vector byte load would make the next
// vmcnt wait cover every row load issued before it). The word never leaves
// the 4-byte-aligned block of the flag, so it stays inside the flag's page.
__device__ __forceinline__ bool uniform_flag(const uint8_t* flags, int64_t r) {
  typedef const __attribute__((address_space(1))) uint32_t* gword;
  const uintptr_t p = (uintptr_t)(flags + r);
  const uint32_t word = *(gword)(p & ~(uintptr_t)3);
  return ((word >> (8 * (p & 3))) & 0xFFu) != 0;
}

struct Work {
  int r, j, L, t0, t1;
  int64_t start;
  int32_t slot;
  bool valid, h;
};

__device__ __forceinline__ bool resolve_work(const ConvArgs& a, int cid, Work& w) {
  if (a.qsl == nullptr) {   // uniform update: batch x q rows
    const int cpr = (a.q + a.chunk - 1) / a.chunk;
    w.r = cid / cpr;
    w.j = cid - w.r * cpr;
    if (w.r >= a.batch) return false;
    w.start = (int64_t)w.r * a.q;
    w.L = a.q;
  } else {
    w.r = find_request(a.qsl, a.batch, cid, a.chunk);
    if (w.r >= a.batch) return false;
    const int s0 = a.qsl[w.r], s1 = a.qsl[w.r + 1];
    if (s0 < 0) return false;
    w.j = cid - (s0 / a.chunk + w.r);
    w.start = s0;
    w.L = s1 - s0;
  }
  if (w.j < 0 || w.L <= 0 || w.start >= a.num_tokens) return false;
  if (w.start + w.L > a.num_tokens) w.L = (int)(a.num_tokens - w.start);
  w.t0 = w.j * a.chunk;
  if (w.t0 >= w.L) return false;
  w.t1 = min(w.L, w.t0 + a.chunk);
  w.slot = a.slots[(int64_t)w.r * a.slot_stride];
  w.valid = w.slot >= 0 && w.slot < a.num_slots;
  w.h = w.valid && (a.has_init ? a.has_init[w.r] != 0 : true);
  return true;
}

// ---------------------------------------------------------------------------
// register-window helpers (all indices compile-time after unrolling)
// ---------------------------------------------------------------------------
template <class E>
__device__ __forceinline__ float widen(uint32_t b) {
  if constexpr (E::VEC == 8) return __uint_as_float(b << 16);
  else return __uint_as_float(b);
}

// element e of a flat array of 16-byte vectors
template <class E>
__device__ __forceinline__ uint32_t get_flat(const u32x4* v, int e) {
  return E::get(v[e / E::VEC], e % E::VEC);
}
template <class E>
__device__ __forceinline__ void set_flat(u32x4* v, int e, uint32_t val) {
  E::set(v[e / E::VEC], e % E::VEC, val);
}

template <class E, int K>
__device__ __forceinline__ void load_weights(const void* w, int c0, float (*wt)[E::VEC]) {
  constexpr int VEC = E::VEC;
  using S = typename E::S;
  const S* wp = (const S*)w + (int64_t)c0 * K;
  float flat[VEC * K];
#pragma unroll
  for (int v = 0; v < K; ++v) E::unpack(ld16(wp + v * VEC), flat + v * VEC);
#pragma unroll
  for (int ch = 0; ch < VEC; ++ch)
#pragma unroll
    for (int k = 0; k < K; ++k) wt[k][ch] = flat[ch * K + k];
}

template <class E, int K, int D, bool SILU>
__device__ __forceinline__ void conv_point(const float (*win)[E::VEC], int pos,
                                           const float (*wt)[E::VEC], const float* bs,
                                           float* z) {
#pragma unroll
  for (int ch = 0; ch < E::VEC; ++ch) {
    float acc = bs[ch];
#pragma unroll
    for (int k = 0; k < K; ++k) acc = __builtin_fmaf(wt[k][ch], win[pos - (K - 1 - k) * D][ch], acc);
    z[ch] = SILU ? silu(acc) : acc;
  }
}

// ---------------------------------------------------------------------------
// row mapping and residual fusion (PLE page, _short_conv / ple_conv)
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool fused(const ConvArgs& a) {
  return a.tok != nullptr || a.outer != nullptr || a.accumulate != 0;
}
// physical row of logical row r; a map entry outside [0, phys_rows) is a
// caller error and is clamped so that no access leaves the tensors
__device__ __forceinline__ int64_t phys_row(const ConvArgs& a, int64_t r) {
  if (!a.tok) return r;
  const int64_t p = a.tok[r];
  return p < 0 ? 0 : (p >= a.phys_rows ? a.phys_rows - 1 : p);
}
// z (one vector of channels at physical row pr, channel c0) plus the residual
// held in out (accumulate) and the outer residual, in that order, in fp32
template <class E>
__device__ __forceinline__ void add_residuals(const ConvArgs& a, int64_t pr, int c0, float* z) {
  using S = typename E::S;
  if (a.accumulate) {
    float r[E::VEC];
    E::unpack(ld16((const S*)a.out + pr * a.out_rs + c0), r);
#pragma unroll
    for (int ch = 0; ch < E::VEC; ++ch) z[ch] += r[ch];
  }
  if (a.outer) {
    float o[E::VEC];
    E::unpack(ld16((const S*)a.outer + pr * a.outer_rs + c0), o);
#pragma unroll
    for (int ch = 0; ch < E::VEC; ++ch) z[ch] += o[ch];
  }
}

// Pair-of-taps dot product on bf16 data (v_dot2c_f32_bf16): acc + w.x over a
// (older, newer) pair, fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t w_pair, uint32_t x_pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w_pair),
                                         __builtin_bit_cast(bf16x2, x_pair), acc, false);
}

// Pair of channel ch's values from rows a (older, low half) and b (newer).
__device__ __forceinline__ uint32_t row_pair(const u32x4& ra, const u32x4& rb, int ch) {
  return __builtin_amdgcn_perm(rb[ch >> 1], ra[ch >> 1], (ch & 1) ? 0x07060302u : 0x05040100u);
}

// Scalar element access for the one-channel-per-lane kernels.
template <class E>
__device__ __forceinline__ uint32_t ld_el(const typename E::S* p) { return (uint32_t)*p; }

template <class E>
__device__ __forceinline__ typename E::S narrow(float v) {
  if constexpr (E::VEC == 8) return __builtin_bit_cast(uint16_t, (__bf16)v);
  else return __float_as_uint(v);
}

}  // namespace sc
