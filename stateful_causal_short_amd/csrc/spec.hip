// Depthwise conv updates on a state buffer widened for speculative rollback.
//
// Operation (GDN page "vllm.model_executor.layers.mamba.ops.cpu.gdn_attention",
// _spec_forward, per-sequence rolling buffer; PLE page
// "vllm.models.qwen4_exp.nvidia.ple_layer", spec mode with a state capacity of
// conv_state_len + num_spec_tokens): each channel keeps S >= H = (K-1)*d
// entries. A speculative request of q tokens whose previous step had `a`
// accepted tokens (clamped to [1, min(q, S-H+1)], the range in which the
// page's slices are well formed) reads the H entries starting at a-1 as its
// history, produces out[t] = act(b + sum_k w[k] * ext[H + t - (K-1-k)*d]) over
// ext = [history, x], and leaves its buffer as the entries from a on, cut to
// S - q, followed by the q new tokens. With a draft count per request (the GDN
// page's loop over spec_query_start_loc) request r owns rows [qsl[r], qsl[r+1])
// and one with no drafts, or more than S, is skipped whole. A plain
// (non-speculative) update on such a buffer uses the first H entries as the
// window and leaves the rest as they were (GDN page, _spec_aware_nonspec: the
// live window is the leading width-1 entries of each row).
//
// Layout: pool (num_slots, C, S). A workgroup takes one request and 256
// vectors of channels; their state rows form one contiguous region of 256 * S
// vectors, which is loaded and stored with unit-stride lanes and staged in LDS.
// Each lane then reads its own channels' entries at the runtime offset a-1 and
// rolls them in place (its region is private to the lane), so a runtime
// acceptance count costs only LDS addressing. The token arithmetic is that of
// the narrow-buffer kernels (tap pairs on v_dot2c_f32_bf16 for the shapes the
// prefill kernel pairs, an fp32 fused multiply-add chain otherwise), so a fully
// accepted speculative chain reproduces the prefill outputs bit for bit.
#include "conv_device.hpp"

namespace sc {

constexpr int kSpecQMax = 8;    // tokens per request on the register path
constexpr int kSpecSMax = 16;   // state entries per channel staged in LDS

// DS pool in LDS: a lane's channels hold 4*S words (S vectors); with one pad
// word per lane the lane stride is odd, so the element-wise window and roll
// accesses of a wave fall in distinct banks. Without room for the pad (S = 16)
// the stride stays 4*S.
__host__ __device__ constexpr int ds_lane_words(int S, int block) {
  return (size_t)block * (4 * S + 1) * 4 <= 65536 ? 4 * S + 1 : 4 * S;
}

template <class E, int K, int D, bool SILU, bool SPEC, bool FUSE>
__global__ __launch_bounds__(kBlock) void conv_rollbuf(ConvArgs a) {
  using St = typename E::S;
  constexpr int H = (K - 1) * D;
  constexpr int VEC = E::VEC;
  constexpr bool PAIRS = VEC == 8 && ((K == 4 && D <= 3) || (K == 2 && D == 1));
  constexpr int NP = K / 2;
  constexpr int QM = kSpecQMax;
  extern __shared__ u32x4 region[];   // SD: kBlock * S vectors; DS: kBlock lanes of ds_lane_words

  const int lb = logical_block(a.n_logical, a.per_xcd);
  if (lb < 0) return;                       // uniform over the workgroup
  const int r = lb / a.n_cblk, cb = lb - r * a.n_cblk;
  if (r >= a.batch) return;
  const int tid = (int)threadIdx.x;
  const int cbase = cb * kBlock * VEC;
  const int c0 = cbase + tid * VEC;
  const bool lane_ok = c0 < a.C;
  const int Sl = a.S;
  int q = a.q;
  int64_t start = (int64_t)r * q;
  if (a.qsl) {   // a draft count per request; a.q bounds them all
    start = a.qsl[r];
    q = a.qsl[r + 1] - a.qsl[r];
    if (q <= 0 || q > a.q || q > Sl || start < 0 || start + q > a.num_tokens) return;
  }
  const int nvec = (min(a.C - cbase, kBlock * VEC) / VEC) * Sl;
  const int lw = ds_lane_words(Sl, kBlock);  // DS: words per lane in LDS
  uint32_t* rw = (uint32_t*)region;

  // weights and bias (independent of the request)
  uint32_t wp[PAIRS ? NP : 1][VEC];
  float wt[PAIRS ? 1 : K][VEC];
  u32x4 bsv = u32x4{0, 0, 0, 0};
  if (lane_ok) {
    if constexpr (PAIRS) {
      u32x4 wv[NP * 2];
#pragma unroll
      for (int v = 0; v < NP * 2; ++v) wv[v] = ld16((const St*)a.w + (int64_t)c0 * K + v * VEC);
#pragma unroll
      for (int ch = 0; ch < VEC; ++ch)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int word = ch * NP + p;
          wp[p][ch] = wv[word >> 2][word & 3];
        }
    } else {
      load_weights<E, K>(a.w, c0, wt);
    }
    if (a.bias) bsv = ld16((const St*)a.bias + c0);
  }

  // physical row of the request's token u (through the row map when fused)
  auto prow = [&](int u) -> int64_t {
    if constexpr (FUSE) return phys_row(a, start + u);
    else return start + u;
  };
  // token rows (and fused residuals), then the slot, then the state region
  u32x4 xr[QM], rres[FUSE ? QM : 1], rout[FUSE ? QM : 1];
#pragma unroll
  for (int u = 0; u < QM; ++u)
    xr[u] = (u < q && lane_ok) ? ld16_stream((const St*)a.x + prow(u) * a.x_rs + c0)
                               : u32x4{0, 0, 0, 0};
  if constexpr (FUSE) {
#pragma unroll
    for (int u = 0; u < QM; ++u) {
      const bool ok = u < q && lane_ok;
      rres[u] = (ok && a.accumulate) ? ld16((const St*)a.out + prow(u) * a.out_rs + c0)
                                     : u32x4{0, 0, 0, 0};
      rout[u] = (ok && a.outer) ? ld16((const St*)a.outer + prow(u) * a.outer_rs + c0)
                                : u32x4{0, 0, 0, 0};
    }
  }
  const int32_t slot = a.slots[(int64_t)r * a.slot_stride];
  const bool valid = slot >= 0 && slot < a.num_slots;
  bool hist = valid;
  int acc = 1;
  if constexpr (SPEC) {
    acc = min(max(a.num_acc[r], 1), min(q, Sl - H + 1));
  } else {
    hist = valid && (a.has_init ? uniform_flag(a.has_init, r) : true);
  }
  // SD pool (num_slots, S, C): entry k of the lane's channels is one vector;
  // the lane keeps its own column region[k * kBlock + tid] (no other lane
  // touches it). DS pool: the workgroup's rows are one contiguous region.
  const bool sd = a.sd != 0;
  if (valid) {
    u32x4 sv[kSpecSMax];
    if (sd) {
      const St* sp = (const St*)a.pool + (int64_t)slot * Sl * a.C + c0;
#pragma unroll
      for (int k = 0; k < kSpecSMax; ++k)
        sv[k] = (k < Sl && lane_ok) ? ld16_stream(sp + (int64_t)k * a.C) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < kSpecSMax; ++k)
        if (k < Sl) region[k * kBlock + tid] = sv[k];
    } else {
      // coalesced loads of the workgroup's contiguous rows; vector vi is entry
      // group vi % S of lane vi / S, stored at that lane's padded offset
      const St* sp = (const St*)a.pool + ((int64_t)slot * a.C + cbase) * Sl;
#pragma unroll
      for (int k = 0; k < kSpecSMax; ++k) {
        const int vi = tid + k * kBlock;
        sv[k] = (k < Sl && vi < nvec) ? ld16_stream(sp + vi * VEC) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int k = 0; k < kSpecSMax; ++k) {
        const int vi = tid + k * kBlock;
        if (k < Sl && vi < nvec) {
          const int ln = vi / Sl;
          uint32_t* wd = rw + ln * lw + 4 * (vi - ln * Sl);
#pragma unroll
          for (int d = 0; d < 4; ++d) wd[d] = sv[k][d];
        }
      }
    }
  }
  __syncthreads();

  St* le = (St*)region;
  const int lbase = tid * lw * (int)(4 / sizeof(St));   // DS: channel c0, entry 0 of this lane
  const int off = SPEC ? acc - 1 : 0;
  u32x4 raw[H + QM];
#pragma unroll
  for (int u = 0; u < H; ++u) {
    raw[u] = u32x4{0, 0, 0, 0};
    if (hist && lane_ok) {
      if (sd) {
        raw[u] = region[(off + u) * kBlock + tid];
      } else {
#pragma unroll
        for (int ch = 0; ch < VEC; ++ch) E::set(raw[u], ch, (uint32_t)le[lbase + ch * Sl + off + u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < QM; ++u) raw[H + u] = xr[u];

  if (lane_ok) {
    float bs[VEC];
    E::unpack(bsv, bs);
    float win[PAIRS ? 1 : H + QM][VEC];
    if constexpr (!PAIRS) {
#pragma unroll
      for (int i = 0; i < H + QM; ++i) E::unpack(raw[i], win[i]);
    }
#pragma unroll
    for (int u = 0; u < QM; ++u) {
      if (u < q) {
        float z[VEC];
        if constexpr (PAIRS) {
#pragma unroll
          for (int ch = 0; ch < VEC; ++ch) {
            float accf = bs[ch];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const int r0 = H + u - (K - 1 - 2 * p) * D;
              accf = dot2_bf16(wp[p][ch], row_pair(raw[r0], raw[r0 + D], ch), accf);
            }
            z[ch] = SILU ? silu(accf) : accf;
          }
        } else {
          conv_point<E, K, D, SILU>(win, H + u, wt, bs, z);
        }
        if constexpr (FUSE) {
          float fr[VEC], fo[VEC];
          E::unpack(rres[u], fr);
          E::unpack(rout[u], fo);
#pragma unroll
          for (int ch = 0; ch < VEC; ++ch) {
            if (a.accumulate) z[ch] += fr[ch];
            if (a.outer) z[ch] += fo[ch];
          }
        }
        st16_stream((St*)a.out + prow(u) * a.out_rs + c0, E::pack(z));
      }
    }
    // new buffer contents, in place in the lane's own entries
    if (valid && sd) {
      if constexpr (SPEC) {
        // ascending j reads entry acc + j > j before it is overwritten
        for (int j = 0; j < Sl - q; ++j) region[j * kBlock + tid] = region[(acc + j) * kBlock + tid];
#pragma unroll
        for (int u = 0; u < QM; ++u)
          if (u < q) region[(Sl - q + u) * kBlock + tid] = xr[u];
      } else {
        // window = ext[q .. q+H) = raw[q .. q+H); entries H .. S-1 keep their values
#pragma unroll
        for (int j = 0; j < H; ++j) {
          u32x4 val = u32x4{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < H + QM; ++e)
            if (e == q + j) val = raw[e];
          region[j * kBlock + tid] = val;
        }
      }
    } else if (valid) {
      if constexpr (SPEC) {
        // ascending j reads entry acc + j > j before it is overwritten; the
        // lane's channels go together, so each step's reads are independent
        for (int j = 0; j < Sl - q; ++j) {
          St v8[VEC];
#pragma unroll
          for (int ch = 0; ch < VEC; ++ch) v8[ch] = le[lbase + ch * Sl + acc + j];
#pragma unroll
          for (int ch = 0; ch < VEC; ++ch) le[lbase + ch * Sl + j] = v8[ch];
        }
      }
#pragma unroll
      for (int ch = 0; ch < VEC; ++ch) {
        St* row = le + lbase + ch * Sl;
        if constexpr (SPEC) {
#pragma unroll
          for (int u = 0; u < QM; ++u)
            if (u < q) row[Sl - q + u] = (St)E::get(xr[u], ch);
        } else {
          // window = ext[q .. q+H); entries H .. S-1 keep their values
#pragma unroll
          for (int j = 0; j < H; ++j) {
            const int e = q + j;
            uint32_t val = 0;
            if (e < H) {
              val = hist ? (uint32_t)row[e] : 0u;
            } else {
#pragma unroll
              for (int u = 0; u < QM; ++u)
                if (u == e - H) val = E::get(xr[u], ch);
            }
            row[j] = (St)val;
          }
        }
      }
    }
  }
  __syncthreads();
  if (valid && sd) {
    St* dp = (St*)a.pool + (int64_t)slot * Sl * a.C + c0;
#pragma unroll
    for (int k = 0; k < kSpecSMax; ++k)
      if (k < Sl && lane_ok) st16_stream(dp + (int64_t)k * a.C, region[k * kBlock + tid]);
  } else if (valid) {
    St* dp = (St*)a.pool + ((int64_t)slot * a.C + cbase) * Sl;
#pragma unroll
    for (int k = 0; k < kSpecSMax; ++k) {
      const int vi = tid + k * kBlock;
      if (k < Sl && vi < nvec) {
        const int ln = vi / Sl;
        const uint32_t* wd = rw + ln * lw + 4 * (vi - ln * Sl);
        st16_stream(dp + vi * VEC, u32x4{wd[0], wd[1], wd[2], wd[3]});
      }
    }
  }
}

// DS pool, K = 4, d = 1 (H = 3), bf16, S entries known at compile time. The
// workgroup's state region is staged through LDS with unit-stride lanes as in
// conv_rollbuf, but each lane then reads its own S vectors whole and turns
// them in registers from channel-major (element ch * S + e) into S entry
// vectors (element ch of entry e, the SD order), so the window read at the
// acceptance offset, the roll and the new tokens are whole 16-byte vectors
// picked by workgroup-uniform selects instead of 16-bit LDS accesses.
// Same arithmetic as conv_rollbuf (tap pairs on v_dot2c).
template <int S, bool SILU, bool SPEC>
__global__ __launch_bounds__(kBlock) void conv_rollbuf_ds(ConvArgs a) {
  using E = BF16;
  using St = E::S;
  constexpr int K = 4, D = 1, H = 3, NP = 2, VEC = 8, QM = kSpecQMax;
  static_assert(S >= H && S <= kSpecSMax, "state length");
  __shared__ u32x4 region[kBlock * S];

  const int lb = logical_block(a.n_logical, a.per_xcd);
  if (lb < 0) return;                       // uniform over the workgroup
  const int r = lb / a.n_cblk, cb = lb - r * a.n_cblk;
  if (r >= a.batch) return;
  const int tid = (int)threadIdx.x;
  const int cbase = cb * kBlock * VEC;
  const int c0 = cbase + tid * VEC;
  const bool lane_ok = c0 < a.C;
  int q = a.q;
  int64_t start = (int64_t)r * q;
  if (a.qsl) {   // a draft count per request; a.q bounds them all
    start = a.qsl[r];
    q = a.qsl[r + 1] - a.qsl[r];
    if (q <= 0 || q > a.q || q > S || start < 0 || start + q > a.num_tokens) return;
  }
  const int nvec = (min(a.C - cbase, kBlock * VEC) / VEC) * S;

  uint32_t wp[NP][VEC];
  u32x4 bsv = u32x4{0, 0, 0, 0};
  if (lane_ok) {
    u32x4 wv[NP * 2];
#pragma unroll
    for (int v = 0; v < NP * 2; ++v) wv[v] = ld16((const St*)a.w + (int64_t)c0 * K + v * VEC);
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int word = ch * NP + p;
        wp[p][ch] = wv[word >> 2][word & 3];
      }
    if (a.bias) bsv = ld16((const St*)a.bias + c0);
  }
  u32x4 xr[QM];
#pragma unroll
  for (int u = 0; u < QM; ++u)
    xr[u] = (u < q && lane_ok) ? ld16_stream((const St*)a.x + (start + u) * a.x_rs + c0)
                               : u32x4{0, 0, 0, 0};
  const int32_t slot = a.slots[(int64_t)r * a.slot_stride];
  const bool valid = slot >= 0 && slot < a.num_slots;
  bool hist = valid;
  int acc = 1;
  if constexpr (SPEC) {
    acc = min(max(a.num_acc[r], 1), min(q, S - H + 1));
  } else {
    hist = valid && (a.has_init ? uniform_flag(a.has_init, r) : true);
  }
  St* const sp = (St*)a.pool + ((int64_t)(valid ? slot : 0) * a.C + cbase) * S;
  if (valid) {
    u32x4 sv[S];
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const int vi = tid + k * kBlock;
      sv[k] = vi < nvec ? ld16_stream(sp + vi * VEC) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const int vi = tid + k * kBlock;
      if (vi < nvec) region[vi] = sv[k];
    }
  }
  __syncthreads();

  // the lane's channel-major vectors, then its entry vectors
  u32x4 ent[S];
  {
    u32x4 cm[S];
#pragma unroll
    for (int k = 0; k < S; ++k)
      cm[k] = (valid && lane_ok) ? region[tid * S + k] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < S; ++e)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int m0 = (2 * w) * S + e, m1 = (2 * w + 1) * S + e;   // channels 2w, 2w+1
        const uint32_t b0 = 2u * (uint32_t)(m0 & 1), b1 = 4u + 2u * (uint32_t)(m1 & 1);
        ent[e][w] = __builtin_amdgcn_perm(cm[m1 >> 3][(m1 & 7) >> 1], cm[m0 >> 3][(m0 & 7) >> 1],
                                          b0 | ((b0 + 1) << 8) | (b1 << 16) | ((b1 + 1) << 24));
      }
  }

  // window: entries acc-1 .. acc+H-2 (speculative) or 0 .. H-1; zeros without history
  u32x4 raw[H + QM];
#pragma unroll
  for (int u = 0; u < H; ++u) {
    u32x4 wv = ent[u];
    if constexpr (SPEC) {
#pragma unroll
      for (int av = 2; av <= S - H + 1; ++av)
        if (acc == av) wv = ent[av - 1 + u];
    }
    raw[u] = hist ? wv : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < QM; ++u) raw[H + u] = xr[u];

  if (lane_ok) {
    float bs[VEC];
    E::unpack(bsv, bs);
#pragma unroll
    for (int u = 0; u < QM; ++u) {
      if (u < q) {
        float z[VEC];
#pragma unroll
        for (int ch = 0; ch < VEC; ++ch) {
          float accf = bs[ch];
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const int r0 = H + u - (K - 1 - 2 * p) * D;
            accf = dot2_bf16(wp[p][ch], row_pair(raw[r0], raw[r0 + D], ch), accf);
          }
          z[ch] = SILU ? silu(accf) : accf;
        }
        st16_stream((St*)a.out + (start + u) * a.out_rs + c0, E::pack(z));
      }
    }
  }
  if (!valid) return;                       // uniform over the workgroup

  // new entries: speculative, entry j = old entry acc + j for j < S - q, then
  // the q tokens; plain, entries j < H = ext[q + j] (ext = window, tokens)
  u32x4 nent[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    if constexpr (SPEC) {
      u32x4 roll = u32x4{0, 0, 0, 0}, tok = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int av = 1; av + j < S; ++av)
        if (acc == av) roll = ent[av + j];
#pragma unroll
      for (int u = 0; u < QM; ++u)
        if (u == j - (S - q)) tok = xr[u];
      nent[j] = j < S - q ? roll : tok;
    } else {
      u32x4 v = ent[j];
      if (j < H) {
#pragma unroll
        for (int e = 0; e < H + QM; ++e)
          if (e == q + j) v = raw[e];
      }
      nent[j] = v;
    }
  }
  // back to channel-major, into the lane's own region slots
  if (lane_ok) {
#pragma unroll
    for (int k = 0; k < S; ++k) {
      u32x4 cm;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int m0 = 8 * k + 2 * w, m1 = m0 + 1;     // elements (channel, entry) = divmod(m, S)
        const int ch0 = m0 / S, e0 = m0 % S, ch1 = m1 / S, e1 = m1 % S;
        const uint32_t b0 = 2u * (uint32_t)(ch0 & 1), b1 = 4u + 2u * (uint32_t)(ch1 & 1);
        cm[w] = __builtin_amdgcn_perm(nent[e1][ch1 >> 1], nent[e0][ch0 >> 1],
                                      b0 | ((b0 + 1) << 8) | (b1 << 16) | ((b1 + 1) << 24));
      }
      region[tid * S + k] = cm;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const int vi = tid + k * kBlock;
    if (vi < nvec) st16_stream(sp + vi * VEC, region[vi]);
  }
}

// Any K <= 8, dilation, S, q and alignment: one channel a lane, entries read
// and rolled in place in global memory.
template <class E, bool SILU>
__global__ __launch_bounds__(kBlock) void conv_spec_generic(ConvArgs a, int K, int D) {
  using St = typename E::S;
  const int lb = logical_block(a.n_logical, a.per_xcd);
  if (lb < 0) return;
  const int r = lb / a.n_cblk, cb = lb - r * a.n_cblk;
  if (r >= a.batch) return;
  const int c = cb * kBlock + (int)threadIdx.x;
  if (c >= a.C) return;
  const int H = (K - 1) * D, Sl = a.S;
  int q = a.q;
  int64_t start = (int64_t)r * q;
  if (a.qsl) {   // a draft count per request; a.q bounds them all
    start = a.qsl[r];
    q = a.qsl[r + 1] - a.qsl[r];
    if (q <= 0 || q > a.q || q > Sl || start < 0 || start + q > a.num_tokens) return;
  }
  float wt[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    wt[k] = k < K ? widen<E>(ld_el<E>((const St*)a.w + (int64_t)c * K + k)) : 0.f;
  const float b = a.bias ? widen<E>(ld_el<E>((const St*)a.bias + c)) : 0.f;
  const int32_t slot = a.slots[(int64_t)r * a.slot_stride];
  const bool valid = slot >= 0 && slot < a.num_slots;
  const int acc = min(max(a.num_acc[r], 1), min(q, Sl - H + 1));
  // state entry u of this channel (DS or SD pool)
  const int32_t vs = valid ? slot : 0;
  auto sref = [&](int u) -> St& {
    St* pool = (St*)a.pool;
    return a.sd ? pool[((int64_t)vs * Sl + u) * a.C + c] : pool[((int64_t)vs * a.C + c) * Sl + u];
  };
  // the request's token u in x / out (through the row map when one is given)
  auto pr = [&](int u) -> int64_t { return phys_row(a, start + u); };
  for (int t = 0; t < q; ++t) {
    float accf = b;
    for (int k = 0; k < K; ++k) {
      const int p = t - (K - 1 - k) * D;
      float v = 0.f;
      if (p >= 0) v = widen<E>(ld_el<E>((const St*)a.x + pr(p) * a.x_rs + c));
      else if (valid) v = widen<E>((uint32_t)sref(acc - 1 + H + p));
      accf = __builtin_fmaf(wt[k], v, accf);
    }
    if (SILU) accf = silu(accf);
    const int64_t ot = pr(t);
    if (a.accumulate) accf += widen<E>(ld_el<E>((const St*)a.out + ot * a.out_rs + c));
    if (a.outer) accf += widen<E>(ld_el<E>((const St*)a.outer + ot * a.outer_rs + c));
    ((St*)a.out)[ot * a.out_rs + c] = narrow<E>(accf);
  }
  if (valid) {
    for (int j = 0; j < Sl - q; ++j) sref(j) = sref(acc + j);
    for (int u = 0; u < q; ++u) sref(Sl - q + u) = *((const St*)a.x + pr(u) * a.x_rs + c);
  }
}

namespace {

bool rollbuf_shape(int K, int D) {
  return (K == 4 && (D == 1 || D == 2 || D == 3)) || (D == 1 && (K == 2 || K == 3));
}

template <class E, bool SILU, bool SPEC, bool FUSE>
hipError_t launch_rollbuf(const ConvArgs& a, int K, int D, dim3 grid, hipStream_t s) {
  const size_t lds = a.sd ? (size_t)kBlock * a.S * sizeof(u32x4)
                          : (size_t)kBlock * ds_lane_words(a.S, kBlock) * 4;
  const dim3 blk(kBlock);
  if constexpr (E::VEC == 8 && !FUSE) {
    // DS pool, width 4, no dilation: entries transposed in registers
    if (!a.sd && K == 4 && D == 1 && a.S >= 3 && a.S <= 10) {
      switch (a.S) {
        case 3: hipLaunchKernelGGL((conv_rollbuf_ds<3, SILU, SPEC>), grid, blk, 0, s, a); break;
        case 4: hipLaunchKernelGGL((conv_rollbuf_ds<4, SILU, SPEC>), grid, blk, 0, s, a); break;
        case 5: hipLaunchKernelGGL((conv_rollbuf_ds<5, SILU, SPEC>), grid, blk, 0, s, a); break;
        case 6: hipLaunchKernelGGL((conv_rollbuf_ds<6, SILU, SPEC>), grid, blk, 0, s, a); break;
        case 7: hipLaunchKernelGGL((conv_rollbuf_ds<7, SILU, SPEC>), grid, blk, 0, s, a); break;
        case 8: hipLaunchKernelGGL((conv_rollbuf_ds<8, SILU, SPEC>), grid, blk, 0, s, a); break;
        case 9: hipLaunchKernelGGL((conv_rollbuf_ds<9, SILU, SPEC>), grid, blk, 0, s, a); break;
        default: hipLaunchKernelGGL((conv_rollbuf_ds<10, SILU, SPEC>), grid, blk, 0, s, a); break;
      }
      return hipGetLastError();
    }
  }
  if (K == 4 && D == 1) hipLaunchKernelGGL((conv_rollbuf<E, 4, 1, SILU, SPEC, FUSE>), grid, blk, lds, s, a);
  else if (K == 4 && D == 2) hipLaunchKernelGGL((conv_rollbuf<E, 4, 2, SILU, SPEC, FUSE>), grid, blk, lds, s, a);
  else if (K == 4 && D == 3) hipLaunchKernelGGL((conv_rollbuf<E, 4, 3, SILU, SPEC, FUSE>), grid, blk, lds, s, a);
  else if (K == 3) hipLaunchKernelGGL((conv_rollbuf<E, 3, 1, SILU, SPEC, FUSE>), grid, blk, lds, s, a);
  else hipLaunchKernelGGL((conv_rollbuf<E, 2, 1, SILU, SPEC, FUSE>), grid, blk, lds, s, a);
  return hipGetLastError();
}

template <bool SPEC>
hipError_t launch_rollbuf_any(const ConvArgs& a, int dtype, int K, int D, bool silu_act,
                              dim3 grid, hipStream_t s) {
  const bool fuse = a.tok != nullptr || a.outer != nullptr || a.accumulate != 0;
  if (fuse) {
    if (dtype == 1)
      return silu_act ? launch_rollbuf<BF16, true, SPEC, true>(a, K, D, grid, s)
                      : launch_rollbuf<BF16, false, SPEC, true>(a, K, D, grid, s);
    return silu_act ? launch_rollbuf<F32, true, SPEC, true>(a, K, D, grid, s)
                    : launch_rollbuf<F32, false, SPEC, true>(a, K, D, grid, s);
  }
  if (dtype == 1)
    return silu_act ? launch_rollbuf<BF16, true, SPEC, false>(a, K, D, grid, s)
                    : launch_rollbuf<BF16, false, SPEC, false>(a, K, D, grid, s);
  return silu_act ? launch_rollbuf<F32, true, SPEC, false>(a, K, D, grid, s)
                  : launch_rollbuf<F32, false, SPEC, false>(a, K, D, grid, s);
}

bool use_rollbuf(const ConvArgs& a, int dtype, int K, int D, bool aligned16) {
  const int vec = dtype == 1 ? 8 : 4;
  const int es = dtype == 1 ? 2 : 4;
  return aligned16 && a.C % vec == 0 && rollbuf_shape(K, D) && a.q >= 1 && a.q <= kSpecQMax &&
         a.S >= (K - 1) * D && a.S <= kSpecSMax && (!a.outer || (a.outer_rs * es) % 16 == 0);
}

// One workgroup per (request, block of channels); fills the grid fields.
hipError_t set_grid(ConvArgs& a, int per_block_ch, dim3& grid) {
  a.n_cblk = (a.C + per_block_ch - 1) / per_block_ch;
  const int64_t n_logical = (int64_t)a.batch * a.n_cblk;
  if (n_logical > 0x7FFFFFF0LL) return hipErrorInvalidValue;
  a.n_logical = (int)n_logical;
  a.per_xcd = (int)((n_logical + kXcds - 1) / kXcds);
  grid = dim3((unsigned)(a.per_xcd * kXcds));
  return hipSuccess;
}

}  // namespace

hipError_t launch_conv_spec(ConvArgs a, int dtype, int K, int D, bool silu_act, bool aligned16,
                            hipStream_t stream) {
  dim3 grid;
  if (use_rollbuf(a, dtype, K, D, aligned16)) {
    const hipError_t e = set_grid(a, kBlock * (dtype == 1 ? 8 : 4), grid);
    if (e != hipSuccess) return e;
    return launch_rollbuf_any<true>(a, dtype, K, D, silu_act, grid, stream);
  }
  const hipError_t e = set_grid(a, kBlock, grid);
  if (e != hipSuccess) return e;
  if (dtype == 1) {
    if (silu_act) hipLaunchKernelGGL((conv_spec_generic<BF16, true>), grid, dim3(kBlock), 0, stream, a, K, D);
    else hipLaunchKernelGGL((conv_spec_generic<BF16, false>), grid, dim3(kBlock), 0, stream, a, K, D);
  } else {
    if (silu_act) hipLaunchKernelGGL((conv_spec_generic<F32, true>), grid, dim3(kBlock), 0, stream, a, K, D);
    else hipLaunchKernelGGL((conv_spec_generic<F32, false>), grid, dim3(kBlock), 0, stream, a, K, D);
  }
  return hipGetLastError();
}

hipError_t launch_update_wide(ConvArgs a, int dtype, int K, int D, bool silu_act, bool aligned16,
                              hipStream_t stream) {
  if (!use_rollbuf(a, dtype, K, D, aligned16)) return hipErrorNotSupported;
  dim3 grid;
  const hipError_t e = set_grid(a, kBlock * (dtype == 1 ? 8 : 4), grid);
  if (e != hipSuccess) return e;
  return launch_rollbuf_any<false>(a, dtype, K, D, silu_act, grid, stream);
}

}  // namespace sc
