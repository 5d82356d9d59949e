// Depthwise stateful causal conv1d kernels for gfx950 (varlen prefill and
// decode / multi-token update), with the state gather, the state write-back
// and the prefill checkpoint export fused into the same pass.
//
// Operation (GDN page "vllm.model_executor.layers.mamba.ops.cpu.gdn_attention",
// _spec_aware_nonspec; PLE page "vllm.models.qwen4_exp.nvidia.ple_layer",
// Qwen4ExpPLELayer): for each request, ext = [history (H = (K-1)*d raw inputs,
// oldest first, zeros without initial state), tokens]; out[t] = act(b +
// sum_k w[k] * ext[H + t - (K-1-k)*d]); the slot then holds the last H entries
// of ext; a checkpoint at offset p (multiple of the grid) receives ext[p..p+H).
//
// Layout: x / out token-major (rows of C channels, channel-contiguous), state
// pool (num_slots, C, H). A lane owns one 16-byte vector of channels (8 bf16 or
// 4 fp32), so a wave reads 1 KiB contiguous per token row. A workgroup (4 waves)
// covers 256 vectors of channels for one chunk of one request's tokens and keeps
// the causal window in registers while it walks the chunk: every input row is
// read once by the chunk plus an H-row halo from the previous chunk.
//
// State hazard: only the chunk holding a request's first tokens reads the
// request's slot (chunks are at least H long, so later chunks take their halo
// from x), and the same lanes write the new state after reading the old one.
#include <atomic>

#include "conv_device.hpp"

namespace sc {


// State I/O in "rows": rows[u] is entry u (oldest first) of the lane's VEC
// channels. In the SD pool (num_slots, S, C) a row is one 16-byte vector
// (coalesced across lanes); in the DS pool (num_slots, C, S) with S == H the
// lane's entries are H contiguous vectors in (channel, entry) order and are
// transposed in registers.
template <class E, int H, bool SD>
__device__ __forceinline__ void load_state_rows(const ConvArgs& a, int32_t slot, int c0,
                                                u32x4* rows) {
  using S = typename E::S;
  if constexpr (SD) {
    const S* base = (const S*)a.pool + (int64_t)slot * a.S * a.C + c0;
#pragma unroll
    for (int u = 0; u < H; ++u) rows[u] = ld16(base + (int64_t)u * a.C);
  } else {
    const S* sp = (const S*)a.pool + ((int64_t)slot * a.C + c0) * H;
    u32x4 old[H];
#pragma unroll
    for (int v = 0; v < H; ++v) old[v] = ld16(sp + v * E::VEC);
#pragma unroll
    for (int u = 0; u < H; ++u) {
      rows[u] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int ch = 0; ch < E::VEC; ++ch) E::set(rows[u], ch, get_flat<E>(old, ch * H + u));
    }
  }
}

template <class E, int H, bool SD>
__device__ __forceinline__ void store_state_rows(const ConvArgs& a, int32_t slot, int c0,
                                                 const u32x4* rows) {
  using S = typename E::S;
  if constexpr (SD) {
    S* base = (S*)a.pool + (int64_t)slot * a.S * a.C + c0;
#pragma unroll
    for (int u = 0; u < H; ++u) st16(base + (int64_t)u * a.C, rows[u]);
  } else {
    S* sp = (S*)a.pool + ((int64_t)slot * a.C + c0) * H;
    u32x4 nv[H];
#pragma unroll
    for (int u = 0; u < H; ++u)
#pragma unroll
      for (int ch = 0; ch < E::VEC; ++ch) set_flat<E>(nv, ch * H + u, E::get(rows[u], ch));
#pragma unroll
    for (int v = 0; v < H; ++v) st16(sp + v * E::VEC, nv[v]);
  }
}

// Store the window of request rows [p-H, p) (all >= 0) into `slot`; xrow(t) is
// the lane's channel vector in the request's row t.
template <class E, int H, bool SD, class XRow>
__device__ __forceinline__ void store_window_rows(const ConvArgs& a, int32_t slot, int c0,
                                                  XRow xrow, int p) {
  u32x4 r[H];
#pragma unroll
  for (int jj = 0; jj < H; ++jj) r[jj] = ld16(xrow(p - H + jj));
  store_state_rows<E, H, SD>(a, slot, c0, r);
}

// New state = ext[L .. L+H) for a request of runtime length L >= 1, where ext
// is [old rows (H), x rows].
template <class E, int H, bool SD, class XRow>
__device__ __forceinline__ void write_state_rows(const ConvArgs& a, int32_t slot, int c0,
                                                 const u32x4* old, int L, XRow xrow) {
  if (L >= H) {
    store_window_rows<E, H, SD>(a, slot, c0, xrow, L);
    return;
  }
  // 1 <= L < H: entries jj < H-L keep old[L + jj], the rest are the L tokens
  u32x4 r[H];
#pragma unroll
  for (int jj = 0; jj < H; ++jj) {
    const int p = L - H + jj;
    u32x4 val = p >= 0 ? ld16(xrow(p)) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int m = 1; m < H; ++m)
      if (m + jj < H && m == L) val = old[m + jj];
    r[jj] = val;
  }
  store_state_rows<E, H, SD>(a, slot, c0, r);
}

// ---------------------------------------------------------------------------
// fast kernel: compile-time K, D; QC > 0 is a compile-time update length
// ---------------------------------------------------------------------------
template <class E, int K, int D, int U, bool SILU, int QC, bool SD>
__global__ __launch_bounds__(kBlock) void conv_fast(ConvArgs a) {
  constexpr int H = (K - 1) * D;
  constexpr int VEC = E::VEC;
  using S = typename E::S;
  static_assert(K >= 2, "K = 1 has no history; use the generic kernel");

  const int lb = logical_block(a.n_logical, a.per_xcd);
  if (lb < 0) return;
  const int cid = lb / a.n_cblk, cb = lb - cid * a.n_cblk;
  Work w;
  if (!resolve_work(a, cid, w)) return;
  const int c0 = (cb * kBlock + (int)threadIdx.x) * VEC;
  if (c0 >= a.C) return;

  float wt[K][VEC], bs[VEC];
  load_weights<E, K>(a.w, c0, wt);
  if (a.bias) {
    E::unpack(ld16((const S*)a.bias + c0), bs);
  } else {
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) bs[ch] = 0.f;
  }

  const int64_t xrs = a.x_rs, ors = a.out_rs;
  const S* xb = (const S*)a.x + w.start * xrs + c0;
  S* ob = (S*)a.out + w.start * ors + c0;
  u32x4 old[H];   // history rows (entry u of this lane's channels)
#pragma unroll
  for (int v = 0; v < H; ++v) old[v] = u32x4{0, 0, 0, 0};
  if (w.j == 0 && w.h) load_state_rows<E, H, SD>(a, w.slot, c0, old);

  if constexpr (QC > 0) {
    // Update of exactly QC tokens (the host launches this only when q == QC).
    u32x4 xr[QC];
#pragma unroll
    for (int u = 0; u < QC; ++u) xr[u] = ld16(xb + (int64_t)u * xrs);
    float win[H + QC][VEC];
#pragma unroll
    for (int u = 0; u < H; ++u) E::unpack(old[u], win[u]);
#pragma unroll
    for (int u = 0; u < QC; ++u) E::unpack(xr[u], win[H + u]);
#pragma unroll
    for (int u = 0; u < QC; ++u) {
      float z[VEC];
      conv_point<E, K, D, SILU>(win, H + u, wt, bs, z);
      st16_stream(ob + (int64_t)u * ors, E::pack(z));
    }
    if (w.valid) {
      u32x4 nr[H];
#pragma unroll
      for (int jj = 0; jj < H; ++jj) {
        const int e = QC + jj;   // ext index of new-state entry jj
        nr[jj] = e < H ? old[e] : xr[e - H];
      }
      store_state_rows<E, H, SD>(a, w.slot, c0, nr);
    }
  } else {
    float win[H + U][VEC];
    if (w.j == 0) {
#pragma unroll
      for (int u = 0; u < H; ++u) E::unpack(old[u], win[u]);
    } else {
#pragma unroll
      for (int u = 0; u < H; ++u) E::unpack(ld16(xb + (int64_t)(w.t0 - H + u) * xrs), win[u]);
    }
    for (int tb = w.t0; tb < w.t1; tb += U) {
      u32x4 xr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = min(tb + u, w.t1 - 1);
        xr[u] = ld16_stream(xb + (int64_t)t * xrs);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) E::unpack(xr[u], win[H + u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (tb + u < w.t1) {
          float z[VEC];
          conv_point<E, K, D, SILU>(win, H + u, wt, bs, z);
          st16_stream(ob + (int64_t)(tb + u) * ors, E::pack(z));
        }
      }
#pragma unroll
      for (int i = 0; i < H; ++i)
#pragma unroll
        for (int ch = 0; ch < VEC; ++ch) win[i][ch] = win[i + U][ch];
    }
    auto xrow = [&](int t) { return xb + (int64_t)t * xrs; };
    if (w.j == 0 && w.valid) write_state_rows<E, H, SD>(a, w.slot, c0, old, w.L, xrow);
    if (a.ckpt_grid > 0 && a.qsl != nullptr) {
      // checkpoints at p = m*g with t0 < p <= t1: the chunk holding token p-1
      const int g = a.ckpt_grid;
      const int cu0 = a.cu_ckpt[w.r], cnt = a.cu_ckpt[w.r + 1] - cu0;
      for (int m = w.t0 / g + 1; m <= cnt && (int64_t)m * g <= w.t1; ++m) {
        const int32_t dst = a.ckpt_slots[cu0 + m - 1];
        if (dst < 0 || dst >= a.num_slots) continue;
        store_window_rows<E, H, SD>(a, dst, c0, xrow, m * g);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 one-pass kernel for an even number of taps: a workgroup handles one
// chunk of at most U tokens in one pass (all rows issued up front), and taps
// are consumed in pairs by v_dot2c_f32_bf16 straight from bf16 data: the pair
// (x[s-D][c], x[s][c]) is built from two token rows with one v_perm_b32 and
// reused by every output that needs it. UPDATE: requests of exactly U tokens.
// ---------------------------------------------------------------------------

template <int K, int D, int U, bool SILU, bool UPDATE, bool FUSE, bool SD>
__global__ __launch_bounds__(kBlock) void conv_pairs(ConvArgs a) {
  using E = BF16;
  using S = E::S;
  constexpr int H = (K - 1) * D;
  constexpr int NP = K / 2;
  constexpr int VEC = 8;
  static_assert(K % 2 == 0 && K >= 2, "pairs of taps");
  static_assert(U >= H, "the chunk must cover the history (halo from x only)");

  const int lb = logical_block(a.n_logical, a.per_xcd);
  if (lb < 0) return;
  const int cid = lb / a.n_cblk, cb = lb - cid * a.n_cblk;
  const int c0 = (cb * kBlock + (int)threadIdx.x) * VEC;
  const bool lane_ok = c0 < a.C;

  // chunk -> request (one round of loads below 64 requests, three from 64 on:
  // two for the request, one for its bounds), bounds and chunk range
  // (the launcher sets a.chunk = U for this kernel; U as a constant turns the
  // divisions below into multiplies)
  int r, s0 = 0, s1 = 0;
  if (UPDATE || a.qsl == nullptr) {
    const int cpr = (a.q + U - 1) / U;
    r = cid / cpr;
    s0 = r * a.q;
    s1 = s0 + a.q;
  } else {
    r = find_request_bounds(a.qsl, a.batch, cid, U, s0, s1);
  }
  if (r >= a.batch || s0 < 0) return;
  const int j = (UPDATE || a.qsl == nullptr) ? cid - r * ((a.q + U - 1) / U) : cid - (s0 / U + r);
  int L = s1 - s0;
  if (j < 0 || L <= 0 || s0 >= a.num_tokens) return;
  if ((int64_t)s0 + L > a.num_tokens) L = (int)(a.num_tokens - s0);
  const int t0 = j * U;
  if (t0 >= L || !lane_ok) return;
  const int t1 = min(L, t0 + U);

  // Loads in the order they are consumed (vmcnt retires in issue order).
  // The weights go out after the request lookup: ahead of it, the wait for
  // the lookup's own load would cover them too, and a workgroup whose chunk
  // id holds no rows would load them for nothing.
  uint32_t wp[NP][VEC];
  u32x4 bsv = u32x4{0, 0, 0, 0};
  {
    u32x4 wv[NP * 2];
#pragma unroll
    for (int v = 0; v < NP * 2; ++v)
      wv[v] = lane_ok ? ld16((const S*)a.w + (int64_t)c0 * K + v * VEC) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int word = ch * NP + p;
        wp[p][ch] = wv[word >> 2][word & 3];
      }
    if (a.bias && lane_ok) bsv = ld16((const S*)a.bias + c0);
  }

  const int64_t xrs = a.x_rs, ors = a.out_rs;
  const S* xb = (const S*)a.x + (int64_t)s0 * xrs + c0;
  S* ob = (S*)a.out + (int64_t)s0 * ors + c0;
  // request row t of x / out (through the row map when fused)
  auto xrow = [&](int t) -> const S* {
    if constexpr (FUSE) return (const S*)a.x + phys_row(a, (int64_t)s0 + t) * xrs + c0;
    else return xb + (int64_t)t * xrs;
  };

  // the slot is needed by the request's first chunk only (history and
  // write-back); its scalar load goes out before the rows so that the state
  // loads, which wait on it, start while the rows are in flight; the
  // has-state flag is read after them and applied to the loaded history
  int32_t slot = -1;
  bool valid = false, hflag = false;
  if (j == 0) {
    slot = a.slots[(int64_t)r * a.slot_stride];
    valid = slot >= 0 && slot < a.num_slots;
  }
  u32x4 raw[H + U];
  if (j > 0) {
#pragma unroll
    for (int u = 0; u < H; ++u) raw[u] = ld16(xrow(t0 - H + u));
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = UPDATE ? u : min(t0 + u, t1 - 1);
    raw[H + u] = ld16_stream(xrow(t));
  }
  u32x4 old[H];
#pragma unroll
  for (int v = 0; v < H; ++v) old[v] = u32x4{0, 0, 0, 0};
  if (valid) load_state_rows<E, H, SD>(a, slot, c0, old);   // history rows
  if (valid) {
    hflag = a.has_init ? uniform_flag(a.has_init, r) : true;
    if (!hflag) {
#pragma unroll
      for (int v = 0; v < H; ++v) old[v] = u32x4{0, 0, 0, 0};
    }
  }
  Work w;
  w.r = r;
  w.j = j;
  w.L = L;
  w.t0 = t0;
  w.t1 = t1;
  w.start = s0;
  w.slot = slot;
  w.valid = valid;
  w.h = hflag;
  // fused residuals, FG rows at a time, one group ahead of the rows computed
  // (all U rows at once would hold 2*U vectors; physical rows are distinct,
  // so a row's residual is read before that row is written)
  constexpr int FG = FUSE ? (U < 4 ? U : 4) : 1;
  static_assert(!FUSE || U % FG == 0, "whole residual groups");
  u32x4 rres[2][FG], rout[2][FG];
  auto load_res = [&](int g) {
#pragma unroll
    for (int k = 0; k < FG; ++k) {
      const int u = g * FG + k;
      const int t = UPDATE ? u : min(t0 + u, t1 - 1);
      const int64_t pr = phys_row(a, (int64_t)s0 + t);
      rres[g & 1][k] = a.accumulate ? ld16((const S*)a.out + pr * ors + c0) : u32x4{0, 0, 0, 0};
      rout[g & 1][k] = a.outer ? ld16((const S*)a.outer + pr * a.outer_rs + c0) : u32x4{0, 0, 0, 0};
    }
  };
  if constexpr (FUSE) load_res(0);
  float bs[VEC];
  E::unpack(bsv, bs);
  if (w.j == 0) {
#pragma unroll
    for (int u = 0; u < H; ++u) raw[u] = old[u];
  }

#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (FUSE) {
      if (u % FG == 0 && u + FG < U) load_res(u / FG + 1);
    }
    if (UPDATE || w.t0 + u < w.t1) {
      float z[VEC];
#pragma unroll
      for (int ch = 0; ch < VEC; ++ch) {
        float acc = bs[ch];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          // taps 2p and 2p+1 sit at rows H+u-(K-1-2p)*D and D later
          const int r0 = H + u - (K - 1 - 2 * p) * D;
          acc = dot2_bf16(wp[p][ch], row_pair(raw[r0], raw[r0 + D], ch), acc);
        }
        z[ch] = SILU ? silu(acc) : acc;
      }
      if constexpr (FUSE) {
        const int64_t pr = phys_row(a, (int64_t)s0 + w.t0 + u);
        float rr[VEC], ro[VEC];
        E::unpack(rres[(u / FG) & 1][u % FG], rr);
        E::unpack(rout[(u / FG) & 1][u % FG], ro);
#pragma unroll
        for (int ch = 0; ch < VEC; ++ch) {
          if (a.accumulate) z[ch] += rr[ch];
          if (a.outer) z[ch] += ro[ch];
        }
        st16_stream((S*)a.out + pr * ors + c0, E::pack(z));
      } else {
        st16_stream(ob + (int64_t)(w.t0 + u) * ors, E::pack(z));
      }
    }
  }

  if (w.j == 0 && w.valid) {
    if constexpr (UPDATE) {
      store_state_rows<E, H, SD>(a, slot, c0, raw + U);   // new state = ext[U .. U+H)
    } else {
      write_state_rows<E, H, SD>(a, slot, c0, old, w.L, xrow);
    }
  }
  if (!UPDATE && a.ckpt_grid > 0 && a.qsl != nullptr) {
    const int g = a.ckpt_grid;
    const int cu0 = a.cu_ckpt[w.r], cnt = a.cu_ckpt[w.r + 1] - cu0;
    for (int m = w.t0 / g + 1; m <= cnt && (int64_t)m * g <= w.t1; ++m) {
      const int32_t dst = a.ckpt_slots[cu0 + m - 1];
      if (dst < 0 || dst >= a.num_slots) continue;
      store_window_rows<E, H, SD>(a, dst, c0, xrow, m * g);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 decode / multi-token update (requests of exactly Q tokens), R requests
// per workgroup. The state rows of a workgroup's channels are contiguous in the
// (slot, C, H) pool; they are loaded and stored with unit-stride lanes and
// transposed to and from the per-lane (channel, tap) order through LDS. The
// weights are loaded once for the R requests. Same tap pairing and dot2 order
// as conv_pairs, so a decode step equals the matching prefill token bit for bit.
// ---------------------------------------------------------------------------
// Requests of a DS update workgroup transposed through LDS together: the
// largest divisor of R whose state regions fit in 48 KiB.
constexpr int ds_batch(int R, int H) {
  int b = R;
  while (b > 1 && (R % b != 0 || b * H * kBlock * 16 > 49152)) --b;
  return b;
}

template <int K, int D, int Q, int R, bool SILU, bool FUSE, bool SD>
__global__ __launch_bounds__(kBlock) void conv_update_pairs(ConvArgs a) {
  using E = BF16;
  using S = E::S;
  constexpr int H = (K - 1) * D;
  constexpr int NP = K / 2;
  constexpr int VEC = 8;
  // DS pool: requests whose state regions are transposed through LDS together
  // (at most 48 KiB of LDS), so the workgroup passes 4 barriers per batch
  constexpr int RB = SD ? 1 : ds_batch(R, H);
  static_assert(R % RB == 0, "whole batches");
  __shared__ u32x4 xch[RB * H * kBlock];

  const int lb = logical_block(a.n_logical, a.per_xcd);
  if (lb < 0) return;                       // uniform over the workgroup
  const int grp = lb / a.n_cblk, cb = lb - grp * a.n_cblk;
  const int tid = (int)threadIdx.x;
  const int cbase = cb * kBlock * VEC;      // first channel of the workgroup
  const int c0 = cbase + tid * VEC;
  const bool lane_ok = c0 < a.C;
  // vectors of the workgroup's state region that exist (partial last block)
  const int nvec = (min(a.C - cbase, kBlock * VEC) / VEC) * H;

  uint32_t wp[NP][VEC];
  u32x4 bsv = u32x4{0, 0, 0, 0};
  if (lane_ok) {
    u32x4 wv[NP * 2];
#pragma unroll
    for (int v = 0; v < NP * 2; ++v) wv[v] = ld16((const S*)a.w + (int64_t)c0 * K + v * VEC);
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int word = ch * NP + p;
        wp[p][ch] = wv[word >> 2][word & 3];
      }
    if (a.bias) bsv = ld16((const S*)a.bias + c0);
  }

  // issue every request's loads: the token rows (independent of the slot),
  // the slot indices and has-state flags (workgroup-uniform scalar loads),
  // then the state (unit stride over the region), which waits on the slots
  // only. With one request per workgroup the slot load goes out before the
  // token rows (6.78 vs 6.90 us on the 128 x 4 update); with several, after
  // them (12.53 vs 12.82 us on the 512-request decode, the state loads then
  // start a few scalar round trips after the rows).
  int32_t slot[R];
  bool valid[R], hflag[R];
  u32x4 st[R][H], xr[R][Q];
  auto load_slots = [&]() {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int r = grp * R + rr;
      slot[rr] = r < a.batch ? a.slots[(int64_t)r * a.slot_stride] : -1;
      valid[rr] = slot[rr] >= 0 && slot[rr] < a.num_slots;
      hflag[rr] = valid[rr] && (a.has_init ? uniform_flag(a.has_init, r) : true);
    }
  };
  if constexpr (R == 1) load_slots();
  // physical row of request r's token u (through the row map when fused)
  auto prow = [&](int r, int u) -> int64_t {
    if constexpr (FUSE) return phys_row(a, (int64_t)r * Q + u);
    else return (int64_t)r * Q + u;
  };
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int r = grp * R + rr;
#pragma unroll
    for (int u = 0; u < Q; ++u)
      xr[rr][u] = (r < a.batch && lane_ok)
                      ? ld16_stream((const S*)a.x + prow(r, u) * a.x_rs + c0)
                      : u32x4{0, 0, 0, 0};
  }
  // fused residuals, issued with the token rows
  u32x4 rres[FUSE ? R : 1][FUSE ? Q : 1], rout[FUSE ? R : 1][FUSE ? Q : 1];
  if constexpr (FUSE) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int r = grp * R + rr;
#pragma unroll
      for (int u = 0; u < Q; ++u) {
        const bool ok = r < a.batch && lane_ok;
        rres[rr][u] = (ok && a.accumulate) ? ld16((const S*)a.out + prow(r, u) * a.out_rs + c0)
                                           : u32x4{0, 0, 0, 0};
        rout[rr][u] = (ok && a.outer) ? ld16((const S*)a.outer + prow(r, u) * a.outer_rs + c0)
                                      : u32x4{0, 0, 0, 0};
      }
    }
  }
  if constexpr (R > 1) load_slots();
  if constexpr (SD) {
    // SD pool: entry k of the lane's channels is one vector, unit stride across lanes
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const S* sp = (const S*)a.pool + (int64_t)(valid[rr] ? slot[rr] : 0) * a.S * a.C + c0;
#pragma unroll
      for (int k = 0; k < H; ++k)
        st[rr][k] = (hflag[rr] && lane_ok) ? ld16_stream(sp + (int64_t)k * a.C) : u32x4{0, 0, 0, 0};
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const S* sp = (const S*)a.pool + ((int64_t)(valid[rr] ? slot[rr] : 0) * a.C + cbase) * H;
#pragma unroll
      for (int k = 0; k < H; ++k) {
        const int vi = tid + k * kBlock;
        st[rr][k] = (hflag[rr] && vi < nvec) ? ld16_stream(sp + vi * VEC) : u32x4{0, 0, 0, 0};
      }
    }
  }
  float bs[VEC];
  E::unpack(bsv, bs);

#pragma unroll
  for (int rb = 0; rb < R; rb += RB) {
    if constexpr (!SD) {
      // the batch's state regions -> per-lane (channel, tap) order
      __syncthreads();
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int k = 0; k < H; ++k) xch[j * H * kBlock + tid + k * kBlock] = st[rb + j][k];
      __syncthreads();
    }
    u32x4 nvb[RB][SD ? 1 : H];   // new state of the batch, (channel, tap) order
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int rr = rb + j;
      const int r = grp * R + rr;
      u32x4 raw[H + Q];
      if constexpr (SD) {
#pragma unroll
        for (int u = 0; u < H; ++u) raw[u] = st[rr][u];
      } else {
        u32x4 old[H];
#pragma unroll
        for (int k = 0; k < H; ++k) old[k] = xch[j * H * kBlock + tid * H + k];
#pragma unroll
        for (int u = 0; u < H; ++u) {
          raw[u] = u32x4{0, 0, 0, 0};
#pragma unroll
          for (int ch = 0; ch < VEC; ++ch) E::set(raw[u], ch, get_flat<E>(old, ch * H + u));
        }
      }
#pragma unroll
      for (int u = 0; u < Q; ++u) raw[H + u] = xr[rr][u];
      if (r < a.batch && lane_ok) {
#pragma unroll
        for (int u = 0; u < Q; ++u) {
          float z[VEC];
#pragma unroll
          for (int ch = 0; ch < VEC; ++ch) {
            float acc = bs[ch];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const int r0 = H + u - (K - 1 - 2 * p) * D;
              acc = dot2_bf16(wp[p][ch], row_pair(raw[r0], raw[r0 + D], ch), acc);
            }
            z[ch] = SILU ? silu(acc) : acc;
          }
          const int64_t pr = prow(r, u);
          if constexpr (FUSE) {
            float fr[VEC], fo[VEC];
            E::unpack(rres[rr][u], fr);
            E::unpack(rout[rr][u], fo);
#pragma unroll
            for (int ch = 0; ch < VEC; ++ch) {
              if (a.accumulate) z[ch] += fr[ch];
              if (a.outer) z[ch] += fo[ch];
            }
          }
          st16_stream((S*)a.out + pr * a.out_rs + c0, E::pack(z));
        }
      }
      // new state = ext[Q .. Q+H)
      if constexpr (SD) {
        if (valid[rr] && lane_ok) {
          S* dp = (S*)a.pool + (int64_t)slot[rr] * a.S * a.C + c0;
#pragma unroll
          for (int k = 0; k < H; ++k) st16_stream(dp + (int64_t)k * a.C, raw[Q + k]);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < H; ++jj)
#pragma unroll
          for (int ch = 0; ch < VEC; ++ch) set_flat<E>(nvb[j], ch * H + jj, E::get(raw[Q + jj], ch));
      }
    }
    if constexpr (!SD) {
      // (channel, tap) order -> region order, then unit-stride stores
      __syncthreads();
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int k = 0; k < H; ++k) xch[j * H * kBlock + tid * H + k] = nvb[j][k];
      __syncthreads();
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const int rr = rb + j;
        if (valid[rr]) {
          S* dp = (S*)a.pool + ((int64_t)slot[rr] * a.C + cbase) * H;
#pragma unroll
          for (int k = 0; k < H; ++k) {
            const int vi = tid + k * kBlock;
            if (vi < nvec) st16_stream(dp + vi * VEC, xch[j * H * kBlock + vi]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// generic kernel: any K <= 8, any dilation, any alignment, state rows of any
// length S >= H (window in the first H entries); one channel a lane, each tap
// read through the cache
// ---------------------------------------------------------------------------

template <class E, bool SILU>
__global__ __launch_bounds__(kBlock) void conv_generic(ConvArgs a, int K, int D) {
  using S = typename E::S;
  const int lb = logical_block(a.n_logical, a.per_xcd);
  if (lb < 0) return;
  const int cid = lb / a.n_cblk, cb = lb - cid * a.n_cblk;
  Work w;
  if (!resolve_work(a, cid, w)) return;
  const int c = cb * kBlock + (int)threadIdx.x;
  if (c >= a.C) return;
  const int H = (K - 1) * D;
  float wt[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    wt[k] = k < K ? widen<E>(ld_el<E>((const S*)a.w + (int64_t)c * K + k)) : 0.f;
  const float b = a.bias ? widen<E>(ld_el<E>((const S*)a.bias + c)) : 0.f;
  const int64_t xrs = a.x_rs, ors = a.out_rs;
  const S* xb = (const S*)a.x + w.start * xrs + c;
  // state entry u of this channel in slot s (DS or SD pool)
  auto sref = [&](int32_t s, int u) -> S& {
    S* pool = (S*)a.pool;
    return a.sd ? pool[((int64_t)s * a.S + u) * a.C + c] : pool[((int64_t)s * a.C + c) * a.S + u];
  };
  const int32_t wslot = w.valid ? w.slot : 0;
  // request row p of x (through the row map when one is given)
  auto xg = [&](int p) -> const S* {
    return a.tok ? (const S*)a.x + phys_row(a, w.start + p) * xrs + c : xb + (int64_t)p * xrs;
  };
  for (int t = w.t0; t < w.t1; ++t) {
    float acc = b;
    for (int k = 0; k < K; ++k) {
      const int p = t - (K - 1 - k) * D;
      float v = 0.f;
      if (p >= 0) v = widen<E>(ld_el<E>(xg(p)));
      else if (w.h) v = widen<E>((uint32_t)sref(wslot, H + p));
      acc = __builtin_fmaf(wt[k], v, acc);
    }
    if (SILU) acc = silu(acc);
    const int64_t pr = a.tok ? phys_row(a, w.start + t) : w.start + t;
    if (a.accumulate) acc += widen<E>(ld_el<E>((const S*)a.out + pr * ors + c));
    if (a.outer) acc += widen<E>(ld_el<E>((const S*)a.outer + pr * a.outer_rs + c));
    ((S*)a.out)[pr * ors + c] = narrow<E>(acc);
  }
  if (w.j == 0 && w.valid) {
    // ascending jj reads old entry L + jj > jj before it is overwritten
    for (int jj = 0; jj < H; ++jj) {
      const int p = w.L - H + jj;
      S v = 0;
      if (p >= 0) v = *xg(p);
      else if (w.h) v = sref(wslot, w.L + jj);
      sref(wslot, jj) = v;
    }
  }
  if (a.ckpt_grid > 0 && a.qsl != nullptr) {
    const int g = a.ckpt_grid;
    const int cu0 = a.cu_ckpt[w.r], cnt = a.cu_ckpt[w.r + 1] - cu0;
    for (int m = w.t0 / g + 1; m <= cnt && (int64_t)m * g <= w.t1; ++m) {
      const int32_t dst = a.ckpt_slots[cu0 + m - 1];
      if (dst < 0 || dst >= a.num_slots) continue;
      for (int jj = 0; jj < H; ++jj) sref(dst, jj) = *xg(m * g - H + jj);
    }
  }
}

// ---------------------------------------------------------------------------
// host-side launch selection
// ---------------------------------------------------------------------------
// Each per-device slot is an atomic that every racing writer sets to the same
// value.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

bool fast_shape(int K, int D) {
  return (K == 4 && (D == 1 || D == 2 || D == 3)) || (D == 1 && (K == 2 || K == 3));
}
bool pairs_shape(int K, int D) {
  return (K == 4 && (D == 1 || D == 2 || D == 3)) || (K == 2 && D == 1);
}

template <class E, int K, int D, bool SILU, bool SD>
hipError_t launch_kd_l(const ConvArgs& a, int qc, dim3 grid, hipStream_t s) {
  constexpr int U = kUnroll;
  switch (qc) {
    case 1: hipLaunchKernelGGL((conv_fast<E, K, D, U, SILU, 1, SD>), grid, dim3(kBlock), 0, s, a); break;
    case 2: hipLaunchKernelGGL((conv_fast<E, K, D, U, SILU, 2, SD>), grid, dim3(kBlock), 0, s, a); break;
    case 4: hipLaunchKernelGGL((conv_fast<E, K, D, U, SILU, 4, SD>), grid, dim3(kBlock), 0, s, a); break;
    default: hipLaunchKernelGGL((conv_fast<E, K, D, U, SILU, 0, SD>), grid, dim3(kBlock), 0, s, a); break;
  }
  return hipGetLastError();
}

template <class E, int K, int D, bool SILU>
hipError_t launch_kd(const ConvArgs& a, int qc, dim3 grid, hipStream_t s) {
  return a.sd ? launch_kd_l<E, K, D, SILU, true>(a, qc, grid, s)
              : launch_kd_l<E, K, D, SILU, false>(a, qc, grid, s);
}

// tokens per one-pass prefill chunk for history length H (must be >= H).
// `small` launches (tokens x channels at most kSmallLaunch) are bound by
// their ramp and drain, where shorter chunks finish sooner; larger ones by
// bandwidth, where longer chunks re-read fewer halo rows. Measured at 8192
// channels: 8 tokens won by 7.8 / 2.5 / 1.1% at 2.6k / 5.3k / 7.4k tokens, 12
// by 1.8 / 3.6 / 6.8% at 9.1k / 11.8k / 15.3k tokens (DS pool); with the
// weights loaded after the request lookup, the same rule holds on an SD pool
// (8 faster by 8% at 2.6k and 3% at 7.4k tokens, 12 by 2–6% at 15k–33k).
constexpr int64_t kSmallLaunch = int64_t(1) << 26;
constexpr int pairs_chunk(int H, bool small) {
  return H <= 4 ? (small ? 8 : kPairsChunkLarge) : (H <= 8 ? 8 : 16);
}
// requests per update workgroup
constexpr int update_reqs(int H, int Q, bool sd) {
  if (H <= 4) return Q == 1 ? (sd ? kUpdateReqsSD : kUpdateReqsDS) : kUpdateReqsMulti;
  return Q == 1 ? 2 : 1;
}


// Requests per one-token update workgroup (H <= 4) by batch size: each
// workgroup is a single round of loads, so the launch should fill the device
// once without splitting it thinner than that. A DS pool (state transposed
// through LDS) is fastest at two workgroups per CU, an SD pool at one; so take
// the largest R in {1, 2, 4, 8} whose workgroup count still reaches that
// target. On a DS pool, when even R = 8 needs more than one round, 4 (two
// LDS batches fewer) measured faster. Measured optimum at 8192 channels on
// 256 CUs: DS R = 1, 1, 2, 4, 8, 4 and SD R = 1, 2, 4, 8, 8, 8 for 64, 128,
// 256, 512, 1024, 2048 requests.
// Longer histories (H > 4) take at most 2 requests per workgroup: for the
// 9-entry PLE history on a DS pool, R = 1, 2, 2~1 were fastest at 64, 256,
// 1024 requests, and R = 4 never was.
int update_reqs_rt(int H, bool sd, int64_t batch, int n_cblk) {
  const int64_t target = (int64_t)device_cus() * (sd ? 1 : 2);
  auto wgs = [&](int R) { return (batch + R - 1) / R * n_cblk; };
  if (H > 4) return wgs(2) >= target ? 2 : 1;
  if (!sd && wgs(8) > target) return 4;
  int R = 8;
  while (R > 1 && wgs(R) < target) R >>= 1;
  return R;
}

template <int K, int D, bool SILU, bool FUSE, bool SD>
hipError_t launch_update1(const ConvArgs& a, dim3 grid, hipStream_t s) {
  constexpr int H = (K - 1) * D;
  if constexpr (H > 4) {
    if (a.ureqs == 1)
      hipLaunchKernelGGL((conv_update_pairs<K, D, 1, 1, SILU, FUSE, SD>), grid, dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL((conv_update_pairs<K, D, 1, 2, SILU, FUSE, SD>), grid, dim3(kBlock), 0, s, a);
  } else {
    switch (a.ureqs) {
      case 1: hipLaunchKernelGGL((conv_update_pairs<K, D, 1, 1, SILU, FUSE, SD>), grid, dim3(kBlock), 0, s, a); break;
      case 2: hipLaunchKernelGGL((conv_update_pairs<K, D, 1, 2, SILU, FUSE, SD>), grid, dim3(kBlock), 0, s, a); break;
      case 4: hipLaunchKernelGGL((conv_update_pairs<K, D, 1, 4, SILU, FUSE, SD>), grid, dim3(kBlock), 0, s, a); break;
      default: hipLaunchKernelGGL((conv_update_pairs<K, D, 1, 8, SILU, FUSE, SD>), grid, dim3(kBlock), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

template <int K, int D, bool SILU, bool FUSE, bool SD>
hipError_t launch_pairs_l(const ConvArgs& a, int qc, dim3 grid, hipStream_t s) {
  constexpr int H = (K - 1) * D;
  if (qc == 0 && a.chunk == pairs_chunk(H, true) && pairs_chunk(H, true) != pairs_chunk(H, false)) {
    hipLaunchKernelGGL((conv_pairs<K, D, pairs_chunk(H, true), SILU, false, FUSE, SD>), grid, dim3(kBlock),
                       kPairsResidencyLds, s, a);
    return hipGetLastError();
  }
  switch (qc) {
    case 1: return launch_update1<K, D, SILU, FUSE, SD>(a, grid, s);
    case 2: hipLaunchKernelGGL((conv_update_pairs<K, D, 2, update_reqs(H, 2, SD), SILU, FUSE, SD>), grid, dim3(kBlock), 0, s, a); break;
    case 4: hipLaunchKernelGGL((conv_update_pairs<K, D, 4, update_reqs(H, 4, SD), SILU, FUSE, SD>), grid, dim3(kBlock), 0, s, a); break;
    default:
      hipLaunchKernelGGL((conv_pairs<K, D, pairs_chunk(H, false), SILU, false, FUSE, SD>), grid,
                         dim3(kBlock), kPairsResidencyLds, s, a);
      break;
  }
  return hipGetLastError();
}

template <int K, int D, bool SILU, bool FUSE>
hipError_t launch_pairs_kd(const ConvArgs& a, int qc, dim3 grid, hipStream_t s) {
  return a.sd ? launch_pairs_l<K, D, SILU, FUSE, true>(a, qc, grid, s)
              : launch_pairs_l<K, D, SILU, FUSE, false>(a, qc, grid, s);
}

template <bool SILU, bool FUSE>
hipError_t launch_pairs(const ConvArgs& a, int K, int D, int qc, dim3 grid, hipStream_t s) {
  if (K == 4 && D == 1) return launch_pairs_kd<4, 1, SILU, FUSE>(a, qc, grid, s);
  if (K == 4 && D == 2) return launch_pairs_kd<4, 2, SILU, FUSE>(a, qc, grid, s);
  if (K == 4 && D == 3) return launch_pairs_kd<4, 3, SILU, FUSE>(a, qc, grid, s);
  return launch_pairs_kd<2, 1, SILU, FUSE>(a, qc, grid, s);
}

template <class E, bool SILU>
hipError_t launch_typed(const ConvArgs& a, int K, int D, bool fast, int qc, dim3 grid,
                        hipStream_t s, bool fuse) {
  if ((a.chunk == pairs_chunk((K - 1) * D, true) || a.chunk == pairs_chunk((K - 1) * D, false)) &&
      fast && E::VEC == 8 && pairs_shape(K, D))
    return fuse ? launch_pairs<SILU, true>(a, K, D, qc, grid, s)
                : launch_pairs<SILU, false>(a, K, D, qc, grid, s);
  if (fast && !fuse) {
    if (K == 4 && D == 1) return launch_kd<E, 4, 1, SILU>(a, qc, grid, s);
    if (K == 4 && D == 3) return launch_kd<E, 4, 3, SILU>(a, qc, grid, s);
    if (K == 4 && D == 2) return launch_kd<E, 4, 2, SILU>(a, qc, grid, s);
    if (K == 3 && D == 1) return launch_kd<E, 3, 1, SILU>(a, qc, grid, s);
    if (K == 2 && D == 1) return launch_kd<E, 2, 1, SILU>(a, qc, grid, s);
  }
  hipLaunchKernelGGL((conv_generic<E, SILU>), grid, dim3(kBlock), 0, s, a, K, D);
  return hipGetLastError();
}



}  // namespace

// Fills the grid fields of `a` and launches. `uniform` = update mode (batch x q).
hipError_t launch_conv(ConvArgs a, int dtype, int K, int D, bool silu_act, bool aligned16,
                       hipStream_t stream, ConvLaunchInfo* info) {
  const int vec = dtype == 1 ? 8 : 4;
  const int H = (K - 1) * D;
  if (a.S <= 0) a.S = H;
  const bool uniform = a.qsl == nullptr;
  if (a.S != H && !a.sd && uniform) {
    // a buffer widened for speculative rollback: plain update on its first H columns
    const hipError_t e = launch_update_wide(a, dtype, K, D, silu_act, aligned16, stream);
    if (e != hipErrorNotSupported) return e;
  }
  // the register-window kernels assume S == H (the lane's state is H vectors);
  // residual fusion and row maps are built into the bf16 pair kernels and the
  // generic one
  const bool fuse = a.tok != nullptr || a.outer != nullptr || a.accumulate != 0;
  // (an SD pool keeps a lane's entries as vectors at any S; a DS one only at S == H)
  const bool rows_ok = a.S == H || a.sd;
  const bool pairs_ok = rows_ok && aligned16 && (a.C % vec == 0) && dtype == 1 &&
                        pairs_shape(K, D) &&
                        (!a.outer || (a.outer_rs * 2) % 16 == 0);
  const bool fast = rows_ok && aligned16 && (a.C % vec == 0) && fast_shape(K, D) &&
                    (!fuse || pairs_ok);
  // the one-pass kernel takes its halo from x: its chunk covers H by construction
  const bool pairs = fast && pairs_ok;
  const bool small = (int64_t)a.num_tokens * a.C <= kSmallLaunch;
  a.chunk = pairs ? pairs_chunk(H, small) : fast ? kChunk : (H > kChunk ? H : kChunk);
  int qc = 0;
  if (fast && uniform && (a.q == 1 || a.q == 2 || a.q == 4) && a.q <= a.chunk) qc = a.q;
  const int64_t per_block_ch = (int64_t)kBlock * (fast ? vec : 1);
  a.n_cblk = (int)((a.C + per_block_ch - 1) / per_block_ch);
  int64_t n_chunks;
  if (pairs && qc) {
    const int R = qc == 1 ? update_reqs_rt(H, a.sd != 0, a.batch, a.n_cblk)
                          : update_reqs(H, qc, a.sd != 0);
    a.ureqs = R;
    n_chunks = (a.batch + R - 1) / R;     // workgroup groups of R requests
  } else if (uniform) {
    n_chunks = (int64_t)a.batch * ((a.q + a.chunk - 1) / a.chunk);
  } else {
    n_chunks = a.num_tokens / a.chunk + a.batch;
  }
  const int64_t n_logical = n_chunks * a.n_cblk;
  if (n_logical > 0x7FFFFFF0LL) return hipErrorInvalidValue;
  a.n_logical = (int)n_logical;
  a.per_xcd = (int)((n_logical + kXcds - 1) / kXcds);
  dim3 grid((unsigned)(a.per_xcd * kXcds));
  if (info) {
    info->fast = fast;
    info->qc = qc;
    info->grid = (int64_t)grid.x;
    info->chunk = a.chunk;
  }
  if (dtype == 1)
    return silu_act ? launch_typed<BF16, true>(a, K, D, fast, qc, grid, stream, fuse)
                    : launch_typed<BF16, false>(a, K, D, fast, qc, grid, stream, fuse);
  return silu_act ? launch_typed<F32, true>(a, K, D, fast, qc, grid, stream, fuse)
                  : launch_typed<F32, false>(a, K, D, fast, qc, grid, stream, fuse);
}

}  // namespace sc
