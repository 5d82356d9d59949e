// Sanitizer driver for the oracle (TEST INFRASTRUCTURE ONLY).
//
// Built together with oracle.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer by oracle/build.py (build_sanitized) and run by
// the CPU test suite. It calls every oracle entry point over the tiny shapes
// the brute-force pins sweep (channels 1..3, widths 1..4, dilations 1..3,
// lengths 0..7 with and without history, padding and out-of-range slots,
// checkpoints, both state layouts, widened and rolling buffers, residual
// fusion with a row map, the CCA path in every depthwise mode, the row
// copies), so that any out-of-bounds access or undefined operation in the
// oracle aborts the run. Values are not checked here; the pins do that.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

extern "C" {
int oracle_conv(int32_t C, int32_t K, int32_t d, int32_t act, int32_t io_dtype,
                int32_t out_dtype, const void* x, int64_t x_rs, void* out, int64_t out_rs,
                double* absum, const void* w, const void* bias, void* pool, int32_t num_slots,
                int32_t state_len, int32_t state_layout, int32_t num_decodes, int32_t q,
                const int32_t* decode_slots, int64_t decode_slot_stride, const uint8_t* decode_h,
                int32_t num_prefills, const int32_t* qsl_p, const int32_t* prefill_slots,
                int64_t prefill_slot_stride, const uint8_t* prefill_h, int32_t ckpt_grid,
                const int32_t* cu_ckpt, const int32_t* ckpt_slots, const uint8_t* row_mask,
                const int32_t* token_indices, const void* resid, int64_t resid_rs,
                const void* outer, int64_t outer_rs, int32_t nthreads);
int oracle_conv_spec(int32_t C, int32_t K, int32_t d, int32_t S, int32_t state_layout,
                     int32_t act, int32_t io_dtype, int32_t out_dtype, const void* x,
                     int64_t x_rs, void* out, int64_t out_rs, double* absum, const void* w,
                     const void* bias, void* pool, int32_t num_slots, int32_t B, int32_t q,
                     const int32_t* slots, int64_t slot_stride, const int32_t* num_accepted,
                     const uint8_t* row_mask, const int32_t* token_indices, const void* resid,
                     int64_t resid_rs, const void* outer, int64_t outer_rs, int32_t nthreads);
int oracle_conv_spec_varlen(int32_t C, int32_t K, int32_t d, int32_t S, int32_t state_layout,
                            int32_t act, int32_t io_dtype, int32_t out_dtype, const void* x,
                            int64_t x_rs, void* out, int64_t out_rs, double* absum,
                            const void* w, const void* bias, void* pool, int32_t num_slots,
                            int32_t B, const int32_t* qsl, const int32_t* slots,
                            int64_t slot_stride, const int32_t* num_accepted,
                            const uint8_t* row_mask, const int32_t* token_indices,
                            const void* resid, int64_t resid_rs, const void* outer,
                            int64_t outer_rs, int32_t nthreads);
int oracle_cca(int32_t nq, int32_t nkv, int32_t hd, int32_t t0, int32_t t1, int32_t io_dtype,
               int32_t out_dtype, int32_t dw_mode, const void* qp, int64_t q_rs, const void* kp,
               int64_t k_rs, const void* vcur, int64_t vc_rs, const void* vdel, int64_t vd_rs,
               void* out, int64_t out_rs, double* absum, const void* w_dw, const void* b_dw,
               const void* w_gr, const void* b_gr, const void* delayed_init, void* conv_state,
               void* delayed_state, int32_t num_slots, int32_t num_decodes,
               const int32_t* decode_slots, int64_t dstride, int32_t num_prefills,
               const int32_t* qsl_p, const int32_t* prefill_slots, int64_t pstride,
               const uint8_t* prefill_h, const uint8_t* row_mask, int64_t* dw_chain_diff,
               double* dw_allow, int32_t nthreads);
int oracle_state_gather(int32_t elsize, int64_t row_elems, const void* pool, int32_t num_slots,
                        const int32_t* idx, int64_t idx_stride, int32_t n, void* dense);
int oracle_state_scatter(int32_t elsize, int64_t row_elems, const void* dense,
                         const int32_t* idx, int64_t idx_stride, int32_t n, void* pool,
                         int32_t num_slots);
}

namespace {

std::mt19937_64 rng(12345);

// Random storage for `n` elements of dtype dt (0 f32, 1 bf16, 2 f64): finite
// values of moderate size.
std::vector<uint8_t> randbuf(int dt, size_t n) {
  const size_t es = dt == 0 ? 4 : dt == 1 ? 2 : 8;
  std::vector<uint8_t> b(n * es + 1);   // +1: never empty
  std::normal_distribution<float> nd(0.f, 1.f);
  for (size_t i = 0; i < n; ++i) {
    const float f = nd(rng);
    if (dt == 0) ((float*)b.data())[i] = f;
    else if (dt == 2) ((double*)b.data())[i] = f;
    else {
      uint32_t u;
      __builtin_memcpy(&u, &f, 4);
      ((uint16_t*)b.data())[i] = (uint16_t)(u >> 16);
    }
  }
  return b;
}

int fails = 0;
void expect(int rc, const char* what) {
  if (rc != 0) {
    std::fprintf(stderr, "%s returned %d\n", what, rc);
    ++fails;
  }
}

// One depthwise batch: decodes then prefills of the given lengths.
void conv_batch(int dt, int C, int K, int d, int S, int sd, const std::vector<int>& lens,
                int nd, int q, int grid, bool fuse, int nthreads) {
  const int H = (K - 1) * d;
  int np = (int)lens.size();
  std::vector<int32_t> qsl(np + 1, 0);
  for (int r = 0; r < np; ++r) qsl[r + 1] = qsl[r] + lens[r];
  const int T = nd * q + qsl[np];
  std::vector<int32_t> cu(np + 1, 0);
  for (int r = 0; r < np; ++r) cu[r + 1] = cu[r] + (grid > 0 ? lens[r] / grid : 0);
  const int nck = cu[np];
  const int slots = nd + np + nck + 2;
  std::vector<int32_t> dsl(nd), psl(np), cks(nck + 1);
  for (int i = 0; i < nd; ++i) dsl[i] = (i == 1) ? -1 : i;          // one padding row
  for (int r = 0; r < np; ++r) psl[r] = (r == 2) ? slots + 3 : nd + r;   // one out of range
  for (int i = 0; i < nck; ++i) cks[i] = nd + np + i;
  std::vector<uint8_t> dh(nd + 1), ph(np + 1), mask(T + 1, 1);
  for (int i = 0; i < nd; ++i) dh[i] = i & 1;
  for (int r = 0; r < np; ++r) ph[r] = (r + 1) & 1;
  if (T > 2) mask[T / 2] = 0;
  std::vector<int32_t> tok(T + 1);
  for (int i = 0; i < T; ++i) tok[i] = T - 1 - i;                   // reversed row map
  auto x = randbuf(dt, (size_t)T * C), w = randbuf(dt, (size_t)C * K), b = randbuf(dt, C);
  auto pool = randbuf(dt, (size_t)slots * C * S), res = randbuf(dt, (size_t)T * C);
  auto outer = randbuf(dt, (size_t)T * C);
  for (int odt : {dt, 2}) {
    auto out = randbuf(odt, (size_t)T * C);
    std::vector<double> ab((size_t)T * C + 1);
    expect(oracle_conv(C, K, d, 1, dt, odt, x.data(), C, out.data(), C, ab.data(), w.data(),
                       b.data(), pool.data(), slots, S, sd, nd, q, dsl.data(), 1, dh.data(), np,
                       qsl.data(), psl.data(), 1, ph.data(), grid, grid ? cu.data() : nullptr,
                       grid ? cks.data() : nullptr, mask.data(), fuse ? tok.data() : nullptr,
                       fuse ? res.data() : nullptr, C, fuse ? outer.data() : nullptr, C,
                       nthreads),
           "oracle_conv");
    (void)H;
  }
}

void spec_batch(int dt, int C, int K, int d, int S, int sd, int B, int q, bool fuse) {
  const int H = (K - 1) * d;
  if (q > S || S < H) return;
  const int T = B * q, slots = B + 2;
  std::vector<int32_t> sl(B + 1), acc(B + 1), qsl(B + 1, 0);
  for (int r = 0; r < B; ++r) {
    sl[r] = r == 1 ? -1 : r;
    acc[r] = (r * 7) % (q + 3) - 1;   // includes values the oracle clamps
    qsl[r + 1] = qsl[r] + (r % (q + 1));
  }
  std::vector<int32_t> tok(T + 1);
  for (int i = 0; i < T; ++i) tok[i] = (i * 5 + 3) % T;
  auto x = randbuf(dt, (size_t)T * C), w = randbuf(dt, (size_t)C * K), b = randbuf(dt, C);
  auto pool = randbuf(dt, (size_t)slots * C * S), out = randbuf(dt, (size_t)T * C);
  auto res = randbuf(dt, (size_t)T * C);
  std::vector<double> ab((size_t)T * C + 1);
  expect(oracle_conv_spec(C, K, d, S, sd, 1, dt, dt, x.data(), C, out.data(), C, ab.data(),
                          w.data(), b.data(), pool.data(), slots, B, q, sl.data(), 1,
                          acc.data(), nullptr, fuse ? tok.data() : nullptr,
                          fuse ? res.data() : nullptr, C, nullptr, 0, 2),
         "oracle_conv_spec");
  auto out64 = randbuf(2, (size_t)T * C);
  expect(oracle_conv_spec_varlen(C, K, d, S, sd, 0, dt, 2, x.data(), C, out64.data(), C,
                                 ab.data(), w.data(), nullptr, pool.data(), slots, B,
                                 qsl.data(), sl.data(), 1, acc.data(), nullptr, nullptr,
                                 nullptr, 0, nullptr, 0, 1),
         "oracle_conv_spec_varlen");
}

void cca_batch(int nq, int nkv, int hd, int t0, int t1, int dw_mode, int odt) {
  const int C = (nq + nkv) * hd, vd = nkv * hd / 2, W = (nq + 2 * nkv) * hd, n = t0 + t1 - 2;
  const int nd = 3;
  std::vector<int32_t> qsl = {0, 1, 1, 5, 12};
  const int np = (int)qsl.size() - 1, T = nd + qsl[np], slots = nd + np + 1;
  std::vector<int32_t> dsl = {0, -1, 2}, psl = {3, 4, slots + 2, 5};
  std::vector<uint8_t> ph = {1, 0, 1, 1}, mask(T, 1);
  mask[4] = 0;
  auto qb = randbuf(1, (size_t)T * nq * hd), kb = randbuf(1, (size_t)T * nkv * hd);
  auto vc = randbuf(1, (size_t)T * vd), vdl = randbuf(1, (size_t)T * vd);
  auto wdw = randbuf(1, (size_t)C * t0), bdw = randbuf(1, C);
  auto wgr = randbuf(1, (size_t)C * hd * t1), bgr = randbuf(1, C), di = randbuf(1, vd);
  auto cs = randbuf(1, (size_t)slots * C * n), ds = randbuf(1, (size_t)slots * vd);
  auto out = randbuf(odt, (size_t)T * W);
  std::vector<double> ab((size_t)T * W), allow((size_t)T * W);
  int64_t diff = -1;
  expect(oracle_cca(nq, nkv, hd, t0, t1, 1, odt, dw_mode, qb.data(), nq * hd, kb.data(),
                    nkv * hd, vc.data(), vd, vdl.data(), vd, out.data(), W, ab.data(),
                    wdw.data(), bdw.data(), wgr.data(), bgr.data(), di.data(), cs.data(),
                    ds.data(), slots, nd, dsl.data(), 1, np, qsl.data(), psl.data(), 1,
                    ph.data(), mask.data(), dw_mode == 2 ? &diff : nullptr, allow.data(), 3),
         "oracle_cca");
}

}  // namespace

int main() {
  // depthwise: the brute-force pin shapes, both dtypes and layouts
  for (int dt : {0, 1})
    for (int C = 1; C <= 3; ++C)
      for (int K = 1; K <= 4; ++K)
        for (int d = 1; d <= 3; ++d)
          for (int sd = 0; sd <= 1; ++sd) {
            const int H = (K - 1) * d;
            conv_batch(dt, C, K, d, H, sd, {0, 1, 2, 3, 7, 5}, 3, 1, 0, false, 1);
            conv_batch(dt, C, K, d, H + 2, sd, {4, 0, 6}, 2, 2, 0, C == 2, 2);
            if (H >= 1) conv_batch(dt, C, K, d, H, sd, {7, H, 2 * H + 1, 1}, 0, 1, H, C == 3, 3);
            for (int q = 1; q <= 3; ++q) spec_batch(dt, C, K, d, H + q + 1, sd, 4, q, q == 2);
          }
  // CCA: both kernel widths of the grouped stage, every depthwise mode
  for (int mode = 0; mode <= 2; ++mode)
    for (int t0 = 1; t0 <= 4; ++t0)
      for (int t1 = 1; t1 <= 3; ++t1) cca_batch(4, 2, 4, t0, t1, mode, mode == 1 ? 1 : 2);
  cca_batch(2, 2, 2, 2, 2, 2, 1);
  // row copies, with padding and out-of-range indices
  std::vector<uint16_t> pool(5 * 6), dense(4 * 6);
  std::vector<int32_t> idx = {4, -1, 9, 0};
  expect(oracle_state_gather(2, 6, pool.data(), 5, idx.data(), 1, 4, dense.data()),
         "oracle_state_gather");
  expect(oracle_state_scatter(2, 6, dense.data(), idx.data(), 1, 4, pool.data(), 5),
         "oracle_state_scatter");
  if (fails) {
    std::fprintf(stderr, "%d oracle calls failed\n", fails);
    return 1;
  }
  std::printf("oracle sanitizer run: ok\n");
  return 0;
}
