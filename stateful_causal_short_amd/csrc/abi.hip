// C ABI of libstatefulconv.so: host-side validation, then one asynchronous
// launch on the caller's stream. Declarations and their defining passages are
// in include/statefulconv.h.
#include <stdint.h>

#include <new>
#include <unordered_set>
#include <vector>

#include "statefulconv.h"
#include "kernels.hpp"
#include "cca.hpp"

namespace {

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Descriptor checks shared by the depthwise entry points. The state-capacity
// rule follows the PLE layer's _short_conv (cache narrower than the window
// raises); a wider state is a buffer sized for speculative rollback.
sc_status check_conv_desc(const sc_conv_desc* d, int* H) {
  if (d->dtype != SC_DTYPE_F32 && d->dtype != SC_DTYPE_BF16) return SC_ERR_DTYPE;
  if (d->channels < 1 || d->width < 1 || d->dilation < 1) return SC_ERR_INVALID_ARG;
  if (d->width > 8) return SC_ERR_UNSUPPORTED;
  if (d->activation != SC_ACT_NONE && d->activation != SC_ACT_SILU) return SC_ERR_INVALID_ARG;
  if (d->x_row_stride < d->channels || d->out_row_stride < d->channels) return SC_ERR_INVALID_ARG;
  if (d->state_indices_stride < 1) return SC_ERR_INVALID_ARG;
  const int64_t h = (int64_t)(d->width - 1) * d->dilation;
  if (h > (1 << 20)) return SC_ERR_INVALID_ARG;
  if (d->state_len < h) return SC_ERR_STATE_CAPACITY;
  if (d->state_len > (1 << 20)) return SC_ERR_INVALID_ARG;
  if (d->state_layout != SC_STATE_DS && d->state_layout != SC_STATE_SD) return SC_ERR_INVALID_ARG;
  *H = (int)h;
  return SC_OK;
}

// Whether every vector access of the fast kernels is 16-byte aligned.
bool conv_aligned(const sc_conv_desc* d, const void* x, const void* out, const void* w,
                  const void* bias, const void* pool) {
  const int64_t es = d->dtype == SC_DTYPE_BF16 ? 2 : 4;
  return al16(x) && al16(out) && al16(w) && (!bias || al16(bias)) && (!pool || al16(pool)) &&
         (d->x_row_stride * es) % 16 == 0 && (d->out_row_stride * es) % 16 == 0;
}

// Descriptor checks of the optional residual fusion / row map.
sc_status check_fuse(const sc_conv_fuse* f, const sc_conv_desc* d) {
  if (!f) return SC_OK;
  if (f->accumulate != 0 && f->accumulate != 1) return SC_ERR_INVALID_ARG;
  if (f->token_indices && f->num_physical_rows < 1) return SC_ERR_INVALID_ARG;
  if (f->outer_residual && f->outer_row_stride < d->channels) return SC_ERR_INVALID_ARG;
  return SC_OK;
}

// Copies the fusion descriptor into the kernel arguments; out must not be the
// outer residual.
sc_status apply_fuse(const sc_conv_fuse* f, const void* out, sc::ConvArgs& a) {
  if (!f) return SC_OK;
  if (f->outer_residual && f->outer_residual == out) return SC_ERR_INVALID_ARG;
  a.tok = f->token_indices;
  a.phys_rows = f->num_physical_rows;
  a.accumulate = f->accumulate;
  a.outer = f->outer_residual;
  a.outer_rs = f->outer_row_stride;
  return SC_OK;
}

sc_status from_hip(hipError_t e) {
  if (e == hipSuccess) return SC_OK;
  if (e == hipErrorNotSupported) return SC_ERR_UNSUPPORTED;
  return SC_ERR_HIP;
}

// host side of sc_validate_metadata: copies the arrays and checks them
sc_status validate_metadata_host(const int32_t* query_start_loc,
                                 const int32_t* state_indices, int64_t idx_stride,
                                 int32_t batch, int64_t num_tokens, int32_t num_slots,
                                 hipStream_t st) {
  if (query_start_loc) {
    std::vector<int32_t> q((size_t)batch + 1);
    if (hipMemcpyAsync(q.data(), query_start_loc, q.size() * sizeof(int32_t),
                       hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return SC_ERR_HIP;
    if (q[0] != 0 || (int64_t)q[(size_t)batch] != num_tokens) return SC_ERR_INVALID_ARG;
    for (int32_t r = 0; r < batch; ++r)
      if (q[(size_t)r + 1] < q[(size_t)r]) return SC_ERR_INVALID_ARG;
  }
  if (state_indices) {
    if (idx_stride > (INT64_MAX / 4 - 1) / batch) return SC_ERR_INVALID_ARG;
    const size_t n = (size_t)(batch - 1) * (size_t)idx_stride + 1;
    std::vector<int32_t> s(n);
    if (hipMemcpyAsync(s.data(), state_indices, n * sizeof(int32_t), hipMemcpyDeviceToHost,
                       st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return SC_ERR_HIP;
    std::unordered_set<int32_t> seen;
    for (int32_t r = 0; r < batch; ++r) {
      const int32_t v = s[(size_t)r * (size_t)idx_stride];
      if (v < 0) continue;
      if (v >= num_slots || !seen.insert(v).second) return SC_ERR_INVALID_ARG;
    }
  }
  return SC_OK;
}

}  // namespace

extern "C" {

int32_t sc_abi_version(void) { return SC_ABI_VERSION; }

sc_status sc_validate_metadata(const int32_t* query_start_loc, const int32_t* state_indices,
                               int64_t idx_stride, int32_t batch, int64_t num_tokens,
                               int32_t num_slots, void* stream) {
  if (batch < 0 || num_tokens < 0 || num_slots < 0 || idx_stride < 1) return SC_ERR_INVALID_ARG;
  if (batch == 0) return SC_OK;
  // the host copies below must not let an allocation failure leave the C ABI
  try {
    return validate_metadata_host(query_start_loc, state_indices, idx_stride, batch,
                                  num_tokens, num_slots, (hipStream_t)stream);
  } catch (const std::bad_alloc&) {
    return SC_ERR_INVALID_ARG;
  }
}


const char* sc_status_string(sc_status s) {
  switch (s) {
    case SC_OK: return "ok";
    case SC_ERR_NULL_ARG: return "a required pointer is NULL";
    case SC_ERR_INVALID_ARG: return "invalid size, stride, enum or grid";
    case SC_ERR_DTYPE: return "unsupported dtype";
    case SC_ERR_STATE_CAPACITY: return "state_len smaller than (width-1)*dilation";
    case SC_ERR_UNSUPPORTED: return "configuration not supported by this library";
    case SC_ERR_HIP: return "HIP runtime error (launch or copy)";
  }
  return "unknown status";
}

sc_status sc_conv_prefill_varlen(const sc_conv_desc* desc, const void* x, void* out,
                                 const void* weight, const void* bias, void* state_pool,
                                 int32_t num_slots, const int32_t* query_start_loc,
                                 const int32_t* state_indices,
                                 const uint8_t* has_initial_state, int32_t batch,
                                 int64_t num_tokens, const sc_ckpt_desc* ckpt,
                                 const sc_conv_fuse* fuse, void* stream) {
  if (!desc) return SC_ERR_NULL_ARG;
  int H = 0;
  sc_status st = check_conv_desc(desc, &H);
  if (st != SC_OK) return st;
  if ((st = check_fuse(fuse, desc)) != SC_OK) return st;
  if (batch < 0 || num_tokens < 0 || num_slots < 0) return SC_ERR_INVALID_ARG;
  int32_t grid = 0;
  if (ckpt && ckpt->grid != 0) {
    // the PLE layer asserts grid >= conv_state_len: a window holds inputs only
    if (ckpt->grid < 0 || ckpt->grid < H) return SC_ERR_INVALID_ARG;
    grid = ckpt->grid;
  }
  // zero work is a no-op before any pointer is required (empty tensors may
  // carry NULL data pointers), as the GDN core returns early on zero tokens
  if (batch == 0 || num_tokens == 0) return SC_OK;
  if (!x || !out || !weight || !query_start_loc || !state_indices || !has_initial_state)
    return SC_ERR_NULL_ARG;
  if (!state_pool && num_slots > 0 && H > 0) return SC_ERR_NULL_ARG;
  if (grid && !ckpt->cu_ckpt) return SC_ERR_NULL_ARG;
  // no destination slots (an empty array: no request is long enough to reach a
  // checkpoint) means nothing to export
  if (grid && !ckpt->ckpt_slots) grid = 0;
  if (x == out) return SC_ERR_INVALID_ARG;
  if (num_tokens > 0x7FFFFFFFLL) return SC_ERR_UNSUPPORTED;
  sc::ConvArgs a{};
  a.x = x;
  a.out = out;
  a.w = weight;
  a.bias = bias;
  a.pool = state_pool;
  a.qsl = query_start_loc;
  a.slots = state_indices;
  a.has_init = has_initial_state;
  a.cu_ckpt = grid ? ckpt->cu_ckpt : nullptr;
  a.ckpt_slots = grid ? ckpt->ckpt_slots : nullptr;
  a.x_rs = desc->x_row_stride;
  a.out_rs = desc->out_row_stride;
  a.slot_stride = desc->state_indices_stride;
  a.num_tokens = num_tokens;
  a.C = desc->channels;
  a.num_slots = (H > 0) ? num_slots : 0;
  a.batch = batch;
  a.q = 0;
  a.ckpt_grid = grid;
  a.S = desc->state_len;
  a.sd = desc->state_layout == SC_STATE_SD ? 1 : 0;
  if ((st = apply_fuse(fuse, out, a)) != SC_OK) return st;
  const bool aligned = conv_aligned(desc, x, out, weight, bias, state_pool) &&
                       (!a.outer || al16(a.outer));
  return from_hip(sc::launch_conv(a, desc->dtype, desc->width, desc->dilation,
                                  desc->activation == SC_ACT_SILU, aligned,
                                  (hipStream_t)stream, nullptr));
}

sc_status sc_conv_update(const sc_conv_desc* desc, const void* x, void* out,
                         const void* weight, const void* bias, void* state_pool,
                         int32_t num_slots, const int32_t* state_indices,
                         const uint8_t* has_initial_state, int32_t batch, int32_t q,
                         const sc_conv_fuse* fuse, void* stream) {
  if (!desc) return SC_ERR_NULL_ARG;
  int H = 0;
  sc_status st = check_conv_desc(desc, &H);
  if (st != SC_OK) return st;
  if ((st = check_fuse(fuse, desc)) != SC_OK) return st;
  if (batch < 0 || q < 0 || num_slots < 0) return SC_ERR_INVALID_ARG;
  if (batch == 0 || q == 0) return SC_OK;
  if (!x || !out || !weight || !state_indices) return SC_ERR_NULL_ARG;
  if (!state_pool && num_slots > 0 && H > 0) return SC_ERR_NULL_ARG;
  if (x == out) return SC_ERR_INVALID_ARG;
  const int64_t T = (int64_t)batch * q;
  if (T > 0x7FFFFFFFLL) return SC_ERR_UNSUPPORTED;
  sc::ConvArgs a{};
  a.x = x;
  a.out = out;
  a.w = weight;
  a.bias = bias;
  a.pool = state_pool;
  a.qsl = nullptr;
  a.slots = state_indices;
  a.has_init = has_initial_state;
  a.x_rs = desc->x_row_stride;
  a.out_rs = desc->out_row_stride;
  a.slot_stride = desc->state_indices_stride;
  a.num_tokens = T;
  a.C = desc->channels;
  a.num_slots = (H > 0) ? num_slots : 0;
  a.batch = batch;
  a.q = q;
  a.ckpt_grid = 0;
  a.S = desc->state_len;
  a.sd = desc->state_layout == SC_STATE_SD ? 1 : 0;
  if ((st = apply_fuse(fuse, out, a)) != SC_OK) return st;
  const bool aligned = conv_aligned(desc, x, out, weight, bias, state_pool) &&
                       (!a.outer || al16(a.outer));
  return from_hip(sc::launch_conv(a, desc->dtype, desc->width, desc->dilation,
                                  desc->activation == SC_ACT_SILU, aligned,
                                  (hipStream_t)stream, nullptr));
}

sc_status sc_conv_update_spec(const sc_conv_desc* desc, const void* x, void* out,
                              const void* weight, const void* bias, void* state_pool,
                              int32_t num_slots, const int32_t* state_indices,
                              const int32_t* num_accepted_tokens, int32_t batch, int32_t q,
                              const sc_conv_fuse* fuse, void* stream) {
  if (!desc) return SC_ERR_NULL_ARG;
  int H = 0;
  sc_status st = check_conv_desc(desc, &H);
  if (st != SC_OK) return st;
  if ((st = check_fuse(fuse, desc)) != SC_OK) return st;
  if (batch < 0 || q < 0 || num_slots < 0) return SC_ERR_INVALID_ARG;
  // the rolled buffer keeps S - q old entries: q drafts must fit in it
  if (q > desc->state_len) return SC_ERR_INVALID_ARG;
  if (batch == 0 || q == 0) return SC_OK;
  if (!x || !out || !weight || !state_indices || !num_accepted_tokens) return SC_ERR_NULL_ARG;
  if (!state_pool && num_slots > 0) return SC_ERR_NULL_ARG;
  if (x == out) return SC_ERR_INVALID_ARG;
  const int64_t T = (int64_t)batch * q;
  if (T > 0x7FFFFFFFLL) return SC_ERR_UNSUPPORTED;
  sc::ConvArgs a{};
  a.x = x;
  a.out = out;
  a.w = weight;
  a.bias = bias;
  a.pool = state_pool;
  a.qsl = nullptr;
  a.slots = state_indices;
  a.has_init = nullptr;
  a.num_acc = num_accepted_tokens;
  a.x_rs = desc->x_row_stride;
  a.out_rs = desc->out_row_stride;
  a.slot_stride = desc->state_indices_stride;
  a.num_tokens = T;
  a.C = desc->channels;
  a.num_slots = num_slots;
  a.batch = batch;
  a.q = q;
  a.ckpt_grid = 0;
  a.S = desc->state_len;
  a.sd = desc->state_layout == SC_STATE_SD ? 1 : 0;
  if ((st = apply_fuse(fuse, out, a)) != SC_OK) return st;
  const bool aligned = conv_aligned(desc, x, out, weight, bias, state_pool) &&
                       (!a.outer || al16(a.outer));
  return from_hip(sc::launch_conv_spec(a, desc->dtype, desc->width, desc->dilation,
                                       desc->activation == SC_ACT_SILU, aligned,
                                       (hipStream_t)stream));
}

sc_status sc_conv_update_spec_varlen(const sc_conv_desc* desc, const void* x, void* out,
                                     const void* weight, const void* bias, void* state_pool,
                                     int32_t num_slots, const int32_t* state_indices,
                                     const int32_t* num_accepted_tokens,
                                     const int32_t* query_start_loc, int32_t batch,
                                     int64_t num_tokens, int32_t max_query_len,
                                     const sc_conv_fuse* fuse, void* stream) {
  if (!desc) return SC_ERR_NULL_ARG;
  int H = 0;
  sc_status st = check_conv_desc(desc, &H);
  if (st != SC_OK) return st;
  if ((st = check_fuse(fuse, desc)) != SC_OK) return st;
  if (batch < 0 || num_tokens < 0 || max_query_len < 0 || num_slots < 0)
    return SC_ERR_INVALID_ARG;
  // the rolled buffer keeps S - q old entries: every request's drafts must fit
  if (max_query_len > desc->state_len) return SC_ERR_INVALID_ARG;
  if (batch == 0 || num_tokens == 0 || max_query_len == 0) return SC_OK;
  if (!x || !out || !weight || !state_indices || !num_accepted_tokens || !query_start_loc)
    return SC_ERR_NULL_ARG;
  if (!state_pool && num_slots > 0) return SC_ERR_NULL_ARG;
  if (x == out) return SC_ERR_INVALID_ARG;
  if (num_tokens > 0x7FFFFFFFLL) return SC_ERR_UNSUPPORTED;
  sc::ConvArgs a{};
  a.x = x;
  a.out = out;
  a.w = weight;
  a.bias = bias;
  a.pool = state_pool;
  a.qsl = query_start_loc;
  a.slots = state_indices;
  a.has_init = nullptr;
  a.num_acc = num_accepted_tokens;
  a.x_rs = desc->x_row_stride;
  a.out_rs = desc->out_row_stride;
  a.slot_stride = desc->state_indices_stride;
  a.num_tokens = num_tokens;
  a.C = desc->channels;
  a.num_slots = num_slots;
  a.batch = batch;
  a.q = max_query_len;
  a.ckpt_grid = 0;
  a.S = desc->state_len;
  a.sd = desc->state_layout == SC_STATE_SD ? 1 : 0;
  if ((st = apply_fuse(fuse, out, a)) != SC_OK) return st;
  const bool aligned = conv_aligned(desc, x, out, weight, bias, state_pool) &&
                       (!a.outer || al16(a.outer));
  return from_hip(sc::launch_conv_spec(a, desc->dtype, desc->width, desc->dilation,
                                       desc->activation == SC_ACT_SILU, aligned,
                                       (hipStream_t)stream));
}

sc_status sc_state_gather(const void* pool, int32_t num_slots, int64_t row_bytes,
                          const int32_t* idx, int64_t idx_stride, int32_t n, void* dense,
                          void* stream) {
  if (num_slots < 0 || row_bytes < 1 || idx_stride < 1 || n < 0) return SC_ERR_INVALID_ARG;
  if (n == 0) return SC_OK;
  if (!idx || !dense || (!pool && num_slots > 0)) return SC_ERR_NULL_ARG;
  return from_hip(sc::launch_state_copy(true, pool, dense, row_bytes, num_slots, idx,
                                        idx_stride, n, (hipStream_t)stream));
}

sc_status sc_state_scatter(const void* dense, int64_t row_bytes, const int32_t* idx,
                           int64_t idx_stride, int32_t n, void* pool, int32_t num_slots,
                           void* stream) {
  if (num_slots < 0 || row_bytes < 1 || idx_stride < 1 || n < 0) return SC_ERR_INVALID_ARG;
  if (n == 0) return SC_OK;
  if (!idx || !dense || (!pool && num_slots > 0)) return SC_ERR_NULL_ARG;
  return from_hip(sc::launch_state_copy(false, dense, pool, row_bytes, num_slots, idx,
                                        idx_stride, n, (hipStream_t)stream));
}

sc_status sc_cca_qk_conv(const sc_cca_desc* desc, const void* q, const void* k,
                         const void* v_cur, const void* v_del, void* out, const void* w_dw,
                         const void* b_dw, const void* w_gr, const void* b_gr,
                         const void* delayed_init, void* conv_state, void* delayed_state,
                         int32_t num_slots, int32_t num_decodes,
                         const int32_t* decode_slots, int32_t num_prefills,
                         const int32_t* prefill_qsl, const int32_t* prefill_slots,
                         const uint8_t* prefill_has_initial_state, int64_t num_tokens,
                         void* stream) {
  if (!desc) return SC_ERR_NULL_ARG;
  if (desc->dtype != SC_DTYPE_BF16) return SC_ERR_DTYPE;
  const int nq = desc->num_q_heads, nkv = desc->num_kv_heads, hd = desc->head_dim;
  if (nq < 1 || nkv < 1 || hd < 2 || nq % nkv != 0 || hd % 2 != 0 || desc->t0 < 1 ||
      desc->t1 < 1)
    return SC_ERR_INVALID_ARG;
  if (num_slots < 0 || num_decodes < 0 || num_prefills < 0 || num_tokens < 0)
    return SC_ERR_INVALID_ARG;
  const int64_t C = (int64_t)(nq + nkv) * hd, vd = (int64_t)nkv * hd / 2;
  const int64_t W = (int64_t)(nq + 2 * nkv) * hd;
  if (desc->q_row_stride < (int64_t)nq * hd || desc->k_row_stride < (int64_t)nkv * hd ||
      desc->v_cur_row_stride < vd || desc->v_del_row_stride < vd || desc->out_row_stride < W)
    return SC_ERR_INVALID_ARG;
  if (desc->decode_slot_stride < 1 || desc->prefill_slot_stride < 1) return SC_ERR_INVALID_ARG;
  if (num_tokens < num_decodes) return SC_ERR_INVALID_ARG;
  if (num_tokens == 0 || (num_decodes == 0 && num_prefills == 0)) return SC_OK;
  if (!q || !k || !v_cur || !v_del || !out || !w_dw || !b_dw || !w_gr || !b_gr)
    return SC_ERR_NULL_ARG;
  if (num_decodes > 0 && !decode_slots) return SC_ERR_NULL_ARG;
  if (num_prefills > 0 && (!prefill_qsl || !prefill_slots || !prefill_has_initial_state))
    return SC_ERR_NULL_ARG;
  // with t0 = t1 = 1 there is no conv history (an empty, possibly NULL, pool)
  const bool has_history = desc->t0 + desc->t1 - 2 > 0;
  if (num_slots > 0 && ((has_history && !conv_state) || !delayed_state)) return SC_ERR_NULL_ARG;
  if (num_tokens > 0x7FFFFFFFLL || C > 0x7FFFFFFFLL) return SC_ERR_UNSUPPORTED;
  sc::CcaArgs a{};
  a.q = q;
  a.k = k;
  a.v_cur = v_cur;
  a.v_del = v_del;
  a.out = out;
  a.w_dw = w_dw;
  a.b_dw = b_dw;
  a.w_gr = w_gr;
  a.b_gr = b_gr;
  a.delayed_init = delayed_init;
  a.conv_state = conv_state;
  a.delayed_state = delayed_state;
  a.decode_slots = decode_slots;
  a.prefill_qsl = prefill_qsl;
  a.prefill_slots = prefill_slots;
  a.prefill_h = prefill_has_initial_state;
  a.q_rs = desc->q_row_stride;
  a.k_rs = desc->k_row_stride;
  a.vc_rs = desc->v_cur_row_stride;
  a.vd_rs = desc->v_del_row_stride;
  a.out_rs = desc->out_row_stride;
  a.dslot_stride = desc->decode_slot_stride;
  a.pslot_stride = desc->prefill_slot_stride;
  a.num_tokens = num_tokens;
  a.nq = nq;
  a.nkv = nkv;
  a.hd = hd;
  a.t0 = desc->t0;
  a.t1 = desc->t1;
  a.num_slots = num_slots;
  a.num_decodes = num_decodes;
  a.num_prefills = num_prefills;
  return from_hip(sc::launch_cca(a, (hipStream_t)stream));
}

}  // extern "C"
