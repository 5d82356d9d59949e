// Kernel argument blocks and launchers shared between the kernel sources and
// the C-ABI layer (abi.hip). Host + device visible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

constexpr int kChunk = 64;   // tokens per prefill chunk (>= H for the fast kernels)

// Depthwise conv launch arguments (by value into the kernel).
struct ConvArgs {
  const void* x;
  void* out;
  const void* w;
  const void* bias;          // nullable
  void* pool;
  const int32_t* qsl;        // nullptr = uniform update (batch x q)
  const int32_t* slots;
  const uint8_t* has_init;   // nullable = all continue their state
  const int32_t* cu_ckpt;
  const int32_t* ckpt_slots;
  int64_t x_rs, out_rs, slot_stride;   // elements
  int64_t num_tokens;
  int32_t C, num_slots, batch, q, ckpt_grid;
  // filled by launch_conv
  int32_t chunk, n_cblk, n_logical, per_xcd;
};

struct ConvLaunchInfo {
  bool fast;
  int qc;
  int64_t grid;
  int chunk;
};

hipError_t launch_conv(ConvArgs a, int dtype, int K, int D, bool silu_act, bool aligned16,
                       hipStream_t stream, ConvLaunchInfo* info);

hipError_t launch_state_copy(bool gather, const void* src, void* dst, int64_t row_bytes,
                             int32_t num_slots, const int32_t* idx, int64_t idx_stride,
                             int32_t n, hipStream_t stream);

// CCA launch arguments.
struct CcaArgs {
  const void* q;
  const void* k;
  const void* v_cur;
  const void* v_del;
  void* out;
  const void* w_dw;
  const void* b_dw;
  const void* w_gr;
  const void* b_gr;
  const void* delayed_init;   // nullable
  void* conv_state;
  void* delayed_state;
  const int32_t* decode_slots;
  const int32_t* prefill_qsl;
  const int32_t* prefill_slots;
  const uint8_t* prefill_h;
  int64_t q_rs, k_rs, vc_rs, vd_rs, out_rs, dslot_stride, pslot_stride;
  int64_t num_tokens;
  int32_t nq, nkv, hd, t0, t1, num_slots, num_decodes, num_prefills;
};

hipError_t launch_cca(const CcaArgs& a, hipStream_t stream);

}  // namespace sc
