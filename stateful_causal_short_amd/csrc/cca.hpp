// CCA kernel argument block and launcher, shared by cca.hip and abi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

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
  // filled by launch_cca: workgroup count and per-XCD share, the main
  // workgroups (S per head group), and the kv-head groups' tail split
  int32_t n_logical, per_xcd, n_main, kv_main_tiles, kv_help;
};

hipError_t launch_cca(const CcaArgs& a, hipStream_t stream);

}  // namespace sc
