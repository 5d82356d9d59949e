// Kernel argument blocks and launchers shared between the kernel sources and
// the C-ABI layer (abi.hip). Host + device visible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

#ifndef SC_PREFILL_CHUNK
#define SC_PREFILL_CHUNK 16
#endif
#ifndef SC_UNROLL_SMALL_H
#define SC_UNROLL_SMALL_H 16
#endif
#ifndef SC_UNROLL_LARGE_H
#define SC_UNROLL_LARGE_H 16
#endif
#ifndef SC_NO_XCD_REMAP
#define SC_NO_XCD_REMAP 0
#endif
#ifndef SC_NT_LOADS
#define SC_NT_LOADS 1   // streaming (non-temporal) loads of token rows read once
#endif
#ifndef SC_LDS_PAD
#define SC_LDS_PAD 0
#endif
#ifndef SC_PAIRS_LDS_RESERVE
// LDS each one-pass prefill workgroup reserves only to cap residency (the
// kernel itself uses none): a gfx950 CU has 160 KiB, so 48 KiB admits three
// 4-wave workgroups per CU. Three measured faster than the five the register
// count allows (and than two or four): fewer streams contend for HBM.
#define SC_PAIRS_LDS_RESERVE 49152
#endif
#ifndef SC_NO_PAIRS
#define SC_NO_PAIRS 0
#endif
#ifndef SC_PAIRS_CHUNK_SMALL
#define SC_PAIRS_CHUNK_SMALL 12
#endif
#ifndef SC_UPDATE_REQS
#define SC_UPDATE_REQS 4
#endif
#ifndef SC_UPDATE_REQS_SD
#define SC_UPDATE_REQS_SD 8   // requests per q = 1 update workgroup on an SD pool (H <= 4)
#endif
#ifndef SC_UPDATE_REQS_MULTI
#define SC_UPDATE_REQS_MULTI 1   // requests per update workgroup for q = 2, 4 (H <= 4)
#endif
constexpr int kChunk = SC_PREFILL_CHUNK;   // tokens per prefill chunk (>= H for the fast kernels)

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
  const int32_t* num_acc;    // speculative update: accepted counts (batch), else nullptr
  const int32_t* tok;        // logical row -> physical row of x / out / outer, or nullptr
  const void* outer;         // added to each result at its physical row, or nullptr
  int64_t outer_rs;          // elements
  int32_t accumulate;        // 1: out rows hold a residual on entry; the result is added to it
  int64_t phys_rows;         // rows of x / out / outer when tok is given (indices are clamped)
  int64_t num_tokens;
  int32_t C, num_slots, batch, q, ckpt_grid;
  int32_t S;                 // state entries per channel (>= H); the window is entries [0, H)
  int32_t sd;                // 1: pool is (num_slots, S, C) ("SD"), else (num_slots, C, S)
  // filled by launch_conv
  int32_t chunk, n_cblk, n_logical, per_xcd;
  int32_t ureqs;             // requests per one-token update workgroup (host side)
};

struct ConvLaunchInfo {
  bool fast;
  int qc;
  int64_t grid;
  int chunk;
};

hipError_t launch_conv(ConvArgs a, int dtype, int K, int D, bool silu_act, bool aligned16,
                       hipStream_t stream, ConvLaunchInfo* info);

// Speculative multi-token update on a rolling buffer of S >= H entries per
// channel (requests of exactly a.q tokens, accepted counts in a.num_acc).
hipError_t launch_conv_spec(ConvArgs a, int dtype, int K, int D, bool silu_act, bool aligned16,
                            hipStream_t stream);
// Plain decode / multi-token update on a buffer wider than H (the window in the
// first H columns); nullptr-free fast path or hipErrorNotSupported.
hipError_t launch_update_wide(ConvArgs a, int dtype, int K, int D, bool silu_act, bool aligned16,
                              hipStream_t stream);

hipError_t launch_state_copy(bool gather, const void* src, void* dst, int64_t row_bytes,
                             int32_t num_slots, const int32_t* idx, int64_t idx_stride,
                             int32_t n, hipStream_t stream);



}  // namespace sc
