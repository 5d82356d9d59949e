// Kernel argument blocks and launchers shared between the kernel sources and
// the C-ABI layer (abi.hip). Host + device visible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

// Launch constants of the depthwise kernels (measured choices, see the
// launchers in conv.hip):
constexpr int kChunk = 16;              // tokens per chunk of the fp32 / generic prefill
constexpr int kUnroll = 16;             // tokens per register-window step of conv_fast
constexpr int kPairsChunkLarge = 12;    // bf16 one-pass prefill chunk on large launches (H <= 4)
constexpr int kUpdateReqsDS = 4;        // requests per one-token update workgroup, DS pool
constexpr int kUpdateReqsSD = 8;        // the same on an SD pool
constexpr int kUpdateReqsMulti = 1;     // requests per workgroup for q = 2, 4 (H <= 4)
// LDS each bf16 one-pass prefill workgroup reserves at launch (dynamic
// shared memory the kernel never touches): a gfx950 CU has 160 KiB, so
// 48 KiB admits three 4-wave workgroups per CU, where the 91 registers alone
// would admit five. LDS and registers are the only per-launch residency
// controls the hardware has; three measured faster than two, four or five
// (fewer row streams contend less for HBM).
constexpr unsigned kPairsResidencyLds = 49152;

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
