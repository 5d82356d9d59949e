// Slot-indexed row copies between a state pool and a dense buffer
// (gather / scatter through state indices, as ZayaCCA._mix_with_state gathers
// `conv_state[slot]` and writes `conv_state[slot] = new_history`).
#include "common.hpp"
#include "kernels.hpp"

namespace sc {

template <typename T>
__device__ __forceinline__ T zero_el() {
  if constexpr (sizeof(T) == 16) return u32x4{0, 0, 0, 0};
  else return T(0);
}

// One or more workgroups per row; `bpr` workgroups share a row. Each thread
// copies up to kCopyUnroll elements per pass, all loads issued before the
// first store so that many are in flight; the rows are streamed through
// (nontemporal loads and stores: a row is touched once).
constexpr int kCopyUnroll = 4;
template <typename T, bool GATHER>
__global__ __launch_bounds__(kBlock) void row_copy(const void* src, void* dst,
                                                   int64_t row_elems, int32_t num_slots,
                                                   const int32_t* idx, int64_t idx_stride,
                                                   int32_t n, int32_t bpr) {
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / bpr;
  const int part = (int)(bid - row * bpr);
  if (row >= n) return;
  const int32_t s = idx[row * idx_stride];
  const bool valid = s >= 0 && s < num_slots;
  if (!GATHER && !valid) return;
  const int64_t src_row = GATHER ? (valid ? (int64_t)s : 0) : row;
  const int64_t dst_row = GATHER ? row : (int64_t)s;
  const T* sp = (const T*)src + src_row * row_elems;
  T* dp = (T*)dst + dst_row * row_elems;
  const int64_t stride = (int64_t)bpr * kBlock;
  for (int64_t e0 = (int64_t)part * kBlock + threadIdx.x; e0 < row_elems;
       e0 += kCopyUnroll * stride) {
    T v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t e = e0 + u * stride;
      v[u] = (valid && e < row_elems) ? __builtin_nontemporal_load(sp + e) : zero_el<T>();
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t e = e0 + u * stride;
      if (e < row_elems) __builtin_nontemporal_store(v[u], dp + e);
    }
  }
}

namespace {
template <typename T>
hipError_t launch_t(bool gather, const void* src, void* dst, int64_t row_bytes,
                    int32_t num_slots, const int32_t* idx, int64_t idx_stride, int32_t n,
                    hipStream_t stream) {
  const int64_t row_elems = row_bytes / (int64_t)sizeof(T);
  int64_t bpr = (row_elems + kCopyUnroll * kBlock - 1) / (kCopyUnroll * kBlock);
  if (bpr < 1) bpr = 1;
  if (bpr > 64) bpr = 64;
  const int64_t blocks = (int64_t)n * bpr;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (gather)
    hipLaunchKernelGGL((row_copy<T, true>), dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                       src, dst, row_elems, num_slots, idx, idx_stride, n, (int32_t)bpr);
  else
    hipLaunchKernelGGL((row_copy<T, false>), dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                       src, dst, row_elems, num_slots, idx, idx_stride, n, (int32_t)bpr);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_state_copy(bool gather, const void* src, void* dst, int64_t row_bytes,
                             int32_t num_slots, const int32_t* idx, int64_t idx_stride,
                             int32_t n, hipStream_t stream) {
  const uintptr_t al = (uintptr_t)src | (uintptr_t)dst;
  if (row_bytes % 16 == 0 && (al & 15) == 0)
    return launch_t<u32x4>(gather, src, dst, row_bytes, num_slots, idx, idx_stride, n, stream);
  if (row_bytes % 4 == 0 && (al & 3) == 0)
    return launch_t<uint32_t>(gather, src, dst, row_bytes, num_slots, idx, idx_stride, n, stream);
  return launch_t<uint8_t>(gather, src, dst, row_bytes, num_slots, idx, idx_stride, n, stream);
}

}  // namespace sc
