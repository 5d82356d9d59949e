// Shared device helpers for the gfx950 kernels: 16-byte vector access and
// element traits (bf16 / fp32 storage, fp32 arithmetic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;      // threads per workgroup (4 wave64)
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round-robin

// Compute units of the current device (host; cached per device, 256 if the
// runtime cannot say); safe to call from several host threads.
int device_cus();

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// Streaming load: read once by this kernel.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Streaming store: the output is not re-read by this kernel.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// bf16 storage: 8 channels per 16-byte vector; element 2i is the low half of
// word i. Widening is exact; narrowing is one round-to-nearest-even
// (v_cvt_pk_bf16_f32 on gfx950).
struct BF16 {
  using S = uint16_t;
  static constexpr int VEC = 8;
  __device__ __forceinline__ static void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static u32x4 pack(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2 p = {f[2 * i], f[2 * i + 1]};
      r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
    }
    return r;
  }
  // raw element e (0..7) of a vector, and its replacement
  __device__ __forceinline__ static uint32_t get(const u32x4& v, int e) {
    return (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
  }
  __device__ __forceinline__ static void set(u32x4& v, int e, uint32_t val) {
    const int sh = 16 * (e & 1);
    v[e >> 1] = (v[e >> 1] & ~(0xFFFFu << sh)) | (val << sh);
  }
};

// fp32 storage: 4 channels per 16-byte vector.
struct F32 {
  using S = uint32_t;
  static constexpr int VEC = 4;
  __device__ __forceinline__ static void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static u32x4 pack(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    return r;
  }
  __device__ __forceinline__ static uint32_t get(const u32x4& v, int e) { return v[e]; }
  __device__ __forceinline__ static void set(u32x4& v, int e, uint32_t val) { v[e] = val; }
};

// SiLU z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

}  // namespace sc
