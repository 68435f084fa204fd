// Device-side types and helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/star_attn.h"

namespace star {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32 (fp32 -> bf16 rounds to nearest even: v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte global load of 8 consecutive elements as bf16x8 (as 4 dwords).
// For fp32 sources, two 16-byte loads are converted to bf16 (RNE).
template <typename T>
struct Load8;

// load: a plain load.  load_stream: the same load with the nontemporal
// hint, for data read exactly once (it streams from HBM ~12% faster than
// plain 16-byte loads on this GPU: 6.5-6.8 against 5.7-6.0 TB/s measured).
template <>
struct Load8<__bf16> {
  static __device__ __forceinline__ u32x4 load(const __bf16* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
  static __device__ __forceinline__ u32x4 load_stream(const __bf16* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
};

template <>
struct Load8<float> {
  static __device__ __forceinline__ u32x4 pack(f32x4 a, f32x4 b) {
    u32x4 r;
    r[0] = pack_bf16(a[0], a[1]);
    r[1] = pack_bf16(a[2], a[3]);
    r[2] = pack_bf16(b[0], b[1]);
    r[3] = pack_bf16(b[2], b[3]);
    return r;
  }
  static __device__ __forceinline__ u32x4 load(const float* p) {
    return pack(reinterpret_cast<const f32x4*>(p)[0], reinterpret_cast<const f32x4*>(p)[1]);
  }
  static __device__ __forceinline__ u32x4 load_stream(const float* p) {
    return pack(__builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)),
                __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1));
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Maps a workgroup id to a logical work-item id so that the work items an
// XCD receives are contiguous in logical order.  Workgroups are handed to the
// 8 XCDs round-robin (id % 8), so neighbouring logical items (which share
// K/V ranges) land in the same XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int n) {
  const int xcd = w & 7, idx = w >> 3;
  const int base = n >> 3, extra = n & 7;
  return xcd * base + (xcd < extra ? xcd : extra) + idx;
}

}  // namespace star
