// RMSNorm of the residual stream in front of the q/k/v projections (the
// Llama-3 attention block of the Star Attention pages' HuggingFace models:
// graphcanon record of NVIDIA/Star-Attention, README).  One wave per row:
// the sum of squares in fp32, one rounding of x * rsqrt(mean + eps) * gamma
// to bf16.  HBM-bound: a row is read once (at the Llama hidden sizes; twice,
// the second time from cache, at other sizes) and written once.
#include "common.h"
#include "internal.h"

namespace star {
namespace {

constexpr int RW = 4;   // rows (waves) per workgroup

__global__ __launch_bounds__(RW * 64) void rmsnorm_kernel(const RmsParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * RW + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int64_t s = row % p.S;
  const int64_t bh = row / p.S;
  const int64_t h = bh % p.H, b = bh / p.H;
  const __bf16* x = reinterpret_cast<const __bf16*>(p.x.data) + b * p.x.sB + h * p.x.sH + s * p.x.sS;
  __bf16* y = reinterpret_cast<__bf16*>(p.y) + b * p.ysB + h * p.ysH + s * p.ysS;
  const int nch = p.D / 8;
  float ss = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const bf16x8 v = as_bf16x8(*reinterpret_cast<const u32x4*>(x + 8 * c));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = (float)v[e];
      ss = __builtin_fmaf(f, f, ss);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  const float r = 1.0f / sqrtf(ss / (float)p.D + p.eps);
  const __bf16* g = reinterpret_cast<const __bf16*>(p.gamma);
  for (int c = lane; c < nch; c += 64) {
    const bf16x8 v = as_bf16x8(*reinterpret_cast<const u32x4*>(x + 8 * c));
    const bf16x8 gv = as_bf16x8(*reinterpret_cast<const u32x4*>(g + 8 * c));
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)((float)v[e] * r * (float)gv[e]);
    *reinterpret_cast<bf16x8*>(y + 8 * c) = out;
  }
}

// The same for D = 512 NC (the Llama hidden sizes): the wave's row stays in
// registers (NC 16-byte chunks per lane, all loads in flight at once), so it
// is read from memory once.  Each lane sums its chunks in the order the
// general kernel does, so the results are the same bits.
template <int NC>
__global__ __launch_bounds__(RW * 64) void rmsnorm_reg_kernel(const RmsParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * RW + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int64_t s = row % p.S;
  const int64_t bh = row / p.S;
  const int64_t h = bh % p.H, b = bh / p.H;
  const __bf16* x = reinterpret_cast<const __bf16*>(p.x.data) + b * p.x.sB + h * p.x.sH + s * p.x.sS;
  __bf16* y = reinterpret_cast<__bf16*>(p.y) + b * p.ysB + h * p.ysH + s * p.ysS;
  const __bf16* g = reinterpret_cast<const __bf16*>(p.gamma);
  u32x4 v[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + 8 * (lane + 64 * i)));
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const bf16x8 f8 = as_bf16x8(v[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = (float)f8[e];
      ss = __builtin_fmaf(f, f, ss);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  const float r = 1.0f / sqrtf(ss / (float)p.D + p.eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    const bf16x8 f8 = as_bf16x8(v[i]);
    const bf16x8 gv = as_bf16x8(*reinterpret_cast<const u32x4*>(g + 8 * c));
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)((float)f8[e] * r * (float)gv[e]);
    *reinterpret_cast<bf16x8*>(y + 8 * c) = out;
  }
}

}  // namespace

hipError_t launch_rmsnorm(RmsParams& p, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  const int64_t grid = (p.rows + RW - 1) / RW;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 gd((unsigned)grid), bd(RW * 64);
  switch (p.D) {
    case 512: hipLaunchKernelGGL(rmsnorm_reg_kernel<1>, gd, bd, 0, stream, p); break;
    case 1024: hipLaunchKernelGGL(rmsnorm_reg_kernel<2>, gd, bd, 0, stream, p); break;
    case 2048: hipLaunchKernelGGL(rmsnorm_reg_kernel<4>, gd, bd, 0, stream, p); break;
    case 4096: hipLaunchKernelGGL(rmsnorm_reg_kernel<8>, gd, bd, 0, stream, p); break;
    case 8192: hipLaunchKernelGGL(rmsnorm_reg_kernel<16>, gd, bd, 0, stream, p); break;
    default: hipLaunchKernelGGL(rmsnorm_kernel, gd, bd, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace star
