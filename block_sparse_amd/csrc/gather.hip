// Row gather dst[b, h, r] = src[b, h, rows[r]]: assembles a Phase-1 prefix
// from context rows that keep their original positions (Pith review of
// Pulsar Attention, "What carries the argument").  Pure data movement: one
// 16-byte load and store per thread, consecutive threads on consecutive
// bytes of a row.
#include "common.h"
#include "internal.h"

namespace star {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void gather_kernel(const GatherParams p) {
  const int esz = p.f32 ? 4 : 2;
  const int tpr = p.D * esz / 16;                 // threads per row
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t row = gid / tpr;                   // over B * H * R
  const int c = (int)(gid - row * tpr);
  if (row >= (int64_t)p.B * p.H * p.R) return;
  const int64_t r = row % p.R;
  const int64_t bh = row / p.R;
  const int64_t h = bh % p.H, b = bh / p.H;
  const int64_t sr = p.rows[r];
  u32x4 v = {0, 0, 0, 0};
  if (sr >= 0 && sr < p.src_rows) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(p.src.data) +
                         (b * p.src.sB + h * p.src.sH + sr * p.src.sS) * esz;
    v = reinterpret_cast<const u32x4*>(src)[c];
  }
  uint8_t* dst = reinterpret_cast<uint8_t*>(p.dst) + (b * p.dsB + h * p.dsH + r * p.dsS) * esz;
  reinterpret_cast<u32x4*>(dst)[c] = v;
}

}  // namespace

hipError_t launch_gather(GatherParams& p, hipStream_t stream) {
  const int64_t tpr = (int64_t)p.D * (p.f32 ? 4 : 2) / 16;
  const int64_t total = (int64_t)p.B * p.H * p.R * tpr;
  const int64_t grid = (total + NT - 1) / NT;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace star
