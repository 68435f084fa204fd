// Exact online-softmax (log-sum-exp) merge of N partials per query row.
//
// The query host combines the hosts' local outputs A_n and statistics s_n
// into exact global attention: s = log sum_n exp(s_n) and
// A = sum_n exp(s_n - s) A_n (Pith review of Star Attention, Referee Report
// minor comment on Algorithm 2, and "Circularity Check").  Partials with
// s_n = -inf (empty chunks, fully masked rows) get weight 0.
//
// One wave per row: lanes split the N statistics for the max and the sum
// (wave reductions), then every lane accumulates D/64 output columns over
// the N partials with coalesced loads of each partial's row.
#include "common.h"
#include "internal.h"

namespace star {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr int PER = D / 64;  // columns per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.R) return;
  const int N = p.N;
  float m = -INFINITY;
  for (int n = lane; n < N; n += 64) m = fmaxf(m, p.lsep[(int64_t)n * p.R + row]);
  m = wave_max(m);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float sum = 0.f;
    for (int n = lane; n < N; n += 64) sum += __expf(p.lsep[(int64_t)n * p.R + row] - m);
    sum = wave_sum(sum);
    lse = m + __logf(sum);
    for (int n = 0; n < N; ++n) {
      const float sn = p.lsep[(int64_t)n * p.R + row];
      if (sn == -INFINITY) continue;
      const float w = __expf(sn - lse);
      const float* src = p.opart + ((int64_t)n * p.R + row) * D + lane * PER;
      if constexpr (PER == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(src);
        acc[0] += w * v[0];
        acc[1] += w * v[1];
      } else {
        acc[0] += w * src[0];
      }
    }
  }
  const int64_t s = row % p.S;
  const int64_t bh = row / p.S;
  const int64_t h = bh % p.H, b = bh / p.H;
  const int64_t off = b * p.osB + h * p.osH + s * p.osS + lane * PER;
  if (p.o_f32) {
    float* o = reinterpret_cast<float*>(p.o) + off;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = acc[i];
  } else {
    __bf16* o = reinterpret_cast<__bf16*>(p.o) + off;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = (__bf16)acc[i];
  }
  if (p.lse != nullptr && lane == 0) p.lse[row] = lse;
}

}  // namespace

hipError_t launch_merge(MergeParams& p, hipStream_t stream) {
  if (p.R <= 0) return hipSuccess;
  const int64_t blocks = (p.R + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (p.D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace star
