// Exact online-softmax (log-sum-exp) merge of N partials per query row.
//
// The query host combines the hosts' local outputs A_n and statistics s_n
// into exact global attention: s = log sum_n exp(s_n) and
// A = sum_n exp(s_n - s) A_n (Pith review of Star Attention, Referee Report
// minor comment on Algorithm 2, and "Circularity Check").  Partials with
// s_n = -inf (empty chunks, fully masked rows) get weight 0.
//
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

constexpr int MW = 8;  // waves per row

// One workgroup per row.  Pass 1: all threads stride the N statistics for
// the max and the sum of exp (block reductions through LDS).  Pass 2: wave w
// takes partials w, w + MW, ...; each lane owns D/64 output columns; eight
// partials' loads are issued before any is used, so a row costs a few
// memory latencies whatever N is.  The MW waves' sums meet in LDS.
template <int D>
__global__ __launch_bounds__(MW * 64) void merge_kernel(const MergeParams p) {
  constexpr int PER = D / 64;
  constexpr int U = 8;
  __shared__ float red[MW];
  __shared__ float part[MW][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int N = p.N;
  const float* ls = p.lsep + row;

  float m = -INFINITY;
  for (int n = tid; n < N; n += MW * 64) m = fmaxf(m, ls[(int64_t)n * p.R]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < MW; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  float lse = -INFINITY;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  if (m != -INFINITY) {
    float sum = 0.f;
    for (int n = tid; n < N; n += MW * 64) sum += __expf(ls[(int64_t)n * p.R] - m);
    sum = wave_sum(sum);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    sum = 0.f;
#pragma unroll
    for (int w = 0; w < MW; ++w) sum += red[w];
    lse = m + __logf(sum);
    const float* ob = p.opart + row * D + lane * PER;
    for (int n0 = wave; n0 < N; n0 += MW * U) {
      float wt[U];
      float v[U][PER];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * MW;
        wt[u] = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) v[u][i] = 0.f;
        if (n < N) {
          const float sn = ls[(int64_t)n * p.R];
          wt[u] = (sn == -INFINITY) ? 0.f : __expf(sn - lse);
          const float* src = ob + (int64_t)n * p.R * D;
#pragma unroll
          for (int i = 0; i < PER; ++i) v[u][i] = src[i];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += wt[u] * v[u][i];
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) part[wave][lane * PER + i] = acc[i];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < MW; ++w) o += part[w][lane * PER + i];
    acc[i] = o;
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
  if (p.R > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)p.R), block(MW * 64);
  if (p.D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace star
