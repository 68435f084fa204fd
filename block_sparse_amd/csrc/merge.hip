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

constexpr int MW = 8;  // waves per row

// One workgroup per row, one pass over the partials.  Wave w takes partials
// w, w + MW, ... in batches of U (their statistics and output columns are
// loaded together, so a batch costs one memory latency) and keeps a running
// (max, sum of exp, weighted output) for them, rescaled when the max grows.
// The MW waves' running values are then merged the same way through LDS.
// Every lane of a wave handles the same partials, so the running max and
// sum are wave-uniform; each lane owns D/64 output columns.
template <int D>
__global__ __launch_bounds__(MW * 64) void merge_kernel(const MergeParams p) {
  constexpr int PER = D / 64;
  constexpr int U = 8;
  __shared__ float wm[MW], ws[MW];
  __shared__ float wacc[MW][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int N = p.N;
  const float* ls = p.lsep + row;
  const float* ob = p.opart + row * D + lane * PER;

  float m = -INFINITY, sum = 0.f;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int n0 = wave; n0 < N; n0 += MW * U) {
    float sn[U];
    float v[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = n0 + u * MW;
      sn[u] = -INFINITY;
#pragma unroll
      for (int i = 0; i < PER; ++i) v[u][i] = 0.f;
      if (n < N) {
        sn[u] = ls[(int64_t)n * p.R];
        const float* src = ob + (int64_t)n * p.R * D;
#pragma unroll
        for (int i = 0; i < PER; ++i) v[u][i] = src[i];
      }
    }
    float bm = sn[0];
#pragma unroll
    for (int u = 1; u < U; ++u) bm = fmaxf(bm, sn[u]);
    if (bm == -INFINITY) continue;            // only empty partials in this batch
    const float nm = fmaxf(m, bm);
    const float f = (m == -INFINITY) ? 0.f : __expf(m - nm);
    sum *= f;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] *= f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = (sn[u] == -INFINITY) ? 0.f : __expf(sn[u] - nm);
      sum += w;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += w * v[u][i];
    }
    m = nm;
  }
  if (lane == 0) {
    wm[wave] = m;
    ws[wave] = sum;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) wacc[wave][lane * PER + i] = acc[i];
  __syncthreads();
  if (wave != 0) return;
  float M = wm[0];
#pragma unroll
  for (int w = 1; w < MW; ++w) M = fmaxf(M, wm[w]);
  float S = 0.f;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < MW; ++w) {
      const float f = (wm[w] == -INFINITY) ? 0.f : __expf(wm[w] - M);
      S += f * ws[w];
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] += f * wacc[w][lane * PER + i];
    }
  }
  const float inv = S > 0.f ? 1.0f / S : 0.f;
  const float lse = S > 0.f ? M + __logf(S) : -INFINITY;
  const int64_t s = row % p.S;
  const int64_t bh = row / p.S;
  const int64_t h = bh % p.H, b = bh / p.H;
  const int64_t off = b * p.osB + h * p.osH + s * p.osS + lane * PER;
  if (p.o_f32) {
    float* out = reinterpret_cast<float*>(p.o) + off;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[i] = o[i] * inv;
  } else {
    __bf16* out = reinterpret_cast<__bf16*>(p.o) + off;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[i] = (__bf16)(o[i] * inv);
  }
  if (p.lse != nullptr && lane == 0) p.lse[row] = lse;
  // device-position decode: advance the position for the next step (the
  // decode launch that read it has completed before this launch started)
  if (p.pos_inc != nullptr && row == 0 && lane == 0) *p.pos_inc += 1;
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
