// Streaming-read reference for the HBM-bound kernels: every byte of a
// buffer is read once with 16-byte nontemporal loads (the fastest plain
// read form measured on this GPU: 6.5-6.8 TB/s, against 5.7-6.0 TB/s with
// the default cache policy), 8 loads in flight per thread,
// and each workgroup writes the XOR of the 32-bit words it read (so the
// loads cannot be dropped, and a caller can check the result).  Not a step
// of the method: it measures what a plain read reaches on this GPU, the
// practical ceiling for the decode kernel.
#include "common.h"
#include "internal.h"

namespace star {
namespace {

constexpr int SU = 8;        // loads in flight per thread
constexpr int ST = 256;      // threads per workgroup

__global__ __launch_bounds__(ST) void stream_read_kernel(const u32x4* __restrict__ src,
                                                         int64_t per, uint32_t* out) {
  // per (16-byte words per workgroup) is a multiple of SU * ST
  const u32x4* b = src + (int64_t)blockIdx.x * per;
  uint32_t acc = 0;
  for (int64_t i = threadIdx.x; i < per; i += SU * ST) {
    u32x4 v[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) v[u] = __builtin_nontemporal_load(b + i + u * ST);
#pragma unroll
    for (int u = 0; u < SU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  __shared__ uint32_t wx[ST / 64];
  if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < ST / 64; ++w) r ^= wx[w];
    out[blockIdx.x] = r;
  }
}

}  // namespace

int64_t stream_read_granule() { return (int64_t)16 * SU * ST; }

hipError_t launch_stream_read(const void* src, int64_t bytes, int32_t workgroups,
                              uint32_t* out, hipStream_t stream) {
  const int64_t per = bytes / 16 / workgroups;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(ST), 0, stream,
                     reinterpret_cast<const u32x4*>(src), per, out);
  return hipGetLastError();
}

}  // namespace star
