// RoPE at original position ids, and the KV-cache append of new tokens.
//
// Every token is rotated at its true position: the anchor block keeps the
// first block's positions and query/generated tokens continue after the
// context (Pith review of Star Attention, "What carries the argument";
// Pith review of Pulsar Attention, "Assumptions & free parameters": original
// position ids preserve RoPE geometry).  Rotate-half form: pair (j, j+D/2)
// turns by pos * theta_j.
//
// The angle, its cos/sin and the rotation are fp64 (rope_math.h), rounded
// once to the output dtype.
//
// Both kernels are HBM-bound streams: a thread owns 8 pairs of one row
// (two 16-byte loads for bf16), computes their cos/sin once and applies them
// to every head of that position, so the trigonometry is amortised over H.
#include "common.h"
#include "internal.h"
#include "rope_math.h"

namespace star {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out);
template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* p, float* out) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16_lo(w[i]);
    out[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* out) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = a[i];
    out[4 + i] = b[i];
  }
}

// 8 fp64 values -> 8 stored elements, each rounded once (nearest even)
template <typename T>
__device__ __forceinline__ void store8(T* p, const double* in);
template <>
__device__ __forceinline__ void store8<__bf16>(__bf16* p, const double* in) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16_f64(in[2 * i], in[2 * i + 1]);
  *reinterpret_cast<u32x4*>(p) = w;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const double* in) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{(float)in[0], (float)in[1], (float)in[2], (float)in[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{(float)in[4], (float)in[5], (float)in[6], (float)in[7]};
}

// rotate 8 pairs (x1[i], x2[i]) by the angles whose cos/sin are cs/sn
__device__ __forceinline__ void rotate8(const float* x1, const float* x2, const double* cs,
                                        const double* sn, double* y1, double* y2) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    rope_rotate64((double)x1[i], (double)x2[i], cs[i], sn[i], y1[i], y2[i]);
}

// copy 8 bf16 values through fp64 (exact both ways)
__device__ __forceinline__ void widen8(const float* x, double* y) {
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (double)x[i];
}

// grid-stride over (head group, b, s, pair-chunk); loop over the heads of
// the group inside.  Long sequences use one group (sin/cos shared by all H
// heads); a handful of rows (decode) spreads the heads over threads.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(const RopeParams p, int hgroups) {
  const int nchunk = p.D / 16;  // chunks of 8 pairs per row
  const int64_t total = (int64_t)p.B * p.S * nchunk * hgroups;
  const int half = p.D / 2;
  const int hper = (p.H + hgroups - 1) / hgroups;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int ch = (int)(idx % nchunk);
    int64_t r = idx / nchunk;
    const int64_t s = r % p.S;
    r /= p.S;
    const int b = (int)(r % p.B);
    const int hg = (int)(r / p.B);
    const int h0 = hg * hper, h1 = min(p.H, h0 + hper);
    const double pos = (double)(p.pos ? p.pos[s] : p.pos0 + s);
    double cs[8], sn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rope_cs(pos, p.inv_freq[8 * ch + i], cs[i], sn[i]);
    const T* xb = reinterpret_cast<const T*>(p.x.data) + (int64_t)b * p.x.sB + s * p.x.sS;
    T* yb = reinterpret_cast<T*>(p.y) + (int64_t)b * p.ysB + s * p.ysS;
    // heads in groups of HG: all of a group's loads go out before the first
    // rotation, so a thread keeps 2 HG loads in flight rather than 2
    constexpr int HG = 4;
    int h = h0;
    for (; h + HG <= h1; h += HG) {
      float x1[HG][8], x2[HG][8];
#pragma unroll
      for (int u = 0; u < HG; ++u) {
        const T* xr = xb + (int64_t)(h + u) * p.x.sH;
        load8<T>(xr + 8 * ch, x1[u]);
        load8<T>(xr + half + 8 * ch, x2[u]);
      }
#pragma unroll
      for (int u = 0; u < HG; ++u) {
        T* yr = yb + (int64_t)(h + u) * p.ysH;
        double y1[8], y2[8];
        rotate8(x1[u], x2[u], cs, sn, y1, y2);
        store8<T>(yr + 8 * ch, y1);
        store8<T>(yr + half + 8 * ch, y2);
      }
    }
    for (; h < h1; ++h) {
      const T* xr = xb + (int64_t)h * p.x.sH;
      T* yr = yb + (int64_t)h * p.ysH;
      float x1[8], x2[8];
      double y1[8], y2[8];
      load8<T>(xr + 8 * ch, x1);
      load8<T>(xr + half + 8 * ch, x2);
      rotate8(x1, x2, cs, sn, y1, y2);
      store8<T>(yr + 8 * ch, y1);
      store8<T>(yr + half + 8 * ch, y2);
    }
  }
}

// one thread per (b, h, t, pair-chunk): rotate k_t, copy v_t, into the cache
__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  const int nchunk = p.D / 16;
  const int64_t total = (int64_t)p.B * p.H * p.T * nchunk;
  const int half = p.D / 2;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int ch = (int)(idx % nchunk);
    int64_t r = idx / nchunk;
    const int64_t t = r % p.T;
    r /= p.T;
    const int h = (int)(r % p.H);
    const int b = (int)(r / p.H);
    const __bf16* kr = reinterpret_cast<const __bf16*>(p.kn.data) + (int64_t)b * p.kn.sB +
                       (int64_t)h * p.kn.sH + t * p.kn.sS;
    const __bf16* vr = reinterpret_cast<const __bf16*>(p.vn.data) + (int64_t)b * p.vn.sB +
                       (int64_t)h * p.vn.sH + t * p.vn.sS;
    __bf16* kc = reinterpret_cast<__bf16*>(p.kc) + (int64_t)b * p.kcsB + (int64_t)h * p.kcsH +
                 (p.slot0 + t) * p.kcsS;
    __bf16* vc = reinterpret_cast<__bf16*>(p.vc) + (int64_t)b * p.vcsB + (int64_t)h * p.vcsH +
                 (p.slot0 + t) * p.vcsS;
    *reinterpret_cast<u32x4*>(vc + 8 * ch) = *reinterpret_cast<const u32x4*>(vr + 8 * ch);
    *reinterpret_cast<u32x4*>(vc + half + 8 * ch) = *reinterpret_cast<const u32x4*>(vr + half + 8 * ch);
    float x1[8], x2[8];
    double y1[8], y2[8];
    load8<__bf16>(kr + 8 * ch, x1);
    load8<__bf16>(kr + half + 8 * ch, x2);
    if (p.rope) {
      const double pos = (double)(p.pos0 + t);
      double cs[8], sn[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rope_cs(pos, p.inv_freq[8 * ch + i], cs[i], sn[i]);
      rotate8(x1, x2, cs, sn, y1, y2);
    } else {
      widen8(x1, y1);
      widen8(x2, y2);
    }
    store8<__bf16>(kc + 8 * ch, y1);
    store8<__bf16>(kc + half + 8 * ch, y2);
  }
}

// rope(q) and the KV append of the same tokens: threads [0, nq) rotate
// query rows, the rest handle K/V rows (one pair-chunk each)
__global__ __launch_bounds__(256) void prepare_kernel(const PrepareParams pp) {
  const AppendParams& p = pp.kv;
  const int nchunk = p.D / 16;
  const int half = p.D / 2;
  const int64_t nq = (int64_t)p.B * pp.Hq * p.T * nchunk;
  const int64_t nkv = (int64_t)p.B * p.H * p.T * nchunk;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nq + nkv;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const bool isq = idx < nq;
    const int64_t li = isq ? idx : idx - nq;
    const int ch = (int)(li % nchunk);
    int64_t r = li / nchunk;
    const int64_t t = r % p.T;
    r /= p.T;
    const int H = isq ? pp.Hq : p.H;
    const int h = (int)(r % H);
    const int b = (int)(r / H);
    const __bf16* src;
    __bf16* dst;
    if (isq) {
      src = reinterpret_cast<const __bf16*>(pp.qn.data) + (int64_t)b * pp.qn.sB +
            (int64_t)h * pp.qn.sH + t * pp.qn.sS;
      dst = reinterpret_cast<__bf16*>(pp.qo) + (int64_t)b * pp.qosB + (int64_t)h * pp.qosH +
            t * pp.qosS;
    } else {
      src = reinterpret_cast<const __bf16*>(p.kn.data) + (int64_t)b * p.kn.sB +
            (int64_t)h * p.kn.sH + t * p.kn.sS;
      dst = reinterpret_cast<__bf16*>(p.kc) + (int64_t)b * p.kcsB + (int64_t)h * p.kcsH +
            (p.slot0 + t) * p.kcsS;
      const __bf16* vr = reinterpret_cast<const __bf16*>(p.vn.data) + (int64_t)b * p.vn.sB +
                         (int64_t)h * p.vn.sH + t * p.vn.sS;
      __bf16* vc = reinterpret_cast<__bf16*>(p.vc) + (int64_t)b * p.vcsB + (int64_t)h * p.vcsH +
                   (p.slot0 + t) * p.vcsS;
      *reinterpret_cast<u32x4*>(vc + 8 * ch) = *reinterpret_cast<const u32x4*>(vr + 8 * ch);
      *reinterpret_cast<u32x4*>(vc + half + 8 * ch) =
          *reinterpret_cast<const u32x4*>(vr + half + 8 * ch);
    }
    float x1[8], x2[8];
    double y1[8], y2[8];
    load8<__bf16>(src + 8 * ch, x1);
    load8<__bf16>(src + half + 8 * ch, x2);
    if (p.rope) {
      const double pos = (double)(p.pos0 + t);
      double cs[8], sn[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rope_cs(pos, p.inv_freq[8 * ch + i], cs[i], sn[i]);
      rotate8(x1, x2, cs, sn, y1, y2);
    } else {
      widen8(x1, y1);
      widen8(x2, y2);
    }
    store8<__bf16>(dst + 8 * ch, y1);
    store8<__bf16>(dst + half + 8 * ch, y2);
  }
}

int grid_for(int64_t total) {
  const int64_t blocks = (total + 255) / 256;
  return (int)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_rope(RopeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.S * (p.D / 16);
  if (rows <= 0 || p.H <= 0) return hipSuccess;
  const int hgroups = rows < 16384 ? p.H : 1;
  const int64_t total = rows * hgroups;
  if (p.f32)
    hipLaunchKernelGGL(rope_kernel<float>, dim3(grid_for(total)), dim3(256), 0, stream, p, hgroups);
  else
    hipLaunchKernelGGL(rope_kernel<__bf16>, dim3(grid_for(total)), dim3(256), 0, stream, p, hgroups);
  return hipGetLastError();
}

hipError_t launch_prepare(PrepareParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.kv.B * (p.Hq + p.kv.H) * p.kv.T * (p.kv.D / 16);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(prepare_kernel, dim3(grid_for(total)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_append(AppendParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.B * p.H * p.T * (p.D / 16);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(grid_for(total)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace star
