// star_decode_step_noalloc: the fused decode step for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The split-KV partials that
// star_decode_step keeps in caller workspaces live here in a file-scope
// device array instead, one copy per GPU.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device (with that device current) and kept.  Only that address
// is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/star_attn.h"
#include "internal.h"

namespace {

constexpr int64_t kScratchBytes = STAR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// device address of this GPU's scratch array (resolved on first use)
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return STAR_ERR_HIP;
  if (dev >= kMaxDevices) return STAR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return STAR_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return STAR_OK;
}

}  // namespace

extern "C" int star_decode_step_noalloc(const star_tensor* q_new, const star_tensor* k_new,
                                        const star_tensor* v_new, const star_tensor* k_cache,
                                        const star_tensor* v_cache, int64_t slot, int64_t pos,
                                        double base, int32_t rope, const int64_t* part_offsets,
                                        int32_t P, int32_t splits, float scale,
                                        const star_tensor* o, float* lse, void* stream) {
  // every argument but the workspaces, as star_decode_step checks them
  int s = star::decode_step_impl(q_new, k_new, v_new, k_cache, v_cache, slot, pos, base, rope,
                                 part_offsets, P, splits, scale, nullptr, nullptr, o, lse,
                                 stream, false);
  if (s != STAR_OK) return s;
  // partials: o_part [P*splits, B, Hq, 1, D] then lse_part [P*splits, B, Hq]
  const int64_t rows = (int64_t)P * splits * q_new->B * q_new->H;
  const int64_t o_bytes = rows * q_new->D * 4;
  const int64_t o_span = (o_bytes + 255) / 256 * 256;   // lse part 256-byte aligned
  if (rows > kScratchBytes / 4 || o_span + rows * 4 > kScratchBytes) return STAR_ERR_UNSUPPORTED;
  void* base_ptr = nullptr;
  if ((s = scratch_address(&base_ptr)) != STAR_OK) return s;
  float* o_part = static_cast<float*>(base_ptr);
  float* lse_part = reinterpret_cast<float*>(static_cast<uint8_t*>(base_ptr) + o_span);
  return star::decode_step_impl(q_new, k_new, v_new, k_cache, v_cache, slot, pos, base, rope,
                                part_offsets, P, splits, scale, o_part, lse_part, o, lse, stream,
                                true);
}
