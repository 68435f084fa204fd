// Host-side launch interfaces between the C ABI (abi.cpp) and the kernels.
// Every struct here is passed to its kernel by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/star_attn.h"

namespace star {

struct TensorRef {
  const void* data;
  int64_t sB, sH, sS;
};

// Flash-style attention over analytic key ranges (Phase 1 and the Phase-2
// query chunk).  Key range A (the anchor or prefix: every row sees all of
// it) is read from pk/pv; key range B (own block or Phase-2 chunk, causal
// by position) from k/v.
struct FlashParams {
  TensorRef q, k, v;
  TensorRef pk, pv;      // source of key range A (k/v themselves for the anchor)
  int64_t pk_rows;       // rows of pk/pv
  int32_t B, Hq, Hkv, g;
  int32_t D;
  int32_t in_f32;        // Q/K/V are fp32 (rounded to bf16 on load)
  int64_t q_rows;        // rows of the q tensor
  int64_t kv_rows;       // rows of the k/v tensors
  int64_t pos_shift;     // position of q row r is r + pos_shift
  float scale;           // softmax scale on raw scores
  float scale_log2;      // scale * log2(e)
  // workgroup geometry (filled by the launcher)
  int32_t gw, npg, hgroups, m_pos;
  int32_t total_items;
  // mode 0: Phase 1 ; mode 1: Phase-2 partials
  int32_t mode;
  // Phase 1
  int64_t L, b, a;
  int32_t nblocks, nqt_full, nqt_last, nqt0;
  int32_t prefix_tab;    // 1: range A of block i is pk/pv rows [offs[i], offs[i] + chunk[i])
  // 1: q holds un-rotated rows; the kernel applies rotate-half RoPE at the
  // row's position with these inverse frequencies (D = 128) before use
  int32_t q_rope;
  double inv_freq[64];
  // Phase 2
  int32_t P, splits, nqt2;
  // Phase 2: partition offsets and split chunk length per partition.
  // Phase 1 with prefix_tab: prefix start (offs) and length (chunk) per block.
  int64_t offs[STAR_MAX_PARTS + 1];
  int64_t chunk[STAR_MAX_PARTS];
  // outputs
  void* o;               // Phase 1 O (bf16)
  int64_t osB, osH, osS;
  float* lse;            // Phase 1 lse (nullable) or Phase-2 lse_part
  float* opart;          // Phase-2 o_part
  // scheduling workspace (STAR_SCHED_INTS int32, device) or NULL: with it
  // the bf16 D = 128 kernel takes its items from per-XCD queues
  int32_t* sched;
};

hipError_t launch_flash(FlashParams& p, hipStream_t stream);
bool flash2_supported(const FlashParams& p);
hipError_t launch_flash2(FlashParams& p, hipStream_t stream);

// Split-KV decode partials (few query rows per KV head).
struct DecodeParams {
  TensorRef q, k, v;
  int32_t B, Hq, Hkv, g, D;
  int32_t in_f32;
  int64_t Lq;
  int64_t kv_rows;
  int64_t q_pos0;
  float scale, scale_log2;
  int32_t P, splits;
  int64_t offs[STAR_MAX_PARTS + 1];
  int64_t chunk[STAR_MAX_PARTS];
  int32_t total_items;
  float* opart;
  float* lse;
  // fused decode step (star_decode_step, one query row per head): rope of
  // q and of the new K row at position q_pos0 and the append of the new K/V
  // row by the workgroup whose chunk holds its slot
  int32_t fused;
  int32_t rope;
  TensorRef kn, vn;        // the new token's K (un-rotated) and V, [B, Hkv, 1, D]
  int64_t slot;            // cache row the new token is written to
  double inv_freq[64];     // theta_j of pair j (fused rope)
  // device-resident position (star_decode_step_devpos): when set, the
  // token's position (= its cache row) is read from *pos_dev at the start
  // of the launch instead of q_pos0 / slot; the last partition then ends
  // right after it.  Positions outside [offs[P - 1], pos_end) make the step
  // write nothing to the cache and produce empty partials.
  const int64_t* pos_dev;
  int64_t pos_end;
};

bool decode_supported(int g, int64_t Lq, int D);
hipError_t launch_decode(DecodeParams& p, hipStream_t stream);

// star_decode_step (abi.cpp): validation, then the fused decode launch and
// the merge; ws_given == false validates everything but the workspaces and
// launches nothing; pos_dev != nullptr: the position is read on the device
// (star_decode_step_devpos) and slot / pos are ignored
int decode_step_impl(const star_tensor* q_new, const star_tensor* k_new,
                     const star_tensor* v_new, const star_tensor* k_cache,
                     const star_tensor* v_cache, int64_t slot, int64_t pos, double base,
                     int32_t rope, const int64_t* part_offsets, int32_t P, int32_t splits,
                     float scale, float* o_part, float* lse_part, const star_tensor* o,
                     float* lse, void* stream, bool ws_given, int64_t* pos_dev = nullptr);

struct RopeParams {
  TensorRef x;
  void* y;
  int64_t ysB, ysH, ysS;
  int32_t B, H, D;
  int64_t S;
  int32_t f32;
  const int64_t* pos;
  int64_t pos0;
  double inv_freq[64];
};

hipError_t launch_rope(RopeParams& p, hipStream_t stream);

struct AppendParams {
  TensorRef kn, vn;
  void* kc;
  void* vc;
  int64_t kcsB, kcsH, kcsS, vcsB, vcsH, vcsS;
  int32_t B, H, D;
  int64_t T, slot0, pos0;
  int32_t rope;
  double inv_freq[64];
};

hipError_t launch_append(AppendParams& p, hipStream_t stream);

// rope(q) + KV append of the same tokens in one launch
struct PrepareParams {
  AppendParams kv;
  TensorRef qn;
  void* qo;
  int64_t qosB, qosH, qosS;
  int32_t Hq;
};

hipError_t launch_prepare(PrepareParams& p, hipStream_t stream);

struct MergeParams {
  const float* opart;
  const float* lsep;
  int32_t N;
  int64_t R;             // rows = B * H * S
  int32_t D;
  int32_t H;
  int64_t S;
  void* o;
  int32_t o_f32;
  int64_t osB, osH, osS;
  float* lse;
  int64_t* pos_inc;      // when set, one thread adds 1 to *pos_inc (device-position decode)
};

hipError_t launch_merge(MergeParams& p, hipStream_t stream);

// dst[b, h, r] = src[b, h, rows[r]] (a zero row where rows[r] is out of range)
struct GatherParams {
  TensorRef src;
  void* dst;
  int64_t dsB, dsH, dsS;
  const int64_t* rows;
  int64_t src_rows, R;
  int32_t B, H, D, f32;
};

hipError_t launch_gather(GatherParams& p, hipStream_t stream);

// streaming-read reference (stream.hip): bytes must be a multiple of
// workgroups * stream_read_granule()
int64_t stream_read_granule();
hipError_t launch_stream_read(const void* src, int64_t bytes, int32_t workgroups,
                              uint32_t* out, hipStream_t stream);

// RMSNorm of every row (length D) of a [B, H, S, D] bf16 tensor
struct RmsParams {
  TensorRef x;
  void* y;
  int64_t ysB, ysH, ysS;
  const void* gamma;     // bf16 [D]
  int64_t rows, S;
  int32_t H, D;
  float eps;
};

hipError_t launch_rmsnorm(RmsParams& p, hipStream_t stream);

}  // namespace star
