// C ABI of the Star Attention hot path: argument validation on the host,
// then dispatch to the gfx950 kernels on the caller's stream.  The entry
// points are declared and documented in include/star_attn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/star_attn.h"
#include "internal.h"

namespace {

using star::TensorRef;

int esize(int32_t dtype) { return dtype == STAR_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Basic checks of one tensor descriptor.
int check_tensor(const star_tensor* t, bool allow_f32) {
  if (t == nullptr || t->data == nullptr) return STAR_ERR_NULL;
  if (t->dtype != STAR_BF16 && !(allow_f32 && t->dtype == STAR_F32)) return STAR_ERR_DTYPE;
  if (t->B < 1 || t->H < 1 || t->S < 0 || t->D < 1) return STAR_ERR_SHAPE;
  if (t->sB < 0 || t->sH < 0 || t->sS < 0) return STAR_ERR_SHAPE;
  const int64_t e = esize(t->dtype);
  if (!aligned16(t->data)) return STAR_ERR_ALIGN;
  if ((t->sB * e) % 16 || (t->sH * e) % 16 || (t->sS * e) % 16) return STAR_ERR_ALIGN;
  return STAR_OK;
}

TensorRef ref(const star_tensor* t) { return TensorRef{t->data, t->sB, t->sH, t->sS}; }

int hip_status(hipError_t e) { return e == hipSuccess ? STAR_OK : STAR_ERR_HIP; }

bool rope_dim_ok(int64_t D) { return D >= 16 && D <= 128 && D % 16 == 0; }

// theta_j = base^(-2j/D), j < D/2: the power in extended precision (x87
// long double, 64-bit significand, error ~2^-63 relative), rounded once to
// fp64, so theta_j is the fp64 value nearest the exact power unless that
// power lies within ~2^-10 ulp of a rounding midpoint.  Every rotating
// kernel forms its angle as the IEEE product pos * theta_j from these.
void fill_inv_freq(double* inv_freq, int64_t D, double base) {
  for (int64_t j = 0; j < D / 2; ++j)
    inv_freq[j] = (double)std::pow((long double)base,
                                   -2.0L * (long double)j / (long double)D);
  for (int64_t j = D / 2; j < 64; ++j) inv_freq[j] = 0.0;
}

// Shared validation of q/k/v for the attention entry points.
int check_qkv(const star_tensor* q, const star_tensor* k, const star_tensor* v) {
  int s;
  if ((s = check_tensor(q, true)) != STAR_OK) return s;
  if ((s = check_tensor(k, true)) != STAR_OK) return s;
  if ((s = check_tensor(v, true)) != STAR_OK) return s;
  if (k->dtype != q->dtype || v->dtype != q->dtype) return STAR_ERR_DTYPE;
  if (q->D != 64 && q->D != 128) return STAR_ERR_UNSUPPORTED;
  if (k->D != q->D || v->D != q->D) return STAR_ERR_SHAPE;
  if (k->B != q->B || v->B != q->B) return STAR_ERR_SHAPE;
  if (k->H != v->H || k->S != v->S) return STAR_ERR_SHAPE;
  if (q->H % k->H != 0) return STAR_ERR_SHAPE;
  if (q->H / k->H > 16) return STAR_ERR_UNSUPPORTED;
  if (q->B > 65535 || q->H > 65535) return STAR_ERR_UNSUPPORTED;
  return STAR_OK;
}

// Partition offsets (host [P + 1]) and the split chunk length per
// partition: c_j = roundup(ceil(n_j / splits), STAR_SPLIT_ALIGN).
int check_parts(const int64_t* part_offsets, int32_t P, int32_t splits, int64_t rows,
                int64_t* chunk) {
  if (part_offsets == nullptr) return STAR_ERR_NULL;
  if (P < 1 || P > STAR_MAX_PARTS || splits < 1 || splits > 1024) return STAR_ERR_SHAPE;
  if (part_offsets[0] < 0 || part_offsets[P] > rows) return STAR_ERR_SHAPE;
  for (int j = 0; j < P; ++j)
    if (part_offsets[j + 1] < part_offsets[j]) return STAR_ERR_SHAPE;
  for (int j = 0; j < P; ++j) {
    const int64_t n = part_offsets[j + 1] - part_offsets[j];
    int64_t c = (n + splits - 1) / splits;
    c = (c + STAR_SPLIT_ALIGN - 1) / STAR_SPLIT_ALIGN * STAR_SPLIT_ALIGN;
    chunk[j] = c;
  }
  return STAR_OK;
}

// Split-KV decode launch parameters common to the partial and fused paths.
void decode_params(star::DecodeParams& p, const star_tensor* q, const star_tensor* k_cache,
                   const star_tensor* v_cache, const int64_t* part_offsets, int32_t P,
                   int32_t splits, const int64_t* chunk, int64_t q_pos0, float scale,
                   float* o_part, float* lse_part) {
  std::memset(&p, 0, sizeof(p));
  p.q = ref(q);
  p.k = ref(k_cache);
  p.v = ref(v_cache);
  p.B = (int32_t)q->B;
  p.Hq = (int32_t)q->H;
  p.Hkv = (int32_t)k_cache->H;
  p.g = (int32_t)(q->H / k_cache->H);
  p.D = (int32_t)q->D;
  p.in_f32 = q->dtype == STAR_F32;
  p.Lq = q->S;
  p.kv_rows = k_cache->S;
  p.q_pos0 = q_pos0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.P = P;
  p.splits = splits;
  for (int j = 0; j <= P; ++j) p.offs[j] = part_offsets[j];
  for (int j = 0; j < P; ++j) p.chunk[j] = chunk[j];
  p.opart = o_part;
  p.lse = lse_part;
}

// Validation shared by the Phase-1 entry points.
int check_phase1(const star_tensor* q, const star_tensor* k, const star_tensor* v,
                 int64_t block_b, float scale, const star_tensor* o, const float* lse,
                 const int32_t* sched) {
  int s;
  if ((s = check_qkv(q, k, v)) != STAR_OK) return s;
  if ((s = check_tensor(o, false)) != STAR_OK) return s;
  if (k->S != q->S) return STAR_ERR_SHAPE;
  if (o->B != q->B || o->H != q->H || o->S != q->S || o->D != q->D) return STAR_ERR_SHAPE;
  if (block_b < 1) return STAR_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return STAR_ERR_SHAPE;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return STAR_ERR_ALIGN;
  if (sched != nullptr && (reinterpret_cast<uintptr_t>(sched) & 3u)) return STAR_ERR_ALIGN;
  return STAR_OK;
}

// Phase-1 launch parameters common to both entry points (key range A is
// filled by the caller).
void phase1_params(star::FlashParams& p, const star_tensor* q, const star_tensor* k,
                   const star_tensor* v, int64_t block_b, float scale, const star_tensor* o,
                   float* lse, int32_t* sched) {
  std::memset(&p, 0, sizeof(p));
  p.q = ref(q);
  p.k = ref(k);
  p.v = ref(v);
  p.B = (int32_t)q->B;
  p.Hq = (int32_t)q->H;
  p.Hkv = (int32_t)k->H;
  p.g = p.Hq / p.Hkv;
  p.D = (int32_t)q->D;
  p.in_f32 = q->dtype == STAR_F32;
  p.q_rows = q->S;
  p.kv_rows = k->S;
  p.pos_shift = 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.mode = 0;
  p.L = q->S;
  p.b = block_b < q->S ? block_b : q->S;
  p.o = o->data;
  p.osB = o->sB;
  p.osH = o->sH;
  p.osS = o->sS;
  p.lse = lse;
  p.sched = sched;
}

}  // namespace

extern "C" {

const char* star_status_string(int status) {
  switch (status) {
    case STAR_OK: return "STAR_OK";
    case STAR_ERR_NULL: return "STAR_ERR_NULL: a required pointer is NULL";
    case STAR_ERR_SHAPE: return "STAR_ERR_SHAPE: inconsistent or out-of-range sizes";
    case STAR_ERR_DTYPE: return "STAR_ERR_DTYPE: unsupported dtype or dtype combination";
    case STAR_ERR_ALIGN: return "STAR_ERR_ALIGN: data or stride not 16-byte aligned";
    case STAR_ERR_UNSUPPORTED: return "STAR_ERR_UNSUPPORTED: valid request this build does not serve";
    case STAR_ERR_HIP: return "STAR_ERR_HIP: the HIP runtime reported a launch error";
    case STAR_ERR_BLAS: return "STAR_ERR_BLAS: the BLAS library reported an error";
    default: return "unknown star_status";
  }
}

int star_abi_version(void) { return 500; }

int star_rope_freqs(int64_t D, double base, double* inv_freq) {
  if (inv_freq == nullptr) return STAR_ERR_NULL;
  if (!rope_dim_ok(D)) return STAR_ERR_UNSUPPORTED;
  if (!(base > 1.0) || !std::isfinite(base)) return STAR_ERR_SHAPE;
  double f[64];
  fill_inv_freq(f, D, base);
  for (int64_t j = 0; j < D / 2; ++j) inv_freq[j] = f[j];
  return STAR_OK;
}

int star_rope_apply(const star_tensor* x_in, const star_tensor* x_out, const int64_t* pos,
                    int64_t pos0, double base, void* stream) {
  int s;
  if ((s = check_tensor(x_in, true)) != STAR_OK) return s;
  if ((s = check_tensor(x_out, true)) != STAR_OK) return s;
  if (x_out->dtype != x_in->dtype) return STAR_ERR_DTYPE;
  if (x_out->B != x_in->B || x_out->H != x_in->H || x_out->S != x_in->S || x_out->D != x_in->D)
    return STAR_ERR_SHAPE;
  if (!rope_dim_ok(x_in->D)) return STAR_ERR_UNSUPPORTED;
  if (!(base > 1.0) || !std::isfinite(base)) return STAR_ERR_SHAPE;
  if (pos == nullptr && pos0 < 0) return STAR_ERR_SHAPE;
  if (x_in->B > 65535 || x_in->H > 65535) return STAR_ERR_UNSUPPORTED;
  if (x_in->S == 0) return STAR_OK;
  star::RopeParams p;
  std::memset(&p, 0, sizeof(p));
  p.x = ref(x_in);
  p.y = x_out->data;
  p.ysB = x_out->sB;
  p.ysH = x_out->sH;
  p.ysS = x_out->sS;
  p.B = (int32_t)x_in->B;
  p.H = (int32_t)x_in->H;
  p.D = (int32_t)x_in->D;
  p.S = x_in->S;
  p.f32 = x_in->dtype == STAR_F32;
  p.pos = pos;
  p.pos0 = pos0;
  fill_inv_freq(p.inv_freq, x_in->D, base);
  return hip_status(star::launch_rope(p, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Validation shared by star_kv_append and star_decode_prepare; fills p.
int prepare_append(const star_tensor* k_new, const star_tensor* v_new, const star_tensor* k_cache,
                   const star_tensor* v_cache, int64_t slot0, int64_t pos0, double base,
                   int32_t rope, star::AppendParams& p) {
  int s;
  if ((s = check_tensor(k_new, false)) != STAR_OK) return s;
  if ((s = check_tensor(v_new, false)) != STAR_OK) return s;
  if ((s = check_tensor(k_cache, false)) != STAR_OK) return s;
  if ((s = check_tensor(v_cache, false)) != STAR_OK) return s;
  const int64_t B = k_new->B, H = k_new->H, T = k_new->S, D = k_new->D;
  if (v_new->B != B || v_new->H != H || v_new->S != T || v_new->D != D) return STAR_ERR_SHAPE;
  if (k_cache->B != B || k_cache->H != H || k_cache->D != D) return STAR_ERR_SHAPE;
  if (v_cache->B != B || v_cache->H != H || v_cache->D != D || v_cache->S != k_cache->S)
    return STAR_ERR_SHAPE;
  if (!rope_dim_ok(D)) return STAR_ERR_UNSUPPORTED;
  if (slot0 < 0 || pos0 < 0 || slot0 + T > k_cache->S) return STAR_ERR_SHAPE;
  if (rope && (!(base > 1.0) || !std::isfinite(base))) return STAR_ERR_SHAPE;
  if (B > 65535 || H > 65535) return STAR_ERR_UNSUPPORTED;
  std::memset(&p, 0, sizeof(p));
  p.kn = ref(k_new);
  p.vn = ref(v_new);
  p.kc = k_cache->data;
  p.vc = v_cache->data;
  p.kcsB = k_cache->sB; p.kcsH = k_cache->sH; p.kcsS = k_cache->sS;
  p.vcsB = v_cache->sB; p.vcsH = v_cache->sH; p.vcsS = v_cache->sS;
  p.B = (int32_t)B;
  p.H = (int32_t)H;
  p.D = (int32_t)D;
  p.T = T;
  p.slot0 = slot0;
  p.pos0 = pos0;
  p.rope = rope != 0;
  if (rope) fill_inv_freq(p.inv_freq, D, base);
  return STAR_OK;
}

}  // namespace

extern "C" {

int star_kv_append(const star_tensor* k_new, const star_tensor* v_new, const star_tensor* k_cache,
                   const star_tensor* v_cache, int64_t slot0, int64_t pos0, double base,
                   int32_t rope, void* stream) {
  star::AppendParams p;
  const int s = prepare_append(k_new, v_new, k_cache, v_cache, slot0, pos0, base, rope, p);
  if (s != STAR_OK) return s;
  if (p.T == 0) return STAR_OK;
  return hip_status(star::launch_append(p, (hipStream_t)stream));
}

int star_decode_prepare(const star_tensor* q_new, const star_tensor* q_out,
                        const star_tensor* k_new, const star_tensor* v_new,
                        const star_tensor* k_cache, const star_tensor* v_cache, int64_t slot0,
                        int64_t pos0, double base, int32_t rope, void* stream) {
  star::PrepareParams p;
  int s = prepare_append(k_new, v_new, k_cache, v_cache, slot0, pos0, base, rope, p.kv);
  if (s != STAR_OK) return s;
  if ((s = check_tensor(q_new, false)) != STAR_OK) return s;
  if ((s = check_tensor(q_out, false)) != STAR_OK) return s;
  if (q_new->B != k_new->B || q_new->S != k_new->S || q_new->D != k_new->D) return STAR_ERR_SHAPE;
  if (q_out->B != q_new->B || q_out->H != q_new->H || q_out->S != q_new->S ||
      q_out->D != q_new->D)
    return STAR_ERR_SHAPE;
  if (q_new->H < 1 || q_new->H > 65535) return STAR_ERR_UNSUPPORTED;
  if (p.kv.T == 0) return STAR_OK;
  p.qn = ref(q_new);
  p.qo = q_out->data;
  p.qosB = q_out->sB;
  p.qosH = q_out->sH;
  p.qosS = q_out->sS;
  p.Hq = (int32_t)q_new->H;
  return hip_status(star::launch_prepare(p, (hipStream_t)stream));
}

int star_phase1_blocklocal(const star_tensor* q, const star_tensor* k, const star_tensor* v,
                           int64_t block_b, int64_t anchor_len, float scale,
                           const star_tensor* o, float* lse, int32_t* sched, void* stream) {
  int s;
  if ((s = check_phase1(q, k, v, block_b, scale, o, lse, sched)) != STAR_OK) return s;
  if (anchor_len < 0 || anchor_len > block_b) return STAR_ERR_SHAPE;
  if (q->S == 0) return STAR_OK;
  star::FlashParams p;
  phase1_params(p, q, k, v, block_b, scale, o, lse, sched);
  p.pk = p.k;
  p.pv = p.v;
  p.pk_rows = k->S;
  p.a = anchor_len < p.b ? anchor_len : p.b;
  if (block_b >= q->S) p.a = 0;  // a single block has no anchor
  return hip_status(star::launch_flash(p, (hipStream_t)stream));
}

int star_phase1_rope(const star_tensor* q, const star_tensor* k, const star_tensor* v,
                     int64_t block_b, int64_t anchor_len, double base, float scale,
                     const star_tensor* o, float* lse, int32_t* sched, void* stream) {
  int s;
  if ((s = check_phase1(q, k, v, block_b, scale, o, lse, sched)) != STAR_OK) return s;
  if (anchor_len < 0 || anchor_len > block_b) return STAR_ERR_SHAPE;
  if (!std::isfinite(base) || !(base > 1.0)) return STAR_ERR_SHAPE;
  if (q->S == 0) return STAR_OK;
  star::FlashParams p;
  phase1_params(p, q, k, v, block_b, scale, o, lse, sched);
  p.pk = p.k;
  p.pv = p.v;
  p.pk_rows = k->S;
  p.a = anchor_len < p.b ? anchor_len : p.b;
  if (block_b >= q->S) p.a = 0;  // a single block has no anchor
  p.q_rope = 1;
  fill_inv_freq(p.inv_freq, q->D, base);
  // the rotation lives in the bf16, D = 128 kernel only
  if (!star::flash2_supported(p)) return STAR_ERR_UNSUPPORTED;
  return hip_status(star::launch_flash(p, (hipStream_t)stream));
}

int star_phase1_prefix(const star_tensor* q, const star_tensor* k, const star_tensor* v,
                       const star_tensor* pk, const star_tensor* pv,
                       const int64_t* prefix_start, const int64_t* prefix_len, int32_t nblocks,
                       int64_t block_b, float scale, const star_tensor* o, float* lse,
                       int32_t* sched, void* stream) {
  int s;
  if ((s = check_phase1(q, k, v, block_b, scale, o, lse, sched)) != STAR_OK) return s;
  if ((s = check_tensor(pk, true)) != STAR_OK) return s;
  if ((s = check_tensor(pv, true)) != STAR_OK) return s;
  if (pk->dtype != q->dtype || pv->dtype != q->dtype) return STAR_ERR_DTYPE;
  if (pk->B != k->B || pk->H != k->H || pk->D != k->D) return STAR_ERR_SHAPE;
  if (pv->B != k->B || pv->H != k->H || pv->D != k->D || pv->S != pk->S) return STAR_ERR_SHAPE;
  const int64_t n = (q->S + block_b - 1) / block_b;
  if (nblocks != n) return STAR_ERR_SHAPE;
  if (n > STAR_MAX_PARTS) return STAR_ERR_UNSUPPORTED;
  if (n > 0 && (prefix_start == nullptr || prefix_len == nullptr)) return STAR_ERR_NULL;
  for (int64_t i = 0; i < n; ++i) {
    if (prefix_start[i] < 0 || prefix_len[i] < 0) return STAR_ERR_SHAPE;
    if (prefix_len[i] > pk->S - prefix_start[i]) return STAR_ERR_SHAPE;
  }
  if (q->S == 0) return STAR_OK;
  star::FlashParams p;
  phase1_params(p, q, k, v, block_b, scale, o, lse, sched);
  p.pk = ref(pk);
  p.pv = ref(pv);
  p.pk_rows = pk->S;
  p.prefix_tab = 1;
  for (int64_t i = 0; i < n; ++i) {
    p.offs[i] = prefix_start[i];
    p.chunk[i] = prefix_len[i];
  }
  return hip_status(star::launch_flash(p, (hipStream_t)stream));
}

int star_stream_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                     void* stream) {
  if (src == nullptr || out == nullptr) return STAR_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 3) != 0)
    return STAR_ERR_ALIGN;
  if (workgroups < 1 || workgroups > 65536 || bytes <= 0) return STAR_ERR_SHAPE;
  const int64_t unit = star::stream_read_granule() * workgroups;
  if (bytes % unit != 0) return STAR_ERR_SHAPE;
  return hip_status(star::launch_stream_read(src, bytes, workgroups, out,
                                             static_cast<hipStream_t>(stream)));
}

int star_gather_rows(const star_tensor* src, const int64_t* rows, const star_tensor* dst,
                     void* stream) {
  int s;
  if ((s = check_tensor(src, true)) != STAR_OK) return s;
  if ((s = check_tensor(dst, true)) != STAR_OK) return s;
  if (dst->dtype != src->dtype) return STAR_ERR_DTYPE;
  if (dst->B != src->B || dst->H != src->H || dst->D != src->D) return STAR_ERR_SHAPE;
  if ((src->D * esize(src->dtype)) % 16) return STAR_ERR_ALIGN;
  if (src->D > 1024) return STAR_ERR_UNSUPPORTED;
  if (dst->S == 0) return STAR_OK;
  if (rows == nullptr) return STAR_ERR_NULL;
  star::GatherParams p;
  std::memset(&p, 0, sizeof(p));
  p.src = ref(src);
  p.dst = dst->data;
  p.dsB = dst->sB;
  p.dsH = dst->sH;
  p.dsS = dst->sS;
  p.rows = rows;
  p.src_rows = src->S;
  p.R = dst->S;
  p.B = (int32_t)src->B;
  p.H = (int32_t)src->H;
  p.D = (int32_t)src->D;
  p.f32 = src->dtype == STAR_F32;
  return hip_status(star::launch_gather(p, (hipStream_t)stream));
}

int star_phase2_partial(const star_tensor* q, const star_tensor* k_cache,
                        const star_tensor* v_cache, const int64_t* part_offsets, int32_t P,
                        int32_t splits, int64_t q_pos0, float scale, float* o_part,
                        float* lse_part, void* stream) {
  int s;
  if ((s = check_qkv(q, k_cache, v_cache)) != STAR_OK) return s;
  if (o_part == nullptr || lse_part == nullptr) return STAR_ERR_NULL;
  int64_t chunk[STAR_MAX_PARTS];
  if ((s = check_parts(part_offsets, P, splits, k_cache->S, chunk)) != STAR_OK) return s;
  if (q_pos0 < 0) return STAR_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return STAR_ERR_SHAPE;
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(lse_part) & 3u)) return STAR_ERR_ALIGN;
  if (q->S == 0) return STAR_OK;
  const int g = (int)(q->H / k_cache->H);
  if (star::decode_supported(g, q->S, (int)q->D)) {
    star::DecodeParams p;
    decode_params(p, q, k_cache, v_cache, part_offsets, P, splits, chunk, q_pos0, scale, o_part,
                  lse_part);
    return hip_status(star::launch_decode(p, (hipStream_t)stream));
  }
  star::FlashParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = ref(q);
  p.k = ref(k_cache);
  p.v = ref(v_cache);
  p.B = (int32_t)q->B;
  p.Hq = (int32_t)q->H;
  p.Hkv = (int32_t)k_cache->H;
  p.g = g;
  p.D = (int32_t)q->D;
  p.in_f32 = q->dtype == STAR_F32;
  p.q_rows = q->S;
  p.kv_rows = k_cache->S;
  p.pos_shift = q_pos0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.mode = 1;
  p.pk = p.k;            // key range A is empty in Phase 2
  p.pv = p.v;
  p.pk_rows = k_cache->S;
  p.P = P;
  p.splits = splits;
  for (int j = 0; j <= P; ++j) p.offs[j] = part_offsets[j];
  for (int j = 0; j < P; ++j) p.chunk[j] = chunk[j];
  p.lse = lse_part;
  p.opart = o_part;
  return hip_status(star::launch_flash(p, (hipStream_t)stream));
}

}  // extern "C"

namespace star {

// star_decode_step's validation and launches.  With ws_given == false the
// workspace pointers are not checked and nothing is launched (the no-alloc
// entry point validates its arguments before it looks up its scratch).
int decode_step_impl(const star_tensor* q_new, const star_tensor* k_new,
                     const star_tensor* v_new, const star_tensor* k_cache,
                     const star_tensor* v_cache, int64_t slot, int64_t pos, double base,
                     int32_t rope, const int64_t* part_offsets, int32_t P, int32_t splits,
                     float scale, float* o_part, float* lse_part, const star_tensor* o,
                     float* lse, void* stream, bool ws_given, int64_t* pos_dev) {
  int s;
  if ((s = check_qkv(q_new, k_cache, v_cache)) != STAR_OK) return s;
  if ((s = check_tensor(k_new, false)) != STAR_OK) return s;
  if ((s = check_tensor(v_new, false)) != STAR_OK) return s;
  if ((s = check_tensor(o, true)) != STAR_OK) return s;
  if (q_new->dtype != STAR_BF16) return STAR_ERR_DTYPE;
  if (ws_given && (o_part == nullptr || lse_part == nullptr)) return STAR_ERR_NULL;
  if (q_new->S != 1 || k_new->S != 1 || v_new->S != 1) return STAR_ERR_SHAPE;
  for (const star_tensor* t : {k_new, v_new})
    if (t->B != k_cache->B || t->H != k_cache->H || t->D != k_cache->D) return STAR_ERR_SHAPE;
  if (o->B != q_new->B || o->H != q_new->H || o->S != 1 || o->D != q_new->D) return STAR_ERR_SHAPE;
  int64_t chunk[STAR_MAX_PARTS];
  if ((s = check_parts(part_offsets, P, splits, k_cache->S, chunk)) != STAR_OK) return s;
  if (pos_dev != nullptr) {
    // the position is read on the device; the host checks only that the
    // last partition can hold one
    if (reinterpret_cast<uintptr_t>(pos_dev) & 7u) return STAR_ERR_ALIGN;
    if (part_offsets[P - 1] >= part_offsets[P]) return STAR_ERR_SHAPE;
    slot = pos = part_offsets[P - 1];
  }
  // position-contiguous cache: the token's row is its position
  if (slot != pos || slot < part_offsets[0] || slot >= part_offsets[P]) return STAR_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return STAR_ERR_SHAPE;
  if (rope && !(std::isfinite(base) && base > 1.0)) return STAR_ERR_SHAPE;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return STAR_ERR_ALIGN;
  if (!ws_given) return STAR_OK;
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(lse_part) & 3u)) return STAR_ERR_ALIGN;
  star::DecodeParams p;
  decode_params(p, q_new, k_cache, v_cache, part_offsets, P, splits, chunk, pos, scale, o_part,
                lse_part);
  p.fused = 1;
  p.rope = rope != 0;
  p.kn = ref(k_new);
  p.vn = ref(v_new);
  p.slot = slot;
  p.pos_dev = pos_dev;
  p.pos_end = part_offsets[P];
  if (p.rope) fill_inv_freq(p.inv_freq, q_new->D, base);
  if ((s = hip_status(star::launch_decode(p, (hipStream_t)stream))) != STAR_OK) return s;
  // the merge runs as the next launch on the same stream: the kernel
  // boundary makes every workgroup's partial visible to it
  star::MergeParams m;
  std::memset(&m, 0, sizeof(m));
  m.opart = o_part;
  m.lsep = lse_part;
  m.N = P * splits;
  m.R = q_new->B * q_new->H;
  m.D = (int32_t)q_new->D;
  m.H = (int32_t)q_new->H;
  m.S = 1;
  m.o = o->data;
  m.o_f32 = o->dtype == STAR_F32;
  m.osB = o->sB;
  m.osH = o->sH;
  m.osS = o->sS;
  m.lse = lse;
  m.pos_inc = pos_dev;
  return hip_status(star::launch_merge(m, (hipStream_t)stream));
}

}  // namespace star

extern "C" {

int star_decode_step(const star_tensor* q_new, const star_tensor* k_new,
                     const star_tensor* v_new, const star_tensor* k_cache,
                     const star_tensor* v_cache, int64_t slot, int64_t pos, double base,
                     int32_t rope, const int64_t* part_offsets, int32_t P, int32_t splits,
                     float scale, float* o_part, float* lse_part, const star_tensor* o,
                     float* lse, void* stream) {
  return star::decode_step_impl(q_new, k_new, v_new, k_cache, v_cache, slot, pos, base, rope,
                                part_offsets, P, splits, scale, o_part, lse_part, o, lse, stream,
                                true, nullptr);
}

int star_decode_step_devpos(const star_tensor* q_new, const star_tensor* k_new,
                            const star_tensor* v_new, const star_tensor* k_cache,
                            const star_tensor* v_cache, int64_t* pos, double base, int32_t rope,
                            const int64_t* part_offsets, int32_t P, int32_t splits, float scale,
                            float* o_part, float* lse_part, const star_tensor* o, float* lse,
                            void* stream) {
  if (pos == nullptr) return STAR_ERR_NULL;
  return star::decode_step_impl(q_new, k_new, v_new, k_cache, v_cache, 0, 0, base, rope,
                                part_offsets, P, splits, scale, o_part, lse_part, o, lse, stream,
                                true, pos);
}

int star_rmsnorm(const star_tensor* x, const void* gamma, float eps, const star_tensor* y,
                 void* stream) {
  int s;
  if ((s = check_tensor(x, false)) != STAR_OK) return s;
  if ((s = check_tensor(y, false)) != STAR_OK) return s;
  if (gamma == nullptr) return STAR_ERR_NULL;
  if (!aligned16(gamma)) return STAR_ERR_ALIGN;
  if (y->B != x->B || y->H != x->H || y->S != x->S || y->D != x->D) return STAR_ERR_SHAPE;
  if (x->D % 8 != 0 || x->D > 65536) return STAR_ERR_UNSUPPORTED;
  if (!std::isfinite(eps) || eps < 0.f) return STAR_ERR_SHAPE;
  star::RmsParams p;
  std::memset(&p, 0, sizeof(p));
  p.x = ref(x);
  p.y = y->data;
  p.ysB = y->sB;
  p.ysH = y->sH;
  p.ysS = y->sS;
  p.gamma = gamma;
  p.rows = x->B * x->H * x->S;
  p.S = x->S;
  p.H = (int32_t)x->H;
  p.D = (int32_t)x->D;
  p.eps = eps;
  return hip_status(star::launch_rmsnorm(p, (hipStream_t)stream));
}

int star_lse_merge(const float* o_part, const float* lse_part, int32_t N, int64_t B,
                   int64_t Hq, int64_t Lq, int64_t D, const star_tensor* o, float* lse,
                   void* stream) {
  if (o_part == nullptr || lse_part == nullptr) return STAR_ERR_NULL;
  int s;
  if ((s = check_tensor(o, true)) != STAR_OK) return s;
  if (N < 1 || N > 65536) return STAR_ERR_SHAPE;
  if (o->B != B || o->H != Hq || o->S != Lq || o->D != D) return STAR_ERR_SHAPE;
  if (o->D != 64 && o->D != 128) return STAR_ERR_UNSUPPORTED;
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(lse_part) & 3u)) return STAR_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return STAR_ERR_ALIGN;
  const int64_t R = o->B * o->H * o->S;
  if (R == 0) return STAR_OK;
  star::MergeParams p;
  std::memset(&p, 0, sizeof(p));
  p.opart = o_part;
  p.lsep = lse_part;
  p.N = N;
  p.R = R;
  p.D = (int32_t)o->D;
  p.H = (int32_t)o->H;
  p.S = o->S;
  p.o = o->data;
  p.o_f32 = o->dtype == STAR_F32;
  p.osB = o->sB;
  p.osH = o->sH;
  p.osS = o->sS;
  p.lse = lse;
  return hip_status(star::launch_merge(p, (hipStream_t)stream));
}

}  // extern "C"
