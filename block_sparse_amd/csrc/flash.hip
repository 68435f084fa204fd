// Flash-style attention on gfx950 bf16 MFMA for Phase 1 (anchor-block
// blockwise-local causal attention) and for Phase-2 query-chunk partials.
//
// Phase 1 (Pith review of Star Attention, "What carries the argument"):
// a row at position p of block i >= 1 attends to the anchor keys [0, a) and
// to its own block's keys up to p; block 1 is plain causal attention.  The
// anchor's K/V are block 1's K/V, read in place (or, with a prefix table,
// any rows of a separate pk/pv pair).  Phase 2 (same review, "Circularity
// Check"): every KV chunk yields a local output and lse.  Both are written
// as "q rows against <= 2 key ranges: every key of range A, and the keys of
// range B up to the row's position", so one kernel serves both.  The mask is analytic: only tiles that cross a range end or
// the diagonal evaluate it.
//
// Work decomposition.  One workgroup = NW waves; wave w owns CB column
// blocks of 32 query rows.  A workgroup covers up to 8 query heads of one
// KV head (GQA heads share every K/V tile it loads) times 32*npg positions.
// Per 64-key tile the workgroup stages K (row-major) and V (transposed,
// keys permuted inside 16-key groups) in LDS, double-buffered with a
// register prefetch of the next tile.  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (rows = keys, so a lane owns one query column:
// the row max/sum are lane-local plus one cross-half exchange), then
// P^T = exp2(S^T*c - m), and O^T += V^T P^T, where P^T is fed straight
// from the S^T accumulator registers as the B operand.  The running max is
// rescaled lazily: O is only rescaled when the max grows by more than 2^8.
#include "common.h"
#include "internal.h"
#include "flash_items.h"


namespace star {
namespace {

constexpr int KT = 64;                    // keys per LDS tile
constexpr float kRescaleLog2 = 8.0f;      // lazy-rescale threshold (log2)

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  constexpr int NCH = D / 8;
  return r * (D * 2) + ((c ^ (r & (NCH - 1))) << 4);
}

// V^T tile: row d holds 64 key slots (128 B); 16-byte chunks are XOR
// swizzled by row so that 8 consecutive rows hit distinct banks.
__device__ __forceinline__ int vt_chunk_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Inside each 16-key group, physical key 8i + 4h + j is stored at slot
// 8h + 4i + j (bits 2 and 3 swapped): a lane of the PV MFMA then reads its
// eight keys as one 16-byte chunk, in the order its S^T registers hold them.
__device__ __forceinline__ int key_slot(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int NW, int CB, typename T>
__global__ __launch_bounds__(NW * 64) void flash_kernel(const FlashParams p) {
  constexpr int NT = NW * 64;
  constexpr int NCH = D / 8;     // 16-byte chunks per K/V row
  constexpr int NDC = D / 16;    // MFMA k-steps along D
  constexpr int NDB = D / 32;    // 32-row blocks of O^T
  constexpr int KBYTES = KT * D * 2;
  constexpr int K_UNITS = KT * NCH;
  constexpr int K_LOADS = (K_UNITS + NT - 1) / NT;
  constexpr int V_UNITS = (KT / 4) * NCH;   // (4-key group, 8-d chunk)
  constexpr int V_LOADS = (V_UNITS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * KBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  Item it;
  flash_get_item(p, xcd_remap(blockIdx.x, p.total_items), it);

  // ---- positions covered by this workgroup and by this wave
  const int64_t qlast = min(it.qr0 + p.m_pos, it.qr_end) - 1;
  const int64_t pmax = qlast + p.pos_shift;  // largest row position in the WG
  // range A (anchor / prefix) precedes every row: only its source bounds it
  it.ra1 = max(min(it.ra1, p.pk_rows), it.ra0);
  it.rb1 = max(min(min(it.rb1, pmax + 1), p.kv_rows), it.rb0);

  int head[CB];
  bool cb_ok[CB];
  int64_t qrow[CB];
  int64_t wave_min = INT64_MAX, wave_max = -1;
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    const int c = CB * wave + u;
    const int hh = c % p.gw, pg = c / p.gw;
    const int hl = it.hg * p.gw + hh;
    const int64_t r0 = it.qr0 + 32 * pg;
    cb_ok[u] = (pg < p.npg) && (hl < p.g) && (r0 < it.qr_end);
    head[u] = it.kvh * p.g + (hl < p.g ? hl : 0);
    qrow[u] = r0 + l32;
    if (cb_ok[u]) {
      wave_min = min(wave_min, r0 + p.pos_shift);
      wave_max = max(wave_max, min(r0 + 31, it.qr_end - 1) + p.pos_shift);
    }
  }

  // ---- Q^T operands (B operand of S^T = K Q^T) straight to registers
  const T* qbase = reinterpret_cast<const T*>(p.q.data) + (int64_t)it.b * p.q.sB;
  bf16x8 qf[CB][NDC];
  int64_t qpos[CB];
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    const bool ok = cb_ok[u] && qrow[u] < it.qr_end;
    qpos[u] = qrow[u] + p.pos_shift;
    const T* qr = qbase + (int64_t)head[u] * p.q.sH + (ok ? qrow[u] : 0) * p.q.sS;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = Load8<T>::load(qr + 16 * dc + 8 * hf);
      qf[u][dc] = as_bf16x8(v);
    }
  }

  f32x16 oacc[CB][NDB];
  float m2[CB], lsum[CB];
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    m2[u] = -INFINITY;
    lsum[u] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[u][db][r] = 0.f;
  }

  const T* kbase = reinterpret_cast<const T*>(p.k.data) + (int64_t)it.b * p.k.sB +
                   (int64_t)it.kvh * p.k.sH;
  const T* vbase = reinterpret_cast<const T*>(p.v.data) + (int64_t)it.b * p.v.sB +
                   (int64_t)it.kvh * p.v.sH;
  const T* pkbase = reinterpret_cast<const T*>(p.pk.data) + (int64_t)it.b * p.pk.sB +
                    (int64_t)it.kvh * p.pk.sH;
  const T* pvbase = reinterpret_cast<const T*>(p.pv.data) + (int64_t)it.b * p.pv.sB +
                    (int64_t)it.kvh * p.pv.sH;

  const int nt0 = (int)((it.ra1 - it.ra0 + KT - 1) / KT);
  const int nt = nt0 + (int)((it.rb1 - it.rb0 + KT - 1) / KT);

  u32x4 kst[K_LOADS];
  u32x4 vst[V_LOADS][4];

  // tile t -> first key; tiles of range 0 come first, then range 1
  const int64_t ra0 = it.ra0, ra1 = it.ra1, rb0 = it.rb0, rb1 = it.rb1;
  auto tile_start = [&](int t) -> int64_t {
    return t < nt0 ? ra0 + (int64_t)KT * t : rb0 + (int64_t)KT * (t - nt0);
  };

  auto issue_loads = [&](int t) {
    const bool A = t < nt0;
    const int64_t kt = tile_start(t);
    // keys past the range end are zero-filled, never read: they may be
    // unwritten memory (0 * NaN in the PV product would poison the output)
    const int64_t rows = A ? ra1 : rb1;
    const T* kbs = A ? pkbase : kbase;
    const T* vbs = A ? pvbase : vbase;
    const int64_t kss = A ? p.pk.sS : p.k.sS;
    const int64_t vss = A ? p.pv.sS : p.v.sS;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int idx = tid + i * NT;
      kst[i] = u32x4{0, 0, 0, 0};
      if (idx < K_UNITS) {
        const int r = idx / NCH, c = idx % NCH;
        const int64_t key = kt + r;
        if (key < rows) kst[i] = Load8<T>::load(kbs + key * kss + 8 * c);
      }
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int u = tid + i * NT;
#pragma unroll
      for (int e = 0; e < 4; ++e) vst[i][e] = u32x4{0, 0, 0, 0};
      if (u < V_UNITS) {
        const int kg = u / NCH, dc = u % NCH;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t key = kt + 4 * kg + e;
          if (key < rows) vst[i][e] = Load8<T>::load(vbs + key * vss + 8 * dc);
        }
      }
    }
  };

  auto store_lds = [&](int buf) {
    uint8_t* kb = smem + buf * KBYTES;
    uint8_t* vb = smem + 2 * KBYTES + buf * KBYTES;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int idx = tid + i * NT;
      if (idx < K_UNITS) {
        const int r = idx / NCH, c = idx % NCH;
        *reinterpret_cast<u32x4*>(kb + k_off<D>(r, c)) = kst[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int u = tid + i * NT;
      if (u < V_UNITS) {
        const int kg = u / NCH, dc = u % NCH;
        const int slot = key_slot(4 * kg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * dc + e;
          const int w = e >> 1;
          uint32_t x0, x1, x2, x3;
          if (e & 1) {
            x0 = vst[i][0][w] >> 16; x1 = vst[i][1][w] & 0xffff0000u;
            x2 = vst[i][2][w] >> 16; x3 = vst[i][3][w] & 0xffff0000u;
          } else {
            x0 = vst[i][0][w] & 0xffffu; x1 = vst[i][1][w] << 16;
            x2 = vst[i][2][w] & 0xffffu; x3 = vst[i][3][w] << 16;
          }
          u32x2 pk = {x0 | x1, x2 | x3};
          const int off = d * (KT * 2) + (((slot >> 3) ^ vt_chunk_swz(d)) << 4) + ((slot & 7) << 1);
          *reinterpret_cast<u32x2*>(vb + off) = pk;
        }
      }
    }
  };

  const float c2 = p.scale_log2;

  if (nt > 0) {
    issue_loads(0);
    store_lds(0);
  }
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int64_t kt = tile_start(t);
    if (t + 1 < nt) issue_loads(t + 1);
    const int buf = t & 1;
    const uint8_t* kb = smem + buf * KBYTES;
    const uint8_t* vb = smem + 2 * KBYTES + buf * KBYTES;
    const int64_t rend = t < nt0 ? ra1 : rb1;

    const bool A = t < nt0;       // range A: no position limit
    if ((A && wave_max >= 0) || kt <= wave_max) {
      const bool need_mask = (kt + KT > rend) || (!A && kt + KT - 1 > wave_min);
      // mask limits relative to the tile start, as 32-bit ints
      const int lim_end = (int)min(rend - kt, (int64_t)KT);
      int lim_pos[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u)
        lim_pos[u] = A ? KT : (int)max(min(qpos[u] - kt, (int64_t)KT), (int64_t)-1);
#pragma unroll 1
      for (int kb2 = 0; kb2 < KT / 32; ++kb2) {
        f32x16 s[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[u][r] = 0.f;
        const int krow = 32 * kb2 + l32;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + k_off<D>(krow, 2 * dc + hf));
#pragma unroll
          for (int u = 0; u < CB; ++u) s[u] = mfma32(a, qf[u][dc], s[u]);
        }
        if (need_mask) {
#pragma unroll
          for (int u = 0; u < CB; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = 32 * kb2 + 8 * (r >> 2) + 4 * hf + (r & 3);
              if (key >= lim_end || key > lim_pos[u]) s[u][r] = -INFINITY;
            }
        }
        bf16x8 pf[CB][2];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
          float mt = s[u][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[u][r]);
          mt = fmaxf(mt, __shfl_xor(mt, 32));
          const float mt2 = mt * c2;
          const bool need = mt2 > m2[u] + kRescaleLog2;
          if (__any(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m2[u] - mt2) : 1.0f;
            if (need) m2[u] = mt2;
            lsum[u] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[u][db][r] *= alpha;
          }
          const float msub = (m2[u] == -INFINITY) ? 0.f : m2[u];
          float pv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][r], c2, -msub));
            lsum[u] += pv[r];
          }
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            bf16x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (__bf16)pv[8 * cc + e];
            pf[u][cc] = x;
          }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + l32;
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const int chunk = 2 * (2 * kb2 + cc) + hf;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                vb + d * (KT * 2) + ((chunk ^ vt_chunk_swz(d)) << 4));
#pragma unroll
            for (int u = 0; u < CB; ++u) oacc[u][db] = mfma32(a, pf[u][cc], oacc[u][db]);
          }
        }
      }
    }
    if (t + 1 < nt) store_lds(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and write
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    const float lt = lsum[u] + __shfl_xor(lsum[u], 32);
    const bool ok = cb_ok[u] && qrow[u] < it.qr_end;
    if (!ok) continue;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const float lse = lt > 0.f ? (m2[u] + __log2f(lt)) * kLn2 : -INFINITY;
    if (p.mode == 0) {
      __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)it.b * p.osB +
                     (int64_t)head[u] * p.osH + qrow[u] * p.osS;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * db + 8 * i + 4 * hf;
          u32x2 w = {pack_bf16(oacc[u][db][4 * i] * inv, oacc[u][db][4 * i + 1] * inv),
                     pack_bf16(oacc[u][db][4 * i + 2] * inv, oacc[u][db][4 * i + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      if (p.lse != nullptr && hf == 0)
        p.lse[((int64_t)it.b * p.Hq + head[u]) * p.L + qrow[u]] = lse;
    } else {
      const int64_t row = (((int64_t)it.cs * p.B + it.b) * p.Hq + head[u]) * p.q_rows + qrow[u];
      float* orow = p.opart + row * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * db + 8 * i + 4 * hf;
          f32x4 w = {oacc[u][db][4 * i] * inv, oacc[u][db][4 * i + 1] * inv,
                     oacc[u][db][4 * i + 2] * inv, oacc[u][db][4 * i + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + d0) = w;
        }
      if (hf == 0) p.lse[row] = lse;
    }
  }
}

template <int D, int NW, int CB>
hipError_t launch_cfg(FlashParams& p, hipStream_t stream) {
  if (!flash_geometry(p, NW * CB)) return hipErrorInvalidValue;
  if (p.total_items == 0) return hipSuccess;
  if (p.in_f32)
    hipLaunchKernelGGL((flash_kernel<D, NW, CB, float>), dim3(p.total_items), dim3(NW * 64), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((flash_kernel<D, NW, CB, __bf16>), dim3(p.total_items), dim3(NW * 64), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

// bf16 inputs with D = 128 take the flash2 kernel; fp32 inputs (rounded to
// bf16 on load) and D = 64 take this one.
hipError_t launch_flash(FlashParams& p, hipStream_t stream) {
  if (flash2_supported(p)) return launch_flash2(p, stream);
  if (p.D == 128) return launch_cfg<128, 8, 1>(p, stream);
  return launch_cfg<64, 8, 1>(p, stream);
}

}  // namespace star
