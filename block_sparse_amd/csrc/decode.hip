// Split-KV Phase-2 partials for few query rows per KV head (decode steps).
//
// A generated token attends globally to every cached token; each KV
// partition returns its local output and log-sum-exp (Pith review of Star
// Attention, "Core claim" and "Circularity Check").  With one query token
// the work is a stream over the whole KV cache, so this kernel is built to
// keep HBM busy: one workgroup owns one long chunk of one partition for one
// KV head and all of its g query heads (GQA heads share each K/V byte read),
// its eight waves walk interleaved 32-key tiles of the chunk, and each wave
// keeps its next two tiles in flight in registers while it computes the
// current one.  Long chunks keep the per-workgroup setup and the number of
// partials (and so the merge that follows) small.
//
// Loads: every load instruction of a wave reads 1 KiB of consecutive bytes
// (whole key rows) with the nontemporal hint.  Each K/V byte is read once,
// and on this GPU that form streams at ~7.0-7.1 TB/s against ~6.2 TB/s for
// the MFMA operand layout (16 rows x 64 B per instruction, which with the
// hint falls to ~5.9 TB/s: half-lines evicted before their other half is
// read).  The tile therefore goes through LDS for K as well as V.
//
// Math on v_mfma_f32_16x16x32_bf16 with the g*Lq query rows padded to 16:
// S^T = K Q^T (A = K read back from the wave's LDS copy in operand layout),
// the row max/sum per lane column, then O^T += V^T P^T where V^T is read
// from the LDS copy of the V tile with ds_read_b64_tr_b16 (keys in the
// order the S^T registers hold them) and P^T comes from the S^T registers.
// The waves merge their (m, l, O) in LDS at the end.
#include "common.h"
#include "internal.h"
#include "rope_math.h"

#include <type_traits>

namespace star {
namespace {

constexpr int NWD = 8;      // waves per workgroup
constexpr int64_t kSplitAlign = STAR_SPLIT_ALIGN;
constexpr int KTD = 32;     // keys per wave tile
constexpr float kRescaleLog2 = 8.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ s16x4 tr_read(const uint8_t* p) {
#if __HIP_DEVICE_COMPILE__
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
#else
  (void)p;
  return s16x4{0, 0, 0, 0};
#endif
}

// 16-byte chunk c of K/V-tile row r is stored at chunk c ^ swz(r & 15): the
// 4-row x 2-chunk footprint of a transpose read of V and the 16-row x
// 1-chunk footprint of a K operand read land on distinct banks (32 or 64
// banks of 4 bytes); a row write covers all banks.
__device__ __forceinline__ int swz(int r) {
  const int k = r & 3;
  const int g = (k << 1) | ((k ^ (k >> 1)) & 1);
  return (2 * g) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
}

template <int D>
__device__ __forceinline__ int v_chunk_off(int row, int chunk) {
  return row * (D * 2) + (((chunk ^ swz(row)) & (D / 8 - 1)) << 4);
}

template <int D, typename T, bool FUSED>
__global__ __launch_bounds__(NWD * 64) void decode_kernel(const DecodeParams p) {
  constexpr int NDC = D / 32;   // k-steps of 32 along D
  constexpr int NDB = D / 16;   // 16-row blocks of O^T
  constexpr int VT = KTD * D * 2;
  // per-wave V tiles during the key loop; reused for the final merge
  static_assert(NWD * 16 * D * 4 <= NWD * VT, "merge buffer must fit");
  // per wave: a V tile and a K tile (row-major, chunk-swizzled)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * NWD * VT];
  __shared__ float red_m[NWD][16];
  __shared__ float red_l[NWD][16];
  float (*red_o)[16][D] = reinterpret_cast<float (*)[16][D]>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;       // query row (column of S^T / O^T)
  const int kg = lane >> 4;      // 8-wide k group of the MFMA operands

  const int lid = xcd_remap(blockIdx.x, p.total_items);
  const int nch = p.P * p.splits;
  const int cs = lid % nch;
  const int rr = lid / nch;
  const int kvh = rr % p.Hkv;
  const int b = rr / p.Hkv;
  const int part = cs / p.splits, sp = cs - part * p.splits;
  // the token's position and cache row: kernel arguments, or read from
  // device memory (then the last partition ends right after the token, and
  // a position outside [offs[P-1], pos_end) leaves every chunk empty and
  // writes no cache row)
  int64_t q_pos0 = p.q_pos0, slot = p.slot;
  int64_t part_end = p.offs[part + 1], chunk = p.chunk[part];
  bool pos_ok = true;
  if constexpr (FUSED) {
    if (p.pos_dev != nullptr) {
      const uint64_t raw = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p.pos_dev),
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)raw);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(raw >> 32));
      q_pos0 = slot = (int64_t)(((uint64_t)hi << 32) | lo);
      pos_ok = q_pos0 >= p.offs[p.P - 1] && q_pos0 < p.pos_end;
      if (part == p.P - 1) {
        part_end = q_pos0 + 1;
        const int64_t n = pos_ok ? part_end - p.offs[part] : 0;
        chunk = ((n + p.splits - 1) / p.splits + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
      }
    }
  }
  const int64_t c0 = p.offs[part] + (int64_t)sp * chunk;
  int64_t c1 = min(c0 + chunk, part_end);
  c1 = min(c1, p.kv_rows);
  // rows after the last query position are visible to no row: never read
  // them (they may be cache slots not written yet)
  c1 = min(c1, q_pos0 + p.Lq);
  if (c1 < c0 || !pos_ok) c1 = c0;

  const int nrows = p.g * (int)p.Lq;
  const bool row_ok = n < nrows;
  const int hh = n % p.g;
  const int qi = n / p.g;
  const int head = kvh * p.g + hh;
  const int64_t qpos = q_pos0 + qi;
  const int64_t min_qpos = q_pos0;     // rows are ordered by query index

  if constexpr (FUSED) {
    // the workgroup whose chunk holds the new token's slot appends its K/V
    // row (K rotated like q, one pair per thread) before any of its waves
    // loads the chunk
    if (pos_ok && slot >= c0 && slot < c1) {
      const int half = D / 2;
      const __bf16* kn = reinterpret_cast<const __bf16*>(p.kn.data) + (int64_t)b * p.kn.sB +
                         (int64_t)kvh * p.kn.sH;
      const __bf16* vn = reinterpret_cast<const __bf16*>(p.vn.data) + (int64_t)b * p.vn.sB +
                         (int64_t)kvh * p.vn.sH;
      __bf16* kc = const_cast<__bf16*>(reinterpret_cast<const __bf16*>(p.k.data)) +
                   (int64_t)b * p.k.sB + (int64_t)kvh * p.k.sH + slot * p.k.sS;
      __bf16* vc = const_cast<__bf16*>(reinterpret_cast<const __bf16*>(p.v.data)) +
                   (int64_t)b * p.v.sB + (int64_t)kvh * p.v.sH + slot * p.v.sS;
      if (tid < half) {
        const int j = tid;
        __bf16 y1 = kn[j], y2 = kn[j + half];
        if (p.rope) {
          double c, sn, r1, r2;
          rope_cs((double)q_pos0, p.inv_freq[j], c, sn);
          rope_rotate64((double)(float)kn[j], (double)(float)kn[j + half], c, sn, r1, r2);
          y1 = f64_to_bf16(r1);
          y2 = f64_to_bf16(r2);
        }
        kc[j] = y1;
        kc[j + half] = y2;
      } else if (tid < half + D / 8) {
        const int ch = tid - half;
        *reinterpret_cast<u32x4*>(vc + 8 * ch) = *reinterpret_cast<const u32x4*>(vn + 8 * ch);
      }
      __syncthreads();   // stores complete and visible to this workgroup's loads
    }
  }

  const T* kbase = reinterpret_cast<const T*>(p.k.data) + (int64_t)b * p.k.sB + (int64_t)kvh * p.k.sH;
  const T* vbase = reinterpret_cast<const T*>(p.v.data) + (int64_t)b * p.v.sB + (int64_t)kvh * p.v.sH;

  const int nt = (int)((c1 - c0 + KTD - 1) / KTD);
  // Workgroups start their walk at evenly spread tiles of their chunks.
  // Chunks begin at equally aligned addresses and all workgroups stream at
  // the same rate, so walking them in lockstep would keep hitting the same
  // HBM channels (measured: 3-4% slower per decode step).  Tile order does
  // not change the result beyond rounding: each wave merges its tiles with
  // the online softmax.
  const int rot = nt > 0 ? (int)(((int64_t)lid * nt) / (p.total_items > 0 ? p.total_items : 1)) : 0;
  auto phys = [&](int t) { const int u = t + rot; return u >= nt ? u - nt : u; };
  uint8_t* vs = smem + wave * VT;
  uint8_t* ks = smem + (NWD + wave) * VT;

  // LDS offsets.  Loads and row writes: instruction i of a tile reads 1 KiB
  // contiguous, RPI whole rows; lane -> row i RPI + lane / CPR, chunk
  // lane % CPR.  V transpose reads: 16-lane group kg, lane j: row
  // 16t + 4kg + (j >> 2), columns 16db + 4(j & 3) .. +3.
  // (the swizzle repeats every 16 rows, so instruction i + WP writes at
  // wofs[i % WP] plus a constant)
  constexpr int CPR = D / 8, RPI = 64 / CPR, NLD = KTD / RPI, WP = 16 / RPI;
  constexpr int ROW16 = 16 * D * 2;   // bytes of 16 rows
  int wofs[WP];
#pragma unroll
  for (int i = 0; i < WP; ++i) wofs[i] = v_chunk_off<D>(RPI * i + lane / CPR, lane % CPR);
  // K reads in MFMA operand layout: row 16 kb + n (kb: + ROW16), chunk 4 dc + kg
  int kofs[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) kofs[dc] = v_chunk_off<D>(n, 4 * dc + kg);
  // (rows 16.. of the tile: + ROW16, the swizzle repeating every 16 rows)
  int rofs[NDB];
  {
    const int j = lane & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int row = 4 * kg + (j >> 2);
      const int col = 16 * db + 4 * (j & 3);
      rofs[db] = v_chunk_off<D>(row, col >> 3) + ((col & 7) << 1);
    }
  }

  // register staging, two tiles deep: [slot][load instruction]
  u32x4 kr[2][NLD], vr[2][NLD];
  auto load_tile = [&](int slot, int t) {
    const int64_t kt = c0 + (int64_t)KTD * phys(t);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int64_t key = kt + RPI * i + lane / CPR;
      const int ch = lane % CPR;
      kr[slot][i] = u32x4{0, 0, 0, 0};
      vr[slot][i] = u32x4{0, 0, 0, 0};
      if (key < c1) {
        kr[slot][i] = Load8<T>::load_stream(kbase + key * p.k.sS + 8 * ch);
        vr[slot][i] = Load8<T>::load_stream(vbase + key * p.v.sS + 8 * ch);
      }
    }
  };

  // fused rope: the workgroup rotates its g query rows once, one pair per
  // thread, into an LDS copy that every wave then reads its Q^T operand
  // from.  The raw pairs are loaded before the tile loads, so waiting for
  // them does not wait for the tiles; the barrier waits only for the LDS
  // writes.
  __shared__ __attribute__((aligned(16))) __bf16 q_rot[16 * D];
  constexpr int NPAIR = (16 * (D / 2) + NWD * 64 - 1) / (NWD * 64);   // pairs per thread
  [[maybe_unused]] __bf16 qx1[NPAIR], qx2[NPAIR];
  [[maybe_unused]] double qth[NPAIR];
  const bool rope_q = FUSED && p.rope;
  if (rope_q) {
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      const int idx = tid + NWD * 64 * i, r = idx / (D / 2), j = idx % (D / 2);
      qx1[i] = qx2[i] = (__bf16)0.f;
      qth[i] = p.inv_freq[j];
      if (r < nrows) {
        const __bf16* qr = reinterpret_cast<const __bf16*>(p.q.data) + (int64_t)b * p.q.sB +
                           (int64_t)(kvh * p.g + r % p.g) * p.q.sH + (int64_t)(r / p.g) * p.q.sS;
        qx1[i] = qr[j];
        qx2[i] = qr[j + D / 2];
      }
    }
  }

  // the first two tiles go out before the query is loaded and rotated
  // this wave's tiles: wave, wave + NWD, ...; two in flight at any time
  if (wave < nt) load_tile(0, wave);
  if (wave + NWD < nt) load_tile(1, wave + NWD);

  if (rope_q) {
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      const int idx = tid + NWD * 64 * i, r = idx / (D / 2), j = idx % (D / 2);
      if (r < 16) {
        double c, sn, y1, y2;
        rope_cs((double)(q_pos0 + r / p.g), qth[i], c, sn);
        rope_rotate64((double)(float)qx1[i], (double)(float)qx2[i], c, sn, y1, y2);
        q_rot[r * D + j] = f64_to_bf16(y1);
        q_rot[r * D + j + D / 2] = f64_to_bf16(y2);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // Q^T as the B operand: lane (row n, group kg) holds d = 32dc + 8kg + e.
  bf16x8 qf[NDC];
  if (rope_q) {
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
      qf[dc] = row_ok ? *reinterpret_cast<const bf16x8*>(q_rot + n * D + 32 * dc + 8 * kg)
                      : as_bf16x8(u32x4{0, 0, 0, 0});
  } else {
    const T* qr = reinterpret_cast<const T*>(p.q.data) + (int64_t)b * p.q.sB +
                  (int64_t)(row_ok ? head : 0) * p.q.sH + (int64_t)(row_ok ? qi : 0) * p.q.sS;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      u32x4 v = {0, 0, 0, 0};
      if (row_ok) v = Load8<T>::load(qr + 32 * dc + 8 * kg);
      qf[dc] = as_bf16x8(v);
    }
  }
  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2 = -INFINITY, lsum = 0.f;
  const float c2 = p.scale_log2;

  // one tile held in staging slot SL; the slot is refilled with the tile
  // two steps ahead right after its registers are consumed
  auto process = [&](auto slc, int t) {
    constexpr int SL = decltype(slc)::value;
    const int64_t kt = c0 + (int64_t)KTD * phys(t);
    // stage K and V (row-major, chunk-swizzled) in this wave's LDS regions;
    // the previous tile's reads were issued before these writes, and LDS
    // executes one wave's instructions in order
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int o = wofs[i % WP] + (i / WP) * ROW16;
      *reinterpret_cast<u32x4*>(ks + o) = kr[SL][i];
      *reinterpret_cast<u32x4*>(vs + o) = vr[SL][i];
    }
    asm volatile("" ::: "memory");
    // S^T = K Q^T for two 16-key blocks, K read back in operand layout
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
        s[kb] = mfma16(as_bf16x8(*reinterpret_cast<const u32x4*>(ks + kofs[dc] + kb * ROW16)),
                       qf[dc], s[kb]);
    }
    // refill the staging slot with the tile two steps ahead (after the K
    // operands are read, so they can use the slot's registers)
    asm volatile("" ::: "memory");
    if (t + 2 * NWD < nt) load_tile(SL, t + 2 * NWD);

    // mask: keys past the chunk end or after the row's position
    if (kt + KTD > c1 || kt + KTD - 1 > min_qpos) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t key = kt + 16 * kb + 4 * kg + j;
          if (key >= c1 || key > qpos) s[kb][j] = -INFINITY;
        }
    }
    float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mt2 = mt * c2;
    const bool need = mt2 > m2 + kRescaleLog2;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m2 - mt2) : 1.0f;
      if (need) m2 = mt2;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    const float msub = (m2 == -INFINITY) ? 0.f : m2;
    bf16x8 pt;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][j], c2, -msub));
        lsum += pv;
        pt[4 * kb + j] = (__bf16)pv;
      }
    // O^T += V^T P^T : lane (d = 16db + n, group kg) supplies keys
    // 4kg + e (e < 4) and 16 + 4kg + (e - 4), matching pt's order.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const s16x4 a0 = tr_read(vs + rofs[db]);
      const s16x4 a1 = tr_read(vs + rofs[db] + ROW16);
      const bf16x8 a =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = mfma16(a, pt, oacc[db]);
    }
    asm volatile("" ::: "memory");
  };

  for (int t = wave; t < nt; t += 2 * NWD) {
    process(std::integral_constant<int, 0>{}, t);
    if (t + NWD >= nt) break;
    process(std::integral_constant<int, 1>{}, t + NWD);
  }

  // ---- merge the waves' (m, l, O^T) and write the chunk partial
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // every wave is done with its V tile
  if (kg == 0) {
    red_m[wave][n] = m2;
    red_l[wave][n] = lsum;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) red_o[wave][n][16 * db + 4 * kg + j] = oacc[db][j];
  __syncthreads();

  // thread -> (row, d) pairs
  for (int idx = tid; idx < 16 * D; idx += NWD * 64) {
    const int r = idx / D, d = idx - r * D;
    if (r >= nrows) continue;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWD; ++w) mm = fmaxf(mm, red_m[w][r]);
    float l = 0.f, o = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NWD; ++w) {
        const float al = (red_m[w][r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(red_m[w][r] - mm);
        l += al * red_l[w][r];
        o += al * red_o[w][r][d];
      }
    }
    const int rh = r % p.g, rq = r / p.g;
    const int64_t row = (((int64_t)cs * p.B + b) * p.Hq + (kvh * p.g + rh)) * p.Lq + rq;
    p.opart[row * D + d] = l > 0.f ? o / l : 0.f;
    if (d == 0) p.lse[row] = l > 0.f ? (mm + log2f(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

bool decode_supported(int g, int64_t Lq, int D) {
  return (D == 64 || D == 128) && g >= 1 && Lq >= 1 && (int64_t)g * Lq <= 16;
}

hipError_t launch_decode(DecodeParams& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.B * p.Hkv * p.P * p.splits;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  p.total_items = (int32_t)items;
  const dim3 grid(p.total_items), block(NWD * 64);
  if (p.fused) {
    if (p.in_f32) return hipErrorInvalidValue;
    if (p.D == 128) hipLaunchKernelGGL((decode_kernel<128, __bf16, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((decode_kernel<64, __bf16, true>), grid, block, 0, stream, p);
  } else if (p.D == 128) {
    if (p.in_f32) hipLaunchKernelGGL((decode_kernel<128, float, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((decode_kernel<128, __bf16, false>), grid, block, 0, stream, p);
  } else {
    if (p.in_f32) hipLaunchKernelGGL((decode_kernel<64, float, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((decode_kernel<64, __bf16, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace star
