// gfx950 flash kernel for bf16 Q/K/V with head dim 128: Phase 1 (anchor
// block + own block, causal) and Phase-2 query-chunk partials.
//
// Same work decomposition and math as flash.hip (see flash_items.h for the
// key ranges each row sees: Pith review of Star Attention, "What carries
// the argument" and "Circularity Check"), re-planned around the costs the
// hardware counters showed: the plain fp32 VALU work of the softmax (max,
// scale, row sums, conversions) does not overlap the MFMAs of its SIMD on
// this chip (only the exps do), so every VALU instruction that is not
// softmax arithmetic is removed, and so is the row max of the common path.
//  * K and V tiles go global -> LDS with global_load_lds_dwordx4 from a
//    scalar base plus a fixed per-lane offset: no staging registers, no
//    ds_write, and per tile only a 64-bit scalar add per base (tiles load in
//    order, so the loader advances running pointers).  A wave's load writes 1 KiB
//    of LDS at consecutive addresses, so the chunk swizzle (see swz) is done
//    by permuting the global source addresses instead.
//  * V stays row-major in LDS; the V^T operand of the PV MFMA is read with
//    ds_read_b64_tr_b16, which transposes 4x4 blocks of 16-bit values
//    across each 16-lane group.
//  * every LDS address is a per-lane register plus an immediate below
//    64 KiB: the tile loop is unrolled over the three buffers, the K tiles
//    and the V tiles sit in two arrays (48 KiB each with 64-key tiles), and
//    each array's address is folded into the per-lane registers, so no LDS
//    read needs an add.
//  * which sub-tiles need the causal / range-end mask is decided from two
//    32-bit thresholds computed once (64-bit compares would go to the VALU).
//  * lazy online softmax tested after the fact: P_j is formed with the
//    current shift, and the lane's sum of its 16 values (needed for the
//    denominator anyway) exceeding 2^8 is the sign that some score passed
//    the shift by more than 8 (log2 units).  Only then is the column max
//    formed (IEEE maximum, v_maximum3_f32: no canonicalisation of the MFMA
//    results), O rescaled and P_j recomputed.  Per 32 keys a wave issues
//    16 MFMAs and 57 other VALU instructions (16 FMA, 16 exp, 16 adds,
//    8 packs, 1 compare).
//  * each step's softmax and next QK MFMAs run at a raised wave priority
//    (s_setprio), the PV MFMAs at the normal one: the two waves of a SIMD
//    then tend to alternate, one's VALU work beside the other's MFMAs
//    (1.8-2.7% faster at 8B-128K than without, same box).  Half of the
//    V^T operands of the PV are read at the start of the step, before the
//    softmax, so the first PV MFMAs find them in registers (another ~1%).
//  * the softmax denominator is summed from the fp32 P before it is rounded
//    to bf16 for the PV MFMA (summing the rounded P would move the lse by up
//    to 2^-9 relative).
//  * with q_rope the kernel rotates Q itself in its prologue, under the
//    first tile loads (per lane, or from a per-workgroup cos/sin table when
//    4 or more query heads share the workgroup's positions).
//  * work items come in a fixed XCD-aware order, or, with a scheduling
//    workspace, from per-XCD queues (sched_grab), so that XCDs running at
//    a higher clock take over the slower ones' remaining items.
// One workgroup = 8 waves, one 32-row column block each; 64-key tiles in
// three LDS buffers (one tile computing, one landing, one free); two waves
// share a SIMD, so one's LDS reads, barrier waits and exps run under the
// other's MFMAs.  Phase-2 query items with at most 4 column blocks run a
// 4-wave instance with 32-key tiles instead: two of its workgroups share a
// CU, so the second wave of a SIMD comes from the other workgroup.
#include "common.h"
#include "internal.h"
#include "flash_items.h"
#include "rope_math.h"

#include <type_traits>

namespace star {
namespace {

constexpr int D = 128;
constexpr int ROWB = D * 2;                 // bytes per K/V row
constexpr float kRescaleLog2 = 8.0f;
constexpr float kRescaleP = 256.0f;          // 2^kRescaleLog2

// s_waitcnt vmcnt(4): all but this wave's last 4 vector-memory ops done
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4] = 7, lgkmcnt[11:8] = 15).
__device__ __forceinline__ void wait_vm_keep4() { __builtin_amdgcn_s_waitcnt(0x0F74); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16-byte chunk c of LDS row r is stored at chunk c ^ swz(r & 15).  swz
// takes the 4-row groups a transpose read touches (rows 4i..4i+3, two or
// four adjacent chunks each) and the 16 rows a K read touches (one chunk
// each) onto distinct banks, whether the LDS has 32 or 64 4-byte banks.
__device__ __forceinline__ int swz(int r) {
  const int k = r & 3;
  const int g = (k << 1) | ((k ^ (k >> 1)) & 1);
  return (2 * g) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// global -> LDS DMA of 16 bytes per lane from base + off (base scalar, off
// a per-lane 32-bit byte offset): lane i's bytes land at LDS address
// lds + 16 i.  Issued from inline asm (inputs only: the offset VGPR and
// base SGPRs are read at issue, M0 is set in the same block) so that the
// compiler does not treat it as a possibly-aliasing LDS store and wait for
// it before every later LDS read; the kernel waits for it explicitly
// (vmcnt(0) + barrier) before any wave reads the buffer.
// M0 is a reserved register: the compiler neither saves it around the asm
// nor needs it here (on gfx950 the LDS reads take no M0), so writing it is
// safe as long as the kernel keeps no M0 value of its own; a host test
// checks the generated code for exactly that.  NT sets the nontemporal
// hint, for K/V that no other workgroup reads again.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(p);
}

template <typename T>
__device__ __forceinline__ const __attribute__((address_space(3))) T* lds_ptr(int addr) {
  return (const __attribute__((address_space(3))) T*)(uintptr_t)(uint32_t)addr;
}

__device__ __forceinline__ s16x4 tr_read(int addr) {
#if __HIP_DEVICE_COMPILE__
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(uint32_t)addr);
#else
  (void)addr;
  return s16x4{0, 0, 0, 0};
#endif
}

// Dynamic item order (when the caller passes a scheduling workspace).  The
// items are cut into 8 queues, queue x being the contiguous range the static
// order gives XCD x (heavy first), and sched[x] counts the tickets handed out
// from it.  A workgroup takes the next ticket of its own XCD's queue; once
// that queue is empty it takes one from another queue, so XCDs that run
// faster (their clocks differ by several percent under this load) take over
// the slower ones' remaining items.  Items are independent, so the order
// changes no result; only relaxed atomics are needed.  Returns -1 when every
// queue is empty (the grid holds more workgroups than items).
__device__ __forceinline__ int sched_grab(const FlashParams& p) {
  const int n = p.total_items, base = n >> 3, extra = n & 7;
  // XCC_ID hardware register (hwreg 20, bits 3:0): this XCD's index
  const int xcd = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7;
  auto first = [&](int x) { return x * base + (x < extra ? x : extra); };
  auto count = [&](int x) { return base + (x < extra ? 1 : 0); };
  if (count(xcd) > 0) {
    const int t = atomicAdd(p.sched + xcd, 1);
    if (t < count(xcd)) return first(xcd) + t;
  }
  // own queue empty: read every counter once and take from a non-empty one
  int seen[8];
#pragma unroll
  for (int x = 0; x < 8; ++x)
    seen[x] = __hip_atomic_load(p.sched + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int v = 1; v < 8; ++v) {
    const int x = (xcd + v) & 7;
    if (seen[x] >= count(x)) continue;
    const int t = atomicAdd(p.sched + x, 1);
    if (t < count(x)) return first(x) + t;
  }
  return -1;
}

__global__ void sched_reset_kernel(int32_t* sched) {
  if (threadIdx.x < STAR_SCHED_INTS) sched[threadIdx.x] = 0;
}

// Rotate-half RoPE of this lane's Q fragments whose frequency falls in one
// pass of a cos/sin table in LDS.  The lane holds d = 16 dc + 8 hf + e
// (frequency j = d) in fragment dc and its partner d + 64 in fragment
// dc + 4.  The pass covers frequencies [j0, j0 + FPP); the fp64 (cos, sin)
// of position r (relative to the item's first row) and frequency j0 + i is
// at tab(i, r) = (i < FPP/2 ? tlo : thi) + ((i mod FPP/2) NR + r) 16 bytes.
// Angles and rotation are the RoPE kernel's (rope_math.h), then one
// rounding to bf16, so the rotated Q is bit for bit the one
// star_rope_apply would store.
__device__ __forceinline__ void rope_q_pass(bf16x8* qf, int j0, int FPP, int r, int hf, int NR,
                                            int tlo, int thi) {
  typedef double f64x2 __attribute__((ext_vector_type(2)));
  const int half = FPP >> 1;
#pragma unroll
  for (int dc = 0; dc < 4; ++dc) {
    const int jb = 16 * dc + 8 * hf;              // this fragment's frequencies jb .. jb + 7
    if (jb < j0 || jb >= j0 + FPP) continue;       // wave-uniform unless FPP = 8
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = jb + e - j0;
      const int addr = (i < half ? tlo + i * NR * 16 : thi + (i - half) * NR * 16) + r * 16;
      const f64x2 cs = *lds_ptr<f64x2>(addr);
      double y1, y2;
      rope_rotate64((double)(float)qf[dc][e], (double)(float)qf[dc + 4][e], cs.x, cs.y, y1, y2);
      qf[dc][e] = f64_to_bf16(y1);
      qf[dc + 4][e] = f64_to_bf16(y2);
    }
  }
}

// NW waves, tiles of KT = 32 SUB keys (SUB 32-key sub-tiles each).  The
// instance <8, 2> serves Phase 1 and the Phase-2 query; <4, 1> serves query
// items whose rows fill at most 4 column blocks: with 48 KiB of LDS two of
// its workgroups share a CU, so no wave computes columns without rows.
// Both keep two waves per SIMD: amdgpu_waves_per_eu(2) holds the 4-wave
// instance to the 256 registers that allows (without it the compiler takes
// 284, and only one of its workgroups fits a CU).
template <int NW, int SUB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void flash2_kernel(const FlashParams p) {
  constexpr int KT = 32 * SUB;
  constexpr int TILE = KT * ROWB;             // 16 KiB (SUB = 2), 8 KiB (SUB = 1)
  constexpr int NBUF = 3;                     // LDS tile buffers
  constexpr int CYC = NBUF * SUB;             // sub-tiles per cycle of the buffer ring
  static_assert(NW * 8 == KT && (SUB == 1 || SUB == 2), "each wave loads 8 rows of a tile");
  // tile buffer b: K rows at smK + b TILE, V rows at smV + b TILE
  __shared__ __attribute__((aligned(1024))) uint8_t smK[NBUF * TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t smV[NBUF * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  int lid;
  if (p.sched != nullptr) {
    __shared__ int s_item;
    if (tid == 0) s_item = sched_grab(p);
    __syncthreads();
    lid = __builtin_amdgcn_readfirstlane(s_item);
    if (lid < 0) return;
  } else {
    lid = xcd_remap(blockIdx.x, p.total_items);
  }
  Item it;
  flash_get_item(p, lid, it);

  const int64_t qlast = min(it.qr0 + p.m_pos, it.qr_end) - 1;
  const int64_t pmax = qlast + p.pos_shift;
  // range A (anchor / prefix) precedes every row: only its source bounds it
  it.ra1 = max(min(it.ra1, p.pk_rows), it.ra0);
  it.rb1 = max(min(min(it.rb1, pmax + 1), p.kv_rows), it.rb0);

  // this wave's column block: 32 consecutive positions of one query head
  const int hh = wave % p.gw, pg = wave / p.gw;
  const int hl = it.hg * p.gw + hh;
  const int64_t r0 = it.qr0 + 32 * pg;
  const bool cb_ok = (pg < p.npg) && (hl < p.g) && (r0 < it.qr_end);
  const int head = it.kvh * p.g + (hl < p.g ? hl : 0);
  const int64_t qrow = r0 + l32;
  const bool row_ok = cb_ok && qrow < it.qr_end;
  const int64_t wave_min = r0 + p.pos_shift;
  const int64_t wave_max = cb_ok ? min(r0 + 31, it.qr_end - 1) + p.pos_shift : -1;
  const int64_t qpos = qrow + p.pos_shift;

  // Q^T operands (B of S^T = K Q^T): lane (query l32, half hf) holds
  // d = 16dc + 8hf .. +7 (loaded in the prologue, beside the first tile)
  bf16x8 qf[D / 16];

  // ---- per-lane constant LDS offsets
  // K read for S^T: row 32kb + l32, logical chunk 2dc + hf
  int kofs[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    kofs[dc] = (int)lds_u32(smK) + l32 * ROWB + (((2 * dc + hf) ^ swz(l32)) << 4);
    asm("" : "+v"(kofs[dc]));   // keep the array address in the register
  }
  // V^T via transpose reads: 16-lane group G = lane >> 4 (h = G >> 1 selects
  // keys 4h.., gsub = G & 1 selects d 16gsub..), lane j = lane & 15 points at
  // row (8t + 4h + (j >> 2)) and columns 32db + 16gsub + 4(j & 3) .. +3
  int vofs[2][D / 32];
  {
    const int j = lane & 15, G = lane >> 4, h = G >> 1, gsub = G & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rr = 8 * t + 4 * h + (j >> 2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * gsub + ((j & 3) >> 1);
        vofs[t][db] = (int)lds_u32(smV) + rr * ROWB + ((c ^ swz(rr)) << 4) + 8 * (j & 1);
        asm("" : "+v"(vofs[t][db]));
      }
    }
  }

  // ---- direct global -> LDS loads: wave w fills rows 8w .. 8w+7 of the
  // K and V tiles, 4 rows (1 KiB) per instruction.  A lane's byte offset
  // inside a tile is fixed (per key range, as the strides may differ); the
  // tile's base address is scalar, so a full tile costs no VALU work.
  const int64_t ksA = p.pk.sS * 2, vsA = p.pv.sS * 2;     // bytes per row
  const int64_t ksB = p.k.sS * 2, vsB = p.v.sS * 2;
  const uint8_t* kbA = reinterpret_cast<const uint8_t*>(p.pk.data) +
                       ((int64_t)it.b * p.pk.sB + (int64_t)it.kvh * p.pk.sH) * 2 + it.ra0 * ksA;
  const uint8_t* vbA = reinterpret_cast<const uint8_t*>(p.pv.data) +
                       ((int64_t)it.b * p.pv.sB + (int64_t)it.kvh * p.pv.sH) * 2 + it.ra0 * vsA;
  const uint8_t* kbB = reinterpret_cast<const uint8_t*>(p.k.data) +
                       ((int64_t)it.b * p.k.sB + (int64_t)it.kvh * p.k.sH) * 2 + it.rb0 * ksB;
  const uint8_t* vbB = reinterpret_cast<const uint8_t*>(p.v.data) +
                       ((int64_t)it.b * p.v.sB + (int64_t)it.kvh * p.v.sH) * 2 + it.rb0 * vsB;
  // rows of each range (already clamped to its source tensor): a tile row
  // past the range end re-reads the range's last row (masked later), so no
  // row outside the range is ever read -- it may be unwritten memory, and
  // 0 * NaN in the PV product would poison the output
  const int64_t rowsA = it.ra1 - it.ra0, rowsB = it.rb1 - it.rb0;
  int lrow[2], lcolb[2];
  uint32_t okA[2], ovA[2], okB[2], ovB[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lrow[i] = 8 * wave + 4 * i + (lane >> 4);
    lcolb[i] = 16 * ((lane & 15) ^ swz(lrow[i]));
    okA[i] = (uint32_t)(lrow[i] * ksA + lcolb[i]);
    ovA[i] = (uint32_t)(lrow[i] * vsA + lcolb[i]);
    okB[i] = (uint32_t)(lrow[i] * ksB + lcolb[i]);
    ovB[i] = (uint32_t)(lrow[i] * vsB + lcolb[i]);
  }

  const int nt0 = (int)((it.ra1 - it.ra0 + KT - 1) / KT);
  const int nt = nt0 + (int)((it.rb1 - it.rb0 + KT - 1) / KT);
  const int nsub = SUB * nt;                      // 32-key sub-tiles

  // Tiles are loaded in order, range A's then range B's.  The loader keeps
  // the next tile's K and V row pointers (advanced by one 64-bit add per
  // tile), the strides and lane offsets of its range, the number of tiles
  // left in the range and how many of them lie wholly inside the range.
  // Rows past the range's end (last tile only) are clamped to its last row
  // and masked later.
  const uint8_t* lk = kbA;
  const uint8_t* lv = vbA;
  int64_t lks = ksA, lvs = vsA, lrows = rowsA;
  uint32_t lok[2] = {okA[0], okA[1]}, lov[2] = {ovA[0], ovA[1]};
  int lleft = nt0;
  int lfull = (int)min((int64_t)nt0, rowsA / KT);
  bool in_a = true;
  auto to_range_b = [&]() {
    lk = kbB;
    lv = vbB;
    lks = ksB;
    lvs = vsB;
    lrows = rowsB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lok[i] = okB[i];
      lov[i] = ovB[i];
    }
    lleft = nt - nt0;
    lfull = (int)min((int64_t)(nt - nt0), rowsB / KT);
    in_a = false;
  };
  if (nt0 == 0) to_range_b();
  // the 4 DMAs of the next tile into buffer buf (every wave issues exactly 4
  // loads per tile: wait_vm_keep4 relies on it).  The 4-wave instance runs
  // only Phase-2 query items, each of which streams its chunk's K/V once
  // from HBM: its loads carry the nontemporal hint (at 8B-1M the query
  // partials then read at 6.4-6.8 TB/s instead of 5.7).  Phase 1 re-reads
  // the anchor's K/V from L2 and the Infinity Cache and keeps plain loads.
  constexpr bool NT = SUB == 1;
  auto load_next = [&](int buf) {
    uint32_t dk[2], dv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int at = buf * TILE + (8 * wave + 4 * i) * ROWB;
      dk[i] = __builtin_amdgcn_readfirstlane(lds_u32(smK + at));
      dv[i] = __builtin_amdgcn_readfirstlane(lds_u32(smV + at));
    }
    if (__builtin_expect(lfull > 0, 1)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        dma16<NT>(lk, lok[i], dk[i]);
        dma16<NT>(lv, lov[i], dv[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t rr = min((int64_t)lrow[i], lrows - 1);
        dma16<NT>(lk, (uint32_t)(rr * lks + lcolb[i]), dk[i]);
        dma16<NT>(lv, (uint32_t)(rr * lvs + lcolb[i]), dv[i]);
      }
    }
    lk += KT * lks;
    lv += KT * lvs;
    lrows -= KT;
    // wave-uniform counters: keep them in scalar registers
    lfull = __builtin_amdgcn_readfirstlane(lfull - 1);
    lleft = __builtin_amdgcn_readfirstlane(lleft - 1);
    if (__builtin_expect(lleft == 0 && in_a, 0)) to_range_b();
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m2 = -INFINITY, lsum = 0.f;
  float msub = 0.f;          // m2 where finite, else 0 (the exp2 shift)
  const float c2 = p.scale_log2;

  // Sub-tile j (32 keys) lives in LDS buffer (j / SUB) % 3, rows 32 (j % SUB) ..
  // The loop below is unrolled over the 3 SUB sub-tiles of one buffer cycle
  // so that every LDS address is a per-lane register plus an immediate.
  auto qk = [&](auto boff) -> f32x16 {
    constexpr int OFF = decltype(boff)::value;
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      s = mfma32(*lds_ptr<bf16x8>(kofs[dc] + OFF), qf[dc], s);
    return s;
  };
  // first key of sub-tile j, relative to the start of its key range, and
  // the range it belongs to
  auto sub_key = [&](int j) -> int64_t {
    const int t = SUB == 2 ? j >> 1 : j;
    return (t < nt0 ? it.ra0 + (int64_t)KT * t : it.rb0 + (int64_t)KT * (t - nt0)) +
           32 * (j & (SUB - 1));
  };
  // keys of sub-tile j past the range end or (range B only) after the row's
  // position -> -inf
  // first sub-tile of each range that needs the mask: range A's sub-tiles
  // reaching past its end; range B's reaching past its end or past the
  // wave's first query position
  const int jmA = (int)((it.ra1 - it.ra0) >> 5);
  int jmB;
  {
    const int64_t xb = wave_min - 31 - it.rb0;
    jmB = SUB * nt0 + (int)min((it.rb1 - it.rb0) >> 5, xb < 0 ? (int64_t)0 : (xb >> 5) + 1);
  }
  auto mask_needed = [&](int j) -> bool { return j >= (j < SUB * nt0 ? jmA : jmB); };
  auto mask = [&](int j, f32x16& s) {
    const bool A = j < SUB * nt0;
    const int64_t ks = sub_key(j);
    const int64_t rend = A ? it.ra1 : it.rb1;
    const int lim_end = (int)min(rend - ks, (int64_t)32);
    const int lim_pos = A ? 32 : (int)max(min(qpos - ks, (int64_t)32), (int64_t)-1);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key >= lim_end || key > lim_pos) s[r] = -INFINITY;
    }
  };
  // column max of S across the lane's 16 keys and the partner half's 16
  auto colmax = [&](const f32x16& sv) -> float {
    float ml = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) ml = __builtin_elementwise_maximum(ml, sv[r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ml), __float_as_uint(ml),
                                                     false, false);
    return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  // P = exp2(S c - msub) of one sub-tile: the bf16 operand of PV, and the
  // sum of the lane's 16 fp32 values (returned)
  auto softmax_p = [&](const f32x16& sv, bf16x8* pf) -> float {
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], c2, -msub));
      ls = e == 0 ? pv : ls + pv;          // (0 + pv would cost an add)
      pf[e >> 3][e & 7] = (__bf16)pv;
    }
    return ls;
  };

  // lane-sum limit that triggers the rescale test: -1 (always) until the
  // column has a finite max, then 2^8
  float plim = -1.f;

  // prologue: tile 0 in flight while Q loads, then tile 1, RoPE, first S
  if (nt > 0) load_next(0);
  {
    // a lane past the last row reads row 0 instead (in bounds; its
    // results are never stored)
    const __bf16* qr = reinterpret_cast<const __bf16*>(p.q.data) + (int64_t)it.b * p.q.sB +
                       (int64_t)head * p.q.sH + (row_ok ? qrow : 0) * p.q.sS;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      qf[dc] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 16 * dc + 8 * hf));
    // complete the Q loads (and tile 0, issued before them) here, so the
    // compiler, which does not count the untracked tile DMAs, has no load of
    // its own left to wait for later
    __builtin_amdgcn_s_waitcnt(0);
  }
  if (nt > 1) load_next(1);
  // RoPE of Q, under the tile loads.  The workgroup's NR = 32 npg positions
  // (32 at g >= 5, 64 at g = 3, 4, up to 256 at g = 1) share each
  // (position, frequency) cos/sin among its waves: it is computed once, in
  // fp64, into a table in the third tile slot (32 KiB, not loaded before the
  // first barrier of the key loop) and read back by every wave of that
  // position.  The table of all 64 frequencies is 16 NR KiB, so it is built
  // and used in passes of FPP = 2048 / NR frequencies.  A pass has 2048
  // entries (i, r) = (frequency, position), entry e = i NR + r; wave w
  // computes entries 256 w + 64 m + lane, m = 0..3.  The frequency of such
  // an entry is wave-uniform for NR >= 64 and takes one of two values for
  // NR = 32, so its loads are scalar ones and the compiler's wait for them
  // does not also wait for the tile DMAs in flight.
  if constexpr (SUB == 2) if (p.q_rope) {
    typedef double f64x2 __attribute__((ext_vector_type(2)));
    const int NR = 32 * p.npg;
    const int FPP = 2048 / NR;
    const int tlo = (int)lds_u32(smK + 2 * TILE), thi = (int)lds_u32(smV + 2 * TILE);
    const int hi32 = (NR == 32) ? (lane >> 5) : 0;
    for (int j0 = 0; j0 < D / 2; j0 += FPP) {
      if (j0 > 0) __syncthreads();                  // every wave done with the last pass
#pragma unroll 1
      for (int m = 0; m < 4; ++m) {
        const int e0 = 256 * wave + 64 * m;         // wave-uniform
        const int i0 = e0 / NR, r0 = e0 - i0 * NR;
        const double th0 = p.inv_freq[j0 + i0];
        const double th1 = p.inv_freq[j0 + min(i0 + 1, FPP - 1)];
        const double th = hi32 ? th1 : th0;
        const int i = i0 + hi32;
        const int r = (NR == 32) ? (lane & 31) : r0 + lane;
        double c, sn;
        rope_cs((double)(it.qr0 + r + p.pos_shift), th, c, sn);
        const int addr = (i < (FPP >> 1) ? tlo + i * NR * 16 : thi + (i - (FPP >> 1)) * NR * 16) +
                         r * 16;
        *(__attribute__((address_space(3))) f64x2*)(uintptr_t)(uint32_t)addr = f64x2{c, sn};
      }
      __syncthreads();
      // (a wave with no column block of its own has no rows to rotate)
      if (cb_ok) rope_q_pass(qf, j0, FPP, 32 * pg + l32, hf, NR, tlo, thi);
    }
  }
  if (nt > 1) wait_vm_keep4(); else __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 s = {};
  if (nsub > 0) {
    s = qk(std::integral_constant<int, 0>{});
    if (mask_needed(0)) mask(0, s);
  }

  // one pipeline step: sub-tile j = CYC c + JJ (buffer JJ / SUB, sub-tile
  // JJ % SUB of it).  On entry s = S_j, masked.
  auto step = [&](auto jjc, int j) {
    constexpr int JJ = decltype(jjc)::value;
    constexpr int CUR = (JJ / SUB) * TILE + (JJ % SUB) * 32 * ROWB;       // this sub-tile
    constexpr int JN = (JJ + 1) % CYC;
    constexpr int NXT = (JN / SUB) * TILE + (JN % SUB) * 32 * ROWB;       // the next one
    const bool more = j + 1 < nsub;
    if constexpr (JJ % SUB == SUB - 1) {
      // the next sub-tile starts a new tile: make it resident, then put the
      // tile after it in flight (its buffer was last read two tiles ago)
      if (more) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int tn = j / SUB + 2;
        if (tn < nt) load_next((JJ / SUB + 2) % NBUF);
      }
    }
    // P_j with the current shift, issued together with the QK MFMAs of
    // S_{j+1} (after the last sub-tile S_{j+1} is unused: its slot may hold
    // stale data).  The wave runs this part at a raised issue priority, so
    // of the two waves of a SIMD the one in its softmax goes ahead while the
    // other is in its PV MFMAs: the two fall into alternating phases.
    bf16x8 pf[2];
    // the V^T operands of the first half of this sub-tile's PV are read
    // first, so that those PV MFMAs need no LDS wait and the reads of the
    // second half complete under them (the sched barrier keeps the early
    // reads here; hoisting all of them, or a quarter or three quarters,
    // measured slower)
    bf16x8 va[D / 32][2];
#pragma unroll
    for (int db = 0; db < D / 64; ++db)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const s16x4 a0 = tr_read(vofs[0][db] + CUR + cc * 16 * ROWB);
        const s16x4 a1 = tr_read(vofs[1][db] + CUR + cc * 16 * ROWB);
        va[db][cc] = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    float ls = softmax_p(s, pf);
    f32x16 sn = qk(std::integral_constant<int, NXT>{});
    __builtin_amdgcn_s_setprio(0);
    // Lazy rescale, tested after the fact: a column whose scores exceed
    // its shift by more than 8 (log2 units) has a P above 2^8, so its lane
    // sum exceeds 2^8.  Only a wave where some lane's sum exceeds plim
    // (or where a column has seen no finite score yet) forms the column max; columns
    // whose max grew by more than 8 rescale O and the row sum and
    // recompute P_j.
    if (__builtin_expect(__any(ls > plim), 0)) {
      const float mt2 = colmax(s) * c2;
      const bool need = mt2 > m2 + kRescaleLog2;
      if (__any(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m2 - mt2) : 1.0f;
        if (need) {
          m2 = mt2;
          msub = mt2;
          plim = kRescaleP;
        }
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        ls = softmax_p(s, pf);
      }
    }
    lsum += ls;
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        if (db >= D / 64) {
          const s16x4 a0 = tr_read(vofs[0][db] + CUR + cc * 16 * ROWB);
          const s16x4 a1 = tr_read(vofs[1][db] + CUR + cc * 16 * ROWB);
          va[db][cc] = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        oacc[db] = mfma32(va[db][cc], pf[cc], oacc[db]);
      }
    if (__builtin_expect(more && mask_needed(j + 1), 0)) mask(j + 1, sn);
    s = sn;
  };

  // whole CYC-sub-tile cycles without an exit in the middle (an exit there
  // makes the compiler materialise the dead loop state of the exit path in
  // every step, stalling on the last MFMA's result), then the remainder
  const int ncyc = nsub / CYC, rem = nsub - CYC * ncyc;
  int j = 0;
  for (int c = 0; c < ncyc; ++c, j += CYC) {
    step(std::integral_constant<int, 0>{}, j);
    step(std::integral_constant<int, 1>{}, j + 1);
    step(std::integral_constant<int, 2>{}, j + 2);
    if constexpr (CYC == 6) {
      step(std::integral_constant<int, 3 % CYC>{}, j + 3);
      step(std::integral_constant<int, 4 % CYC>{}, j + 4);
      step(std::integral_constant<int, 5 % CYC>{}, j + 5);
    }
  }
  if (rem > 0) step(std::integral_constant<int, 0>{}, j);
  if (rem > 1) step(std::integral_constant<int, 1>{}, j + 1);
  if constexpr (CYC == 6) {
    if (rem > 2) step(std::integral_constant<int, 2>{}, j + 2);
    if (rem > 3) step(std::integral_constant<int, 3 % CYC>{}, j + 3);
    if (rem > 4) step(std::integral_constant<int, 4 % CYC>{}, j + 4);
  }

  // ---- epilogue
  const float lt = lsum + __shfl_xor(lsum, 32);
  if (!row_ok) return;
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const float lse = lt > 0.f ? (m2 + log2f(lt)) * kLn2 : -INFINITY;
  if (p.mode == 0) {
    __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)it.b * p.osB +
                   (int64_t)head * p.osH + qrow * p.osS;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * hf;
        u32x2 w = {pack_bf16(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv),
                   pack_bf16(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (p.lse != nullptr && hf == 0) p.lse[((int64_t)it.b * p.Hq + head) * p.L + qrow] = lse;
  } else {
    const int64_t row = (((int64_t)it.cs * p.B + it.b) * p.Hq + head) * p.q_rows + qrow;
    float* orow = p.opart + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * hf;
        f32x4 w = {oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv,
                   oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + d0) = w;
      }
    if (hf == 0) p.lse[row] = lse;
  }
}

}  // namespace

// The tile DMAs address a lane's bytes with a 32-bit offset from a scalar
// base: 64 rows of every source must span less than 2 GiB.
bool flash2_supported(const FlashParams& p) {
  const int64_t lim = (int64_t)1 << 31;
  for (int64_t s : {p.k.sS, p.v.sS, p.pk.sS, p.pv.sS})
    if (s * 2 * 64 >= lim) return false;
  return p.D == 128 && !p.in_f32;
}

hipError_t launch_flash2(FlashParams& p, hipStream_t stream) {
  // Phase-2 query items of at most 4 column blocks (g <= 4 heads x their
  // rows): the 4-wave instance, two workgroups per CU
  const bool small = p.mode == 1 && !p.q_rope && p.g <= 4 && (int64_t)p.g * p.q_rows <= 128;
  const int NW = small ? 4 : 8;
  if (!flash_geometry(p, NW)) return hipErrorInvalidValue;
  if (p.total_items == 0) return hipSuccess;
  int grid = p.total_items;
  if (p.sched != nullptr) {
    // one eighth more workgroups than items: the spare ones serve the XCDs
    // that empty their own queue first, the rest find nothing and exit
    const int spare = ((p.total_items / 8 + 7) / 8) * 8 + 8;
    if (p.total_items > 0x7fffffff - spare) return hipErrorInvalidValue;
    grid += spare;
    hipLaunchKernelGGL(sched_reset_kernel, dim3(1), dim3(64), 0, stream, p.sched);
  }
  if (small)
    hipLaunchKernelGGL((flash2_kernel<4, 1>), dim3(grid), dim3(4 * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((flash2_kernel<8, 2>), dim3(grid), dim3(8 * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace star
