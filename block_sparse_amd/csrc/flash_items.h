// Work items of the flash-style attention kernels: which query rows a
// workgroup owns and which key ranges those rows see.
//
// Phase 1 (Pith review of Star Attention, "What carries the argument"): a
// row of block i >= 1 sees the anchor keys [0, a) and its own block's keys
// up to itself; block 1 is causal within itself.  With a prefix table the
// anchor is replaced by any per-block list of rows that all precede the
// block (the anchor ablations of the Star Attention pages; Pulsar's sink and
// summaries, Pith review of Pulsar Attention, "What carries the argument").
// Phase 2: each chunk of a KV partition is one key range, visible to a row
// up to its position.
#pragma once

#include "common.h"
#include "internal.h"

namespace star {

struct Item {
  int b, kvh, hg;
  int64_t qr0, qr_end;   // first q row of the tile, end of valid q rows
  int64_t ra0, ra1;      // key range A (the anchor; may be empty)
  int64_t rb0, rb1;      // key range B (own block / Phase-2 chunk)
  int cs;                // Phase-2 chunk index
};

__device__ __forceinline__ void flash_get_item(const FlashParams& p, int lid, Item& it) {
  if (p.mode == 0) {
    const int T_tot = (p.nblocks >= 2)
                          ? (p.nblocks - 2) * p.nqt_full + p.nqt_last + p.nqt0
                          : p.nqt0;
    const int grp = lid / T_tot;
    const int t = lid - grp * T_tot;
    it.hg = grp % p.hgroups;
    const int r = grp / p.hgroups;
    it.kvh = r % p.Hkv;
    it.b = r / p.Hkv;
    // heavy tiles first: blocks 2..n (anchor + long causal prefix), the
    // last q tile of each block first; block 1 (no anchor) last.
    int blk, j;
    if (p.nblocks == 1) {
      blk = 0;
      j = p.nqt0 - 1 - t;
    } else {
      const int nmid = (p.nblocks - 2) * p.nqt_full;
      if (t < nmid) {
        blk = 1 + t / p.nqt_full;
        j = p.nqt_full - 1 - (t - (blk - 1) * p.nqt_full);
      } else if (t < nmid + p.nqt_last) {
        blk = p.nblocks - 1;
        j = p.nqt_last - 1 - (t - nmid);
      } else {
        blk = 0;
        j = p.nqt0 - 1 - (t - nmid - p.nqt_last);
      }
    }
    const int64_t bs = (int64_t)blk * p.b;
    const int64_t be = min(bs + p.b, p.L);
    it.qr0 = bs + (int64_t)j * p.m_pos;
    it.qr_end = be;
    if (p.prefix_tab) {
      it.ra0 = p.offs[blk];
      it.ra1 = p.offs[blk] + p.chunk[blk];
    } else {
      it.ra0 = 0;
      it.ra1 = (blk > 0) ? p.a : 0;
    }
    it.rb0 = bs;
    it.rb1 = be;
    it.cs = 0;
  } else {
    const int per = p.P * p.splits * p.nqt2;
    const int grp = lid / per;
    const int t = lid - grp * per;
    it.hg = grp % p.hgroups;
    const int r = grp / p.hgroups;
    it.kvh = r % p.Hkv;
    it.b = r / p.Hkv;
    const int qt = t % p.nqt2;
    const int cs = t / p.nqt2;
    const int part = cs / p.splits, sp = cs - part * p.splits;
    const int64_t c0 = p.offs[part] + (int64_t)sp * p.chunk[part];
    const int64_t c1 = min(c0 + p.chunk[part], p.offs[part + 1]);
    it.qr0 = (int64_t)qt * p.m_pos;
    it.qr_end = p.q_rows;
    it.ra0 = it.ra1 = 0;
    it.rb0 = c0;
    it.rb1 = c1 > c0 ? c1 : c0;
    it.cs = cs;
  }
}

// Host side: workgroup geometry and item count for NCB column blocks (of 32
// query rows) per workgroup.  Returns false if the grid would not fit.
inline bool flash_geometry(FlashParams& p, int NCB) {
  p.gw = p.g < NCB ? p.g : NCB;
  p.npg = NCB / p.gw;
  p.hgroups = (p.g + p.gw - 1) / p.gw;
  p.m_pos = 32 * p.npg;
  int64_t items;
  if (p.mode == 0) {
    p.nblocks = (int32_t)((p.L + p.b - 1) / p.b);
    p.nqt_full = (int32_t)((p.b + p.m_pos - 1) / p.m_pos);
    const int64_t last = p.L - (int64_t)(p.nblocks - 1) * p.b;
    p.nqt_last = (int32_t)((last + p.m_pos - 1) / p.m_pos);
    p.nqt0 = (p.nblocks == 1) ? p.nqt_last : p.nqt_full;
    const int64_t per = (p.nblocks >= 2)
                            ? (int64_t)(p.nblocks - 2) * p.nqt_full + p.nqt_last + p.nqt0
                            : p.nqt0;
    items = per * p.B * p.Hkv * p.hgroups;
  } else {
    p.nqt2 = (int32_t)((p.q_rows + p.m_pos - 1) / p.m_pos);
    items = (int64_t)p.P * p.splits * p.nqt2 * p.B * p.Hkv * p.hgroups;
  }
  if (items < 0 || items > 0x7fffffff) return false;
  p.total_items = (int32_t)items;
  return true;
}

}  // namespace star
