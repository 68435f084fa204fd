"""Host-side driver of one pass of the two-phase hot path for one layer.

It owns the device buffers (allocated once, resident in HBM) and issues the
library calls in the order the method runs them (Star Attention, pith
review "What carries the argument"; atlas.scime.ai summary "Approach"):

  Phase 1  rope(Q) and rope(K) at original positions (K straight into the
           position-contiguous KV cache), then block-local attention with
           the anchor.  The anchor's KV is never copied: it is block 1's KV
           in the cache, so after Phase 1 the cache holds exactly L entries.
  Phase 2  query tokens: rope(q) at L.., append their K/V to the last
           partition (the query host), partials over every partition and
           the LSE merge.  Then each generated token repeats the same with
           one row, attending to everything cached so far: rope, append and
           partials in one launch per token, then the merge.

Phase-1 variants (same cache afterwards, so Phase 2 is unchanged):
  anchor at other position ids  the anchor's un-rotated keys re-rotated per
           block at given positions (atlas.scime.ai summary, "Measured
           effects reported in the paper");
  Pulsar   a 64-token sink plus the Max-IDF summaries of every earlier block
           at their original positions, gathered from the cache (Pith review
           of Pulsar Attention, "What carries the argument").

All buffers are caller-visible torch tensors; every computation runs in the
library's kernels.
"""
from __future__ import annotations

import math

import torch

from . import (decode_prepare, decode_step, decode_step_devpos, gather_rows, kv_append,
               lse_merge, phase1_blocklocal, phase1_prefix, phase1_rope, phase2_partial,
               pulsar_prefix, rope_apply, sched_workspace)


def partition_offsets(L: int, b: int, cache_len: int):
    """Partition j = block j's cache rows; the last one extends to cache_len."""
    offs = list(range(0, L, b)) + [cache_len]
    return offs


def choose_splits(B: int, Hkv: int, P: int, part_len: int, target_wg: int,
                  min_chunk: int, row_groups: int = 1) -> int:
    """Chunks per partition so that B*Hkv*P*splits*row_groups workgroups
    fill the chip without cutting chunks below ``min_chunk`` keys
    (``row_groups``: workgroups per chunk, one per 256 query rows of a KV
    head in the flash kernel)."""
    want = max(1, math.ceil(target_wg / max(1, B * Hkv * P * row_groups)))
    cap = max(1, math.ceil(part_len / min_chunk))
    return int(min(want, cap, 1024))


class StarAttentionStep:
    """Buffers and call sequence of one Star Attention layer pass."""

    def __init__(self, B, Hq, Hkv, D, L, b, Lq, T, anchor=None, rope=True,
                 base=500000.0, device="cuda", want_lse=True,
                 splits_query=None, splits_decode=None, fused_decode=True,
                 fuse_q_rope=False, dynamic_schedule=True):
        self.B, self.Hq, self.Hkv, self.D = B, Hq, Hkv, D
        self.L, self.b, self.Lq, self.T = L, b, Lq, T
        self.a = b if anchor is None else anchor
        self.rope, self.base = rope, base
        self.scale = 1.0 / math.sqrt(D)
        bf = torch.bfloat16
        S = L + Lq + T
        self.S = S
        dev = torch.device(device)
        self.qr = torch.empty((B, Hq, L, D), dtype=bf, device=dev)
        self.kc = torch.empty((B, Hkv, S, D), dtype=bf, device=dev)
        self.vc = torch.empty((B, Hkv, S, D), dtype=bf, device=dev)
        self.o1 = torch.empty((B, Hq, L, D), dtype=bf, device=dev)
        self.lse1 = torch.empty((B, Hq, L), dtype=torch.float32, device=dev) if want_lse else None
        self.qq_r = torch.empty((B, Hq, max(Lq, 1), D), dtype=bf, device=dev)
        self.qd_r = torch.empty((B, Hq, max(T, 1), D), dtype=bf, device=dev)
        self.o2 = torch.empty((B, Hq, Lq, D), dtype=torch.float32, device=dev)
        self.lse2 = torch.empty((B, Hq, Lq), dtype=torch.float32, device=dev)
        self.od = torch.empty((B, Hq, max(T, 1), D), dtype=torch.float32, device=dev)
        self.lsed = torch.empty((max(T, 1), B, Hq), dtype=torch.float32, device=dev)
        self.P = -(-L // b)
        part_len = min(b, L)
        # query chunks: one workgroup per CU (256 at 8B-128K) -- measured
        # 164 us against 190 us for two rounds of half-length chunks.  With
        # g <= 4 heads of at most 128 rows together (D = 128) the query runs
        # the 4-wave flash instance, two workgroups per CU: 512 of them.
        g = Hq // Hkv
        rows = g * max(Lq, 1)
        two_per_cu = D == 128 and g <= 4 and 16 < rows <= 128
        self.sq = splits_query or choose_splits(B, Hkv, self.P, part_len,
                                                512 if two_per_cu else 256, 512,
                                                1 if rows <= 16 else math.ceil(rows / 256))
        self.sd = splits_decode or choose_splits(B, Hkv, self.P, part_len, 256, 512)
        nq = self.P * self.sq
        nd = self.P * self.sd
        self.op_q = torch.empty((nq, B, Hq, max(Lq, 1), D), dtype=torch.float32, device=dev)
        self.lp_q = torch.empty((nq, B, Hq, max(Lq, 1)), dtype=torch.float32, device=dev)
        self.op_d = torch.empty((nd, B, Hq, 1, D), dtype=torch.float32, device=dev)
        self.lp_d = torch.empty((nd, B, Hq, 1), dtype=torch.float32, device=dev)
        # rope + append + partials in one launch per token (star_decode_step)
        self.fused_decode = fused_decode
        # fuse_q_rope: Phase 1 rotates the context Q itself
        # (star_phase1_rope) instead of a RoPE pass over Q into self.qr
        # before star_phase1_blocklocal.  Both give the same bits; measured
        # at 8B-128K on three boxes, the separate pass plus the attention-only
        # kernel took the same or less time (by 0.2-1.6%), so it is the
        # default.
        self.fuse_q_rope = bool(fuse_q_rope and rope and D == 128)
        # Phase-1 work items from per-XCD queues (the calls of one step run
        # in order on one stream, so one workspace serves them all)
        self.sched = sched_workspace(dev) if dynamic_schedule else None
        self._qraw = None
        self._qr_ok = False

    # -- inputs -----------------------------------------------------------
    def load_context(self, v):
        """Place the context V in the cache (V needs no rotation)."""
        self.vc[:, :, :self.L].copy_(v)

    # -- phases -----------------------------------------------------------
    def rope_context(self, q, k):
        L = self.L
        self._qraw, self._qr_ok = q, False
        if self.rope:
            if not self.fuse_q_rope:
                rope_apply(q, pos0=0, base=self.base, out=self.qr)
                self._qr_ok = True
            rope_apply(k, pos0=0, base=self.base, out=self.kc[:, :, :L])
        else:
            self.qr.copy_(q)
            self._qr_ok = True
            self.kc[:, :, :L].copy_(k)

    def rotated_q(self):
        """The context Q at its positions (made on first use when Phase 1
        rotates Q itself)."""
        if not self._qr_ok:
            rope_apply(self._qraw, pos0=0, base=self.base, out=self.qr)
            self._qr_ok = True
        return self.qr

    def phase1(self):
        L = self.L
        if self.fuse_q_rope:
            phase1_rope(self._qraw, self.kc[:, :, :L], self.vc[:, :, :L], self.b, self.a,
                        self.base, self.scale, out=self.o1, lse=self.lse1, sched=self.sched)
        else:
            phase1_blocklocal(self.qr, self.kc[:, :, :L], self.vc[:, :, :L], self.b, self.a,
                              self.scale, out=self.o1, lse=self.lse1, sched=self.sched)

    def pulsar_setup(self, tokens, m: int = 32, sink: int = 64, k: int = 16):
        """Host-side Max-IDF selection for every sequence (``tokens[B, L]``)
        and device buffers for the gathered prefix rows."""
        self.pulsar = []
        for bb in range(self.B):
            rows, st, ln = pulsar_prefix(tokens[bb], self.L, self.b, m, sink, k)
            R = max(int(rows.size), 1)
            dev = self.qr.device
            rows_d = torch.from_numpy(rows).to(dev)
            pk = torch.empty((1, self.Hkv, R, self.D), dtype=torch.bfloat16, device=dev)
            pv = torch.empty_like(pk)
            self.pulsar.append((rows_d, st, ln, pk, pv))

    def phase1_pulsar(self):
        """Phase 1 with Pulsar's prefix: gather the sink and summary rows of
        the rotated cache, then block-local attention over [prefix ; block]."""
        L = self.L
        qr = self.rotated_q()
        for bb, (rows_d, st, ln, pk, pv) in enumerate(self.pulsar):
            sl = slice(bb, bb + 1)
            if rows_d.numel():
                gather_rows(self.kc[sl, :, :L], rows_d, out=pk)
                gather_rows(self.vc[sl, :, :L], rows_d, out=pv)
            lse = None if self.lse1 is None else self.lse1[sl]
            phase1_prefix(qr[sl], self.kc[sl, :, :L], self.vc[sl, :, :L], pk, pv, st, ln,
                          self.b, self.scale, out=self.o1[sl], lse=lse, sched=self.sched)

    def anchor_remap_setup(self, positions):
        """Buffers for the anchor at other position ids: ``positions[i]``
        (a ids each) are block i's anchor positions (block 0 unused)."""
        n, a = self.P, self.a
        dev = self.qr.device
        self.apos = [torch.as_tensor(p, dtype=torch.int64).to(dev) for p in positions]
        self.apk = torch.empty((self.B, self.Hkv, n * a, self.D), dtype=torch.bfloat16,
                               device=dev)
        self.apv = torch.empty_like(self.apk)
        self.arows = torch.arange(a, dtype=torch.int64, device=dev).repeat(n)
        self.ast = [i * a for i in range(n)]
        self.aln = [0] + [a] * (n - 1)

    def phase1_anchor_remap(self, k_pre):
        """Phase 1 whose anchor keys (``k_pre[..., :a, :]``, un-rotated) are
        rotated at each block's own anchor positions."""
        L, a = self.L, self.a
        for i in range(1, self.P):
            rope_apply(k_pre[:, :, :a], pos=self.apos[i], base=self.base,
                       out=self.apk[:, :, i * a:(i + 1) * a])
        gather_rows(self.vc[:, :, :L], self.arows, out=self.apv)
        phase1_prefix(self.rotated_q(), self.kc[:, :, :L], self.vc[:, :, :L], self.apk, self.apv,
                      self.ast, self.aln, self.b, self.scale, out=self.o1, lse=self.lse1,
                      sched=self.sched)

    def query(self, qq, kq, vq, events=None):
        """The query tokens (inputs [B, H, Lq, D]).  ``events``: an optional
        pair of timing events recorded on the stream right before and after
        the partials call."""
        L, Lq = self.L, self.Lq
        if Lq == 0:
            return
        if self.rope:
            rope_apply(qq, pos0=L, base=self.base, out=self.qq_r[:, :, :Lq])
        else:
            self.qq_r[:, :, :Lq].copy_(qq)
        kv_append(kq, vq, self.kc, self.vc, slot0=L, pos0=L, base=self.base, rope=self.rope)
        offs = partition_offsets(L, self.b, L + Lq)
        if events is not None:
            events[0].record()
        op, lp = phase2_partial(self.qq_r[:, :, :Lq], self.kc, self.vc, offs, self.sq,
                                q_pos0=L, scale=self.scale,
                                o_part=self.op_q, lse_part=self.lp_q)
        if events is not None:
            events[1].record()
        lse_merge(op, lp, out=self.o2, lse=self.lse2)

    def decode(self, t, qd, kd, vd):
        """Generated token t (inputs are views [B, H, 1, D])."""
        pos = self.L + self.Lq + t
        if self.fused_decode:
            offs = partition_offsets(self.L, self.b, pos + 1)
            decode_step(qd, kd, vd, self.kc, self.vc, pos, pos, offs, self.sd, self.op_d,
                        self.lp_d, self.od[:, :, t:t + 1], self.lsed[t],
                        base=self.base, rope=self.rope, scale=self.scale)
            return
        qv = self.qd_r[:, :, t:t + 1]
        decode_prepare(qd, qv, kd, vd, self.kc, self.vc, slot0=pos, pos0=pos, base=self.base,
                       rope=self.rope)
        offs = partition_offsets(self.L, self.b, pos + 1)
        phase2_partial(qv, self.kc, self.vc, offs, self.sd, q_pos0=pos, scale=self.scale,
                       o_part=self.op_d, lse_part=self.lp_d)
        lse_merge(self.op_d, self.lp_d, out=self.od[:, :, t:t + 1], lse=self.lsed[t])

    def run(self, q, k, qq, kq, vq, qd, kd, vd):
        """One whole pass: Phase 1, the query, then every decode step."""
        self.rope_context(q, k)
        self.phase1()
        self.query(qq, kq, vq)
        for t in range(self.T):
            self.decode(t, qd[:, :, t:t + 1], kd[:, :, t:t + 1], vd[:, :, t:t + 1])


class DecodeGraph:
    """Decode steps replayed from one captured HIP graph
    (star_decode_step_devpos): the token's position lives in device memory
    (``pos``) and every step advances it, so the graph's arguments never
    change.  ``steps`` consecutive steps are captured together (a per-token
    graph of a model would hold one step per attention layer; each graph
    launch costs the runtime a gap of a few microseconds).

    Before each :meth:`replay`, write the next tokens' un-rotated q/k/v into
    ``q_in``, ``k_in``, ``v_in`` ([B, H, steps, D]); afterwards ``out`` and
    ``lse`` ([B, Hq, steps, D] and [steps, B, Hq]) hold their attention
    outputs.  Positions run from ``first`` to ``st.S - 1``."""

    def __init__(self, st: "StarAttentionStep", first: int, steps: int = 1):
        if not (st.L <= first and first + steps <= st.S):
            raise ValueError("positions outside the cache")
        B, Hq, Hkv, D = st.B, st.Hq, st.Hkv, st.D
        dev = st.kc.device
        bf = torch.bfloat16
        self.st, self.first, self.steps = st, first, steps
        self.q_in = torch.zeros((B, Hq, steps, D), dtype=bf, device=dev)
        self.k_in = torch.zeros((B, Hkv, steps, D), dtype=bf, device=dev)
        self.v_in = torch.zeros((B, Hkv, steps, D), dtype=bf, device=dev)
        self.out = torch.empty((B, Hq, steps, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((steps, B, Hq), dtype=torch.float32, device=dev)
        self.pos = torch.full((1,), first, dtype=torch.int64, device=dev)
        offs = partition_offsets(st.L, st.b, st.S)     # the last partition may grow to S
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(steps):
                decode_step_devpos(self.q_in[:, :, i:i + 1], self.k_in[:, :, i:i + 1],
                                   self.v_in[:, :, i:i + 1], st.kc, st.vc, self.pos, offs,
                                   st.sd, st.op_d, st.lp_d, self.out[:, :, i:i + 1],
                                   self.lse[i], base=st.base, rope=st.rope, scale=st.scale)

    def set_position(self, p: int):
        """Position of the next step (an eager fill, not part of the graph)."""
        self.pos.fill_(p)

    def replay(self):
        self.graph.replay()
