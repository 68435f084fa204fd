"""GPU tests of what the kernels must not touch and must not read.

* Unwritten memory next to the inputs: cache rows past the partitions' end
  (decode slots not written yet) and prefix rows outside a block's prefix
  range may hold anything, NaN and Inf included.  No kernel may read them:
  a masked key still enters the PV product as 0 * V, and 0 * NaN = NaN.
* Canaries around every output: O, lse, the partials and the merged output,
  a strided attention view like the layer's, and the decode step's cache
  row.  Every byte outside the written region must be unchanged.
* Rows that see very few keys, where the lse is essentially one score: with
  Q and K rotated exactly (fp64, one rounding), their lse error is far
  below the 1e-3 bound.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_amd as sa
import oracle.star_oracle as so
from block_sparse_amd.pipeline import StarAttentionStep
from gpu_util import check_lse, check_out, f64, host64, rand_tensor, to_dev

pytestmark = pytest.mark.gpu

# bf16 bit patterns: quiet NaN, +Inf, -Inf, a large finite value
POISON16 = np.array([0x7FC0, 0x7F80, 0xFF80, 0x7F7F], dtype=np.uint16)
CANARY16 = 0x5A5A          # bf16 ~1.5e16: never a result here
CANARY32 = 0x5A5A5A5A      # fp32 ~1.5e16


def poison_rows(t: torch.Tensor, r0: int):
    """Fill rows r0.. of a [B, H, S, D] bf16 tensor with NaN / Inf patterns."""
    n = t.shape[2] - r0
    if n <= 0:
        return
    pat = np.resize(POISON16, t.shape[0] * t.shape[1] * n * t.shape[3])
    src = torch.from_numpy(pat.view(np.int16)).view(torch.bfloat16).cuda()
    t[:, :, r0:].copy_(src.view(t.shape[0], t.shape[1], n, t.shape[3]))


def canary_like(shape, dtype, margin_elems):
    """A flat buffer with ``margin_elems`` canary elements on both sides of a
    contiguous region of ``shape``; returns (buffer, view)."""
    n = int(np.prod(shape))
    if dtype == torch.bfloat16:
        buf = torch.full((n + 2 * margin_elems,), CANARY16, dtype=torch.int16,
                         device="cuda").view(torch.bfloat16)
    else:
        buf = torch.full((n + 2 * margin_elems,), CANARY32, dtype=torch.int32,
                         device="cuda").view(torch.float32)
    return buf, buf[margin_elems:margin_elems + n].view(shape)


def untouched(buf: torch.Tensor, written: torch.Tensor) -> bool:
    """Every element of ``buf`` outside the (possibly strided) view
    ``written`` still holds the canary."""
    raw = buf.view(torch.int16 if buf.dtype == torch.bfloat16 else torch.int32).reshape(-1)
    mask = torch.ones(raw.numel(), dtype=torch.bool, device=buf.device)
    # mark the view's elements by their offsets
    off0 = written.data_ptr() - buf.data_ptr()
    es = buf.element_size()
    assert off0 % es == 0
    idx = torch.zeros(written.shape, dtype=torch.int64, device=buf.device)
    for d, (n, st) in enumerate(zip(written.shape, written.stride())):
        shp = [1] * written.dim()
        shp[d] = n
        idx += (torch.arange(n, device=buf.device) * st).view(shp)
    mask[(idx + off0 // es).flatten()] = False
    want = CANARY16 if buf.dtype == torch.bfloat16 else CANARY32
    return bool((raw[mask] == want).all())


def written_everywhere(view: torch.Tensor) -> bool:
    """No element of ``view`` still holds the canary (an empty chunk's lse
    is -inf, so finiteness is not the test)."""
    raw = view.contiguous().view(torch.int16 if view.dtype == torch.bfloat16 else torch.int32)
    want = CANARY16 if view.dtype == torch.bfloat16 else CANARY32
    return not bool((raw == want).any())


# ---------------------------------------------------------------------------
# unwritten memory is never read
# ---------------------------------------------------------------------------
P2_POISON_CASES = [
    # B, Hq, Hkv, D, L, Lq, b, splits, bf16   (path)
    (1, 32, 8, 128, 1000, 64, 300, 2, True),      # flash2 (D = 128 bf16), ragged last tile
    (1, 16, 4, 128, 777, 33, 200, 3, True),       # flash2, chunk ends at 32 mod 64
    (1, 32, 8, 128, 1000, 32, 300, 2, True),      # flash2 4-wave (g * Lq = 128), ragged tile
    (1, 8, 4, 128, 777, 20, 200, 3, True),        # flash2 4-wave, g = 2
    (1, 8, 2, 64, 700, 40, 256, 2, True),         # flash.hip (D = 64)
    (1, 16, 2, 128, 500, 16, 128, 2, False),      # flash.hip (fp32 inputs)
    (2, 8, 2, 128, 777, 1, 200, 4, True),         # decode kernel (g * Lq = 4)
    (1, 4, 1, 64, 300, 1, 100, 8, True),          # decode kernel, D = 64
]


@pytest.mark.parametrize("case", P2_POISON_CASES, ids=[str(i) for i in range(len(P2_POISON_CASES))])
def test_phase2_ignores_rows_past_the_partitions(case):
    """Cache rows at and after part_offsets[P] hold NaN / Inf: the partials
    and the merged output still equal the oracle's over the valid rows."""
    B, Hq, Hkv, D, L, Lq, b, splits, bf16 = case
    print(f"phase2 poison case {case}", flush=True)
    g = Hq // Hkv
    N = L + Lq
    sc = 1.0 if bf16 else 0.125
    q = rand_tensor(61, 3, B, Hq, Lq, D, sc, bf16)
    kc = rand_tensor(61, 4, B, Hkv, N, D, sc, bf16)
    vc = rand_tensor(61, 5, B, Hkv, N, D, sc, bf16)
    extra = 200
    kd = torch.empty((B, Hkv, N + extra, D), dtype=torch.bfloat16 if bf16 else torch.float32,
                     device="cuda")
    vd = torch.empty_like(kd)
    kd[:, :, :N].copy_(to_dev(kc))
    vd[:, :, :N].copy_(to_dev(vc))
    if bf16:
        poison_rows(kd, N)
        poison_rows(vd, N)
    else:
        kd[:, :, N:] = float("nan")
        vd[:, :, N:] = float("inf")
    parts = so.partitions(L, b, N)
    offs = [p[0] for p in parts] + [parts[-1][1]]
    op, lp = sa.phase2_partial(to_dev(q), kd, vd, offs, splits, q_pos0=L)
    o, l = sa.lse_merge(op, lp)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(op).all()), "a partial read a poisoned row"
    qpos = L + np.arange(Lq)
    for bb in range(B):
        for h in range(Hq):
            ro, rl, _, _ = so.phase2(f64(q)[bb, h], qpos, f64(kc)[bb, h // g],
                                     f64(vc)[bb, h // g], parts, 1 / math.sqrt(D))
            check_out(host64(o)[bb, h], ro, f"O merged b{bb} h{h}")
            check_lse(host64(l)[bb, h], rl, f"LSE merged b{bb} h{h}")


def test_decode_step_ignores_rows_past_its_position():
    """The cache is allocated for every future token: the rows after the
    decode token's own slot are NaN / Inf and must not be read, even though
    the last partition's offset reaches the end of the allocation."""
    B, Hq, Hkv, D, L, b = 1, 32, 8, 128, 1500, 512
    T = 3
    print("decode step with poisoned future slots", flush=True)
    q = rand_tensor(62, 0, B, Hq, L, D)
    k = rand_tensor(62, 1, B, Hkv, L, D)
    v = rand_tensor(62, 2, B, Hkv, L, D)
    qd, kd, vd = (rand_tensor(62, t, B, H, T, D) for t, H in ((6, Hq), (7, Hkv), (8, Hkv)))
    st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, T, base=500000.0, splits_decode=4)
    st.load_context(to_dev(v))
    st.rope_context(to_dev(q), to_dev(k))
    poison_rows(st.kc, L)
    poison_rows(st.vc, L)
    dq, dk, dv = to_dev(qd), to_dev(kd), to_dev(vd)
    S = st.kc.shape[2]
    for t in range(T):
        pos = L + t
        # the last partition spans the whole allocation, not just pos + 1
        offs = list(range(0, L, b)) + [S]
        sa.decode_step(dq[:, :, t:t + 1], dk[:, :, t:t + 1], dv[:, :, t:t + 1], st.kc, st.vc,
                       pos, pos, offs, 4, st.op_d, st.lp_d, st.od[:, :, t:t + 1], st.lsed[t])
    torch.cuda.synchronize()
    rot = lambda x, p: so.round_bf16(so.rope(x, p, 500000.0))
    K = np.concatenate([rot(f64(k), np.arange(L)), rot(f64(kd), L + np.arange(T))], axis=2)
    V = np.concatenate([f64(v), f64(vd)], axis=2)
    Qd = rot(f64(qd), L + np.arange(T))
    for t in range(T):
        for h in range(Hq):
            ro, rl, _, _ = so.phase2(Qd[0, h, t:t + 1], np.array([L + t]), K[0, h // 4],
                                     V[0, h // 4], so.partitions(L, b, L + t + 1),
                                     1 / math.sqrt(D))
            check_out(host64(st.od)[0, h, t:t + 1], ro, f"decode O t{t} h{h}")
            check_lse(host64(st.lsed)[t, 0, h:h + 1], rl, f"decode LSE t{t} h{h}")


@pytest.mark.parametrize("D,bf16", [(128, True), (64, True), (128, False)])
def test_phase1_prefix_ignores_rows_outside_the_ranges(D, bf16):
    """Prefix rows outside every block's [start, start + len) are NaN / Inf
    (the table may point into a larger buffer): they are never read."""
    B, Hq, Hkv, L, b, R = 1, 8, 2, 600, 200, 500
    print(f"phase1 prefix poison D={D} bf16={bf16}", flush=True)
    sc = 1.0 if bf16 else 0.125
    q = rand_tensor(63, 0, B, Hq, L, D, sc, bf16)
    k = rand_tensor(63, 1, B, Hkv, L, D, sc, bf16)
    v = rand_tensor(63, 2, B, Hkv, L, D, sc, bf16)
    pk = rand_tensor(63, 3, B, Hkv, R, D, sc, bf16)
    pv = rand_tensor(63, 4, B, Hkv, R, D, sc, bf16)
    # prefix ranges [10, 43), [100, 227), [250, 250 + 95): lengths not multiples of 64
    st, ln = [0, 100, 250], [0, 127, 95]
    st[0], ln[0] = 10, 33
    pkd, pvd = to_dev(pk), to_dev(pv)
    keep = np.zeros(R, bool)
    for s0, n in zip(st, ln):
        keep[s0:s0 + n] = True
    bad = torch.from_numpy(np.nonzero(~keep)[0]).cuda()
    fill = float("nan")
    pkd[:, :, bad] = fill
    pvd[:, :, bad] = float("inf")
    o, lse = sa.phase1_prefix(to_dev(q), to_dev(k), to_dev(v), pkd, pvd, st, ln, b,
                              want_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = so.phase1_prefix(f64(q), f64(k), f64(v), f64(pk), f64(pv), st, ln, b,
                                    1 / math.sqrt(D))
    wabs, _ = so.phase1_prefix(f64(q), f64(k), np.abs(f64(v)), f64(pk), np.abs(f64(pv)), st, ln,
                               b, 1 / math.sqrt(D))
    check_out(host64(o), ref_o, "O", bf16_out=True, wabs=wabs)
    check_lse(host64(lse), ref_l, "LSE")


# ---------------------------------------------------------------------------
# canaries: nothing outside an output is written
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Lq", [40, 24], ids=["8-wave", "4-wave"])
def test_outputs_keep_their_canaries(Lq):
    """(g * Lq = 160 runs the 8-wave query instance, 96 the 4-wave one.)"""
    B, Hq, Hkv, D, L, b = 1, 16, 4, 128, 700, 256
    print(f"canaries Lq={Lq}", flush=True)
    q, k, v = (to_dev(rand_tensor(64, t, B, H, L, D)) for t, H in ((0, Hq), (1, Hkv), (2, Hkv)))
    M = 64
    # Phase-1 O through a strided view laid out like the attention layer's
    # output buffer ([B, L, Hq*D + pad] viewed as [B, Hq, L, D]), lse with margins
    att = torch.empty((B, L, Hq * D + M), dtype=torch.int16, device="cuda")
    att.fill_(CANARY16)
    att = att.view(torch.bfloat16)
    o_view = att[:, :, :Hq * D].view(B, L, Hq, D).permute(0, 2, 1, 3)
    lbuf, lse = canary_like((B, Hq, L), torch.float32, M)
    sched = sa.sched_workspace(q.device)
    sa.phase1_rope(q, k, v, b, b, out=o_view, lse=lse, sched=sched)
    # Phase 2: partials and merge, each with margins; merged O strided
    qq = to_dev(rand_tensor(64, 3, B, Hq, Lq, D))
    kc = torch.cat([k, to_dev(rand_tensor(64, 4, B, Hkv, Lq, D))], dim=2).contiguous()
    vc = torch.cat([v, to_dev(rand_tensor(64, 5, B, Hkv, Lq, D))], dim=2).contiguous()
    offs = list(range(0, L, b)) + [L + Lq]
    splits = 3
    N = (len(offs) - 1) * splits
    opbuf, op = canary_like((N, B, Hq, Lq, D), torch.float32, M)
    lpbuf, lp = canary_like((N, B, Hq, Lq), torch.float32, M)
    sa.phase2_partial(qq, kc, vc, offs, splits, q_pos0=L, o_part=op, lse_part=lp)
    obig = torch.full((B, Hq, Lq, D + M), 0, dtype=torch.int32, device="cuda")
    obig.fill_(CANARY32)
    obig = obig.view(torch.float32)
    o_m = obig[..., :D]
    lmbuf, l_m = canary_like((B, Hq, Lq), torch.float32, M)
    sa.lse_merge(op, lp, out=o_m, lse=l_m)
    torch.cuda.synchronize()
    for buf, view, what in ((att, o_view, "Phase-1 O (layer view)"), (lbuf, lse, "Phase-1 lse"),
                            (opbuf, op, "o_part"), (lpbuf, lp, "lse_part"),
                            (obig, o_m, "merged O"), (lmbuf, l_m, "merged lse")):
        assert untouched(buf, view), f"{what}: a canary was overwritten"
        assert written_everywhere(view), f"{what}: not fully written"


def test_decode_step_writes_only_its_row():
    """The fused decode step writes the new token's K/V row and nothing else
    of the cache; its partials and outputs keep their canaries."""
    B, Hq, Hkv, D, L, b, T = 1, 32, 8, 128, 900, 300, 2
    print("decode step canaries", flush=True)
    st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, T, splits_decode=3)
    st.load_context(to_dev(rand_tensor(65, 2, B, Hkv, L, D)))
    st.rope_context(to_dev(rand_tensor(65, 0, B, Hq, L, D)),
                    to_dev(rand_tensor(65, 1, B, Hkv, L, D)))
    st.kc[:, :, L:].fill_(3.0)
    st.vc[:, :, L:].fill_(-3.0)
    torch.cuda.synchronize()
    kc0, vc0 = st.kc.clone(), st.vc.clone()
    qd, kd, vd = (to_dev(rand_tensor(65, t, B, H, 1, D)) for t, H in ((6, Hq), (7, Hkv), (8, Hkv)))
    M = 64
    nd = st.op_d.shape[0]
    opbuf, op = canary_like((nd, B, Hq, 1, D), torch.float32, M)
    lpbuf, lp = canary_like((nd, B, Hq, 1), torch.float32, M)
    obuf, o = canary_like((B, Hq, 1, D), torch.float32, M)
    lbuf, l = canary_like((B, Hq), torch.float32, M)
    pos = L
    offs = list(range(0, L, b)) + [pos + 1]
    sa.decode_step(qd, kd, vd, st.kc, st.vc, pos, pos, offs, 3, op, lp, o, l)
    torch.cuda.synchronize()
    changed_k = (st.kc != kc0).any(dim=-1)
    changed_v = (st.vc != vc0).any(dim=-1)
    rows_k = torch.nonzero(changed_k.any(dim=(0, 1))).flatten().tolist()
    rows_v = torch.nonzero(changed_v.any(dim=(0, 1))).flatten().tolist()
    assert rows_k == [pos] and rows_v == [pos], (rows_k, rows_v)
    for buf, view, what in ((opbuf, op, "o_part"), (lpbuf, lp, "lse_part"), (obuf, o, "O"),
                            (lbuf, l, "lse")):
        assert untouched(buf, view), f"{what}: a canary was overwritten"


# ---------------------------------------------------------------------------
# rows that see one to four keys
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_phase1_few_key_rows_lse(seed):
    """Positions 0..3 of block 1 see 1..4 keys, and with no anchor so does
    the start of every block: their lse is essentially one score.  With Q
    rotated in the kernel and K by star_rope_apply, both exactly (fp64, one
    rounding), the only error left is the fp32 accumulation of the scores,
    so the lse error there is far below the 1e-3 bound."""
    B, Hq, Hkv, D, L, b = 1, 32, 8, 128, 2048, 512
    base = 500000.0
    print(f"few-key rows seed {seed}", flush=True)
    q = rand_tensor(70 + seed, 0, B, Hq, L, D)
    k = rand_tensor(70 + seed, 1, B, Hkv, L, D)
    v = rand_tensor(70 + seed, 2, B, Hkv, L, D)
    kd = sa.rope_apply(to_dev(k), pos0=0, base=base, out=torch.empty_like(to_dev(k)))
    pos = np.arange(L)
    Q = so.round_bf16(so.rope(f64(q), pos, base))
    K = so.round_bf16(so.rope(f64(k), pos, base))
    starts = np.arange(0, L, b)
    few = np.concatenate([s + np.arange(4) for s in starts])
    for a in (b, 0):
        o, lse = sa.phase1_rope(to_dev(q), kd, to_dev(v), b, a, base, want_lse=True)
        torch.cuda.synchronize()
        ref_o, ref_l = so.phase1(Q, K, f64(v), b, a, 1 / math.sqrt(D))
        rows = few if a == 0 else np.arange(4)
        err = np.abs(host64(lse)[..., rows] - ref_l[..., rows])
        assert err.max() <= 2e-5, (a, float(err.max()))
        wabs, _ = so.phase1(Q, K, np.abs(f64(v)), b, a, 1 / math.sqrt(D))
        check_out(host64(o), ref_o, f"O a={a}", bf16_out=True, wabs=wabs)
        check_lse(host64(lse), ref_l, f"LSE a={a}")


def test_concurrent_streams_match_sequential_results():
    """The library keeps no mutable state between calls: two Phase-1 calls
    (each with its own scheduling workspace) and two decode steps (own
    workspaces) issued together on two streams give the same bits as the
    same calls one after the other."""
    from block_sparse_amd.pipeline import partition_offsets
    B, Hq, Hkv, D, L, b = 1, 16, 4, 128, 3000, 1024
    print("concurrent streams: two Phase-1 calls and two decode steps", flush=True)
    ins = []
    for seed in (91, 92):
        q = to_dev(rand_tensor(seed, 0, B, Hq, L, D))
        k = to_dev(rand_tensor(seed, 1, B, Hkv, L + 1, D))
        v = to_dev(rand_tensor(seed, 2, B, Hkv, L + 1, D))
        qd = to_dev(rand_tensor(seed, 6, B, Hq, 1, D))
        kd = to_dev(rand_tensor(seed, 7, B, Hkv, 1, D))
        vd = to_dev(rand_tensor(seed, 8, B, Hkv, 1, D))
        ins.append((q, k, v, qd, kd, vd))
    offs = partition_offsets(L, b, L + 1)
    splits = 3
    P = len(offs) - 1

    def run(i, stream):
        q, k, v, qd, kd, vd = ins[i]
        with torch.cuda.stream(stream):
            kc, vc = k.clone(), v.clone()        # on this stream: ordered before the calls
            ws = sa.sched_workspace(q.device)
            o1, l1 = sa.phase1_blocklocal(q, kc[:, :, :L], vc[:, :, :L], b, b, want_lse=True,
                                          sched=ws)
            op = torch.empty((P * splits, B, Hq, 1, D), dtype=torch.float32, device="cuda")
            lp = torch.empty((P * splits, B, Hq, 1), dtype=torch.float32, device="cuda")
            od = torch.empty((B, Hq, 1, D), dtype=torch.float32, device="cuda")
            ld = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
            sa.decode_step(qd, kd, vd, kc, vc, L, L, offs, splits, op, lp, od, ld)
        return o1, l1, od, ld, kc

    s0 = torch.cuda.current_stream()
    seq = [run(i, s0) for i in (0, 1)]
    torch.cuda.synchronize()
    sa_, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa_.wait_stream(s0)
    sb.wait_stream(s0)
    par = [run(0, sa_), run(1, sb)]
    torch.cuda.synchronize()
    for i in (0, 1):
        for x, y in zip(seq[i], par[i]):
            assert torch.equal(x, y), f"call set {i} differs when run concurrently"
