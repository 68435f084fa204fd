"""The decode step with its position in device memory
(star_decode_step_devpos): eager calls and a captured HIP graph replayed
once per generated token, against star_decode_step at the same positions.

Both entry points run the same kernels with the same chunking of the
partitions, so every output, lse and cache row must be the same bits; the
first case is also checked against the oracle.  Positions outside the
partitions' bound must leave the cache untouched and give empty results.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_amd as sa
import oracle.star_oracle as so
from gpu_util import check_lse, check_out, f64, host64, rand_tensor, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, D, L, b, splits, steps, rope
    (1, 32, 8, 128, 3000, 1024, 4, 5, True),
    (2, 8, 2, 64, 500, 128, 2, 4, True),
    (1, 16, 16, 128, 1000, 1000, 3, 3, False),
]


def setup(case, seed):
    B, Hq, Hkv, D, L, b, splits, n, rope = case
    S = L + n + 2
    k = np.concatenate([rand_tensor(seed, 1, B, Hkv, L, D),
                        np.zeros((B, Hkv, S - L, D), dtype=np.uint16)], axis=2)
    v = np.concatenate([rand_tensor(seed, 2, B, Hkv, L, D),
                        np.zeros((B, Hkv, S - L, D), dtype=np.uint16)], axis=2)
    steps = {name: rand_tensor(seed, t, B, H, n, D)
             for name, t, H in (("q", 6, Hq), ("k", 7, Hkv), ("v", 8, Hkv))}
    offs = list(range(0, L, b)) + [S]
    return k, v, steps, offs


def reference(case, k, v, steps, offs, base):
    """star_decode_step at positions L, L+1, ...: outputs, lse, final cache."""
    B, Hq, Hkv, D, L, b, splits, n, rope = case
    P = len(offs) - 1
    kc, vc = to_dev(k), to_dev(v)
    op = torch.empty((P * splits, B, Hq, 1, D), dtype=torch.float32, device="cuda")
    lp = torch.empty((P * splits, B, Hq, 1), dtype=torch.float32, device="cuda")
    outs, lses = [], []
    for t in range(n):
        pos = L + t
        o = torch.empty((B, Hq, 1, D), dtype=torch.float32, device="cuda")
        l = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        sl = slice(t, t + 1)
        sa.decode_step(to_dev(steps["q"][:, :, sl]), to_dev(steps["k"][:, :, sl]),
                       to_dev(steps["v"][:, :, sl]), kc, vc, pos, pos, offs[:-1] + [pos + 1],
                       splits, op, lp, o, l, base=base, rope=rope)
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    return outs, lses, kc, vc


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_devpos_eager_equals_decode_step(ci):
    case = CASES[ci]
    B, Hq, Hkv, D, L, b, splits, n, rope = case
    print(f"devpos eager: case {case}", flush=True)
    base = 500000.0
    k, v, steps, offs = setup(case, 40 + ci)
    r_o, r_l, r_k, r_v = reference(case, k, v, steps, offs, base)
    P = len(offs) - 1
    kc, vc = to_dev(k), to_dev(v)
    op = torch.empty((P * splits, B, Hq, 1, D), dtype=torch.float32, device="cuda")
    lp = torch.empty((P * splits, B, Hq, 1), dtype=torch.float32, device="cuda")
    pos = torch.tensor([L], dtype=torch.int64, device="cuda")
    for t in range(n):
        o = torch.full((B, Hq, 1, D), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        sl = slice(t, t + 1)
        sa.decode_step_devpos(to_dev(steps["q"][:, :, sl]), to_dev(steps["k"][:, :, sl]),
                              to_dev(steps["v"][:, :, sl]), kc, vc, pos, offs, splits, op, lp,
                              o, l, base=base, rope=rope)
        torch.cuda.synchronize()
        assert torch.equal(o, r_o[t]) and torch.equal(l, r_l[t]), f"step {t} differs"
    assert int(pos.item()) == L + n
    assert torch.equal(kc, r_k) and torch.equal(vc, r_v), "cache differs"
    if ci == 0:
        # the last step against the oracle, every head; the context rows are
        # attended as the cache holds them (this test stores them as drawn)
        rot = (lambda x, p: so.round_bf16(so.rope(x, p, base))) if rope else (lambda x, p: x)
        Kc = np.concatenate([f64(k[:, :, :L]), rot(f64(steps["k"]), L + np.arange(n))], axis=2)
        Vc = np.concatenate([f64(v[:, :, :L]), f64(steps["v"])], axis=2)
        pl = L + n - 1
        qr = rot(f64(steps["q"][:, :, n - 1:n]), [pl])
        g = Hq // Hkv
        got_o, got_l = host64(r_o[-1]), host64(r_l[-1])
        for bb in range(B):
            for h in range(Hq):
                ro, rl, _, _ = so.phase2(qr[bb, h], np.array([pl]), Kc[bb, h // g],
                                         Vc[bb, h // g], so.partitions(L, b, pl + 1),
                                         1 / math.sqrt(D))
                check_out(got_o[bb, h], ro, f"devpos O b{bb} h{h}")
                check_lse(got_l[bb, h:h + 1], rl, f"devpos LSE b{bb} h{h}")


# the 8B-128K decode shape (8 partitions x 4 chunks x 8 KV heads = 256 workgroups)
FULL = (1, 32, 8, 128, 131072, 16384, 4, 3, True)


@pytest.mark.parametrize("ci", [0, 1, "full"])
def test_devpos_graph_replays(ci):
    """One step captured in a HIP graph, replayed once per token with the
    token's inputs copied into the captured buffers in between (eager work
    and a synchronisation between replays): every replay equals
    star_decode_step at that position."""
    case = FULL if ci == "full" else CASES[ci]
    B, Hq, Hkv, D, L, b, splits, n, rope = case
    print(f"devpos graph: case {case}", flush=True)
    base = 500000.0
    k, v, steps, offs = setup(case, 50 + (9 if ci == "full" else ci))
    r_o, r_l, r_k, r_v = reference(case, k, v, steps, offs, base)
    P = len(offs) - 1
    kc, vc = to_dev(k), to_dev(v)
    op = torch.empty((P * splits, B, Hq, 1, D), dtype=torch.float32, device="cuda")
    lp = torch.empty((P * splits, B, Hq, 1), dtype=torch.float32, device="cuda")
    qb = torch.zeros((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros((B, Hkv, 1, D), dtype=torch.bfloat16, device="cuda")
    vb = torch.zeros((B, Hkv, 1, D), dtype=torch.bfloat16, device="cuda")
    ob = torch.zeros((B, Hq, 1, D), dtype=torch.float32, device="cuda")
    lb = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    pos = torch.tensor([L], dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.decode_step_devpos(qb, kb, vb, kc, vc, pos, offs, splits, op, lp, ob, lb, base=base,
                              rope=rope)
    torch.cuda.synchronize()
    # capturing ran nothing: the position and the cache are as they were
    assert int(pos.item()) == L
    assert torch.equal(kc, to_dev(k))
    for t in range(n):
        sl = slice(t, t + 1)
        qb.copy_(to_dev(steps["q"][:, :, sl]))
        kb.copy_(to_dev(steps["k"][:, :, sl]))
        vb.copy_(to_dev(steps["v"][:, :, sl]))
        ob.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ob, r_o[t]) and torch.equal(lb, r_l[t]), f"replay {t} differs"
        assert int(pos.item()) == L + t + 1
    assert torch.equal(kc, r_k) and torch.equal(vc, r_v), "cache differs"
    del graph


def test_devpos_out_of_range_positions():
    """A position outside [part_offsets[P-1], part_offsets[P]) writes no
    cache row, gives o = 0 and lse = -inf, and is still advanced."""
    B, Hq, Hkv, D, L, b, splits = 1, 8, 2, 128, 600, 256, 2
    k, v, steps, offs = setup((B, Hq, Hkv, D, L, b, splits, 1, True), 60)
    kc, vc = to_dev(k), to_dev(v)
    P = len(offs) - 1
    op = torch.empty((P * splits, B, Hq, 1, D), dtype=torch.float32, device="cuda")
    lp = torch.empty((P * splits, B, Hq, 1), dtype=torch.float32, device="cuda")
    for p0 in (offs[-1], offs[-2] - 1, -5):
        print(f"devpos out of range: pos {p0}", flush=True)
        pos = torch.tensor([p0], dtype=torch.int64, device="cuda")
        o = torch.full((B, Hq, 1, D), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        sa.decode_step_devpos(to_dev(steps["q"]), to_dev(steps["k"]), to_dev(steps["v"]), kc, vc,
                              pos, offs, splits, op, lp, o, l)
        torch.cuda.synchronize()
        assert int(pos.item()) == p0 + 1
        assert bool((o == 0).all()) and bool(torch.isneginf(l).all())
        assert torch.equal(kc, to_dev(k)) and torch.equal(vc, to_dev(v))


def test_devpos_never_reads_past_the_token():
    """The last partition ends right after the device-side position: cache
    rows past the token hold NaN and +-Inf patterns, and every step still
    gives star_decode_step's bits (computed with zero rows there)."""
    case = CASES[0]
    B, Hq, Hkv, D, L, b, splits, n, rope = case
    base = 500000.0
    k, v, steps, offs = setup(case, 70)
    r_o, r_l, _, _ = reference(case, k, v, steps, offs, base)
    poison = np.array([0x7FC0, 0x7F80, 0xFF80, 0xFFC1], dtype=np.uint16)   # NaN, +Inf, -Inf, NaN
    kp, vp = k.copy(), v.copy()
    S = k.shape[2]
    kp[:, :, L:] = np.resize(poison, (B, Hkv, S - L, D))
    vp[:, :, L:] = np.resize(poison[::-1], (B, Hkv, S - L, D))
    kc, vc = to_dev(kp), to_dev(vp)
    P = len(offs) - 1
    op = torch.empty((P * splits, B, Hq, 1, D), dtype=torch.float32, device="cuda")
    lp = torch.empty((P * splits, B, Hq, 1), dtype=torch.float32, device="cuda")
    pos = torch.tensor([L], dtype=torch.int64, device="cuda")
    for t in range(n):
        print(f"devpos poison: step {t}", flush=True)
        o = torch.full((B, Hq, 1, D), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        sl = slice(t, t + 1)
        sa.decode_step_devpos(to_dev(steps["q"][:, :, sl]), to_dev(steps["k"][:, :, sl]),
                              to_dev(steps["v"][:, :, sl]), kc, vc, pos, offs, splits, op, lp,
                              o, l, base=base, rope=rope)
        torch.cuda.synchronize()
        assert torch.equal(o, r_o[t]) and torch.equal(l, r_l[t]), f"step {t} differs"


def test_decode_graph_helper():
    """pipeline.DecodeGraph: 3 steps per graph, replayed twice with new
    inputs written in between, equals 6 eager star_decode_step calls bit for
    bit (outputs, lse and the cache)."""
    from block_sparse_amd.pipeline import DecodeGraph, StarAttentionStep
    B, Hq, Hkv, D, L, b, splits = 1, 16, 4, 128, 2500, 1024, 3
    n, per = 6, 3
    print(f"decode graph helper: L={L} steps={n}", flush=True)
    q = rand_tensor(80, 0, B, Hq, L, D)
    k = rand_tensor(80, 1, B, Hkv, L, D)
    v = rand_tensor(80, 2, B, Hkv, L, D)
    qd, kd, vd = (rand_tensor(80, t, B, H, n, D) for t, H in ((6, Hq), (7, Hkv), (8, Hkv)))
    runs = []
    for use_graph in (False, True):
        st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, n, splits_decode=splits)
        st.load_context(to_dev(v))
        st.rope_context(to_dev(q), to_dev(k))
        if not use_graph:
            for t in range(n):
                sl = slice(t, t + 1)
                st.decode(t, to_dev(qd[:, :, sl]), to_dev(kd[:, :, sl]), to_dev(vd[:, :, sl]))
            torch.cuda.synchronize()
            runs.append((st.od.clone(), st.lsed.clone(), st.kc.clone(), st.vc.clone()))
            continue
        dg = DecodeGraph(st, L, per)
        od = torch.empty_like(st.od)
        ld = torch.empty_like(st.lsed)
        for r in range(n // per):
            sl = slice(r * per, (r + 1) * per)
            dg.q_in.copy_(to_dev(qd[:, :, sl]))
            dg.k_in.copy_(to_dev(kd[:, :, sl]))
            dg.v_in.copy_(to_dev(vd[:, :, sl]))
            dg.replay()
            torch.cuda.synchronize()
            od[:, :, sl] = dg.out
            ld[sl] = dg.lse
        assert int(dg.pos.item()) == L + n
        runs.append((od, ld, st.kc.clone(), st.vc.clone()))
    (o0, l0, k0, v0), (o1, l1, k1, v1) = runs
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "graph steps differ from eager ones"
    assert torch.equal(k0, k1) and torch.equal(v0, v1), "cache differs"
