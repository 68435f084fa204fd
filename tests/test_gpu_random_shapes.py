"""GPU parity on seeded random shapes, beyond the hand-picked cases: ragged
context lengths, block sizes that are not multiples of the 64-key tile,
anchors from 0 to b, every GQA ratio the kernels take, D = 64 and 128,
split counts that leave chunks empty, and Phase-1 work queues on or off.
Each case is compared with the oracle element by element, to the same
tolerances as the other parity tests."""
import math

import numpy as np
import pytest
import torch

import block_sparse_amd as sa
import oracle.star_oracle as so
from block_sparse_amd.pipeline import StarAttentionStep
from gpu_util import check_lse, check_out, chunk_ranges, f64, host64, rand_tensor, to_dev

pytestmark = pytest.mark.gpu

BASE = 500000.0


def _p1_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        Hkv = int(rng.integers(1, 3))
        B = int(rng.integers(1, 3))
        L = int(rng.integers(1, 1600))
        b = int(rng.integers(16, 800))
        a = b if rng.random() < 0.5 else int(rng.integers(0, b + 1))
        sched = bool(rng.random() < 0.5)
        out.append((B, g * Hkv, Hkv, D, L, b, a, sched))
    return out


P1_RANDOM = _p1_cases(12, 7001)


@pytest.mark.parametrize("case", P1_RANDOM, ids=[str(i) for i in range(len(P1_RANDOM))])
def test_phase1_random_shapes(case):
    B, Hq, Hkv, D, L, b, a, sched = case
    print(f"phase1 random case {case}", flush=True)
    q = rand_tensor(31, 0, B, Hq, L, D)
    k = rand_tensor(31, 1, B, Hkv, L, D)
    v = rand_tensor(31, 2, B, Hkv, L, D)
    ws = sa.sched_workspace(torch.device("cuda")) if sched else None
    o, lse = sa.phase1_blocklocal(to_dev(q), to_dev(k), to_dev(v), b, a, want_lse=True, sched=ws)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(D)
    aa = a if b < L else 0
    ref_o, ref_l = so.phase1(f64(q), f64(k), f64(v), b, aa, scale)
    wabs, _ = so.phase1(f64(q), f64(k), np.abs(f64(v)), b, aa, scale)
    check_out(host64(o), ref_o, "O", bf16_out=True, wabs=wabs)
    check_lse(host64(lse), ref_l, "LSE")


P1_ROPE_RANDOM = [c for c in _p1_cases(24, 7002) if c[3] == 128][:8]


@pytest.mark.parametrize("case", P1_ROPE_RANDOM, ids=[str(i) for i in range(len(P1_ROPE_RANDOM))])
def test_phase1_rope_random_shapes(case):
    """Q rotated inside the kernel at positions 0..L-1; K rotated by the
    oracle (exact rotation rounded to bf16) and passed in."""
    B, Hq, Hkv, D, L, b, a, sched = case
    print(f"phase1 rope random case {case}", flush=True)
    q = rand_tensor(32, 0, B, Hq, L, D)
    k = rand_tensor(32, 1, B, Hkv, L, D)
    v = rand_tensor(32, 2, B, Hkv, L, D)
    pos = np.arange(L)
    k_rot = so.round_bf16(so.rope(f64(k), pos, BASE))
    kd = to_dev(k_rot.astype(np.float32)).to(torch.bfloat16)
    ws = sa.sched_workspace(torch.device("cuda")) if sched else None
    o, lse = sa.phase1_rope(to_dev(q), kd, to_dev(v), b, a, BASE, want_lse=True, sched=ws)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(D)
    aa = a if b < L else 0
    q_rot = so.round_bf16(so.rope(f64(q), pos, BASE))
    ref_o, ref_l = so.phase1(q_rot, k_rot, f64(v), b, aa, scale)
    wabs, _ = so.phase1(q_rot, k_rot, np.abs(f64(v)), b, aa, scale)
    check_out(host64(o), ref_o, "O", bf16_out=True, wabs=wabs)
    check_lse(host64(lse), ref_l, "LSE")


def _p2_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 3))
        B = int(rng.integers(1, 3))
        L = int(rng.integers(1, 1500))
        Lq = int(rng.choice([1, 2, 3, 7, 16, 33]))
        b = int(rng.integers(16, 600))
        splits = int(rng.choice([1, 2, 3, 5, 8]))
        out.append((B, g * Hkv, Hkv, D, L, Lq, b, splits))
    return out


def _p2_flash_cases(n, seed):
    """bf16 D = 128 query partials on the flash kernel (g * Lq > 16): both
    the 4-wave instance (g <= 4, g * Lq <= 128) and the 8-wave one."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        g = int(rng.choice([1, 2, 3, 4, 8]))
        small = i % 2 == 0 and g <= 4          # alternate the two instances
        if small:                              # 16 < g * Lq <= 128
            Lq = int(rng.integers(16 // g + 1, 128 // g + 1))
        else:                                  # 128 < g * Lq <= 200 + g
            Lq = int(rng.integers(128 // g + 1, 200 // g + 2))
        Hkv = int(rng.integers(1, 3))
        B = int(rng.integers(1, 3))
        L = int(rng.integers(1, 1500))
        b = int(rng.integers(16, 600))
        splits = int(rng.choice([1, 2, 3, 5, 8]))
        out.append((B, g * Hkv, Hkv, 128, L, Lq, b, splits))
    return out


P2_RANDOM = _p2_cases(12, 7003) + _p2_flash_cases(10, 7005)


@pytest.mark.parametrize("case", P2_RANDOM, ids=[str(i) for i in range(len(P2_RANDOM))])
def test_phase2_random_shapes(case):
    """Partials (decode kernel when g*Lq <= 16, flash kernel otherwise) and
    their merge."""
    B, Hq, Hkv, D, L, Lq, b, splits = case
    print(f"phase2 random case {case}", flush=True)
    g = Hq // Hkv
    N = L + Lq
    q = rand_tensor(33, 3, B, Hq, Lq, D)
    kc = rand_tensor(33, 4, B, Hkv, N, D)
    vc = rand_tensor(33, 5, B, Hkv, N, D)
    parts = so.partitions(L, b, N)
    offs = [p[0] for p in parts] + [parts[-1][1]]
    scale = 1 / math.sqrt(D)
    op, lp = sa.phase2_partial(to_dev(q), to_dev(kc), to_dev(vc), offs, splits, q_pos0=L)
    o, l = sa.lse_merge(op, lp)
    torch.cuda.synchronize()
    ranges = chunk_ranges(offs, splits)
    qf, kf, vf = f64(q), f64(kc), f64(vc)
    qpos = L + np.arange(Lq)
    ref_op, ref_lp = np.zeros(op.shape), np.zeros(lp.shape)
    ref_o, ref_l = np.zeros(o.shape), np.zeros(l.shape)
    for bb in range(B):
        for h in range(Hq):
            for c, (k0, k1) in enumerate(ranges):
                ref_op[c, bb, h], ref_lp[c, bb, h] = so.partial(
                    qf[bb, h], qpos, kf[bb, h // g], vf[bb, h // g], k0, k1, scale)
            ro, rl, _, _ = so.phase2(qf[bb, h], qpos, kf[bb, h // g], vf[bb, h // g], parts, scale)
            ref_o[bb, h], ref_l[bb, h] = ro, rl
    check_out(host64(op), ref_op, "o_part")
    check_lse(host64(lp), ref_lp, "lse_part")
    check_out(host64(o), ref_o, "O merged")
    check_lse(host64(l), ref_l, "LSE merged")


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = (128, 64)[i % 2]
        g = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.integers(1, 3))
        L = int(rng.integers(1, 1200))
        b = int(rng.integers(16, 500))
        splits = int(rng.choice([1, 2, 4, 7]))
        T = int(rng.integers(1, 5))
        out.append((int(rng.integers(1, 3)), g * Hkv, Hkv, D, L, b, splits, T))
    return out


DEC_RANDOM = _decode_cases(8, 7004)


@pytest.mark.parametrize("case", DEC_RANDOM, ids=[str(i) for i in range(len(DEC_RANDOM))])
def test_decode_step_random_shapes(case):
    """Consecutive fused decode steps (rope, append, partials, merge) after a
    rotated context, through the pipeline: outputs, lse and the appended
    cache rows."""
    B, Hq, Hkv, D, L, b, splits, T = case
    print(f"decode random case {case}", flush=True)
    g = Hq // Hkv
    q = rand_tensor(34, 0, B, Hq, L, D)
    k = rand_tensor(34, 1, B, Hkv, L, D)
    v = rand_tensor(34, 2, B, Hkv, L, D)
    qd = rand_tensor(34, 6, B, Hq, T, D)
    kd = rand_tensor(34, 7, B, Hkv, T, D)
    vd = rand_tensor(34, 8, B, Hkv, T, D)
    st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, T, base=BASE, splits_decode=splits)
    st.load_context(to_dev(v))
    st.rope_context(to_dev(q), to_dev(k))
    dq, dk, dv = to_dev(qd), to_dev(kd), to_dev(vd)
    for t in range(T):
        st.decode(t, dq[:, :, t:t + 1], dk[:, :, t:t + 1], dv[:, :, t:t + 1])
    torch.cuda.synchronize()
    rot = lambda x, p: so.round_bf16(so.rope(x, p, BASE))
    pos_d = L + np.arange(T)
    K = np.concatenate([rot(f64(k), np.arange(L)), rot(f64(kd), pos_d)], axis=2)
    V = np.concatenate([f64(v), f64(vd)], axis=2)
    assert np.array_equal(host64(st.kc[:, :, :L + T]), K), "cache K differs"
    assert np.array_equal(host64(st.vc[:, :, :L + T]), V), "cache V differs"
    Qd = rot(f64(qd), pos_d)
    ref_o, ref_l = np.zeros((B, Hq, T, D)), np.zeros((T, B, Hq))
    for t in range(T):
        parts = so.partitions(L, b, L + t + 1)
        for bb in range(B):
            for h in range(Hq):
                o, l, _, _ = so.phase2(Qd[bb, h, t:t + 1], pos_d[t:t + 1], K[bb, h // g],
                                       V[bb, h // g], parts, 1 / math.sqrt(D))
                ref_o[bb, h, t], ref_l[t, bb, h] = o[0], l[0]
    check_out(host64(st.od)[:, :, :T], ref_o, "decode O")
    check_lse(host64(st.lsed)[:T], ref_l, "decode LSE")
