"""GPU parity on small shapes: every entry point of the C ABI against the CPU
oracle, element by element, including ragged tails, anchor variants, GQA
ratios, empty chunks and fully masked rows."""
import math

import numpy as np
import pytest
import torch

import block_sparse_amd as sa
import oracle.star_oracle as so
from gpu_util import (check_lse, check_out, chunk_ranges, f64, host64, rand_tensor,
                      to_dev, with_wabs)

pytestmark = pytest.mark.gpu


def _qkv(seed, B, Hq, Hkv, L, D, bf16=True, scale=1.0):
    q = rand_tensor(seed, 0, B, Hq, L, D, scale, bf16)
    k = rand_tensor(seed, 1, B, Hkv, L, D, scale, bf16)
    v = rand_tensor(seed, 2, B, Hkv, L, D, scale, bf16)
    return q, k, v


P1_CASES = [
    # B, Hq, Hkv, D, L, b, a, bf16, scale
    (1, 2, 1, 64, 512, 128, 128, True, 0.125),     # tiny workload, bf16
    (1, 2, 1, 64, 512, 128, 128, False, 0.125),    # tiny workload, fp32 inputs
    (2, 8, 2, 128, 700, 200, 200, True, 1.0),      # ragged tail, b % 64 != 0
    (1, 4, 1, 128, 333, 1000, 1000, True, 1.0),    # single block (b >= L)
    (1, 8, 1, 128, 640, 128, 0, True, 1.0),        # no anchor (block-diagonal)
    (1, 4, 4, 64, 600, 256, 100, True, 1.0),       # smaller anchor, MHA
    (1, 16, 1, 128, 300, 128, 128, True, 1.0),     # g = 16
    (1, 24, 8, 128, 300, 100, 100, True, 1.0),     # g = 3
    (1, 5, 5, 64, 97, 32, 32, True, 1.0),          # L < one key tile
    (1, 8, 2, 128, 1, 16, 16, True, 1.0),          # one token
    (1, 8, 2, 128, 600, 200, 200, False, 0.125),   # D = 128, fp32 inputs (flash.hip)
]


@pytest.mark.parametrize("case", P1_CASES, ids=[str(i) for i in range(len(P1_CASES))])
def test_phase1_parity(case):
    B, Hq, Hkv, D, L, b, a, bf16, sc = case
    print(f"phase1 case {case}", flush=True)
    q, k, v = _qkv(11, B, Hq, Hkv, L, D, bf16, sc)
    scale = 1 / math.sqrt(D)
    o, lse = sa.phase1_blocklocal(to_dev(q), to_dev(k), to_dev(v), b, a, want_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = so.phase1(f64(q), f64(k), f64(v), b, a if b < L else 0, scale)
    wabs, _ = so.phase1(f64(q), f64(k), np.abs(f64(v)), b, a if b < L else 0, scale)
    check_out(host64(o), ref_o, "O", bf16_out=True, wabs=wabs)
    check_lse(host64(lse), ref_l, "LSE")


P1_ROPE_CASES = [
    # B, Hq, Hkv, L, b, a
    (2, 8, 2, 700, 200, 200),      # ragged tail, b % 64 != 0
    (1, 32, 8, 1000, 256, 256),    # Llama-8B heads
    (1, 8, 1, 333, 1000, 1000),    # one block
    (1, 16, 16, 130, 64, 0),       # MHA, no anchor
    (1, 8, 4, 450, 128, 128),      # g = 2: per-lane angles, 128 positions per workgroup
    (1, 32, 2, 300, 100, 100),     # g = 16: cos/sin table, two head groups per KV head
]


@pytest.mark.parametrize("case", P1_ROPE_CASES, ids=[str(i) for i in range(len(P1_ROPE_CASES))])
def test_phase1_rope_parity(case):
    """Phase 1 with the RoPE of Q done in the kernel against the oracle
    (Q rotated exactly in fp64 at positions 0..L-1, rounded to bf16), and
    against the two-pass GPU path (star_rope_apply, then Phase 1), which it
    must equal bit for bit."""
    B, Hq, Hkv, L, b, a = case
    D, base = 128, 500000.0
    print(f"phase1 rope case {case}", flush=True)
    q, k, v = _qkv(17, B, Hq, Hkv, L, D, True, 1.0)
    pos = np.arange(L)
    k_rot = so.round_bf16(so.rope(f64(k), pos, base))
    kd = to_dev(k_rot.astype(np.float32)).to(torch.bfloat16)
    qd, vd = to_dev(q), to_dev(v)
    scale = 1 / math.sqrt(D)
    o, lse = sa.phase1_rope(qd, kd, vd, b, a, base, want_lse=True)
    qr = sa.rope_apply(qd, pos0=0, base=base, out=torch.empty_like(qd))
    o2, lse2 = sa.phase1_blocklocal(qr, kd, vd, b, a,
                                    want_lse=True)
    torch.cuda.synchronize()
    q_rot = so.round_bf16(so.rope(f64(q), pos, base))
    ref_o, ref_l = so.phase1(q_rot, k_rot, f64(v), b, a if b < L else 0, scale)
    wabs, _ = so.phase1(q_rot, k_rot, np.abs(f64(v)), b, a if b < L else 0, scale)
    check_out(host64(o), ref_o, "O (fused rope)", bf16_out=True, wabs=wabs)
    check_lse(host64(lse), ref_l, "LSE (fused rope)")
    check_out(host64(o2), ref_o, "O (two passes)", bf16_out=True, wabs=wabs)
    check_lse(host64(lse2), ref_l, "LSE (two passes)")
    # the in-kernel rotation is the RoPE kernel's, bit for bit
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


SCHED_CASES = [
    # B, Hq, Hkv, D, L, b, a, bf16
    (1, 32, 8, 128, 8192, 1024, 1024, True),   # 1024 items: queues drain and steal
    (2, 8, 2, 128, 700, 200, 200, True),       # ragged tail
    (1, 8, 1, 128, 100, 64, 64, True),         # 2 items: most queues empty
    (1, 4, 4, 64, 600, 256, 100, True),        # D = 64 kernel (ignores sched)
    (1, 2, 1, 64, 512, 128, 128, False),       # fp32 inputs (ignores sched)
]


@pytest.mark.parametrize("case", SCHED_CASES, ids=[str(i) for i in range(len(SCHED_CASES))])
def test_phase1_sched_identical(case):
    """With a scheduling workspace the items are handed out from per-XCD
    queues instead of a fixed order; the items are independent, so O and lse
    must be bit for bit those of the fixed order.  The workspace starts with
    junk (the call clears it itself) and is reused by back-to-back calls of
    all three Phase-1 entry points."""
    B, Hq, Hkv, D, L, b, a, bf16 = case
    print(f"phase1 sched case {case}", flush=True)
    q, k, v = (to_dev(t) for t in _qkv(23, B, Hq, Hkv, L, D, bf16, 1.0))
    sched = torch.full((sa.SCHED_INTS,), 12345, dtype=torch.int32, device=q.device)
    sched[::3] = -7

    def nan_out():
        # outputs start as NaN, so an item the queues never hand out shows
        o = torch.full((B, Hq, L, D), float("nan"), dtype=torch.bfloat16, device=q.device)
        return o, torch.full((B, Hq, L), float("nan"), dtype=torch.float32, device=q.device)

    o0, l0 = sa.phase1_blocklocal(q, k, v, b, a, want_lse=True)
    for rep in range(3):
        o1, l1 = nan_out()
        sa.phase1_blocklocal(q, k, v, b, a, out=o1, lse=l1, sched=sched)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1), f"blocklocal, call {rep}"
    n = -(-L // b)
    st, ln = [0] * n, [0] + [min(a, L)] * (n - 1)
    p0, pl0 = sa.phase1_prefix(q, k, v, k, v, st, ln, b, want_lse=True)
    p1, pl1 = nan_out()
    sa.phase1_prefix(q, k, v, k, v, st, ln, b, out=p1, lse=pl1, sched=sched)
    torch.cuda.synchronize()
    assert torch.equal(p0, p1) and torch.equal(pl0, pl1), "prefix"
    if D == 128 and bf16:
        r0, rl0 = sa.phase1_rope(q, k, v, b, a, want_lse=True)
        r1, rl1 = nan_out()
        sa.phase1_rope(q, k, v, b, a, out=r1, lse=rl1, sched=sched)
        torch.cuda.synchronize()
        assert torch.equal(r0, r1) and torch.equal(rl0, rl1), "rope"


def test_phase1_sched_argument_checks():
    q, k, v = (to_dev(t) for t in _qkv(5, 1, 2, 1, 64, 128, True, 1.0))
    for bad in (torch.zeros(sa.SCHED_INTS, dtype=torch.int64, device=q.device),
                torch.zeros(sa.SCHED_INTS - 1, dtype=torch.int32, device=q.device),
                torch.zeros(sa.SCHED_INTS),
                torch.zeros(2 * sa.SCHED_INTS, dtype=torch.int32, device=q.device)[::2]):
        with pytest.raises(ValueError):
            sa.phase1_blocklocal(q, k, v, 16, 16, sched=bad)


# (q scale, k scale at position 0, k scale at the last position)
RESCALE_CASES = [(2.0, 2.0, 8.0), (2.0, 8.0, 2.0), (6.0, 6.0, 6.0)]


@pytest.mark.parametrize("case", RESCALE_CASES, ids=["growing", "shrinking", "overflow"])
def test_phase1_rescale_stress(case):
    """Large scores for the lazy online softmax: scores that keep growing
    along the keys (the running max passes its shift many times), that keep
    shrinking, and that are large enough (std ~52 in log2 units) that P of
    the first sub-tile, formed before any shift is known, overflows fp32.
    V is drawn at scale 0.5 so that the bf16 rounding of P (2^-9 of each
    weight) stays inside the output bound when the attention is peaked."""
    qs, k0, k1 = case
    B, Hq, Hkv, D, L, b, a = 1, 8, 2, 128, 1100, 300, 300
    print(f"phase1 rescale case {case}", flush=True)
    q = so.round_bf16(rand_tensor(41, 0, B, Hq, L, D, qs, False).astype(np.float64))
    ramp = np.linspace(k0, k1, L)[None, None, :, None]
    k = so.round_bf16(rand_tensor(41, 1, B, Hkv, L, D, 1.0, False).astype(np.float64) * ramp)
    v = so.round_bf16(rand_tensor(41, 2, B, Hkv, L, D, 0.5, False).astype(np.float64))
    dev = lambda t: to_dev(t.astype(np.float32)).to(torch.bfloat16)
    scale = 1 / math.sqrt(D)
    o, lse = sa.phase1_blocklocal(dev(q), dev(k), dev(v), b, a, want_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = so.phase1(q, k, v, b, a, scale)
    wabs, _ = so.phase1(q, k, np.abs(v), b, a, scale)
    check_out(host64(o), ref_o, "O", bf16_out=True, wabs=wabs)
    check_lse(host64(lse), ref_l, "LSE")


@pytest.mark.parametrize("wg,mib", [(64, 4), (1, 1), (4096, 128)])
def test_stream_read_checksum(wg, mib):
    """The streaming-read aid reads every 32-bit word once: workgroup i's
    result is the XOR of the words of slice i (bit-exact)."""
    g = torch.Generator().manual_seed(wg)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (mib << 18,), dtype=torch.int32, generator=g)
    out = sa.stream_read(words.cuda(), workgroups=wg)
    torch.cuda.synchronize()
    ref = np.bitwise_xor.reduce(words.numpy().view(np.uint32).reshape(wg, -1), axis=1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref)


P2_CASES = [
    # B, Hq, Hkv, D, L, Lq, b, splits
    (1, 2, 1, 64, 512, 16, 128, 1),     # tiny workload query phase (flash path)
    (1, 2, 1, 64, 512, 16, 128, 3),
    (1, 32, 8, 128, 1000, 64, 300, 2),  # flash path, ragged partitions
    (2, 8, 2, 128, 777, 1, 200, 4),     # decode path (g*Lq = 4)
    (1, 16, 2, 128, 500, 2, 128, 3),    # decode path, g*Lq = 16
    (1, 4, 1, 64, 300, 1, 100, 8),      # decode path, D = 64, empty chunks
    (1, 24, 8, 128, 400, 5, 90, 2),     # decode path, g = 3, Lq = 5
    (1, 8, 1, 128, 300, 3, 64, 16),     # flash path (g*Lq = 24), many empty chunks
    (2, 8, 2, 128, 777, 1, 200, 4, False),   # decode path, fp32 inputs (rounded at load)
    (1, 4, 1, 64, 300, 1, 100, 8, False),    # decode path, D = 64, fp32 inputs
    (1, 16, 2, 128, 500, 16, 128, 2, False),  # flash path (g*Lq = 128), D = 128, fp32 inputs
    # 4-wave flash instance (g <= 4, g*Lq <= 128, bf16, D = 128)
    (1, 32, 8, 128, 1000, 32, 300, 2),  # g = 4, 128 rows, ragged chunks (5 tiles + tail)
    (1, 8, 2, 128, 384, 32, 192, 2),    # chunks of 96 keys: whole 3-tile cycles
    (1, 8, 2, 128, 512, 32, 256, 2),    # chunks of 128 keys: one tile past a cycle
    (1, 8, 4, 128, 777, 20, 200, 3),    # g = 2, 40 rows: two column blocks per head
    (2, 12, 4, 128, 901, 9, 256, 5),    # g = 3: the fourth wave has no column block
    (1, 4, 4, 128, 640, 40, 160, 2),    # g = 1, 40 rows: waves 2, 3 idle
    (1, 8, 2, 128, 500, 33, 128, 2),    # g*Lq = 132: just past it, the 8-wave instance
]


@pytest.mark.parametrize("case", P2_CASES, ids=[str(i) for i in range(len(P2_CASES))])
def test_phase2_partials_and_merge(case):
    B, Hq, Hkv, D, L, Lq, b, splits = case[:8]
    bf16 = case[8] if len(case) > 8 else True
    print(f"phase2 case {case}", flush=True)
    g = Hq // Hkv
    N = L + Lq
    # fp32 inputs are rounded to bf16 at load while the oracle reads them
    # exactly; at the Tiny workload's scale that quantisation stays inside
    # the tolerances
    sc = 1.0 if bf16 else 0.125
    q = rand_tensor(21, 3, B, Hq, Lq, D, sc, bf16)
    kc = rand_tensor(21, 4, B, Hkv, N + 7, D, sc, bf16)   # spare rows past the cache end
    vc = rand_tensor(21, 5, B, Hkv, N + 7, D, sc, bf16)
    parts = so.partitions(L, b, N)
    offs = [p[0] for p in parts] + [parts[-1][1]]
    scale = 1 / math.sqrt(D)
    op, lp = sa.phase2_partial(to_dev(q), to_dev(kc), to_dev(vc), offs, splits, q_pos0=L)
    o, l = sa.lse_merge(op, lp)
    torch.cuda.synchronize()
    ranges = chunk_ranges(offs, splits)
    assert len(ranges) == op.shape[0]
    qf, kf, vf = f64(q), f64(kc), f64(vc)
    qpos = L + np.arange(Lq)
    ref_op = np.zeros(op.shape)
    ref_lp = np.zeros(lp.shape)
    ref_o = np.zeros(o.shape)
    ref_l = np.zeros(l.shape)
    for bb in range(B):
        for h in range(Hq):
            for c, (k0, k1) in enumerate(ranges):
                ro, rl = so.partial(qf[bb, h], qpos, kf[bb, h // g], vf[bb, h // g], k0, k1, scale)
                ref_op[c, bb, h], ref_lp[c, bb, h] = ro, rl
            ro, rl, _, _ = so.phase2(qf[bb, h], qpos, kf[bb, h // g], vf[bb, h // g], parts, scale)
            ref_o[bb, h], ref_l[bb, h] = ro, rl
    check_out(host64(op), ref_op, "o_part")
    check_lse(host64(lp), ref_lp, "lse_part")
    check_out(host64(o), ref_o, "O merged")
    check_lse(host64(l), ref_l, "LSE merged")


@pytest.mark.parametrize("N,D,out_bf16", [(4, 64, False), (37, 128, True), (300, 128, False)])
def test_merge_parity(N, D, out_bf16):
    """Merge partials the oracle produced (random key ranges, some empty)."""
    rng = np.random.default_rng(N)
    B, H, S, M = 1, 3, 5, 200
    q = rng.standard_normal((B, H, S, D))
    k = rng.standard_normal((M, D))
    v = rng.standard_normal((M, D))
    cuts = np.sort(rng.integers(0, M + 1, size=N - 1))
    bounds = [0, *cuts.tolist(), M]
    op = np.zeros((N, B, H, S, D))
    lp = np.zeros((N, B, H, S))
    for n in range(N):
        for h in range(H):
            o, l = so.attend(q[0, h], k[bounds[n]:bounds[n + 1]], v[bounds[n]:bounds[n + 1]],
                             np.ones((S, bounds[n + 1] - bounds[n]), bool), 1 / math.sqrt(D))
            op[n, 0, h], lp[n, 0, h] = o, l
    ref_o, ref_l = so.lse_merge(op, lp)
    o, l = sa.lse_merge(torch.from_numpy(op.astype(np.float32)).cuda(),
                        torch.from_numpy(lp.astype(np.float32)).cuda(),
                        out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    check_out(host64(o), ref_o, "merged O")
    check_lse(host64(l), ref_l, "merged LSE")


def bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a device tensor (uint16 for bf16, uint32 for fp32)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def rot_bits(x64: np.ndarray, pos, base: float, f32: bool) -> np.ndarray:
    """The oracle's exact rotation rounded once to the stored dtype, as bits."""
    r = so.rope(x64, np.asarray(pos), base)
    if f32:
        return r.astype(np.float32).view(np.uint32)           # one RNE rounding
    return so.round_bf16(r).astype(np.float32).view(np.uint32) >> 16


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str):
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, f"{what}: {bad[0].size} elements differ, first at {list(zip(*bad))[:6]}"


ROPE_BIT_CASES = [
    # D, f32, positions
    (128, False, np.arange(0, 4096)),                          # block starts, small angles
    (128, False, np.arange(131072 - 2048, 131072 + 192)),      # the 128K context end
    (128, False, np.arange(1048576 - 64, 1048576 + 64)),       # around 2^20
    (128, True, np.arange(1048576 - 64, 1048576 + 64)),
    (64, False, np.sort(np.random.default_rng(3).choice(2 ** 21, 3000, replace=False))),
    (16, True, np.arange(0, 300) * 7919),
]


@pytest.mark.parametrize("case", ROPE_BIT_CASES, ids=[str(i) for i in range(len(ROPE_BIT_CASES))])
def test_rope_bit_exact(case):
    """star_rope_apply stores the exact rotation rounded once (nearest even)
    to the tensor's dtype: the same bits as the oracle's fp64 rotation
    rounded once, over context, query and million-token positions, with a
    contiguous range and with a position list."""
    D, f32, pos = case
    base = 500000.0
    B, H, S = 2, 8, pos.size
    x = rand_tensor(31, 0, B, H, S, D, bf16=not f32)
    xd = to_dev(x)
    contiguous = bool(np.all(np.diff(pos) == 1))
    out1 = sa.rope_apply(xd, pos0=int(pos[0]), base=base, out=torch.empty_like(xd)) \
        if contiguous else None
    out2 = sa.rope_apply(xd, pos=torch.from_numpy(pos).cuda(), base=base,
                         out=torch.empty_like(xd))
    torch.cuda.synchronize()
    ref = rot_bits(f64(x), pos, base, f32)
    for o in (out1, out2):
        if o is not None:
            got = bits(o).astype(np.uint32)
            assert_bits_equal(got, ref, f"rope D={D} f32={f32}")


def test_rope_freqs_match_the_oracle():
    for D in (16, 64, 128):
        assert sa.rope_freqs(D, 500000.0) == so.rope_theta(D, 500000.0).tolist()


def test_kv_append_parity():
    B, H, T, D, S = 2, 4, 5, 128, 40
    kn = rand_tensor(41, 7, B, H, T, D)
    vn = rand_tensor(41, 8, B, H, T, D)
    kc = torch.zeros((B, H, S, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    sa.kv_append(to_dev(kn), to_dev(vn), kc, vc, slot0=30, pos0=123456, base=500000.0)
    torch.cuda.synchronize()
    got = bits(kc).astype(np.uint32)
    assert_bits_equal(got[:, :, 30:35], rot_bits(f64(kn), 123456 + np.arange(T), 500000.0, False),
                      "appended K")
    assert np.array_equal(host64(vc)[:, :, 30:35], f64(vn))
    assert (host64(kc)[:, :, :30] == 0).all() and (host64(kc)[:, :, 35:] == 0).all()


@pytest.mark.parametrize("rope", [True, False])
def test_decode_prepare_parity(rope):
    """rope(q) + KV append in one launch stores the oracle's rotation rounded
    once, bit for bit, and leaves the rest of the cache untouched."""
    B, Hq, Hkv, T, D, S = 2, 8, 2, 3, 128, 50
    qn = rand_tensor(43, 6, B, Hq, T, D)
    kn = rand_tensor(43, 7, B, Hkv, T, D)
    vn = rand_tensor(43, 8, B, Hkv, T, D)
    qo = torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, S, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pos0 = 1048000
    sa.decode_prepare(to_dev(qn), qo, to_dev(kn), to_dev(vn), kc, vc, slot0=40, pos0=pos0,
                      base=500000.0, rope=rope)
    torch.cuda.synchronize()
    pos = pos0 + np.arange(T)
    if rope:
        assert_bits_equal(bits(qo).astype(np.uint32), rot_bits(f64(qn), pos, 500000.0, False), "q")
        assert_bits_equal(bits(kc).astype(np.uint32)[:, :, 40:43],
                          rot_bits(f64(kn), pos, 500000.0, False), "k")
    else:
        assert np.array_equal(host64(qo), f64(qn))
        assert np.array_equal(host64(kc)[:, :, 40:43], f64(kn))
    assert np.array_equal(host64(vc)[:, :, 40:43], f64(vn))
    assert (host64(kc)[:, :, :40] == 0).all() and (host64(kc)[:, :, 43:] == 0).all()


DSTEP_CASES = [
    # B, Hq, Hkv, D, L, b, splits, rope, T
    (2, 8, 2, 128, 777, 200, 4, True, 5),
    (1, 16, 1, 64, 300, 100, 8, False, 3),      # g = 16, D = 64, empty chunks
    (1, 32, 8, 128, 2000, 512, 3, True, 4),
    (1, 4, 4, 128, 70, 64, 1, True, 2),         # MHA, short context
]


@pytest.mark.parametrize("case", DSTEP_CASES, ids=[str(i) for i in range(len(DSTEP_CASES))])
def test_decode_step_parity(case):
    """The fused decode step (rope, append and partials in one launch, then
    the merge) against the oracle's global attention and cache over several
    consecutive tokens, and against the unfused call sequence."""
    from block_sparse_amd.pipeline import StarAttentionStep
    B, Hq, Hkv, D, L, b, splits, rope, T = case
    print(f"decode_step case {case}", flush=True)
    g = Hq // Hkv
    base = 500000.0
    q = rand_tensor(51, 0, B, Hq, L, D)
    k = rand_tensor(51, 1, B, Hkv, L, D)
    v = rand_tensor(51, 2, B, Hkv, L, D)
    qd = rand_tensor(51, 6, B, Hq, T, D)
    kd = rand_tensor(51, 7, B, Hkv, T, D)
    vd = rand_tensor(51, 8, B, Hkv, T, D)
    outs = []
    for fused in (True, False):
        st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, T, rope=rope, base=base,
                               splits_decode=splits, fused_decode=fused)
        st.load_context(to_dev(v))
        st.rope_context(to_dev(q), to_dev(k))
        dq, dk, dv = to_dev(qd), to_dev(kd), to_dev(vd)
        for t in range(T):
            st.decode(t, dq[:, :, t:t + 1], dk[:, :, t:t + 1], dv[:, :, t:t + 1])
        torch.cuda.synchronize()
        outs.append((host64(st.od), host64(st.lsed), host64(st.kc), host64(st.vc)))
    (o_f, l_f, kc_f, vc_f), (o_u, l_u, kc_u, vc_u) = outs
    pos_c = np.arange(L)
    pos_d = L + np.arange(T)
    rot = (lambda x, p: so.round_bf16(so.rope(x, p, base))) if rope else (lambda x, p: x)
    K = np.concatenate([rot(f64(k), pos_c), rot(f64(kd), pos_d)], axis=2)
    V = np.concatenate([f64(v), f64(vd)], axis=2)
    # the appended rows: rotated k (the exact rotation rounded once, the same
    # bits on the fused and unfused paths) and v
    assert np.array_equal(kc_f[:, :, L:L + T], K[:, :, L:])
    assert np.array_equal(kc_u[:, :, L:L + T], K[:, :, L:])
    assert np.array_equal(vc_f[:, :, L:L + T], f64(vd))
    Qd = rot(f64(qd), pos_d)
    ref_o = np.zeros((B, Hq, T, D))
    ref_l = np.zeros((T, B, Hq))
    for t in range(T):
        parts = so.partitions(L, b, L + t + 1)
        for bb in range(B):
            for h in range(Hq):
                o, l, _, _ = so.phase2(Qd[bb, h, t:t + 1], pos_d[t:t + 1], K[bb, h // g],
                                       V[bb, h // g], parts, 1 / math.sqrt(D))
                ref_o[bb, h, t], ref_l[t, bb, h] = o[0], l[0]
    check_out(o_f[:, :, :T], ref_o, "fused O")
    check_lse(l_f[:T], ref_l, "fused LSE")
    check_out(o_u[:, :, :T], ref_o, "unfused O")
    assert np.abs(o_f[:, :, :T] - o_u[:, :, :T]).max() < 2e-3
    assert np.abs(l_f[:T] - l_u[:T]).max() < 2e-4


def test_phase1_many_small_blocks():
    """640 blocks of 16 tokens (anchor 16): far more blocks than the prefix
    table allows, on the analytic anchor path."""
    B, Hq, Hkv, D, L, b = 1, 8, 2, 128, 10240, 16
    print("phase1 640 blocks", flush=True)
    q, k, v = _qkv(81, B, Hq, Hkv, L, D)
    o, lse = sa.phase1_blocklocal(to_dev(q), to_dev(k), to_dev(v), b, b, want_lse=True)
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(0, 48), np.arange(5000, 5040), np.arange(L - 40, L)])
    for h in (0, 5):
        qq = f64(q)[0, h][pos]
        ro, rl, wabs = with_wabs(so.phase1_rows, f64(v)[0, h // 4], qq, pos, f64(k)[0, h // 4],
                                 b, b, 1 / math.sqrt(D), v_index=3)
        check_out(host64(o)[0, h][pos], ro, "O", bf16_out=True, wabs=wabs)
        check_lse(host64(lse)[0, h][pos], rl, "LSE")


def test_phase1_prefix_at_the_block_limit():
    """A prefix table of STAR_MAX_PARTS = 128 blocks."""
    B, Hq, Hkv, D, b = 1, 4, 1, 128, 32
    L = 128 * b
    R = 200
    print("phase1 prefix 128 blocks", flush=True)
    q, k, v = _qkv(82, B, Hq, Hkv, L, D)
    pk, pv = rand_tensor(82, 3, B, Hkv, R, D), rand_tensor(82, 4, B, Hkv, R, D)
    rng = np.random.default_rng(82)
    st = rng.integers(0, R, size=128)
    ln = np.array([rng.integers(0, R - s + 1) for s in st])
    o, lse = sa.phase1_prefix(to_dev(q), to_dev(k), to_dev(v), to_dev(pk), to_dev(pv), st, ln,
                              b, want_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = so.phase1_prefix(f64(q), f64(k), f64(v), f64(pk), f64(pv), st, ln, b,
                                    1 / math.sqrt(D))
    wabs, _ = so.phase1_prefix(f64(q), f64(k), np.abs(f64(v)), f64(pk), np.abs(f64(pv)), st, ln,
                               b, 1 / math.sqrt(D))
    check_out(host64(o), ref_o, "O", bf16_out=True, wabs=wabs)
    check_lse(host64(lse), ref_l, "LSE")
    with pytest.raises(sa.StarError):                   # 133 blocks: refused before any launch
        sa.phase1_prefix(to_dev(q), to_dev(k), to_dev(v), to_dev(pk), to_dev(pv),
                         np.zeros(133, np.int64), np.zeros(133, np.int64), 31)


@pytest.mark.parametrize("Lq,splits", [(1, 8), (64, 2)])
def test_phase2_at_the_partition_limit(Lq, splits):
    """128 partitions (the limit) x splits chunks, merged: decode and flash
    paths; the merge combines up to 1024 partials per row."""
    B, Hq, Hkv, D, b = 1, 8, 2, 128, 64
    L = 128 * b - 30                                  # ragged last partition
    print(f"phase2 128 partitions Lq={Lq} splits={splits}", flush=True)
    N = L + Lq
    q = rand_tensor(83, 3, B, Hq, Lq, D)
    kc = rand_tensor(83, 4, B, Hkv, N, D)
    vc = rand_tensor(83, 5, B, Hkv, N, D)
    parts = so.partitions(L, b, N)
    assert len(parts) == 128
    offs = [p[0] for p in parts] + [parts[-1][1]]
    op, lp = sa.phase2_partial(to_dev(q), to_dev(kc), to_dev(vc), offs, splits, q_pos0=L)
    o, l = sa.lse_merge(op, lp)
    torch.cuda.synchronize()
    qpos = L + np.arange(Lq)
    for h in (0, 7):
        ro, rl, _, _ = so.phase2(f64(q)[0, h], qpos, f64(kc)[0, h // 4], f64(vc)[0, h // 4],
                                 parts, 1 / math.sqrt(D))
        check_out(host64(o)[0, h], ro, "O merged")
        check_lse(host64(l)[0, h], rl, "LSE merged")


def test_decode_step_max_splits():
    """One partition cut into the maximum 1024 chunks (most of them empty)."""
    from block_sparse_amd.pipeline import StarAttentionStep
    B, Hq, Hkv, D, L, b = 1, 4, 1, 128, 700, 1000
    print("decode_step splits=1024", flush=True)
    q = rand_tensor(84, 0, B, Hq, L, D)
    k = rand_tensor(84, 1, B, Hkv, L, D)
    v = rand_tensor(84, 2, B, Hkv, L, D)
    qd, kd, vd = (rand_tensor(84, t, B, H, 1, D) for t, H in ((6, Hq), (7, Hkv), (8, Hkv)))
    st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, 1, splits_decode=1024)
    st.load_context(to_dev(v))
    st.rope_context(to_dev(q), to_dev(k))
    st.decode(0, to_dev(qd), to_dev(kd), to_dev(vd))
    torch.cuda.synchronize()
    rot = lambda x, p: so.round_bf16(so.rope(x, p, st.base))
    K = np.concatenate([rot(f64(k), np.arange(L)), rot(f64(kd), [L])], axis=2)
    V = np.concatenate([f64(v), f64(vd)], axis=2)
    qr = rot(f64(qd), [L])
    for h in range(Hq):
        ro, rl, _, _ = so.phase2(qr[0, h], np.array([L]), K[0, 0], V[0, 0],
                                 so.partitions(L, b, L + 1), 1 / math.sqrt(D))
        check_out(host64(st.od)[0, h, :1], ro, "decode O")
        check_lse(host64(st.lsed)[0, 0, h:h + 1], rl, "decode LSE")
