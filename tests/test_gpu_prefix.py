"""GPU parity of the Phase-1 prefix variants through the C ABI: the
explicit per-block prefix table (flash kernels of both head dims and both
input dtypes), the row gather, the anchor at other position ids and the
Pulsar prefix (host-side Max-IDF selection + gather + prefix attention),
each against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import block_sparse_amd as sa
import oracle.star_oracle as so
from block_sparse_amd.pipeline import StarAttentionStep
from gpu_util import check_lse, check_out, f64, host64, rand_tensor, to_dev
from workloads import anchor_positions, token_ids

pytestmark = pytest.mark.gpu

PREFIX_CASES = [
    # B, Hq, Hkv, D, L, b, R, bf16, seed
    (1, 8, 2, 128, 700, 200, 300, True, 1),      # flash2 path, ragged tail
    (2, 4, 4, 128, 512, 128, 64, True, 2),       # MHA, short prefixes
    (1, 6, 2, 64, 450, 100, 500, True, 3),       # D = 64 (v1 kernel)
    (1, 4, 1, 128, 333, 64, 97, False, 4),       # fp32 inputs (v1 kernel), tiny's N(0,1)/8
    (1, 16, 1, 128, 130, 1000, 50, True, 5),     # one block with a prefix
]


def _table(seed, n, R, bf):
    rng = np.random.default_rng(seed)
    st = rng.integers(0, R, size=n)
    ln = np.array([rng.integers(0, R - s + 1) for s in st])
    if n > 2:
        ln[1] = 0                                   # a block without prefix
        st[2], ln[2] = R - 1, 1                     # a one-key prefix at the end
    return st, ln


@pytest.mark.parametrize("case", PREFIX_CASES, ids=[str(i) for i in range(len(PREFIX_CASES))])
def test_phase1_prefix_parity(case):
    B, Hq, Hkv, D, L, b, R, bf, seed = case
    print(f"phase1_prefix case {case}", flush=True)
    # fp32 inputs are the tiny workload's (N(0,1)/8): the kernels round them
    # to bf16 on load, and the tolerance covers that only at that scale
    sc = 1.0 if bf else 0.125
    q = rand_tensor(seed, 0, B, Hq, L, D, sc, bf16=bf)
    k = rand_tensor(seed, 1, B, Hkv, L, D, sc, bf16=bf)
    v = rand_tensor(seed, 2, B, Hkv, L, D, sc, bf16=bf)
    pk = rand_tensor(seed, 3, B, Hkv, R, D, sc, bf16=bf)
    pv = rand_tensor(seed, 4, B, Hkv, R, D, sc, bf16=bf)
    n = -(-L // b)
    st, ln = _table(seed, n, R, bf)
    o, lse = sa.phase1_prefix(to_dev(q), to_dev(k), to_dev(v), to_dev(pk), to_dev(pv), st, ln,
                              b, want_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = so.phase1_prefix(f64(q), f64(k), f64(v), f64(pk), f64(pv), st, ln, b,
                                    1 / math.sqrt(D))
    wabs, _ = so.phase1_prefix(f64(q), f64(k), np.abs(f64(v)), f64(pk), np.abs(f64(pv)), st, ln,
                               b, 1 / math.sqrt(D))
    check_out(host64(o), ref_o, "O", bf16_out=True, wabs=wabs)
    check_lse(host64(lse), ref_l, "LSE")


@pytest.mark.parametrize("D,a", [(128, 200), (128, 57), (64, 100)])
def test_prefix_table_of_the_anchor_equals_blocklocal(D, a):
    """The anchor expressed as a prefix table (pk = k) runs the same key
    ranges as star_phase1_blocklocal: identical bits."""
    B, Hq, Hkv, L, b = 1, 8, 2, 650, 200
    print(f"anchor table D={D} a={a}", flush=True)
    q, k, v = (to_dev(rand_tensor(6, t, B, H, L, D)) for t, H in ((0, Hq), (1, Hkv), (2, Hkv)))
    st, ln = so.anchor_prefix_table(L, b, a)
    o1, l1 = sa.phase1_prefix(q, k, v, k, v, st, ln, b, want_lse=True)
    o2, l2 = sa.phase1_blocklocal(q, k, v, b, a, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("bf16,D", [(True, 128), (False, 64), (True, 64)])
def test_gather_rows_parity(bf16, D):
    B, H, S, R = 2, 3, 100, 37
    print(f"gather bf16={bf16} D={D}", flush=True)
    src = rand_tensor(7, 0, B, H, S, D, bf16=bf16)
    rows = np.random.default_rng(8).integers(0, S, size=R)
    rows[3], rows[10], rows[20] = -1, S, S + 1000       # out of range -> zero rows
    big = torch.full((B, H, R + 5, D), 7.0, dtype=torch.bfloat16 if bf16 else torch.float32,
                     device="cuda")
    dst = big[:, :, 2:2 + R]                            # a strided view
    sa.gather_rows(to_dev(src), torch.from_numpy(rows).cuda(), out=dst)
    torch.cuda.synchronize()
    ref = f64(src)[:, :, np.clip(rows, 0, S - 1)]
    ref[:, :, (rows < 0) | (rows >= S)] = 0.0
    assert np.array_equal(host64(dst), ref)             # pure data movement: bit-exact
    assert (host64(big[:, :, :2]) == 7.0).all() and (host64(big[:, :, 2 + R:]) == 7.0).all()


def test_anchor_at_other_positions_parity():
    """Anchor keys re-rotated at seeded random positions before each block
    (the position-id ablation), through the pipeline's own calls."""
    B, Hq, Hkv, D, L, b = 1, 8, 2, 128, 1024, 256
    print("anchor remap", flush=True)
    q = rand_tensor(9, 0, B, Hq, L, D)
    k = rand_tensor(9, 1, B, Hkv, L, D)
    v = rand_tensor(9, 2, B, Hkv, L, D)
    st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, 0)
    st.load_context(to_dev(v))
    st.rope_context(to_dev(q), to_dev(k))
    pos = anchor_positions(9, L, b, b)
    st.anchor_remap_setup(pos)
    st.phase1_anchor_remap(to_dev(k))
    torch.cuda.synchronize()
    P = np.arange(L)
    Q = so.round_bf16(so.rope(f64(q), P, st.base))
    K = so.round_bf16(so.rope(f64(k), P, st.base))
    PK = so.remapped_anchor(f64(k), pos, st.base)
    PV = np.concatenate([f64(v)[..., :b, :]] * len(pos), axis=-2)
    tab = (np.arange(len(pos)) * b, [0] + [b] * (len(pos) - 1))
    ref_o, ref_l = so.phase1_prefix(Q, K, f64(v), PK, PV, *tab, b, 1 / math.sqrt(D))
    wabs, _ = so.phase1_prefix(Q, K, np.abs(f64(v)), PK, np.abs(PV), *tab, b, 1 / math.sqrt(D))
    check_out(host64(st.o1), ref_o, "O", bf16_out=True, wabs=wabs)
    check_lse(host64(st.lse1), ref_l, "LSE")


@pytest.mark.parametrize("B,L,b,k", [(1, 2048, 512, 2), (2, 1500, 400, 3)])
def test_pulsar_phase1_parity(B, L, b, k):
    """Pulsar's Phase 1: library selection + gather + prefix attention vs the
    oracle's selection and attention."""
    Hq, Hkv, D = 8, 2, 128
    print(f"pulsar B={B} L={L} b={b} k={k}", flush=True)
    q = rand_tensor(10, 0, B, Hq, L, D)
    kk = rand_tensor(10, 1, B, Hkv, L, D)
    v = rand_tensor(10, 2, B, Hkv, L, D)
    tok = token_ids(10, B, L)
    st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, 0)
    st.load_context(to_dev(v))
    st.rope_context(to_dev(q), to_dev(kk))
    st.pulsar_setup(tok, 32, 64, k)
    st.phase1_pulsar()
    torch.cuda.synchronize()
    P = np.arange(L)
    Q = so.round_bf16(so.rope(f64(q), P, st.base))
    K = so.round_bf16(so.rope(f64(kk), P, st.base))
    V = f64(v)
    for bb in range(B):
        rows, s0, l0 = so.pulsar_prefix(tok[bb], L, b, 32, 64, k)
        ref_o, ref_l = so.phase1_prefix(Q[bb:bb + 1], K[bb:bb + 1], V[bb:bb + 1],
                                        K[bb:bb + 1][:, :, rows], V[bb:bb + 1][:, :, rows],
                                        s0, l0, b, 1 / math.sqrt(D))
        Va = np.abs(V[bb:bb + 1])
        wabs, _ = so.phase1_prefix(Q[bb:bb + 1], K[bb:bb + 1], Va, K[bb:bb + 1][:, :, rows],
                                   Va[:, :, rows], s0, l0, b, 1 / math.sqrt(D))
        check_out(host64(st.o1[bb:bb + 1]), ref_o, f"O b={bb}", bf16_out=True, wabs=wabs)
        check_lse(host64(st.lse1[bb:bb + 1]), ref_l, f"LSE b={bb}")
