"""Pins of the oracle's Phase-1 prefix variants: the explicit prefix table,
the re-rotated anchor of the position-id ablation and the Pulsar prefix
(attention sink + Max-IDF chunk summaries).  Each function is checked
against something other than itself: torch's SDPA in float64, the Star
oracle it must reduce to, rotation-group identities, hand-derived chunk
selections and the lengths the Pulsar review prints."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.star_oracle as so

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------
# prefix table
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,b,a", [(300, 64, 64), (300, 64, 20), (256, 64, 0), (100, 128, 128)])
def test_prefix_table_reduces_to_star_anchor(L, b, a):
    B, Hq, Hkv, D = 1, 4, 2, 16
    Q, K, V = rnd(1, B, Hq, L, D), rnd(2, B, Hkv, L, D), rnd(3, B, Hkv, L, D)
    st, ln = so.anchor_prefix_table(L, b, a)
    o1, l1 = so.phase1_prefix(Q, K, V, K, V, st, ln, b, 0.25)
    o2, l2 = so.phase1(Q, K, V, b, a if b < L else 0, 0.25)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


def test_prefix_matches_sdpa_on_materialised_blocks():
    """Every block equals SDPA over [PK rows ; own block] with the explicit
    mask (prefix all visible, block causal)."""
    B, Hq, Hkv, D, L, b, R = 2, 6, 2, 32, 200, 48, 90
    Q, K, V = rnd(4, B, Hq, L, D), rnd(5, B, Hkv, L, D), rnd(6, B, Hkv, L, D)
    PK, PV = rnd(7, B, Hkv, R, D), rnd(8, B, Hkv, R, D)
    n = -(-L // b)
    rng = np.random.default_rng(9)
    st = rng.integers(0, R, size=n)
    ln = np.array([rng.integers(0, R - s + 1) for s in st])
    ln[1] = 0                                      # one block without prefix
    scale = 1 / math.sqrt(D)
    O, LSE = so.phase1_prefix(Q, K, V, PK, PV, st, ln, b, scale)
    g = Hq // Hkv
    for i, s in enumerate(range(0, L, b)):
        e = min(s + b, L)
        p0, p1 = st[i], st[i] + ln[i]
        for bb in range(B):
            for h in range(Hq):
                kv = h // g
                kk = torch.from_numpy(np.concatenate([PK[bb, kv, p0:p1], K[bb, kv, s:e]]))
                vv = torch.from_numpy(np.concatenate([PV[bb, kv, p0:p1], V[bb, kv, s:e]]))
                nb, npf = e - s, p1 - p0
                m = torch.ones(nb, npf + nb, dtype=torch.bool)
                m[:, npf:] = torch.tril(torch.ones(nb, nb, dtype=torch.bool))
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(Q[bb, h, s:e])[None], kk[None], vv[None],
                    attn_mask=m[None], scale=scale)[0].numpy()
                assert np.allclose(O[bb, h, s:e], ref, atol=1e-12)
                sc = (Q[bb, h, s:e] @ kk.numpy().T) * scale
                sc = np.where(m.numpy(), sc, -np.inf)
                mx = sc.max(1)
                lse = mx + np.log(np.exp(sc - mx[:, None]).sum(1))
                assert np.allclose(LSE[bb, h, s:e], lse, atol=1e-12)


def test_prefix_closed_form_two_keys():
    """Row 0 of a block with a one-key prefix sees exactly two keys."""
    D, L, b = 8, 64, 32
    Q, K, V = rnd(10, 1, 1, L, D), rnd(11, 1, 1, L, D), rnd(12, 1, 1, L, D)
    PK, PV = rnd(13, 1, 1, 5, D), rnd(14, 1, 1, 5, D)
    st, ln = np.array([0, 3]), np.array([0, 1])
    O, LSE = so.phase1_prefix(Q, K, V, PK, PV, st, ln, b, 1.0)
    q = Q[0, 0, 32]
    s1, s2 = q @ PK[0, 0, 3], q @ K[0, 0, 32]
    w1, w2 = math.exp(s1), math.exp(s2)
    assert np.allclose(O[0, 0, 32], (w1 * PV[0, 0, 3] + w2 * V[0, 0, 32]) / (w1 + w2))
    assert math.isclose(LSE[0, 0, 32], math.log(w1 + w2), rel_tol=1e-12)
    # block 0 has no prefix: its row 0 sees only itself
    assert np.allclose(O[0, 0, 0], V[0, 0, 0])
    assert math.isclose(LSE[0, 0, 0], Q[0, 0, 0] @ K[0, 0, 0], rel_tol=1e-12)


def test_prefix_rows_match_full():
    D, L, b, R = 16, 150, 40, 30
    Q, K, V = rnd(15, 1, 1, L, D), rnd(16, 1, 1, L, D), rnd(17, 1, 1, L, D)
    PK, PV = rnd(18, 1, 1, R, D), rnd(19, 1, 1, R, D)
    st, ln = np.array([0, 5, 0, 10]), np.array([0, 20, 30, 7])
    O, LSE = so.phase1_prefix(Q, K, V, PK, PV, st, ln, b, 0.3)
    pos = np.array([0, 39, 40, 41, 79, 80, 119, 120, 149])
    o, l = so.phase1_prefix_rows(Q[0, 0, pos], pos, K[0, 0], V[0, 0], PK[0, 0], PV[0, 0],
                                 st, ln, b, 0.3)
    assert np.allclose(o, O[0, 0, pos], atol=1e-12) and np.allclose(l, LSE[0, 0, pos], atol=1e-12)


# ----------------------------------------------------------------------------
# anchor with other position ids
# ----------------------------------------------------------------------------
def test_remapped_anchor_at_original_positions_is_star():
    B, Hq, Hkv, D, L, b = 1, 4, 2, 32, 256, 64
    Qp, Kp, V = rnd(20, B, Hq, L, D), rnd(21, B, Hkv, L, D), rnd(22, B, Hkv, L, D)
    pos = np.arange(L)
    Q = so.round_bf16(so.rope(Qp, pos, 1e4))
    K = so.round_bf16(so.rope(Kp, pos, 1e4))
    n = L // b
    PK = so.remapped_anchor(Kp, [np.arange(b)] * n, 1e4)
    PV = np.concatenate([V[..., :b, :]] * n, axis=-2)
    st = np.arange(n) * b
    ln = np.array([0] + [b] * (n - 1))
    o1, l1 = so.phase1_prefix(Q, K, V, PK, PV, st, ln, b, 1 / math.sqrt(D))
    o2, l2 = so.phase1(Q, K, V, b, b, 1 / math.sqrt(D))
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


def test_remapped_anchor_rotation_composes():
    """R(p) k = R(p - p0) R(p0) k: an anchor key re-rotated at p equals the
    originally rotated key turned further by p - p0 (RoPE is a rotation
    group per frequency pair)."""
    D, a = 64, 16
    Kp = rnd(23, 1, 1, a, D)
    newpos = np.sort(np.random.default_rng(24).choice(5000, size=a, replace=False))
    got = so.remapped_anchor(Kp, [newpos], 5e5, store_bf16=False)
    orig = so.rope(Kp, np.arange(a), 5e5)
    th = so.rope_theta(D, 5e5)
    h = D // 2
    ang = (newpos - np.arange(a))[:, None] * th[None]
    z = (orig[..., :h] + 1j * orig[..., h:]) * np.exp(1j * ang)
    assert np.allclose(got, np.concatenate([z.real, z.imag], axis=-1), atol=1e-9)


# ----------------------------------------------------------------------------
# Pulsar: Max-IDF summaries and the prefix they form
# ----------------------------------------------------------------------------
def planted_tokens():
    """4 blocks of 128 tokens (4 chunks of 32 each), all the common token 7
    (in every block: IDF = log(4/4) = 0) except planted ids:
      block 0: 4004 in chunk 0 (inside the 64-token sink), 4005 in chunk 3
      block 1: 2002 in chunk 0 (also in block 3: IDF log 2), 1001 in chunk 2 (IDF log 4)
      block 2: 3003 in chunk 1 and 3004 in chunk 3 (both IDF log 4: a tie)
      block 3: 2002 in chunk 1 (IDF log 2)."""
    t = np.full(512, 7, dtype=np.int64)
    t[5] = 4004
    t[96 + 3] = 4005
    t[128 + 10] = 2002
    t[128 + 64 + 1] = 1001
    t[256 + 32 + 31] = 3003
    t[256 + 96] = 3004
    t[384 + 32 + 2] = 2002
    return t


def test_document_frequency_counts_blocks():
    t = planted_tokens()
    t2 = t.copy()
    t2[140:150] = 1001                      # repeats inside one block: still df 1
    df = so.document_frequency(t2, 512, 128)
    assert df[7] == 4 and df[1001] == 1 and df[2002] == 2 and df[3003] == 1
    n = 4
    assert so.maxidf_score(t[128 + 64: 128 + 96], df, n) == math.log(4)
    assert so.maxidf_score(t[128: 160], df, n) == math.log(2)
    assert so.maxidf_score(np.full(32, 7), df, n) == 0.0


def test_maxidf_summaries_hand_derived():
    t = planted_tokens()
    s1 = so.maxidf_summaries(t, 512, 128, m=32, sink=64, k=1)
    # block 0: chunks 0/1 overlap the sink; chunk 3 (4005) beats chunk 2
    assert np.array_equal(s1[0], np.arange(96, 128))
    # block 1: chunk 2 (log 4) beats chunk 0 (log 2)
    assert np.array_equal(s1[1], np.arange(192, 224))
    # block 2: tie between chunks 1 and 3 -> the earlier one
    assert np.array_equal(s1[2], np.arange(288, 320))
    assert np.array_equal(s1[3], np.arange(416, 448))
    s2 = so.maxidf_summaries(t, 512, 128, m=32, sink=64, k=2)
    assert np.array_equal(s2[0], np.arange(64, 128))                 # the only 2 candidates
    assert np.array_equal(s2[1], np.r_[128:160, 192:224])            # positional order
    assert np.array_equal(s2[2], np.r_[288:320, 352:384])
    assert np.array_equal(s2[3], np.r_[384:416, 416:448])            # chunk 1 + earliest 0-score


def test_pulsar_prefix_layout():
    t = planted_tokens()
    rows, st, ln = so.pulsar_prefix(t, 512, 128, m=32, sink=64, k=1)
    assert np.array_equal(rows, np.r_[0:64, 96:128, 192:224, 288:320])
    assert np.array_equal(st, [0, 0, 0, 0])
    assert np.array_equal(ln, [0, 96, 128, 160])
    # every prefix row precedes the block that reads it
    for i in range(1, 4):
        assert rows[st[i]:st[i] + ln[i]].max() < 128 * i
    # the KV the hosts keep is still exactly L entries (the prefix is dropped)
    assert so.kv_cache_entries(512, 128) == 512


def test_pulsar_prefix_ragged_chunks():
    """b not a multiple of m: the last chunk of a block is shorter."""
    L, b = 230, 70
    t = np.arange(L) % 50             # df varies; deterministic
    sums = so.maxidf_summaries(t, L, b, m=32, sink=64, k=3)
    assert [c for c in so.chunks_of_block(70, 140, 32)] == [(70, 102), (102, 134), (134, 140)]
    for i, s in enumerate(sums):
        s0, e0 = i * b, min(i * b + b, L)
        assert (s >= s0).all() and (s < e0).all() and np.all(np.diff(s) > 0)
    assert sums[0].size == 6          # only chunk [64, 70) is a candidate in block 0


def test_pulsar_host_lengths_match_printed_numbers():
    g = json.load(open(os.path.join(GOLD, "pulsar_lengths.json")))
    L, hosts, sink = g["L"], g["hosts"], g["sink"]
    b = L // hosts
    assert 2 * b == g["n_star"]
    for c in g["cases"]:
        n = so.pulsar_host_length(L, b, sink, c["summary_tokens"], hosts - 1)
        assert n == c["n_pulsar"]
        assert round((2 * b / n) ** 2, 1 if c["flops_ratio_vs_star"] == 3.3 else 2) == \
            c["flops_ratio_vs_star"]
    # 12.5% of the block, 16 chunks of 32 for a 4096-token block
    assert 16 * g["chunk_tokens"] == g["summary_fraction_of_block"] * 4096
    # asymptote with s = 0.125 * b: (b + 3 s) / L -> 0.34375
    big = 1 << 40
    bb = big // 4
    n = so.pulsar_host_length(big, bb, sink, bb // 8, 3)
    assert abs(n / big - g["asymptote"]["n_pulsar_over_L"]) < 1e-9
    assert round((2 * bb / n) ** 2, 2) == g["asymptote"]["flops_ratio_vs_star"]


def test_pulsar_prefix_lengths_agree_with_host_length():
    """With every block offering k full chunks, host i's prefix + block is
    b + sink + i*s."""
    L, b, m, sink, k = 1024, 256, 32, 64, 2
    t = np.random.default_rng(25).integers(0, 300, size=L)
    rows, st, ln = so.pulsar_prefix(t, L, b, m=m, sink=sink, k=k)
    for i in range(4):
        assert ln[i] + b == so.pulsar_host_length(L, b, sink, k * m, i)


def test_pulsar_planted_mistake_is_caught():
    """A plausible slip (ranking by the minimum IDF instead of the maximum)
    changes the hand-derived selection."""
    t = planted_tokens()
    df = so.document_frequency(t, 512, 128)
    wrong = min(math.log(4 / max(df.get(int(x), 0), 1)) for x in t[192:224])
    right = so.maxidf_score(t[192:224], df, 4)
    assert wrong == 0.0 and right == math.log(4)


def test_pulsar_16k_prefix_is_1600_entries():
    """At 16K with 4 hosts, 16 chunks of 32 per block: the last host's
    prefix (sink + 3 summaries) is the 1,600 entries the Pulsar review
    speaks of, and its Phase-1 length is L/4 + 1600."""
    g = json.load(open(os.path.join(GOLD, "pulsar_lengths.json")))["fixed_budget_16k"]
    L, hosts = g["L"], g["hosts"]
    b = L // hosts
    t = np.random.default_rng(26).integers(0, 5000, size=L)
    rows, st, ln = so.pulsar_prefix(t, L, b, m=32, sink=64, k=g["summary_tokens"] // 32)
    assert rows.size == ln[-1] == g["prefix_entries_last_host"]
    assert so.pulsar_host_length(L, b, 64, g["summary_tokens"], hosts - 1) == L // 4 + 1600
