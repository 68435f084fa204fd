"""Pins for the CPU oracle: checks against facts the pages and mathematics
fix, never against the oracle's own formulas retyped.

Each pin is chosen so that a plausible mistake in the oracle (a dropped
anchor, a wrong mask index, a RoPE sign or pairing slip, a wrong GQA map, a
bad merge weight) fails at least one of them; ``test_planted_mistakes``
plants such mistakes in the oracle on the CPU and checks that the pins catch
them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.star_oracle as so
from workloads import TINY, as_f64, inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "star_counts.json")
RNG = np.random.default_rng(1234)


def rand(*shape):
    return RNG.standard_normal(shape)


def sdpa(q, k, v, causal=False, mask=None):
    """torch scaled_dot_product_attention in float64 on the CPU (library
    routine; default scale 1/sqrt(D))."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, is_causal=causal)
    return out.numpy()


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------
def test_rope_d2_is_rotation_by_position():
    # D = 2: theta_0 = 1, so position p rotates (x, y) by exactly p radians.
    for p in [0, 1, 7, 12345, 1048575]:
        out = so.rope(np.array([[1.0, 0.0]]), np.array([p]), 500000.0)
        assert np.allclose(out[0], [math.cos(p), math.sin(p)], atol=1e-12)
        out = so.rope(np.array([[0.0, 1.0]]), np.array([p]), 500000.0)
        assert np.allclose(out[0], [-math.sin(p), math.cos(p)], atol=1e-12)


def test_rope_pairs_and_frequencies():
    # D = 4, base 100: theta = (1, 100^(-1/2) = 0.1).  Pair (1, 3) at
    # position 10 rotates by 1 rad; pair (0, 2) by 10 rad.
    x = np.array([[0.0, 1.0, 0.0, 0.0]])
    out = so.rope(x, np.array([10]), 100.0)
    assert np.allclose(out[0], [0.0, math.cos(1.0), 0.0, math.sin(1.0)], atol=1e-12)
    x = np.array([[1.0, 0.0, 0.0, 0.0]])
    out = so.rope(x, np.array([10]), 100.0)
    assert np.allclose(out[0], [math.cos(10.0), 0.0, math.sin(10.0), 0.0], atol=1e-12)


def test_rope_theta_is_the_nearest_float64():
    """theta_j = base^(-2j/D), each the float64 nearest the exact power.
    Bases that are powers of two give exactly representable frequencies
    (2^16 at D = 8: theta_j = 2^(-4j)); theta_0 = 1 for any base; and for
    the bases and head dims the workloads use, the C library's pow (a
    separate routine, correctly rounded on these inputs) gives the same
    bits -- numpy's vectorised power does not on AVX-512 hosts, which is why
    the oracle avoids it."""
    assert so.rope_theta(8, 65536.0).tolist() == [1.0, 2.0 ** -4, 2.0 ** -8, 2.0 ** -12]
    assert so.rope_theta(2, 12345.0).tolist() == [1.0]
    for base in (100.0, 10000.0, 500000.0, 1e6):
        for D in (2, 4, 16, 64, 128):
            th = so.rope_theta(D, base)
            ref = [math.pow(base, -2.0 * j / D) for j in range(D // 2)]
            assert th.tolist() == ref, (base, D)
    # a slip in the exponent (-j/D instead of -2j/D) is caught
    assert so.rope_theta(8, 65536.0)[1] != 2.0 ** -2


def test_rope_identity_norm_relative_complex():
    D, S = 128, 33
    x = rand(S, D)
    pos = np.arange(S) * 4099 + 3
    assert np.allclose(so.rope(x, np.zeros(S, dtype=np.int64), 500000.0), x)
    r = so.rope(x, pos, 500000.0)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1))
    # equals the complex multiply (x_j + i x_{j+D/2}) * exp(i p theta_j)
    j = np.arange(D // 2)
    theta = np.exp(-(2.0 * j / D) * math.log(500000.0))
    z = (x[:, :D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * pos[:, None] * theta[None])
    assert np.allclose(r, np.concatenate([z.real, z.imag], axis=1), atol=1e-9)
    # <R(p) q, R(p') k> depends only on p - p'
    q, k = rand(1, D), rand(1, D)
    for p, pp, d in [(5, 2, 1000), (131071, 17, 900001)]:
        a = so.rope(q, np.array([p]), 5e5) @ so.rope(k, np.array([pp]), 5e5).T
        b = so.rope(q, np.array([p + d]), 5e5) @ so.rope(k, np.array([pp + d]), 5e5).T
        assert abs(a - b) < 1e-9


# ----------------------------------------------------------------------------
# masked attention primitive
# ----------------------------------------------------------------------------
def brute_attention(q, k, v, mask, scale):
    """Pure-Python loops (tiny inputs only)."""
    n, m, D = len(q), len(k), len(v[0])
    o = [[0.0] * D for _ in range(n)]
    lse = [-math.inf] * n
    for r in range(n):
        sc = [sum(q[r][d] * k[c][d] for d in range(len(q[r]))) * scale
              for c in range(m) if mask[r][c]]
        idx = [c for c in range(m) if mask[r][c]]
        if not sc:
            continue
        mx = max(sc)
        ws = [math.exp(s - mx) for s in sc]
        tot = sum(ws)
        lse[r] = mx + math.log(tot)
        for w, c in zip(ws, idx):
            for d in range(D):
                o[r][d] += w / tot * v[c][d]
    return np.array(o), np.array(lse)


def test_attend_bruteforce_and_sdpa():
    n, m, D = 5, 7, 4
    q, k, v = rand(n, D), rand(m, D), rand(m, D)
    mask = RNG.random((n, m)) < 0.6
    mask[0] = False
    mask[1] = True
    o, l = so.attend(q, k, v, mask, 0.5)
    ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), mask.tolist(), 0.5)
    assert np.allclose(o, ob, atol=1e-12)
    assert np.array_equal(np.isinf(l), np.isinf(lb))
    assert np.allclose(l[np.isfinite(l)], lb[np.isfinite(lb)], atol=1e-12)
    assert np.all(o[0] == 0) and l[0] == -np.inf
    live = mask.any(axis=1)
    ref = sdpa(q[None, live], k[None], v[None], mask=mask[None, live])
    o2, _ = so.attend(q[live], k, v, mask[live], 1.0 / math.sqrt(D))
    assert np.allclose(o2, ref[0], atol=1e-12)


def test_attend_closed_forms():
    D = 8
    q, k, v = rand(1, D), rand(1, D), rand(1, D)
    o, l = so.attend(q, k, v, np.ones((1, 1), bool), 0.3)
    assert np.allclose(o, v) and np.isclose(l[0], 0.3 * (q @ k.T).item())
    # equal scores (q = 0): lse = ln n, o = mean of the visible values
    n = 9
    k, v = rand(n, D), rand(n, D)
    o, l = so.attend(np.zeros((1, D)), k, v, np.ones((1, n), bool), 0.3)
    assert np.isclose(l[0], math.log(n)) and np.allclose(o[0], v.mean(axis=0))


# ----------------------------------------------------------------------------
# Phase 1
# ----------------------------------------------------------------------------
def expand_kv(K, g):
    """HF repeat-kv convention: KV head j serves query heads j*g .. j*g+g-1."""
    return np.repeat(K, g, axis=1)


def _p1_inputs(B=2, Hq=4, Hkv=2, L=40, D=8):
    return rand(B, Hq, L, D), rand(B, Hkv, L, D), rand(B, Hkv, L, D)


def test_phase1_single_block_equals_dense_causal():
    """b >= L: Phase 1 is plain causal attention (I1)."""
    Q, K, V = _p1_inputs()
    D = Q.shape[-1]
    for b in (40, 64):
        O, LSE = so.phase1(Q, K, V, b, b, 1 / math.sqrt(D))
        ref = sdpa(Q, expand_kv(K, 2), expand_kv(V, 2), causal=True)
        assert np.allclose(O, ref, atol=1e-12)
        o, l = so.dense_causal(Q[1, 3], K[1, 1], V[1, 1], 1 / math.sqrt(D))
        assert np.allclose(O[1, 3], o) and np.allclose(LSE[1, 3], l)


def p1_pin_error(b, a, L=44):
    """Max error of the oracle's Phase 1 against SDPA run causally on the
    materialised augmented block [anchor ; c_i] (I2 / I4)."""
    Q, K, V = _p1_inputs(L=L)
    D = Q.shape[-1]
    O, _ = so.phase1(Q, K, V, b, a, 1 / math.sqrt(D))
    Ke, Ve = expand_kv(K, 2), expand_kv(V, 2)
    err = 0.0
    for i, s in enumerate(range(0, L, b)):
        e = min(s + b, L)
        if i == 0 or a == 0:
            ref = sdpa(Q[:, :, s:e], Ke[:, :, s:e], Ve[:, :, s:e], causal=True)
        else:
            cat = lambda X: np.concatenate([X[:, :, :a], X[:, :, s:e]], axis=2)
            ref = sdpa(cat(Q), cat(Ke), cat(Ve), causal=True)[:, :, a:]
        err = max(err, np.abs(O[:, :, s:e] - ref).max())
    return err


@pytest.mark.parametrize("b,a", [(8, 8), (12, 12), (8, 5), (8, 0), (16, 16)])
def test_phase1_block_equals_causal_over_augmented_block(b, a):
    """Each block's rows equal dense causal attention over the materialised
    [anchor ; block] sequence (last n_i rows); a = 0 is block-diagonal (I2, I4).
    L = 44 leaves a ragged tail block for every b here."""
    assert p1_pin_error(b, a) < 1e-12


def test_visible_key_counts_and_golden_counts():
    """I6: r+1 visible keys in block 1, a+r+1 in later blocks; exactly L KV
    entries kept; per-host length 2b as the pages state."""
    with open(GOLDEN) as f:
        gold = {e["name"]: e for e in json.load(f)["entries"]}
    L, b, a = 50, 8, 8
    for i, (s, e) in enumerate(so.blocks(L, b)):
        keys, mask = so.phase1_block_keys(i, L, b, a)
        r = np.arange(e - s)
        want = r + 1 if i == 0 else a + r + 1
        assert np.array_equal(mask.sum(axis=1), want)
        assert np.array_equal(keys[mask[-1]], np.concatenate(
            [np.arange(0, a) if i else np.arange(0), np.arange(s, e)]))
    assert so.kv_cache_entries(L, b) == L * gold["kv_entries_after_phase1"]["value_in_L"]
    g = gold["per_host_tokens_star_64k_4hosts"]
    assert g["b"] == g["L"] * gold["block_size_rule_up_to_128k"]["value"]
    nb = len(so.blocks(g["L"], g["b"]))
    assert nb == g["hosts"]
    longest = max(so.phase1_block_keys(i, g["L"], g["b"], g["anchor"])[0].size
                  for i in range(nb))
    assert longest == g["value"]
    first = so.phase1_block_keys(0, g["L"], g["b"], g["anchor"])[0].size
    assert first == g["b"] * gold["first_block_tokens"]["value_in_b"]
    assert longest == g["b"] * gold["later_block_tokens"]["value_in_b"]


def test_phase1_closed_forms():
    """I7: the first row of block 1 sees one key (o = v_0, lse = its score);
    with a = 0 the first row of every block sees only itself."""
    Q, K, V = _p1_inputs(L=24)
    sc = 1 / math.sqrt(Q.shape[-1])
    O, LSE = so.phase1(Q, K, V, 8, 0, sc)
    for s in (0, 8, 16):
        assert np.allclose(O[0, 2, s], V[0, 1, s])
        assert np.isclose(LSE[0, 2, s], sc * Q[0, 2, s] @ K[0, 1, s])


def test_phase1_row_is_merge_of_anchor_and_own_block():
    """I9: a block-i row equals the LSE merge of an anchor-only partial and
    an own-block causal partial (ties Phase 1 to the Phase 2 machinery)."""
    Q, K, V = _p1_inputs(B=1, Hq=2, Hkv=1, L=30)
    sc = 1 / math.sqrt(Q.shape[-1])
    b = a = 10
    O, LSE = so.phase1(Q, K, V, b, a, sc)
    for p in (10, 15, 29):
        s = (p // b) * b
        oa, la = so.attend(Q[0, 1, p:p + 1], K[0, 0, :a], V[0, 0, :a],
                           np.ones((1, a), bool), sc)
        ob, lb = so.partial(Q[0, 1, p:p + 1], [p], K[0, 0], V[0, 0], s, s + b, sc)
        o, l = so.lse_merge(np.stack([oa, ob]), np.stack([la, lb]))
        assert np.allclose(o[0], O[0, 1, p]) and np.isclose(l[0], LSE[0, 1, p])


def test_phase1_rows_matches_phase1():
    Q, K, V = _p1_inputs(B=1, Hq=2, Hkv=1, L=37)
    sc = 1 / math.sqrt(Q.shape[-1])
    O, LSE = so.phase1(Q, K, V, 8, 6, sc)
    pos = np.array([0, 3, 8, 9, 20, 36])
    o, l = so.phase1_rows(Q[0, 1, pos], pos, K[0, 0], V[0, 0], 8, 6, sc)
    assert np.allclose(o, O[0, 1, pos]) and np.allclose(l, LSE[0, 1, pos])


# ----------------------------------------------------------------------------
# Phase 2 and the merge
# ----------------------------------------------------------------------------
def merge_pin_error(seed):
    """Merge of a random partition of the keys (random split points, empty
    parts, permuted order) against monolithic attention (I3)."""
    r = np.random.default_rng(seed)
    n, m, D = 6, int(r.integers(1, 40)), 8
    q, k, v = r.standard_normal((n, D)), r.standard_normal((m, D)), r.standard_normal((m, D))
    mask = r.random((n, m)) < 0.7
    full_o, full_l = so.attend(q, k, v, mask, 0.4)
    cuts = np.sort(r.integers(0, m + 1, size=int(r.integers(0, 6))))
    bounds = [0, *cuts.tolist(), m]
    parts = [(bounds[i], bounds[i + 1]) for i in range(len(bounds) - 1)]
    r.shuffle(parts)
    ops, lps = [], []
    for k0, k1 in parts:
        o, l = so.attend(q, k[k0:k1], v[k0:k1], mask[:, k0:k1], 0.4)
        ops.append(o)
        lps.append(l)
    o, l = so.lse_merge(np.stack(ops), np.stack(lps))
    fin = np.isfinite(full_l)
    assert np.array_equal(np.isfinite(l), fin)
    return max(np.abs(o - full_o).max(), np.abs(l[fin] - full_l[fin]).max(initial=0))


@pytest.mark.parametrize("seed", range(25))
def test_merge_of_any_partition_is_exact(seed):
    assert merge_pin_error(seed) < 1e-12


def test_merge_weights_bruteforce():
    # two partials with lse 0 and ln 3: weights 1/4 and 3/4, lse ln 4
    o, l = so.lse_merge(np.array([[[1.0, 0.0]], [[0.0, 1.0]]]),
                        np.array([[0.0], [math.log(3.0)]]))
    assert np.allclose(o[0], [0.25, 0.75]) and np.isclose(l[0], math.log(4.0))
    o, l = so.lse_merge(np.array([[[5.0]], [[7.0]]]), np.array([[-np.inf], [-np.inf]]))
    assert o[0, 0] == 0.0 and l[0] == -np.inf


def test_phase2_equals_global_attention():
    """I8 and the Phase-2 definition: the merged partials over every
    partition equal attention of the query over the whole cache, which is
    the last rows of causal SDPA over the full sequence."""
    L, b, Lq, D = 40, 12, 5, 8
    N = L + Lq
    Kc, Vc = rand(N, D), rand(N, D)
    Qf = rand(N, D)
    qpos = np.arange(L, N)
    ref = sdpa(Qf[None], Kc[None], Vc[None], causal=True)[0, L:]
    for parts in (so.partitions(L, b, N), [(0, N)]):
        o, l, op, lp = so.phase2(Qf[L:], qpos, Kc, Vc, parts, 1 / math.sqrt(D))
        assert np.allclose(o, ref, atol=1e-12)
    assert so.partitions(L, b, N) == [(0, 12), (12, 24), (24, 36), (36, 45)]


def test_tiny_pipeline_decode_and_gqa():
    """The whole pipeline on a shrunken tiny workload with decode steps:
    every decode output equals causal SDPA over the full cache with the KV
    heads expanded by the repeat-kv convention."""
    w = TINY.replace(L=96, b=32, Lq=4, T=3, Hq=4, Hkv=2, rope=True, base=10000.0)
    x = {k: as_f64(t) for k, t in inputs(w, as_bf16=True).items()}
    r = so.star_attention(w, x)
    N = w.L + w.Lq + w.T
    Qf = np.concatenate([r["Q"], r["qq"], r["qd"]], axis=2)
    ref = sdpa(Qf, expand_kv(r["Kc"], 2), expand_kv(r["Vc"], 2), causal=True)
    assert np.allclose(r["O2"], ref[:, :, w.L:w.L + w.Lq], atol=1e-12)
    assert np.allclose(r["OD"], ref[:, :, w.L + w.Lq:N], atol=1e-12)
    assert r["Kc"].shape[2] == N
    # Phase-1 block 1 equals the dense causal prefix of the same sequence
    assert np.allclose(r["O1"][:, :, :w.b], ref[:, :, :w.b], atol=1e-12)


# ----------------------------------------------------------------------------
# planted mistakes: the pins above must catch them
# ----------------------------------------------------------------------------
def test_planted_mistakes(monkeypatch):
    # 1. anchor dropped from later blocks
    orig_keys = so.phase1_block_keys

    def no_anchor(i, L, b, a):
        return orig_keys(i, L, b, 0)
    with monkeypatch.context() as m:
        m.setattr(so, "phase1_block_keys", no_anchor)
        assert p1_pin_error(8, 8) > 1e-3
    # 2. causal mask off by one (row sees the next key)
    def shifted(i, L, b, a):
        keys, mask = orig_keys(i, L, b, a)
        n = mask.shape[0]
        mask = mask.copy()
        mask[:, mask.shape[1] - n:] = np.tril(np.ones((n, n), bool), 1)
        return keys, mask
    with monkeypatch.context() as m:
        m.setattr(so, "phase1_block_keys", shifted)
        assert p1_pin_error(8, 8) > 1e-3
    # 3. merge weight without the global normaliser
    orig_merge = so.lse_merge

    def bad_merge(o_parts, lse_parts):
        o, l = orig_merge(o_parts, lse_parts)
        w = np.exp(np.asarray(lse_parts))
        return (w[..., None] * np.asarray(o_parts)).sum(axis=0), l
    with monkeypatch.context() as m:
        m.setattr(so, "lse_merge", bad_merge)
        assert max(merge_pin_error(s) for s in range(5)) > 1e-3
    # 4. RoPE with the opposite rotation sense
    orig_rope = so.rope
    with monkeypatch.context() as m:
        m.setattr(so, "rope", lambda x, pos, base: orig_rope(x, -np.asarray(pos), base))
        with pytest.raises(AssertionError):
            test_rope_d2_is_rotation_by_position()
    # 5. wrong GQA map (query head h reading KV head Hkv-1-h//g)
    orig_phase1 = so.phase1

    def phase1_wrong_gqa(Q, K, V, b, a, scale):
        return orig_phase1(Q, K[:, ::-1].copy(), V[:, ::-1].copy(), b, a, scale)
    with monkeypatch.context() as m:
        m.setattr(so, "phase1", phase1_wrong_gqa)
        with pytest.raises(AssertionError):
            test_phase1_single_block_equals_dense_causal()


def test_round_bf16_matches_torch_and_ties():
    """bf16 rounding of the rotated tensors: equals torch's float32->bfloat16
    cast (round to nearest even) on float32 inputs, and rounds float64
    values directly (no double rounding through float32)."""
    r = np.random.default_rng(5)
    x = np.concatenate([r.standard_normal(50000) * 10.0 ** r.integers(-30, 30, 50000),
                        [0.0, -0.0, 1.0, 1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 3e38]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(so.round_bf16(x32.astype(np.float64)), ref)
    assert so.round_bf16(np.array([1 + 2**-8 + 2**-40]))[0] == 1 + 2**-7
    assert so.round_bf16(np.array([1 + 2**-8 - 2**-40]))[0] == 1.0
    assert so.round_bf16(np.array([1 + 2**-8]))[0] == 1.0   # tie to even
