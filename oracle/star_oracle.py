"""CPU oracle for Star Attention's two-phase attention hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in ``oracle/``.  The HIP library never calls it and
shares no code with it: the only thing both sides use is the seeded input
generator in ``workloads/``, which holds none of the method's arithmetic.

Everything here is plain float64 numpy: explicit boolean masks, one matmul
per score matrix, no tiling, no fusion, no reordering beyond what the
definitions state.  Every function is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force, library routines (torch SDPA in float64)
or facts the pages fix; no function here is "parity unpinned".

Sources (cited by page title and section):
  [SA-pith]   Pith review of "Star Attention: Efficient LLM Inference over
              Long Sequences" (pith.science) -- "What carries the argument",
              "Core claim", "Referee Report", "Circularity Check",
              "Assumptions & free parameters", the abstract.
  [SA-atlas]  atlas.scime.ai summary of the same paper -- "Approach",
              "Measured effects reported in the paper".
  [SA-repo]   graphcanon record of the NVIDIA/Star-Attention repository --
              README excerpt (Phase 1 / Phase 2 description; HuggingFace
              Transformers implementation).
  [Pulsar]    Pith review of "Dropping the Anchor ... Pulsar Attention" --
              "Core claim", "Assumptions & free parameters" (restates Star's
              KV-cache identity and the exactness of the online-softmax merge).

Readings where the pages leave a step open (all listed in the design notes):
  * causality inside an augmented block: causal over the concatenation
    [anchor ; block], so every block row sees the whole anchor;
  * the anchor is the first ``a`` context tokens at their original positions
    (a = b by default), hence its keys/values are block 1's rotated K/V;
  * a tail block shorter than b when b does not divide L; b >= L is one block;
  * softmax scale 1/sqrt(D); GQA query head h reads KV head h // g;
  * the softmax statistic is the natural-log log-sum-exp of the scaled scores;
  * the query host is the last partition: it also holds the query and decode
    tokens' KV, and a token attends to itself;
  * RoPE is rotate-half with theta_j = base^(-2j/D), angles in exact (fp64)
    arithmetic, no frequency scaling;
  * a prefix (anchor variant or Pulsar sink + summaries) precedes its block:
    every block row sees every prefix key;
  * Pulsar: host 0 is plain causal; block 0's chunks that overlap the sink
    are not summary candidates; equal Max-IDF scores go to the earlier chunk;
    the last chunk of a block may be shorter than m;
  * the attention layer is the Llama-3 block: RMSNorm (eps 1e-5), q/k/v
    projections, RoPE, attention, output projection and the residual add;
    every stored activation is bf16 (one rounding per stored tensor).
"""
from __future__ import annotations

import functools
import math

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# RoPE at original position ids
# ----------------------------------------------------------------------------
def rope_theta(D: int, base: float) -> np.ndarray:
    """Rotation frequencies theta_j = base^(-2j/D), j = 0..D/2-1: each one
    the float64 value nearest the exact power.

    The power is evaluated as exp(-(2j/D) ln(base)) in 40-digit decimal
    arithmetic and rounded once to float64 (Python's Decimal -> float
    conversion rounds to nearest).  numpy's vectorised ``power`` is not
    used: on hosts with AVX-512 it dispatches to a SIMD routine that is off
    by one ulp for some j (2 of the 64 frequencies at base 500000, D = 128),
    so its angles, and the bf16 rounding of rotated values, would depend on
    the host the oracle runs on.
    """
    return np.array(_rope_theta_exact(int(D), float(base)), dtype=np.float64)


@functools.lru_cache(maxsize=64)
def _rope_theta_exact(D: int, base: float) -> tuple:
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = 40
        ln_base = Decimal(base).ln()                 # Decimal(float) is exact
        return tuple(float((ln_base * Decimal(-2 * j) / Decimal(D)).exp())
                     for j in range(D // 2))


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE of ``x[..., S, D]`` at integer positions ``pos[S]``.

    Pair (j, j + D/2) is rotated by the angle pos * theta_j.  Positions are
    the tokens' original (global) ids: [SA-pith] "What carries the argument"
    (the anchor keeps the first block's positional indices) and [Pulsar]
    "Assumptions & free parameters" (original position ids preserve RoPE
    geometry).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_theta(D, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float64.  bfloat16 keeps 8 significant bits: with x = m * 2^e,
    0.5 <= |m| < 1, the result is rint(m * 2^8) * 2^(e-8) (numpy's rint
    rounds half to even).  Exponents below bfloat16's normal range keep the
    subnormal quantum 2^-133.

    Rotated Q/K are stored in the model's bfloat16 dtype (the KV cache
    dtype) before attention reads them ([SA-repo] README: HuggingFace
    Transformers LLMs; the attention inputs are bf16), so the oracle rounds
    its exact rotation here.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


# ----------------------------------------------------------------------------
# masked softmax attention: the one primitive every step uses
# ----------------------------------------------------------------------------
def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
           scale: float):
    """Softmax attention of rows ``q[n, D]`` over ``k, v[m, D]`` where
    ``mask[n, m]`` marks the visible keys.

    Returns ``(o[n, D], lse[n])`` with ``lse`` the natural-log log-sum-exp of
    the scaled visible scores.  A row with no visible key gets o = 0 and
    lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, m = q.shape[0], k.shape[0]
    assert mask.shape == (n, m)
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, NEG_INF, dtype=np.float64)
    if n == 0 or m == 0:
        return o, lse
    s = (q @ k.T) * scale
    s = np.where(mask, s, NEG_INF)
    mx = s.max(axis=1)
    live = np.isfinite(mx)
    if not live.any():
        return o, lse
    s, mx = s[live], mx[live]
    p = np.exp(s - mx[:, None])
    l = p.sum(axis=1)
    o[live] = (p @ v) / l[:, None]
    lse[live] = mx + np.log(l)
    return o, lse


# ----------------------------------------------------------------------------
# Phase 1: blockwise-local attention with the anchor block
# ----------------------------------------------------------------------------
def blocks(L: int, b: int):
    """Context blocks c_1..c_n as [start, end) token ranges; the last one is
    shorter when b does not divide L ([SA-pith] "What carries the argument":
    the context is split into blocks of b tokens)."""
    return [(s, min(s + b, L)) for s in range(0, L, b)]


def phase1_block_keys(i: int, L: int, b: int, a: int, rows=None):
    """Key ids and explicit mask of the augmented block c'_i (0-based i).

    c'_1 = c_1 is plain causal attention over b tokens ([SA-pith] "Referee
    Report", minor comment on section 2.1: only blocks after the first carry
    the anchor).  For i >= 1 the augmented block is [anchor ; c_i]: every row
    sees all ``a`` anchor tokens (the first ``a`` context tokens at their
    original positions) plus its own block's tokens up to itself.
    Returns (key_ids[m], mask[n, m]); ``rows`` (indices inside the block)
    selects which mask rows to build, default all n_i rows.
    """
    s, e = blocks(L, b)[i]
    n = e - s
    own = np.arange(s, e)
    r = np.arange(n) if rows is None else np.asarray(rows)
    causal = own[None, :] - s <= r[:, None]
    if i == 0:
        return own, causal
    anc = np.arange(0, min(a, L))
    mask = np.concatenate([np.ones((r.size, anc.size), dtype=bool), causal], axis=1)
    return np.concatenate([anc, own]), mask


def phase1(Q, K, V, b: int, a: int, scale: float):
    """Phase 1 context encoding ([SA-pith] "What carries the argument",
    "Referee Report" summary; [SA-repo] README, Phase 1).

    Q [B, Hq, L, D], K/V [B, Hkv, L, D] (already rotated).  Each block's rows
    attend within their augmented block only.  Returns O [B, Hq, L, D] and
    LSE [B, Hq, L].  The anchor's own outputs are not produced: block 1's
    rows are the only outputs for those tokens.
    """
    B, Hq, L, D = Q.shape
    g = Hq // K.shape[1]
    O = np.zeros((B, Hq, L, D))
    LSE = np.full((B, Hq, L), NEG_INF)
    for i, (s, e) in enumerate(blocks(L, b)):
        keys, mask = phase1_block_keys(i, L, b, a)
        for bb in range(B):
            for h in range(Hq):
                o, l = attend(Q[bb, h, s:e], K[bb, h // g, keys],
                              V[bb, h // g, keys], mask, scale)
                O[bb, h, s:e], LSE[bb, h, s:e] = o, l
    return O, LSE


def phase1_rows(q_rows, pos, K, V, b: int, a: int, scale: float):
    """Phase 1 outputs for selected rows of one (batch, query head).

    ``q_rows[n, D]`` are rotated query rows at context positions ``pos[n]``;
    ``K, V [L, D]`` are that head's KV head.  Each row is computed over the
    same key set and the same mask row as in :func:`phase1`.
    """
    L = K.shape[0]
    pos = np.asarray(pos)
    o = np.zeros((pos.size, V.shape[1]))
    lse = np.full(pos.size, NEG_INF)
    for i, (s, e) in enumerate(blocks(L, b)):
        sel = np.nonzero((pos >= s) & (pos < e))[0]
        if sel.size == 0:
            continue
        keys, mask = phase1_block_keys(i, L, b, a, rows=pos[sel] - s)
        oo, ll = attend(q_rows[sel], K[keys], V[keys], mask, scale)
        o[sel], lse[sel] = oo, ll
    return o, lse


def kv_cache_entries(L: int, b: int) -> int:
    """Number of KV entries kept after Phase 1: each host keeps only its own
    block and the anchor's KV is discarded ([SA-atlas] "Approach"; [Pulsar]
    "Core claim": exactly L entries across hosts)."""
    return sum(e - s for s, e in blocks(L, b))


# ----------------------------------------------------------------------------
# Phase 2: per-partition partials and the exact LSE merge
# ----------------------------------------------------------------------------
def partitions(L: int, b: int, cache_len: int):
    """KV partitions ("hosts"): partition j holds block j's KV; the last one
    (the query host) also holds the query and generated tokens' KV
    ([SA-pith] "What carries the argument": a designated query host)."""
    parts = blocks(L, b)
    s, _ = parts[-1]
    parts[-1] = (s, cache_len)
    return parts


def partial(q, q_pos, Kc, Vc, k0: int, k1: int, scale: float):
    """Local attention of query rows over cache entries [k0, k1): the
    per-host output A_h and statistic s_h ([SA-pith] "Circularity Check":
    each host computes a local attention output and softmax denominator).

    ``q[n, D]`` rotated rows at positions ``q_pos[n]``; ``Kc, Vc [N, D]``.
    A key at cache index c (= its position) is visible to a row at position
    p when c <= p.
    """
    keys = np.arange(k0, k1)
    mask = keys[None, :] <= np.asarray(q_pos)[:, None]
    return attend(q, Kc[k0:k1], Vc[k0:k1], mask, scale)


def lse_merge(o_parts, lse_parts):
    """Exact online-softmax merge of N partials ([SA-pith] "Referee Report",
    minor comment on Algorithm 2: the weight of A_h is exp(s_h - s_global);
    "Circularity Check": the reweighting is an exact identity).

    ``o_parts[N, ..., D]``, ``lse_parts[N, ...]``.  s = log sum_h exp(s_h);
    A = sum_h exp(s_h - s) A_h.  Partials with s_h = -inf carry no weight; if
    every partial is -inf the row is o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    live = np.isfinite(m)
    msafe = np.where(live, m, 0.0)
    w = np.exp(lse_parts - msafe[None])          # exp(-inf) = 0
    tot = w.sum(axis=0)
    lse = np.where(live, msafe + np.log(np.where(live, tot, 1.0)), NEG_INF)
    wn = np.where(live[None], w / np.where(live, tot, 1.0)[None], 0.0)
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse


def phase2(q, q_pos, Kc, Vc, parts, scale: float):
    """Sequence-global attention of query rows via per-partition partials
    and the LSE merge ([SA-pith] "Referee Report" summary, Eqs. 3-4;
    [SA-repo] README, Phase 2).  Returns (o, lse, o_parts, lse_parts)."""
    op, lp = [], []
    for (k0, k1) in parts:
        o, l = partial(q, q_pos, Kc, Vc, k0, k1, scale)
        op.append(o)
        lp.append(l)
    op, lp = np.stack(op), np.stack(lp)
    o, l = lse_merge(op, lp)
    return o, l, op, lp


# ----------------------------------------------------------------------------
# textbook references used only as pins
# ----------------------------------------------------------------------------
def dense_causal(Q, K, V, scale: float):
    """Plain dense causal attention of one head, [S, D] each (global
    attention, the method's baseline)."""
    S = Q.shape[0]
    return attend(Q, K, V, np.tril(np.ones((S, S), dtype=bool)), scale)


# ----------------------------------------------------------------------------
# the whole hot path on one workload (small workloads only)
# ----------------------------------------------------------------------------
def star_attention(w, x: dict, store_bf16: bool = True):
    """Run both phases on a workload's inputs (see ``workloads.inputs``).

    ``x`` maps names to float64 arrays.  With ``store_bf16`` the rotated
    Q/K are rounded to bfloat16, the dtype the model stores them in, before
    attention (see :func:`round_bf16`).  Returns a dict with the rotated
    tensors, Phase-1 O/LSE, the query-phase partials and merged output, and
    one merged output per decode step.
    """
    B, Hq, Hkv, D, L = w.B, w.Hq, w.Hkv, w.D, w.L
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    def rot(t, pos):
        if not w.rope:
            return np.asarray(t, np.float64)
        r = rope(t, pos, w.base)
        return round_bf16(r) if store_bf16 else r
    pos_ctx = np.arange(L)
    pos_q = L + np.arange(w.Lq)
    pos_d = L + w.Lq + np.arange(w.T)
    Q, K = rot(x["q"], pos_ctx), rot(x["k"], pos_ctx)
    V = np.asarray(x["v"], np.float64)
    O1, LSE1 = phase1(Q, K, V, w.b, w.a, scale)
    qq, kq = rot(x["qq"], pos_q), rot(x["kq"], pos_q)
    qd, kd = rot(x["qd"], pos_d), rot(x["kd"], pos_d)
    Kc = np.concatenate([K, kq, kd], axis=2)
    Vc = np.concatenate([V, np.asarray(x["vq"], np.float64),
                         np.asarray(x["vd"], np.float64)], axis=2)
    res = {"Q": Q, "K": K, "V": V, "O1": O1, "LSE1": LSE1, "Kc": Kc, "Vc": Vc,
           "qq": qq, "qd": qd}
    parts_q = partitions(L, w.b, L + w.Lq)
    O2 = np.zeros((B, Hq, w.Lq, D))
    L2 = np.zeros((B, Hq, w.Lq))
    P2o = np.zeros((len(parts_q), B, Hq, w.Lq, D))
    P2l = np.zeros((len(parts_q), B, Hq, w.Lq))
    OD = np.zeros((B, Hq, w.T, D))
    LD = np.zeros((B, Hq, w.T))
    for bb in range(B):
        for h in range(Hq):
            kv = h // g
            o, l, op, lp = phase2(qq[bb, h], pos_q, Kc[bb, kv], Vc[bb, kv],
                                  parts_q, scale)
            O2[bb, h], L2[bb, h], P2o[:, bb, h], P2l[:, bb, h] = o, l, op, lp
            for t in range(w.T):
                parts_t = partitions(L, w.b, L + w.Lq + t + 1)
                o, l, _, _ = phase2(qd[bb, h, t:t + 1], pos_d[t:t + 1],
                                    Kc[bb, kv], Vc[bb, kv], parts_t, scale)
                OD[bb, h, t], LD[bb, h, t] = o[0], l[0]
    res.update(O2=O2, LSE2=L2, P2o=P2o, P2l=P2l, OD=OD, LSED=LD)
    return res


# ----------------------------------------------------------------------------
# Phase 1 with an explicit per-block prefix (anchor variants and Pulsar)
# ----------------------------------------------------------------------------
def phase1_prefix_keys(n_prefix: int, n_block: int, rows=None):
    """Mask of one augmented block [prefix ; own block]: every row sees all
    ``n_prefix`` prefix keys (they precede the block) and its own block's
    keys up to itself.  Returns mask[len(rows), n_prefix + n_block]."""
    r = np.arange(n_block) if rows is None else np.asarray(rows)
    causal = np.arange(n_block)[None, :] <= r[:, None]
    return np.concatenate([np.ones((r.size, n_prefix), dtype=bool), causal], axis=1)


def phase1_prefix(Q, K, V, PK, PV, starts, lens, b: int, scale: float):
    """Phase 1 where block i's prefix is rows [starts[i], starts[i] + lens[i])
    of PK/PV instead of the fixed anchor.

    This is the common form of the anchor variants the Star Attention pages
    ablate ([SA-atlas] "Measured effects reported in the paper": no anchor,
    anchor with other position ids, anchor with other content) and of the
    Pulsar prefix ([Pulsar] "What carries the argument": host i encodes
    [sink || summaries of blocks 0..i-1 || B_i] and then drops the prefix
    KV).  Q [B, Hq, L, D]; K/V [B, Hkv, L, D]; PK/PV [B, Hkv, R, D].
    Returns O [B, Hq, L, D] and LSE [B, Hq, L].
    """
    B, Hq, L, D = Q.shape
    g = Hq // K.shape[1]
    O = np.zeros((B, Hq, L, D))
    LSE = np.full((B, Hq, L), NEG_INF)
    for i, (s, e) in enumerate(blocks(L, b)):
        p0, p1 = int(starts[i]), int(starts[i]) + int(lens[i])
        mask = phase1_prefix_keys(p1 - p0, e - s)
        for bb in range(B):
            for h in range(Hq):
                kv = h // g
                keys = np.concatenate([PK[bb, kv, p0:p1], K[bb, kv, s:e]])
                vals = np.concatenate([PV[bb, kv, p0:p1], V[bb, kv, s:e]])
                o, l = attend(Q[bb, h, s:e], keys, vals, mask, scale)
                O[bb, h, s:e], LSE[bb, h, s:e] = o, l
    return O, LSE


def phase1_prefix_rows(q_rows, pos, K, V, PK, PV, starts, lens, b: int, scale: float):
    """:func:`phase1_prefix` for selected rows of one (batch, query head):
    ``q_rows[n, D]`` at context positions ``pos[n]``; K/V [L, D] and PK/PV
    [R, D] are that head's KV head."""
    L = K.shape[0]
    pos = np.asarray(pos)
    o = np.zeros((pos.size, V.shape[1]))
    lse = np.full(pos.size, NEG_INF)
    for i, (s, e) in enumerate(blocks(L, b)):
        sel = np.nonzero((pos >= s) & (pos < e))[0]
        if sel.size == 0:
            continue
        p0, p1 = int(starts[i]), int(starts[i]) + int(lens[i])
        mask = phase1_prefix_keys(p1 - p0, e - s, rows=pos[sel] - s)
        keys = np.concatenate([PK[p0:p1], K[s:e]])
        vals = np.concatenate([PV[p0:p1], V[s:e]])
        oo, ll = attend(q_rows[sel], keys, vals, mask, scale)
        o[sel], lse[sel] = oo, ll
    return o, lse


def anchor_prefix_table(L: int, b: int, a: int):
    """The Star anchor as a prefix table over the context K/V themselves:
    block 0 has none, block i >= 1 has rows [0, a) ([SA-pith] "What carries
    the argument")."""
    n = len(blocks(L, b))
    starts = np.zeros(n, dtype=np.int64)
    lens = np.array([0] + [min(a, L)] * (n - 1), dtype=np.int64)
    return starts, lens


def remapped_anchor(K_pre, pos_per_block, base: float, store_bf16: bool = True):
    """Anchor keys re-rotated at other position ids, one copy per block.

    The position-id ablation ([SA-atlas] "Measured effects reported in the
    paper"; [SA-pith] "Core claim": the content of the anchor matters, its
    position ids much less) keeps the anchor's content (the first ``a``
    context tokens, un-rotated keys ``K_pre[..., :a, :]``) and rotates it at
    ``pos_per_block[i]`` (``a`` positions) for block i.  Row block i of the
    result (rows [i*a, (i+1)*a)) is that block's anchor; block 0's slot is
    unused.  Values need no rotation: the anchor V is block 1's V.
    """
    K_pre = np.asarray(K_pre, dtype=np.float64)
    out = []
    for pos in pos_per_block:
        pos = np.asarray(pos)
        r = rope(K_pre[..., :pos.size, :], pos, base)
        out.append(round_bf16(r) if store_bf16 else r)
    return np.concatenate(out, axis=-2)


# ----------------------------------------------------------------------------
# Pulsar: attention sink + Max-IDF chunk summaries of the earlier blocks
# ----------------------------------------------------------------------------
def chunks_of_block(s: int, e: int, m: int):
    """Chunks of m consecutive tokens of block [s, e) ([Pulsar] "What
    carries the argument": chunks of 32 tokens); the last one is shorter
    when m does not divide the block length."""
    return [(c, min(c + m, e)) for c in range(s, e, m)]


def document_frequency(tokens, L: int, b: int) -> dict:
    """df(t) = number of blocks that contain token t ([Pulsar] "What carries
    the argument")."""
    df = {}
    for s, e in blocks(L, b):
        for t in set(int(x) for x in tokens[s:e]):
            df[t] = df.get(t, 0) + 1
    return df


def maxidf_score(chunk_tokens, df: dict, n: int) -> float:
    """score(C) = max over the chunk's tokens of IDF(t) = log(n / max(df(t), 1))
    ([Pulsar] "What carries the argument")."""
    return max(math.log(n / max(df.get(int(t), 0), 1)) for t in chunk_tokens)


def maxidf_summaries(tokens, L: int, b: int, m: int, sink: int, k: int):
    """Summary Sigma_i of every block: its k best chunks by Max-IDF score,
    listed in positional order ([Pulsar] "What carries the argument", "Core
    claim").  Readings: equal scores go to the earlier chunk; block 0's
    chunks that overlap the sink are not candidates (those tokens are already
    in every prefix); a block with fewer candidates than k keeps them all.
    Returns a list of token-index arrays, one per block.
    """
    bl = blocks(L, b)
    n = len(bl)
    df = document_frequency(tokens, L, b)
    out = []
    for i, (s, e) in enumerate(bl):
        cands = [(c0, c1) for (c0, c1) in chunks_of_block(s, e, m)
                 if not (i == 0 and c0 < sink)]
        scored = [(-maxidf_score(tokens[c0:c1], df, n), c0, c1) for (c0, c1) in cands]
        best = sorted(scored)[:k]                      # highest score, then earliest
        best = sorted(best, key=lambda t: t[1])        # positional order
        rows = [np.arange(c0, c1) for (_, c0, c1) in best]
        out.append(np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64))
    return out


def pulsar_prefix(tokens, L: int, b: int, m: int = 32, sink: int = 64, k: int = 16):
    """Host i's prefix [sink || Sigma_0 || ... || Sigma_{i-1}] ([Pulsar] "What
    carries the argument") as one list of context rows plus a per-block
    table into it: block i's prefix is rows[starts[i] : starts[i] + lens[i]].
    Reading: host 0 is plain causal over its own block (its sink is its own
    first tokens), as Star's first block carries no anchor.
    Returns (rows[R], starts[n], lens[n]).
    """
    sums = maxidf_summaries(tokens, L, b, m, sink, k)
    n = len(sums)
    sink_rows = np.arange(min(sink, L, b))
    rows = [sink_rows] + sums[:-1]
    rows = np.concatenate(rows).astype(np.int64)
    starts = np.zeros(n, dtype=np.int64)
    lens = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        lens[i] = sink_rows.size + sum(x.size for x in sums[:i])
    return rows, starts, lens


def pulsar_host_length(L: int, b: int, sink: int, s: int, i: int) -> int:
    """Tokens host i encodes in Phase 1 when every summary has s tokens:
    b + sink + i*s (host 0: b) ([Pulsar] "Referee Report", major comment 1,
    and Eq. 4 as restated there)."""
    n_i = min(b, L - i * b)
    return n_i if i == 0 else n_i + sink + i * s


# ----------------------------------------------------------------------------
# The attention layer around Phase 1 (Llama-3 attention block, any weights)
# ----------------------------------------------------------------------------
def rmsnorm(x, gamma, eps: float):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma (the
    Llama-3 input normalisation; [SA-repo] README: HuggingFace Llama
    models)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def _maybe_bf16(t, store_bf16: bool):
    return round_bf16(t) if store_bf16 else t


def layer_projections(xs, w, Hq: int, Hkv: int, D: int, eps: float, store_bf16: bool = True):
    """h = rmsnorm(x); q, k, v = h Wq^T, h Wk^T, h Wv^T for xs [B, n, H].
    Returns q [B, Hq, n, D], k and v [B, Hkv, n, D] (un-rotated).  Every
    stored tensor is bf16 in the model, so with ``store_bf16`` h and the
    projections are rounded to bf16."""
    B, n, _ = xs.shape
    h = _maybe_bf16(rmsnorm(xs, w["gamma"], eps), store_bf16)
    def proj(W, H):
        y = _maybe_bf16(h @ np.asarray(W, np.float64).T, store_bf16)
        return y.reshape(B, n, H, D).transpose(0, 2, 1, 3)
    return proj(w["wq"], Hq), proj(w["wk"], Hkv), proj(w["wv"], Hkv)


def layer_output(xs, O, w, store_bf16: bool = True):
    """out = x + O_flat Wo^T: the output projection and the residual add.
    O [B, Hq, n, D] is the attention output (stored in bf16)."""
    B, Hq, n, D = O.shape
    of = np.asarray(O, np.float64).transpose(0, 2, 1, 3).reshape(B, n, Hq * D)
    return _maybe_bf16(np.asarray(xs, np.float64) + of @ np.asarray(w["wo"], np.float64).T,
                       store_bf16)


def attention_layer_phase1(x, w, Hq: int, Hkv: int, D: int, b: int, a: int, base: float,
                           eps: float, rope_on: bool = True, store_bf16: bool = True,
                           round_output: bool = True):
    """One attention layer over the whole context with Phase-1 attention, as
    one device computes it: every token's q/k/v once, the anchor's K/V read
    from block 1's rows ([SA-pith] "What carries the argument").

    x [B, L, H] (H = Hq*D); w: gamma [H], wq [Hq*D, H], wk/wv [Hkv*D, H],
    wo [H, Hq*D].  Returns (out [B, L, H], K [B, Hkv, L, D] rotated,
    V [B, Hkv, L, D]).  ``round_output=False`` leaves the final output in
    float64 (the intermediate stored tensors are still rounded).
    """
    B, L, _ = x.shape
    q, k, v = layer_projections(x, w, Hq, Hkv, D, eps, store_bf16)
    pos = np.arange(L)
    if rope_on:
        q = _maybe_bf16(rope(q, pos, base), store_bf16)
        k = _maybe_bf16(rope(k, pos, base), store_bf16)
    O, _ = phase1(q, k, v, b, a if b < L else 0, 1.0 / math.sqrt(D))
    O = _maybe_bf16(O, store_bf16)
    return layer_output(x, O, w, store_bf16 and round_output), k, v


def causal_layer(xs, pos, w, Hq: int, Hkv: int, D: int, base: float, eps: float,
                 rope_on: bool = True, store_bf16: bool = True):
    """One attention layer with plain causal attention over the sequence xs
    [B, n, H] whose tokens sit at positions ``pos[n]`` (sequence order is
    causal order)."""
    B, n, _ = xs.shape
    q, k, v = layer_projections(xs, w, Hq, Hkv, D, eps, store_bf16)
    if rope_on:
        q = _maybe_bf16(rope(q, pos, base), store_bf16)
        k = _maybe_bf16(rope(k, pos, base), store_bf16)
    g = Hq // Hkv
    mask = np.tril(np.ones((n, n), dtype=bool))
    O = np.zeros_like(q)
    for bb in range(B):
        for h in range(Hq):
            O[bb, h], _ = attend(q[bb, h], k[bb, h // g], v[bb, h // g], mask, 1.0 / math.sqrt(D))
    return layer_output(xs, _maybe_bf16(O, store_bf16), w, store_bf16)


def star_context_per_host(x, layers, Hq: int, Hkv: int, D: int, b: int, a: int, base: float,
                          eps: float, rope_on: bool = True, store_bf16: bool = True):
    """Phase-1 context encoding through a stack of layers exactly as the
    pages describe it, host by host ([SA-pith] "What carries the argument",
    [SA-atlas] "Approach"): host 1 runs block 1 through every layer with
    causal attention; host i >= 2 runs [anchor ; block i] (the anchor = the
    first a tokens at their original positions) through every layer with
    causal attention over that augmented sequence and keeps only block i's
    rows.  Returns the final hidden states [B, L, H]."""
    B, L, H = x.shape
    out = np.zeros((B, L, H))
    for i, (s, e) in enumerate(blocks(L, b)):
        if i == 0 or a == 0:
            idx = np.arange(s, e)
        else:
            idx = np.concatenate([np.arange(min(a, L)), np.arange(s, e)])
        xs = np.asarray(x, np.float64)[:, idx]
        for w in layers:
            xs = causal_layer(xs, idx, w, Hq, Hkv, D, base, eps, rope_on, store_bf16)
        out[:, s:e] = xs[:, idx.size - (e - s):]
    return out


def star_context_layers(x, layers, Hq: int, Hkv: int, D: int, b: int, a: int, base: float,
                        eps: float, rope_on: bool = True, store_bf16: bool = True):
    """The same stack computed as one device does: every layer applies
    :func:`attention_layer_phase1` to all L tokens, so the anchor's K/V at
    every layer are block 1's own rows of that layer."""
    xs = np.asarray(x, np.float64)
    for w in layers:
        xs, _, _ = attention_layer_phase1(xs, w, Hq, Hkv, D, b, a, base, eps, rope_on, store_bf16)
    return xs
