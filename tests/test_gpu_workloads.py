"""GPU parity on the five workloads at their full sizes, run through the same
call sequence the benchmark times (block_sparse_amd.pipeline).

Tiny is compared on every output element, in both its fp32 and bf16 forms.
The Llama-shaped workloads are compared for every (batch, query head), on
the call sequence the benchmark times (Q rotated in a pass of its own before
Phase 1), and Phase 1 with Q rotated inside the kernel is checked bit for bit
against it at full size:
  * the rotated K cache (context, query and decode rows): bit for bit
    against the oracle's exact rotation rounded once to bf16;
  * Phase 1: llama8b-16k on every row; the larger ones on the first two and
    last two rows of every block plus 64 seeded random rows of every block,
    each computed exactly by the oracle over all its visible keys;
  * Phase 2: every query row and every decode step;
and on properties that hold at any size (every Phase-1 output and lse of
every head finite).  The Phase-1 variants (Pulsar's sink + Max-IDF summaries,
the anchor at other position ids) are checked the same way at the 8B-128K
and 70B-64K shapes.
"""
import math
import time

import numpy as np
import pytest
import torch

import block_sparse_amd as sa
import oracle.star_oracle as so
from block_sparse_amd.pipeline import StarAttentionStep, partition_offsets
from gpu_util import check_lse, check_out, chunk_ranges, f64, host64, to_dev
from workloads import TINY, WORKLOADS, as_f64, f32_to_bf16_bits, inputs

pytestmark = pytest.mark.gpu


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "fp32"])
def test_tiny_full(bf16):
    w = TINY
    log(f"tiny bf16={bf16}: inputs")
    x = inputs(w, as_bf16=bf16)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    o1, l1 = sa.phase1_blocklocal(q, k, v, w.b, w.a, want_lse=True)
    kc = torch.cat([k, to_dev(x["kq"])], dim=2).contiguous()
    vc = torch.cat([v, to_dev(x["vq"])], dim=2).contiguous()
    offs = partition_offsets(w.L, w.b, w.L + w.Lq)
    op, lp = sa.phase2_partial(to_dev(x["qq"]), kc, vc, offs, splits=1, q_pos0=w.L)
    o2, l2 = sa.lse_merge(op, lp)
    torch.cuda.synchronize()
    xf = {n: as_f64(t) for n, t in x.items()}
    ref = so.star_attention(w, xf)
    wabs, _ = so.phase1(xf["q"], xf["k"], np.abs(xf["v"]), w.b, w.a, 1 / math.sqrt(w.D))
    check_out(host64(o1), ref["O1"], "phase1 O", bf16_out=True, wabs=wabs)
    check_lse(host64(l1), ref["LSE1"], "phase1 LSE")
    check_out(host64(op), ref["P2o"], "phase2 partials")
    check_lse(host64(lp), ref["P2l"], "phase2 partial lse")
    check_out(host64(o2), ref["O2"], "phase2 O")
    check_lse(host64(l2), ref["LSE2"], "phase2 LSE")


# name -> (random rows per block, every Phase-1 row?)
LLAMA = {
    "llama8b-16k": (0, True),
    "llama8b-128k": (64, False),
    "llama70b-64k": (64, False),
    "llama8b-1m": (64, False),
}


def sample_rows(w, rows_per_block, seed):
    rng = np.random.default_rng(seed)
    pos = []
    for s, e in so.blocks(w.L, w.b):
        n = e - s
        pos += [s, s + 1, e - 2, e - 1]
        if rows_per_block:
            pos += (s + rng.choice(n, size=min(rows_per_block, n), replace=False)).tolist()
    return np.unique(np.array(pos, dtype=np.int64))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name", list(LLAMA))
def test_llama_workload(name):
    w = WORKLOADS[name]
    rows_per_block, full_rows = LLAMA[name]
    g = w.g
    scale = 1.0 / math.sqrt(w.D)
    log(f"{name}: generating inputs")
    x = inputs(w, as_bf16=True)
    log(f"{name}: GPU pass")
    st = StarAttentionStep(w.B, w.Hq, w.Hkv, w.D, w.L, w.b, w.Lq, w.T, rope=True, base=w.base)
    dev = {n: to_dev(t) for n, t in x.items() if n != "v"}
    st.load_context(to_dev(x["v"]))
    st.run(dev["q"], dev["k"], dev["qq"], dev["kq"], dev["vq"], dev["qd"], dev["kd"], dev["vd"])
    torch.cuda.synchronize()
    # the step rotates Q in a pass of its own; the Phase-1 form that rotates
    # Q inside the kernel gives the same bits at full size
    log(f"{name}: Phase 1 with the rotation of Q inside the kernel")
    of = torch.empty_like(st.o1)
    lf = torch.empty_like(st.lse1)
    sa.phase1_rope(dev["q"], st.kc[:, :, :w.L], st.vc[:, :, :w.L], w.b, w.a, w.base, scale,
                   out=of, lse=lf, sched=st.sched)
    torch.cuda.synchronize()
    assert torch.equal(of.view(torch.int16), st.o1.view(torch.int16)), "fused-RoPE O differs"
    assert torch.equal(lf.view(torch.int32), st.lse1.view(torch.int32)), "fused-RoPE lse differs"
    del of, lf
    # properties over every head at full size
    assert bool(torch.isfinite(st.o1).all()), "non-finite Phase-1 output"
    assert bool(torch.isfinite(st.lse1).all()), "non-finite Phase-1 lse"
    assert bool(torch.isfinite(st.o2).all()) and bool(torch.isfinite(st.od).all())
    del dev
    pos = np.arange(w.L) if full_rows else sample_rows(w, rows_per_block, w.seed)
    pos_t = torch.from_numpy(pos).cuda()
    pos_c = np.arange(w.L)
    pos_q = w.L + np.arange(w.Lq)
    pos_d = w.L + w.Lq + np.arange(w.T)
    parts = so.partitions(w.L, w.b, w.cache_len)
    worst = {}
    for bb in range(w.B):
        for kvh in range(w.Hkv):
            log(f"{name}: oracle b={bb} kv head {kvh}")
            # rotated Q/K are stored in bf16 (the cache dtype) before attention
            rot = lambda t, p: so.round_bf16(so.rope(t, p, w.base))
            K = rot(f64(x["k"][bb, kvh]), pos_c)
            V = f64(x["v"][bb, kvh])
            Kc = np.concatenate([K, rot(f64(x["kq"][bb, kvh]), pos_q),
                                 rot(f64(x["kd"][bb, kvh]), pos_d)])
            Vc = np.concatenate([V, f64(x["vq"][bb, kvh]), f64(x["vd"][bb, kvh])])
            # the rotated cache rows, bit for bit (context, query and decode keys)
            got_k = bf16_bits(st.kc[bb, kvh])
            ref_k = f32_to_bf16_bits(Kc.astype(np.float32))
            bad = np.nonzero(got_k != ref_k)
            assert bad[0].size == 0, (f"{name}: {bad[0].size} rotated K elements differ from the "
                                      f"oracle's at (row, d) {list(zip(*bad))[:8]}")
            # [V | |V|]: one softmax gives the output and the average of |V|
            # (the compute term of the bf16 output's bound)
            Vw = np.concatenate([V, np.abs(V)], axis=-1)
            for h in range(kvh * g, (kvh + 1) * g):
                qrows = rot(f64(x["q"][bb, h][pos]), pos)
                rw, rl = so.phase1_rows(qrows, pos, K, Vw, w.b, w.a, scale)
                ro, wabs = rw[:, :w.D], rw[:, w.D:]
                go = host64(st.o1[bb, h].index_select(0, pos_t))
                gl = host64(st.lse1[bb, h].index_select(0, pos_t))
                e1 = check_out(go, ro, f"{name} phase1 O b{bb} h{h}", bf16_out=True, wabs=wabs)
                e2 = check_lse(gl, rl, f"{name} phase1 LSE b{bb} h{h}")
                # query rows and every decode step, against global attention
                qq = rot(f64(x["qq"][bb, h]), pos_q)
                qd = rot(f64(x["qd"][bb, h]), pos_d)
                rows = np.concatenate([qq, qd])
                rpos = np.concatenate([pos_q, pos_d])
                o, l, _, _ = so.phase2(rows, rpos, Kc, Vc, parts, scale)
                e3 = check_out(host64(st.o2[bb, h]), o[:w.Lq], f"{name} query O b{bb} h{h}")
                e4 = check_lse(host64(st.lse2[bb, h]), l[:w.Lq], f"{name} query LSE b{bb} h{h}")
                e5 = check_out(host64(st.od[bb, h, :w.T]), o[w.Lq:], f"{name} decode O b{bb} h{h}")
                e6 = check_lse(host64(st.lsed[:w.T, bb, h]), l[w.Lq:], f"{name} decode LSE b{bb} h{h}")
                for key, val in zip(("p1O", "p1mean", "p1L", "qO", "qL", "dO", "dL"),
                                    (e1[0], e1[1], e2, e3[0], e4, e5[0], e6)):
                    worst[key] = max(worst.get(key, 0.0), val)
    log(f"{name}: worst errors {worst} over {pos.size} Phase-1 rows per head, "
        f"{w.B * w.Hq} heads; rotated K bit-exact over {w.cache_len} rows x {w.B * w.Hkv} heads")


# Phase-1 variants at full size: (workload, variant)
VARIANTS = [("llama8b-128k", "pulsar"), ("llama8b-128k", "anchor_remap"),
            ("llama70b-64k", "pulsar")]


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name,variant", VARIANTS, ids=[f"{n}-{v}" for n, v in VARIANTS])
def test_llama_phase1_variants(name, variant):
    """Pulsar's prefix and the anchor at other position ids, at the
    workloads' full shapes, on sampled rows (block edges plus 32 seeded rows
    per block) of every (batch, query head)."""
    from workloads import anchor_positions, pulsar_params, token_ids
    w = WORKLOADS[name]
    g = w.g
    scale = 1.0 / math.sqrt(w.D)
    log(f"{name} {variant}: generating inputs")
    x = inputs(w, as_bf16=True)
    st = StarAttentionStep(w.B, w.Hq, w.Hkv, w.D, w.L, w.b, 0, 0, rope=True, base=w.base)
    st.load_context(to_dev(x["v"]))
    kdev = to_dev(x["k"])
    st.rope_context(to_dev(x["q"]), kdev)
    pp = pulsar_params(w)
    tok = token_ids(w.seed, w.B, w.L)
    apos = anchor_positions(w.seed, w.L, w.b, w.a)
    log(f"{name} {variant}: GPU pass")
    if variant == "pulsar":
        st.pulsar_setup(tok, pp.m, pp.sink, pp.k)
        st.phase1_pulsar()
    else:
        st.anchor_remap_setup(apos)
        st.phase1_anchor_remap(kdev)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(st.o1).all()) and bool(torch.isfinite(st.lse1).all())
    pos = sample_rows(w, 32, w.seed + 100)
    kv_heads = range(w.Hkv)
    pos_t = torch.from_numpy(pos).cuda()
    rot = lambda t, p: so.round_bf16(so.rope(t, p, w.base))
    worst = [0.0, 0.0]
    for bb in range(w.B):
        if variant == "pulsar":
            rows, pst, pln = so.pulsar_prefix(tok[bb], w.L, w.b, pp.m, pp.sink, pp.k)
        for kvh in kv_heads:
            log(f"{name} {variant}: oracle b={bb} kv head {kvh}")
            K = rot(f64(x["k"][bb, kvh]), np.arange(w.L))
            V = f64(x["v"][bb, kvh])
            if variant == "pulsar":
                PK, PV = K[rows], V[rows]
            else:
                PK = so.remapped_anchor(f64(x["k"][bb, kvh]), apos, w.base)
                PV = np.concatenate([V[:w.a]] * len(apos))
                pst = np.arange(len(apos)) * w.a
                pln = np.array([0] + [w.a] * (len(apos) - 1))
            Vw = np.concatenate([V, np.abs(V)], axis=-1)
            PVw = np.concatenate([PV, np.abs(PV)], axis=-1)
            for h in range(kvh * g, (kvh + 1) * g):
                qrows = rot(f64(x["q"][bb, h][pos]), pos)
                rw, rl = so.phase1_prefix_rows(qrows, pos, K, Vw, PK, PVw, pst, pln, w.b, scale)
                ro, wabs = rw[:, :w.D], rw[:, w.D:]
                e1 = check_out(host64(st.o1[bb, h].index_select(0, pos_t)), ro,
                               f"{name} {variant} O b{bb} h{h}", bf16_out=True, wabs=wabs)
                e2 = check_lse(host64(st.lse1[bb, h].index_select(0, pos_t)), rl,
                               f"{name} {variant} LSE b{bb} h{h}")
                worst = [max(worst[0], e1[0]), max(worst[1], e2)]
    log(f"{name} {variant}: worst O {worst[0]:.3e} LSE {worst[1]:.3e} over {pos.size} rows/head")
