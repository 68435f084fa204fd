"""Benchmark of the Star Attention two-phase hot path on one MI355X.

One step = one whole pass over one batch of synthetic input, resident in HBM:
RoPE of the context Q/K at original positions (K straight into the KV cache),
Phase-1 anchor-block blockwise-local attention, the Phase-2 query (RoPE, KV
append, partials over every partition, LSE merge) and every decode step
(same, one token each).  Default workload: Llama-3.1-8B layer shapes at
131072-token context, b = 16384 (8 KV partitions), 64 query tokens, 128
decode steps.

Prints ONE JSON line.  ``value`` is whole-step context tokens/s
(B*L per step / step time).  ``phase1`` / ``decode`` hold the per-phase
rates; ``roofline`` is for the dominant kernel (the Phase-1 flash kernel,
bf16 MFMA), timed with HIP events on the stream it is launched on;
``cpu_baseline`` is the fp64 CPU oracle timed on a bounded sample;
``phase1.separate_rope`` times the step's Phase 1 (the rotation of Q as a
pass of its own) against the form that rotates Q inside the kernel.  Beside
them: ``decode_cold`` (each step after a cache-flushing read),
``decode_graph`` (steps replayed from captured HIP graphs),
``phase2_query`` (the query partials against their roofline),
``hbm_stream`` (the streaming-read reference), ``phase1_variants``,
``phase1_layer`` and ``per_config`` (one record per workload with the errors
of a sampled parity check against the oracle).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --cpu-full [NAMES] [--cpu-full-only]   # whole-oracle timings
    python bench.py --trace-summary DIR                    # rocprofv3 csv -> table
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Phase1 context tokens/s + TFLOP/s; Phase2 decode GB/s (8B shapes, 128K ctx)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PMC_SUMMARY = os.path.join(ROOT, "profiles", "phase1_flash_llama8b-128k_pmc.txt")
FLASH_SRC = os.path.join(ROOT, "block_sparse_amd", "csrc", "flash2.hip")


def progress(msg: str):
    """One line per finished stage, on stderr (the JSON line owns stdout)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def phase1_pairs(L: int, b: int, a: int) -> int:
    """Useful (query, key) pairs of Phase 1 per head: block 1 is causal over
    itself; block i >= 2 sees a anchor keys plus its causal prefix."""
    tot = 0
    for i, s in enumerate(range(0, L, b)):
        n = min(s + b, L) - s
        tot += n * (n + 1) // 2 + (a * n if i > 0 else 0)
    return tot


def phase1_flops(w) -> float:
    return 4.0 * w.D * w.Hq * w.B * phase1_pairs(w.L, w.b, w.a)


def decode_bytes(w, t: int) -> int:
    """K and V bytes a decode step must read: every visible cached token."""
    return (w.L + w.Lq + t + 1) * w.Hkv * w.B * w.D * 2 * 2


def pmc_traffic():
    """HBM traffic per Phase-1 launch from the committed rocprofv3 counter
    summary, or None when it is absent or the kernel source changed since."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m = re.search(r"flash_src_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t:
        return None
    cur = hashlib.sha256(open(FLASH_SRC, "rb").read()).hexdigest()
    return float(t.group(1)) if m.group(1) == cur else None


def _blas_threads() -> int:
    """Threads the host BLAS uses (the oracle's matmuls run there)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(w, x, heads: int = 4, rows_per_call: int = 4096):
    """Time the CPU oracle (as it stands) on a bounded sample of Phase 1:
    every row of block 2 (anchor plus its causal prefix) for the first
    ``heads`` query heads of batch 0 (one GQA group: they share KV head 0),
    in calls of ``rows_per_call`` rows, including the RoPE of the sampled
    rows and of that KV head.  About 10-15 s on 16 host threads at the
    8B-128K shape.  Scaled to whole-workload context tokens/s by the ratio
    of useful (query, key) pairs."""
    import numpy as np

    import oracle.star_oracle as so
    from workloads import as_f64
    cores = _blas_threads()
    scale = 1.0 / math.sqrt(w.D)
    blk = 1 if w.L > w.b else 0
    s = blk * w.b
    e = min(s + w.b, w.L)
    heads = min(heads, w.g)
    t0 = time.perf_counter()
    kv = 0
    K = so.rope(as_f64(x["k"][0, kv]), np.arange(w.L), w.base) if w.rope else as_f64(x["k"][0, kv])
    V = as_f64(x["v"][0, kv])
    for h in range(heads):
        for r0 in range(s, e, rows_per_call):
            pos = np.arange(r0, min(r0 + rows_per_call, e))
            q = as_f64(x["q"][0, h][pos])
            q = so.rope(q, pos, w.base) if w.rope else q
            so.phase1_rows(q, pos, K, V, w.b, w.a, scale)
    dt = time.perf_counter() - t0
    sample_pairs = heads * sum((w.a if blk > 0 else 0) + (p - s + 1) for p in range(s, e))
    total_pairs = phase1_pairs(w.L, w.b, w.a) * w.Hq * w.B
    tokens_per_s = w.B * w.L / (dt * total_pairs / sample_pairs)
    return {"value": tokens_per_s, "unit": "context tokens/s (Phase 1, extrapolated)",
            "cores": int(cores), "affinity_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": (f"fp64 numpy oracle, Phase 1 of all {e - s} rows of block {blk + 1} "
                       f"(positions {s}-{e - 1}) for {heads} query heads of KV head 0, incl. "
                       f"RoPE; {dt:.1f} s; scaled by useful (q,k) pairs {sample_pairs:.3e} of "
                       f"{total_pairs:.3e}")}


def pages_host_pairs(L: int, b: int, a: int) -> int:
    """(query, key) pairs per head as the pages' hosts compute them: host 1
    runs causal attention over its block, host i >= 2 over its augmented
    block [anchor ; block i] of a + n_i tokens, the anchor's rows included
    (one GPU skips those rows, so they are not in the useful count)."""
    tot = 0
    for i, s in enumerate(range(0, L, b)):
        m = min(s + b, L) - s + (a if i > 0 else 0)
        tot += m * (m + 1) // 2
    return tot


def prefix_pairs(L: int, b: int, lens) -> int:
    """Useful (query, key) pairs per head of Phase 1 with a per-block prefix
    of lens[i] keys: every row sees its block's prefix and its causal
    prefix within the block."""
    tot = 0
    for i, s in enumerate(range(0, L, b)):
        n = min(s + b, L) - s
        tot += n * (n + 1) // 2 + int(lens[i]) * n
    return tot


def phase1_variants(st, dev, w, x, ev, reps=3):
    """Phase-1 time of the prefix variants on the same context (after the
    timed region): Pulsar's sink + Max-IDF summaries (gather + prefix
    attention; the host-side selection runs once, before timing) and the
    anchor re-rotated at other position ids (per-block RoPE of the anchor
    keys + gather of the anchor values + prefix attention)."""
    import numpy as np
    import torch

    from workloads import anchor_positions, pulsar_params, token_ids
    out = {}
    pp = pulsar_params(w)
    t0 = time.perf_counter()
    st.pulsar_setup(token_ids(w.seed, w.B, w.L), pp.m, pp.sink, pp.k)
    sel_ms = (time.perf_counter() - t0) * 1e3
    st.anchor_remap_setup(anchor_positions(w.seed, w.L, w.b, w.a))
    runs = {"pulsar": st.phase1_pulsar, "anchor_random_positions": lambda: st.phase1_anchor_remap(dev["k"])}
    for name, fn in runs.items():
        fn()
        torch.cuda.synchronize()
        e = [(ev(), ev()) for _ in range(reps)]
        for e0, e1 in e:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in e]))
        if name == "pulsar":
            pairs = sum(prefix_pairs(w.L, w.b, ln) for (_, _, ln, _, _) in st.pulsar) * w.Hq
            extra = {"prefix_rows_last_block": int(st.pulsar[0][2][-1]),
                     "host_selection_ms": sel_ms,
                     "params": {"chunk": pp.m, "sink": pp.sink, "chunks_per_block": pp.k}}
        else:
            pairs = prefix_pairs(w.L, w.b, st.aln) * w.Hq * w.B
            extra = {}
        fl = 4.0 * w.D * pairs
        out[name] = {"ms": ms, "context_tokens_per_s": w.B * w.L / (ms * 1e-3),
                     "tflops": fl / (ms * 1e-3) / 1e12, "algorithmic_flops": fl, **extra}
    # the Star Phase 1 leaves o1 as the timed pass did: restore it
    st.phase1()
    return out


def phase1_layer(w, ev, reps=3):
    """One Llama-3 attention layer around Phase 1 on the same shapes (seeded
    input stream and random weights): RMSNorm, the fused q/k/v projection
    (rocBLAS), RoPE, Phase 1 and the output projection with the residual,
    timed per stage with HIP events after one warm-up pass."""
    import numpy as np
    import torch

    from block_sparse_amd.layer import AttentionLayers
    from workloads import RMS_EPS, layer_inputs
    inp = layer_inputs(w, 1)
    todev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    layers = [{k: todev(v) for k, v in inp["layers"][0].items()}]
    x = todev(inp["x"])
    del inp
    st = AttentionLayers(w.B, w.Hq, w.Hkv, w.D, w.L, w.b, layers, anchor=w.a, rope=w.rope,
                         base=w.base, eps=RMS_EPS)
    st.forward(x)
    torch.cuda.synchronize()
    runs = []
    for _ in range(reps):
        marks = [("start", ev())]
        marks[0][1].record()
        def mark(name):
            e = ev()
            e.record()
            marks.append((name, e))
        st.forward(x, mark)
        runs.append(marks)
    torch.cuda.synchronize()
    stages = {}
    for marks in runs:
        for (_, e0), (name, e1) in zip(marks, marks[1:]):
            stages.setdefault(name, []).append(e0.elapsed_time(e1))
    st_ms = {k: float(np.mean(v)) for k, v in stages.items()}
    total = sum(st_ms.values())
    gf = st.gemm_flops()
    af = phase1_flops(w)
    gemm_ms = st_ms["qkv_proj"] + st_ms["o_proj"]
    out = {"ms": total, "stages_ms": st_ms,
           "context_tokens_per_s": w.B * w.L / (total * 1e-3),
           "gemm_tflops": gf / (gemm_ms * 1e-3) / 1e12,
           "phase1_tflops": af / (st_ms["phase1"] * 1e-3) / 1e12,
           "layer_tflops": (gf + af) / (total * 1e-3) / 1e12,
           "gemm_flops": gf, "note": "projections in rocBLAS (bf16, fp32 accumulate)"}
    del st, x, layers
    torch.cuda.empty_cache()
    return out


def decode_cold(st, dev, w, ev, samples=16):
    """Decode steps with cold caches: each step runs right after a 1 GiB
    device read that evicts the L2 caches and the 256 MiB Infinity Cache, so
    every K/V byte comes from HBM.  The flush reads rather than writes: a
    written flush leaves dirty lines whose write-back then competes with the
    timed reads (it halves a plain streaming read's rate on this chip).

    An event recorded between the flush and the step would itself cost
    several microseconds (the command processor finishes the flush and the
    marker before it dispatches the step), so the step is timed as the
    difference of two interleaved sequences: [event, flush, step, event] and
    [event, flush, event].  Re-runs decode steps spread over 0..T-1 after
    the timed pass (the cache rows they append hold the same values)."""
    import numpy as np
    import torch

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    ts = sorted(set(np.linspace(0, w.T - 1, min(samples, w.T)).astype(int).tolist()))
    # untimed round first: the first reduction loads its kernel
    for _ in range(2):
        torch.sum(flush, dim=0, out=sink)
        st.decode(ts[0], dev["qd"][:, :, ts[0]:ts[0] + 1], dev["kd"][:, :, ts[0]:ts[0] + 1],
                  dev["vd"][:, :, ts[0]:ts[0] + 1])
    torch.cuda.synchronize()
    with_step, flush_only = [], []
    for t in ts:
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record()
        torch.sum(flush, dim=0, out=sink)
        st.decode(t, dev["qd"][:, :, t:t + 1], dev["kd"][:, :, t:t + 1],
                  dev["vd"][:, :, t:t + 1])
        e1.record()
        e2.record()
        torch.sum(flush, dim=0, out=sink)
        e3.record()
        with_step.append((t, e0, e1))
        flush_only.append((e2, e3))
    torch.cuda.synchronize()
    a = [e0.elapsed_time(e1) for _, e0, e1 in with_step]
    f = [e2.elapsed_time(e3) for e2, e3 in flush_only]
    step_ms = float(np.median(a) - np.median(f))
    byts = float(np.mean([decode_bytes(w, t) for t, _, _ in with_step]))
    gbps = byts / (step_ms * 1e-3) / 1e9
    del flush
    return {"us_per_step": step_ms * 1e3, "gbps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBS,
            "steps_sampled": len(ts), "flush_us": float(np.median(f)) * 1e3,
            "flush_us_std": float(np.std(f)) * 1e3,
            "note": "each step right after a 1 GiB read that flushes L2 and Infinity Cache; "
                    "median of [flush + step] minus median of [flush] over interleaved "
                    "samples"}


def query_flops(w) -> float:
    """Algorithmic FLOPs of the Phase-2 query partials: query row r (at
    position L + r) sees L + r + 1 keys, 4 D FLOPs per (row, key) pair."""
    return 4.0 * w.D * w.Hq * w.B * sum(w.L + r + 1 for r in range(w.Lq))


def query_bytes(w) -> int:
    """K and V bytes the query partials read: every key once per KV head."""
    return (w.L + w.Lq) * w.Hkv * w.B * w.D * 2 * 2


def phase2_query(st, w, ev, in_step_ms, reps=20):
    """The Phase-2 query partials (the flash kernel in partial mode) against
    min(MFMA peak, arithmetic intensity x HBM peak).

    ``in_step_ms``: the partials call's duration inside each timed step
    (events recorded right around it), the reported figure (None: report
    the sustained rate).  The call runs
    once per step, right after Phase 1; timed back to back instead, the
    kernel's clock moves with the chip's power management (a trace at
    8B-128K shows ~135 us for the first dozen launches, then 160-200 us), so
    that sustained rate (median of 3 x ``reps``) is reported beside it."""
    import numpy as np
    import torch

    from block_sparse_amd import phase2_partial
    from block_sparse_amd.pipeline import partition_offsets
    offs = partition_offsets(w.L, w.b, w.L + w.Lq)

    def timed(n):
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(n):
            phase2_partial(st.qq_r[:, :, :w.Lq], st.kc, st.vc, offs, st.sq, q_pos0=w.L,
                           scale=st.scale, o_part=st.op_q, lse_part=st.lp_q)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    timed(1)
    sustained = [timed(reps) for _ in range(3)]
    ms = float(np.median(in_step_ms if in_step_ms else sustained))
    fl, by = query_flops(w), query_bytes(w)
    tflops = fl / (ms * 1e-3) / 1e12
    gbps = by / (ms * 1e-3) / 1e9
    ai = fl / by
    roof = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3)
    sus = float(np.median(sustained))
    return {"us": ms * 1e3, "tflops": tflops, "gbps": gbps, "flops": fl, "bytes": by,
            "arith_intensity": ai, "roofline_tflops": roof, "frac_of_roofline": tflops / roof,
            "samples": len(in_step_ms) if in_step_ms else 0,
            "sustained_us": sus * 1e3,
            "sustained_frac_of_roofline": fl / (sus * 1e-3) / 1e12 / roof,
            "splits": st.sq,
            "note": "star_phase2_partial for the query rows: median over the timed steps "
                    "(events around the call inside each step); sustained = "
                    f"{reps} back to back; roofline = min(bf16 MFMA peak, flop/byte x HBM peak)"}


def decode_graph(st, w, ev, n):
    """Decode steps replayed from captured HIP graphs (pipeline.DecodeGraph:
    star_decode_step_devpos and its merge, the position in device memory),
    against the eager steps whose host-side launch work can exceed a short
    step's GPU time.
      sequence: ``n`` consecutive steps captured in one graph and replayed
        once, as a per-token graph of a model with ``n`` attention layers
        would hold them: the runtime's gap between graph launches is paid
        once.
      one_step: a graph of one step, replayed ``n`` times back to back.
    Writes cache rows L + Lq .. L + Lq + n - 1, as the timed steps do."""
    import numpy as np
    import torch

    from block_sparse_amd.pipeline import DecodeGraph
    p0 = w.L + w.Lq
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    out = {}
    for name, steps, replays in (("one_step", 1, n), ("sequence", n, 1)):
        dg = DecodeGraph(st, p0, steps)
        for t in (dg.q_in, dg.k_in, dg.v_in):
            t.copy_(torch.randn(t.shape, device="cuda", generator=gen))
        dg.replay()                                 # untimed first replay
        dg.set_position(p0)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(replays):
            dg.replay()
        e1.record()
        torch.cuda.synchronize()
        if int(dg.pos.item()) != p0 + n:
            raise RuntimeError("device position did not advance once per step")
        out[name] = e0.elapsed_time(e1) / n
        del dg
    byts = float(np.mean([decode_bytes(w, t) for t in range(n)]))
    ms = out["sequence"]
    return {"us_per_step": ms * 1e3, "gbps": byts / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "one_step_graph_us_per_step": out["one_step"] * 1e3, "steps": n,
            "note": f"{n} decode steps (star_decode_step_devpos + merge) captured in one HIP "
                    "graph and replayed; one_step_graph: a one-step graph replayed "
                    f"{n} times (each replay adds the runtime's gap between graph launches)"}


def phase1_separate_rope(st, dev, w, ev, reps=5):
    """The same box, interleaved: Phase 1 with Q rotated inside the kernel
    (star_phase1_rope) against the step's form, the rotation of Q as a pass
    of its own (star_rope_apply) followed by star_phase1_blocklocal on the
    rotated Q.  Both give the same bits; the second kernel does attention
    only."""
    import numpy as np
    import torch

    import block_sparse_amd as sa
    L = w.L
    t = {"fused": [], "rope_q": [], "blocklocal": []}
    for _ in range(reps):
        e = [ev() for _ in range(4)]
        e[0].record()
        sa.phase1_rope(dev["q"], st.kc[:, :, :L], st.vc[:, :, :L], st.b, st.a, w.base,
                       st.scale, out=st.o1, lse=st.lse1, sched=st.sched)
        e[1].record()
        sa.rope_apply(dev["q"], pos0=0, base=w.base, out=st.qr)
        e[2].record()
        sa.phase1_blocklocal(st.qr, st.kc[:, :, :L], st.vc[:, :, :L], st.b, st.a, st.scale,
                             out=st.o1, lse=st.lse1, sched=st.sched)
        e[3].record()
        torch.cuda.synchronize()
        for k, (a, b) in zip(t, ((0, 1), (1, 2), (2, 3))):
            t[k].append(e[a].elapsed_time(e[b]))
    med = {k: float(np.median(v)) for k, v in t.items()}
    fl = phase1_flops(w)
    return {"fused_ms": med["fused"], "rope_q_ms": med["rope_q"],
            "blocklocal_ms": med["blocklocal"],
            "separate_total_ms": med["rope_q"] + med["blocklocal"],
            "blocklocal_tflops": fl / (med["blocklocal"] * 1e-3) / 1e12,
            "blocklocal_frac_of_peak": fl / (med["blocklocal"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "reps": reps,
            "note": "medians of interleaved launches: star_phase1_rope against the step's "
                    "star_rope_apply on Q + star_phase1_blocklocal (same output bits; that "
                    "kernel does attention only)"}


def config_record(name, ev, rows_per_block=8, decode_steps=16):
    """One record per workload: Phase-1 time and rate, the Phase-2 query
    and warm decode-step times, and the parity errors of a small sampled
    check against the oracle.  The device inputs are seeded normal draws;
    batch 0's KV head 0 and its query heads are the seeded workload draws
    (workloads.draw_tensor), so the oracle regenerates exactly those slices
    and checks: block edges plus ``rows_per_block`` seeded rows of every
    block of Phase 1, every query row, and the timed decode steps."""
    import numpy as np
    import torch

    import oracle.star_oracle as so
    from block_sparse_amd.pipeline import StarAttentionStep
    from workloads import (T_K, T_KD, T_KQ, T_Q, T_QD, T_QQ, T_V, T_VD, T_VQ, WORKLOADS,
                           bf16_bits_to_f32, draw_tensor)
    w = WORKLOADS[name]
    g = w.g
    n_dec = min(w.T, decode_steps)
    gen = torch.Generator(device="cuda").manual_seed(1000 + w.seed)
    host = {}

    def make(key, tid, H, S):
        t = torch.empty((w.B, H, S, w.D), dtype=torch.bfloat16, device="cuda")
        for bb in range(w.B):
            for h in range(H):
                t[bb, h].copy_(torch.randn((S, w.D), generator=gen, device="cuda") * w.scale)
        nh = g if H == w.Hq else 1          # batch 0: KV head 0 and its query heads
        bits = draw_tensor(w.seed, tid, 1, nh, S, w.D, w.scale)
        host[key] = bf16_bits_to_f32(bits[0]).astype(np.float64)
        t[0, :nh].copy_(torch.from_numpy(bits[0].view(np.int16)).view(torch.bfloat16))
        return t

    q, k, v = make("q", T_Q, w.Hq, w.L), make("k", T_K, w.Hkv, w.L), make("v", T_V, w.Hkv, w.L)
    qq, kq, vq = (make("qq", T_QQ, w.Hq, w.Lq), make("kq", T_KQ, w.Hkv, w.Lq),
                  make("vq", T_VQ, w.Hkv, w.Lq))
    qd, kd, vd = (make("qd", T_QD, w.Hq, n_dec), make("kd", T_KD, w.Hkv, n_dec),
                  make("vd", T_VD, w.Hkv, n_dec))
    st = StarAttentionStep(w.B, w.Hq, w.Hkv, w.D, w.L, w.b, w.Lq, n_dec, rope=w.rope,
                           base=w.base)
    st.load_context(v)
    st.rope_context(q, k)
    # warm-up: Phase 1 back to back for at least 0.2 s (a short kernel right
    # after the host-side work of the previous record would otherwise run
    # before the clock has ramped up), then the median of 5 launches, 2 at
    # the 1M shape
    t_w = time.perf_counter()
    while True:
        st.phase1()
        torch.cuda.synchronize()
        if time.perf_counter() - t_w >= 0.2:
            break
    e = [(ev(), ev()) for _ in range(2 if w.L >= (1 << 20) else 5)]
    for e0, e1 in e:
        e0.record()
        st.phase1()
        e1.record()
    torch.cuda.synchronize()
    p1_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in e]))
    fl = phase1_flops(w)
    rec = {"workload": name, "phase1_ms": p1_ms,
           "phase1_tflops": fl / (p1_ms * 1e-3) / 1e12,
           "phase1_frac_of_peak": fl / (p1_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "context_tokens_per_s": w.B * w.L / (p1_ms * 1e-3)}
    st.query(qq, kq, vq)
    if w.Lq > 0:
        pq = phase2_query(st, w, ev, None, reps=5)
        rec.update({"query_us": pq["us"], "query_frac_of_roofline": pq["frac_of_roofline"],
                    "query_splits": pq["splits"]})
    if n_dec:
        # one untimed pass over the same steps first (each step rewrites its
        # own cache row with the same values and sees only rows up to it, so
        # the timed pass computes the same results), then the timed pass
        for t in range(n_dec):
            st.decode(t, qd[:, :, t:t + 1], kd[:, :, t:t + 1], vd[:, :, t:t + 1])
        e0, e1 = ev(), ev()
        e0.record()
        for t in range(n_dec):
            st.decode(t, qd[:, :, t:t + 1], kd[:, :, t:t + 1], vd[:, :, t:t + 1])
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / n_dec
        byts = sum(decode_bytes(w, t) for t in range(n_dec)) / n_dec
        rec.update({"decode_us_per_step": dms * 1e3, "decode_gbps": byts / (dms * 1e-3) / 1e9,
                    "decode_frac_of_hbm_peak": byts / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                    "decode_steps_timed": n_dec})
    torch.cuda.synchronize()
    # parity on the seeded slices
    scale = 1.0 / math.sqrt(w.D)
    rng = np.random.default_rng(w.seed)
    pos = []
    for s0, e0_ in so.blocks(w.L, w.b):
        pos += [s0, s0 + 1, e0_ - 2, e0_ - 1]
        pos += (s0 + rng.choice(e0_ - s0, min(rows_per_block, e0_ - s0), replace=False)).tolist()
    pos = np.unique(np.clip(np.array(pos), 0, w.L - 1))
    rot = (lambda x, p: so.round_bf16(so.rope(x, p, w.base))) if w.rope else (lambda x, p: x)
    K = rot(host["k"][0], np.arange(w.L))
    V = host["v"][0]
    pq = w.L + np.arange(w.Lq)
    pd = w.L + w.Lq + np.arange(n_dec)
    Kc = np.concatenate([K, rot(host["kq"][0], pq), rot(host["kd"][0], pd)])
    Vc = np.concatenate([V, host["vq"][0], host["vd"][0]])
    parts = so.partitions(w.L, w.b, w.L + w.Lq + n_dec)
    Vw = np.concatenate([V, np.abs(V)], axis=-1)
    pos_t = torch.from_numpy(pos).cuda()
    err = {"phase1_max_abs": 0.0, "phase1_mean_abs": 0.0, "phase1_lse": 0.0,
           "query_max_abs": 0.0, "query_lse": 0.0, "decode_max_abs": 0.0, "decode_lse": 0.0}
    ok = True
    oracle_p2 = 0.0
    for h in range(g):
        rw, rl = so.phase1_rows(rot(host["q"][h][pos], pos), pos, K, Vw, w.b, w.a, scale)
        ro, wabs = rw[:, :w.D], rw[:, w.D:]
        go = st.o1[0, h].index_select(0, pos_t).float().cpu().numpy().astype(np.float64)
        gl = st.lse1[0, h].index_select(0, pos_t).cpu().numpy().astype(np.float64)
        d = np.abs(go - ro)
        ok &= bool((d <= np.maximum(1e-2, 2.0 ** -8 * np.abs(ro) + 2.0 ** -9 * wabs + 1e-4)).all())
        err["phase1_max_abs"] = max(err["phase1_max_abs"], float(d.max()))
        err["phase1_mean_abs"] = max(err["phase1_mean_abs"], float(d.mean()))
        err["phase1_lse"] = max(err["phase1_lse"], float(np.abs(gl - rl).max()))
        rows = np.concatenate([rot(host["qq"][h], pq), rot(host["qd"][h], pd)])
        t_p2 = time.perf_counter()
        o, l, _, _ = so.phase2(rows, np.concatenate([pq, pd]), Kc, Vc, parts, scale)
        oracle_p2 += time.perf_counter() - t_p2
        if w.Lq:
            err["query_max_abs"] = max(err["query_max_abs"], float(np.abs(
                st.o2[0, h].cpu().numpy() - o[:w.Lq]).max()))
            err["query_lse"] = max(err["query_lse"], float(np.abs(
                st.lse2[0, h].cpu().numpy() - l[:w.Lq]).max()))
        if n_dec:
            err["decode_max_abs"] = max(err["decode_max_abs"], float(np.abs(
                st.od[0, h, :n_dec].cpu().numpy() - o[w.Lq:]).max()))
            err["decode_lse"] = max(err["decode_lse"], float(np.abs(
                st.lsed[:n_dec, 0, h].cpu().numpy() - l[w.Lq:]).max()))
    ok &= (err["phase1_mean_abs"] <= 1e-3 and err["phase1_lse"] <= 1e-3
           and err["query_max_abs"] <= 1e-2 and err["query_lse"] <= 1e-3
           and err["decode_max_abs"] <= 1e-2 and err["decode_lse"] <= 1e-3)
    rec["parity"] = {**err, "within_tolerance": bool(ok), "heads_checked": g,
                     "phase1_rows_per_head": int(pos.size), "query_rows": w.Lq,
                     "decode_steps": n_dec,
                     "checked": "batch 0, KV head 0 and its query heads, vs the fp64 oracle"}
    # (the whole oracle's Phase 1 is timed by --cpu-full: a few sampled rows
    # per call carry fixed costs that do not scale with the rows)
    rec["oracle_cores"] = _blas_threads()
    if w.Lq + n_dec:
        # the oracle's merged Phase-2 attention per token, every head
        rec["oracle_phase2_ms_per_token"] = (oracle_p2 / (g * (w.Lq + n_dec)) * w.B * w.Hq * 1e3)
    if n_dec:
        # after the parity check: the replays overwrite the decode rows
        gr = decode_graph(st, w, ev, n_dec)
        rec.update({"decode_graph_us_per_step": gr["us_per_step"],
                    "decode_graph_frac_of_hbm_peak": gr["frac_of_hbm_peak"],
                    "decode_one_step_graph_us_per_step": gr["one_step_graph_us_per_step"]})
    del st, q, k, v, qq, kq, vq, qd, kd, vd
    torch.cuda.empty_cache()
    return rec


def hbm_stream(ev, mib=1024, reps=5):
    """Achievable streaming-read rate on this GPU: the library's plain
    streaming read (16-byte nontemporal loads, every byte once) over 1 GiB, four times
    the 256 MiB Infinity Cache, so every pass reads HBM; best of three grid
    sizes.  Reported beside the decode rate as the practical ceiling of an
    HBM-bound kernel."""
    import torch

    import block_sparse_amd as sa

    buf = torch.ones(mib << 18, dtype=torch.int32, device="cuda")
    best = None
    for wg in (2048, 4096, 8192):
        out = torch.empty(wg, dtype=torch.int32, device="cuda")
        sa.stream_read(buf, wg, out)
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            sa.stream_read(buf, wg, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        if best is None or ms < best[0]:
            best = (ms, wg)
    gbps = (mib << 20) / (best[0] * 1e-3) / 1e9
    del buf
    return {"gbps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBS, "bytes": mib << 20,
            "workgroups": best[1],
            "note": "star_stream_read over 1 GiB (a plain streaming read, 16-byte nontemporal loads)"}


FULL_ORACLE = ("tiny", "llama8b-16k", "llama8b-128k", "llama70b-64k", "llama8b-1m")


def oracle_flops(w, blocks=None) -> float:
    """fp64 FLOPs the oracle executes for Phase 1 (its explicit masks make
    every block a full rectangle: n_i rows x (n_i or a + n_i) keys, QK^T and
    PV) and for Phase 2 (every query and decode row over its cache), all
    heads.  ``blocks``: count only the first ``blocks`` blocks' Phase 1."""
    per_head = 0
    for i, s0 in enumerate(range(0, w.L, w.b)):
        if blocks is not None and i >= blocks:
            break
        n = min(s0 + w.b, w.L) - s0
        per_head += 4 * w.D * n * (n + (w.a if i > 0 else 0))
    if blocks is None:
        per_head += 4 * w.D * (w.Lq * (w.L + w.Lq) + sum(w.L + w.Lq + t + 1 for t in range(w.T)))
    return float(per_head * w.Hq * w.B)


def cpu_full_oracle(names=FULL_ORACLE):
    """Whole-oracle CPU timings (the oracle as it stands, fp64 numpy, on the
    host's BLAS threads); only the oracle calls are timed, not the input
    draws.
      tiny, llama8b-16k: one call over the whole workload.
      llama8b-128k, llama70b-64k: one (batch, KV head) group at a time, so
        that memory stays bounded and progress shows: the oracle's heads are
        independent and each group's inputs are the workload's own slices,
        so the groups together are the whole workload (RoPE, Phase 1, the
        query, every decode step).
      llama8b-1m: Phase 1 only, extrapolated: blocks 1 and 2 of every head
        are timed, and each later block costs what block 2 does (the anchor
        plus a causal block of the same size)."""
    import dataclasses

    import numpy as np

    import oracle.star_oracle as so
    from workloads import WORKLOADS, as_f64, draw_rows, f32_to_bf16_bits, group_inputs, inputs
    from workloads import T_K, T_Q, T_V
    out = {}
    for name in names:
        w = WORKLOADS[name]
        if name == "llama8b-1m":
            scale = 1.0 / math.sqrt(w.D)
            rows = 2 * w.b
            f64 = lambda tid, b, h: as_f64(f32_to_bf16_bits(
                draw_rows(w.seed, tid, b, h, w.L, w.D, w.scale, 0, rows)))
            t_blocks = [0.0, 0.0]
            for b in range(w.B):
                for kvh in range(w.Hkv):
                    k, v = f64(T_K, b, kvh), f64(T_V, b, kvh)
                    qs = [f64(T_Q, b, h) for h in range(kvh * w.g, (kvh + 1) * w.g)]
                    for blk in (0, 1):
                        t0 = time.perf_counter()
                        pos_k = np.arange(rows)
                        K = so.round_bf16(so.rope(k, pos_k, w.base))
                        for q in qs:
                            for r0 in range(blk * w.b, (blk + 1) * w.b, 4096):
                                pos = np.arange(r0, r0 + 4096)
                                qr = so.round_bf16(so.rope(q[pos], pos, w.base))
                                so.phase1_rows(qr, pos, K, v, w.b, w.a, scale)
                        t_blocks[blk] += time.perf_counter() - t0
                    progress(f"oracle {name}: blocks 1-2 of group b{b} kv{kvh} done")
            total = t_blocks[0] + (w.n_blocks - 1) * t_blocks[1]
            out[name] = {"seconds": total, "context_tokens_per_s": w.B * w.L / total,
                         "fp64_gflops": oracle_flops(w, 2) / sum(t_blocks) / 1e9,
                         "note": f"Phase 1 only, extrapolated: blocks 1 and 2 of every head took "
                                 f"{t_blocks[0]:.1f} s and {t_blocks[1]:.1f} s; "
                                 f"{w.n_blocks - 2} more blocks at block 2's cost"}
            continue
        dt, groups = 0.0, 0
        if w.B * w.Hkv == 1 or name in ("tiny", "llama8b-16k"):
            x = {n: as_f64(t) for n, t in inputs(w, as_bf16=True).items()}
            t0 = time.perf_counter()
            so.star_attention(w, x)
            dt, groups = time.perf_counter() - t0, 1
        else:
            wg = dataclasses.replace(w, B=1, Hq=w.g, Hkv=1)
            for b in range(w.B):
                for kvh in range(w.Hkv):
                    x = {n: as_f64(t) for n, t in group_inputs(w, b, kvh).items()}
                    t0 = time.perf_counter()
                    so.star_attention(wg, x)
                    dt += time.perf_counter() - t0
                    groups += 1
                    progress(f"oracle {name}: group b{b} kv{kvh} done ({dt:.0f} s so far)")
        progress(f"oracle {name}: {dt:.1f} s")
        out[name] = {"seconds": dt, "context_tokens_per_s": w.B * w.L / dt, "groups": groups,
                     "fp64_gflops": oracle_flops(w) / dt / 1e9,
                     "note": "fp64 numpy oracle, whole workload incl. RoPE, Phase 1, query "
                             "and every decode step"}
    return out


def _short_kernel_name(name: str) -> str:
    """Kernel name without namespace noise and argument list.  rocprofv3
    leaves some names with a __bf16 template argument mangled (``_ZN4star
    12_GLOBAL__N_111rope_kernelIDF16bEE...``): their nested name and simple
    template arguments are decoded here."""
    if name.startswith("_ZN"):
        parts, i = [], 3
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            n = int(name[i:j])
            parts.append(name[j:j + n])
            i = j + n
        targs = ""
        if name[i:i + 1] == "I":
            # template arguments: types (f, d, i, DF16b) and literals
            # (L <type> <value> E: Li8E, Lb1E), up to the list's closing E
            args, i = [], i + 1
            types = {"DF16b": "__bf16", "f": "float", "d": "double", "i": "int", "b": "bool"}
            while i < len(name) and name[i] != "E":
                if name[i] == "L":
                    j = name.index("E", i)
                    lit = name[i + 1:j]
                    t = "b" if lit[:1] == "b" else lit[:1]
                    v = lit[1:]
                    args.append({"0": "false", "1": "true"}[v] if t == "b" else v.replace("n", "-"))
                    i = j + 1
                    continue
                code = next((c for c in types if name.startswith(c, i)), None)
                if code is None:
                    break
                args.append(types[code])
                i += len(code)
            targs = "<" + ", ".join(args) + ">" if args else ""
        return "::".join(x for x in parts if not x.startswith("_GLOBAL__N")) + targs
    short = name.replace("(anonymous namespace)::", "")
    if short.endswith(")"):                       # drop the argument list
        depth = 0
        for i in range(len(short) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(short[i], 0)
            if depth == 0:
                short = short[:i]
                break
    return re.sub(r"^void ", "", short)


def _trace_sequences(files) -> list:
    """Launch-order figures of a step trace: each decode partials launch
    with the merge launch that follows it, split into the cold samples (the
    launch right before the decode launch is the cache-flushing reduction)
    and the others (step passes and graph replays), each with its median
    decode, merge and decode-start-to-merge-end times and the gap between
    the two launches; and the Phase-2 query partials (flash kernel launches
    below its largest grid) in launch order."""
    import csv
    import statistics
    ev = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                try:
                    grid = int(r.get("Grid_Size_X", 0))
                    wg = int(r.get("Workgroup_Size_X", 1))
                    ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                               _short_kernel_name(r.get("Kernel_Name", "?")), grid // max(wg, 1)))
                except (KeyError, ValueError):
                    continue
    ev.sort()
    out = []
    pairs = {"cold": [], "other": []}
    for i, (s0, e0, n, _) in enumerate(ev):
        if not n.startswith("star::decode_kernel") or i + 1 >= len(ev):
            continue
        s1, e1, n1, _ = ev[i + 1]
        if not n1.startswith("star::merge_kernel"):
            continue
        cold = i > 0 and ev[i - 1][2].startswith("at::native::reduce_kernel")
        pairs["cold" if cold else "other"].append(((e0 - s0) / 1e3, (e1 - s1) / 1e3,
                                                   (e1 - s0) / 1e3, (s1 - e0) / 1e3))
    for k, label in (("cold", "decode steps right after the cache-flushing read"),
                     ("other", "other decode steps (step passes, graph replays)")):
        v = pairs[k]
        if v:
            med = [statistics.median(x[j] for x in v) for j in range(4)]
            out.append(f"{label}: {len(v)} launches; median decode {med[0]:.2f} us, merge "
                       f"{med[1]:.2f} us, decode start to merge end {med[2]:.2f} us, gap "
                       f"between the launches {med[3]:.2f} us")
    fl = [(s0, e0, g) for s0, e0, n, g in ev if n.startswith("star::flash2_kernel")]
    if fl:
        big = max(g for _, _, g in fl)
        q = [(e0 - s0) / 1e3 for s0, e0, g in fl if g < big]
        if q:
            out.append("Phase-2 query partials (flash kernel below its largest grid), first "
                       f"{min(len(q), 8)} in launch order: " + ", ".join(f"{x:.1f}" for x in q[:8])
                       + " us")
    return ([""] + out) if out else []


def trace_summary(root: str) -> str:
    """Per-kernel count, mean, median and min duration (us) from the
    kernel_trace.csv files a ``rocprofv3 --kernel-trace --output-format csv``
    run wrote under ``root``, one line per (kernel, workgroup count)."""
    import csv
    import glob
    import statistics
    files = glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return f"no *kernel_trace.csv under {root}"
    agg = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name", "?")
                try:
                    grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)))
                    wg = int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", 1)))
                    d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                except (KeyError, ValueError):
                    continue
                short = _short_kernel_name(name)
                agg.setdefault((short[:60], grid // max(wg, 1)), []).append(d)
    tot = sum(sum(v) for v in agg.values())
    lines = [f"{'kernel':60s} {'workgroups':>10s} {'calls':>6s} {'mean_us':>10s} "
             f"{'median_us':>10s} {'min_us':>10s} {'share':>6s}"]
    for (n, wg), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{n:60s} {wg:10d} {len(v):6d} {statistics.mean(v):10.2f} "
                     f"{statistics.median(v):10.2f} {min(v):10.2f} {100 * sum(v) / tot:5.1f}%")
    lines += _trace_sequences(files)
    stats = glob.glob(os.path.join(root, "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        lines += ["", "rocprofv3 --stats (one line per kernel name: every grid size together)",
                  f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
        for f in stats:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    try:
                        lines.append(f"{_short_kernel_name(r['Name'])[:60]:60s} {int(r['Calls']):6d} "
                                     f"{float(r['AverageNs']) / 1e3:10.2f} "
                                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}")
                    except (KeyError, ValueError):
                        continue
    return "\n".join(lines)


def counter_summary(roots, calib_mib: int = 1024) -> str:
    """Per-dispatch means of the counters in the counter_collection.csv
    files that ``rocprofv3 --pmc ... --output-format csv`` runs wrote under
    ``roots`` (one run per counter set), one line per (kernel, workgroup
    count, counter); then, from the same numbers:
      * byte counters scaled by the plain device copy of ``calib_mib`` MiB
        the ``--copy-calib`` run issues first (__amd_rocclr_copyBuffer: its
        bytes read and written are known), and the Phase-1 launch's
        ``traffic_bytes_per_launch`` with the flash kernel's source hash (the
        lines the benchmark's ``roofline.traffic`` reads);
      * SQ ratios of the Phase-1 flash launch (the flash kernel's largest
        grid) when its SQ counters are there."""
    import csv
    import glob
    import statistics
    agg = {}
    dur = {}
    for root in roots:
        files = glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    try:
                        grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)))
                        wg = int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", 1)))
                        val = float(r["Counter_Value"])
                        cname = r["Counter_Name"]
                    except (KeyError, ValueError):
                        continue
                    key = (_short_kernel_name(r.get("Kernel_Name", "?"))[:60], grid // max(wg, 1))
                    agg.setdefault(key, {}).setdefault(cname, []).append(val)
                    try:
                        dur[(key, r["Dispatch_Id"], root)] = (
                            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                    except (KeyError, ValueError):
                        pass
    if not agg:
        return f"no *counter_collection.csv under {roots}"
    lines = [f"{'kernel':60s} {'workgroups':>10s} {'counter':28s} {'dispatches':>10s} "
             f"{'mean':>14s} {'min':>14s} {'max':>14s}"]
    for (n, wg), cs in sorted(agg.items()):
        for c, v in sorted(cs.items()):
            lines.append(f"{n:60s} {wg:10d} {c:28s} {len(v):10d} {statistics.mean(v):14.6g} "
                         f"{min(v):14.6g} {max(v):14.6g}")
    mean = {k: {c: statistics.mean(v) for c, v in cs.items()} for k, cs in agg.items()}
    # the calibration copy: the largest copyBuffer dispatch (a step also
    # issues small host-to-device copies through the same kernel)
    copy = max((cs for (n, _), cs in mean.items() if n.startswith("__amd_rocclr_copyBuffer")
                and cs.get("FETCH_SIZE", cs.get("WRITE_SIZE", 0)) > 0),
               key=lambda cs: cs.get("FETCH_SIZE", 0) + cs.get("WRITE_SIZE", 0), default=None)
    flash = [k for k in mean if k[0].startswith("star::flash2_kernel")]
    p1 = max(flash, key=lambda k: k[1]) if flash else None
    nbytes = calib_mib * (1 << 20)
    if copy is not None:
        lines += ["", f"calibration copy: {calib_mib} MiB read and written"]
        scale = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in copy:
                scale[c] = nbytes / (copy[c] * 1024.0)
                lines.append(f"  {c} {copy[c]:.0f} KiB -> scale {scale[c]:.4f}")
        lines.append("scaled bytes per dispatch (counter KiB x 1024 x scale):")
        for (n, wg), cs in sorted(mean.items()):
            parts = [f"{c} {cs[c] * 1024 * scale[c] / 1e9:.4f} GB" for c in scale if c in cs]
            if parts:
                lines.append(f"  {n:60s} {wg:10d}  " + ", ".join(parts))
        if p1 is not None and all(c in mean[p1] for c in ("FETCH_SIZE", "WRITE_SIZE")) \
                and len(scale) == 2:
            tr = sum(mean[p1][c] * 1024 * scale[c] for c in scale)
            src = hashlib.sha256(open(FLASH_SRC, "rb").read()).hexdigest()
            lines += [f"Phase-1 launch ({p1[0]}, {p1[1]} workgroups): "
                      f"read {mean[p1]['FETCH_SIZE'] * 1024 * scale['FETCH_SIZE'] / 1e9:.3f} GB, "
                      f"written {mean[p1]['WRITE_SIZE'] * 1024 * scale['WRITE_SIZE'] / 1e9:.3f} GB",
                      f"traffic_bytes_per_launch: {tr:.6e}",
                      f"flash_src_sha256: {src}"]
    if p1 is not None:
        c = mean[p1]
        need = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA")
        if all(x in c for x in need):
            kc = c["GRBM_GUI_ACTIVE"] / 8.0
            d = [("kernel cycles per XCD (GRBM_GUI_ACTIVE / 8)", kc)]
            ns = [v for (k, _, _), v in dur.items() if k == p1]
            if ns:
                d += [("launch duration in the counter runs (ms)", statistics.mean(ns) / 1e6),
                      ("clock (those cycles / that duration, GHz)",
                       kc / statistics.mean(ns))]
            d += [
                 ("MFMA busy / SIMD cycles (1024 SIMDs)",
                  c["SQ_VALU_MFMA_BUSY_CYCLES"] / (kc * 1024)),
                 ("MFMA busy cycles / MFMA instruction",
                  c["SQ_VALU_MFMA_BUSY_CYCLES"] / c["SQ_INSTS_MFMA"])]
            for label, num in (("VALU instructions / MFMA (incl. MFMA)", "SQ_INSTS_VALU"),
                               ("exp2 (trans) / MFMA", "SQ_INSTS_VALU_TRANS_F32"),
                               ("LDS instructions / MFMA", "SQ_INSTS_LDS"),
                               ("SALU instructions / MFMA", "SQ_INSTS_SALU")):
                if num in c:
                    d.append((label, c[num] / c["SQ_INSTS_MFMA"]))
            if all(x in c for x in ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY")):
                wc = c["SQ_WAVE_CYCLES"]
                d += [("wave cycles waiting (SQ_WAIT_ANY)", c["SQ_WAIT_ANY"] / wc),
                      ("wave cycles ready, not issued",
                       (wc - c["SQ_WAIT_ANY"] - c["SQ_ACTIVE_INST_ANY"]) / wc),
                      ("wave cycles issuing", c["SQ_ACTIVE_INST_ANY"] / wc)]
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
                d.append(("MFMA/VALU co-execution / MFMA busy",
                          c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"]))
            lines += ["", f"derived, Phase-1 launch ({p1[0]}, {p1[1]} workgroups):"]
            lines += [f"  {label:42s} {v:.4g}" for label, v in d]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b-128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache decode timing")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the attention-layer timing (projections + Phase 1)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the Phase-1 prefix variants (Pulsar, anchor positions)")
    ap.add_argument("--splits-decode", type=int, default=None,
                    help="chunks per KV partition for the decode partials")
    ap.add_argument("--splits-query", type=int, default=None,
                    help="chunks per KV partition for the query partials")
    ap.add_argument("--phase1-only", action="store_true",
                    help="time only RoPE + Phase 1 (for counter runs)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of this many MiB first "
                         "(reference kernel for rocprofv3 byte counters)")
    ap.add_argument("--no-separate-rope", action="store_true",
                    help="skip timing Phase 1 with Q rotated inside the kernel beside the "
                         "step's form (keeps a kernel trace to the step's launches)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload records (timing + sampled parity)")
    ap.add_argument("--configs", default=None,
                    help="comma-separated workloads for the per-workload records "
                         "(default: all five)")
    ap.add_argument("--cpu-full", nargs="?", const=",".join(FULL_ORACLE), default=None,
                    metavar="NAMES",
                    help="also time the whole oracle on these workloads (default: tiny, "
                         "8B-16K, 8B-128K and 70B-64K whole, 8B-1M Phase 1 extrapolated "
                         "from two blocks; ~10 minutes each for the large ones on 16 host "
                         "threads)")
    ap.add_argument("--cpu-full-only", action="store_true",
                    help="with --cpu-full: time the oracle only (no GPU work) and print "
                         "one JSON line")
    ap.add_argument("--counter-summary", nargs="+", default=None, metavar="DIR",
                    help="print per-kernel counter means from the rocprofv3 --pmc csv runs "
                         "under the DIRs (with byte scaling by the --copy-calib copy and the "
                         "Phase-1 launch's ratios), then exit (no GPU)")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="print the per-kernel summary of a rocprofv3 --output-format csv "
                         "kernel trace found under DIR, then exit (no GPU)")
    args = ap.parse_args()
    if args.counter_summary:
        print(counter_summary(args.counter_summary, args.copy_calib or 1024))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.cpu_full_only:
        if not args.cpu_full:
            ap.error("--cpu-full-only needs --cpu-full")
        print(json.dumps({"cpu_full_oracle": cpu_full_oracle(args.cpu_full.split(",")),
                          "cores": _blas_threads(),
                          "affinity_cores": len(os.sched_getaffinity(0))}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_amd.pipeline import StarAttentionStep
    from workloads import WORKLOADS, inputs

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    x = inputs(w, as_bf16=True)
    dev = {n: torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).cuda() for n, t in x.items()}
    st = StarAttentionStep(w.B, w.Hq, w.Hkv, w.D, w.L, w.b, w.Lq, w.T, rope=w.rope, base=w.base,
                           splits_query=args.splits_query, splits_decode=args.splits_decode)
    st.load_context(dev["v"])
    if args.copy_calib:
        n = args.copy_calib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(rec=None):
        if rec is not None:
            rec["p1"][0].record()
        st.rope_context(dev["q"], dev["k"])
        if rec is not None:
            rec["p1"][1].record()
        st.phase1()
        if rec is not None:
            rec["p1"][2].record()
        if args.phase1_only:
            return
        st.query(dev["qq"], dev["kq"], dev["vq"], events=None if rec is None else rec["q"])
        if rec is not None:
            rec["dec"][0].record()
        for t in range(w.T):
            st.decode(t, dev["qd"][:, :, t:t + 1], dev["kd"][:, :, t:t + 1],
                      dev["vd"][:, :, t:t + 1])
        if rec is not None:
            rec["dec"][1].record()

    progress(f"{w.name}: inputs resident")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    progress("warm-up done")
    recs = [{"p1": [ev(), ev(), ev()], "q": [ev(), ev()], "dec": [ev(), ev()]}
            for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in recs:
        step(r)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    ms_step = total * 1e3 / args.steps
    progress(f"timed steps done: {ms_step:.2f} ms per step")

    rope_ms = np.mean([r["p1"][0].elapsed_time(r["p1"][1]) for r in recs])
    p1_samples = [r["p1"][1].elapsed_time(r["p1"][2]) for r in recs]
    p1_ms = np.mean(p1_samples)
    flops = phase1_flops(w)
    p1_tflops = flops / (p1_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": w.B * w.L * args.steps / total,
        "unit": "context tokens/s (whole two-phase step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "context": w.L, "block": w.b, "anchor": w.a,
                   "query_tokens": w.Lq, "decode_steps": w.T, "rope_base": w.base,
                   "splits_query": st.sq, "splits_decode": st.sd,
                   "phase1_only": bool(args.phase1_only)},
        "phase1": {"kernel_ms": p1_ms, "kernel_median_ms": float(np.median(p1_samples)),
                   "kernel_min_ms": float(np.min(p1_samples)), "rope_ms": rope_ms,
                   "context_tokens_per_s": w.B * w.L / (p1_ms * 1e-3),
                   "context_tokens_per_s_with_rope": w.B * w.L / ((p1_ms + rope_ms) * 1e-3),
                   "tflops": p1_tflops, "algorithmic_flops": flops,
                   "pages_host_flops": 4 * w.D * w.Hq * w.B * pages_host_pairs(w.L, w.b, w.a),
                   "note": "algorithmic_flops counts useful (query, key) pairs; "
                           "pages_host_flops is the pages' per-host count (every host also "
                           "recomputes its anchor rows), for information"},
        "roofline": {"bound": "mfma", "achieved": p1_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": p1_tflops / PEAK_BF16_TFLOPS,
                     "traffic": pmc_traffic(),
                     "kernel": "flash2_kernel<8, 2> (Phase 1)"},
    }
    if w.rope and w.D == 128 and not args.phase1_only and not args.no_separate_rope:
        out["phase1"]["separate_rope"] = phase1_separate_rope(st, dev, w, ev)
        progress("Phase 1 with and without the rotation of Q inside the kernel done")
    if not args.phase1_only and w.T > 0:
        dec_ms = np.mean([r["dec"][0].elapsed_time(r["dec"][1]) for r in recs])
        byts = sum(decode_bytes(w, t) for t in range(w.T))
        out["decode"] = {"us_per_step": dec_ms * 1e3 / w.T,
                         "gbps": byts / (dec_ms * 1e-3) / 1e9,
                         "frac_of_hbm_peak": byts / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "note": "whole decode step (RoPE, KV append, partials, merge), "
                                 "K+V bytes of every visible token"}
    if not args.phase1_only and w.Lq > 0:
        out["phase2_query"] = phase2_query(
            st, w, ev, [r["q"][0].elapsed_time(r["q"][1]) for r in recs])
    if not args.phase1_only and w.T > 0 and not args.no_cold:
        out["decode_cold"] = decode_cold(st, dev, w, ev)
        progress("cold decode done")
    if not args.phase1_only and w.T > 0:
        out["decode_graph"] = decode_graph(st, w, ev, w.T)
        progress("graph decode done")
    if not args.phase1_only and w.T > 0:
        out["hbm_stream"] = hbm_stream(ev)
    if w.rope and not args.no_variants:
        out["phase1_variants"] = phase1_variants(st, dev, w, x, ev)
        progress("Phase-1 variants done")
    if not args.no_layer:
        out["phase1_layer"] = phase1_layer(w, ev)
        progress("attention layer done")
    del st, dev
    torch.cuda.empty_cache()
    if not args.no_configs:
        names = args.configs.split(",") if args.configs else list(WORKLOADS)
        out["per_config"] = []
        for n in names:
            out["per_config"].append(config_record(n, ev))
            progress(f"per-workload record {n} done")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
        progress("cpu baseline done")
        if args.cpu_full:
            full = cpu_full_oracle(args.cpu_full.split(","))
            ref = full.get(w.name)
            if ref is not None and "extrapolated" not in ref["note"]:
                ref["oracle_over_gpu_step"] = ref["seconds"] / (ms_step * 1e-3)
            out["cpu_full_oracle"] = full
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
