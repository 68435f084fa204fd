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
``cpu_baseline`` is the fp64 CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
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
            "cores": int(cores), "kind": "oracle",
            "sample": (f"fp64 numpy oracle, Phase 1 of all {e - s} rows of block {blk + 1} "
                       f"(positions {s}-{e - 1}) for {heads} query heads of KV head 0, incl. "
                       f"RoPE; {dt:.1f} s; scaled by useful (q,k) pairs {sample_pairs:.3e} of "
                       f"{total_pairs:.3e}")}


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
    """Decode steps timed one at a time, each after a 1 GiB device read that
    evicts the L2 caches and the 256 MiB Infinity Cache, so every K/V byte
    comes from HBM.  The flush reads rather than writes: a written flush
    leaves dirty lines whose write-back then competes with the timed reads
    (it halves a plain streaming read's rate on this chip).  Re-runs decode
    steps spread over 0..T-1 after the timed pass (the cache rows they
    append hold the same values)."""
    import numpy as np
    import torch

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    ts = sorted(set(np.linspace(0, w.T - 1, min(samples, w.T)).astype(int).tolist()))
    recs = []
    for i, t in enumerate(ts):
        torch.sum(flush, dim=0, out=sink)
        e0, e1 = ev(), ev()
        e0.record()
        st.decode(t, dev["qd"][:, :, t:t + 1], dev["kd"][:, :, t:t + 1],
                  dev["vd"][:, :, t:t + 1])
        e1.record()
        recs.append((t, e0, e1))
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for _, e0, e1 in recs]
    byts = [decode_bytes(w, t) for t, _, _ in recs]
    us = float(np.mean(ms)) * 1e3
    gbps = float(np.sum(byts) / (np.sum(ms) * 1e-3) / 1e9)
    del flush
    return {"us_per_step": us, "gbps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBS,
            "steps_sampled": len(ts),
            "note": "each step after a 1 GiB read that flushes L2 and Infinity Cache"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
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
    args = ap.parse_args()
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
        st.query(dev["qq"], dev["kq"], dev["vq"])
        if rec is not None:
            rec["dec"][0].record()
        for t in range(w.T):
            st.decode(t, dev["qd"][:, :, t:t + 1], dev["kd"][:, :, t:t + 1],
                      dev["vd"][:, :, t:t + 1])
        if rec is not None:
            rec["dec"][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = [{"p1": [ev(), ev(), ev()], "dec": [ev(), ev()]} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in recs:
        step(r)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    ms_step = total * 1e3 / args.steps

    rope_ms = np.mean([r["p1"][0].elapsed_time(r["p1"][1]) for r in recs])
    p1_ms = np.mean([r["p1"][1].elapsed_time(r["p1"][2]) for r in recs])
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
        "phase1": {"kernel_ms": p1_ms, "rope_ms": rope_ms,
                   "context_tokens_per_s": w.B * w.L / (p1_ms * 1e-3),
                   "context_tokens_per_s_with_rope": w.B * w.L / ((p1_ms + rope_ms) * 1e-3),
                   "tflops": p1_tflops, "algorithmic_flops": flops},
        "roofline": {"bound": "mfma", "achieved": p1_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": p1_tflops / PEAK_BF16_TFLOPS,
                     "traffic": pmc_traffic(),
                     "kernel": "flash2_kernel (Phase 1)"},
    }
    if not args.phase1_only and w.T > 0:
        dec_ms = np.mean([r["dec"][0].elapsed_time(r["dec"][1]) for r in recs])
        byts = sum(decode_bytes(w, t) for t in range(w.T))
        out["decode"] = {"us_per_step": dec_ms * 1e3 / w.T,
                         "gbps": byts / (dec_ms * 1e-3) / 1e9,
                         "frac_of_hbm_peak": byts / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "note": "whole decode step (RoPE, KV append, partials, merge), "
                                 "K+V bytes of every visible token"}
    if not args.phase1_only and w.T > 0 and not args.no_cold:
        out["decode_cold"] = decode_cold(st, dev, w, ev)
    if not args.phase1_only and w.T > 0:
        out["hbm_stream"] = hbm_stream(ev)
    if w.rope and not args.no_variants:
        out["phase1_variants"] = phase1_variants(st, dev, w, x, ev)
    if not args.no_layer:
        out["phase1_layer"] = phase1_layer(w, ev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
