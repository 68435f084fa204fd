"""Host-side checks of bench.py (no GPU): the one-GPU guard, and the
algorithmic work it divides by (useful Phase-1 pairs, decode bytes), pinned
by brute-force counting over (query, key) positions and by the sizes the
workload table states (8B-128K: 4.838e13 FLOP per Phase-1 launch, 537.7 MB
per decode step)."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("L,b,a", [(700, 200, 200), (512, 128, 0), (333, 1000, 1000),
                                   (97, 32, 16), (1, 16, 16)])
def test_phase1_pairs_brute_force(L, b, a):
    """Query q (block i = q // b) sees key k when k is in its own block and
    k <= q, or when i >= 1 and k < a (the anchor)."""
    bench = load_bench()
    q = np.arange(L)[:, None]
    k = np.arange(L)[None, :]
    own = (k // b == q // b) & (k <= q)
    anchor = (q // b >= 1) & (k < a)
    assert bench.phase1_pairs(L, b, a) == int((own | anchor).sum())


def test_workload_work_figures():
    bench = load_bench()
    from workloads import WORKLOADS
    w = WORKLOADS["llama8b-128k"]
    assert bench.phase1_flops(w) == pytest.approx(4.838e13, rel=1e-3)
    assert bench.decode_bytes(w, w.T - 1) == pytest.approx(537.7e6, rel=1e-3)
    w = WORKLOADS["llama8b-1m"]
    assert bench.phase1_flops(w) == pytest.approx(8.268e14, rel=1e-3)
    assert bench.decode_bytes(w, w.T - 1) == pytest.approx(4.295e9, rel=1e-3)


def test_traffic_only_for_the_profiled_kernel(tmp_path, monkeypatch):
    """The HBM traffic figure is reported only while the kernel source is the
    one the counter summary was taken from."""
    bench = load_bench()
    t = bench.pmc_traffic()
    assert t is None or t > 0
    other = tmp_path / "flash2.hip"
    other.write_text("// another kernel\n")
    monkeypatch.setattr(bench, "FLASH_SRC", str(other))
    assert bench.pmc_traffic() is None


def test_query_work_figures():
    """Query row r at position L + r sees every key up to itself (L + r + 1
    keys); K and V are each read once per KV head."""
    bench = load_bench()
    from workloads import WORKLOADS
    w = WORKLOADS["llama8b-128k"]
    pairs = sum(len(range(0, w.L + r + 1)) for r in range(w.Lq))
    assert bench.query_flops(w) == 4.0 * w.D * w.Hq * w.B * pairs
    assert bench.query_flops(w) == pytest.approx(1.3747e11, rel=1e-3)
    assert bench.query_bytes(w) == (w.L + w.Lq) * w.Hkv * w.D * 4


def test_trace_summary_reads_rocprof_csv(tmp_path):
    """The per-kernel summary of a rocprofv3 csv kernel trace: count, mean,
    median and min per (kernel, workgroup count)."""
    bench = load_bench()
    hdr = ("Kind,Agent_Id,Queue_Id,Stream_Id,Thread_Id,Dispatch_Id,Kernel_Id,Kernel_Name,"
           "Correlation_Id,Start_Timestamp,End_Timestamp,Private_Segment_Size,"
           "Group_Segment_Size,Workgroup_Size_X,Workgroup_Size_Y,Workgroup_Size_Z,"
           "Grid_Size_X,Grid_Size_Y,Grid_Size_Z\n")
    rows = []
    for i, d in enumerate((10_000, 30_000, 20_000)):
        rows.append(f'KERNEL_DISPATCH,1,1,1,1,{i},1,"star::(anonymous namespace)::k(star::P)",'
                    f'{i},{1000 * i},{1000 * i + d},0,0,512,1,1,{512 * 256},1,1\n')
    (tmp_path / "run_kernel_trace.csv").write_text(hdr + "".join(rows))
    out = bench.trace_summary(str(tmp_path)).splitlines()
    assert out[1].split()[:6] == ["star::k", "256", "3", "20.00", "20.00", "10.00"]


def test_short_kernel_names():
    """Namespace noise and argument lists go; names rocprofv3 leaves mangled
    (a __bf16 template argument) are decoded."""
    bench = load_bench()
    f = bench._short_kernel_name
    assert f("_ZN4star12_GLOBAL__N_111rope_kernelIDF16bEEvNS_10RopeParamsEi") == \
        "star::rope_kernel<__bf16>"
    assert f("_ZN4star12_GLOBAL__N_111rope_kernelIfEEvNS_10RopeParamsEi") == \
        "star::rope_kernel<float>"
    assert f("star::(anonymous namespace)::stream_read_kernel(unsigned int __vector(4) const*, "
             "long, unsigned int*)") == "star::stream_read_kernel"
    assert f("void star::(anonymous namespace)::merge_kernel<128>(star::MergeParams)") == \
        "star::merge_kernel<128>"
    assert f("_ZN4star12_GLOBAL__N_113flash2_kernelILi4ELi1EEEvNS_11FlashParamsE") == \
        "star::flash2_kernel<4, 1>"
    assert f("_ZN4star12_GLOBAL__N_113decode_kernelILi128EDF16bLb1EEEvNS_12DecodeParamsE") == \
        "star::decode_kernel<128, __bf16, true>"
    assert f("void star::(anonymous namespace)::flash2_kernel<8, 2>(star::FlashParams)") == \
        "star::flash2_kernel<8, 2>"


def test_pages_host_flops():
    """The pages' per-host count (causal over the 2b-token augmented block,
    anchor rows included): 6.38e13 FLOP at 8B-128K, and a brute-force count
    on a small ragged case."""
    bench = load_bench()
    from workloads import WORKLOADS
    w = WORKLOADS["llama8b-128k"]
    assert 4 * w.D * w.Hq * w.B * bench.pages_host_pairs(w.L, w.b, w.a) == pytest.approx(6.38e13, rel=1e-3)
    L, b, a = 23, 7, 7
    brute = 0
    for s in range(0, L, b):
        n = min(s + b, L) - s
        m = n + (a if s > 0 else 0)
        brute += sum(r + 1 for r in range(m))
    assert bench.pages_host_pairs(L, b, a) == brute


def test_oracle_flops_follow_the_oracles_key_sets():
    """The oracle's executed Phase-1 FLOPs: every block is a full rectangle
    of its rows by the key set the oracle builds for it."""
    import dataclasses
    import oracle.star_oracle as so
    from workloads import WORKLOADS
    bench = load_bench()
    w = dataclasses.replace(WORKLOADS["llama8b-16k"], L=1000, b=300, T=0, Lq=0)
    per_head = 0
    for i, (s, e) in enumerate(so.blocks(w.L, w.b)):
        keys, mask = so.phase1_block_keys(i, w.L, w.b, w.a)
        per_head += 4 * w.D * mask.shape[0] * mask.shape[1]
    assert bench.oracle_flops(w) == per_head * w.Hq * w.B
    assert bench.oracle_flops(w, 2) < bench.oracle_flops(w)


def _trace_row(i, name, start, end, wg=256, block=512):
    return (f'KERNEL_DISPATCH,1,1,1,1,{i},1,"{name}",{i},{start},{end},0,0,{block},1,1,'
            f'{block * wg},1,1\n')


def test_trace_sequences_cold_and_query(tmp_path):
    """Launch-order figures: a decode launch right after the flushing
    reduction is a cold sample, its merge follows it; flash launches below the
    largest grid are the query partials, in launch order."""
    bench = load_bench()
    hdr = ("Kind,Agent_Id,Queue_Id,Stream_Id,Thread_Id,Dispatch_Id,Kernel_Id,Kernel_Name,"
           "Correlation_Id,Start_Timestamp,End_Timestamp,Private_Segment_Size,"
           "Group_Segment_Size,Workgroup_Size_X,Workgroup_Size_Y,Workgroup_Size_Z,"
           "Grid_Size_X,Grid_Size_Y,Grid_Size_Z\n")
    dec = "void star::(anonymous namespace)::decode_kernel<128, __bf16, true>(star::DecodeParams)"
    mrg = "void star::(anonymous namespace)::merge_kernel<128>(star::MergeParams)"
    red = "void at::native::reduce_kernel<512, 1>(int)"
    fl = "star::(anonymous namespace)::flash2_kernel(star::FlashParams)"
    rows, t, i = [], 0, 0

    def add(name, dur_ns, wg=256, gap=0):
        nonlocal t, i
        rows.append(_trace_row(i, name, t + gap, t + gap + dur_ns, wg))
        t += gap + dur_ns
        i += 1
    add(fl, 40_000_000, wg=18440)
    add(fl, 140_000, gap=5000)
    add(fl, 150_000, gap=5000)
    for cold in (True, False, True, False):
        if cold:
            add(red, 270_000, wg=1, gap=3000)
        add(dec, 88_000 if cold else 86_000, gap=2000)
        add(mrg, 4_000, wg=32, gap=500)
    (tmp_path / "run_kernel_trace.csv").write_text(hdr + "".join(rows))
    out = bench.trace_summary(str(tmp_path))
    cold = next(l for l in out.splitlines() if l.startswith("decode steps right after"))
    warm = next(l for l in out.splitlines() if l.startswith("other decode steps"))
    assert "2 launches; median decode 88.00 us, merge 4.00 us" in cold
    assert "decode start to merge end 92.50 us, gap between the launches 0.50 us" in cold
    assert "2 launches; median decode 86.00 us" in warm
    q = next(l for l in out.splitlines() if l.startswith("Phase-2 query partials"))
    assert q.endswith("first 2 in launch order: 140.0, 150.0 us")


def _counter_rows(name, grid_wg, counters, start=0):
    out = []
    for c, v in counters.items():
        out.append(f'{start},{start},"Agent 1",1,1,1,{grid_wg * 512},1,"{name}",512,0,0,128,0,96,'
                   f'"{c}",{v},{start},{start + 10}\n')
    return out


def test_counter_summary_scales_bytes_by_the_copy(tmp_path):
    """Byte counters are scaled by the plain copy of known size (fetch read
    at half: scale 2, writes at full: scale 1), and the Phase-1 launch's
    traffic line carries the flash kernel's source hash, as the benchmark's
    roofline reads it.  A smaller copyBuffer dispatch (a host copy of the
    step) is not taken for the calibration."""
    import hashlib
    bench = load_bench()
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
           '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
           '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
           '"Counter_Value","Start_Timestamp","End_Timestamp"\n')
    fl = "star::(anonymous namespace)::flash2_kernel(star::FlashParams)"
    for sub, c, copy_v, fl_v in (("f", "FETCH_SIZE", 524288, 1_000_000),
                                 ("w", "WRITE_SIZE", 1048576, 500_000)):
        d = tmp_path / sub
        d.mkdir()
        # a small host copy through the same kernel comes first: the
        # calibration is the large one
        rows = (_counter_rows("__amd_rocclr_copyBuffer", 1, {c: 3}, 1)
                + _counter_rows("__amd_rocclr_copyBuffer", 256, {c: copy_v}, 2)
                + _counter_rows(fl, 256, {c: 7}, 5) + _counter_rows(fl, 18440, {c: fl_v}, 9))
        (d / "run_counter_collection.csv").write_text(hdr + "".join(rows))
    out = bench.counter_summary([str(tmp_path / "f"), str(tmp_path / "w")], 1024)
    want = (1_000_000 * 2.0 + 500_000 * 1.0) * 1024
    line = next(l for l in out.splitlines() if l.startswith("traffic_bytes_per_launch:"))
    assert abs(float(line.split(":")[1]) - want) / want < 1e-6
    src = hashlib.sha256(open(os.path.join(ROOT, "block_sparse_amd", "csrc", "flash2.hip"),
                              "rb").read()).hexdigest()
    assert f"flash_src_sha256: {src}" in out


def test_counter_summary_sq_ratios(tmp_path):
    """The Phase-1 launch's SQ ratios: MFMA busy over the SIMD cycles of the
    launch (GRBM_GUI_ACTIVE summed over 8 XCDs, 1024 SIMDs) and per-MFMA
    instruction counts."""
    bench = load_bench()
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
           '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
           '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
           '"Counter_Value","Start_Timestamp","End_Timestamp"\n')
    fl = "star::(anonymous namespace)::flash2_kernel(star::FlashParams)"
    c = {"GRBM_GUI_ACTIVE": 8 * 1000, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1000 * 1024,
         "SQ_INSTS_MFMA": 500, "SQ_INSTS_VALU": 2000, "SQ_WAVE_CYCLES": 100,
         "SQ_WAIT_ANY": 30, "SQ_ACTIVE_INST_ANY": 45}
    (tmp_path / "run_counter_collection.csv").write_text(hdr + "".join(_counter_rows(fl, 18440, c)))
    out = bench.counter_summary([str(tmp_path)])
    val = {l.rsplit(None, 1)[0].strip(): float(l.split()[-1]) for l in out.splitlines()
           if l.startswith("  ") and l.split()[-1][0].isdigit()}
    assert val["MFMA busy / SIMD cycles (1024 SIMDs)"] == pytest.approx(0.5)
    assert val["VALU instructions / MFMA (incl. MFMA)"] == pytest.approx(4.0)
    assert val["wave cycles waiting (SQ_WAIT_ANY)"] == pytest.approx(0.30)
    assert val["wave cycles ready, not issued"] == pytest.approx(0.25)
