"""Host-side checks of the generated gfx950 code (no GPU).

The Phase-1 kernel issues its global -> LDS tile loads from inline asm that
sets M0, a register the compiler reserves and does not preserve around asm.
That is only sound while the compiled kernel keeps no M0 value of its own:
every write of M0 must be one of those loads' set-ups, directly followed by
its global_load_lds_dwordx4, and nothing else may read M0.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def device_asm(src: str, tmp_path) -> str:
    from block_sparse_amd import build as B
    out = tmp_path / "k.s"
    cmd = [B.hipcc(), *B.COMMON, *B.DEVICE_FLAGS, "-x", "hip", "--cuda-device-only", "-S",
           src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-2000:])
    return out.read_text()


def test_m0_only_set_for_the_tile_loads(tmp_path):
    asm = device_asm(os.path.join(ROOT, "block_sparse_amd", "csrc", "flash2.hip"), tmp_path)
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    code = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    writes = 0
    for i, l in enumerate(code):
        if not re.search(r"\bm0\b", l):
            continue
        assert re.match(r"s_mov_b32 m0, s\d+$", l), f"unexpected use of M0: {l}"
        nxt = code[i + 1] if i + 1 < len(code) else ""
        assert nxt.startswith("global_load_lds_dwordx4"), f"M0 set but not for a tile load: {nxt}"
        writes += 1
    assert writes > 0


def kernel_meta(asm: str) -> dict:
    """name -> {vgpr_count, vgpr_spill_count, sgpr_spill_count} from the
    code object metadata of the generated assembly."""
    meta, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            cur = m.group(1)
            meta[cur] = {}
            continue
        m = re.match(r"\s+\.(vgpr_count|vgpr_spill_count|sgpr_spill_count):\s+(\d+)", line)
        if m and cur is not None:
            meta[cur][m.group(1)] = int(m.group(2))
    return meta


@pytest.mark.parametrize("src,kernels", [
    ("flash2.hip", ["flash2_kernel"]),
    ("decode.hip", ["decode_kernelILi128EDF16bLb1E", "decode_kernelILi128EDF16bLb0E",
                    "decode_kernelILi64EDF16bLb1E"]),
])
def test_hot_kernels_do_not_spill(src, kernels, tmp_path):
    """The timed kernels fit the register file of two waves per SIMD
    (256 VGPRs) without scratch: a spill in the key loop would cost far
    more than any change that caused it could gain."""
    meta = kernel_meta(device_asm(os.path.join(ROOT, "block_sparse_amd", "csrc", src), tmp_path))
    for k in kernels:
        hits = [n for n in meta if k in n]
        assert hits, f"no kernel named like {k}"
        for n in hits:
            assert "vgpr_count" in meta[n] and "vgpr_spill_count" in meta[n], (n, meta[n])
            assert meta[n]["vgpr_spill_count"] == 0, (n, meta[n])
            assert 0 < meta[n]["vgpr_count"] <= 256, (n, meta[n])
