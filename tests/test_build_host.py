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
