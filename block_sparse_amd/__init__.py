"""MI355X (gfx950) Star Attention hot path.

Thin PyTorch-facing binding of the C ABI in ``include/star_attn.h``: the
functions below only turn torch tensors into ``star_tensor`` descriptors,
pick the current HIP stream and call the library.  Every step of the
computation runs in the library's HIP kernels.  PyTorch provides device
memory and streams only; tensors must live on a ROCm device.

Phase 1 -- anchor-block blockwise-local causal attention (context encoding),
           or the same with any per-block prefix (anchor ablations, Pulsar's
           sink + Max-IDF summaries).
Phase 2 -- per-partition partials + exact LSE merge (query and decode).
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import STAR_MAX_PARTS, STAR_SPLIT_ALIGN, StarError  # noqa: F401

__all__ = ["rope_apply", "rope_freqs", "kv_append", "decode_prepare", "phase1_blocklocal", "phase1_rope",
           "phase1_prefix", "sched_workspace", "SCHED_INTS",
           "gather_rows", "pulsar_prefix", "phase2_partial", "lse_merge", "decode_step",
           "decode_step_devpos", "decode_step_noalloc",
           "Context", "rmsnorm", "linear", "split_ranges", "stream_read",
           "StarError", "library"]


def library():
    return _lib.load()


def _desc(t: torch.Tensor) -> _lib.StarTensor:
    if t.dim() != 4:
        raise ValueError(f"expected a [B, H, S, D] tensor, got shape {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    if t.dtype == torch.bfloat16:
        dt = _lib.STAR_BF16
    elif t.dtype == torch.float32:
        dt = _lib.STAR_F32
    else:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the head dim must be contiguous")
    B, H, S, D = t.shape
    return _lib.StarTensor(t.data_ptr(), dt, 0, B, H, S, D,
                           t.stride(0), t.stride(1), t.stride(2))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# int32 count of a Phase-1 scheduling workspace (STAR_SCHED_INTS)
SCHED_INTS = 16


def sched_workspace(device=None) -> torch.Tensor:
    """A Phase-1 scheduling workspace: ``SCHED_INTS`` int32 on ``device``.
    Passed as ``sched=`` to the Phase-1 calls, it lets the kernel hand out
    its items from per-XCD queues (faster XCDs take over the slower ones'
    remaining items); results are identical with or without it.  One
    workspace must not serve two calls that may run at the same time."""
    return torch.zeros(SCHED_INTS, dtype=torch.int32, device=device)


def _sched_ptr(sched, like: torch.Tensor):
    if sched is None:
        return None
    if (not isinstance(sched, torch.Tensor) or sched.dtype != torch.int32
            or sched.numel() < SCHED_INTS or not sched.is_contiguous()
            or sched.device != like.device):
        raise ValueError(f"sched must be a contiguous int32 tensor of at least {SCHED_INTS} "
                         "elements on the inputs' device")
    return ctypes.c_void_p(sched.data_ptr())


def rope_apply(x: torch.Tensor, pos: torch.Tensor | None = None, pos0: int = 0,
               base: float = 500000.0, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rotate-half RoPE of ``x[B, H, S, D]`` at positions ``pos[S]`` (int64,
    device) or ``pos0 + s``.  In place when ``out`` is None."""
    out = x if out is None else out
    if pos is not None:
        if pos.dtype != torch.int64 or pos.numel() != x.shape[2] or not pos.is_contiguous():
            raise ValueError("pos must be a contiguous int64 tensor of length S")
    a, b = _desc(x), _desc(out)
    st = library().star_rope_apply(ctypes.byref(a), ctypes.byref(b), _ptr(pos), int(pos0),
                                   float(base), _stream(x))
    _lib.check("star_rope_apply", st)
    return out


def rope_freqs(D: int, base: float = 500000.0):
    """The RoPE frequencies theta_j (fp64, j < D/2) every rotating entry
    point uses, as a list of floats (host call, no GPU needed)."""
    out = (ctypes.c_double * max(D // 2, 1))()
    _lib.check("star_rope_freqs", library().star_rope_freqs(int(D), float(base), out))
    return list(out)[:D // 2]


def kv_append(k_new, v_new, k_cache, v_cache, slot0: int, pos0: int,
              base: float = 500000.0, rope: bool = True):
    """Rotate ``k_new`` at positions ``pos0 + t`` and write it, with
    ``v_new``, into cache rows ``slot0 + t``."""
    d = [_desc(t) for t in (k_new, v_new, k_cache, v_cache)]
    st = library().star_kv_append(*[ctypes.byref(x) for x in d], int(slot0), int(pos0),
                                  float(base), int(bool(rope)), _stream(k_new))
    _lib.check("star_kv_append", st)


def decode_prepare(q_new, q_out, k_new, v_new, k_cache, v_cache, slot0: int, pos0: int,
                   base: float = 500000.0, rope: bool = True):
    """One launch: rotate ``q_new`` at positions ``pos0 + t`` into ``q_out``
    and append ``k_new``/``v_new`` to the cache rows ``slot0 + t``."""
    d = [_desc(t) for t in (q_new, q_out, k_new, v_new, k_cache, v_cache)]
    st = library().star_decode_prepare(*[ctypes.byref(x) for x in d], int(slot0), int(pos0),
                                       float(base), int(bool(rope)), _stream(q_new))
    _lib.check("star_decode_prepare", st)


def phase1_blocklocal(q, k, v, block_b: int, anchor_len: int | None = None,
                      scale: float | None = None, out=None, lse=None,
                      want_lse: bool = False, sched=None):
    """Phase 1 context encoding.  Returns ``(o, lse)`` (lse None unless
    ``want_lse`` or an ``lse`` buffer is given).  ``sched``: optional
    scheduling workspace (:func:`sched_workspace`)."""
    B, Hq, L, D = q.shape
    if anchor_len is None:
        anchor_len = block_b
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.numel() != B * Hq * L):
        raise ValueError("lse must be a contiguous fp32 [B, Hq, L] tensor")
    dq, dk, dv, do = _desc(q), _desc(k), _desc(v), _desc(out)
    st = library().star_phase1_blocklocal(
        ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(block_b), int(anchor_len),
        float(scale), ctypes.byref(do), _ptr(lse), _sched_ptr(sched, q), _stream(q))
    _lib.check("star_phase1_blocklocal", st)
    return out, lse


def phase1_rope(q, k, v, block_b: int, anchor_len: int | None = None,
                base: float = 500000.0, scale: float | None = None, out=None, lse=None,
                want_lse: bool = False, sched=None):
    """Phase 1 with the RoPE of ``q`` fused in: ``q`` holds un-rotated rows
    (rotated in the kernel at positions 0..L-1), ``k`` is already rotated.
    bf16, D = 128.  Returns ``(o, lse)`` like :func:`phase1_blocklocal`."""
    B, Hq, L, D = q.shape
    if anchor_len is None:
        anchor_len = block_b
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.numel() != B * Hq * L):
        raise ValueError("lse must be a contiguous fp32 [B, Hq, L] tensor")
    dq, dk, dv, do = _desc(q), _desc(k), _desc(v), _desc(out)
    st = library().star_phase1_rope(
        ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(block_b), int(anchor_len),
        float(base), float(scale), ctypes.byref(do), _ptr(lse), _sched_ptr(sched, q), _stream(q))
    _lib.check("star_phase1_rope", st)
    return out, lse


def phase1_prefix(q, k, v, pk, pv, prefix_start, prefix_len, block_b: int,
                  scale: float | None = None, out=None, lse=None, want_lse: bool = False,
                  sched=None):
    """Phase 1 where block i attends to all of ``pk/pv`` rows
    ``[prefix_start[i], prefix_start[i] + prefix_len[i])`` and then causally
    within itself.  ``prefix_start``/``prefix_len`` are host sequences of
    ceil(L / block_b) ints.  Returns ``(o, lse)``."""
    B, Hq, L, D = q.shape
    n = -(-L // block_b)
    if len(prefix_start) != n or len(prefix_len) != n:
        raise ValueError(f"prefix table needs {n} entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, L, D), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.numel() != B * Hq * L):
        raise ValueError("lse must be a contiguous fp32 [B, Hq, L] tensor")
    st_arr = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in prefix_start])
    ln_arr = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in prefix_len])
    d = [_desc(t) for t in (q, k, v, pk, pv)]
    do = _desc(out)
    st = library().star_phase1_prefix(*[ctypes.byref(x) for x in d], st_arr, ln_arr, int(n),
                                      int(block_b), float(scale), ctypes.byref(do), _ptr(lse),
                                      _sched_ptr(sched, q), _stream(q))
    _lib.check("star_phase1_prefix", st)
    return out, lse


def gather_rows(src, rows, out=None):
    """``out[b, h, r] = src[b, h, rows[r]]`` (``rows`` device int64)."""
    if rows.dtype != torch.int64 or not rows.is_contiguous() or rows.dim() != 1:
        raise ValueError("rows must be a contiguous 1-D int64 tensor")
    B, H, _, D = src.shape
    if out is None:
        out = torch.empty((B, H, rows.numel(), D), dtype=src.dtype, device=src.device)
    if out.shape[2] != rows.numel():
        raise ValueError("out must have one row per index")
    a, b = _desc(src), _desc(out)
    st = library().star_gather_rows(ctypes.byref(a), _ptr(rows), ctypes.byref(b), _stream(src))
    _lib.check("star_gather_rows", st)
    return out


def stream_read(buf: torch.Tensor, workgroups: int = 4096, out=None):
    """Plain streaming read of ``buf`` (a measurement aid, not a step of the
    method): returns the per-workgroup XOR of the 32-bit words read, device
    uint32 [workgroups] as int32."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if out is None:
        out = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    st = library().star_stream_read(_ptr(buf), buf.numel() * buf.element_size(),
                                    int(workgroups), _ptr(out), _stream(buf))
    _lib.check("star_stream_read", st)
    return out


def pulsar_prefix(tokens, L: int, block_b: int, chunk_m: int = 32, sink: int = 64,
                  k: int = 16):
    """Pulsar's prefix rows and per-block table from host token ids (the
    library's host-side Max-IDF selection).  Returns numpy int64
    ``(rows[R], prefix_start[n], prefix_len[n])``."""
    import numpy as np
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    if tok.shape != (L,):
        raise ValueError("tokens must be a 1-D array of L ids")
    n = -(-L // block_b)
    st = np.zeros(max(n, 1), dtype=np.int64)
    ln = np.zeros(max(n, 1), dtype=np.int64)
    nrows = ctypes.c_int64(0)
    P64 = ctypes.POINTER(ctypes.c_int64)
    tptr = tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    lib = library()
    args = (tptr, int(L), int(block_b), int(chunk_m), int(sink), int(k))
    # at most the sink plus k chunks of every block but the last
    cap = min(L, min(sink, block_b, L) + max(n - 1, 0) * max(k, 0) * chunk_m)
    rows = np.zeros(max(cap, 1), dtype=np.int64)
    r = lib.star_pulsar_prefix(*args, rows.ctypes.data_as(P64), int(rows.size),
                               ctypes.byref(nrows), st.ctypes.data_as(P64),
                               ln.ctypes.data_as(P64), int(n))
    if r == _lib.STATUS_CODE["STAR_ERR_SHAPE"] and nrows.value > rows.size:
        rows = np.zeros(nrows.value, dtype=np.int64)
        r = lib.star_pulsar_prefix(*args, rows.ctypes.data_as(P64), int(rows.size),
                                   ctypes.byref(nrows), st.ctypes.data_as(P64),
                                   ln.ctypes.data_as(P64), int(n))
    _lib.check("star_pulsar_prefix", r)
    return rows[:nrows.value], st[:n], ln[:n]


def split_ranges(part_offsets, splits: int):
    """The [start, end) key range of every chunk, in o_part order: partition
    j is cut into chunks of roundup(ceil(n_j / splits), 64) keys."""
    out = []
    for j in range(len(part_offsets) - 1):
        a, b = int(part_offsets[j]), int(part_offsets[j + 1])
        c = -(-(b - a) // splits)
        c = -(-c // STAR_SPLIT_ALIGN) * STAR_SPLIT_ALIGN
        for s in range(splits):
            lo = a + s * c
            out.append((min(lo, b), min(lo + c, b)))
    return out


def phase2_partial(q, k_cache, v_cache, part_offsets, splits: int = 1, q_pos0: int = 0,
                   scale: float | None = None, o_part=None, lse_part=None):
    """Per-chunk partials of query rows ``q[B, Hq, Lq, D]`` (at positions
    ``q_pos0 + r``) over the cache partitions ``part_offsets[P + 1]``.
    Returns ``(o_part[P*splits, B, Hq, Lq, D], lse_part[P*splits, B, Hq, Lq])``."""
    B, Hq, Lq, D = q.shape
    P = len(part_offsets) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    N = P * splits
    if o_part is None:
        o_part = torch.empty((N, B, Hq, Lq, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((N, B, Hq, Lq), dtype=torch.float32, device=q.device)
    for t, n in ((o_part, N * B * Hq * Lq * D), (lse_part, N * B * Hq * Lq)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < n:
            raise ValueError("o_part / lse_part must be contiguous fp32 buffers of the full size")
    offs = (ctypes.c_int64 * (P + 1))(*[int(x) for x in part_offsets])
    dq, dk, dv = _desc(q), _desc(k_cache), _desc(v_cache)
    st = library().star_phase2_partial(
        ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), offs, int(P), int(splits),
        int(q_pos0), float(scale), _ptr(o_part), _ptr(lse_part), _stream(q))
    _lib.check("star_phase2_partial", st)
    return o_part, lse_part


def lse_merge(o_part, lse_part, out=None, lse=None, out_dtype=torch.float32,
              want_lse: bool = True):
    """Exact LSE merge over the leading (partial) dim of ``o_part[N, B, H, S, D]``.
    Returns ``(o[B, H, S, D], lse[B, H, S])``."""
    N, B, H, S, D = o_part.shape
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("o_part and lse_part must be contiguous")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise TypeError("partials are fp32")
    if tuple(lse_part.shape) != (N, B, H, S):
        raise ValueError("lse_part shape mismatch")
    if out is None:
        out = torch.empty((B, H, S, D), dtype=out_dtype, device=o_part.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=o_part.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.numel() != B * H * S):
        raise ValueError("lse must be a contiguous fp32 tensor of B*H*S rows")
    do = _desc(out)
    st = library().star_lse_merge(_ptr(o_part), _ptr(lse_part), int(N), int(B), int(H), int(S),
                                  int(D), ctypes.byref(do), _ptr(lse), _stream(o_part))
    _lib.check("star_lse_merge", st)
    return out, lse


def decode_step(q_new, k_new, v_new, k_cache, v_cache, slot: int, pos: int, part_offsets,
                splits: int, o_part, lse_part, out, lse=None, base: float = 500000.0,
                rope: bool = True, scale: float | None = None):
    """One generated token: rope of its q/k at ``pos``, its K/V appended at
    cache row ``slot`` and the split-KV partials over ``part_offsets`` in one
    launch, then their merge into ``out[B, Hq, 1, D]`` (and ``lse`` [B, Hq]).
    ``o_part``/``lse_part`` are fp32 workspaces of phase2_partial's sizes."""
    B, Hq, _, D = q_new.shape
    P = len(part_offsets) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    N = P * splits
    for t, n in ((o_part, N * B * Hq * D), (lse_part, N * B * Hq)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < n:
            raise ValueError("o_part / lse_part must be contiguous fp32 buffers of the full size")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.numel() != B * Hq):
        raise ValueError("lse must be a contiguous fp32 [B, Hq] tensor")
    offs = (ctypes.c_int64 * (P + 1))(*[int(x) for x in part_offsets])
    d = [_desc(t) for t in (q_new, k_new, v_new, k_cache, v_cache)]
    do = _desc(out)
    st = library().star_decode_step(*[ctypes.byref(x) for x in d], int(slot), int(pos),
                                    float(base), int(bool(rope)), offs, int(P), int(splits),
                                    float(scale), _ptr(o_part), _ptr(lse_part),
                                    ctypes.byref(do), _ptr(lse), _stream(q_new))
    _lib.check("star_decode_step", st)
    return out, lse


def decode_step_devpos(q_new, k_new, v_new, k_cache, v_cache, pos_dev, part_offsets,
                       splits: int, o_part, lse_part, out, lse=None, base: float = 500000.0,
                       rope: bool = True, scale: float | None = None):
    """:func:`decode_step` with the token's position in device memory
    (``pos_dev``: a one-element int64 device tensor, read at the start of
    the step and advanced by one at its end), so that a captured graph of
    the call serves every step.  ``part_offsets[-1]`` bounds the positions
    the call may run at (star_decode_step_devpos)."""
    B, Hq, _, D = q_new.shape
    P = len(part_offsets) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if (pos_dev.dtype != torch.int64 or pos_dev.numel() != 1 or pos_dev.device.type != "cuda"):
        raise ValueError("pos_dev must be a one-element int64 device tensor")
    N = P * splits
    for t, n in ((o_part, N * B * Hq * D), (lse_part, N * B * Hq)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < n:
            raise ValueError("o_part / lse_part must be contiguous fp32 buffers of the full size")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.numel() != B * Hq):
        raise ValueError("lse must be a contiguous fp32 [B, Hq] tensor")
    offs = (ctypes.c_int64 * (P + 1))(*[int(x) for x in part_offsets])
    d = [_desc(t) for t in (q_new, k_new, v_new, k_cache, v_cache)]
    do = _desc(out)
    st = library().star_decode_step_devpos(*[ctypes.byref(x) for x in d], _ptr(pos_dev),
                                           float(base), int(bool(rope)), offs, int(P),
                                           int(splits), float(scale), _ptr(o_part),
                                           _ptr(lse_part), ctypes.byref(do), _ptr(lse),
                                           _stream(q_new))
    _lib.check("star_decode_step_devpos", st)
    return out, lse


def decode_step_noalloc(q_new, k_new, v_new, k_cache, v_cache, slot: int, pos: int,
                        part_offsets, splits: int, out, lse=None, base: float = 500000.0,
                        rope: bool = True, scale: float | None = None):
    """:func:`decode_step` without caller workspaces: the partials live in the
    library's per-GPU scratch array (star_decode_step_noalloc; nothing is
    allocated).  Calls that may overlap on one GPU must not be issued."""
    B, Hq, _, D = q_new.shape
    P = len(part_offsets) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.numel() != B * Hq):
        raise ValueError("lse must be a contiguous fp32 [B, Hq] tensor")
    offs = (ctypes.c_int64 * (P + 1))(*[int(x) for x in part_offsets])
    d = [_desc(t) for t in (q_new, k_new, v_new, k_cache, v_cache)]
    do = _desc(out)
    st = library().star_decode_step_noalloc(*[ctypes.byref(x) for x in d], int(slot), int(pos),
                                            float(base), int(bool(rope)), offs, int(P),
                                            int(splits), float(scale), ctypes.byref(do),
                                            _ptr(lse), _stream(q_new))
    _lib.check("star_decode_step_noalloc", st)
    return out, lse


class Context:
    """Owner of the library's rocBLAS handle (star_context); needed by
    :func:`linear`.  Create once and reuse; ``close()`` releases it."""

    def __init__(self):
        self._ptr = ctypes.c_void_p()
        _lib.check("star_context_create", library().star_context_create(ctypes.byref(self._ptr)))

    @property
    def handle(self):
        return self._ptr

    def close(self):
        if self._ptr:
            library().star_context_destroy(self._ptr)
            self._ptr = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


def _mat(t: torch.Tensor) -> _lib.StarTensor:
    """[M, K] bf16 matrix (unit column stride) as a [1, 1, M, K] descriptor."""
    if t.dim() != 2:
        raise ValueError(f"expected a matrix, got shape {tuple(t.shape)}")
    if t.dtype != torch.bfloat16 or t.device.type != "cuda":
        raise TypeError("matrices are bf16 device tensors")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("matrix rows must be contiguous")
    M, K = t.shape
    return _lib.StarTensor(t.data_ptr(), _lib.STAR_BF16, 0, 1, 1, M, K, M * t.stride(0),
                           M * t.stride(0), t.stride(0))


def rmsnorm(x, gamma, eps: float = 1e-5, out=None):
    """Row RMSNorm of ``x`` ([B, H, S, D] or a [M, D] matrix) by ``gamma[D]``."""
    out = torch.empty_like(x) if out is None else out
    if gamma.dtype != torch.bfloat16 or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous bf16 vector")
    a = _desc(x) if x.dim() == 4 else _mat(x)
    b = _desc(out) if out.dim() == 4 else _mat(out)
    st = library().star_rmsnorm(ctypes.byref(a), _ptr(gamma), float(eps), ctypes.byref(b),
                                _stream(x))
    _lib.check("star_rmsnorm", st)
    return out


def linear(ctx: Context, x, w, residual=None, out=None):
    """``out[M, N] = x[M, K] w[N, K]^T (+ residual)`` in rocBLAS (bf16, fp32
    accumulation)."""
    if out is None:
        out = torch.empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16, device=x.device)
    dx, dw, dy = _mat(x), _mat(w), _mat(out)
    dr = None if residual is None else _mat(residual)
    st = library().star_linear(ctx.handle, ctypes.byref(dx), ctypes.byref(dw),
                               None if dr is None else ctypes.byref(dr), ctypes.byref(dy),
                               _stream(x))
    _lib.check("star_linear", st)
    return out
