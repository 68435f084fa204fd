"""Seeded synthetic workloads for the Star Attention hot path.

This module holds the workload shapes and the seeded random draws that both
the CPU oracle (``oracle/``) and the HIP library's tests and benchmark use.
It deliberately contains none of the method's arithmetic: no RoPE, no
attention, no softmax, no merge.  It only produces the input tensors.

Shapes follow the configurations the method is evaluated on: Llama-3.1-8B
and -70B single-layer attention shapes (32/8 and 64/8 query/KV heads, head
dim 128) at 16K-1M context, plus a tiny case (Star Attention review page,
"Assumptions & free parameters": block size is a quarter of the sequence up
to 128K and 32K beyond; anchor size equals block size).  The pages evaluate
on RULER / BABILong / InfiniteBench with real model weights; those are not
available, so every tensor here is an i.i.d. normal draw of the same shape.

Draws
-----
Every tensor is generated in row chunks of ``CHUNK_ROWS`` rows.  Chunk
``c`` of (tensor ``tid``, batch ``b``, head ``h``) is

    numpy.random.Generator(PCG64(SeedSequence([seed, tid, b, h, c])))
        .standard_normal((rows, D), dtype=float32) * scale

so any slice can be regenerated independently and chunks can be generated in
parallel threads.  ``scale`` is 1 for the Llama-shaped workloads and 1/8
(= 1/sqrt(64), exact in fp32) for the tiny one.  bf16 inputs are the fp32
draws rounded to nearest-even.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 4096

# tensor ids used in the seed sequence
T_Q, T_K, T_V = 0, 1, 2            # context Q/K/V (pre-RoPE)
T_QQ, T_KQ, T_VQ = 3, 4, 5         # query tokens (Phase 2)
T_QD, T_KD, T_VD = 6, 7, 8         # decode tokens (Phase 2, one per step)
T_TOK = 9                          # context token ids (Pulsar chunk scoring)
T_APOS = 10                        # anchor position ids (position-id ablation)
T_X, T_WQ, T_WK, T_WV, T_WO, T_G = 11, 12, 13, 14, 15, 16   # attention layer
RMS_EPS = 1e-5                     # Llama-3 RMSNorm epsilon

VOCAB = 128256                     # Llama-3 vocabulary size
ZIPF_S = 1.1                       # exponent of the token-rank distribution


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int          # batch (independent sequences)
    Hq: int         # query heads
    Hkv: int        # KV heads
    D: int          # head dim
    L: int          # context length
    b: int          # block size
    Lq: int         # query tokens attending globally in Phase 2
    T: int          # decode steps
    seed: int
    scale: float    # std of the normal draws
    rope: bool      # apply RoPE at original position ids
    base: float = 500000.0
    anchor: int | None = None  # anchor length; None means a = b

    @property
    def a(self) -> int:
        return self.b if self.anchor is None else self.anchor

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_blocks(self) -> int:
        return -(-self.L // self.b)

    @property
    def cache_len(self) -> int:
        """KV entries after the query and every decode step are appended."""
        return self.L + self.Lq + self.T

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the hot path.  Seeds 0..4 in this order.
TINY = Workload("tiny", B=1, Hq=2, Hkv=1, D=64, L=512, b=128, Lq=16, T=0,
                seed=0, scale=0.125, rope=False)
L8B_16K = Workload("llama8b-16k", B=1, Hq=32, Hkv=8, D=128, L=16384, b=4096,
                   Lq=64, T=32, seed=1, scale=1.0, rope=True)
L8B_128K = Workload("llama8b-128k", B=1, Hq=32, Hkv=8, D=128, L=131072,
                    b=16384, Lq=64, T=128, seed=2, scale=1.0, rope=True)
L70B_64K = Workload("llama70b-64k", B=2, Hq=64, Hkv=8, D=128, L=65536,
                    b=8192, Lq=64, T=64, seed=3, scale=1.0, rope=True)
L8B_1M = Workload("llama8b-1m", B=1, Hq=32, Hkv=8, D=128, L=1048576,
                  b=32768, Lq=32, T=32, seed=4, scale=1.0, rope=True)

WORKLOADS = {w.name: w for w in (TINY, L8B_16K, L8B_128K, L70B_64K, L8B_1M)}


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# bf16 round-to-nearest-even on the host (input preparation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaNs stay NaN (quiet).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# seeded draws
# ----------------------------------------------------------------------------
def draw_rows(seed: int, tid: int, b: int, h: int, rows: int, D: int,
              scale: float, row0: int = 0, row1: int | None = None) -> np.ndarray:
    """float32 draws for rows [row0, row1) of one (tensor, batch, head) slice
    whose full length is ``rows``."""
    if row1 is None:
        row1 = rows
    out = np.empty((row1 - row0, D), dtype=np.float32)
    c0, c1 = row0 // CHUNK_ROWS, -(-row1 // CHUNK_ROWS)
    for c in range(c0, c1):
        lo = c * CHUNK_ROWS
        n = min(CHUNK_ROWS, rows - lo)
        rng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([seed, tid, b, h, c])))
        blk = rng.standard_normal((n, D), dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        s0, s1 = max(row0, lo), min(row1, lo + n)
        out[s0 - row0:s1 - row0] = blk[s0 - lo:s1 - lo]
    return out


def draw_tensor(seed: int, tid: int, B: int, H: int, S: int, D: int,
                scale: float, as_bf16: bool = True) -> np.ndarray:
    """Full [B, H, S, D] tensor.  bf16 bit patterns (uint16) if ``as_bf16``,
    else float32.  Generated chunk-parallel over threads."""
    dtype = np.uint16 if as_bf16 else np.float32
    out = np.empty((B, H, S, D), dtype=dtype)
    jobs = [(b, h, c) for b in range(B) for h in range(H)
            for c in range(-(-S // CHUNK_ROWS))]

    def work(job):
        b, h, c = job
        lo, hi = c * CHUNK_ROWS, min(S, (c + 1) * CHUNK_ROWS)
        x = draw_rows(seed, tid, b, h, S, D, scale, lo, hi)
        out[b, h, lo:hi] = f32_to_bf16_bits(x) if as_bf16 else x

    if len(jobs) == 1:
        work(jobs[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, jobs))
    return out


def inputs(w: Workload, as_bf16: bool = True) -> dict:
    """All input tensors of a workload, keyed by name.

    Context ``q, k, v``: [B, H, L, D]; query-phase ``qq, kq, vq``:
    [B, H, Lq, D]; decode ``qd, kd, vd``: [B, H, T, D].  Values are bf16
    bit patterns (uint16) when ``as_bf16``, else float32 draws.
    """
    spec = {
        "q": (T_Q, w.Hq, w.L), "k": (T_K, w.Hkv, w.L), "v": (T_V, w.Hkv, w.L),
        "qq": (T_QQ, w.Hq, w.Lq), "kq": (T_KQ, w.Hkv, w.Lq),
        "vq": (T_VQ, w.Hkv, w.Lq),
        "qd": (T_QD, w.Hq, w.T), "kd": (T_KD, w.Hkv, w.T),
        "vd": (T_VD, w.Hkv, w.T),
    }
    return {name: draw_tensor(w.seed, tid, w.B, H, S, w.D, w.scale, as_bf16)
            for name, (tid, H, S) in spec.items()}


def group_inputs(w: Workload, b: int, kvh: int, as_bf16: bool = True) -> dict:
    """The tensors of one (batch, KV head) group: KV head ``kvh`` of batch
    ``b`` and its g query heads, every slice drawn exactly as :func:`inputs`
    draws it (same seeds), with shapes [1, g, S, D] (query heads) and
    [1, 1, S, D] (the KV head)."""
    g = w.g
    spec = {
        "q": (T_Q, True, w.L), "k": (T_K, False, w.L), "v": (T_V, False, w.L),
        "qq": (T_QQ, True, w.Lq), "kq": (T_KQ, False, w.Lq), "vq": (T_VQ, False, w.Lq),
        "qd": (T_QD, True, w.T), "kd": (T_KD, False, w.T), "vd": (T_VD, False, w.T),
    }
    out = {}
    for name, (tid, is_q, S) in spec.items():
        heads = range(kvh * g, (kvh + 1) * g) if is_q else [kvh]
        arr = np.empty((1, len(heads), S, w.D), dtype=np.uint16 if as_bf16 else np.float32)
        for i, h in enumerate(heads):
            x = draw_rows(w.seed, tid, b, h, S, w.D, w.scale)
            arr[0, i] = f32_to_bf16_bits(x) if as_bf16 else x
        out[name] = arr
    return out


def as_f64(t: np.ndarray) -> np.ndarray:
    """Exact float64 view of a tensor from ``inputs`` (bf16 bits or fp32)."""
    if t.dtype == np.uint16:
        return bf16_bits_to_f32(t).astype(np.float64)
    return t.astype(np.float64)


# ----------------------------------------------------------------------------
# inputs of the Phase-1 prefix variants
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PulsarParams:
    """Pulsar's free parameters (Pulsar review page, "Assumptions & free
    parameters"): chunk of m tokens, a sink of ``sink`` tokens, and k chunks
    per block, i.e. a summary budget of 12.5% of the block (16 chunks of 32
    for a 4096-token block, scaled with the block)."""
    m: int = 32
    sink: int = 64
    k: int = 16


def pulsar_params(w: Workload) -> PulsarParams:
    return PulsarParams(m=32, sink=64, k=max(1, w.b // 256))


def token_ids(seed: int, B: int, L: int) -> np.ndarray:
    """Synthetic context token ids [B, L] (int32).  Token ranks follow a
    Zipf law p(r) ~ r^-ZIPF_S over the VOCAB ranks (a few frequent tokens,
    a long tail of rare ones, as in text); ranks map to ids through a seeded
    permutation.  The pages score chunks by the rarity of their tokens, so
    only the frequency structure matters, not which ids carry it."""
    ranks = np.arange(1, VOCAB + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** -ZIPF_S)
    cdf /= cdf[-1]
    out = np.empty((B, L), dtype=np.int32)
    for b in range(B):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, T_TOK, b])))
        perm = rng.permutation(VOCAB)
        r = np.searchsorted(cdf, rng.random(L), side="right")
        out[b] = perm[np.minimum(r, VOCAB - 1)]
    return out


def anchor_positions(seed: int, L: int, b: int, a: int) -> list:
    """Position ids for the anchor of every block in the position-id
    ablation: for block i >= 1, ``a`` distinct positions drawn uniformly
    from [0, i*b) (positions before the block), sorted.  Block 0 (no
    anchor) gets its original positions 0..a-1 as a placeholder."""
    n = -(-L // b)
    a = min(a, L)
    out = [np.arange(a, dtype=np.int64)]
    for i in range(1, n):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, T_APOS, i])))
        out.append(np.sort(rng.choice(i * b, size=a, replace=False)).astype(np.int64))
    return out


# ----------------------------------------------------------------------------
# inputs of the attention layer around Phase 1 (random weights)
# ----------------------------------------------------------------------------
def layer_inputs(w: Workload, n_layers: int = 1, as_bf16: bool = True) -> dict:
    """Residual-stream input x [B, L, H] (H = Hq*D, N(0,1)) and, per layer,
    RMSNorm gain gamma [H] (1 + N(0, 0.1^2)) and projection weights in the
    [out, in] layout: wq [Hq*D, H], wk and wv [Hkv*D, H], wo [H, Hq*D], each
    N(0, 1/H) so that projections keep unit scale.  Layer i's weights are
    draws with batch index i.  bf16 bit patterns when ``as_bf16``."""
    H = w.Hq * w.D
    s = float(1.0 / np.sqrt(H))
    x = draw_tensor(w.seed, T_X, w.B, 1, w.L, H, 1.0, as_bf16)[:, 0]
    def mat(tid, rows, cols):
        return draw_tensor(w.seed, tid, n_layers, 1, rows, cols, s, as_bf16)[:, 0]
    g = draw_tensor(w.seed, T_G, n_layers, 1, 1, H, 0.1, as_bf16=False)[:, 0, 0]
    g = (g + np.float32(1.0)).astype(np.float32)
    gamma = f32_to_bf16_bits(g) if as_bf16 else g
    wq, wk, wv = mat(T_WQ, w.Hq * w.D, H), mat(T_WK, w.Hkv * w.D, H), mat(T_WV, w.Hkv * w.D, H)
    wo = mat(T_WO, H, w.Hq * w.D)
    layers = [{"gamma": gamma[i], "wq": wq[i], "wk": wk[i], "wv": wv[i], "wo": wo[i]}
              for i in range(n_layers)]
    return {"x": x, "layers": layers}
