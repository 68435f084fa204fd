"""GPU parity of the attention layer around Phase 1 (RMSNorm, rocBLAS
projections, RoPE, Phase-1 attention, output projection + residual) against
the CPU oracle: each building block on its own, stacks of 1-2 layers on small
shapes element by element, and one layer at the 8B-16K shape on sampled
rows."""
import math
import time

import numpy as np
import pytest
import torch

import block_sparse_amd as sa
import oracle.star_oracle as so
from block_sparse_amd.layer import AttentionLayers
from gpu_util import check_out, f64, host64, rand_tensor, to_dev
from workloads import RMS_EPS, WORKLOADS, Workload, layer_inputs

pytestmark = pytest.mark.gpu


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.mark.parametrize("rows,D", [(300, 4096), (77, 512), (50, 8192), (40, 1000)])
def test_rmsnorm_parity(rows, D):
    """The register-resident kernel (D = 512 .. 8192, powers of two) and the
    general one (D = 1000)."""
    x = rand_tensor(61, 0, 1, 1, rows, D)[0, 0]
    g = rand_tensor(61, 1, 1, 1, 1, D, 0.5)[0, 0, 0]
    y = sa.rmsnorm(to_dev(x), to_dev(g), RMS_EPS)
    torch.cuda.synchronize()
    ref = so.rmsnorm(f64(x), f64(g), RMS_EPS)
    got = host64(y)
    # one bf16 rounding of the fp32 result: half an ulp, 2^-8 relative
    assert (np.abs(got - ref) <= np.abs(ref) * 2.0**-8 + 1e-6).all()


@pytest.mark.parametrize("M,K,N,res", [(300, 256, 384, False), (1000, 1024, 512, True),
                                       (64, 4096, 6144, True)])
def test_linear_parity(M, K, N, res):
    x = rand_tensor(62, 0, 1, 1, M, K)[0, 0]
    w = rand_tensor(62, 1, 1, 1, N, K, 1 / math.sqrt(K))[0, 0]
    r = rand_tensor(62, 2, 1, 1, M, N)[0, 0]
    ctx = sa.Context()
    y = sa.linear(ctx, to_dev(x), to_dev(w), residual=to_dev(r) if res else None)
    torch.cuda.synchronize()
    ref = f64(x) @ f64(w).T + (f64(r) if res else 0.0)
    check_out(host64(y), ref, "linear", bf16_out=True, layer=True)
    ctx.close()


SMALL = [
    # B, Hq, Hkv, D, L, b, a, layers, rope
    (2, 4, 2, 64, 300, 64, 64, 2, True),
    (1, 8, 2, 128, 700, 200, 200, 2, True),
    (1, 2, 1, 64, 512, 128, 128, 1, False),     # tiny's shapes (no RoPE)
    (1, 8, 8, 128, 333, 100, 37, 1, True),      # MHA, a < b, ragged tail
]


def run_layer_staged(layer: AttentionLayers, x):
    """One forward pass of a one-layer stack, keeping each stage's actual
    output as stored in bf16 (copied on the stream as the stages run, before
    RoPE rotates k in place): h, the q/k/v projection (un-rotated), the
    attention output and the layer output."""
    saved = {}

    def mark(name):
        if name == "rmsnorm":
            saved["h"] = layer.h.clone()
        elif name == "qkv_proj":
            saved["qkv"] = layer.qkv.clone()
        elif name == "phase1":
            saved["attn"] = layer.attn.clone()
    out = layer.forward(x, mark).clone()
    torch.cuda.synchronize()
    return {k: host64(v) for k, v in saved.items()}, out


def check_layer_stages(st, x64, lw, Hq, Hkv, D, b, a, base, rope, rows=None, what="layer"):
    """Each stage of one layer against the oracle fed that stage's actual
    input (the GPU's bf16 output of the stage before), so every stage has
    the bound of its own arithmetic: RMSNorm and the q/k/v projection; the
    attention (Q and K rotated exactly and rounded once, as the GPU does bit
    for bit) with the bf16-weight compute term; the output projection with
    the residual.  ``rows``: check only these context rows (all if None)."""
    B = x64.shape[0]
    L = x64.shape[1]
    H = Hq * D
    w64 = {k: f64(v) for k, v in lw.items()}
    sel = np.arange(L) if rows is None else np.asarray(rows)
    # RMSNorm (one rounding of an fp32 result)
    h_ref = so.rmsnorm(x64[:, sel], w64["gamma"], RMS_EPS)
    h_got = st["h"].reshape(B, L, H)[:, sel]
    assert (np.abs(h_got - h_ref) <= np.abs(h_ref) * 2.0 ** -8 + 1e-6).all(), f"{what} rmsnorm"
    # q/k/v projection of the GPU's h
    wqkv = np.concatenate([w64["wq"], w64["wk"], w64["wv"]], axis=0)
    hg = st["h"].reshape(B, L, H)
    p_ref = hg[:, sel] @ wqkv.T
    p_got = st["qkv"].reshape(B, L, -1)[:, sel]
    check_out(p_got, p_ref, f"{what} qkv", bf16_out=True, layer=True)
    # attention over the GPU's q/k/v (rotated exactly, rounded once)
    qkv = st["qkv"].reshape(B, L, Hq + 2 * Hkv, D).transpose(0, 2, 1, 3)
    q, k, v = qkv[:, :Hq][:, :, sel], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]
    if rope:
        q = so.round_bf16(so.rope(q, sel, base))
        k = so.round_bf16(so.rope(k, np.arange(L), base))
    g = Hq // Hkv
    scale = 1 / math.sqrt(D)
    A_ref = np.zeros((B, Hq, sel.size, D))
    A_w = np.zeros_like(A_ref)
    for bb in range(B):
        for h in range(Hq):
            vw = np.concatenate([v[bb, h // g], np.abs(v[bb, h // g])], axis=-1)
            o, _ = so.phase1_rows(q[bb, h], sel, k[bb, h // g], vw, b, a if b < L else 0,
                                  scale)
            A_ref[bb, h], A_w[bb, h] = o[:, :D], o[:, D:]
    A_got = st["attn"].reshape(B, L, Hq, D).transpose(0, 2, 1, 3)[:, :, sel]
    check_out(A_got, A_ref, f"{what} attention", bf16_out=True, wabs=A_w)
    # output projection + residual of the GPU's attention output
    o_ref = so.layer_output(x64[:, sel], A_got, w64, store_bf16=False)
    return o_ref


SMALL = [
    # B, Hq, Hkv, D, L, b, a, layers, rope
    (2, 4, 2, 64, 300, 64, 64, 2, True),
    (1, 8, 2, 128, 700, 200, 200, 2, True),
    (1, 2, 1, 64, 512, 128, 128, 1, False),     # tiny's shapes (no RoPE)
    (1, 8, 8, 128, 333, 100, 37, 1, True),      # MHA, a < b, ragged tail
]


@pytest.mark.parametrize("case", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_layer_stack_parity(case):
    """Every stage of every layer of a stack against the oracle fed that
    stage's actual input (the GPU's output of the stage before, as stored in
    bf16), element by element; and the stack equal, bit for bit, to its
    layers chained one at a time.  (The oracle pins the stack itself against
    the host-by-host encoding; comparing a whole stack, or a whole layer,
    here would add bf16 rounding flips of intermediate tensors to the
    bound.)"""
    B, Hq, Hkv, D, L, b, a, n_layers, rope = case
    log(f"layer stack {case}")
    w = Workload("t", B, Hq, Hkv, D, L, b, 0, 0, 71, 1.0, rope, anchor=a)
    inp = layer_inputs(w, n_layers)
    layers = [{k: to_dev(v) for k, v in lw.items()} for lw in inp["layers"]]
    x = to_dev(inp["x"])
    whole = AttentionLayers(B, Hq, Hkv, D, L, b, layers, anchor=a, rope=rope, eps=RMS_EPS)
    out = whole.forward(x).clone()
    cur = x
    for i, lw in enumerate(inp["layers"]):
        one = AttentionLayers(B, Hq, Hkv, D, L, b, [layers[i]], anchor=a, rope=rope, eps=RMS_EPS)
        stages, nxt = run_layer_staged(one, cur)
        ref = check_layer_stages(stages, host64(cur), lw, Hq, Hkv, D, b, a, w.base, rope,
                                 what=f"layer {i}")
        check_out(host64(nxt), ref, f"layer {i} out", bf16_out=True, layer=True)
        cur = nxt
    assert torch.equal(out, cur), "stack differs from its layers chained"


@pytest.mark.timeout(1500)
def test_layer_8b_16k_sampled_rows():
    """One layer at the Llama-3.1-8B shape, 16K context (4 blocks of 4096):
    every row of the output is finite; every stage of rows of blocks 1 and 4
    (edges plus seeded random rows) matches the oracle fed the stage's
    actual input."""
    w = WORKLOADS["llama8b-16k"]
    log("8b-16k layer: inputs")
    inp = layer_inputs(w, 1)
    lw = inp["layers"][0]
    layers = [{k: to_dev(v) for k, v in lw.items()}]
    st = AttentionLayers(w.B, w.Hq, w.Hkv, w.D, w.L, w.b, layers, rope=True, base=w.base,
                         eps=RMS_EPS)
    log("8b-16k layer: GPU pass")
    stages, out = run_layer_staged(st, to_dev(inp["x"]))
    assert bool(torch.isfinite(out).all())
    rng = np.random.default_rng(5)
    blocks = so.blocks(w.L, w.b)
    chk = []
    for i in (0, len(blocks) - 1):
        s, e = blocks[i]
        chk += [s, s + 1, e - 2, e - 1] + (s + rng.choice(e - s, 12, replace=False)).tolist()
    chk = np.unique(np.array(chk))
    log("8b-16k layer: oracle")
    ref = check_layer_stages(stages, f64(inp["x"]), lw, w.Hq, w.Hkv, w.D, w.b, w.a, w.base,
                             True, rows=chk, what="8b-16k layer")
    got = host64(out[0].index_select(0, torch.from_numpy(chk).cuda()))[None]
    e = check_out(got, ref, "8b-16k layer out", bf16_out=True, layer=True)
    log(f"8b-16k layer: worst max-abs {e[0]:.3e} over {chk.size} rows")
