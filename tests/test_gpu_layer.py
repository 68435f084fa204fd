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


def test_rmsnorm_parity():
    x = rand_tensor(61, 0, 1, 1, 300, 4096)[0, 0]
    g = rand_tensor(61, 1, 1, 1, 1, 4096, 0.5)[0, 0, 0]
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
    check_out(host64(y), ref, "linear", bf16_out=True)
    ctx.close()


SMALL = [
    # B, Hq, Hkv, D, L, b, a, layers, rope
    (2, 4, 2, 64, 300, 64, 64, 2, True),
    (1, 8, 2, 128, 700, 200, 200, 2, True),
    (1, 2, 1, 64, 512, 128, 128, 1, False),     # tiny's shapes (no RoPE)
    (1, 8, 8, 128, 333, 100, 37, 1, True),      # MHA, a < b, ragged tail
]


@pytest.mark.parametrize("case", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_layer_stack_parity(case):
    """Every layer of a stack against the oracle fed that layer's actual
    input (the GPU output of the layer before, as stored in bf16), element
    by element; and the stack equal, bit for bit, to its layers chained one
    at a time.  (The oracle pins the stack itself against the host-by-host
    encoding; comparing a whole stack here would add one bf16 rounding flip
    of the residual stream per layer to the bound.)"""
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
        nxt = one.forward(cur).clone()
        torch.cuda.synchronize()
        ref, _, _ = so.attention_layer_phase1(host64(cur), {k: f64(v) for k, v in lw.items()},
                                              Hq, Hkv, D, b, a, w.base, RMS_EPS, rope_on=rope,
                                              round_output=False)
        check_out(host64(nxt), ref, f"layer {i} out", bf16_out=True)
        cur = nxt
    assert torch.equal(out, cur), "stack differs from its layers chained"


@pytest.mark.timeout(1500)
def test_layer_8b_16k_sampled_rows():
    """One layer at the Llama-3.1-8B shape, 16K context (4 blocks of 4096):
    every row of the output is finite; rows of blocks 1 and 4 (edges plus
    seeded random rows) match the oracle, which computes them from the
    projections of just the anchor and those blocks (projections are
    row-wise)."""
    w = WORKLOADS["llama8b-16k"]
    log("8b-16k layer: inputs")
    inp = layer_inputs(w, 1)
    lw = inp["layers"][0]
    layers = [{k: to_dev(v) for k, v in lw.items()}]
    st = AttentionLayers(w.B, w.Hq, w.Hkv, w.D, w.L, w.b, layers, rope=True, base=w.base,
                         eps=RMS_EPS)
    log("8b-16k layer: GPU pass")
    out = st.forward(to_dev(inp["x"]))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rng = np.random.default_rng(5)
    blocks = so.blocks(w.L, w.b)
    chk = []
    for i in (0, len(blocks) - 1):
        s, e = blocks[i]
        chk += [s, s + 1, e - 2, e - 1] + (s + rng.choice(e - s, 12, replace=False)).tolist()
    chk = np.unique(np.array(chk))
    # tokens whose projections the checked rows need: the anchor and the checked blocks
    s_last, e_last = blocks[-1]
    need = np.unique(np.concatenate([np.arange(0, w.b), np.arange(s_last, e_last)]))
    log("8b-16k layer: oracle")
    x64 = f64(inp["x"])[0]
    w64 = {k: f64(v) for k, v in lw.items()}
    q, k, v = so.layer_projections(x64[need][None], w64, w.Hq, w.Hkv, w.D, RMS_EPS)
    q = so.round_bf16(so.rope(q, need, w.base))
    k = so.round_bf16(so.rope(k, need, w.base))
    K = np.zeros((w.Hkv, w.L, w.D))
    V = np.zeros((w.Hkv, w.L, w.D))
    K[:, need], V[:, need] = k[0], v[0]
    sel = np.searchsorted(need, chk)
    O = np.zeros((1, w.Hq, chk.size, w.D))
    g = w.g
    for h in range(w.Hq):
        o, _ = so.phase1_rows(q[0, h, sel], chk, K[h // g], V[h // g], w.b, w.a,
                              1 / math.sqrt(w.D))
        O[0, h] = so.round_bf16(o)
    ref = so.layer_output(x64[chk][None], O, w64, store_bf16=False)[0]
    got = host64(out[0].index_select(0, torch.from_numpy(chk).cuda()))
    e = check_out(got, ref, "8b-16k layer out", bf16_out=True)
    log(f"8b-16k layer: worst max-abs {e[0]:.3e} over {chk.size} rows")
