"""Pins of the oracle's attention layer around Phase 1: the layer against a
textbook Llama attention block written with torch's own RMSNorm, linear,
complex-number RoPE and causal SDPA (all float64), and the one-device
formulation (anchor K/V = block 1's rows at every layer) against the pages'
host-by-host formulation ([anchor ; block] through every layer)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.star_oracle as so


def weights(seed, Hq, Hkv, D, scale=None):
    rng = np.random.default_rng(seed)
    H = Hq * D
    s = 1 / math.sqrt(H) if scale is None else scale
    return {"gamma": 1 + 0.1 * rng.standard_normal(H),
            "wq": rng.standard_normal((Hq * D, H)) * s,
            "wk": rng.standard_normal((Hkv * D, H)) * s,
            "wv": rng.standard_normal((Hkv * D, H)) * s,
            "wo": rng.standard_normal((H, Hq * D)) * s}


def torch_layer(x, w, Hq, Hkv, D, base, eps):
    """A dense causal Llama attention block in torch float64."""
    xt = torch.from_numpy(x)
    B, L, H = xt.shape
    h = F.rms_norm(xt, (H,), torch.from_numpy(w["gamma"]), eps)
    q = F.linear(h, torch.from_numpy(w["wq"])).view(B, L, Hq, D).transpose(1, 2)
    k = F.linear(h, torch.from_numpy(w["wk"])).view(B, L, Hkv, D).transpose(1, 2)
    v = F.linear(h, torch.from_numpy(w["wv"])).view(B, L, Hkv, D).transpose(1, 2)
    # RoPE as a complex multiply of the pairs (j, j + D/2)
    j = torch.arange(D // 2, dtype=torch.float64)
    ang = torch.arange(L, dtype=torch.float64)[:, None] * base ** (-2 * j / D)[None]
    rot = torch.polar(torch.ones_like(ang), ang)
    def rope_c(t):
        z = torch.complex(t[..., :D // 2], t[..., D // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)
    q, k = rope_c(q), rope_c(k)
    g = Hq // Hkv
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    o = o.transpose(1, 2).reshape(B, L, Hq * D)
    return (xt + F.linear(o, torch.from_numpy(w["wo"]))).numpy()


@pytest.mark.parametrize("Hq,Hkv,D,L", [(4, 2, 16, 37), (2, 2, 8, 20), (6, 1, 16, 25)])
def test_single_block_layer_is_the_textbook_block(Hq, Hkv, D, L):
    x = np.random.default_rng(1).standard_normal((2, L, Hq * D))
    w = weights(2, Hq, Hkv, D)
    got, _, _ = so.attention_layer_phase1(x, w, Hq, Hkv, D, b=L, a=L, base=1e4, eps=1e-5,
                                          store_bf16=False)
    ref = torch_layer(x, w, Hq, Hkv, D, 1e4, 1e-5)
    assert np.allclose(got, ref, atol=1e-10)


def test_rmsnorm_closed_form_and_torch():
    x = np.random.default_rng(3).standard_normal((3, 5, 12))
    g = np.random.default_rng(4).standard_normal(12)
    ref = F.rms_norm(torch.from_numpy(x), (12,), torch.from_numpy(g), 1e-5).numpy()
    assert np.allclose(so.rmsnorm(x, g, 1e-5), ref, atol=1e-14)
    c = np.full((1, 8), -3.0)
    assert np.allclose(so.rmsnorm(c, np.ones(8), 0.0), -1.0)
    assert np.allclose(so.rmsnorm(c, np.ones(8), 7.0), -3.0 / 4.0)   # sqrt(9 + 7) = 4


def test_zero_output_projection_is_the_residual():
    x = np.random.default_rng(5).standard_normal((1, 30, 32))
    w = weights(6, 4, 2, 8)
    w["wo"] = np.zeros_like(w["wo"])
    out, _, _ = so.attention_layer_phase1(x, w, 4, 2, 8, b=10, a=10, base=1e4, eps=1e-5,
                                          store_bf16=False)
    assert np.array_equal(out, x)


@pytest.mark.parametrize("n_layers,L,b,a", [(1, 40, 16, 16), (2, 40, 16, 16), (3, 50, 16, 16),
                                            (2, 45, 20, 7), (2, 40, 16, 0)])
def test_one_device_stack_equals_host_by_host(n_layers, L, b, a):
    """Through any number of layers, block i's rows computed with the anchor
    K/V read from block 1's rows equal the pages' host-by-host encoding of
    [anchor ; block i]: the anchor is causal and first, so its hidden states
    (and K/V) equal host 1's at every layer."""
    Hq, Hkv, D = 4, 2, 8
    x = np.random.default_rng(7).standard_normal((1, L, Hq * D))
    layers = [weights(10 + i, Hq, Hkv, D, scale=0.5) for i in range(n_layers)]
    one = so.star_context_layers(x, layers, Hq, Hkv, D, b, a, 1e4, 1e-5, store_bf16=False)
    per = so.star_context_per_host(x, layers, Hq, Hkv, D, b, a, 1e4, 1e-5, store_bf16=False)
    assert np.allclose(one, per, atol=1e-10)


def test_host_by_host_without_the_anchor_differs():
    """Planted mistake: dropping the anchor from the hosts' sequences changes
    every block after the first (so the pin above is not vacuous)."""
    Hq, Hkv, D, L, b = 4, 2, 8, 40, 16
    x = np.random.default_rng(8).standard_normal((1, L, Hq * D))
    layers = [weights(20 + i, Hq, Hkv, D, scale=0.5) for i in range(2)]
    one = so.star_context_layers(x, layers, Hq, Hkv, D, b, b, 1e4, 1e-5, store_bf16=False)
    wrong = so.star_context_per_host(x, layers, Hq, Hkv, D, b, 0, 1e4, 1e-5, store_bf16=False)
    assert np.allclose(one[:, :b], wrong[:, :b], atol=1e-10)
    assert np.abs(one[:, b:] - wrong[:, b:]).max() > 1e-3
