"""The no-allocation decode step (star_decode_step_noalloc) against the
workspace one (star_decode_step), through the C ABI: two calls in a row on
one GPU, the second with a smaller problem (other heads, head dim and
partition count), so the second reuses the scratch the first filled.  The
two entry points share their kernels and the partials' layout, so the
outputs must be the same bits; both are also checked against the oracle."""
import math

import numpy as np
import pytest
import torch

import block_sparse_amd as sa
import oracle.star_oracle as so
from block_sparse_amd.pipeline import StarAttentionStep
from gpu_util import check_lse, check_out, f64, host64, rand_tensor, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, D, L, b, splits   (first call, then a smaller one)
    (2, 32, 8, 128, 3000, 1024, 4),
    (1, 8, 2, 64, 500, 128, 2),
]


def one_case(B, Hq, Hkv, D, L, b, splits, seed):
    base = 500000.0
    q = rand_tensor(seed, 0, B, Hq, L, D)
    k = rand_tensor(seed, 1, B, Hkv, L, D)
    v = rand_tensor(seed, 2, B, Hkv, L, D)
    qd, kd, vd = (rand_tensor(seed, t, B, H, 1, D) for t, H in ((6, Hq), (7, Hkv), (8, Hkv)))
    st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, 1, base=base, splits_decode=splits)
    st.load_context(to_dev(v))
    st.rope_context(to_dev(q), to_dev(k))
    pos = L
    offs = list(range(0, L, b)) + [pos + 1]
    dq, dk, dv = to_dev(qd), to_dev(kd), to_dev(vd)
    o_ref = torch.empty((B, Hq, 1, D), dtype=torch.float32, device="cuda")
    l_ref = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    sa.decode_step(dq, dk, dv, st.kc, st.vc, pos, pos, offs, splits, st.op_d, st.lp_d, o_ref,
                   l_ref, base=base)
    o_na = torch.full((B, Hq, 1, D), float("nan"), dtype=torch.float32, device="cuda")
    l_na = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    sa.decode_step_noalloc(dq, dk, dv, st.kc, st.vc, pos, pos, offs, splits, o_na, l_na,
                           base=base)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref), "differs from star_decode_step"
    rot = lambda x, p: so.round_bf16(so.rope(x, p, base))
    K = np.concatenate([rot(f64(k), np.arange(L)), rot(f64(kd), [L])], axis=2)
    V = np.concatenate([f64(v), f64(vd)], axis=2)
    qr = rot(f64(qd), [L])
    g = Hq // Hkv
    for bb in range(B):
        for h in range(Hq):
            ro, rl, _, _ = so.phase2(qr[bb, h], np.array([L]), K[bb, h // g], V[bb, h // g],
                                     so.partitions(L, b, L + 1), 1 / math.sqrt(D))
            check_out(host64(o_na)[bb, h], ro, f"no-alloc O b{bb} h{h}")
            check_lse(host64(l_na)[bb, h:h + 1], rl, f"no-alloc LSE b{bb} h{h}")


def test_noalloc_decode_step_two_calls():
    print("no-alloc decode step: two calls, the second smaller", flush=True)
    for i, case in enumerate(CASES):
        one_case(*case, seed=90 + i)


def test_noalloc_rejects_partials_beyond_the_scratch():
    """P * splits * B * Hq rows of D + 1 floats beyond the array: refused
    on the host with STAR_ERR_UNSUPPORTED, nothing launched."""
    B, Hq, Hkv, D, b = 1, 64, 8, 128, 64
    L = 128 * b
    st = StarAttentionStep(B, Hq, Hkv, D, L, b, 0, 1, splits_decode=1)
    qd, kd, vd = (torch.zeros((B, H, 1, D), dtype=torch.bfloat16, device="cuda")
                  for H in (Hq, Hkv, Hkv))
    o = torch.empty((B, Hq, 1, D), dtype=torch.float32, device="cuda")
    offs = list(range(0, L, b)) + [L + 1]
    with pytest.raises(sa.StarError) as e:
        sa.decode_step_noalloc(qd, kd, vd, st.kc, st.vc, L, L, offs, 8, o)
    assert e.value.status == -5
