"""The seeded input generator: determinism, slicing, bf16 rounding."""
import numpy as np
import torch

from workloads import (CHUNK_ROWS, L8B_128K, TINY, WORKLOADS, bf16_bits_to_f32,
                       draw_rows, draw_tensor, f32_to_bf16_bits)


def test_bf16_rne_matches_torch_and_ties():
    # exact ties round to even; torch's float32 -> bfloat16 cast is RNE
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 3.0e38,
                  np.inf, -np.inf, 1e-40, -0.0, 65504.0], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80 and bits[2] == 0x3F82
    assert bits[3] == 0xBF80
    r = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 100
    x = np.concatenate([x, r])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    nan = f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(bf16_bits_to_f32(nan))[0]


def test_widen_is_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    fin = np.isfinite(f)
    assert np.array_equal(f32_to_bf16_bits(f[fin]), bits[fin])


def test_draws_deterministic_and_sliceable():
    S, D = 2 * CHUNK_ROWS + 100, 16
    full = draw_tensor(7, 1, 1, 2, S, D, 1.0, as_bf16=False)
    again = draw_tensor(7, 1, 1, 2, S, D, 1.0, as_bf16=False)
    assert np.array_equal(full, again)
    part = draw_rows(7, 1, 0, 1, S, D, 1.0, CHUNK_ROWS - 5, CHUNK_ROWS + 300)
    assert np.array_equal(part, full[0, 1, CHUNK_ROWS - 5:CHUNK_ROWS + 300])
    other = draw_tensor(7, 2, 1, 2, S, D, 1.0, as_bf16=False)
    assert not np.array_equal(full, other)
    assert abs(full.std() - 1.0) < 0.02 and abs(full.mean()) < 0.02


def test_tiny_scale_and_bf16():
    t = draw_tensor(TINY.seed, 0, 1, 1, 512, 64, TINY.scale, as_bf16=False)
    assert abs(t.std() - 0.125) < 0.005
    b = draw_tensor(TINY.seed, 0, 1, 1, 512, 64, TINY.scale, as_bf16=True)
    assert np.array_equal(b, f32_to_bf16_bits(t))


def test_workload_table():
    assert [w.name for w in WORKLOADS.values()] == [
        "tiny", "llama8b-16k", "llama8b-128k", "llama70b-64k", "llama8b-1m"]
    w = L8B_128K
    assert (w.n_blocks, w.g, w.a, w.cache_len) == (8, 4, 16384, 131072 + 64 + 128)


def test_token_ids_seeded_and_zipf_shaped():
    from workloads import VOCAB, token_ids
    a, b = token_ids(2, 2, 4096), token_ids(2, 2, 4096)
    assert a.dtype == np.int32 and a.shape == (2, 4096)
    assert np.array_equal(a, b) and not np.array_equal(a[0], a[1])
    assert a.min() >= 0 and a.max() < VOCAB
    # a heavy head and a long tail: the most frequent id is far above the
    # median count, and many ids occur once
    _, counts = np.unique(a[0], return_counts=True)
    assert counts.max() > 20 * np.median(counts) and (counts == 1).sum() > 500


def test_anchor_positions_precede_their_block():
    from workloads import anchor_positions
    L, b, a = 1000, 200, 150
    pos = anchor_positions(3, L, b, a)
    assert len(pos) == 5 and np.array_equal(pos[0], np.arange(a))
    for i in range(1, 5):
        p = pos[i]
        assert p.size == a and np.all(np.diff(p) > 0) and p.min() >= 0 and p.max() < i * b
    assert all(np.array_equal(x, y) for x, y in zip(pos, anchor_positions(3, L, b, a)))


def test_group_inputs_are_the_workload_slices():
    """One (batch, KV head) group's tensors equal the matching slices of the
    whole workload's draws: KV head kvh and query heads kvh*g .. kvh*g+g-1."""
    import dataclasses
    from workloads import group_inputs, inputs
    w = dataclasses.replace(WORKLOADS["llama8b-16k"], name="small", B=2, Hq=8, Hkv=2, L=4100,
                            b=1024, Lq=5, T=3)
    full = inputs(w)
    for b in range(w.B):
        for kvh in range(w.Hkv):
            grp = group_inputs(w, b, kvh)
            for name, t in grp.items():
                hs = slice(kvh * w.g, (kvh + 1) * w.g) if name.startswith("q") else slice(kvh, kvh + 1)
                assert np.array_equal(t, full[name][b:b + 1, hs]), (name, b, kvh)
