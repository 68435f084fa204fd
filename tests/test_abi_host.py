"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and rejects invalid arguments before anything is enqueued.
No call here reaches a kernel launch, so this runs without a GPU."""
import ctypes
import os
import re

import pytest

from block_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "star_attn.h")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced on the host


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(star_\w+)\s*\(", text, re.M)))


def T(B=1, H=2, S=64, D=64, dtype=0, data=FAKE, strides=None):
    if strides is None:
        strides = (H * S * D, S * D, D)
    return _lib.StarTensor(data, dtype, 0, B, H, S, D, *strides)


@pytest.fixture(scope="module")
def lib():
    """The built library; built here (hipcc cross-compiles without a GPU)
    when it is missing, and a failed build fails the tests."""
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert set(syms) == set(_lib.EXPORTS)
    for s in syms:
        assert hasattr(lib, s), s
    assert lib.star_abi_version() == 500


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.star_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.star_status_string(-99)


def p1(lib, q, k, v, o, b=16, a=16, scale=0.125, lse=None, sched=None):
    return lib.star_phase1_blocklocal(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), b, a,
                                      scale, ctypes.byref(o), lse, sched, None)


def test_phase1_validation(lib):
    ok = dict(B=1, H=2, S=64, D=64)
    q, k, v, o = T(**ok), T(B=1, H=1, S=64, D=64), T(B=1, H=1, S=64, D=64), T(**ok)
    assert lib.star_phase1_blocklocal(None, ctypes.byref(k), ctypes.byref(v), 16, 16, 0.1,
                                      ctypes.byref(o), None, None, None) == -1
    assert p1(lib, T(**ok, data=0), k, v, o) == -1
    assert p1(lib, T(**ok, dtype=7), k, v, o) == -3
    assert p1(lib, q, k, v, T(**ok, dtype=1)) == -3            # O must be bf16
    assert p1(lib, T(**ok, data=FAKE + 2), k, v, o) == -4
    assert p1(lib, T(**ok, strides=(8192, 4096, 63)), k, v, o) == -4
    assert p1(lib, T(B=1, H=2, S=64, D=96), T(B=1, H=1, S=64, D=96),
              T(B=1, H=1, S=64, D=96), T(B=1, H=2, S=64, D=96)) == -5
    assert p1(lib, T(B=1, H=3, S=64, D=64), T(B=1, H=2, S=64, D=64),
              T(B=1, H=2, S=64, D=64), T(B=1, H=3, S=64, D=64)) == -2
    assert p1(lib, T(B=1, H=32, S=64, D=64), k, v, T(B=1, H=32, S=64, D=64)) == -5  # g > 16
    assert p1(lib, q, k, v, o, b=0) == -2
    assert p1(lib, q, k, v, o, b=16, a=17) == -2
    assert p1(lib, q, k, v, o, a=-1) == -2
    assert p1(lib, q, k, v, o, scale=float("nan")) == -2
    assert p1(lib, q, T(B=1, H=1, S=63, D=64), T(B=1, H=1, S=63, D=64), o) == -2
    assert p1(lib, q, k, v, T(B=1, H=2, S=32, D=64)) == -2
    assert p1(lib, q, k, v, o, lse=ctypes.c_void_p(FAKE + 1)) == -4
    assert p1(lib, q, k, v, o, sched=ctypes.c_void_p(FAKE + 2)) == -4   # int32 workspace
    # empty context: nothing to do, nothing enqueued
    z = dict(B=1, S=0, D=64)
    assert p1(lib, T(H=2, **z), T(H=1, **z), T(H=1, **z), T(H=2, **z)) == 0


def test_phase1_rope_validation(lib):
    """The fused-RoPE Phase 1 shares the Phase-1 checks, requires a finite
    base above 1 and serves only bf16 with D = 128 (no launch here)."""
    ok = dict(B=1, H=2, S=64, D=128)
    q, k, v, o = T(**ok), T(B=1, H=1, S=64, D=128), T(B=1, H=1, S=64, D=128), T(**ok)
    r = lambda q=q, k=k, v=v, o=o, b=16, a=16, base=500000.0, scale=0.1: lib.star_phase1_rope(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), b, a, base, scale,
        ctypes.byref(o), None, None, None)
    assert lib.star_phase1_rope(None, ctypes.byref(k), ctypes.byref(v), 16, 16, 500000.0, 0.1,
                                ctypes.byref(o), None, None, None) == -1
    assert lib.star_phase1_rope(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 16, 16,
                                500000.0, 0.1, ctypes.byref(o), None, ctypes.c_void_p(FAKE + 1),
                                None) == -4
    assert r(base=1.0) == -2
    assert r(base=float("nan")) == -2
    assert r(b=16, a=17) == -2
    assert r(scale=-1.0) == -2
    small = dict(B=1, S=64, D=64)
    assert r(q=T(H=2, **small), k=T(H=1, **small), v=T(H=1, **small), o=T(H=2, **small)) == -5
    assert r(q=T(**ok, dtype=1), k=T(B=1, H=1, S=64, D=128, dtype=1),
             v=T(B=1, H=1, S=64, D=128, dtype=1)) == -5            # fp32 inputs
    z = dict(B=1, S=0, D=128)
    assert r(q=T(H=2, **z), k=T(H=1, **z), v=T(H=1, **z), o=T(H=2, **z)) == 0


def p2(lib, q, kc, vc, offs, P=None, splits=1, qpos=0, scale=0.1, op=FAKE, lp=FAKE):
    P = len(offs) - 1 if P is None else P
    arr = (ctypes.c_int64 * len(offs))(*offs)
    return lib.star_phase2_partial(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(vc), arr,
                                   P, splits, qpos, scale, op, lp, None)


def test_phase2_validation(lib):
    q = T(B=1, H=4, S=3, D=128)
    kc = T(B=1, H=1, S=100, D=128)
    vc = T(B=1, H=1, S=100, D=128)
    assert p2(lib, q, kc, vc, [0, 50, 100], op=None) == -1
    assert p2(lib, q, kc, vc, [0, 50, 40]) == -2             # non-monotone
    assert p2(lib, q, kc, vc, [0, 50, 101]) == -2            # past the cache
    assert p2(lib, q, kc, vc, [-1, 50, 100]) == -2
    assert p2(lib, q, kc, vc, [0, 100], splits=0) == -2
    assert p2(lib, q, kc, vc, [0, 100], splits=1025) == -2
    assert p2(lib, q, kc, vc, list(range(0, 130)), P=129) == -2
    assert p2(lib, q, kc, vc, [0, 100], qpos=-1) == -2
    assert p2(lib, q, kc, vc, [0, 100], op=FAKE + 4) == -4
    assert p2(lib, q, T(B=1, H=1, S=100, D=128, dtype=1), vc, [0, 100]) == -3
    assert p2(lib, T(B=1, H=4, S=0, D=128), kc, vc, [0, 100]) == 0


def test_merge_rope_append_validation(lib):
    o = T(B=1, H=2, S=4, D=64)

    def m(n, oo=o, op=FAKE, lp=FAKE, shape=None):
        B, H, S, D = shape or (oo.B, oo.H, oo.S, oo.D)
        return lib.star_lse_merge(op, lp, n, B, H, S, D, ctypes.byref(oo), None, None)
    assert m(1, op=None) == -1
    assert m(0) == -2
    assert m(70000) == -2
    assert m(2, oo=T(B=1, H=2, S=4, D=80)) == -5
    assert m(2, op=FAKE + 8) == -4
    assert m(2, oo=T(B=1, H=2, S=0, D=64)) == 0
    # the sizes given must be the output's
    assert m(2, shape=(2, 2, 4, 64)) == -2
    assert m(2, shape=(1, 1, 4, 64)) == -2
    assert m(2, shape=(1, 2, 5, 64)) == -2
    assert m(2, shape=(1, 2, 4, 128)) == -2
    x = T(B=1, H=2, S=8, D=128)
    r = lambda a, b, pos=None, pos0=0, base=5e5: lib.star_rope_apply(
        ctypes.byref(a), ctypes.byref(b), pos, pos0, base, None)
    assert r(x, T(B=1, H=2, S=8, D=128, dtype=1)) == -3
    assert r(x, T(B=1, H=2, S=9, D=128)) == -2
    assert r(T(B=1, H=2, S=8, D=72), T(B=1, H=2, S=8, D=72)) == -5
    assert r(x, x, base=1.0) == -2
    assert r(x, x, pos0=-3) == -2
    assert r(T(B=1, H=2, S=0, D=128), T(B=1, H=2, S=0, D=128)) == 0
    kn, vn = T(B=1, H=2, S=3, D=128), T(B=1, H=2, S=3, D=128)
    kc, vc = T(B=1, H=2, S=10, D=128), T(B=1, H=2, S=10, D=128)
    a = lambda slot, kk=kc: lib.star_kv_append(ctypes.byref(kn), ctypes.byref(vn),
                                               ctypes.byref(kk), ctypes.byref(vc), slot, 5,
                                               5e5, 1, None)
    assert a(8) == -2
    assert a(-1) == -2
    assert a(0, kk=T(B=1, H=2, S=11, D=128)) == -2
    qn, qo = T(B=1, H=8, S=3, D=128), T(B=1, H=8, S=3, D=128)
    dp = lambda q_in, q_o, slot=0: lib.star_decode_prepare(
        ctypes.byref(q_in), ctypes.byref(q_o), ctypes.byref(kn), ctypes.byref(vn),
        ctypes.byref(kc), ctypes.byref(vc), slot, 5, 5e5, 1, None)
    assert dp(qn, T(B=1, H=8, S=4, D=128)) == -2
    assert dp(T(B=1, H=8, S=2, D=128), T(B=1, H=8, S=2, D=128)) == -2
    assert dp(qn, qo, slot=8) == -2
    assert dp(T(B=1, H=8, S=3, D=128, data=0), qo) == -1


def test_phase1_prefix_validation(lib):
    ok = dict(B=1, H=2, S=64, D=64)
    q, o = T(**ok), T(**ok)
    k, v = T(B=1, H=1, S=64, D=64), T(B=1, H=1, S=64, D=64)
    pk, pv = T(B=1, H=1, S=10, D=64), T(B=1, H=1, S=10, D=64)

    def pp(pk=pk, pv=pv, st=(0, 0, 0, 0), ln=(0, 5, 5, 10), n=None, b=16, q=q, sched=None):
        n = len(st) if n is None else n
        sa = (ctypes.c_int64 * len(st))(*st)
        la = (ctypes.c_int64 * len(ln))(*ln)
        return lib.star_phase1_prefix(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                      ctypes.byref(pk), ctypes.byref(pv), sa, la, n, b, 0.1,
                                      ctypes.byref(o), None, sched, None)
    assert pp(ln=(0, 5, 5, 11)) == -2                  # past the prefix rows
    assert pp(st=(0, 0, 6, 0)) == -2                   # 6 + 5 > 10
    assert pp(st=(0, -1, 0, 0)) == -2
    assert pp(ln=(0, -1, 0, 0)) == -2
    assert pp(n=3) == -2                               # table size != ceil(L/b)
    assert pp(pk=T(B=1, H=1, S=10, D=64, dtype=1)) == -3
    assert pp(pv=T(B=1, H=1, S=11, D=64)) == -2        # pk/pv rows differ
    assert pp(pk=T(B=1, H=2, S=10, D=64), pv=T(B=1, H=2, S=10, D=64)) == -2
    assert pp(pk=T(B=1, H=1, S=10, D=64, data=FAKE + 8)) == -4
    assert pp(sched=ctypes.c_void_p(FAKE + 3)) == -4
    st = [0] * 129
    assert pp(st=st, ln=st, b=1, q=T(B=1, H=2, S=129, D=64)) == -2   # k has 64 rows
    assert lib.star_phase1_prefix(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                  ctypes.byref(pk), ctypes.byref(pv), None, None, 4, 16, 0.1,
                                  ctypes.byref(o), None, None, None) == -1
    z = dict(B=1, S=0, D=64)
    assert lib.star_phase1_prefix(ctypes.byref(T(H=2, **z)), ctypes.byref(T(H=1, **z)),
                                  ctypes.byref(T(H=1, **z)), ctypes.byref(pk), ctypes.byref(pv),
                                  None, None, 0, 16, 0.1, ctypes.byref(T(H=2, **z)), None,
                                  None, None) == 0


def test_phase1_prefix_too_many_blocks(lib):
    L, b = 1290, 10                                    # 129 blocks
    q, o = T(B=1, H=2, S=L, D=64), T(B=1, H=2, S=L, D=64)
    k, v = T(B=1, H=1, S=L, D=64), T(B=1, H=1, S=L, D=64)
    z = (ctypes.c_int64 * 129)(*([0] * 129))
    assert lib.star_phase1_prefix(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                  ctypes.byref(k), ctypes.byref(v), z, z, 129, b, 0.1,
                                  ctypes.byref(o), None, None, None) == -5


def test_gather_validation(lib):
    src, dst = T(B=1, H=2, S=50, D=128), T(B=1, H=2, S=7, D=128)
    g = lambda s=src, d=dst, rows=FAKE: lib.star_gather_rows(ctypes.byref(s), rows,
                                                             ctypes.byref(d), None)
    assert g(rows=None) == -1
    assert g(d=T(B=1, H=2, S=7, D=128, dtype=1)) == -3
    assert g(d=T(B=1, H=3, S=7, D=128)) == -2
    assert g(d=T(B=1, H=2, S=7, D=64)) == -2
    assert g(d=T(B=1, H=2, S=0, D=128), rows=None) == 0


def test_stream_read_validation(lib):
    """Argument checks of the streaming-read aid (all before any launch)."""
    fake = ctypes.c_void_p(FAKE)
    r = lambda src=fake, n=1 << 20, wg=32, out=fake: lib.star_stream_read(src, n, wg, out, None)
    assert r(src=None) == -1
    assert r(out=None) == -1
    assert r(src=ctypes.c_void_p(FAKE + 8)) == -4
    assert r(out=ctypes.c_void_p(FAKE + 2)) == -4
    assert r(wg=0) == -2
    assert r(wg=65537) == -2
    assert r(n=0) == -2
    assert r(n=(1 << 20) + 16) == -2          # not a multiple of 32 * 32768
    assert r(n=32768 * 31, wg=32) == -2


def test_pulsar_prefix_host_matches_oracle(lib):
    """The library's host-side Max-IDF selection equals the oracle's,
    index for index (integer work: bit-exact), on Zipf-distributed token
    ids at three block shapes, including a ragged tail and b % 32 != 0."""
    import numpy as np

    import block_sparse_amd as sa
    import oracle.star_oracle as so
    from workloads import token_ids
    for (L, b, m, sink, k) in [(16384, 4096, 32, 64, 16), (5000, 700, 32, 64, 5),
                               (2048, 100, 24, 40, 3), (300, 400, 32, 64, 2)]:
        tok = token_ids(7, 1, L)[0]
        r1, s1, l1 = sa.pulsar_prefix(tok, L, b, m, sink, k)
        r2, s2, l2 = so.pulsar_prefix(tok, L, b, m, sink, k)
        assert np.array_equal(r1, r2) and np.array_equal(s1, s2) and np.array_equal(l1, l2)
        # ids outside a dense vocabulary range (negative, >= 2^24) take the
        # library's hash-map path: same selection
        wide = np.where(tok % 3 == 0, -tok - 1, tok * 1000 + 7).astype(np.int64)
        wide = np.where(wide > 2 ** 31 - 1, wide % (2 ** 31 - 1), wide).astype(np.int32)
        assert len(np.unique(wide)) == len(np.unique(tok))     # still a relabelling
        r3, s3, l3 = sa.pulsar_prefix(wide, L, b, m, sink, k)
        assert np.array_equal(r3, r2) and np.array_equal(s3, s2) and np.array_equal(l3, l2)


def test_pulsar_prefix_host_validation(lib):
    import numpy as np
    tok = np.zeros(100, dtype=np.int32)
    tp = tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    n = ctypes.c_int64(0)
    a = (ctypes.c_int64 * 4)()
    P = lambda L=100, b=25, m=32, s=64, k=1, rows=None, cap=0, nb=4, nr=ctypes.byref(n): \
        lib.star_pulsar_prefix(tp, L, b, m, s, k, rows, cap, nr, a, a, nb)
    assert P(nr=None) == -1
    assert P(b=0) == -2 and P(m=0) == -2 and P(k=-1) == -2 and P(nb=3) == -2
    assert P(cap=0) == -2 and n.value > 0            # too small: reports the size
    rows = (ctypes.c_int64 * n.value)()
    assert P(rows=rows, cap=n.value) == 0


def test_decode_step_validation(lib):
    qn = T(B=1, H=8, S=1, D=128)
    kn, vn = T(B=1, H=2, S=1, D=128), T(B=1, H=2, S=1, D=128)
    kc, vc = T(B=1, H=2, S=100, D=128), T(B=1, H=2, S=100, D=128)
    o = T(B=1, H=8, S=1, D=128, dtype=1)

    def ds(q=qn, k=kn, oo=o, slot=50, pos=50, offs=(0, 40, 51), splits=2, op=FAKE, lp=FAKE,
           base=5e5, rope=1):
        arr = (ctypes.c_int64 * len(offs))(*offs)
        return lib.star_decode_step(ctypes.byref(q), ctypes.byref(k), ctypes.byref(vn),
                                    ctypes.byref(kc), ctypes.byref(vc), slot, pos, base, rope,
                                    arr, len(offs) - 1, splits, 0.1, op, lp, ctypes.byref(oo),
                                    None, None)
    assert ds(slot=51, pos=51) == -2               # slot outside the partitions
    assert ds(slot=-1, pos=-1) == -2
    assert ds(pos=-1) == -2
    # the cache is position-contiguous: the token's row is its position
    assert ds(slot=49, pos=50) == -2
    assert ds(slot=50, pos=49) == -2
    assert ds(q=T(B=1, H=8, S=2, D=128)) == -2     # one token per call
    assert ds(k=T(B=1, H=2, S=1, D=64)) == -2
    assert ds(oo=T(B=1, H=8, S=2, D=128)) == -2
    assert ds(q=T(B=1, H=8, S=1, D=128, dtype=1)) == -3
    assert ds(op=None) == -1
    assert ds(op=FAKE + 4) == -4
    assert ds(offs=(0, 60, 51)) == -2
    assert ds(offs=(0, 40, 101)) == -2
    assert ds(base=1.0) == -2
    assert ds(splits=0) == -2


def test_rope_freqs_are_the_nearest_float64(lib):
    """The frequencies every rotating kernel uses equal the oracle's (the
    float64 nearest base^(-2j/D), from decimal arithmetic) bit for bit, at
    every head dim the RoPE entry points accept and several bases."""
    import oracle.star_oracle as so
    for base in (100.0, 10000.0, 500000.0, 1e6, 1234567.0):
        for D in range(16, 129, 16):
            out = (ctypes.c_double * (D // 2))()
            assert lib.star_rope_freqs(D, base, out) == 0
            assert list(out) == so.rope_theta(D, base).tolist(), (base, D)
    out = (ctypes.c_double * 64)()
    assert lib.star_rope_freqs(128, 5e5, None) == -1
    assert lib.star_rope_freqs(72, 5e5, out) == -5
    assert lib.star_rope_freqs(8, 5e5, out) == -5
    assert lib.star_rope_freqs(128, 1.0, out) == -2
    assert lib.star_rope_freqs(128, float("inf"), out) == -2


def test_decode_step_noalloc_validation(lib):
    """The no-allocation decode step checks its arguments exactly as
    star_decode_step does, then refuses partials beyond its scratch array,
    all before it touches the GPU."""
    qn = T(B=1, H=8, S=1, D=128)
    kn, vn = T(B=1, H=2, S=1, D=128), T(B=1, H=2, S=1, D=128)
    kc, vc = T(B=1, H=2, S=100, D=128), T(B=1, H=2, S=100, D=128)
    o = T(B=1, H=8, S=1, D=128, dtype=1)

    def na(q=qn, oo=o, slot=50, pos=50, offs=(0, 40, 51), splits=2, cache=(kc, vc)):
        arr = (ctypes.c_int64 * len(offs))(*offs)
        return lib.star_decode_step_noalloc(ctypes.byref(q), ctypes.byref(kn), ctypes.byref(vn),
                                            ctypes.byref(cache[0]), ctypes.byref(cache[1]),
                                            slot, pos, 5e5, 1, arr, len(offs) - 1, splits, 0.1,
                                            ctypes.byref(oo), None, None)
    assert na(slot=49) == -2
    assert na(q=T(B=1, H=8, S=2, D=128)) == -2
    assert na(oo=T(B=1, H=8, S=2, D=128)) == -2
    assert na(q=T(B=1, H=8, S=1, D=128, dtype=1)) == -3
    assert na(offs=(0, 60, 51)) == -2
    assert na(splits=0) == -2
    # 128 partitions x 8 chunks x 64 heads x 129 floats: far past the 4 MiB array
    big = (T(B=1, H=8, S=9000, D=128), T(B=1, H=8, S=9000, D=128))
    q64, o64 = T(B=1, H=64, S=1, D=128), T(B=1, H=64, S=1, D=128, dtype=1)
    kn8 = T(B=1, H=8, S=1, D=128)
    arr = (ctypes.c_int64 * 129)(*(list(range(0, 8192, 64)) + [8193]))
    assert lib.star_decode_step_noalloc(ctypes.byref(q64), ctypes.byref(kn8), ctypes.byref(kn8),
                                        ctypes.byref(big[0]), ctypes.byref(big[1]), 8192, 8192,
                                        5e5, 1, arr, 128, 8, 0.1, ctypes.byref(o64), None,
                                        None) == -5
    assert _lib.STAR_NOALLOC_SCRATCH_BYTES == 4 << 20


def test_decode_step_devpos_validation(lib):
    """The device-position decode step checks everything star_decode_step
    checks except the position itself (read on the device), plus its
    pointer: NULL, misaligned, and a last partition that can hold no token."""
    qn = T(B=1, H=8, S=1, D=128)
    kn, vn = T(B=1, H=2, S=1, D=128), T(B=1, H=2, S=1, D=128)
    kc, vc = T(B=1, H=2, S=100, D=128), T(B=1, H=2, S=100, D=128)
    o = T(B=1, H=8, S=1, D=128, dtype=1)

    def dp(q=qn, oo=o, pos=FAKE, offs=(0, 40, 100), splits=2, op=FAKE, base=5e5):
        arr = (ctypes.c_int64 * len(offs))(*offs)
        return lib.star_decode_step_devpos(ctypes.byref(q), ctypes.byref(kn), ctypes.byref(vn),
                                           ctypes.byref(kc), ctypes.byref(vc), pos, base, 1, arr,
                                           len(offs) - 1, splits, 0.1, op, FAKE,
                                           ctypes.byref(oo), None, None)
    assert dp(pos=None) == -1
    assert dp(pos=FAKE + 4) == -4
    assert dp(offs=(0, 40, 40)) == -2          # the last partition holds no position
    assert dp(offs=(0, 40, 101)) == -2         # past the cache
    assert dp(offs=(0, 60, 50)) == -2
    assert dp(q=T(B=1, H=8, S=2, D=128)) == -2
    assert dp(oo=T(B=1, H=8, S=2, D=128)) == -2
    assert dp(q=T(B=1, H=8, S=1, D=128, dtype=1)) == -3
    assert dp(op=None) == -1
    assert dp(splits=0) == -2
    assert dp(base=1.0) == -2
