"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one piece of the format definition (FMT-1..9) against a closed
form, a hand-worked value, a library routine or brute force, so that a dropped
term, a wrong sign, a wrong index or a transposed operand fails at least one.
"""
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import exl3_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- Hadamard --
def test_hadamard_orthogonal_integer():
    H = O.hadamard()
    assert H.shape == (128, 128)
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(H, H.T)


def test_hadamard_matches_library_sylvester():
    # scipy builds the Sylvester matrix by recursive doubling, not by popcount
    assert np.array_equal(O.hadamard(), scipy.linalg.hadamard(128).astype(np.int64))


def test_hadamard_special_vectors():
    H = O.hadamard()
    e0 = np.zeros(128, dtype=np.int64)
    e0[0] = 1
    assert np.array_equal(H @ e0, np.ones(128, dtype=np.int64))
    assert np.array_equal(H @ np.ones(128, dtype=np.int64), 128 * e0)


def _fwht(v):
    """Iterative butterfly, a different algorithm from the dense definition."""
    v = np.array(v, dtype=np.float64)
    h = 1
    while h < v.shape[-1]:
        a = v.reshape(v.shape[:-1] + (-1, 2, h))
        s = a[..., 0, :] + a[..., 1, :]
        d = a[..., 0, :] - a[..., 1, :]
        v = np.stack([s, d], axis=-2).reshape(v.shape)
        h *= 2
    return v


def test_rotate_blockwise_matches_butterfly_and_parseval():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 512))
    sign = rng.choice([-1.0, 1.0], 512)
    xr = O.rotate(x, sign)
    ref = _fwht((x * sign).reshape(3, 4, 128)).reshape(3, 512)
    np.testing.assert_allclose(xr, ref, rtol=0, atol=1e-12)
    # blockwise Parseval: |H v|^2 = 128 |v|^2 per 128-block
    np.testing.assert_allclose((xr.reshape(3, 4, 128) ** 2).sum(-1),
                               128 * (x.reshape(3, 4, 128) ** 2).sum(-1), rtol=1e-12)


def test_rotate_sign_flip_invariance():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 256))
    sign = rng.choice([-1.0, 1.0], 256)
    flip = rng.choice([-1.0, 1.0], 256)
    np.testing.assert_array_equal(O.rotate(x, sign), O.rotate(x * flip, sign * flip))


# ---------------------------------------------------------------- codebook --
def _golden_codebook():
    rows = []
    with open(os.path.join(GOLDEN, "codebook_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            s, p, q, bits, val = line.split()
            rows.append((int(s, 16), int(p, 16), int(q, 16), int(bits, 16), float(val)))
    return rows


def test_codebook_hand_worked_examples():
    for s, p, q, bits, val in _golden_codebook():
        c = O.codebook(np.array([s], dtype=np.uint16))
        assert int(O.fp16_bits(c)[0]) == bits, hex(s)
        assert float(c[0]) == val
        assert O.codebook_scalar(s) == val
        lo, hi = O.codebook_halves(np.array([s], dtype=np.uint16))
        assert int(lo.view(np.uint16)[0]) == q & 0xFFFF
        assert int(hi.view(np.uint16)[0]) == q >> 16


def test_codebook_constant_constraints():
    assert O.CB_A % 2 == 1 and O.CB_A < (1 << 16)
    assert O.CB_X & O.CB_M == 0
    for half in (O.CB_X & 0xFFFF, O.CB_X >> 16):
        assert (half >> 10) & 0x1F == 0b01100      # planted exponent bits 011xx
    for half in (O.CB_M & 0xFFFF, O.CB_M >> 16):
        assert (half >> 14) & 1 == 0 and (half >> 12) & 3 == 0   # top exponent bits planted


def test_codebook_statistics_all_states():
    s = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    c = O.codebook(s).astype(np.float64)
    assert np.isfinite(c).all()
    nz = np.abs(c[c != 0])
    assert nz.min() >= 2.0 ** -14          # no subnormal sums
    assert abs(c.mean()) <= 0.01
    assert abs(c.var() - 1.0) <= 0.02
    lo, hi = O.codebook_halves(s)
    for h in (lo.astype(np.float64), hi.astype(np.float64)):
        assert (np.abs(h) >= 0.125).all() and (np.abs(h) < 2).all()


def test_codebook_vectorised_equals_scalar_all_states():
    s = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    c = O.codebook(s).astype(np.float64)
    cs = np.array([O.codebook_scalar(int(v)) for v in range(65536)])
    np.testing.assert_array_equal(c, cs)


# ------------------------------------------------- byte-sum codebook (FMT-10) --
def _golden_codebook1():
    rows = []
    with open(os.path.join(GOLDEN, "codebook1_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            s, p, t, bits, val = line.split()
            rows.append((int(s, 16), int(p, 16), int(t), int(bits, 16), float(val)))
    return rows


def test_codebook1_hand_worked_examples():
    rows = _golden_codebook1()
    assert len(rows) == 4
    for s, p, t, bits, val in rows:
        c = O.codebook(np.array([s], dtype=np.uint16), cb=1)
        assert int(O.fp16_bits(c)[0]) == bits, hex(s)
        assert float(c[0]) == val
        assert O.codebook_scalar(s, cb=1) == val
        assert int(O.byte_sums(np.array([s]))[0]) == t
        assert (s * O.CB1_A + O.CB1_B) % (1 << 32) == p


def test_codebook1_byte_sums_by_byte_view():
    # the byte sum read back through a little-endian byte view of p: catches a
    # wrong shift, mask or byte count in byte_sums
    s = np.arange(65536, dtype=np.uint64)
    p = ((s * np.uint64(O.CB1_A) + np.uint64(O.CB1_B)) & np.uint64(0xFFFFFFFF)).astype("<u4")
    t = p.view(np.uint8).reshape(-1, 4).astype(np.int64).sum(axis=1)
    np.testing.assert_array_equal(O.byte_sums(s), t)


def test_codebook1_constants_and_statistics():
    assert O.CB1_A % 2 == 1 and O.CB1_A < (1 << 16)
    # G and C are fp16 values; C = -10.375 exactly, G = 1773/262144 exactly
    G = float(np.array([O.CB1_G], np.uint16).view(np.float16)[0])
    C = float(np.array([O.CB1_C], np.uint16).view(np.float16)[0])
    assert G == 1773 / 262144 and C == -10.375
    s = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = O.byte_sums(s).astype(np.float64)
    # four uniform bytes: mean 4 * 255/2 = 510, variance 4 * (256^2 - 1)/12 = 21845
    assert abs(t.mean() - 510) / 510 < 1e-3 and abs(t.var() - 21845) / 21845 < 2e-3
    c = O.codebook(s, cb=1).astype(np.float64)
    assert np.isfinite(c).all()
    assert np.abs(c).min() >= 2.0 ** -14          # no subnormal value
    assert abs(c.mean()) <= 0.01 and abs(c.var() - 1.0) <= 0.02
    assert len(np.unique(c)) > 800


def test_codebook1_single_rounding_all_states():
    # exact rational (1024 + t) * G + C, rounded once to fp16 (Fraction path), on every state
    s = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    c = O.codebook(s, cb=1).astype(np.float64)
    cs = np.array([O.codebook_scalar(int(v), cb=1) for v in range(65536)])
    np.testing.assert_array_equal(c, cs)


def test_codebook1_is_affine_in_the_byte_sum():
    # equal byte sums give equal values; values increase with the byte sum
    s = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = O.byte_sums(s)
    c = O.codebook(s, cb=1).astype(np.float64)
    order = np.argsort(t, kind="stable")
    assert np.all(np.diff(c[order]) >= 0)
    for tv in np.unique(t)[::50]:
        assert np.unique(c[t == tv]).size == 1


def test_codebook_rejects_unknown_codebook():
    with pytest.raises(ValueError):
        O.codebook(np.array([0]), cb=2)


# ------------------------------------------------------------------ states --
@pytest.mark.parametrize("K", range(1, 9))
def test_states_zero_and_ones_streams(K):
    z = np.zeros(16 * K, dtype=np.uint16)
    assert (O.tile_states(z, K) == 0).all()
    o = np.full(16 * K, 0xFFFF, dtype=np.uint16)
    assert (O.tile_states(o, K) == 0xFFFF).all()
    dz = O.decode_tiles(z, K)
    assert (O.fp16_bits(dz) == 0xB1E7).all()


@pytest.mark.parametrize("K", range(1, 9))
def test_states_periodic_stream_is_rotation(K):
    rng = np.random.default_rng(K)
    for w in rng.integers(0, 65536, 8):
        words = np.full(16 * K, w, dtype=np.uint16)
        st = O.tile_states(words, K)
        for i in range(256):
            r = (i * K) % 16
            expect = ((int(w) >> r) | (int(w) << (16 - r))) & 0xFFFF
            assert int(st[i]) == expect


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 7, 8])
def test_states_one_hot_stream(K):
    nbits = 256 * K
    for p in [0, 1, 5, 15, 16, 17, 100, nbits - 1, nbits - 16, nbits - 17]:
        words = np.zeros(16 * K, dtype=np.uint16)
        words[p // 16] = 1 << (p % 16)
        st = O.tile_states(words, K)
        for i in range(256):
            e = (p - i * K) % nbits
            expect = (1 << e) if e < 16 else 0
            assert int(st[i]) == expect, (K, p, i)


@pytest.mark.parametrize("K", range(1, 9))
def test_states_vectorised_equals_scalar(K):
    rng = np.random.default_rng(100 + K)
    words = rng.integers(0, 65536, 16 * K, dtype=np.uint16)
    st = O.tile_states(words, K)
    for i in range(256):
        assert int(st[i]) == O.state_scalar(words, K, i)


@pytest.mark.parametrize("K", range(1, 9))
def test_row_states_equal_tile_states(K):
    # the row decode reads a (K+1)-word window of the stream: every row of
    # random tiles, and of a one-hot stream at each bit near the tile's wrap,
    # against the full-tile states and the scalar bit walk
    rng = np.random.default_rng(300 + K)
    words = rng.integers(0, 65536, (5, 16 * K), dtype=np.uint16)
    full = O.tile_states(words, K)
    for r in range(16):
        np.testing.assert_array_equal(O.tile_row_states(words, K, r), full[:, 16 * r:16 * r + 16])
    rr = rng.integers(0, 16, 5)  # a row per tile
    got = O.tile_row_states(words, K, rr)
    for t in range(5):
        for c in (0, 7, 15):
            assert int(got[t, c]) == O.state_scalar(words[t], K, 16 * int(rr[t]) + c)
    nbits = 256 * K
    for p in list(range(0, 20)) + list(range(nbits - 20, nbits)):
        w = np.zeros(16 * K, np.uint16)
        w[p // 16] = 1 << (p % 16)
        st = O.tile_states(w, K)
        for r in (0, 1, 14, 15):
            np.testing.assert_array_equal(O.tile_row_states(w, K, r), st[16 * r:16 * r + 16])


def test_states_sliding_recurrence():
    # s_{i+1} = (s_i >> K) | (next K stream bits << (16 - K)), cyclic
    for K in (2, 3, 6):
        rng = np.random.default_rng(K)
        words = rng.integers(0, 65536, 16 * K, dtype=np.uint16)
        st = O.tile_states(words, K).astype(np.int64)
        bits = [(int(words[j // 16]) >> (j % 16)) & 1 for j in range(256 * K)]
        for i in range(256):
            nxt = 0
            for b in range(K):
                nxt |= bits[(i * K + 16 + b) % (256 * K)] << b
            assert st[(i + 1) % 256] == (st[i] >> K) | (nxt << (16 - K))


# --------------------------------------------------------------- placement --
def test_tiles_to_matrix_placement():
    to, ti = 3, 5
    ids = np.arange(to * ti * 256, dtype=np.int64).reshape(to, ti, 256)
    W = O.tiles_to_matrix(ids)
    for tr in range(to):
        for tc in range(ti):
            for i in (0, 1, 15, 16, 17, 255):
                assert W[16 * tr + (i >> 4), 16 * tc + (i & 15)] == ids[tr, tc, i]


def test_single_nonzero_tile_touches_only_its_strip():
    K = 3
    words, x, sign, scale = synth.random_case(256, 64, K, 2, 11)
    base = O.linear(x, words, sign, scale, K)
    w2 = words.copy()
    w2[2, 1] ^= np.uint16(0x5A5A)
    y2 = O.linear(x, w2, sign, scale, K)
    diff = np.abs(y2 - base).max(axis=0)
    assert (diff[:32] == 0).all() and (diff[48:] == 0).all()
    assert (diff[32:48] > 0).any()


# ------------------------------------------------------------- the product --
@pytest.mark.parametrize("K", range(1, 9))
def test_linear_brute_force_tiny(K):
    n_out = 32 if K in (3, 8) else 16
    m = 1 + K % 3
    words, x, sign, scale = synth.random_case(128, n_out, K, m, 200 + K)
    y = O.linear(x, words, sign, scale, K)
    rng = np.random.default_rng(K)
    for _ in range(6):
        r = int(rng.integers(0, m))
        o = int(rng.integers(0, n_out))
        ys = O.y_scalar(x, words, sign, scale, K, r, o)
        assert abs(y[r, o] - ys) <= 1e-9 * max(1.0, abs(ys))


@pytest.mark.parametrize("K", [2, 5, 8])
def test_linear_brute_force_tiny_codebook1(K):
    words, x, sign, scale = synth.random_case(128, 16, K, 2, 250 + K)
    y = O.linear(x, words, sign, scale, K, cb=1)
    assert not np.allclose(y, O.linear(x, words, sign, scale, K))  # the codebook matters
    rng = np.random.default_rng(K)
    for _ in range(4):
        r, o = int(rng.integers(0, 2)), int(rng.integers(0, 16))
        ys = O.y_scalar(x, words, sign, scale, K, r, o, cb=1)
        assert abs(y[r, o] - ys) <= 1e-9 * max(1.0, abs(ys))
    rows = np.array([0, 7, 15])
    np.testing.assert_allclose(O.linear_rows(x, words, sign, scale, K, rows, cb=1), y[:, rows], rtol=0, atol=1e-12)


def test_linear_unit_input_closed_form():
    K = 4
    words, x, sign, scale = synth.random_case(256, 32, K, 1, 7)
    sign = np.ones_like(sign)
    W = O.dequant(words, K).astype(np.float64)
    H = O.hadamard()
    for k in (0, 5, 130, 255):
        e = np.zeros((1, 256), dtype=np.float16)
        e[0, k] = 1
        y = O.linear(e, words, sign, scale, K)[0]
        b, j = divmod(k, 128)
        expect = scale.astype(np.float64) * (W[:, 128 * b:128 * b + 128] @ H[:, j].astype(np.float64))
        np.testing.assert_allclose(y, expect, rtol=1e-13, atol=0)


def test_linear_scale_and_sign_invariants():
    K = 2
    words, x, sign, scale = synth.random_case(256, 48, K, 3, 9)
    y = O.linear(x, words, sign, scale, K)
    y2 = O.linear(x, words, sign, (scale.astype(np.float32) * 2).astype(np.float16), K)
    np.testing.assert_array_equal(y2, 2 * y)
    flip = np.where(np.arange(256) % 3 == 0, -1, 1).astype(np.float16)
    y3 = O.linear(x * flip, words, sign * flip, scale, K)
    np.testing.assert_array_equal(y3, y)


@pytest.mark.parametrize("K", range(1, 9))
def test_linear_rows_matches_full(K):
    # any rows, in any order, repeated, across chunk boundaries; both codebooks
    words, x, sign, scale = synth.random_case(384, 80, K, 2, [13, K])
    rows = np.array([0, 7, 16, 33, 79, 64, 7, 15, 48, 31])
    for cb in (0, 1):
        y = O.linear(x, words, sign, scale, K, strip_block=2, cb=cb)
        np.testing.assert_allclose(O.linear_rows(x, words, sign, scale, K, rows, cb=cb, chunk=3), y[:, rows],
                                   rtol=1e-12, atol=0)
        W = O.dequant(words, K, cb)
        np.testing.assert_array_equal(O.fp16_bits(O.weight_rows(words, K, rows, cb)), O.fp16_bits(W[rows]))


def test_oracle_rejects_bad_arguments():
    words, x, sign, scale = synth.random_case(128, 16, 2, 1, 1)
    with pytest.raises(ValueError):
        O.linear(x, words, sign, scale, 3)
    with pytest.raises(ValueError):
        O.tile_states(words[0, 0], 9)
