"""Pins of the CPU oracle's encoder (the tail-biting Viterbi search).

Reference: "ExLlamaV3 inference speed: EXL3 GEMM kernel and fused Viterbi
encoding", section "Viterbi encoding kernel": a forward Viterbi pass over the
trellis keeps the accumulated cost of every edge and takes the minimum-cost
path; the tail-biting boundary is closed by enumerating start states so that
the codeword's head and tail agree.
"""
import itertools

import numpy as np
import pytest

from oracle import exl3_oracle as O


def _tiny(L, K, T, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(T).astype(np.float32), rng.standard_normal(1 << L).astype(np.float32)


@pytest.mark.parametrize("L,K,T", [(6, 2, 6), (5, 1, 10), (8, 3, 5), (6, 3, 4), (7, 2, 7), (4, 1, 12)])
def test_exact_tail_biting_equals_brute_force(L, K, T):
    for seed in range(3):
        w, vals = _tiny(L, K, T, 100 * L + 10 * K + seed)
        bp, bc = O.brute_force_tail_biting(w, vals, L, K)
        ep, ec = O.tail_biting_exact(w, vals, L, K)
        assert ec == bc
        assert O.path_cost(w, vals, ep) == ec


@pytest.mark.parametrize("L,K,T", [(6, 2, 6), (5, 1, 8), (8, 4, 4)])
def test_free_viterbi_equals_brute_force_over_all_paths(L, K, T):
    # without the tail-biting constraint every start state and every K-bit
    # extension is allowed: enumerate them all
    w, vals = _tiny(L, K, T, 7 * L + K)
    best = None
    for s0 in range(1 << L):
        for ext in itertools.product(range(1 << K), repeat=T - 1):
            path = [s0]
            for b in ext:
                path.append((path[-1] >> K) | (b << (L - K)))
            c = O.path_cost(w, vals, path)
            if best is None or c < best:
                best = c
    path, c = O.trellis_viterbi(w, vals, L, K)
    assert c == best and O.path_cost(w, vals, path) == c
    for i in range(1, T):  # the path follows the trellis
        assert path[i] & ((1 << (L - K)) - 1) == path[i - 1] >> K


@pytest.mark.parametrize("L,K,T", [(6, 2, 6), (6, 3, 4), (7, 2, 8), (8, 3, 6)])
def test_two_pass_is_tail_biting_and_not_below_the_optimum(L, K, T):
    for seed in range(4):
        w, vals = _tiny(L, K, T, 31 * L + K + seed)
        path, c = O.tail_biting_two_pass(w, vals, L, K)
        low = (1 << (L - K)) - 1
        assert path[-1] >> K == path[0] & low        # head and tail agree
        assert c >= O.tail_biting_exact(w, vals, L, K)[1]
        assert O.path_cost(w, vals, path) == c


@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_encode_tile_round_trip(K):
    # decoding the packed stream gives back the states of the search and the
    # reported cost
    rng = np.random.default_rng(40 + K)
    w = rng.standard_normal(256).astype(np.float32)
    words, cost = O.encode_tile(w, K)
    assert words.shape == (16 * K,) and words.dtype == np.uint16
    dec = O.decode_tiles(words, K).astype(np.float32)
    d = w - dec
    assert O.path_cost(w, O.codebook(np.arange(65536)).astype(np.float32), O.tile_states(words, K)) == cost
    assert abs(float((d.astype(np.float64) ** 2).sum()) - float(cost)) <= 1e-5 * float(cost)


def test_encode_mse_falls_with_bits():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((3, 256)).astype(np.float32)
    mse = []
    for K in range(1, 9):
        _, costs = O.encode_tiles(W, K)
        mse.append(float(costs.mean()) / 256)
    assert all(a > b for a, b in zip(mse, mse[1:])), mse
    assert mse[0] < 1.0 and mse[-1] < 1e-3   # better than zero and close to lossless at 8 bits


def test_encode_beats_the_best_single_value_per_weight_at_low_rate():
    # at K = 2 the trellis reaches values a 2-bit scalar code cannot: its error
    # is below the best 4-level scalar quantiser of a unit Gaussian (~0.1175)
    rng = np.random.default_rng(11)
    W = rng.standard_normal((4, 256)).astype(np.float32)
    _, costs = O.encode_tiles(W, 2)
    assert float(costs.mean()) / 256 < 0.1175


def test_encode_codebook1():
    rng = np.random.default_rng(12)
    w = rng.standard_normal(256).astype(np.float32)
    words, cost = O.encode_tile(w, 3, cb=1)
    dec = O.decode_tiles(words, 3, cb=1).astype(np.float64)
    assert abs(((w - dec) ** 2).sum() - float(cost)) <= 1e-5 * float(cost)


# ------------------------------ the two-pass reading against the exact optimum
GAP_FILE = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "encoder_tail_biting_gap.txt")


def _gap_rows():
    rows = []
    with open(GAP_FILE) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                K, t, c2, ce = ln.split()
                rows.append((int(K), int(t), np.float32(c2), np.float32(ce)))
    return rows


def _gap_target(K, t):
    # the targets make_encoder_gap.py drew (its recipe, restated)
    return np.random.default_rng([0, 9, K, t]).standard_normal(256).astype(np.float32)


def test_two_pass_costs_recorded_and_never_below_the_exact_optimum():
    # 28 unit-Gaussian tiles at K = 5..8 (16-bit state): the encoder's two-pass
    # search, rerun here, gives the recorded cost, which is never below the
    # recorded exact tail-biting optimum (the best of all 2^(16-K) constrained
    # searches); on these tiles the two are equal
    vals = O.codebook(np.arange(65536)).astype(np.float32)
    rows = _gap_rows()
    assert len(rows) == 28 and {r[0] for r in rows} == {5, 6, 7, 8}
    for K, t, c2, ce in rows:
        path, c = O.tail_biting_two_pass(_gap_target(K, t), vals, 16, K)
        assert c == c2, (K, t, c, c2)
        assert c2 >= ce, (K, t)
        assert path[-1] >> K == path[0] & ((1 << (16 - K)) - 1)


def test_recorded_exact_optimum_k8():
    # one recorded exact optimum recomputed (256 constrained searches)
    vals = O.codebook(np.arange(65536)).astype(np.float32)
    K, t, _, ce = _gap_rows()[-8]
    assert K == 8
    assert O.tail_biting_exact(_gap_target(K, t), vals, 16, K)[1] == ce
