"""Writes encoder_tail_biting_gap.txt: for unit-Gaussian 16x16 tiles at K = 5, 6,
7 and 8, the cost of the encoder's two-pass tail-biting search and of the exact
tail-biting optimum (the best of the 2^(16-K) searches constrained to each
value of the overlap bits), both from the CPU oracle only.

The pages ("ExLlamaV3 inference speed: EXL3 GEMM kernel and fused Viterbi
encoding", section "Viterbi encoding kernel") close the tail-biting boundary by
enumerating start states; the encoder takes two passes instead.  This file
measures what that reading costs.

Run from the repository root:  python tests/golden/make_encoder_gap.py
(about 25 CPU-minutes, spread over the host's cores).
"""
import multiprocessing as mp
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

TILES = {5: 4, 6: 8, 7: 8, 8: 8}  # tiles per bit width


def target(K, t):
    """Unit-Gaussian targets of tile t at K bits (seeded, float32)."""
    return np.random.default_rng([0, 9, K, t]).standard_normal(256).astype(np.float32)


def one(args):
    from oracle import exl3_oracle as O
    K, t = args
    w = target(K, t)
    vals = O.codebook(np.arange(65536)).astype(np.float32)
    _, c2 = O.tail_biting_two_pass(w, vals, 16, K)
    _, ce = O.tail_biting_exact(w, vals, 16, K)
    return K, t, float(c2), float(ce)


if __name__ == "__main__":
    jobs = [(K, t) for K, n in TILES.items() for t in range(n)]
    with mp.get_context("fork").Pool(min(len(jobs), len(os.sched_getaffinity(0)))) as pool:
        rows = pool.map(one, jobs)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "encoder_tail_biting_gap.txt")
    with open(out, "w") as f:
        f.write("# Encoder two-pass tail-biting cost against the exact tail-biting optimum, codebook 0, 16-bit state.\n")
        f.write("# Targets: numpy default_rng([0, 9, K, tile]).standard_normal(256) as float32.\n")
        f.write("# Written by tests/golden/make_encoder_gap.py (CPU oracle only); costs are float32 sums of squares.\n")
        f.write("# K tile two_pass_cost exact_cost\n")
        for K, t, c2, ce in rows:
            f.write(f"{K} {t} {c2!r} {ce!r}\n")
    print(open(out).read())
