"""Seeded synthetic inputs for the EXL3 decode-matmul workloads.

Shared by the tests, the benchmark and the smoke check.  This module holds no
part of the method's arithmetic: it only draws random packed words, inputs,
signs and scales (NumPy PCG64) in a fixed order, so that the CPU oracle and the
GPU path see the same bytes.

Draw order for one matmul (one generator per matmul):
  1. words     uint16 [n_out/16, n_in/16, 16K], uniform over 0..65535
               (every bit string is a valid tail-biting walk)
  2. x         fp16 [m, n_in] ~ N(0, 1), rounded to nearest even
  3. sign      fp16 [n_in], uniform +-1
  4. out_scale fp16 [n_out] ~ U(0.5, 1.5) * 0.02 (= U(0.01, 0.03))

Seeds: the single 4096x4096 layer uses default_rng(0); every other matmul uses
default_rng([0, workload, index]).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Matmul:
    name: str
    n_in: int
    n_out: int
    K: int
    m: int
    seed: object

    @property
    def trellis_bytes(self) -> int:
        return self.n_in * self.n_out * self.K // 8


def draw(mm: Matmul, with_words: bool = True):
    """Return (words, x, sign, out_scale) for one matmul, in the fixed draw order."""
    rng = np.random.default_rng(mm.seed)
    words = None
    if with_words:
        words = rng.integers(0, 65536, size=(mm.n_out // 16, mm.n_in // 16, 16 * mm.K),
                             dtype=np.uint16)
    else:  # keep the stream position identical without materialising the words
        n = (mm.n_out // 16) * (mm.n_in // 16) * 16 * mm.K
        chunk = 1 << 24
        while n > 0:
            rng.integers(0, 65536, size=min(n, chunk), dtype=np.uint16)
            n -= chunk
    x = rng.standard_normal((mm.m, mm.n_in)).astype(np.float16)
    sign = (2 * rng.integers(0, 2, mm.n_in) - 1).astype(np.float16)
    out_scale = (rng.uniform(0.5, 1.5, mm.n_out) * 0.02).astype(np.float16)
    return words, x, sign, out_scale


def words_only(n_in: int, n_out: int, K: int, seed) -> np.ndarray:
    """Packed words alone (first draw of the recipe) for an extra weight matrix."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 65536, size=(n_out // 16, n_in // 16, 16 * K), dtype=np.uint16)


def random_case(n_in: int, n_out: int, K: int, m: int, seed) -> tuple:
    """Arbitrary-shape case with the same recipe (used for small parity shapes)."""
    return draw(Matmul("case", n_in, n_out, K, m, seed))


# --- the five workloads -----------------------------------------------------
def single_layer() -> list[Matmul]:
    """One 4096->4096 linear layer at K=4, m=1, seed 0."""
    return [Matmul("layer4096_k4", 4096, 4096, 4, 1, 0)]


def llama8b_mlp(ms=(1, 4, 8), Ks=(2, 3, 4)) -> list[Matmul]:
    """Llama-3.1-8B-shaped MLP GEMVs: gate/up 4096->14336, down 14336->4096."""
    out = []
    idx = 0
    for K in (2, 3, 4):
        for m in (1, 4, 8):
            for name, n_in, n_out in (("gate_up", 4096, 14336), ("down", 14336, 4096)):
                if K in Ks and m in ms:
                    out.append(Matmul(f"{name}_k{K}_m{m}", n_in, n_out, K, m, [0, 2, idx]))
                idx += 1
    return out


def llama70b_decode() -> list[Matmul]:
    """70B-shaped decode GEMVs at m=1."""
    cases = [("gate_up_k2", 8192, 28672, 2), ("gate_up_k3", 8192, 28672, 3),
             ("down_k2", 28672, 8192, 2), ("down_k3", 28672, 8192, 3),
             ("attn_k4", 8192, 8192, 4)]
    return [Matmul(n, i, o, K, 1, [0, 3, idx]) for idx, (n, i, o, K) in enumerate(cases)]


def prefill_gemm(m: int = 2048) -> list[Matmul]:
    """Prefill GEMMs: 8192->8192 at K=4 and 8192->28672 at K=3, m tokens."""
    return [Matmul("attn_8192_k4", 8192, 8192, 4, m, [0, 4, 0]),
            Matmul("gate_up_28672_k3", 8192, 28672, 3, m, [0, 4, 1])]


STACK_PROJ = (("q", 4096, 4096, True), ("k", 4096, 1024, True), ("v", 4096, 1024, True),
              ("o", 4096, 4096, True), ("gate", 4096, 14336, False),
              ("up", 4096, 14336, False), ("down", 14336, 4096, False))


def llama8b_stack(n_layers: int = 32) -> list[Matmul]:
    """32-layer Llama-3.1-8B-shaped linear stack at m=1 (224 matmuls).

    One bit width K_b per block b drawn from {2..6}; q/k/v/o use K_b + 1.
    """
    kb = np.random.default_rng([0, 5, 999]).integers(2, 7, n_layers)
    out = []
    for b in range(n_layers):
        for j, (name, n_in, n_out, attn) in enumerate(STACK_PROJ):
            K = int(kb[b]) + (1 if attn else 0)
            out.append(Matmul(f"L{b}.{name}_k{K}", n_in, n_out, K, 1, [0, 5, 7 * b + j]))
    return out


# --- the launches the benchmark times ----------------------------------------
# A launch is one call: a GEMV launch may serve several projections that read
# the same input (gate and up, q/k/v), drawn member by member with their own
# seeds by `draw_group` (the first member's x and sign serve the launch).
@dataclass
class Launch:
    name: str
    members: list

    @property
    def K(self) -> int:
        return self.members[0].K

    @property
    def n_in(self) -> int:
        return self.members[0].n_in

    @property
    def m(self) -> int:
        return self.members[0].m

    @property
    def n_outs(self) -> list:
        return [mm.n_out for mm in self.members]


def mlp_launches(K: int, m: int = 1) -> list[Launch]:
    """The Llama-3.1-8B MLP at K bits and m rows as it is launched: gate and up
    (4096->14336 each) in one fused launch, then down (14336->4096)."""
    gate = Matmul(f"gate_k{K}_m{m}", 4096, 14336, K, m, [0, 2, K, m, 0])
    up = Matmul(f"up_k{K}_m{m}", 4096, 14336, K, m, [0, 2, K, m, 1])
    down = Matmul(f"down_k{K}_m{m}", 14336, 4096, K, m, [0, 2, K, m, 2])
    return [Launch(f"gate_up_k{K}", [gate, up]), Launch(f"down_k{K}", [down])]


def llama70b_launches() -> list[Launch]:
    """70B-shaped decode launches at m=1: gate and up (8192->28672 each) fused
    at K=2 and K=3, down (28672->8192) at K=2 and K=3, and the 8192->8192
    attention projection at K=4."""
    out = []
    for K in (2, 3):
        out.append(Launch(f"gate_up_k{K}", [Matmul(f"gate70_k{K}", 8192, 28672, K, 1, [0, 3, K, 0]),
                                            Matmul(f"up70_k{K}", 8192, 28672, K, 1, [0, 3, K, 1])]))
    for K in (2, 3):
        out.append(Launch(f"down_k{K}", [Matmul(f"down70_k{K}", 28672, 8192, K, 1, [0, 3, K, 2])]))
    out.append(Launch("attn_k4", [Matmul("attn70_k4", 8192, 8192, 4, 1, [0, 3, 4, 3])]))
    return out


def medium_m(m: int, n_in: int = 4096, n_out: int = 14336, K: int = 4) -> Matmul:
    """Batched decode and chunked prefill sizes of the 8B gate projection."""
    return Matmul(f"medium_m{m}", n_in, n_out, K, m, [0, 8, n_in, n_out, K, m])


# --- projections fed by one input (one fused GEMV launch) ---------------------
STACK_GROUPS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",)))


def llama8b_stack_groups(n_layers: int = 32) -> list[list[Matmul]]:
    """The 224 stack matmuls grouped by the input they read: per layer q/k/v,
    o, gate/up and down (128 groups).  Members keep their own seeds."""
    by_name = {mm.name: mm for mm in llama8b_stack(n_layers)}
    groups = []
    for b in range(n_layers):
        for _, members in STACK_GROUPS:
            groups.append([next(v for k, v in by_name.items() if k.startswith(f"L{b}.{nm}_k"))
                           for nm in members])
    return groups


def draw_group(mms: list[Matmul], with_words: bool = True):
    """(words list, x, sign, out_scale list) for projections sharing one input.

    Every member is drawn by `draw` with its own seed; the first member's x and
    sign serve the whole group (one input, one rotation), the others' are
    discarded.
    """
    words, scales = [], []
    x = sign = None
    for i, mm in enumerate(mms):
        w, xi, si, sc = draw(mm, with_words)
        words.append(w)
        scales.append(sc)
        if i == 0:
            x, sign = xi, si
    return words, x, sign, scales
