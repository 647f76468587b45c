"""GPU parity of the named workloads and of every launch the benchmark times,
at their full sizes and in the launch configuration the benchmark uses (fused
gate/up and q/k/v through exl3_gemv_multi, the rest through exl3_gemv,
exl3_gemm or exl3_linear), against the float64 CPU oracle.

Large outputs are compared on one output feature of every 16-row strip plus
the first and last strips whole (every strip, and every 256-wide GEMM block,
is looked at); the single 4096x4096 layer and the 2048x8192x8192 GEMM are
compared whole.  The bar (tests/_parity.py): relative Frobenius error <= 1e-3
and every element within 1e-2 of the reference's root mean square.
"""
import numpy as np
import pytest

import synth
from _parity import assert_close, log, run_launch, strip_rows
from oracle import exl3_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ex():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gemm_exl3_amd as ex
    ex.load()
    return ex


@pytest.fixture(scope="module")
def torch_cuda(ex):
    import torch
    return torch


def check_launch(torch, ex, launch, fn, seed, ws=None, cb=0):
    """Run one launch (all its projections) and compare every projection on
    its strip-sampled rows."""
    words, x, sign, scales = synth.draw_group(launch.members)
    log(f"{fn} {launch.name}: n_in={launch.n_in} n_outs={launch.n_outs} K={launch.K} m={launch.m} codebook={cb}")
    ys = run_launch(torch, ex, fn, words, x, sign, scales, launch.K, ws=ws, cb=cb)
    rng = np.random.default_rng(seed)
    for mm, w, sc, y in zip(launch.members, words, scales, ys):
        rows = strip_rows(mm.n_out, rng)
        assert_close(y[:, rows], O.linear_rows(x, w, sign, sc, mm.K, rows, cb=cb), (launch.name, mm.name))


# ------------------------------------------------ 1: one 4096x4096 layer ----
def test_single_layer_whole_output(torch_cuda, ex):
    mm = synth.single_layer()[0]
    words, x, sign, scale = synth.draw(mm)
    ref = O.linear(x, words, sign, scale, mm.K)
    ws = ex.Workspace(mm.n_in, mm.n_out, mm.K, 1)
    for fn in ("gemv", "gemm", "linear"):
        log(f"{fn} single 4096x4096 K=4 m=1, whole output")
        y = run_launch(torch_cuda, ex, fn, [words], x, sign, [scale], mm.K, ws=ws)[0]
        assert_close(y, ref, fn)


# ------------------------------------------- 2: the Llama-3.1-8B MLP --------
@pytest.mark.parametrize("m", [1, 4, 8])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_mlp_launches(torch_cuda, ex, K, m):
    ws = ex.Workspace(14336, 14336, 8, 8)
    gate_up, down = synth.mlp_launches(K, m)
    check_launch(torch_cuda, ex, gate_up, "gemv_multi", [1, K, m], ws=ws)
    check_launch(torch_cuda, ex, down, "gemv", [2, K, m], ws=ws)


def test_mlp_launches_codebook1(torch_cuda, ex):
    ws = ex.Workspace(14336, 14336, 8, 1)
    gate_up, down = synth.mlp_launches(4, 1)
    check_launch(torch_cuda, ex, gate_up, "gemv_multi", [3], ws=ws, cb=1)
    check_launch(torch_cuda, ex, down, "gemv", [4], ws=ws, cb=1)


# ----------------------------------------------- 3: 70B decode launches ----
def test_llama70b_launches(torch_cuda, ex):
    ws = ex.Workspace(28672, 28672, 8, 1)
    for i, launch in enumerate(synth.llama70b_launches()):
        check_launch(torch_cuda, ex, launch, "gemv_multi" if len(launch.members) > 1 else "gemv", [5, i], ws=ws)


# ------------------------------------------------------ 4: prefill GEMM ----
def test_prefill_gemm_8192_whole_output(torch_cuda, ex):
    mm = synth.prefill_gemm()[0]
    words, x, sign, scale = synth.draw(mm)
    log("gemm 2048x8192x8192 K=4, whole output")
    y = run_launch(torch_cuda, ex, "gemm", [words], x, sign, [scale], mm.K, ws=ex.Workspace(8192, 8192, 4, 2048))[0]
    assert_close(y, O.linear(x, words, sign, scale, mm.K), mm.name)


def test_prefill_gemm_28672_and_codebook1(torch_cuda, ex):
    ws = ex.Workspace(8192, 28672, 8, 2048)
    mm = synth.prefill_gemm()[1]
    check_launch(torch_cuda, ex, synth.Launch(mm.name, [mm]), "gemm", [6], ws=ws)
    mm0 = synth.prefill_gemm()[0]
    check_launch(torch_cuda, ex, synth.Launch(mm0.name, [mm0]), "gemm", [7], ws=ws, cb=1)


# --------------------------------------- medium m through exl3_linear -------
@pytest.mark.parametrize("m", [16, 32, 64, 128, 256])
def test_medium_m_linear(torch_cuda, ex, m):
    mm = synth.medium_m(m)
    check_launch(torch_cuda, ex, synth.Launch(mm.name, [mm]), "linear", [8, m], ws=ex.Workspace(4096, 14336, 4, 256))


# -------------------------------- 5: the 32-layer Llama-3.1-8B stack --------
def test_stack_all_layers_fused(torch_cuda, ex):
    # all 224 matmuls, as the benchmark runs them: per layer q/k/v in one
    # launch, o, gate/up in one launch, down
    ws = ex.Workspace(14336, 14336, 8, 1)
    groups = synth.llama8b_stack_groups()
    assert sum(len(g) for g in groups) == 224
    for i, grp in enumerate(groups):
        launch = synth.Launch("+".join(mm.name for mm in grp), grp)
        check_launch(torch_cuda, ex, launch, "gemv_multi", [9, i], ws=ws)


def test_stack_all_layers_unfused(torch_cuda, ex):
    # the same 224 matmuls one launch each, each with its own input
    ws = ex.Workspace(14336, 14336, 8, 1)
    for i, mm in enumerate(synth.llama8b_stack()):
        check_launch(torch_cuda, ex, synth.Launch(mm.name, [mm]), "gemv", [10, i], ws=ws)
