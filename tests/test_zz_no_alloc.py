"""exl3_linear_noalloc (the entry point that allocates nothing: its scratch is
a static per-GPU array in the library) against exl3_linear with a workspace of
the size exl3_pack_info gives, through the C ABI.  The two take the same path
and split, so their outputs must agree bit for bit; both are also checked
against the CPU oracle.  Two calls in a row, the second with a smaller input,
so the second runs over the scratch the first one left behind."""
import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O

pytestmark = pytest.mark.gpu

TOL = 1e-3
SCRATCH = 64 << 20  # EXL3_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gemm_exl3_amd as ex
    ex.load()
    return torch


def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def rel_fro(y, ref):
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


# (n_in, n_out, K, m) pairs: the first call larger than the second.  GEMM with
# the 256-row kernel and a split input dimension, then the 64-row kernel;
# the split 128-row kernel, then the GEMV; the GEMV with its rotation pre-pass
# into the scratch (m = 8 rows of 14336 inputs), then a plain GEMV.
SEQUENCES = [
    [(4096, 1024, 3, 300), (4096, 1024, 3, 40)],
    [(2048, 4112, 4, 100), (2048, 4112, 4, 2)],
    [(14336, 512, 2, 8), (14336, 512, 2, 1)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_linear(torch_cuda, seq):
    import decode_gemm_exl3_amd as ex
    torch = torch_cuda
    for call, (n_in, n_out, K, m) in enumerate(SEQUENCES[seq]):
        print(f"[case] noalloc seq={seq} call={call} n_in={n_in} n_out={n_out} K={K} m={m}", flush=True)
        # the same split in both: the workspace exl3_linear gets fits the scratch
        assert ex.pack_info(n_in, n_out, K, m)["workspace_bytes"] <= SCRATCH
        words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [61, seq, call])
        d = [to_dev(torch, a) for a in (x, words, sign, scale)]
        y_na = torch.full((m, n_out), float("nan"), dtype=torch.float16, device="cuda")
        ex.linear_noalloc(*d, K, y=y_na)
        ws = ex.Workspace(n_in, n_out, K, m)
        y_ref = ex.linear(*d, K, workspace=ws)
        torch.cuda.synchronize()
        a, b = y_na.cpu().numpy(), y_ref.cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (seq, call)
        assert rel_fro(a, O.linear(x, words, sign, scale, K)) <= TOL, (seq, call)


def test_noalloc_at_its_limit(torch_cuda):
    # 4096 rows of 8192 inputs: the rotated input fills the 64 MiB scratch
    # exactly, so the input dimension is not split; exl3_linear given a
    # workspace of the same 64 MiB takes the same plan and gives the same bits
    import decode_gemm_exl3_amd as ex
    torch = torch_cuda
    n_in, n_out, K, m = 8192, 32, 2, 4096
    print(f"[case] noalloc at the limit n_in={n_in} n_out={n_out} K={K} m={m}", flush=True)
    words, _, sign, scale = synth.random_case(n_in, n_out, K, 1, [62])
    x = torch.randn((m, n_in), device="cuda").half()
    d = [x] + [to_dev(torch, a) for a in (words, sign, scale)]
    y_na = torch.full((m, n_out), float("nan"), dtype=torch.float16, device="cuda")
    ex.linear_noalloc(*d, K, y=y_na)

    class Ws:  # a workspace of exactly the scratch's size
        buf = torch.empty(SCRATCH, dtype=torch.uint8, device="cuda")
        nbytes = SCRATCH

    y_ref = ex.linear(*d, K, workspace=Ws())
    torch.cuda.synchronize()
    assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16))
    sel = np.unique(np.concatenate([np.arange(8), m - 8 + np.arange(8), np.random.default_rng(62).integers(0, m, 48)]))
    selt = torch.from_numpy(sel).cuda()
    assert rel_fro(y_na[selt].cpu().numpy(), O.linear(x[selt].cpu().numpy(), words, sign, scale, K)) <= TOL
