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
# into the scratch (m = 2..8, n_in >= 12288), then a plain GEMV.
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
