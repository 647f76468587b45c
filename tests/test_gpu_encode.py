"""GPU parity of the tail-biting Viterbi encoder (exl3_encode_tiles) against
the CPU oracle: the same fp32 decisions, so the streams and the costs must be
identical bit for bit."""
import numpy as np
import pytest

from oracle import exl3_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gemm_exl3_amd as ex
    ex.load()
    return torch


def log(msg):
    print(f"[case] {msg}", flush=True)


def encode_gpu(torch, W, K, cb=0, slots=256):
    import decode_gemm_exl3_amd as ex
    w = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).cuda()
    words, costs = ex.encode_tiles(w, K, codebook=cb, slots=slots)
    torch.cuda.synchronize()
    return words.cpu().numpy().view(np.uint16), costs.cpu().numpy()


def targets(n, seed):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((n, 256)).astype(np.float32)
    W[0] = 0.0                      # all-zero targets: many equal-cost paths (tie rule)
    return W


@pytest.mark.parametrize("K", range(1, 9))
def test_encode_matches_oracle(torch_cuda, K):
    log(f"encode K={K}")
    W = targets(3, 600 + K)
    words, costs = encode_gpu(torch_cuda, W, K)
    ref_w, ref_c = O.encode_tiles(W, K)
    assert np.array_equal(words, ref_w), (K, np.argwhere(words != ref_w)[:4])
    assert np.array_equal(costs.view(np.uint32), ref_c.view(np.uint32)), (K, costs, ref_c)


@pytest.mark.parametrize("K", [2, 5])
def test_encode_codebook1_matches_oracle(torch_cuda, K):
    log(f"encode codebook 1 K={K}")
    W = targets(2, 700 + K)
    words, costs = encode_gpu(torch_cuda, W, K, cb=1)
    ref_w, ref_c = O.encode_tiles(W, K, cb=1)
    assert np.array_equal(words, ref_w) and np.array_equal(costs, ref_c)


def test_encode_round_trip_through_decode(torch_cuda):
    import decode_gemm_exl3_amd as ex
    log("encode -> decode round trip K=3")
    torch = torch_cuda
    W = targets(4, 800)
    words, costs = encode_gpu(torch, W, 3)
    dec = ex.decode_tile(torch.from_numpy(words.view(np.int16)).cuda(), 3)
    torch.cuda.synchronize()
    d = W.astype(np.float64) - dec.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose((d ** 2).sum(axis=1), costs.astype(np.float64), rtol=1e-5)


def test_encode_many_tiles_any_workspace(torch_cuda):
    # the persistent workgroups reuse their slots across tiles: few slots and
    # many slots give the same streams; a sample is checked against the oracle
    log("encode 300 tiles K=4, 7 slots vs 300 slots")
    W = targets(300, 900)
    a_w, a_c = encode_gpu(torch_cuda, W, 4, slots=7)
    b_w, b_c = encode_gpu(torch_cuda, W, 4, slots=300)
    assert np.array_equal(a_w, b_w) and np.array_equal(a_c, b_c)
    idx = [0, 1, 150, 299]
    ref_w, ref_c = O.encode_tiles(W[idx], 4)
    assert np.array_equal(a_w[idx], ref_w) and np.array_equal(a_c[idx], ref_c)
    assert 0.005 < float(a_c[1:].mean()) / 256 < 0.02     # 4 bits per Gaussian weight
