"""The Python binding checks the tensors it hands to the library (element
type, shape, element count, contiguity, 16-byte alignment, device) and raises
before anything is launched.  CPU only: every case fails before a device is touched."""
import numpy as np
import pytest
import torch

import decode_gemm_exl3_amd as ex


def case(n_in=256, n_out=32, K=3, m=2):
    x = torch.zeros((m, n_in), dtype=torch.float16)
    tr = torch.zeros((n_out // 16, n_in // 16, 16 * K), dtype=torch.int16)
    sign = torch.ones(n_in, dtype=torch.float16)
    sc = torch.ones(n_out, dtype=torch.float16)
    y = torch.empty((m, n_out), dtype=torch.float16)
    return x, tr, sign, sc, y


@pytest.mark.parametrize("fn", ["gemv", "gemm", "linear"])
def test_linear_rejects_bad_tensors(fn):
    f = getattr(ex, fn)
    x, tr, sign, sc, y = case()
    with pytest.raises(ex.Exl3Error, match="x: dtype"):
        f(x.float(), tr, sign, sc, 3, y=y)
    with pytest.raises(ex.Exl3Error, match="sign: .*elements"):
        f(x, tr, sign[:128], sc, 3, y=y)
    with pytest.raises(ex.Exl3Error, match="trellis.*elements"):
        f(x, tr[:, :8], sign, sc, 3, y=y)
    with pytest.raises(ex.Exl3Error, match="trellis.*dtype"):
        f(x, tr.float(), sign, sc, 3, y=y)
    with pytest.raises(ex.Exl3Error, match="y.*shape"):
        f(x, tr, sign, sc, 3, y=y[:1])
    with pytest.raises(ex.Exl3Error, match="x: must be contiguous"):
        f(torch.zeros((256, 2), dtype=torch.float16).t(), tr, sign, sc, 3, y=y)
    with pytest.raises(ex.Exl3Error, match="x: data must be 16-byte aligned"):
        f(torch.zeros(2 * 256 + 1, dtype=torch.float16)[1:].view(2, 256), tr, sign, sc, 3, y=y)
    with pytest.raises(ex.Exl3Error, match=r"y(\[0\])?: data must be 16-byte aligned"):
        f(x, tr, sign, sc, 3, y=torch.empty(2 * 32 + 4, dtype=torch.float16)[4:].view(2, 32))
    with pytest.raises(ex.Exl3Error, match="must be on a GPU device"):
        f(x, tr, sign, sc, 3, y=y)


def test_gemv_multi_rejects_bad_tensors():
    x, tr, sign, sc, y = case()
    with pytest.raises(ex.Exl3Error, match="ys: 1 outputs for 2 projections"):
        ex.gemv_multi(x, [(tr, sc), (tr, sc)], sign, 3, ys=[y])
    with pytest.raises(ex.Exl3Error, match=r"trellis\[1\].*elements"):
        ex.gemv_multi(x, [(tr, sc), (tr[:1], sc)], sign, 3, ys=[y, y.clone()])
    with pytest.raises(ex.Exl3Error, match="must be on a GPU device"):
        ex.gemv_multi(x, [(tr, sc)], sign, 3, ys=[y])


def test_decode_and_encode_reject_bad_tensors():
    words = torch.zeros((4, 48), dtype=torch.int16)
    with pytest.raises(ex.Exl3Error, match="words.*elements"):
        ex.decode_tile(words, 4, out=torch.empty((4, 256), dtype=torch.float16))
    with pytest.raises(ex.Exl3Error, match="out: dtype"):
        ex.decode_tile(words, 3, out=torch.empty((4, 256), dtype=torch.float32))
    w = torch.zeros((4, 256), dtype=torch.float32)
    ws = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(ex.Exl3Error, match="w: dtype"):
        ex.encode_tiles(w.double(), 3, workspace=ws)
    with pytest.raises(ex.Exl3Error, match="costs.*elements"):
        ex.encode_tiles(w, 3, workspace=ws, costs=torch.empty(3, dtype=torch.float32))
    with pytest.raises(ex.Exl3Error, match="must be on a GPU device"):
        ex.encode_tiles(w, 3, workspace=ws)


def test_gemv_without_workspace_allocates_none(monkeypatch):
    # gemv() hands the library a null workspace instead of allocating one per
    # call (the GEMV needs none); gemm() and linear() still size one
    calls = []

    class FakeLib:
        def __getattr__(self, name):
            def f(*args):
                calls.append((name, args))
                return 0
            return f

    def no_workspace(*a, **k):
        raise AssertionError("a workspace was allocated")

    monkeypatch.setattr(ex, "load", lambda: FakeLib())
    monkeypatch.setattr(ex, "_on_gpu", lambda **t: None)
    monkeypatch.setattr(ex, "_stream", lambda s: 0)
    monkeypatch.setattr(ex, "Workspace", no_workspace)
    x, tr, sign, sc, y = case()
    ex.gemv(x, tr, sign, sc, 3, y=y)
    name, args = calls[-1]
    assert name == "exl3_gemv" and args[9] == 0 and args[10] == 0
    with pytest.raises(AssertionError, match="workspace was allocated"):
        ex.gemm(x, tr, sign, sc, 3, y=y)
