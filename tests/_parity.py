"""Helpers of the GPU parity tests: device copies, the launches through the
binding, the rows compared and the bar they are held to.

The bar for a GEMV or GEMM output against the float64 oracle, on the outputs
compared: a relative Frobenius error of at most 1e-3, and every element within
1e-2 of the root mean square of the reference (so that one wrong element,
whose share of the Frobenius norm over thousands of outputs is tiny, still
fails).  The per-element budget of a correct result is about 4e-3 of the rms:
the rotated input rounded to fp16 (2^-12 relative per term, ~2.4e-4 of the rms
as a standard deviation, ~1.2e-3 at five deviations) plus the fp16 rounding of
the output (2^-11 of |y|, up to ~2.4e-3 of the rms at |y| = 5 rms).
"""
import numpy as np

TOL_FRO = 1e-3
TOL_ELEM = 1e-2


def log(msg):
    print(f"[case] {msg}", flush=True)


def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def rel_fro(y, ref):
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def worst_elem(y, ref):
    """Largest |y - ref| over the root mean square of ref."""
    y = np.asarray(y, np.float64)
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(y - ref)) / max(rms, 1e-300))


def assert_close(y, ref, what):
    y = np.asarray(y, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.isfinite(y).all(), what
    err, worst = rel_fro(y, ref), worst_elem(y, ref)
    assert err <= TOL_FRO and worst <= TOL_ELEM, (what, err, worst)
    return err, worst


def strip_rows(n_out, rng):
    """Output features compared on a large output: one drawn at random from
    every 16-row strip (so every strip and every 256-wide GEMM block is
    looked at), plus the first and the last strip whole."""
    n_strips = n_out // 16
    rows = np.arange(n_strips) * 16 + rng.integers(0, 16, n_strips)
    return np.unique(np.concatenate([np.arange(16), n_out - 16 + np.arange(16), rows]))


def run_launch(torch, ex, fn, words_list, x, sign, scales, K, ws=None, cb=0):
    """One call: gemv_multi for a fused group, else the named single-projection
    call.  Returns the outputs as NumPy fp16 arrays."""
    if fn == "gemv_multi":
        ys = ex.gemv_multi(to_dev(torch, x), [(to_dev(torch, w), to_dev(torch, sc)) for w, sc in zip(words_list, scales)],
                           to_dev(torch, sign), K, workspace=ws, codebook=cb)
    else:
        ys = [getattr(ex, fn)(to_dev(torch, x), to_dev(torch, words_list[0]), to_dev(torch, sign),
                              to_dev(torch, scales[0]), K, workspace=ws, codebook=cb)]
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]
