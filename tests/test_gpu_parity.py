"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

decode_tile must match bit for bit; gemv / gemm must be within a relative
Frobenius error of 1e-3 of the float64 oracle, every element within 1e-2 of
the reference's root mean square (tests/_parity.py).  Every input comes from the
seeded generators in `synth`; every expected value from `oracle`.
"""
import numpy as np
import pytest

import synth
from _parity import assert_close, strip_rows
from oracle import exl3_oracle as O

pytestmark = pytest.mark.gpu

TOL = 1e-3


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


def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def rel_fro(y, ref):
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def run_linear(torch, fn, words, x, sign, scale, K, ws=None, cb=0):
    import decode_gemm_exl3_amd as ex
    y = getattr(ex, fn)(to_dev(torch, x), to_dev(torch, words), to_dev(torch, sign), to_dev(torch, scale), K,
                        workspace=ws, codebook=cb)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# --------------------------------------------------------------- decode -----
def decode_gpu(torch, words, K, cb=0):
    import decode_gemm_exl3_amd as ex
    w = to_dev(torch, words.reshape(-1, 16 * K))
    out = ex.decode_tile(w, K, codebook=cb)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("K", range(1, 9))
def test_decode_random_tiles_bit_exact(torch_cuda, K):
    log(f"decode random K={K}")
    rng = np.random.default_rng(1000 + K)
    for T in (1, 3, 4, 17, 1000):  # ragged tile counts
        words = rng.integers(0, 65536, (T, 16 * K), dtype=np.uint16)
        got = decode_gpu(torch_cuda, words, K)
        ref = O.fp16_bits(O.decode_tiles(words, K))
        assert np.array_equal(got, ref), (K, T, np.argwhere(got != ref)[:5])


@pytest.mark.parametrize("K", range(1, 9))
def test_decode_structured_streams(torch_cuda, K):
    log(f"decode structured K={K}")
    nbits = 256 * K
    tiles = [np.zeros(16 * K, np.uint16), np.full(16 * K, 0xFFFF, np.uint16),
             np.full(16 * K, 0xA5C3, np.uint16), np.full(16 * K, 0x0001, np.uint16)]
    for p in list(range(0, 40)) + [nbits - 20, nbits - 16, nbits - 1] + list(range(16 * K - 8, 16 * K + 8)):
        w = np.zeros(16 * K, np.uint16)
        w[(p % nbits) // 16] = 1 << (p % 16)
        tiles.append(w)
    words = np.stack(tiles)
    got = decode_gpu(torch_cuda, words, K)
    ref = O.fp16_bits(O.decode_tiles(words, K))
    assert np.array_equal(got, ref)
    assert (got[0] == 0xB1E7).all() and (got[1] == 0xBEB4).all()


def test_decode_all_states_k8(torch_cuda):
    # at K=8, state i = byte_i | byte_{i+1} << 8: tiles of bytes (a, b0, a, b1, ...)
    # visit every (lo, hi) byte pair, i.e. all 65536 states, in 512 tiles
    log("decode all states K=8")
    tiles = []
    for a in range(256):
        for half in range(2):
            bts = np.zeros(256, np.uint8)
            bts[0::2] = a
            bts[1::2] = np.arange(128) + 128 * half
            tiles.append(bts.view(np.uint16))
    words = np.stack(tiles)
    st = O.tile_states(words, 8)
    assert len(np.unique(st)) == 65536
    got = decode_gpu(torch_cuda, words, 8)
    assert np.array_equal(got, O.fp16_bits(O.decode_tiles(words, 8)))


def test_decode_deterministic(torch_cuda):
    rng = np.random.default_rng(3)
    words = rng.integers(0, 65536, (4096, 48), dtype=np.uint16)
    a = decode_gpu(torch_cuda, words, 3)
    b = decode_gpu(torch_cuda, words, 3)
    assert np.array_equal(a, b)


# --------------------------------------------------- byte-sum codebook -----
@pytest.mark.parametrize("K", range(1, 9))
def test_decode_codebook1_bit_exact(torch_cuda, K):
    log(f"decode codebook 1 K={K}")
    rng = np.random.default_rng(1100 + K)
    for T in (1, 5, 1000):
        words = rng.integers(0, 65536, (T, 16 * K), dtype=np.uint16)
        got = decode_gpu(torch_cuda, words, K, cb=1)
        ref = O.fp16_bits(O.decode_tiles(words, K, cb=1))
        assert np.array_equal(got, ref), (K, T, np.argwhere(got != ref)[:5])
    zero = decode_gpu(torch_cuda, np.zeros((1, 16 * K), np.uint16), K, cb=1)
    assert (zero == 0xB168).all()  # c'(0), worked by hand in tests/golden/codebook1_examples.txt


def test_decode_codebook1_all_states_k8(torch_cuda):
    log("decode codebook 1 all states K=8")
    tiles = []
    for a in range(256):
        for half in range(2):
            bts = np.zeros(256, np.uint8)
            bts[0::2] = a
            bts[1::2] = np.arange(128) + 128 * half
            tiles.append(bts.view(np.uint16))
    words = np.stack(tiles)
    got = decode_gpu(torch_cuda, words, 8, cb=1)
    assert np.array_equal(got, O.fp16_bits(O.decode_tiles(words, 8, cb=1)))


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("fn", ["gemv", "gemm"])
def test_linear_codebook1_small_shapes(torch_cuda, fn, K):
    for (n_in, n_out) in [(128, 16), (384, 272), (1024, 1040)]:
        for m in ((1, 3, 8, 16) if fn == "gemv" else (1, 33, 300)):
            log(f"{fn} codebook 1 K={K} n_in={n_in} n_out={n_out} m={m}")
            words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [17, K, n_in, n_out, m])
            ref = O.linear(x, words, sign, scale, K, cb=1)
            y = run_linear(torch_cuda, fn, words, x, sign, scale, K, cb=1)
            assert np.isfinite(y).all()
            assert_close(y, ref, (fn, K, n_in, n_out, m))
            if fn == "gemv" and m == 16:  # the pre-rotated instance: same bits
                import decode_gemm_exl3_amd as ex
                y_pre = run_linear(torch_cuda, fn, words, x, sign, scale, K, ws=ex.Workspace(n_in, n_out, K, m), cb=1)
                assert np.array_equal(y_pre.view(np.uint16), y.view(np.uint16)), ("pre-pass", K, n_in, n_out, m)
            if n_in == 1024:  # the codebook is in use: codebook 0 gives another result
                assert rel_fro(y, O.linear(x, words, sign, scale, K)) > 0.5


def test_codebook1_workloads(torch_cuda):
    import decode_gemm_exl3_amd as ex
    rng = np.random.default_rng(4)
    cases = [("gemv", synth.Matmul("gate_k4_cb1", 4096, 14336, 4, 1, [0, 6, 0])),
             ("gemv", synth.Matmul("down_k3_cb1_m8", 14336, 4096, 3, 8, [0, 6, 1])),
             ("gemm", synth.Matmul("attn_8192_k4_cb1", 8192, 8192, 4, 2048, [0, 6, 2]))]
    ws = ex.Workspace(14336, 14336, 8, 2048)
    for fn, mm in cases:
        log(f"{fn} codebook 1 {mm.name}")
        words, x, sign, scale = synth.draw(mm)
        y = run_linear(torch_cuda, fn, words, x, sign, scale, mm.K, ws=ws, cb=1)
        rows = strip_rows(mm.n_out, rng)
        assert_close(y[:, rows], O.linear_rows(x, words, sign, scale, mm.K, rows, cb=1), mm.name)


def test_gemv_multi_codebook1(torch_cuda):
    import decode_gemm_exl3_amd as ex
    words, x, sign, scales = group_case(1024, (272, 48, 16), 5, 2, 500)
    ys = ex.gemv_multi(to_dev(torch_cuda, x), [(to_dev(torch_cuda, w), to_dev(torch_cuda, sc)) for w, sc in zip(words, scales)],
                       to_dev(torch_cuda, sign), 5, codebook=1)
    torch_cuda.cuda.synchronize()
    for w, sc, y in zip(words, scales, ys):
        assert_close(y.cpu().numpy(), O.linear(x, w, sign, sc, 5, cb=1), 'gemv_multi codebook 1')


# ----------------------------------------------------------------- gemv -----
TINY = [(128, 16), (128, 32), (256, 48), (384, 272), (1024, 1040)]


@pytest.mark.parametrize("K", range(1, 9))
@pytest.mark.parametrize("fn", ["gemv", "gemm"])
def test_linear_small_shapes(torch_cuda, fn, K):
    for (n_in, n_out) in TINY:
        for m in ((1, 2, 3, 4, 5, 8, 9, 13, 16) if fn == "gemv" else (1, 7, 16, 33)):
            log(f"{fn} K={K} n_in={n_in} n_out={n_out} m={m}")
            words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [7, K, n_in, n_out, m])
            ref = O.linear(x, words, sign, scale, K)
            y = run_linear(torch_cuda, fn, words, x, sign, scale, K)
            assert np.isfinite(y).all()
            assert_close(y, ref, (fn, K, n_in, n_out, m))
            if fn == "gemv" and m >= 14:
                # with a workspace these rows are rotated by the pre-pass and
                # copied (the kernel instance for pre-rotated input): same bits
                import decode_gemm_exl3_amd as ex
                y_pre = run_linear(torch_cuda, fn, words, x, sign, scale, K, ws=ex.Workspace(n_in, n_out, K, m))
                assert np.array_equal(y_pre.view(np.uint16), y.view(np.uint16)), ("pre-pass", K, n_in, n_out, m)


def test_gemv_split_and_ragged(torch_cuda):
    # long inputs (several LDS chunks at m = 8) and strip counts that leave the
    # persistent workgroups with unequal strip counts
    import decode_gemm_exl3_amd as ex
    for (n_in, n_out, K, m) in [(4096, 1040, 3, 1), (2048, 4112, 2, 6), (14336, 256, 4, 8), (8192, 48, 5, 3)]:
        log(f"gemv split n_in={n_in} n_out={n_out} K={K} m={m}")
        words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [8, n_in, n_out, K, m])
        ref = O.linear(x, words, sign, scale, K)
        ws = ex.Workspace(n_in, n_out, K, 8)
        for rep in range(2):  # the same workspace twice in a row
            y = run_linear(torch_cuda, "gemv", words, x, sign, scale, K, ws=ws)
            assert_close(y, ref, (n_in, n_out, K, m, rep))


def test_gemv_rotation_pre_pass_and_in_kernel(torch_cuda):
    # with a workspace, an input of m >= 14 rows, or a long one of m >= 2 rows,
    # is rotated once by a pre-pass; without one every workgroup rotates it:
    # both against the oracle, on chunked and unchunked inputs, with row counts
    # that leave the copy's last batch of groups part-filled, and the two
    # results against each other
    import decode_gemm_exl3_amd as ex
    torch = torch_cuda
    for (n_in, n_out, K, m) in [(14336, 272, 3, 8), (28672, 64, 2, 2), (12288, 4112, 5, 5), (4096, 528, 4, 16),
                                (8192, 1040, 4, 4), (14336, 4096, 2, 7), (28672, 208, 3, 3), (4096, 1024, 2, 14),
                                (28672, 96, 5, 16)]:
        log(f"gemv rotation paths n_in={n_in} n_out={n_out} K={K} m={m}")
        words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [21, n_in, n_out, K, m])
        ref = O.linear(x, words, sign, scale, K)
        y_pre = run_linear(torch, "gemv", words, x, sign, scale, K, ws=ex.Workspace(n_in, n_out, K, m))
        y_in = ex.gemv_multi(to_dev(torch, x), [(to_dev(torch, words), to_dev(torch, scale))], to_dev(torch, sign), K)[0]
        torch.cuda.synchronize()
        y_in = y_in.cpu().numpy()
        assert_close(y_pre, ref, ("pre-pass", n_in, n_out, K, m))
        assert_close(y_in, ref, ("in-kernel", n_in, n_out, K, m))
        # the same rotation arithmetic in both places: the same bits
        assert np.array_equal(y_pre.view(np.uint16), y_in.view(np.uint16)), (n_in, n_out, K, m)


def test_workspace_reuse_across_shapes_and_m(torch_cuda):
    import decode_gemm_exl3_amd as ex
    ws = ex.Workspace(4096, 4096, 8, 64)
    torch = torch_cuda
    for (fn, m, K) in [("gemm", 40, 3), ("gemv", 8, 4), ("gemv", 1, 2), ("gemm", 3, 5), ("gemv", 5, 3)]:
        log(f"reuse {fn} m={m} K={K}")
        words, x, sign, scale = synth.random_case(4096, 4096, K, m, [9, m, K])
        ref = O.linear(x, words, sign, scale, K)
        y = run_linear(torch, fn, words, x, sign, scale, K, ws=ws)
        assert_close(y, ref, (fn, m, K))
    # a workspace full of garbage must not matter
    ws.buf.fill_(0xA5)
    words, x, sign, scale = synth.random_case(4096, 4096, 3, 2, [9, 2, 3])
    y = run_linear(torch, "gemv", words, x, sign, scale, 3, ws=ws)
    assert_close(y, O.linear(x, words, sign, scale, 3), 'garbage workspace')


def test_gemv_gemm_agree_and_deterministic(torch_cuda):
    words, x, sign, scale = synth.random_case(2048, 1024, 4, 4, 77)
    ref = O.linear(x, words, sign, scale, 4)
    y1 = run_linear(torch_cuda, "gemv", words, x, sign, scale, 4)
    y2 = run_linear(torch_cuda, "gemv", words, x, sign, scale, 4)
    y3 = run_linear(torch_cuda, "gemm", words, x, sign, scale, 4)
    assert_close(y1, ref, "gemv")
    assert_close(y3, ref, "gemm")
    assert rel_fro(y1.astype(np.float64), y3.astype(np.float64)) <= 2 * TOL
    # the waves' partial sums are added in a fixed order: repeated calls agree bit for bit
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_graph_replays_match_eager(torch_cuda):
    """A GEMV, a fused two-projection GEMV and a split-k GEMM (m = 300: the
    256-row kernel, its rotation pre-pass and the ordered reduce) captured in one
    HIP graph and replayed with new inputs copied in before each replay, eager
    launches of the same calls in between: every replay equals the eager result
    bit for bit, and the eager results match the oracle."""
    import decode_gemm_exl3_amd as ex
    torch = torch_cuda
    w1, x1, s1, c1 = synth.random_case(4096, 1024, 3, 1, [31, 1])
    wm, xm, sm, cm = group_case(2048, (512, 256), 4, 2, 32)
    w3, x3, s3, c3 = synth.random_case(4096, 256, 2, 300, [33, 300])
    d = {k: to_dev(torch, v) for k, v in dict(w1=w1, s1=s1, c1=c1, w3=w3, s3=s3, c3=c3,
                                              wm0=wm[0], wm1=wm[1], cm0=cm[0], cm1=cm[1], sm=sm).items()}
    xs = {"x1": to_dev(torch, x1), "xm": to_dev(torch, xm), "x3": to_dev(torch, x3)}
    ws_graph, ws_eager = ex.Workspace(4096, 256, 2, 300), ex.Workspace(4096, 256, 2, 300)
    f16 = dict(dtype=torch.float16, device="cuda")
    yg = [torch.empty((1, 1024), **f16), torch.empty((2, 512), **f16), torch.empty((2, 256), **f16),
          torch.empty((300, 256), **f16)]
    ye = [torch.empty_like(y) for y in yg]

    def calls(y, ws):
        ex.gemv(xs["x1"], d["w1"], d["s1"], d["c1"], 3, y=y[0])
        ex.gemv_multi(xs["xm"], [(d["wm0"], d["cm0"]), (d["wm1"], d["cm1"])], d["sm"], 4, ys=[y[1], y[2]])
        ex.gemm(xs["x3"], d["w3"], d["s3"], d["c3"], 2, workspace=ws, y=y[3])

    calls(ye, ws_eager)  # outside capture first: one-time per-device set-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(yg, ws_graph)
    torch.cuda.synchronize()
    rng = np.random.default_rng(34)
    for rep in range(4):
        log(f"graph replay {rep}")
        new = {"x1": rng.standard_normal(x1.shape), "xm": rng.standard_normal(xm.shape),
               "x3": rng.standard_normal(x3.shape)}
        new = {k: v.astype(np.float16) for k, v in new.items()}
        for k, v in new.items():
            xs[k].copy_(to_dev(torch, v))
        calls(ye, ws_eager)
        for y in yg:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(yg, ye)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rep, i)
        if rep == 0:
            ref = [O.linear(new["x1"], w1, s1, c1, 3), O.linear(new["xm"], wm[0], sm, cm[0], 4),
                   O.linear(new["xm"], wm[1], sm, cm[1], 4), O.linear(new["x3"], w3, s3, c3, 2)]
            for i, (y, r) in enumerate(zip(ye, ref)):
                assert_close(y.cpu().numpy(), r, i)


def test_zero_m_is_noop(torch_cuda):
    import decode_gemm_exl3_amd as ex
    torch = torch_cuda
    words, x, sign, scale = synth.random_case(128, 16, 2, 1, 1)
    y = torch.full((0, 16), 7, dtype=torch.float16, device="cuda")
    ex.gemv(to_dev(torch, x[:0]), to_dev(torch, words), to_dev(torch, sign), to_dev(torch, scale), 2, y=y)
    torch.cuda.synchronize()


# ------------------------------------------- fused multi-projection GEMV -----
def run_multi(torch, words, x, sign, scales, K, ws=None):
    import decode_gemm_exl3_amd as ex
    ys = ex.gemv_multi(to_dev(torch, x), [(to_dev(torch, w), to_dev(torch, sc)) for w, sc in zip(words, scales)],
                       to_dev(torch, sign), K, workspace=ws)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def group_case(n_in, n_outs, K, m, seed):
    mms = [synth.Matmul(f"p{i}", n_in, n_out, K, m, [seed, i]) for i, n_out in enumerate(n_outs)]
    return synth.draw_group(mms)


@pytest.mark.parametrize("K", range(1, 9))
def test_gemv_multi_small_shapes(torch_cuda, K):
    for n_in, n_outs in [(128, (16,)), (256, (16, 48)), (512, (272, 16, 32)), (1024, (64, 1040, 16, 48))]:
        for m in (1, 3, 8):
            log(f"gemv_multi K={K} n_in={n_in} n_outs={n_outs} m={m}")
            words, x, sign, scales = group_case(n_in, n_outs, K, m, 300 + K)
            ys = run_multi(torch_cuda, words, x, sign, scales, K)
            for i, (w, sc, y) in enumerate(zip(words, scales, ys)):
                assert y.shape == (m, sc.shape[0])
                assert_close(y, O.linear(x, w, sign, sc, K), (K, n_in, n_outs, m, i))
    # 16 rows with a workspace: the pre-pass and the pre-rotated instance over
    # several projections, bit for bit the in-kernel rotation's result
    import decode_gemm_exl3_amd as ex
    n_in, n_outs, m = 1024, (64, 1040, 16, 48), 16
    words, x, sign, scales = group_case(n_in, n_outs, K, m, 310 + K)
    ys = run_multi(torch_cuda, words, x, sign, scales, K)
    ys_pre = run_multi(torch_cuda, words, x, sign, scales, K, ws=ex.Workspace(n_in, max(n_outs), K, m))
    for i, (w, sc, y, yp) in enumerate(zip(words, scales, ys, ys_pre)):
        assert_close(y, O.linear(x, w, sign, sc, K), (K, n_in, n_outs, m, i))
        assert np.array_equal(yp.view(np.uint16), y.view(np.uint16)), ("pre-pass", K, i)


def test_gemv_multi_matches_separate_calls(torch_cuda):
    # one launch over q/k/v-like and gate/up-like groups against one gemv per projection
    for n_in, n_outs, K, m in [(4096, (4096, 1024, 1024), 5, 1), (4096, (14336, 14336), 3, 4)]:
        log(f"gemv_multi vs gemv n_in={n_in} n_outs={n_outs} K={K} m={m}")
        words, x, sign, scales = group_case(n_in, n_outs, K, m, 400)
        ys = run_multi(torch_cuda, words, x, sign, scales, K)
        rng = np.random.default_rng(2)
        for w, sc, y in zip(words, scales, ys):
            y1 = run_linear(torch_cuda, "gemv", w, x, sign, sc, K)
            assert_close(y.astype(np.float64), y1.astype(np.float64), 'gemv_multi against gemv')
            rows = strip_rows(sc.shape[0], rng)
            assert_close(y[:, rows], O.linear_rows(x, w, sign, sc, K, rows), (n_in, n_outs, K, m))


# ------------------------------------- medium m and the GEMM's row blocks -----
def check_case(torch, mm, fn, ws):
    log(f"{fn} {mm.name} n_in={mm.n_in} n_out={mm.n_out} K={mm.K} m={mm.m}")
    words, x, sign, scale = synth.draw(mm)
    y = run_linear(torch, fn, words, x, sign, scale, mm.K, ws=ws)
    rows = strip_rows(mm.n_out, np.random.default_rng(1))
    assert_close(y[:, rows], O.linear_rows(x, words, sign, scale, mm.K, rows), mm.name)


def test_medium_m_gemv_and_split_gemm(torch_cuda):
    # batched decode / chunked prefill sizes: the GEMV up to 16 rows, the GEMM
    # with its input dimension split across workgroups below ~256 blocks
    import decode_gemm_exl3_amd as ex
    ws = ex.Workspace(14336, 14336, 8, 256)
    rng = np.random.default_rng(5)
    for fn, n_in, n_out, K, m in [("gemv", 4096, 14336, 3, 12), ("gemv", 14336, 4096, 4, 16),
                                  ("gemm", 4096, 14336, 3, 17), ("gemm", 14336, 4096, 2, 64),
                                  ("gemm", 4096, 4096, 4, 256), ("gemm", 4096, 1024, 5, 100)]:
        mm = synth.Matmul(f"{fn}_m{m}", n_in, n_out, K, m, [0, 7, n_in, n_out, m])
        check_case(torch_cuda, mm, fn, ws)


def test_gemm_row_block_boundaries(torch_cuda):
    # 64-, 128- and 256-row blocks are chosen by m: both sides of each switch,
    # with split and unsplit input dimensions
    for n_in, n_out, K in [(1024, 528, 3), (2048, 4112, 4)]:
        for m in (63, 64, 65, 127, 128, 129):
            log(f"gemm blocks n_in={n_in} n_out={n_out} K={K} m={m}")
            words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [23, n_in, m])
            y = run_linear(torch_cuda, "gemm", words, x, sign, scale, K)
            assert_close(y, O.linear(x, words, sign, scale, K), (n_in, n_out, K, m))


@pytest.mark.parametrize("K", range(1, 9))
def test_gemm_256_row_blocks(torch_cuda, K):
    # the four-wave 256-row kernel (m > 128): ragged and whole row blocks, output
    # counts that leave a block partly empty, both codebooks, and the input
    # dimension split into 1-step pieces (the main loop's one-step tail only),
    # into two 5-step pieces (two passes of the two-step loop, then the tail) and
    # not split (256 blocks, one pass of the loop)
    for n_in, n_out, m, cb in [(128, 272, 129, 0), (384, 48, 256, 1), (1024, 528, 513, 1),
                               (640, 4096, 2048, 0), (128, 4096, 4096, 1)]:
        log(f"gemm 256-row blocks K={K} n_in={n_in} n_out={n_out} m={m} codebook={cb}")
        words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [29, K, n_in, m])
        y = run_linear(torch_cuda, "gemm", words, x, sign, scale, K, cb=cb)
        assert np.isfinite(y).all()
        assert_close(y, O.linear(x, words, sign, scale, K, cb=cb), (K, n_in, n_out, m, cb))
        if m == 513:  # no atomics, splits added in order: the same bits every time
            y2 = run_linear(torch_cuda, "gemm", words, x, sign, scale, K, cb=cb)
            assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


def test_gemm_seeded_random_shapes(torch_cuda):
    # shapes drawn once from a fixed seed across both GEMM kernels, bits,
    # codebooks, ragged m and output counts, split and unsplit inputs
    rng = np.random.default_rng(2024)
    for case in range(24):
        K = int(rng.integers(1, 9))
        cb = int(rng.integers(0, 2))
        n_in = 128 * int(rng.integers(1, 13))
        n_out = 16 * int(rng.integers(1, 130))
        m = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(129, 700))]))
        log(f"gemm random case {case}: K={K} cb={cb} n_in={n_in} n_out={n_out} m={m}")
        words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [43, case])
        y = run_linear(torch_cuda, "gemm", words, x, sign, scale, K, cb=cb)
        assert_close(y, O.linear(x, words, sign, scale, K, cb=cb), (K, cb, n_in, n_out, m))


def test_gemv_seeded_random_shapes(torch_cuda):
    # fused launches of 1..4 projections drawn from a fixed seed: bits,
    # codebooks, m up to 16, input lengths up to 40 blocks (several LDS chunks
    # at larger m), output counts that leave workgroups unevenly loaded
    import decode_gemm_exl3_amd as ex
    rng = np.random.default_rng(2025)
    for case in range(16):
        K = int(rng.integers(1, 9))
        cb = int(rng.integers(0, 2))
        n_in = 128 * int(rng.integers(1, 41))
        m = int(rng.integers(1, 17))
        n_outs = tuple(16 * int(rng.integers(1, 200)) for _ in range(int(rng.integers(1, 5))))
        log(f"gemv random case {case}: K={K} cb={cb} n_in={n_in} n_outs={n_outs} m={m}")
        words, x, sign, scales = group_case(n_in, n_outs, K, m, 600 + case)
        ys = ex.gemv_multi(to_dev(torch_cuda, x), [(to_dev(torch_cuda, w), to_dev(torch_cuda, sc))
                                                     for w, sc in zip(words, scales)], to_dev(torch_cuda, sign), K,
                           codebook=cb)
        torch_cuda.cuda.synchronize()
        for w, sc, y in zip(words, scales, ys):
            assert_close(y.cpu().numpy(), O.linear(x, w, sign, sc, K, cb=cb), (K, cb, n_in, n_outs, m))


def test_linear_dispatch(torch_cuda):
    # the measured table: GEMV for small m * n_in, the split GEMM beyond
    for n_in, n_out, K, m in [(1024, 272, 3, 1), (1024, 272, 3, 16), (4096, 48, 4, 33), (14336, 64, 2, 12),
                              (4096, 528, 4, 14), (2048, 64, 2, 13), (8192, 272, 3, 13)]:
        log(f"linear n_in={n_in} n_out={n_out} K={K} m={m}")
        words, x, sign, scale = synth.random_case(n_in, n_out, K, m, [19, n_in, m])
        y = run_linear(torch_cuda, "linear", words, x, sign, scale, K)
        assert_close(y, O.linear(x, words, sign, scale, K), (n_in, n_out, K, m))


# ------------------------------------------------------------- edge cases ----
def test_degenerate_inputs(torch_cuda):
    # x = 0 and out_scale = 0 give exactly zero on every path; inputs near the
    # top of the fp16 range do not overflow the rotated input (x'/128 is never
    # larger than max|x|), checked against the oracle with a small scale
    for fn, m in (("gemv", 1), ("gemv", 5), ("gemm", 40), ("gemm", 300)):
        words, x, sign, scale = synth.random_case(1024, 272, 3, m, [71, m])
        log(f"degenerate {fn} m={m}")
        y = run_linear(torch_cuda, fn, words, np.zeros_like(x), sign, scale, 3)
        assert (y.view(np.uint16) & 0x7FFF == 0).all()
        y = run_linear(torch_cuda, fn, words, x, sign, np.zeros_like(scale), 3)
        assert (y.view(np.uint16) & 0x7FFF == 0).all()
        big = (np.sign(x.astype(np.float32)) * 60000).astype(np.float16)  # all-same-magnitude, worst case for x'
        tiny = np.full_like(scale, 1e-4)
        y = run_linear(torch_cuda, fn, words, big, sign, tiny, 3)
        assert_close(y, O.linear(big, words, sign, tiny, 3), (fn, m, "large inputs"))


def test_largest_weight_matrix(torch_cuda):
    # the largest weight one call takes at K = 8 (32768 x 65488, just under the
    # 2^31 - 2^20 bytes read through 32-bit offsets), one output per strip
    # compared; one more strip is refused
    import decode_gemm_exl3_amd as ex
    n_in, n_out, K = 32768, 65488, 8
    assert n_in * n_out * K // 8 < (1 << 31) - (1 << 20) <= n_in * (n_out + 16) * K // 8
    log(f"largest weight {n_in}x{n_out} K={K}")
    words, x, sign, scale = synth.random_case(n_in, n_out, K, 1, [73])
    y = run_linear(torch_cuda, "gemv", words, x, sign, scale, K)
    rows = strip_rows(n_out, np.random.default_rng(73))
    assert_close(y[:, rows], O.linear_rows(x, words, sign, scale, K, rows), "largest weight")
    lib = ex.load()
    A = 1 << 20
    assert lib.exl3_gemv(A, 1, A, A, A, n_in, n_out + 16, K, A + 64, None, 0, None) == -2


def test_gemm_largest_m(torch_cuda):
    # the most rows the GEMM takes at n_in = 8192 (130816: the rotated input
    # just under 2^31 - 2^20 bytes), sampled rows of the output compared; one
    # more block of rows is refused
    import decode_gemm_exl3_amd as ex
    torch = torch_cuda
    n_in, n_out, K, m = 8192, 16, 4, 130816
    log(f"gemm largest m={m} n_in={n_in}")
    words, _, sign, scale = synth.random_case(n_in, n_out, K, 1, [74])
    x = torch.randn((m, n_in), device="cuda").half()
    ws = ex.Workspace(n_in, n_out, K, m)
    y = ex.gemm(x, to_dev(torch, words), to_dev(torch, sign), to_dev(torch, scale), K, workspace=ws)
    torch.cuda.synchronize()
    sel = np.unique(np.concatenate([np.arange(64), m - 64 + np.arange(64),
                                    np.random.default_rng(74).integers(0, m, 256)]))
    xs = x[torch.from_numpy(sel).cuda()].cpu().numpy()
    assert_close(y[torch.from_numpy(sel).cuda()].cpu().numpy(), O.linear(xs, words, sign, scale, K), "largest m")
    lib = ex.load()
    A = 1 << 20
    assert lib.exl3_gemm(A, m + 256, A, A, A, n_in, n_out, K, A + 64, A + 128, 1 << 40, None) == -2
