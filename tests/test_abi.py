"""Host-side checks of the C ABI: the library loads, exports what the header
declares, sizes packed weights and workspaces, and rejects bad arguments before
touching the GPU.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import decode_gemm_exl3_amd as ex

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exl3.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(exl3_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ex.lib_path()):
        pytest.fail("libexl3.so is not built (run __graft_entry__.build())")
    return ex.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == {"exl3_pack_info", "exl3_decode_tile", "exl3_gemv", "exl3_gemv_multi", "exl3_gemm",
                          "exl3_linear", "exl3_linear_noalloc", "exl3_encode_slot_bytes", "exl3_encode_tiles",
                          "exl3_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_pack_info_sizes(lib):
    for n_in, n_out, K, mm in [(4096, 4096, 4, 1), (14336, 4096, 3, 8), (8192, 28672, 2, 2048), (128, 16, 1, 1)]:
        info = ex.pack_info(n_in, n_out, K, mm)
        assert info["tiles_in"] == n_in // 16 and info["tiles_out"] == n_out // 16
        assert info["words_per_tile"] == 16 * K
        assert info["trellis_words"] == (n_in // 16) * (n_out // 16) * 16 * K
        assert info["trellis_bytes"] == n_in * n_out * K // 8 == 2 * info["trellis_words"]
        assert info["workspace_bytes"] >= mm * n_in * 2              # gemm: rotated input
    assert ex.pack_info(4096, 4096, 4, 1)["workspace_bytes"] < ex.pack_info(4096, 4096, 4, 64)["workspace_bytes"]
    # beyond 128 rows the GEMM stages its rotated input in whole 256-row blocks
    for mm in (129, 300, 513):
        rows = (mm + 255) // 256 * 256
        assert ex.pack_info(1024, 4096, 4, mm)["workspace_bytes"] >= rows * 1024 * 2


@pytest.mark.parametrize("args", [(100, 16, 4, 1), (128, 17, 4, 1), (128, 16, 0, 1), (128, 16, 9, 1),
                                  (128, 16, 4, 0), (0, 16, 4, 1), (-128, 16, 4, 1)])
def test_pack_info_rejects(lib, args):
    info = ex._PackInfo()
    assert lib.exl3_pack_info(*args, ctypes.byref(info)) == -1
    assert lib.exl3_pack_info(128, 16, 4, 1, None) == -1


def test_codebook_flag_in_bits(lib):
    info = ex._PackInfo()
    flag = ex.CODEBOOK_BYTE_SUM
    assert flag == 0x100
    assert lib.exl3_pack_info(4096, 4096, 4 | flag, 1, ctypes.byref(info)) == 0
    assert info.bits == 4 | flag and info.words_per_tile == 64 and info.trellis_bytes == 4096 * 4096 // 2
    for bad in (0 | flag, 9 | flag, 4 | 0x200, 4 | 0x10000, -4):
        assert lib.exl3_pack_info(4096, 4096, bad, 1, ctypes.byref(info)) == -1, hex(bad)
        assert lib.exl3_decode_tile(1, bad, 1, 2, None) == -1
        assert _gemv_call(lib, "exl3_gemv", bits=bad) == -1
        assert _gemv_call(lib, "exl3_gemm", bits=bad) == -1
    assert ex.bits_arg(3, 1) == 3 | flag and ex.bits_arg(3) == 3
    with pytest.raises(ex.Exl3Error):
        ex.bits_arg(3, 2)


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, 7):
        s = ex.status_string(code)
        assert isinstance(s, str) and s
    assert ex.status_string(-3).startswith("workspace")


def _gemv_call(lib, fn, x=0x1000, m=1, tr=0x2000, sg=0x3000, sc=0x4000, n_in=128, n_out=16, bits=4, y=0x5000,
               ws=0x6000, wsb=1 << 30):
    return getattr(lib, fn)(x, m, tr, sg, sc, n_in, n_out, bits, y, ws, wsb, None)


@pytest.mark.parametrize("fn", ["exl3_gemv", "exl3_gemm", "exl3_linear"])
def test_linear_argument_errors_return_before_launch(lib, fn):
    # every case is rejected on the host, so fake non-null pointers are never used
    assert _gemv_call(lib, fn, m=-1) == -1
    assert _gemv_call(lib, fn, n_in=100) == -1
    assert _gemv_call(lib, fn, n_out=24) == -1
    assert _gemv_call(lib, fn, bits=0) == -1
    assert _gemv_call(lib, fn, bits=9) == -1
    assert _gemv_call(lib, fn, x=None) == -1
    assert _gemv_call(lib, fn, tr=None) == -1
    assert _gemv_call(lib, fn, sg=None) == -1
    assert _gemv_call(lib, fn, sc=None) == -1
    assert _gemv_call(lib, fn, y=None) == -1
    assert _gemv_call(lib, fn, x=0x5000, y=0x5000) == -1  # aliasing
    for arg in ("x", "tr", "sg", "sc", "y", "ws"):  # every pointer 16-byte aligned
        assert _gemv_call(lib, fn, **{arg: 0x7008}) == -1, arg
    assert _gemv_call(lib, fn, m=0, x=None, y=None) == 0  # m == 0 is a no-op
    # weights of 2 GiB or more are refused (32-bit buffer offsets)
    assert _gemv_call(lib, fn, n_in=65536, n_out=65536, bits=4) == -2


def test_gemm_workspace_errors(lib):
    # gemm stages the rotated input in the workspace; gemv needs none
    assert _gemv_call(lib, "exl3_gemm", ws=None) == -3
    assert _gemv_call(lib, "exl3_gemm", wsb=16) == -3
    # exl3_linear sends large m to the GEMM
    assert _gemv_call(lib, "exl3_linear", m=64, ws=None) == -3


def test_pack_info_workspace_covers_split_partials(lib):
    # few output blocks (medium m) split the input dimension: the workspace
    # holds the rotated input and fp32 partial sums of up to 16 splits
    info = ex.pack_info(4096, 4096, 4, 256)
    assert info["workspace_bytes"] >= 256 * 4096 * 2 + 16 * 256 * 4096 * 4
    assert ex.pack_info(8192, 8192, 4, 2048)["workspace_bytes"] >= 2048 * 8192 * 2


def test_gemv_rejects_m_above_16(lib):
    assert _gemv_call(lib, "exl3_gemv", m=17) == -1


def _multi_call(lib, projs, x=0x1000, m=1, sg=0x1010, n_in=128, bits=4, n_proj=None, ws=None):
    arr = (ex._Proj * max(len(projs), 1))(*[ex._Proj(*p_) for p_ in projs])
    return lib.exl3_gemv_multi(x, m, sg, n_in, bits, arr if projs else None,
                               len(projs) if n_proj is None else n_proj, ws, 0, None)


def test_gemv_multi_argument_errors(lib):
    # (trellis, out_scale, y, n_out, reserved); fake pointers, never dereferenced
    good = [(0x110, 0x120, 0x130, 16, 0), (0x210, 0x220, 0x230, 32, 0)]
    assert _multi_call(lib, good, m=-1) == -1
    assert _multi_call(lib, good, m=17) == -1
    assert _multi_call(lib, good, n_in=100) == -1
    assert _multi_call(lib, good, bits=0) == -1
    assert _multi_call(lib, good, bits=9) == -1
    assert _multi_call(lib, [], n_proj=0) == -1
    assert _multi_call(lib, good, n_proj=5) == -1
    assert _multi_call(lib, good * 3) == -1                       # 6 > EXL3_GEMV_MAX_PROJ
    assert _multi_call(lib, good, x=None) == -1
    assert _multi_call(lib, good, sg=None) == -1
    assert _multi_call(lib, [(0, 0x120, 0x130, 16, 0)]) == -1
    assert _multi_call(lib, [(0x110, 0, 0x130, 16, 0)]) == -1
    assert _multi_call(lib, [(0x110, 0x120, 0, 16, 0)]) == -1
    assert _multi_call(lib, [(0x110, 0x120, 0x130, 24, 0)]) == -1          # n_out % 16
    assert _multi_call(lib, [(0x110, 0x120, 0x130, 0, 0)]) == -1
    assert _multi_call(lib, [(0x110, 0x120, 0x1000, 16, 0)]) == -1         # y aliases x
    assert _multi_call(lib, [(0x110, 0x120, 0x130, 16, 0), (0x210, 0x220, 0x130, 16, 0)]) == -1  # same y twice
    assert _multi_call(lib, good, m=0, x=None, sg=None) == 0              # m == 0 is a no-op
    assert _multi_call(lib, [(0x110, 0x120, 0x130, 65536, 0)], n_in=65536) == -2  # >= 2 GiB of weights
    # every pointer 16-byte aligned
    assert _multi_call(lib, good, x=0x1008) == -1
    assert _multi_call(lib, good, sg=0x1018) == -1
    assert _multi_call(lib, good, ws=0x2004) == -1
    for bad in ((0x118, 0x120, 0x130, 16, 0), (0x110, 0x122, 0x130, 16, 0), (0x110, 0x120, 0x131, 16, 0)):
        assert _multi_call(lib, [bad]) == -1


def test_encode_sizes_and_argument_errors(lib):
    for K in range(1, 9):
        assert lib.exl3_encode_slot_bytes(K) == 256 * (1 << (16 - K))
        assert lib.exl3_encode_slot_bytes(K | ex.CODEBOOK_BYTE_SUM) == 256 * (1 << (16 - K))
    assert lib.exl3_encode_slot_bytes(0) == -1 and lib.exl3_encode_slot_bytes(9) == -1
    big = 1 << 30
    w, words, ws = 0x1000, 0x2000, 0x3000  # fake pointers, never dereferenced
    assert lib.exl3_encode_tiles(w, 1, 0, words, None, ws, big, None) == -1       # bad bits
    assert lib.exl3_encode_tiles(w, -1, 4, words, None, ws, big, None) == -1      # n_tiles < 0
    assert lib.exl3_encode_tiles(None, 1, 4, words, None, ws, big, None) == -1
    assert lib.exl3_encode_tiles(w, 1, 4, None, None, ws, big, None) == -1
    assert lib.exl3_encode_tiles(w, 1, 4, words, None, None, big, None) == -3    # no workspace
    assert lib.exl3_encode_tiles(w, 1, 4, words, None, ws, 1000, None) == -3     # below one slot
    assert lib.exl3_encode_tiles(None, 0, 4, None, None, None, 0, None) == 0     # no tiles: no-op
    for args in ((w + 4, words, None, ws), (w, words + 2, None, ws), (w, words, 0x4004, ws), (w, words, None, ws + 8)):
        assert lib.exl3_encode_tiles(args[0], 1, 4, args[1], args[2], args[3], big, None) == -1  # misaligned


def test_decode_tile_argument_errors(lib):
    words, out = 0x1000, 0x2000  # fake pointers, never dereferenced
    assert lib.exl3_decode_tile(words, 0, 1, out, None) == -1
    assert lib.exl3_decode_tile(words, 9, 1, out, None) == -1
    assert lib.exl3_decode_tile(words, 4, -1, out, None) == -1
    assert lib.exl3_decode_tile(None, 4, 1, out, None) == -1
    assert lib.exl3_decode_tile(words, 4, 1, None, None) == -1
    assert lib.exl3_decode_tile(None, 4, 0, None, None) == 0
    assert lib.exl3_decode_tile(words + 2, 4, 1, out, None) == -1  # misaligned
    assert lib.exl3_decode_tile(words, 4, 1, out + 8, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("EXL3_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ex, "_LIB", None)
    with pytest.raises(ex.Exl3Error):
        ex.load()


def test_noalloc_rejects_before_any_launch(lib):
    # argument errors, and a GEMM input whose rotation would not fit the static
    # scratch (8192 rows of 8192 inputs: 128 MiB), return before any HIP call;
    # m == 0 is a no-op
    A = 1 << 20  # 16-byte aligned stand-ins: no call below reaches the device
    f = lib.exl3_linear_noalloc
    assert f(A, 8192, A, A, A, 8192, 16, 4, A + 64, None) == -2
    assert f(A, 4097, A, A, A, 8192, 16, 4, A + 64, None) == -2   # 4352 rows: 68 MiB
    assert f(A, 0, A, A, A, 8192, 16, 4, A + 64, None) == 0
    assert f(A, -1, A, A, A, 8192, 16, 4, A + 64, None) == -1
    assert f(A, 4, A, A, A, 100, 16, 4, A + 64, None) == -1
    assert f(A, 4, A, A, A, 8192, 16, 4, A + 8, None) == -1   # misaligned y
    assert f(A, 4, 0, A, A, 8192, 16, 4, A + 64, None) == -1  # null trellis


def test_gemm_rejects_rotated_input_of_2_gib(lib):
    # the rotated input is read through 32-bit offsets: 131072 rows of 8192
    # inputs (2 GiB) is refused before any launch, with any workspace
    A = 1 << 20
    big = 1 << 40
    assert lib.exl3_gemm(A, 131072, A, A, A, 8192, 16, 4, A + 64, A + 128, big, None) == -2
    assert lib.exl3_linear(A, 131072, A, A, A, 8192, 16, 4, A + 64, A + 128, big, None) == -2
