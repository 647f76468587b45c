"""Python binding of the EXL3 decode-matmul library (libexl3.so, HIP for gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/exl3.h.  PyTorch supplies device
memory and the current stream.  If the library has not been built, every call
raises; there is no other implementation behind these names.

Tensors:
  words / trellis : int16 (uint16 bit patterns), trellis shape [n_out/16, n_in/16, 16*bits]
  x               : float16 [m, n_in]
  sign            : float16 [n_in] (+-1)
  out_scale       : float16 [n_out]
  result y        : float16 [m, n_out]
Every call takes the bit width K and, as a keyword, the codebook (0: multiply,
mask-and-plant, half sum; 1: byte sum), passed to the ABI as one bits argument.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["Exl3Error", "lib_path", "load", "pack_info", "Workspace", "decode_tile", "gemv", "gemv_multi",
           "gemm", "linear", "linear_noalloc", "status_string", "MAX_PROJ", "CODEBOOK_BYTE_SUM", "bits_arg", "encode_slot_bytes",
           "encode_tiles"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None
MAX_PROJ = 4  # EXL3_GEMV_MAX_PROJ
GEMV_MAX_M = 16  # EXL3_GEMV_MAX_M
CODEBOOK_BYTE_SUM = 0x100  # EXL3_CODEBOOK_BYTE_SUM: flag in the bits argument selecting codebook 1


class Exl3Error(RuntimeError):
    pass


def lib_path() -> str:
    return os.environ.get("EXL3_LIB", os.path.join(_PKG, "libexl3.so"))


class _PackInfo(ctypes.Structure):
    _fields_ = [("n_in", ctypes.c_int32), ("n_out", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("max_m", ctypes.c_int32), ("tiles_in", ctypes.c_int32), ("tiles_out", ctypes.c_int32),
                ("words_per_tile", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("trellis_words", ctypes.c_int64), ("trellis_bytes", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64)]


class _Proj(ctypes.Structure):
    _fields_ = [("trellis", ctypes.c_void_p), ("out_scale", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n_out", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def load() -> ctypes.CDLL:
    """Load libexl3.so once; raise if it is missing (no fallback path exists)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise Exl3Error(f"{path} not found: build it with decode_gemm_exl3_amd._build.build()")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.exl3_pack_info.argtypes = [i32, i32, i32, i32, ctypes.POINTER(_PackInfo)]
    lib.exl3_pack_info.restype = ctypes.c_int
    lib.exl3_decode_tile.argtypes = [vp, i32, i64, vp, vp]
    lib.exl3_decode_tile.restype = ctypes.c_int
    for name in ("exl3_gemv", "exl3_gemm", "exl3_linear"):
        f = getattr(lib, name)
        f.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    lib.exl3_linear_noalloc.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, vp, vp]
    lib.exl3_linear_noalloc.restype = ctypes.c_int
    lib.exl3_gemv_multi.argtypes = [vp, i32, vp, i32, i32, ctypes.POINTER(_Proj), i32, vp, sz, vp]
    lib.exl3_gemv_multi.restype = ctypes.c_int
    lib.exl3_encode_slot_bytes.argtypes = [i32]
    lib.exl3_encode_slot_bytes.restype = i64
    lib.exl3_encode_tiles.argtypes = [vp, i64, i32, vp, vp, vp, sz, vp]
    lib.exl3_encode_tiles.restype = ctypes.c_int
    lib.exl3_status_string.argtypes = [ctypes.c_int]
    lib.exl3_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def bits_arg(bits: int, codebook: int = 0) -> int:
    """The C ABI's bits argument: K, with the flag of codebook 1 when asked for."""
    if codebook not in (0, 1):
        raise Exl3Error(f"codebook must be 0 or 1, got {codebook}")
    return int(bits) | (CODEBOOK_BYTE_SUM if codebook == 1 else 0)


def status_string(status: int) -> str:
    return load().exl3_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise Exl3Error(f"{what}: {status_string(status)} ({status})")


def pack_info(n_in: int, n_out: int, bits: int, max_m: int = 1) -> dict:
    info = _PackInfo()
    _check(load().exl3_pack_info(n_in, n_out, bits, max_m, ctypes.byref(info)), "exl3_pack_info")
    return {f: getattr(info, f) for f, _ in _PackInfo._fields_ if f != "reserved"}


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _need(t, name: str, dtypes, numel: int | None = None, shape=None) -> None:
    """The library reads and writes raw device memory: check what it will be
    handed (contiguous, of the element type and size the call implies; the
    device is checked by _on_gpu) and raise before anything is launched."""
    if not hasattr(t, "data_ptr") or not hasattr(t, "is_cuda"):
        raise Exl3Error(f"{name}: expected a torch tensor")
    if t.dtype not in dtypes:
        raise Exl3Error(f"{name}: dtype {t.dtype}, expected one of {tuple(str(d) for d in dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise Exl3Error(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise Exl3Error(f"{name}: {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise Exl3Error(f"{name}: must be contiguous")
    if t.numel() > 0 and t.data_ptr() % 16 != 0:
        raise Exl3Error(f"{name}: data must be 16-byte aligned (a view at an offset is not)")


def _on_gpu(**tensors) -> None:
    """The device check, after the type and size checks of every tensor."""
    for name, t in tensors.items():
        if not t.is_cuda:
            raise Exl3Error(f"{name}: must be on a GPU device")


def _word_dtypes():
    import torch
    return tuple(d for d in (torch.int16, getattr(torch, "uint16", None)) if d is not None)


def _check_linear(x, trellis, sign, out_scale, bits: int, y, n_outs=None) -> None:
    import torch
    if x.dim() != 2:
        raise Exl3Error(f"x: expected [m, n_in], got shape {tuple(x.shape)}")
    m, n_in = x.shape
    _need(x, "x", (torch.float16,))
    _need(sign, "sign", (torch.float16,), numel=n_in)
    K = int(bits)
    pairs = list(zip(trellis, out_scale, y)) if n_outs is not None else [(trellis, out_scale, y)]
    for i, (tr, sc, yy) in enumerate(pairs):
        n_out = sc.numel()
        _need(sc, f"out_scale[{i}]", (torch.float16,))
        if n_in % 128 == 0 and n_out % 16 == 0 and 1 <= K <= 8:
            _need(tr, f"trellis[{i}]", _word_dtypes(), numel=(n_out // 16) * (n_in // 16) * 16 * K)
        _need(yy, f"y[{i}]", (torch.float16,), shape=(m, n_out))
    _on_gpu(x=x, sign=sign)
    for i, (tr, sc, yy) in enumerate(pairs):
        _on_gpu(**{f"trellis[{i}]": tr, f"out_scale[{i}]": sc, f"y[{i}]": yy})


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class Workspace:
    """Device scratch sized by exl3_pack_info for (n_in, n_out, bits, max_m).

    Needs no initialisation; one workspace per stream of concurrent calls.
    """

    def __init__(self, n_in: int, n_out: int, bits: int, max_m: int, device="cuda"):
        import torch
        self.info = pack_info(n_in, n_out, bits, max_m)
        self.nbytes = int(self.info["workspace_bytes"])
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)

    def fits(self, n_in: int, n_out: int, bits: int, m: int) -> bool:
        return pack_info(n_in, n_out, bits, max(m, 1))["workspace_bytes"] <= self.nbytes


def decode_tile(words, bits: int, out=None, stream=None, codebook: int = 0):
    """Decode packed tiles [T, 16*bits] (int16) to fp16 [T, 256] in trellis order."""
    import torch
    T = words.shape[0]
    if out is None:
        out = torch.empty((T, 256), dtype=torch.float16, device=words.device)
    if 1 <= int(bits) <= 8:
        _need(words, "words", _word_dtypes(), numel=T * 16 * int(bits))
    _need(out, "out", (torch.float16,), numel=T * 256)
    _on_gpu(words=words, out=out)
    _check(load().exl3_decode_tile(_ptr(words), bits_arg(bits, codebook), T, _ptr(out), _stream(stream)),
           "exl3_decode_tile")
    return out


def _linear(fn: str, x, trellis, sign, out_scale, bits: int, workspace=None, y=None, stream=None, codebook=0):
    import torch
    m, n_in = x.shape
    n_out = out_scale.shape[0]
    if y is None:
        y = torch.empty((m, n_out), dtype=torch.float16, device=x.device)
    _check_linear(x, trellis, sign, out_scale, bits, y)
    if workspace is None and fn != "exl3_gemv":  # the GEMV needs none: it then rotates in every workgroup
        workspace = Workspace(n_in, n_out, bits, max(m, 1), device=x.device)
    ws_ptr = 0 if workspace is None else _ptr(workspace.buf)
    ws_bytes = 0 if workspace is None else workspace.nbytes
    rc = getattr(load(), fn)(_ptr(x), m, _ptr(trellis), _ptr(sign), _ptr(out_scale), n_in, n_out,
                             bits_arg(bits, codebook), _ptr(y), ws_ptr, ws_bytes, _stream(stream))
    _check(rc, fn)
    return y


def gemv(x, trellis, sign, out_scale, bits: int, workspace=None, y=None, stream=None, codebook: int = 0):
    """y = out_scale * (H128(sign * x) @ W^T) for 1 <= m <= 16 (fp16 out).

    Without a workspace nothing beyond y (when not given) is allocated."""
    return _linear("exl3_gemv", x, trellis, sign, out_scale, bits, workspace, y, stream, codebook)


def gemv_multi(x, weights, sign, bits: int, ys=None, workspace=None, stream=None, codebook: int = 0):
    """One launch for several projections of the same x (1 <= m <= 16).

    weights: sequence of (trellis, out_scale) pairs sharing n_in and bits; the
    same sign vector applies to all.  Returns the list of y, fp16 [m, n_out_i].
    """
    import torch
    m, n_in = x.shape
    n = len(weights)
    if ys is None:
        ys = [torch.empty((m, sc.shape[0]), dtype=torch.float16, device=x.device) for _, sc in weights]
    if len(ys) != n:
        raise Exl3Error(f"ys: {len(ys)} outputs for {n} projections")
    _check_linear(x, [tr for tr, _ in weights], sign, [sc for _, sc in weights], bits, ys, n_outs=True)
    arr = (_Proj * max(n, 1))()
    for i, ((tr, sc), y) in enumerate(zip(weights, ys)):
        arr[i] = _Proj(_ptr(tr), _ptr(sc), _ptr(y), int(sc.shape[0]), 0)
    ws = 0 if workspace is None else _ptr(workspace.buf)
    wsb = 0 if workspace is None else workspace.nbytes
    rc = load().exl3_gemv_multi(_ptr(x), m, _ptr(sign), n_in, bits_arg(bits, codebook), arr, n, ws, wsb,
                                _stream(stream))
    _check(rc, "exl3_gemv_multi")
    return ys


def linear(x, trellis, sign, out_scale, bits: int, workspace=None, y=None, stream=None, codebook: int = 0):
    """Any m >= 1: the GEMV or the GEMM, as the library's measured table picks."""
    return _linear("exl3_linear", x, trellis, sign, out_scale, bits, workspace, y, stream, codebook)


def linear_noalloc(x, trellis, sign, out_scale, bits: int, y, stream=None, codebook: int = 0):
    """exl3_linear_noalloc: linear() into a caller-given y, with the library's
    static per-GPU scratch instead of a workspace (nothing is allocated)."""
    m, n_in = x.shape
    n_out = out_scale.shape[0]
    _check_linear(x, trellis, sign, out_scale, bits, y)
    rc = load().exl3_linear_noalloc(_ptr(x), m, _ptr(trellis), _ptr(sign), _ptr(out_scale), n_in, n_out,
                                    bits_arg(bits, codebook), _ptr(y), _stream(stream))
    _check(rc, "exl3_linear_noalloc")
    return y


def encode_slot_bytes(bits: int, codebook: int = 0) -> int:
    """Workspace bytes of exl3_encode_tiles per tile in flight."""
    n = int(load().exl3_encode_slot_bytes(bits_arg(bits, codebook)))
    if n < 0:
        _check(n, "exl3_encode_slot_bytes")
    return n


def encode_tiles(w, bits: int, codebook: int = 0, workspace=None, words=None, costs=None, slots: int = 256,
                 stream=None):
    """Quantise fp32 tiles [T, 256] to trellis streams: returns (words [T, 16K] int16, costs [T] fp32).

    workspace: a uint8 device tensor; by default `slots` tiles in flight.
    """
    import torch
    T = w.shape[0]
    if words is None:
        words = torch.empty((T, 16 * bits), dtype=torch.int16, device=w.device)
    if costs is None:
        costs = torch.empty((T,), dtype=torch.float32, device=w.device)
    if workspace is None:
        workspace = torch.empty(encode_slot_bytes(bits, codebook) * max(1, min(slots, T)), dtype=torch.uint8,
                                device=w.device)
    _need(w, "w", (torch.float32,), numel=T * 256)
    if 1 <= int(bits) <= 8:
        _need(words, "words", _word_dtypes(), numel=T * 16 * int(bits))
    _need(costs, "costs", (torch.float32,), numel=T)
    _need(workspace, "workspace", (torch.uint8,))
    _on_gpu(w=w, words=words, costs=costs, workspace=workspace)
    rc = load().exl3_encode_tiles(_ptr(w), T, bits_arg(bits, codebook), _ptr(words), _ptr(costs), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    _check(rc, "exl3_encode_tiles")
    return words, costs


def gemm(x, trellis, sign, out_scale, bits: int, workspace=None, y=None, stream=None, codebook: int = 0):
    """The same result for any m >= 1 through the matrix-core GEMM path."""
    return _linear("exl3_gemm", x, trellis, sign, out_scale, bits, workspace, y, stream, codebook)
