"""CPU oracle for the EXL3 trellis decode-matmul.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  The product path (the HIP library and its Python
binding) never calls it, and it shares no code, constant table or helper with
that path: every constant below is restated from the format definition.

What is computed (all sources are the pages of the ExLlamaV3 / EXL3 articles):

* "ExLlamaV3 inference speed: EXL3 GEMM kernel and fused Viterbi encoding"
  (czykbl.com), section "Viterbi encoding kernel": weights are quantised in
  16x16 blocks of 256 elements, each block is one tail-biting trellis codeword,
  and the code is packed as a sequence of 16-bit words.
* Same page, section "GEMM kernel": the input A is rotated by a 128-point
  Hadamard transform at kernel start; an index turns into a half value through
  one integer multiply and one three-input bit operation, with no table.
* Same page, section "conclusion first": three GPU instructions per codebook
  value; the decode side is table-free.
* "ExLlamaV3 overview" (discosf.com), section "EXL3 format": a streamlined
  variant of QTIP with a procedural codebook and a tail-biting trellis,
  bit widths K = 1..8.

The pages fix none of the constants, bit orders or scalings.  The readings used
here (one per FMT item) are:

FMT-1  y[r][o] = out_scale[o] * sum_k x'[r][k] * W[o][k],  x' = H_blk(sign * x[r])
FMT-2  W is [n_out][n_in]; tile (tr, tc) covers rows 16tr.., cols 16tc..; storage
       trellis[tr][tc][w], w < 16K; tile element i -> (row i>>4, col i&15).
FMT-3  stream bit j of a tile = bit (j & 15) of word j >> 4 (LSB first).
FMT-4  state s_i = sum_{b<16} bit((iK + b) mod 256K) << b, i = 0..255 (the
       window wraps at the tile end: tail-biting).
FMT-5  p = (s*A + B) mod 2^32; q = (p & M) | X; lo, hi = fp16 halves of q;
       c(s) = RNE16(lo + hi).  A = 0xBFD3, B = 0x201784FF, M = 0x8D7F8DFF,
       X = 0x30003000 (X & M = 0).  No post-scale (g = 1).
FMT-6  H = 128x128 Sylvester matrix, H[i][j] = (-1)^popcount(i & j), unnormalised;
       applied to each 128-wide block of the input features.
FMT-7  sign is +-1 per input feature, out_scale one fp16 per output feature.
FMT-8  gemv: 1 <= m <= 8; gemm: any m >= 1.  Same result definition.
FMT-9  K in 1..8.
FMT-10 (the "dp4a" codebook the "GEMM kernel" section names as the alternative
       to the multiply-and-lop3 one): p = (s*A' + B') mod 2^32; t = the sum of
       p's four bytes (0..1020); c'(s) = RNE16((1024 + t) * G + C), one rounding,
       with fp16 constants G = 1773/262144 (bits 0x1EED) and C = -10.375 (0xC930).
       A' = 0xFEC5, B' = 0x77C40AA0.  Selected per call as codebook 1.

The matrix product itself (FMT-1) has a plain definition, so the oracle is that
definition evaluated in float64 after an exact decode.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# FMT-5 constants (the procedural codebook).  Chosen by enumerating all 65536
# states: A odd and below 2^16, X disjoint from M, both fp16 halves planted with
# exponent field 0b011xx (magnitude in [1/8, 2)), mean ~ 0 and variance ~ 1.
# ---------------------------------------------------------------------------
CB_A = 0xBFD3
CB_B = 0x201784FF
CB_M = 0x8D7F8DFF
CB_X = 0x30003000

# FMT-10 constants (the byte-sum codebook).  Chosen by enumerating all 65536
# states: A' odd and below 2^16; the byte sum of p has mean 510.009 and variance
# 21835 (four independent uniform bytes: 510 and 21845); G and C are the fp16
# pair that then gives mean 2e-4 and variance 0.9988; no result is subnormal.
CB1_A = 0xFEC5
CB1_B = 0x77C40AA0
CB1_G = 0x1EED
CB1_C = 0xC930

CODEBOOKS = (0, 1)  # 0: multiply + mask-and-plant + half sum (FMT-5); 1: byte sum (FMT-10)

TILE = 16
TILE_ELEMS = 256
HAD = 128


def words_per_tile(K: int) -> int:
    """Number of uint16 words in one packed 16x16 tile at K bits/weight (FMT-2/3)."""
    _check_k(K)
    return 16 * K


def _check_k(K: int) -> None:
    if not (1 <= int(K) <= 8):
        raise ValueError(f"K must be in 1..8, got {K}")


# ---------------------------------------------------------------------------
# FMT-3 / FMT-4: trellis states of a tile stream
# ---------------------------------------------------------------------------
def tile_states(words: np.ndarray, K: int) -> np.ndarray:
    """Trellis states of packed tiles.

    words: uint16 array [..., 16K] (one tile per last-axis row).
    returns uint16 array [..., 256]: s_i = bits [iK, iK+16) of the cyclic,
    LSB-first stream of the tile (FMT-3, FMT-4).
    """
    _check_k(K)
    words = np.ascontiguousarray(words, dtype=np.uint16)
    if words.shape[-1] != 16 * K:
        raise ValueError("last axis must hold 16*K words")
    lead = words.shape[:-1]
    flat = words.reshape(-1, 16 * K)
    # bit j of the stream = bit (j & 15) of word (j >> 4): unpack each word LSB first
    bits = ((flat[:, :, None] >> np.arange(16, dtype=np.uint16)) & 1).astype(np.uint8)
    bits = bits.reshape(flat.shape[0], 256 * K)
    nbits = 256 * K
    idx = (np.arange(256)[:, None] * K + np.arange(16)[None, :]) % nbits  # [256, 16]
    window = bits[:, idx]  # [T, 256, 16]
    weights = (1 << np.arange(16, dtype=np.uint32)).astype(np.uint32)
    states = (window.astype(np.uint32) * weights).sum(axis=-1).astype(np.uint16)
    return states.reshape(lead + (256,))


def tile_row_states(words: np.ndarray, K: int, r) -> np.ndarray:
    """States 16r .. 16r+15 of packed tiles: one 16-element row of each tile.

    words: uint16 [..., 16K]; r: row index (0..15), broadcastable to
    words.shape[:-1].  Returns uint16 [..., 16], element c = s_{16r+c}.
    By FMT-3/4, s_{16r+c} is the 16-bit window at stream bit (16r + c)K; the 16
    windows of a row lie in the K + 1 words that start at word rK, taken
    cyclically (row 15 wraps into word 0), so the row is read from that
    sub-stream: its bit q is stream bit 16rK + q, i.e. bit q % 16 of its word
    q // 16.  Equal to tile_states(words, K)[..., 16r:16r+16] (pinned in the
    tests).
    """
    _check_k(K)
    words = np.ascontiguousarray(words, dtype=np.uint16)
    if words.shape[-1] != 16 * K:
        raise ValueError("last axis must hold 16*K words")
    r = np.asarray(r, dtype=np.int64)
    widx = (r[..., None] * K + np.arange(K + 1)) % (16 * K)        # words of the sub-stream
    widx = np.broadcast_to(widx, words.shape[:-1] + (K + 1,))
    sub = np.take_along_axis(words, widx, axis=-1).astype(np.uint32)  # [..., K+1]
    states = np.empty(sub.shape[:-1] + (16,), dtype=np.uint16)
    for c in range(16):
        # sub-stream bits [cK, cK + 16) lie in words w0, w0 + 1 (LSB first),
        # i.e. bits sh .. sh + 15 of the little-endian pair
        w0, sh = divmod(c * K, 16)
        pair = sub[..., w0] | (sub[..., w0 + 1] << np.uint32(16))
        states[..., c] = (pair >> np.uint32(sh)) & np.uint32(0xFFFF)
    return states


# ---------------------------------------------------------------------------
# FMT-5: procedural codebook
# ---------------------------------------------------------------------------
def codebook_halves(states: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The two planted fp16 halves (lo, hi) of the codebook word for each state."""
    s = np.asarray(states, dtype=np.uint64)
    p = (s * np.uint64(CB_A) + np.uint64(CB_B)) & np.uint64(0xFFFFFFFF)
    q = (p & np.uint64(CB_M)) | np.uint64(CB_X)
    lo = (q & np.uint64(0xFFFF)).astype(np.uint16).view(np.float16)
    hi = (q >> np.uint64(16)).astype(np.uint16).view(np.float16)
    return lo, hi


def byte_sums(states: np.ndarray) -> np.ndarray:
    """t(s) = sum of the four bytes of p = (s*A' + B') mod 2^32 (FMT-10), int64."""
    s = np.asarray(states, dtype=np.uint64)
    p = (s * np.uint64(CB1_A) + np.uint64(CB1_B)) & np.uint64(0xFFFFFFFF)
    t = np.zeros(p.shape, dtype=np.uint64)
    for k in range(4):
        t += (p >> np.uint64(8 * k)) & np.uint64(0xFF)
    return t.astype(np.int64)


def codebook(states: np.ndarray, cb: int = 0) -> np.ndarray:
    """The codebook value of each state as float16.

    cb = 0 (FMT-5): c(s) = RNE16(lo + hi).  The float32 sum of two fp16 values
    whose exponents differ by at most 3 is exact, so casting it to float16
    (NumPy rounds to nearest even) is one correctly rounded fp16 addition.
    cb = 1 (FMT-10): c'(s) = RNE16((1024 + t) * G + C).  With t < 2^10 and G, C
    fp16, the float64 value is exact, so one cast is the single rounding.
    """
    if cb == 0:
        lo, hi = codebook_halves(states)
        return (lo.astype(np.float32) + hi.astype(np.float32)).astype(np.float16)
    if cb == 1:
        G = float(np.array([CB1_G], np.uint16).view(np.float16)[0])
        C = float(np.array([CB1_C], np.uint16).view(np.float16)[0])
        v = (1024.0 + byte_sums(states).astype(np.float64)) * G + C
        return v.astype(np.float16)
    raise ValueError(f"codebook must be one of {CODEBOOKS}, got {cb}")


def decode_tiles(words: np.ndarray, K: int, cb: int = 0) -> np.ndarray:
    """Decode packed tiles to fp16 values in trellis order: [..., 16K] -> [..., 256]."""
    return codebook(tile_states(words, K), cb)


# ---------------------------------------------------------------------------
# FMT-2: tile grid
# ---------------------------------------------------------------------------
def tiles_to_matrix(tiles: np.ndarray) -> np.ndarray:
    """[n_out/16, n_in/16, 256] tile values -> W [n_out, n_in] (row-major tiles)."""
    to, ti, e = tiles.shape
    assert e == 256
    return tiles.reshape(to, ti, 16, 16).transpose(0, 2, 1, 3).reshape(to * 16, ti * 16)


def dequant(trellis: np.ndarray, K: int, cb: int = 0) -> np.ndarray:
    """Full fp16 weight matrix W [n_out, n_in] from trellis [n_out/16, n_in/16, 16K]."""
    return tiles_to_matrix(decode_tiles(trellis, K, cb))


# ---------------------------------------------------------------------------
# FMT-6: Hadamard rotation
# ---------------------------------------------------------------------------
def hadamard(n: int = HAD) -> np.ndarray:
    """Sylvester Hadamard matrix by definition: H[i][j] = (-1)^popcount(i & j)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    a = i & j
    pc = np.zeros_like(a)
    while np.any(a):
        pc += a & 1
        a = a >> 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def rotate(x: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """x' = blockdiag(H128) (sign * x) along the last axis, in float64 (FMT-6, FMT-7)."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.asarray(sign, dtype=np.float64)
    n_in = x.shape[-1]
    if n_in % HAD:
        raise ValueError("n_in must be a multiple of 128")
    H = hadamard().astype(np.float64)
    xs = (x * sign).reshape(x.shape[:-1] + (n_in // HAD, HAD))
    return (xs @ H.T).reshape(x.shape)


# ---------------------------------------------------------------------------
# FMT-1: the decode-matmul
# ---------------------------------------------------------------------------
def _check_shapes(x, trellis, sign, out_scale, K):
    _check_k(K)
    m, n_in = x.shape
    to, ti, w = trellis.shape
    if w != 16 * K or ti * 16 != n_in or sign.shape != (n_in,) or out_scale.shape != (to * 16,):
        raise ValueError("inconsistent shapes")
    if n_in % HAD:
        raise ValueError("n_in must be a multiple of 128")
    return m, n_in, to * 16


def linear(x, trellis, sign, out_scale, K, strip_block: int = 64, cb: int = 0) -> np.ndarray:
    """y = out_scale * (x' @ W^T) in float64 (FMT-1).

    x: fp16 [m, n_in]; trellis: uint16 [n_out/16, n_in/16, 16K];
    sign: fp16 [n_in]; out_scale: fp16 [n_out].  Returns float64 [m, n_out].
    The weight matrix is decoded strip block by strip block to bound memory.
    """
    m, n_in, n_out = _check_shapes(x, trellis, sign, out_scale, K)
    xr = rotate(np.asarray(x, np.float64), np.asarray(sign, np.float64))
    y = np.empty((m, n_out), dtype=np.float64)
    for t0 in range(0, n_out // 16, strip_block):
        t1 = min(n_out // 16, t0 + strip_block)
        W = dequant(trellis[t0:t1], K, cb).astype(np.float64)
        y[:, 16 * t0:16 * t1] = xr @ W.T
    return y * np.asarray(out_scale, np.float64)[None, :]


def weight_rows(trellis, K, rows, cb: int = 0) -> np.ndarray:
    """Rows W[rows] of the decoded weight matrix as float16 [len(rows), n_in]:
    row o is row o % 16 of every tile of strip o // 16 (FMT-2), element c of
    tile column tc at column 16 tc + c."""
    rows = np.asarray(rows, dtype=np.int64)
    words = np.asarray(trellis)[rows // 16]                       # [R, tiles_in, 16K]
    st = tile_row_states(words, K, (rows % 16)[:, None])          # [R, tiles_in, 16]
    return codebook(st, cb).reshape(rows.size, -1)


def linear_rows(x, trellis, sign, out_scale, K, rows: np.ndarray, cb: int = 0,
                chunk: int = 256) -> np.ndarray:
    """Selected output features only: y[:, rows] in float64 (decodes only those
    rows of W, `chunk` rows at a time)."""
    m, n_in, n_out = _check_shapes(x, trellis, sign, out_scale, K)
    rows = np.asarray(rows, dtype=np.int64)
    xr = rotate(np.asarray(x, np.float64), np.asarray(sign, np.float64))
    out = np.empty((m, rows.size), dtype=np.float64)
    for a in range(0, rows.size, chunk):
        W = weight_rows(trellis, K, rows[a:a + chunk], cb).astype(np.float64)
        out[:, a:a + chunk] = xr @ W.T
    return out * np.asarray(out_scale, np.float64)[rows][None, :]


# ---------------------------------------------------------------------------
# Scalar forms, written independently of the vectorised ones above, for
# brute-force pins on tiny inputs.  Plain Python integers and floats.
# ---------------------------------------------------------------------------
def state_scalar(words, K: int, i: int) -> int:
    """s_i by walking the 16 bits of the window one at a time (FMT-3, FMT-4)."""
    nbits = 256 * K
    s = 0
    for b in range(16):
        j = (i * K + b) % nbits
        bit = (int(words[j // 16]) >> (j % 16)) & 1
        s |= bit << b
    return s


def _fp16_bits_to_float(h: int) -> float:
    """IEEE binary16 bit pattern -> Python float, from the format's definition."""
    sgn = -1.0 if (h >> 15) & 1 else 1.0
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    if e == 0:
        return sgn * f * 2.0 ** -24
    if e == 31:
        return sgn * (float("inf") if f == 0 else float("nan"))
    return sgn * (1.0 + f / 1024.0) * 2.0 ** (e - 15)


def round_to_fp16(v: float) -> float:
    """Round a finite Python float to the nearest binary16 value, ties to even.

    Normal range only (the codebook sums never leave it); written from the
    format's definition: 11 significant bits.
    """
    if v == 0.0:
        return 0.0
    import math
    mant, ex = math.frexp(abs(v))  # abs(v) = mant * 2^ex, mant in [0.5, 1)
    scaled = mant * 2048.0          # 11 significant bits
    r = math.floor(scaled)
    rem = scaled - r
    if rem > 0.5 or (rem == 0.5 and r % 2 == 1):
        r += 1
    out = r / 2048.0 * 2.0 ** ex
    if not (2.0 ** -14 <= out < 65520.0):
        raise ValueError("value outside the fp16 normal range")
    return math.copysign(out, v)


def codebook_scalar(s: int, cb: int = 0) -> float:
    """c(s) via Python integers: FMT-5 (cb = 0) or FMT-10 (cb = 1)."""
    if cb == 1:
        from fractions import Fraction
        p = (s * CB1_A + CB1_B) % (1 << 32)
        t = sum((p >> (8 * k)) & 0xFF for k in range(4))
        G = Fraction(_fp16_bits_to_float(CB1_G))
        C = Fraction(_fp16_bits_to_float(CB1_C))
        return round_to_fp16(float((1024 + t) * G + C))  # the rational is exact in a double
    p = (s * CB_A + CB_B) % (1 << 32)
    q = (p & CB_M) | CB_X
    lo = _fp16_bits_to_float(q & 0xFFFF)
    hi = _fp16_bits_to_float(q >> 16)
    return round_to_fp16(lo + hi)


def hadamard_entry(i: int, j: int) -> int:
    return -1 if bin(i & j).count("1") % 2 else 1


def y_scalar(x, trellis, sign, out_scale, K: int, r: int, o: int, cb: int = 0) -> float:
    """One output element straight from the definitions (FMT-1..7), pure Python.

    Quadratic in n_in: for tiny shapes only.
    """
    n_in = len(sign)
    tr, rr = divmod(o, 16)
    acc = 0.0
    for k in range(n_in):
        b, i = divmod(k, HAD)
        xr = 0.0
        for jj in range(HAD):
            col = b * HAD + jj
            xr += hadamard_entry(i, jj) * float(sign[col]) * float(x[r][col])
        tc, cc = divmod(k, 16)
        elem = rr * 16 + cc
        w = codebook_scalar(state_scalar(trellis[tr][tc], K, elem), cb)
        acc += xr * w
    return float(out_scale[o]) * acc


def fp16_bits(a: np.ndarray) -> np.ndarray:
    """View fp16 values as their uint16 bit patterns (for bit-exact comparison)."""
    return np.asarray(a, dtype=np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# Encoding: the tail-biting Viterbi search ("ExLlamaV3 inference speed", section
# "Viterbi encoding kernel": each 16x16 block is one codeword found by a forward
# Viterbi pass over the trellis, keeping the accumulated cost of every edge and
# the minimum-cost path; the tail-biting boundary is closed by enumerating start
# states so that the codeword's head and tail agree).
#
# Trellis: an L-bit state; state i+1 = (state i >> K) | (b << (L - K)) for the K
# new bits b.  So the predecessors of s are the 2^K states (u << K) | j with
# u = s & (2^(L-K) - 1), and one step is
#     M[u]     = min_j cost[(u << K) | j]     (the first j on ties)
#     cost'[s] = M[s & (2^(L-K) - 1)] + (w_i - value[s])^2.
# Decisions are taken in float32 with the subtraction, the square and the sum
# each rounded (no fused multiply-add), so a GPU encoder can match them bit
# for bit.  A stream is tail-biting when state T-1's top L-K bits equal state
# 0's low L-K bits (the window wraps at the end of the stream).
# ---------------------------------------------------------------------------
def trellis_viterbi(w, values, L: int, K: int, v=None):
    """Minimum-cost state path for targets w [T] over codebook values [2^L].

    v None: free start and end.  v given: start states with low L-K bits == v
    and end states with high L-K bits == v (a tail-biting path).
    Returns (path int64 [T], cost float32).
    """
    w = np.asarray(w, dtype=np.float32)
    values = np.asarray(values, dtype=np.float32)
    T, S = w.shape[0], 1 << L
    low = (1 << (L - K)) - 1
    s = np.arange(S, dtype=np.int64)

    def err(i):
        d = np.float32(w[i]) - values          # float32 subtract
        return d * d                            # float32 square

    cost = err(0)
    if v is not None:
        cost = np.where((s & low) == v, cost, np.float32(np.inf)).astype(np.float32)
    back = np.empty((T, low + 1), dtype=np.int64)
    for i in range(1, T):
        blocks = cost.reshape(low + 1, 1 << K)
        j = np.argmin(blocks, axis=1)            # first minimum on ties
        M = blocks[np.arange(low + 1), j]
        back[i] = j
        cost = (M[s & low] + err(i)).astype(np.float32)
    if v is None:
        end = int(np.argmin(cost))
    else:
        cand = (v << K) + np.arange(1 << K)
        end = int(cand[np.argmin(cost[cand])])
    path = np.empty(T, dtype=np.int64)
    path[T - 1] = end
    for i in range(T - 1, 0, -1):
        u = path[i] & low
        path[i - 1] = (u << K) | back[i][u]
    return path, np.float32(cost[end])


def tail_biting_exact(w, values, L: int, K: int):
    """Optimal tail-biting path: the best of the constrained searches over every
    value of the L-K overlap bits (the full enumeration of start states)."""
    best = None
    for v in range(1 << (L - K)):
        path, c = trellis_viterbi(w, values, L, K, v)
        if best is None or c < best[1]:
            best = (path, c)
    return best


def tail_biting_two_pass(w, values, L: int, K: int):
    """The encoder's search: a free pass over the targets rotated by T/2 picks
    the overlap bits (the low L-K bits of its state at the original position
    0), then one constrained pass returns a tail-biting path with them."""
    w = np.asarray(w, dtype=np.float32)
    T = w.shape[0]
    h = T // 2
    path_r, _ = trellis_viterbi(np.roll(w, -h), values, L, K)
    v = int(path_r[T - h] & ((1 << (L - K)) - 1))
    return trellis_viterbi(w, values, L, K, v)


def path_cost(w, values, path) -> np.float32:
    """Cost of a path with the search's float32 rounding and summation order."""
    w = np.asarray(w, dtype=np.float32)
    values = np.asarray(values, dtype=np.float32)
    c = np.float32(0)
    for i, s in enumerate(path):
        d = np.float32(w[i]) - values[s]
        c = np.float32(c + np.float32(d * d)) if i else np.float32(d * d)
    return c


def pack_path(path, K: int) -> np.ndarray:
    """Tile stream of a tail-biting path of 256 states: stream bits [iK, iK+K)
    are the low K bits of state i (FMT-3, FMT-4), as 16K uint16 words."""
    path = np.asarray(path, dtype=np.int64)
    assert path.shape == (256,)
    bits = ((path[:, None] >> np.arange(K)[None, :]) & 1).reshape(-1)  # stream bit iK + b
    return np.packbits(bits.astype(np.uint8), bitorder="little").view("<u2").astype(np.uint16)


def encode_tile(w, K: int, cb: int = 0):
    """Encode one tile (256 targets in trellis order, float32) at K bits per
    weight: the two-pass tail-biting search over the 16-bit trellis with the
    codebook's values.  Returns (words uint16 [16K], cost float32)."""
    _check_k(K)
    values = codebook(np.arange(65536), cb).astype(np.float32)
    path, cost = tail_biting_two_pass(np.asarray(w, np.float32).reshape(256), values, 16, K)
    return pack_path(path, K), cost


def encode_tiles(W, K: int, cb: int = 0):
    """encode_tile over [n, 256] targets: (words [n, 16K], costs [n])."""
    W = np.asarray(W, dtype=np.float32).reshape(-1, 256)
    out = np.empty((W.shape[0], 16 * K), dtype=np.uint16)
    costs = np.empty(W.shape[0], dtype=np.float32)
    for t in range(W.shape[0]):
        out[t], costs[t] = encode_tile(W[t], K, cb)
    return out, costs


def brute_force_tail_biting(w, values, L: int, K: int):
    """Minimum cost over every cyclic stream of T*K bits (tiny T*K only): state
    i is the L-bit window at bit iK, wrapping at the end (pure Python)."""
    w = [float(np.float32(x)) for x in w]
    T = len(w)
    n = T * K
    best = None
    for stream in range(1 << n):
        path = []
        for i in range(T):
            st = 0
            for b in range(L):
                st |= ((stream >> ((i * K + b) % n)) & 1) << b
            path.append(st)
        c = path_cost(w, values, path)
        if best is None or c < best[1]:
            best = (path, c)
    return best
