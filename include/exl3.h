/*
 * exl3.h - C ABI of the EXL3 trellis decode-matmul library for MI355X (gfx950).
 *
 * The operation (pages: "ExLlamaV3 inference speed: EXL3 GEMM kernel and fused
 * Viterbi encoding", sections "GEMM kernel", "small-batch GEMV" and "Viterbi
 * encoding kernel"; "ExLlamaV3 overview", section "EXL3 format"):
 *
 *     y[r][o] = out_scale[o] * sum_k x'[r][k] * W[o][k],
 *     x'[r]   = blockdiag(H128) (sign * x[r])       (Hadamard rotation of the input)
 *
 * W is never stored: each 16x16 tile of W is a tail-biting bitshift trellis
 * stream of 256*K bits (K bits per weight), packed into 16*K little-endian
 * uint16 words and decoded on the fly by a table-free codebook.
 *
 * Format (the pages leave these open; this library fixes them):
 *   - W is [n_out][n_in] (y = x' W^T).  Tile (tr, tc) covers rows 16tr..16tr+15
 *     and columns 16tc..16tc+15.  trellis[tr][tc][w], w < 16K, so one 16-row
 *     strip (fixed tr) is contiguous.  Tile element i is W[16tr + i/16][16tc + i%16].
 *   - Stream bit j of a tile is bit (j % 16) of word j / 16.  State
 *     s_i = bits [iK, iK+16) of the stream, taken cyclically (i = 0..255).
 *   - Codebook 0 (the multiply and three-input bit operation of "GEMM kernel"):
 *     p = s*0xBFD3 + 0x201784FF (mod 2^32); q = (p & 0x8D7F8DFF) | 0x30003000;
 *     the value is the fp16 sum, rounded to nearest even, of q's two fp16 halves.
 *   - Codebook 1 (the dp4a alternative the same section names): p = s*0xFEC5 +
 *     0x77C40AA0 (mod 2^32); t = the sum of p's four bytes; the value is
 *     (1024 + t) * G + C rounded once to fp16 (nearest even), G = fp16 0x1EED
 *     (1773/262144), C = fp16 0xC930 (-10.375).
 *     A call selects it with EXL3_CODEBOOK_BYTE_SUM in its `bits` argument.
 *   - H128 is the unnormalised 128x128 Sylvester matrix, H[i][j] = (-1)^popcount(i&j),
 *     applied to each block of 128 consecutive input features.
 *   - fp16 values travel as uint16_t bit patterns.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers owned by the caller; the library allocates
 *     nothing and keeps no per-call state.  Tensors (and workspaces) are
 *     contiguous, row-major, and at least 16-byte aligned: a call given a
 *     misaligned pointer returns EXL3_EINVAL.  x and y must not alias.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous: argument errors are returned synchronously, before any
 *     launch; launch failures are reported as EXL3_EHIP from hipGetLastError
 *     right after the launch; device faults surface at the caller's next
 *     synchronisation.
 *   - No C++ exception crosses this interface.  Calls on different streams
 *     may run concurrently if each has its own workspace.
 */
#ifndef EXL3_H
#define EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The `bits` argument of every call: K (1..8) in the low byte, optionally OR-ed
 * with EXL3_CODEBOOK_BYTE_SUM to select codebook 1.  Any other bit is EXL3_EINVAL.
 * Sizes (trellis, workspace) depend on K only. */
#define EXL3_CODEBOOK_BYTE_SUM 0x100

enum exl3_status {
    EXL3_OK = 0,
    EXL3_EINVAL = -1,       /* null pointer, bad shape, bad bit width, bad m        */
    EXL3_EUNSUPPORTED = -2, /* valid request that this build cannot serve           */
    EXL3_EWORKSPACE = -3,   /* workspace missing or smaller than exl3_pack_info says */
    EXL3_EHIP = -4          /* a HIP runtime call or a kernel launch failed          */
};

typedef struct exl3_pack_info_t {
    int32_t n_in, n_out, bits, max_m; /* echo of the arguments (bits with its flag)    */
    int32_t tiles_in, tiles_out;      /* n_in / 16, n_out / 16                         */
    int32_t words_per_tile;           /* 16 * K                                        */
    int32_t reserved;
    int64_t trellis_words;            /* tiles_in * tiles_out * words_per_tile         */
    int64_t trellis_bytes;            /* n_in * n_out * K / 8                          */
    int64_t workspace_bytes;          /* enough for exl3_gemv and exl3_gemm, any m <= max_m */
} exl3_pack_info_t;

/*
 * exl3_pack_info: sizes of the packed weight and of the workspace (pages:
 * "Viterbi encoding kernel" - the weight is quantised in 16x16 blocks, each
 * block's code packed as a sequence of 16-bit indices; here 16*K words per
 * block, K bits per weight).
 *   n_in % 128 == 0, n_out % 16 == 0, 1 <= K <= 8, max_m >= 1.
 *   out : filled on success; max_m is echoed, reserved is set to 0.
 * Host-only; never touches the GPU.  Returns EXL3_EINVAL on bad arguments
 * (out untouched).
 */
int exl3_pack_info(int32_t n_in, int32_t n_out, int32_t bits, int32_t max_m,
                   exl3_pack_info_t* out);

/*
 * exl3_decode_tile: decode n_tiles packed tiles (pages: "Viterbi encoding
 * kernel" packs each 16x16 block as a 16-bit index sequence; "GEMM kernel"
 * turns an index into a half with a multiply and a bit operation).
 *   words : uint16 [n_tiles][16*K], device.
 *   out   : fp16 bits [n_tiles][256], device; element i of tile t at out[256t + i]
 *           (trellis order = row-major over the 16x16 tile).  Bit-exact.
 * n_tiles == 0 is a no-op.  EXL3_EINVAL for null pointers, n_tiles < 0 or a bad
 * bits argument.
 */
int exl3_decode_tile(const uint16_t* words, int32_t bits, int64_t n_tiles,
                     uint16_t* out, void* stream);

/* Largest m the GEMV calls take (the rows of one matrix-core tile). */
#define EXL3_GEMV_MAX_M 16

/*
 * exl3_gemv: the decode-matmul for 1 <= m <= EXL3_GEMV_MAX_M (pages: "small-batch
 * GEMV", where small m makes the weight stream the bottleneck).
 *   x         : fp16 [m][n_in]
 *   trellis   : uint16 [n_out/16][n_in/16][16*K]
 *   sign      : fp16 [n_in], entries +-1
 *   out_scale : fp16 [n_out]
 *   y         : fp16 [m][n_out] (overwritten; fp32 accumulation, round to nearest even)
 *   workspace : optional device scratch (NULL and 0 are accepted).  With at
 *               least m*n_in*2 bytes (rounded up to 256; the size
 *               exl3_pack_info gives for max_m >= m always suffices) an input
 *               of m >= 2 rows with m >= 14, or with n_in >= 8192 and
 *               m * n_in >= 28672, is rotated once by a pre-pass into it;
 *               otherwise every workgroup rotates the input itself.
 *               Both give the same y bit for bit.  Its contents need no
 *               initialisation and are meaningless after the call; it must not
 *               overlap x, y or the weights.  Calls that may run at the same
 *               time (different streams) need separate workspaces.
 * m == 0 is a no-op.  m > EXL3_GEMV_MAX_M or m < 0 gives EXL3_EINVAL (use exl3_gemm).
 */
int exl3_gemv(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
              const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits,
              uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* Most projections one exl3_gemv_multi call serves. */
#define EXL3_GEMV_MAX_PROJ 4

/* One projection of an exl3_gemv_multi call (host memory; read during the call only). */
typedef struct exl3_proj_t {
    const uint16_t* trellis;   /* uint16 [n_out/16][n_in/16][16*K], device      */
    const uint16_t* out_scale; /* fp16 [n_out], device                          */
    uint16_t* y;               /* fp16 [m][n_out], device, overwritten          */
    int32_t n_out;             /* n_out % 16 == 0                               */
    int32_t reserved;          /* set to 0                                      */
} exl3_proj_t;

/*
 * exl3_gemv_multi: exl3_gemv for up to EXL3_GEMV_MAX_PROJ projections of the
 * same input in one launch, e.g. q/k/v or gate/up of a decoder layer (pages:
 * "small-batch GEMV" for the path, and the summary's point that the kernels
 * fuse work so that intermediate tensors and passes over memory disappear).
 *   x, m, sign, n_in, bits : shared by every projection, as in exl3_gemv; the
 *                            projections must have been quantised with the
 *                            same input sign vector (one rotated input).
 *   proj[0..n_proj-1]      : per projection trellis, out_scale, y and n_out.
 *                            The y buffers must not overlap each other or x.
 *   workspace              : as exl3_gemv (optional; used for the rotation pre-pass).
 * Each proj[i].y equals what exl3_gemv gives for that projection, up to fp32
 * summation order.  m == 0 is a no-op.  EXL3_EINVAL for m outside 0..EXL3_GEMV_MAX_M, n_proj
 * outside 1..EXL3_GEMV_MAX_PROJ, a null pointer, a bad shape or two identical y.
 */
int exl3_gemv_multi(const uint16_t* x, int32_t m, const uint16_t* sign, int32_t n_in, int32_t bits,
                    const exl3_proj_t* proj, int32_t n_proj, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * exl3_gemm: the same result for any m >= 1, built for larger m (pages: "GEMM
 * kernel", where the Hadamard rotation of the input and the decode are fused
 * with a tiled matrix product).  Arguments and workspace rules as exl3_gemv;
 * the workspace holds the rotated input and, when the input dimension is split
 * across workgroups (few output blocks), fp32 partial sums: a workspace of the
 * size exl3_pack_info gives always suffices, a smaller one (at least
 * rows*n_in*2 bytes rounded up to 256, with rows = m for m <= 128 and m rounded
 * up to a multiple of 256 beyond) splits less.  EXL3_EUNSUPPORTED, before any
 * launch, when the rotated input (rows*n_in*2 bytes) reaches 2^31 - 2^20 bytes
 * (it is read through 32-bit offsets; e.g. n_in = 8192 at m > 130816) or
 * m > 65535*64: split such a call into row blocks.
 */
int exl3_gemm(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
              const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits,
              uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * exl3_linear: the same result for any m >= 1, through exl3_gemv or exl3_gemm as
 * a measured table picks (pages: "GEMM kernel" - the kernel map chooses tile
 * sizes and concurrency by architecture and shape; "small-batch GEMV" - small m
 * goes to the GEMV).  The GEMV serves m <= 12 while m * n_in <= 2^17 and
 * m <= 14 while m * n_in <= 2^16, the GEMM
 * (64-, 128- or 256-row blocks by m, its input dimension split across
 * workgroups when the output blocks alone leave compute units idle) the rest.  Arguments and workspace as
 * exl3_gemm.
 */
int exl3_linear(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
                const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits,
                uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static scratch exl3_linear_noalloc uses on each GPU. */
#define EXL3_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * exl3_linear_noalloc: exl3_linear with no workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It allocates nothing and calls no
 * allocating routine: its scratch (the GEMM's rotated input and split partial
 * sums, the GEMV's rotation pre-pass) is a static device array of
 * EXL3_NOALLOC_SCRATCH_BYTES in the library, one per GPU, which that GPU holds
 * from the first call until the process ends.  The array's address on a device
 * is looked up on the first call on it (with it current).
 *   Arguments and result as exl3_linear; the caller still owns x, the weights,
 *   sign, out_scale and y.
 *   EXL3_EUNSUPPORTED, before any launch, when a GEMM call's rotated input
 *   (rows * n_in * 2 bytes, rows = m for m <= 128, else m rounded up to a
 *   multiple of 256) exceeds EXL3_NOALLOC_SCRATCH_BYTES; split partial sums
 *   that do not fit beside it make the input dimension split less.
 *   EXL3_EHIP if the scratch's address cannot be looked up.
 * Given the same split, y equals exl3_linear's bit for bit.  Nothing in the
 * scratch needs to start at zero, and it keeps the last call's contents.  Calls
 * on one GPU share its array: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 */
int exl3_linear_noalloc(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
                        const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits, uint16_t* y,
                        void* stream);

/*
 * exl3_encode_slot_bytes: workspace bytes exl3_encode_tiles needs per tile in
 * flight (256 * 2^(16-K): the choice of every trellis step), or EXL3_EINVAL for
 * a bad bits argument.  Host-only.
 */
int64_t exl3_encode_slot_bytes(int32_t bits);

/*
 * exl3_encode_tiles: quantise tiles to trellis streams (pages: "Viterbi encoding
 * kernel": one thread block per 16x16 block of 256 weights, a forward Viterbi
 * pass that keeps the accumulated cost of every edge and takes the
 * minimum-cost path, the tail-biting boundary closed over the start states so
 * that the codeword's head and tail agree; instances per (K, codebook)).
 *   w         : fp32 [n_tiles][256] targets, element i of a tile = row i/16,
 *               column i%16 (the format's tile order), device.
 *   words     : uint16 [n_tiles][16*K] output streams in the format above, device.
 *   costs     : fp32 [n_tiles] sum of squared errors of each tile, device, or NULL.
 *   workspace : at least exl3_encode_slot_bytes(bits) bytes; more lets more
 *               tiles run at once.  Contents need no initialisation.
 * The search: state i+1 = (state i >> K) | (b << (16-K)); a step keeps, for every
 * state, the cheapest predecessor (first on ties) and adds (w_i - c(state))^2,
 * each operation rounded in fp32 with no fused multiply-add.  A free pass over
 * the targets rotated by 128 fixes the 16-K overlap bits (the low bits of its
 * state at position 0); a second pass starts in the states with those low bits
 * and ends in those whose top bits equal them, so every stream is a valid
 * tail-biting walk.  The result is deterministic.  n_tiles == 0 is a no-op;
 * EXL3_EINVAL for null w or words, n_tiles < 0 or a bad bits argument;
 * EXL3_EWORKSPACE for a workspace below one slot.
 */
int exl3_encode_tiles(const float* w, int64_t n_tiles, int32_t bits, uint16_t* words, float* costs,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Text for a status code (static storage; never NULL). */
const char* exl3_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXL3_H */
