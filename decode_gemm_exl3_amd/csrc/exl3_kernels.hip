// exl3_kernels.hip - decode, input rotation and GEMV kernels for gfx950.
#include <atomic>
#include <type_traits>

#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// ---------------------------------------------------------------------------
// decode_tile: one wave decodes 4 tiles, lane (n, g) = row n of tile 4*wave + g.
// Output is the bit-exact fp16 codebook value, in trellis order: element 16n + c
// of the tile.
// ---------------------------------------------------------------------------
template <int K, int CB>
__global__ __launch_bounds__(256) void decode_tile_kernel(const uint16_t* __restrict__ words,
                                                          int64_t n_tiles, uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    constexpr int64_t TILE_B = RowGeom<K>::DW_PER_TILE * 4;
    const int64_t tile0 = (int64_t)blockIdx.x * 16;
    const int64_t tile = tile0 + (threadIdx.x >> 6) * 4 + (lane >> 4);
    const bool valid = tile < n_tiles;
    const CbRegs cr = cb_regs<CB>();
    // tiles past the end read as zero through the buffer range check
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const char*>(words) + tile0 * TILE_B, (n_tiles - tile0) * TILE_B);
    uint32_t b[RowGeom<K>::NB];
    load_row<K>(rs, (uint32_t)((tile - tile0) * TILE_B) + row_offset<K>(n), 0u, b);
    finish_row<K>(n, b);  // every lane takes part in the DPP
    uint32_t q[16];
    decode_row<K, CB>(b, q, cr);
    if (valid) {
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = cb_pack<CB>(q[2 * j], q[2 * j + 1]);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + tile * 256 + n * 16);
        dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
        dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
    }
}

// 128-point Hadamard of one block held by 16 lanes (one DPP row), 8 values per
// lane: lane l16 holds inputs 8*l16 + e, e = 0..7.  H128 = H16 (x) H8 on
// (l16, e), so the three stages on e run inside the lane and the 16-point
// transform across the lanes of the row.
//
// Across lanes, any four butterfly stages whose partner masks form a basis of
// GF(2)^4 give the 16-point Walsh-Hadamard transform up to a permutation and
// signs of the outputs.  The masks 15, 7, 1, 2 are each one DPP pattern (row
// mirror, half-row mirror, two quad permutes).  Stage i pairs lane l with
// l ^ m_i; with b_i a bit set in m_i (3, 2, 0, 1), the lane with bit b_i clear
// keeps v + v', the other v' - v.  Keeping instead u = sigma * v per lane, with
// sigma the product of the stages' signs so far, every stage becomes
// u += c_i(l) * u(l ^ m_i) with c_i(l) = -1 exactly when bit b_i of l is set:
// one v_fmac_f32 with a DPP source per value.  After the four stages lane l
// holds, up to the sign s(l), outputs 8 * pos(l) + e, where
// pos(l) = 5 l0 ^ 6 l1 ^ 12 l2 ^ 8 l3 (l0..l3 the bits of l) and s(l) = -1 for
// the lanes of the mask 0xF9F6.  Both were derived by carrying the unit
// vectors through the stages; the parity tests check the result against the
// Hadamard matrix itself.
struct RowFwht {
    float c[4];  // +-1.0: the partner's factor in cross-lane stage i
    float osc;   // s(l) / 128: the sign the stages leave, and the x'/128 scale
    int pos;     // the 8-input group of the block this lane ends up holding
};

__device__ __forceinline__ RowFwht row_fwht_consts(int l16) {
    RowFwht k;
    k.c[0] = (l16 & 8) ? -1.0f : 1.0f;
    k.c[1] = (l16 & 4) ? -1.0f : 1.0f;
    k.c[2] = (l16 & 1) ? -1.0f : 1.0f;
    k.c[3] = (l16 & 2) ? -1.0f : 1.0f;
    k.osc = ((0xF9F6 >> l16) & 1) ? -1.0f / 128.0f : 1.0f / 128.0f;
    k.pos = ((l16 & 1) ? 5 : 0) ^ ((l16 & 2) ? 6 : 0) ^ ((l16 & 4) ? 12 : 0) ^ ((l16 & 8) ? 8 : 0);
    return k;
}

// u[e] += c * u[e] of the partner lane, for the 8 values.  v_fmac_f32 takes a
// DPP source only in assembly (the compiler folds DPP into adds and multiplies,
// not into the accumulating multiply-add).  The leading s_nop gives the wait
// states a DPP read needs after a vector write of its source (2) or of EXEC
// (5); within the block each value is read once, by the instruction that
// rewrites it.
#define EXL3_XLANE_STAGE(DPP)                                                                             \
    asm volatile("s_nop 4\n"                                                                              \
                 "v_fmac_f32_dpp %0, %0, %8 " DPP " row_mask:0xf bank_mask:0xf\n"                       \
                 "v_fmac_f32_dpp %1, %1, %8 " DPP " row_mask:0xf bank_mask:0xf\n"                       \
                 "v_fmac_f32_dpp %2, %2, %8 " DPP " row_mask:0xf bank_mask:0xf\n"                       \
                 "v_fmac_f32_dpp %3, %3, %8 " DPP " row_mask:0xf bank_mask:0xf\n"                       \
                 "v_fmac_f32_dpp %4, %4, %8 " DPP " row_mask:0xf bank_mask:0xf\n"                       \
                 "v_fmac_f32_dpp %5, %5, %8 " DPP " row_mask:0xf bank_mask:0xf\n"                       \
                 "v_fmac_f32_dpp %6, %6, %8 " DPP " row_mask:0xf bank_mask:0xf\n"                       \
                 "v_fmac_f32_dpp %7, %7, %8 " DPP " row_mask:0xf bank_mask:0xf"                         \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), \
                   "+v"(v[7])                                                                             \
                 : "v"(cc))

// Sign flip and first stage straight from the packed fp16 input: x * sign is
// exact in fp16 (sign is +-1), and the sum and difference of two fp16 values
// are exact in fp32.
__device__ __forceinline__ void row_load_pairs(const u32x4_t& xv, const u32x4_t& sv, float (&v)[8]) {
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        // (element copies first: a bit cast straight from a vector element reads element 0)
        const uint32_t xw = xv[d], sw = sv[d];
        const h2_t p = __builtin_bit_cast(h2_t, xw) * __builtin_bit_cast(h2_t, sw);
        const float a = (float)p[0], b = (float)p[1];
        v[2 * d] = a + b;
        v[2 * d + 1] = a - b;
    }
}

// The remaining stages: in-lane on e bits 1 and 2, then the four cross-lane
// stages.  Afterwards v[e] * k.osc = x'[8 * k.pos + e] / 128 of the block.
__device__ __forceinline__ void fwht128_row(float (&v)[8], const RowFwht& k) {
#pragma unroll
    for (int h = 2; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((e & h) == 0) {
                const float a = v[e], b = v[e + h];
                v[e] = a + b;
                v[e + h] = a - b;
            }
    float cc = k.c[0];
    EXL3_XLANE_STAGE("row_mirror");
    cc = k.c[1];
    EXL3_XLANE_STAGE("row_half_mirror");
    cc = k.c[2];
    EXL3_XLANE_STAGE("quad_perm:[1,0,3,2]");
    cc = k.c[3];
    EXL3_XLANE_STAGE("quad_perm:[2,3,0,1]");
}
#undef EXL3_XLANE_STAGE

// fp16(x'/128) of two values, packed (RNE, one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const h2_t h = h2_t{(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------------------
// rotate: xr[r][k] = fp16((H128 (sign * x[r]))[k] / 128).  16 lanes per block,
// 8 inputs per lane (one 16-byte load and store); a workgroup covers 16
// blocks of a row (blockIdx.x) and walks rows blockIdx.y, + gridDim.y, ...
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rotate_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ sign, int m, int n_in,
                                                     uint16_t* __restrict__ xr) {
    const int l16 = threadIdx.x & 15;
    const int bb = blockIdx.x * 16 + (threadIdx.x >> 4);  // 128-input block within the row
    // whole rows of 16 lanes leave together, so the DPP rows stay complete
    if (bb >= (n_in >> 7)) return;
    const int col = bb * 128 + l16 * 8;
    const RowFwht k = row_fwht_consts(l16);
    const u32x4_t sv = *reinterpret_cast<const u32x4_t*>(sign + col);
    for (int row = blockIdx.y; row < m; row += gridDim.y) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(x + (int64_t)row * n_in + col);
        float v[8];
        row_load_pairs(xv, sv, v);
        fwht128_row(v, k);
        u32x4_t o;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = pack_half2(v[2 * d] * k.osc, v[2 * d + 1] * k.osc);
        *reinterpret_cast<u32x4_t*>(xr + (int64_t)row * n_in + bb * 128 + k.pos * 8) = o;
    }
}

// ---------------------------------------------------------------------------
// rotate, group-major: the same values laid out xr[k / 8][r][k % 8] over
// `rows` >= m rows, the rows past m zero (the 256-row GEMM stages one 16-byte
// group of each row).  A workgroup rotates one 128-input block (blockIdx.x) of
// 16 rows (blockIdx.y), one row per 16 lanes, and transposes through LDS so
// that each group of 8 outputs leaves as one 256-byte run of 16 rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rotate_gm_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ sign, int m, int n_in,
                                                        uint16_t* __restrict__ xr, int rows) {
    __shared__ u32x4_t T[16][16];  // [group of the block][row]
    const int l16 = threadIdx.x & 15, rr = threadIdx.x >> 4;
    const int bb = blockIdx.x;
    const int row = blockIdx.y * 16 + rr;
    const RowFwht k = row_fwht_consts(l16);
    u32x4_t o = u32x4_t{0u, 0u, 0u, 0u};
    if (row < m) {  // whole 16-lane rows agree, so the DPP rows stay complete
        const int col = bb * 128 + l16 * 8;
        const u32x4_t sv = *reinterpret_cast<const u32x4_t*>(sign + col);
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(x + (int64_t)row * n_in + col);
        float v[8];
        row_load_pairs(xv, sv, v);
        fwht128_row(v, k);
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = pack_half2(v[2 * d] * k.osc, v[2 * d + 1] * k.osc);
    }
    T[k.pos][rr] = o;
    __syncthreads();
    const int g = threadIdx.x >> 4, r = threadIdx.x & 15;  // write side: group g, row r
    const int orow = blockIdx.y * 16 + r;
    if (orow < rows)
        *reinterpret_cast<u32x4_t*>(xr + ((int64_t)(bb * 16 + g) * rows + orow) * 8) = T[g][r];
}

// ---------------------------------------------------------------------------
// GEMV (small m).
//
// Matrix-core mapping (v_mfma_f32_16x16x32_f16, D[16x16] += A[16x32] B[32x16]):
//   B = weights.  Lane (n, g) supplies column n and the k slots of lane group g:
//       row n of tile 4*step + g of a strip, 4 weights per MFMA, each weight as
//       its two fp16 codebook halves in two k slots, so the matrix core also adds
//       the halves.  Each lane decodes its whole row (16 weights) per step.
//   A = rotated input.  Row r < m of A holds x'[r] (duplicated to match the two
//       halves) for the inputs of each lane group; rows r >= m are zero.
//   D[r][n] accumulates y[r][16*strip + n]; lane (n, g) holds D[4g + i][n].
// A step is one wave-wide load of 4 consecutive tiles of a strip (4 * 32K
// contiguous bytes).
//
// One launch may serve several projections of the same input (x, sign, n_in
// and K shared): their strips are numbered one after the other and handed out
// as one list, so q/k/v or gate/up cost one launch and one rotation of x.
//
// Persistent workgroups: workgroup b owns strips b, b + G, b + 2G, ... (G =
// grid size, about one workgroup per CU).  The input dimension is cut into
// chunks whose rotated input fits in LDS (usually one chunk).  For each chunk
// the workgroup rotates x into LDS once and then walks its strips; within a
// strip the W waves take consecutive runs of nsw steps.  Every wave keeps PF
// steps in flight and its load stream runs on across strip and chunk
// boundaries, so memory latency is paid once per launch rather than once per
// strip.  Per-wave partial sums live in LDS (each wave owns its slots, no
// barrier); at the end the waves' sums are added and y is written.  One kernel,
// no cross-workgroup reduction.  With PRE the input comes rotated from the
// pre-pass and is copied into LDS instead of rotated there.
// ---------------------------------------------------------------------------
template <int K, int PF, int CB, bool PRE>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvParams p) {
    // LDS: x' rows [m][xcols] | zero block [PF * 64] | partial sums [nj][W][m][16]
    extern __shared__ __align__(16) uint32_t xs[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int M = p.m;
    const int W = p.waves;
    const int nsw = p.nsw;                 // steps per wave per (strip, chunk), a multiple of PF
    // dwords per LDS row: the x' columns plus 4, so that the rows the 16 lanes
    // of a fragment read start 16 bytes apart in the banks (an unpadded stride
    // is a multiple of 256 bytes and puts all 16 rows on the same banks)
    const int xcols = W * nsw * 64 + GEMV_ROW_PAD;
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int nj = (p.n_strips - b + G - 1) / G;   // strips of this workgroup

    uint32_t* zero = xs + M * xcols;
    float* red = reinterpret_cast<float*>(zero + PF * 64);

    // Weight rows come through one buffer resource per projection: the per-step
    // offset is a scalar, the lane offset fixed; reads past the end (prefetch
    // after the last segment) return zero.
    constexpr uint32_t TILE_B = RowGeom<K>::DW_PER_TILE * 4;
    constexpr uint32_t STEP_B = 4 * TILE_B;
    const uint32_t loff = (uint32_t)g * TILE_B + row_offset<K>(n);
    const int col0 = 4 * wave * nsw;  // first tile column of this wave inside a chunk
    // projection of global strip s (uniform), and the strips before it
    auto proj_of = [&](int s) -> int {
        return (s >= p.strip_end[0]) + (s >= p.strip_end[1]) + (s >= p.strip_end[2]);
    };
    auto proj_begin = [&](int pi) -> int { return pi == 0 ? 0 : p.strip_end[pi - 1]; };
    // segment (c, j) = (chunk c, strip b + j * G), taken in the order (0, 0),
    // (0, 1), .., (1, 0), ..: its projection's resource, the byte offset of its
    // step 0 and the offset of the projection's last step.  Step offsets are
    // clamped to that last step, so a wave's padding steps past the end of the
    // last strip re-read real weights (they meet zero inputs) instead of
    // leaving the buffer.
    struct Seg {
        __amdgpu_buffer_rsrc_t rs;
        uint32_t off, lim;
    };
    auto seg_at = [&](int c, int j) -> Seg {
        if (c >= p.n_kchunks) return Seg{make_rsrc(p.trellis[0], 0), 0u, 0u};  // past the end: an empty buffer reads zeros
        const int s = b + j * G;
        const int pi = proj_of(s);
        const int ls = s - proj_begin(pi);
        const int64_t bytes = (int64_t)(p.n_out[pi] >> 4) * p.tiles_in * TILE_B;
        return Seg{make_rsrc(p.trellis[pi], bytes), (uint32_t)(((int64_t)ls * p.tiles_in + c * p.kc + col0) * TILE_B),
                   (uint32_t)(bytes - STEP_B)};
    };

    // Per-projection values for a lane's own projection index, picked with
    // selects from scalar registers: an indexed read of the argument block is a
    // vector load, and its wait would also cover the weight loads in flight.
    // The empty asm keeps the compiler from folding the selects back into one.
    static_assert(GEMV_MAX_PROJ == 4, "the selects below name every projection");
    auto sel4 = [](int pi, auto a0, auto a1, auto a2, auto a3) {
        asm volatile("" : "+s"(a0), "+s"(a1), "+s"(a2), "+s"(a3));
        return pi == 0 ? a0 : pi == 1 ? a1 : pi == 2 ? a2 : a3;
    };
    auto scale_of = [&](int pi) {
        return sel4(pi, p.out_scale[0], p.out_scale[1], p.out_scale[2], p.out_scale[3]);
    };
    auto y_of = [&](int pi) { return sel4(pi, p.y[0], p.y[1], p.y[2], p.y[3]); };
    auto n_out_of = [&](int pi) { return sel4(pi, p.n_out[0], p.n_out[1], p.n_out[2], p.n_out[3]); };
    auto begin_of = [&](int pi) { return sel4(pi, 0, p.strip_end[0], p.strip_end[1], p.strip_end[2]); };
    const RowFwht fk = row_fwht_consts(lane & 15);
    // 16 lanes per 128-input block, 8 inputs per lane (one 16-byte load of x
    // and of sign): rotate block blk of a chunk of nblk blocks (row blk / nblk)
    // into the chunk's LDS rows, xs[r][k] = dup(fp16(x'/128))
    auto rotate_block = [&](int blk, int nblk, const u32x4_t& xv, const u32x4_t& sv) {
        const int r = blk / nblk, bb = blk % nblk;
        float v[8];
        row_load_pairs(xv, sv, v);
        fwht128_row(v, fk);
        uint32_t d[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float t = v[e] * fk.osc;
            d[e] = pack_half2(t, t);  // duplicated for the two codebook halves
        }
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(xs + r * xcols + bb * 128 + fk.pos * 8);
        dst[0] = u32x4_t{d[0], d[1], d[2], d[3]};
        dst[1] = u32x4_t{d[4], d[5], d[6], d[7]};
    };
    auto block_col = [&](int blk, int nblk, int tc0) { return tc0 * 16 + (blk % nblk) * 128 + (lane & 15) * 8; };

    // ---- first loads: x and sign of this thread's first rotation block, the
    // weight stream, the scale of its first output in the final write.  The
    // first block is rotated in straight-line code, so that its wait covers
    // only the x and sign loads and the rotation runs under the weight burst;
    // the scale's latency hides behind the whole stream.
    const int nblk0 = (min(p.kc, p.tiles_in) * 16) >> 7;  // 128-input blocks of chunk 0
    const bool xpre = !PRE && !p.xr && (tid >> 4) < M * nblk0;
    u32x4_t xv0{}, sv0{};
    if (xpre) {
        const int blk = tid >> 4, col = block_col(blk, nblk0, 0);
        xv0 = *reinterpret_cast<const u32x4_t*>(p.x + (int64_t)(blk / nblk0) * p.n_in + col);
        sv0 = *reinterpret_cast<const u32x4_t*>(p.sign + col);
    }
    // Pre-rotated input (PRE): a chunk's rows are copied in 16-byte groups of
    // 8 inputs, taken row by row, XB per thread at a time with their loads
    // issued together; (xr_row, xr_grp) is the thread's next group.  The first
    // batch of chunk 0 is loaded here, ahead of the weight burst, so that its
    // wait does not cover the weight loads.
    constexpr int XB = 4;
    struct XBatch {
        u32x4_t v[XB];
        int r[XB], c8[XB];
    };
    auto xr_first = [&](int per_row, int& r, int& c8) {
        r = 0;
        c8 = tid;
        while (c8 >= per_row && r < M) {
            c8 -= per_row;
            ++r;
        }
    };
    auto xr_issue = [&](int tc0, int per_row, int& r, int& c8, XBatch& bt) {
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            bt.r[u] = r;
            bt.c8[u] = c8;
            if (r < M) bt.v[u] = *reinterpret_cast<const u32x4_t*>(p.xr + (int64_t)r * p.n_in + tc0 * 16 + c8 * 8);
            c8 += 64 * W;
            while (c8 >= per_row && r < M) {
                c8 -= per_row;
                ++r;
            }
        }
    };
    auto xr_store = [&](const XBatch& bt) {
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            if (bt.r[u] < M) {
                uint32_t d[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w2 = bt.v[u][e];
                    d[2 * e] = (w2 & 0xFFFFu) | (w2 << 16);  // duplicated for the two codebook halves
                    d[2 * e + 1] = (w2 >> 16) | (w2 & 0xFFFF0000u);
                }
                u32x4_t* dst = reinterpret_cast<u32x4_t*>(xs + bt.r[u] * xcols + bt.c8[u] * 8);
                dst[0] = u32x4_t{d[0], d[1], d[2], d[3]};
                dst[1] = u32x4_t{d[4], d[5], d[6], d[7]};
            }
        }
    };
    int xr_row = 0, xr_grp = 0;
    XBatch xb0;
    if constexpr (PRE) {
        const int per_row0 = min(p.kc, p.tiles_in) * 2;
        xr_first(per_row0, xr_row, xr_grp);
        xr_issue(0, per_row0, xr_row, xr_grp, xb0);
    }
    uint32_t buf[PF][RowGeom<K>::NB];
    {
        const Seg s0 = seg_at(0, 0);
#pragma unroll
        for (int u = 0; u < PF; ++u) load_row<K>(s0.rs, loff, min(s0.off + u * STEP_B, s0.lim), buf[u]);
    }
    // Loaded by every thread (those past the last output re-read output 0, so
    // the count of loads in flight does not depend on the thread), from global
    // memory (a flat load would make the next wait cover every load), and
    // converted where it is used, so that nothing waits for it here.
    uint16_t sc0;
    {
        const int t = tid < nj * M * 16 ? tid : 0;
        const int s = b + (t / (M * 16)) * G, pi = proj_of(s);
        using gu16 = const __attribute__((address_space(1))) uint16_t*;
        sc0 = *(gu16)(scale_of(pi) + (s - begin_of(pi)) * 16 + (t & 15));
    }
    if (xpre) rotate_block(tid >> 4, nblk0, xv0, sv0);
    for (int i = tid; i < PF * 64; i += 64 * W) zero[i] = 0u;

    const bool adata = n < M;
    const CbRegs cr = cb_regs<CB>();
    for (int c = 0; c < p.n_kchunks; ++c) {
        const int tc0 = c * p.kc;
        const int kcount = min(p.kc, p.tiles_in - tc0);
        // ---- rotate chunk c of x into LDS: xs[r][k] = dup(fp16(x'/128)) -------
        if (c > 0) __syncthreads();  // every wave is done with the previous chunk
        for (int i = kcount * 16 + tid; i < xcols; i += 64 * W)
            for (int r = 0; r < M; ++r) xs[r * xcols + i] = 0u;
        if (PRE || p.xr) {
            // rotated once by the pre-pass: copy the chunk, 8 inputs per lane,
            // each duplicated for the two codebook halves
            const int per_row = kcount * 2;  // 16-byte groups of a row in this chunk
            if constexpr (PRE) {
                if (c == 0)
                    xr_store(xb0);
                else
                    xr_first(per_row, xr_row, xr_grp);
                while (xr_row < M) {
                    XBatch bt;
                    xr_issue(tc0, per_row, xr_row, xr_grp, bt);
                    xr_store(bt);
                }
            } else {
                // one group per thread at a time: the launcher sends a
                // pre-rotated input to the PRE instance, so this is reached
                // only by a direct launch of this one with p.xr set
                for (int r = 0; r < M; ++r)
                    for (int c8 = tid; c8 < per_row; c8 += 64 * W) {
                        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p.xr + (int64_t)r * p.n_in + tc0 * 16 + c8 * 8);
                        uint32_t d[8];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t w2 = v[e];
                            d[2 * e] = (w2 & 0xFFFFu) | (w2 << 16);
                            d[2 * e + 1] = (w2 >> 16) | (w2 & 0xFFFF0000u);
                        }
                        u32x4_t* dst = reinterpret_cast<u32x4_t*>(xs + r * xcols + c8 * 8);
                        dst[0] = u32x4_t{d[0], d[1], d[2], d[3]};
                        dst[1] = u32x4_t{d[4], d[5], d[6], d[7]};
                    }
            }
        } else {
            // chunk 0's first block of each thread was rotated at the start
            const int nblk = (kcount * 16) >> 7;
            for (int blk = (tid >> 4) + (c == 0 ? 4 * W : 0); blk < M * nblk; blk += 4 * W) {
                const int col = block_col(blk, nblk, tc0);
                const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(p.x + (int64_t)(blk / nblk) * p.n_in + col);
                const u32x4_t sv = *reinterpret_cast<const u32x4_t*>(p.sign + col);
                rotate_block(blk, nblk, xv, sv);
            }
        }
        __syncthreads();

        Seg cur = seg_at(c, 0);
        for (int j = 0; j < nj; ++j) {
            // this segment's x' fragments: data lanes walk their row, others read zeros
            const uint32_t* ap = adata ? xs + n * xcols + wave * nsw * 64 + g * 16 : zero;
            const int astep = adata ? PF * 64 : 0;
            const Seg nxt = j + 1 < nj ? seg_at(c, j + 1) : seg_at(c + 1, 0);
            f32x4_t acc[4];  // one accumulator per MFMA of a step: no back-to-back dependent MFMAs
            // one round of PF steps; the first round of a segment starts the
            // accumulators from zero inside its first MFMAs
            auto round = [&](int st, auto first) {
                // refills of this round target the next round: same segment or the next
                const bool same = st + PF < nsw;
                const uint32_t roff = same ? cur.off + (st + PF) * STEP_B : nxt.off;
                const uint32_t rlim = same ? cur.lim : nxt.lim;
                const __amdgpu_buffer_rsrc_t rref = same ? cur.rs : nxt.rs;
#pragma unroll
                for (int u = 0; u < PF; ++u) {
                    // x' fragments first: their LDS latency hides behind the decode
                    u32x4_t av[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) av[t] = *reinterpret_cast<const u32x4_t*>(ap + u * 64 + 4 * t);
                    // decode in place, then refill the same registers: no copies,
                    // so the wait before each step covers only its own load
                    finish_row<K>(n, buf[u]);
                    uint32_t qq[16];
                    decode_row<K, CB>(buf[u], qq, cr);
                    __builtin_amdgcn_sched_barrier(0);
                    load_row<K>(rref, loff, min(roff + u * STEP_B, rlim), buf[u]);
                    // the refill stays here: the scheduler would otherwise sink the
                    // loads of the round to its end and expose the memory latency
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const u32x4_t bv = u32x4_t{qq[4 * t], qq[4 * t + 1], qq[4 * t + 2], qq[4 * t + 3]};
                        const f32x4_t cin = (decltype(first)::value && u == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[t];
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av[t]),
                                                                         __builtin_bit_cast(half8_t, bv), cin, 0, 0, 0);
                    }
                }
                ap += astep;
            };
            round(0, std::true_type{});
            for (int st = PF; st < nsw; st += PF) round(st, std::false_type{});
            // this wave's partial for strip j (its own slots: no barrier needed);
            // the first chunk writes every slot, later chunks add to it
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                if (r < M) {
                    const float v = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
                    float* slot = red + ((j * W + wave) * M + r) * 16 + n;
                    if (c == 0)
                        *slot = v;
                    else
                        *slot += v;
                }
            }
            cur = nxt;
        }
    }

    // ---- add the W waves' partial sums and write y ------------------------------
    __syncthreads();
    for (int idx = tid; idx < nj * M * 16; idx += 64 * W) {
        const int j = idx / (M * 16), r = (idx >> 4) % M, cc = idx & 15;
        float v = 0.f;
        for (int w = 0; w < W; ++w) v += red[((j * W + w) * M + r) * 16 + cc];
        const int s = b + j * G, pi = proj_of(s);
        const int o = (s - begin_of(pi)) * 16 + cc;
        const float sc = __half2float(__ushort_as_half(idx == tid ? sc0 : scale_of(pi)[o])) * 128.0f;
        y_of(pi)[(int64_t)r * n_out_of(pi) + o] = __half_as_ushort(__float2half_rn(sc * v));
    }
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <int K, int CB>
static hipError_t launch_decode_k(const uint16_t* words, int64_t n_tiles, uint16_t* out, hipStream_t s) {
    const int64_t blocks = (n_tiles + 15) / 16;
    hipLaunchKernelGGL((decode_tile_kernel<K, CB>), dim3((unsigned)blocks), dim3(256), 0, s, words, n_tiles, out);
    return hipGetLastError();
}

template <int CB>
static hipError_t launch_decode_cb(int K, const uint16_t* words, int64_t n_tiles, uint16_t* out, hipStream_t s) {
    switch (K) {
        case 1: return launch_decode_k<1, CB>(words, n_tiles, out, s);
        case 2: return launch_decode_k<2, CB>(words, n_tiles, out, s);
        case 3: return launch_decode_k<3, CB>(words, n_tiles, out, s);
        case 4: return launch_decode_k<4, CB>(words, n_tiles, out, s);
        case 5: return launch_decode_k<5, CB>(words, n_tiles, out, s);
        case 6: return launch_decode_k<6, CB>(words, n_tiles, out, s);
        case 7: return launch_decode_k<7, CB>(words, n_tiles, out, s);
        case 8: return launch_decode_k<8, CB>(words, n_tiles, out, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(int K, int cb, const uint16_t* words, int64_t n_tiles, uint16_t* out, hipStream_t s) {
    return cb == 0 ? launch_decode_cb<0>(K, words, n_tiles, out, s) : launch_decode_cb<1>(K, words, n_tiles, out, s);
}

hipError_t launch_rotate(const uint16_t* x, const uint16_t* sign, int m, int n_in, uint16_t* xr, hipStream_t s,
                         int rows) {
    if (rows > 0) {
        if (rows < m || rows % 16 != 0 || rows / 16 > 65535) return hipErrorInvalidValue;
        hipLaunchKernelGGL(rotate_gm_kernel, dim3((unsigned)(n_in >> 7), (unsigned)(rows / 16)), dim3(256), 0, s, x,
                           sign, m, n_in, xr, rows);
        return hipGetLastError();
    }
    const unsigned gx = (unsigned)(((n_in >> 7) + 15) / 16);
    const unsigned gy = (unsigned)(m < 65535 ? m : 65535);
    hipLaunchKernelGGL(rotate_kernel, dim3(gx, gy), dim3(256), 0, s, x, sign, m, n_in, xr);
    return hipGetLastError();
}

// PRE: the input was rotated by the pre-pass (p.xr).  A kernel instance of its
// own: it carries the batched copy and no rotation code, and the instance that
// rotates in the kernel keeps the instruction stream it has without them.
template <int K, int PF, int CB, bool PRE>
static hipError_t launch_gemv_kpp(const GemvParams& p, hipStream_t s) {
    const size_t lds = gemv_lds_bytes(p.m, p.waves, p.nsw, PF, (p.n_strips + p.grid - 1) / p.grid);
    // allow more than 64 KB of dynamic LDS, once per device
    static std::atomic<unsigned long long> attr_set{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const unsigned long long bit = 1ull << (dev & 63);
    if (!(attr_set.load(std::memory_order_acquire) & bit)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_kernel<K, PF, CB, PRE>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, GEMV_LDS_BUDGET);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit, std::memory_order_release);
    }
    hipLaunchKernelGGL((gemv_kernel<K, PF, CB, PRE>), dim3(p.grid), dim3(64 * p.waves), lds, s, p);
    return hipGetLastError();
}

template <int K, int PF, int CB>
static hipError_t launch_gemv_kp(const GemvParams& p, hipStream_t s) {
    return p.xr ? launch_gemv_kpp<K, PF, CB, true>(p, s) : launch_gemv_kpp<K, PF, CB, false>(p, s);
}

template <int K, int CB>
static hipError_t launch_gemv_k(const GemvParams& p, hipStream_t s) {
    switch (p.pf) {
        case 2: return launch_gemv_kp<K, 2, CB>(p, s);
        case 4: return launch_gemv_kp<K, 4, CB>(p, s);
        case 8: return launch_gemv_kp<K, 8, CB>(p, s);
    }
    return hipErrorInvalidValue;
}

template <int CB>
static hipError_t launch_gemv_cb(int K, const GemvParams& p, hipStream_t s) {
    switch (K) {
        case 1: return launch_gemv_k<1, CB>(p, s);
        case 2: return launch_gemv_k<2, CB>(p, s);
        case 3: return launch_gemv_k<3, CB>(p, s);
        case 4: return launch_gemv_k<4, CB>(p, s);
        case 5: return launch_gemv_k<5, CB>(p, s);
        case 6: return launch_gemv_k<6, CB>(p, s);
        case 7: return launch_gemv_k<7, CB>(p, s);
        case 8: return launch_gemv_k<8, CB>(p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int K, int cb, const GemvParams& p, hipStream_t s) {
    return cb == 0 ? launch_gemv_cb<0>(K, p, s) : launch_gemv_cb<1>(K, p, s);
}

}  // namespace exl3
