// exl3_gemm.hip - decode-matmul for larger m on the matrix cores (gfx950).
//
// The input is rotated once by a pre-pass (x'/128 in fp16, workspace).  Two
// kernels: for m <= 128 an eight-wave workgroup owns a BM x 256 block of y
// (BM = 64 or 128, below); for m > 128 a four-wave workgroup owns a 256 x 256
// block (gemm4_kernel, further down).
//
// Eight-wave kernel: wave w owns rows BM/2 (w >> 2) .. +BM/2-1 and outputs
// 64 (w & 3) .. +63 (4 strips).  The input dimension is walked in steps of
// BK = 64 (4 tile columns).
//
// Each weight is decoded once per workgroup and used for BM rows: of the two
// waves that own the same outputs (w and w ^ 4, which share a SIMD), one
// decodes the first 32 inputs of the step and the other the last 32, each
// straight into v_mfma B fragments (lane (n, g): half row g & 1 of row n of
// tile column g >> 1, halves summed to fp16) and writes them to LDS, where both
// read them.  x' is staged in LDS too.
// Both LDS buffers are double-buffered, so a step needs one barrier.
//
// The decode is vector-ALU work and the product matrix-core work; the two only
// overlap across waves.  So the partners run out of phase: after the barrier
// of step s, the first decodes step s + 1 and then runs its MFMAs of step s,
// the second runs its MFMAs first and then decodes.  While one decodes, the
// other keeps the matrix core busy.  The two are separate copies of the main
// loop, so neither has a data-dependent branch.
#include <type_traits>

#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

constexpr int GM_BN = GEMM_BN;        // 16 strips, 64 outputs per wave
constexpr int GM_BK = 64;             // 4 tile columns
constexpr int GM_LD = GM_BK + 8;      // padded LDS row stride in halves (144 bytes)
constexpr int GM_B_FRAGS = 2 * 4 * 4 * 64;  // [k half][output quarter][fragment][lane], 16 bytes each
constexpr int GM_TLD = 72;   // halves per row of a wave's 16 x 64 fp16 output fragment in LDS (144 bytes)
constexpr int GM_TLDF = 68;  // floats per row of the same in fp32 (272 bytes)
static_assert(8 * 16 * GM_TLDF * 4 <= 2 * GM_B_FRAGS * 16, "output fragments of 8 waves fit the B buffers");

// fp16 pair (RNE), first value in the low half.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2_t{(_Float16)a, (_Float16)b});
}

// The value of lane n ^ 1 (DPP quad_perm [1, 0, 3, 2]).
__device__ __forceinline__ float lane_pair_swap(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}

// BM = 64 rows per block for m <= 64, 128 for m <= 128 (the decode of each
// weight is most of the work at such m, and larger blocks would multiply
// padding rows).
template <int K, int CB, int BM>
__global__ __launch_bounds__(512, 1) void gemm_kernel(GemmParams p) {
    constexpr int WR = BM / 2;   // rows per wave
    constexpr int RF = BM / 32;  // 16-row fragments per wave
    constexpr int AL = BM / 64;  // x' staging loads per lane per step
    __shared__ __align__(16) uint16_t As[2][BM * GM_LD];
    __shared__ __align__(16) u32x4_t Bs[2][GM_B_FRAGS];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int mh = wave >> 2, nq = wave & 3;  // row half, output quarter
    // XCD-aware block order: consecutive workgroups go to different XCDs (round
    // robin), so hand each XCD a contiguous run of the m-major block order; its
    // L2 then keeps the x' rows of one m-block while it sweeps the outputs.
    const int nbx = gridDim.x, total = gridDim.x * gridDim.y;
    int lin = blockIdx.x + blockIdx.y * nbx;
    if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
    const int m0 = (lin / nbx) * BM;
    const int s0 = (lin % nbx) * (GM_BN / 16) + 4 * nq;  // first strip of this wave
    // this workgroup's tile columns (split-k): [t0, t1)
    const int t0 = blockIdx.z * p.kz;
    const int t1 = min(p.tiles_in, t0 + p.kz);
    const CbRegs cr = cb_regs<CB>();

    // ---- weights: fragment j = strip s0 + j, tile column 2 mh + (g >> 1) of the
    // step, half g & 1 of row n.  Lane offsets are fixed; strip and step go in
    // the scalar offset.  Both are clamped to the last strip and the last step,
    // so no load leaves the weights: strips past the end re-read the last strip
    // (their outputs are never written) and the prefetch past the last step
    // re-reads it (its decode is never used).
    constexpr int KDH = HalfGeom<K>::KDH;
    constexpr uint32_t TILE_B = RowGeom<K>::DW_PER_TILE * 4;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.trellis, (int64_t)p.n_strips * p.tiles_in * TILE_B);
    const int h = g & 1;
    uint32_t voff[KDH];
#pragma unroll
    for (int i = 0; i < KDH; ++i) voff[i] = (uint32_t)(g >> 1) * TILE_B + half_dword<K>(n, h, i) * 4;
    const uint32_t bsh = half_shift<K>(n, h);
    const uint32_t strip_b = (uint32_t)p.tiles_in * TILE_B;
    uint32_t rows[4][KDH];  // the next step to decode
    const int last_tc = p.tiles_in - 4;  // first tile column of the last step
    auto load_frag = [&](int j, int tc) {
        const uint32_t so = (uint32_t)min(s0 + j, p.n_strips - 1) * strip_b + (uint32_t)(min(tc, last_tc) + 2 * mh) * TILE_B;
#pragma unroll
        for (int i = 0; i < KDH; ++i) rows[j][i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff[i], so, kNT);
    };
    // decode this wave's 4 fragments of the step held in rows[] into LDS, and
    // refill rows[] with tile column tc_next
    auto decode_step = [&](int tc_next, int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t d[KDH];
            if constexpr (HalfGeom<K>::ALIGNED) {
#pragma unroll
                for (int i = 0; i < KDH; ++i) d[i] = rows[j][i];
            } else {
#pragma unroll
                for (int i = 0; i < KDH; ++i)
                    d[i] = __builtin_amdgcn_alignbit(rows[j][i + 1 < KDH ? i + 1 : i], rows[j][i], bsh);
            }
            uint32_t q[8];
            decode_half<K, CB>(d, q, cr);
            // refill after the decode has consumed the rows, into the same
            // registers (the fences keep the scheduler from hoisting the loads,
            // which would force copies and a wait for them)
            __builtin_amdgcn_sched_barrier(0);
            load_frag(j, tc_next);
            __builtin_amdgcn_sched_barrier(0);
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = cb_pack<CB>(q[2 * e], q[2 * e + 1]);
            Bs[buf][((mh * 4 + nq) * 4 + j) * 64 + lane] = u32x4_t{o[0], o[1], o[2], o[3]};
        }
    };

    // ---- x' staging: each load instruction of a wave covers 8 whole rows of the
    // step (8 lanes x 16 bytes per row), so wave w stages rows (BM / 8) w ..
    // + BM / 8 - 1 in BM / 64 loads.  Rows past m read as zero through the
    // buffer range check (the row is in the lane offset); the column goes in the
    // scalar offset, clamped to the last step so that no load leaves its row.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.xr + (int64_t)m0 * p.n_in, ((int64_t)p.m - m0) * p.n_in * 2);
    const int arow = (BM / 8) * wave + (lane >> 3), acol = (lane & 7) * 8;  // row of load c: arow + 8c; col in halves
    const uint32_t aoff = (uint32_t)arow * p.n_in * 2 + acol * 2;
    const uint32_t arow8 = 8u * p.n_in * 2;  // bytes between the rows of consecutive loads
    u32x4_t areg[AL];
    auto load_a = [&](int tc) {
#pragma unroll
        for (int c = 0; c < AL; ++c)  // past the end: range check
            areg[c] = __builtin_bit_cast(u32x4_t,
                                         __builtin_amdgcn_raw_buffer_load_b128(ra, aoff + c * arow8,
                                                                               min(tc, last_tc) * 32, 0));
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int c = 0; c < AL; ++c)
            *reinterpret_cast<u32x4_t*>(&As[buf][(arow + 8 * c) * GM_LD + acol]) = areg[c];
    };

    f32x4_t acc[RF][4];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // 32 inputs (k half kk) of a step: RF row fragments x 4 output fragments;
    // the B fragments of k half kk were decoded by the wave with mh == kk
    auto mfma_half = [&](int buf, int kk) {
        // all 4 B and 8 A fragments of the half are read first: one LDS latency,
        // then 32 back-to-back MFMAs
        half8_t b[4], af[RF];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = __builtin_bit_cast(half8_t, Bs[buf][((kk * 4 + nq) * 4 + j) * 64 + lane]);
        const uint16_t* abase = &As[buf][(WR * mh + n) * GM_LD + 32 * kk + 8 * g];
#pragma unroll
        for (int i = 0; i < RF; ++i) af[i] = *reinterpret_cast<const half8_t*>(abase + i * 16 * GM_LD);
#pragma unroll
        for (int i = 0; i < RF; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], b[j], acc[i][j], 0, 0, 0);
    };

    // ---- prologue: step t0 decoded and staged
#pragma unroll
    for (int j = 0; j < 4; ++j) load_frag(j, t0);
    load_a(t0);
    decode_step(t0 + 4, 0);
    store_a(0);
    load_a(t0 + 4);
    __syncthreads();

    // One copy of the main loop per partner, with its phase fixed at compile
    // time and no condition inside: the decode and the x' staging run every
    // step (in the last step they fetch past the end, decode zeros and stage
    // data that nothing reads), so the trellis rows and the staged x' each have
    // one definition and their loads stay in flight across the step.
    auto main_loop = [&](auto phase) {
        constexpr int MH = decltype(phase)::value;
        int buf = 0;
        for (int tc = t0; tc < t1; tc += 4, buf ^= 1) {
            // the next step's x' goes to the other buffer: its last readers were
            // in the previous step, before this step's barrier
            store_a(buf ^ 1);
            load_a(tc + 8);
            if constexpr (MH == 0) {  // decode the next step, then this step's MFMAs
                decode_step(tc + 8, buf ^ 1);
                mfma_half(buf, 0);
                mfma_half(buf, 1);
            } else {  // MFMAs first, then decode the next step
                mfma_half(buf, 1);
                mfma_half(buf, 0);
                decode_step(tc + 8, buf ^ 1);
            }
            __syncthreads();
        }
    };
    if (mh == 0)
        main_loop(std::integral_constant<int, 0>{});
    else
        main_loop(std::integral_constant<int, 1>{});
    // D[4g + r][n] of fragment (i, j): row WR mh + 16i + 4g + r, output 16 (s0 + j) + n.
    // The results leave through LDS (the B buffers, free after the last
    // barrier), one 16-row fragment at a time in a region of each wave's own,
    // in 16-byte runs of rows rather than 2- or 4-byte pieces.  A wave reads
    // back only what it wrote, and its LDS operations run in order.
    if (p.zsplit > 1) {  // fp32 partial sums of this split; the reduction scales them
        float* part = p.part + (int64_t)blockIdx.z * p.m * p.n_out;
        float* T = reinterpret_cast<float*>(&Bs[0][0]) + wave * 16 * GM_TLDF;
#pragma unroll
        for (int i = 0; i < RF; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) T[(4 * g + r) * GM_TLDF + 16 * j + n] = acc[i][j][r];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = lane + 64 * t, row = c >> 4, q = c & 15;  // 16 runs of 4 outputs per row
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(T + row * GM_TLDF + q * 4);
                const int grow = m0 + WR * mh + 16 * i + row, o = 16 * s0 + 4 * q;
                if (grow < p.m && o < p.n_out) *reinterpret_cast<u32x4_t*>(part + (int64_t)grow * p.n_out + o) = v;
            }
        }
        return;
    }
    uint16_t* T = reinterpret_cast<uint16_t*>(&Bs[0][0]) + wave * 16 * GM_TLD;
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int o = (s0 + j) * 16 + n;
        sc[j] = o < p.n_out ? __half2float(__ushort_as_half(p.out_scale[o])) * 128.0f : 0.0f;
    }
    // lanes n and n ^ 1 hold the same four rows of neighbouring outputs: the
    // even lane writes rows 0 and 1 of the pair of outputs, the odd lane rows
    // 2 and 3, each as fp16 pairs, after trading two values across the pair
    const bool odd = (n & 1) != 0;
#pragma unroll
    for (int i = 0; i < RF; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = sc[j] * acc[i][j][r];
            const float x0 = odd ? v[0] : v[2], x1 = odd ? v[1] : v[3];
            const float t0 = lane_pair_swap(x0), t1 = lane_pair_swap(x1);
            uint32_t* dst = reinterpret_cast<uint32_t*>(T + (4 * g + (odd ? 2 : 0)) * GM_TLD + 16 * j + (n & ~1));
            dst[0] = odd ? pack_h2(t0, v[2]) : pack_h2(v[0], t0);
            dst[GM_TLD / 2] = odd ? pack_h2(t1, v[3]) : pack_h2(v[1], t1);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int c = lane + 64 * t, row = c >> 3, q = c & 7;  // 8 runs of 8 outputs per row
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(T + row * GM_TLD + q * 8);
            const int grow = m0 + WR * mh + 16 * i + row, o = 16 * s0 + 8 * q;
            if (grow < p.m && o < p.n_out) *reinterpret_cast<u32x4_t*>(p.y + (int64_t)grow * p.n_out + o) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Row blocks of 256 (m > 128): four waves, one per SIMD.  Wave w owns the
// outputs of strips 4w .. 4w + 3 of the block (64 outputs) for all 256 rows,
// so each weight is decoded once per workgroup, by the wave that uses it,
// straight into its MFMA B operands: no weight goes through LDS.  The 256
// accumulators per lane (16 row tiles x 4 strips) sit in the accumulation
// registers.  Only x' is shared, staged in LDS in four buffers.
//
// Input order inside a step of 64 inputs (4 tile columns): lane (n, g) of a
// B operand decodes the whole row n of tile column g (16 weights, the
// row-owning lane layout of the GEMV) and feeds its first 8 weights to the
// MFMAs of k half 0 and the last 8 to those of k half 1.  So the MFMA's k
// slots 8g..8g+7 of half h hold step inputs 16g + 8h .. +7: the 16-byte group
// 2g + h.  The A operands read the same groups, which the rotation pre-pass
// lays out group-major (x'[k / 8][row][k % 8]) so that a block's step is 8
// contiguous 4 KB runs.
//
// A step runs its 64 MFMAs of k half 0, then the 64 of k half 1.  During half
// 0 the wave decodes the half-1 weights of the same step (states 8..15 of its
// rows); during half 1, the half-0 weights of the next step (states 0..7 of
// the next rows).  So each B operand is rewritten only after the MFMAs that
// read it, and one set of B registers serves every step.  A step's rows are
// loaded once, about a step and a half before their first use, into one of two
// sets that alternate with the step's parity (the main loop holds two steps).
// x' goes from memory straight into LDS (buffer loads to LDS, no registers)
// three steps ahead, into the fourth of four buffers; the barrier that ends a
// step waits only for the loads issued a step earlier.  A fragments are read
// two row tiles ahead.  Scheduling fences keep each unit of that work next to
// one MFMA, so the vector ALU work issues while the matrix core runs: with one
// wave per SIMD nothing else covers a stall.  One barrier per step.
// ---------------------------------------------------------------------------
constexpr int G4_BUFS = 4;  // x' buffers in LDS, 32 KB each: [group 8][row 256] x 16 bytes
constexpr int G4_TLD = 72;  // halves per row of a wave's 256 x 64 output tile in LDS (144 bytes: rows of a
                            // 16-byte read stay aligned, rows 4 apart fall on different banks)
constexpr int G4_TLDF = 68;  // floats per row of a wave's 128 x 64 fp32 half tile (272 bytes, same reasons)
constexpr int G4_LDS = (G4_BUFS * 8 * 256 * 16 > 4 * GEMM_BM * G4_TLD * 2) ? G4_BUFS * 8 * 256 * 16
                                                                            : 4 * GEMM_BM * G4_TLD * 2;
static_assert(4 * (GEMM_BM / 2) * G4_TLDF * 4 <= G4_LDS, "fp32 half tiles fit the LDS of the kernel");

#define G4_FENCE __builtin_amdgcn_sched_barrier(0)

// v_mad_u32_u16 of the codebook for state c of a finished row (state c at bit
// cK of b[]): the product word p.  Windows that two states of the same half
// share (K divides 16) are kept in win[] by the first.
template <int K, int CB>
__device__ __forceinline__ uint32_t g4_mad(int c, const uint32_t (&b)[RowGeom<K>::NB], uint32_t (&win)[16],
                                          const CbRegs& r) {
    constexpr int NB = RowGeom<K>::NB;
    constexpr uint32_t A = CB == 0 ? CB_A : CB1_A;
    const int P = c * K, dw = P >> 5, sh = P & 31;
    uint32_t w = b[dw];
    bool hi = false;
    if (sh == 16) {
        hi = true;
    } else if (sh != 0) {
        const int partner = c - 16 / K;  // state whose window holds this one in its high half
        if ((16 % K) == 0 && sh > 16 && partner >= (c & 8)) {
            w = win[partner];
            hi = true;
        } else {
            w = __builtin_amdgcn_alignbit(b[(dw + 1 < NB) ? dw + 1 : dw], b[dw], (uint32_t)sh);
            win[c] = w;
        }
    }
    uint32_t p;
    if (hi)
        asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(p) : "v"(w), "s"(A), "v"(r.vB));
    else
        asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(p) : "v"(w), "s"(A), "v"(r.vB));
    return p;
}

// Two values as one fp16x2 dword.  Codebook 0: lo already holds the first
// value (high half zero); the second is summed from its word straight into the
// high half (SDWA, the low half preserved): one instruction, not an add, an
// add and a merge.
template <int CB>
__device__ __forceinline__ uint32_t g4_pack(uint32_t lo, uint32_t q1) {
    if constexpr (CB == 0) {
        asm("s_nop 0\n\t"
            "v_add_f16_sdwa %0, %1, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0 src1_sel:WORD_1"
            : "+v"(lo)
            : "v"(q1));
        return lo;
    } else {
        return cb_pack<CB>(lo, q1);
    }
}

// D += A B with D in accumulation registers.  In assembly so that the
// register allocator keeps all 256 accumulators in place (with the builtin it
// moves them between register files every step).  The compiler does not see
// this MFMA, so the schedule keeps its hazards away: every B operand is
// written by the vector ALU at least two MFMAs before it is read, A operands
// come from LDS (the wait counts see the asm operands), and the accumulators
// are read only after the main loop, behind explicit wait states.
__device__ __forceinline__ void g4_mfma(f32x4_t& d, const half8_t& a, const u32x4_t& b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

template <int K, int CB>
__global__ __launch_bounds__(256, 1) void gemm4_kernel(GemmParams p) {
    __shared__ __align__(16) u32x4_t As[G4_LDS / 16];  // x' staging, then the output tiles
    constexpr int NB = RowGeom<K>::NB;
    constexpr uint32_t TILE_B = RowGeom<K>::DW_PER_TILE * 4;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    // XCD-aware block order (as the eight-wave kernel)
    const int nbx = gridDim.x, total = gridDim.x * gridDim.y;
    int lin = blockIdx.x + blockIdx.y * nbx;
    if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
    const int m0 = (lin / nbx) * GEMM_BM;
    const int s0 = (lin % nbx) * (GEMM_BN / 16) + 4 * wave;  // first strip of this wave
    const int k0 = blockIdx.z * (p.kz / 4);                   // steps of this split: [k0, k1)
    const int k1 = min(p.tiles_in / 4, k0 + p.kz / 4);
    const CbRegs cr = cb_regs<CB>();

    // weights: lane (n, g) loads row n of tile column 4 ks + g of strips s0 .. s0 + 3.
    // The strip and the step go in the scalar offset, clamped to the last strip
    // and the last step, so no load leaves the weights: strips past the end
    // re-read the last strip (their outputs are never written), steps past the
    // last re-read it (their decode is never used).
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.trellis, (int64_t)p.n_strips * p.tiles_in * TILE_B);
    const uint32_t voff = (uint32_t)g * TILE_B + row_offset<K>(n);
    const uint32_t strip_b = (uint32_t)p.tiles_in * TILE_B;
    uint32_t rows[2][4][NB];  // [step parity][strip]
    uint32_t bq[2][4][4];     // B operands [k half][strip]
    const int last_ks = p.tiles_in / 4 - 1;
    auto load_rows = [&](uint32_t (&rr)[4][NB], int j, int ks) {
        load_row<K>(rs, voff, (uint32_t)min(s0 + j, p.n_strips - 1) * strip_b + (uint32_t)min(ks, last_ks) * 4 * TILE_B,
                    rr[j]);
    };

    // x': wave w stages groups 2w and 2w + 1 of a step, 64 rows per load,
    // straight from memory into LDS (buffer loads to LDS: M0 holds the wave's
    // destination, lane i writes 16 bytes at +16 i).  The group goes in the
    // scalar offset, its step clamped to the last, so the staging past the last
    // step re-reads it (into a buffer nothing reads) instead of leaving x'.
    const int64_t xrows = p.rows;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.xr, xrows * p.n_in * 2);
    const uint32_t avoff = (uint32_t)(m0 + lane) * 16;
    const uint32_t agrp = (uint32_t)xrows * 16;  // bytes between groups
    auto stage_a = [&](int i, int ks, int buf) {  // load i of 8: group 2w + (i >> 2), rows 64 (i & 3) ..
        const int c = 2 * wave + (i >> 2), q = i & 3;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(As + buf * 2048 + c * 256 + q * 64), 16,
            avoff + (uint32_t)q * 1024, (uint32_t)(min(ks, last_ks) * 8 + c) * agrp, 0, 0);
    };
    // fragment (row tile rt, k half h) of a buffer: lane (n, g) reads group 2g + h of row 16 rt + n
    const int afrag = 2 * g * 256 + n;

    f32x4_t acc[16][4];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: x' of steps k0 .. k0 + 2 into buffers 0 .. 2; half 0 of
    // step k0 decoded from rows[0] (finished), rows[1] hold step k0 + 1
#pragma unroll
    for (int j = 0; j < 4; ++j) load_rows(rows[0], j, k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) load_rows(rows[1], j, k0 + 1);
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i) stage_a(i, k0 + t, t);
    {
        uint32_t win[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            finish_row<K>(n, rows[0][j]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t pa = g4_mad<K, CB>(2 * e, rows[0][j], win, cr);
                const uint32_t pb = g4_mad<K, CB>(2 * e + 1, rows[0][j], win, cr);
                bq[0][j][e] = cb_pack<CB>(cb_word<CB>(pa, cr), cb_word<CB>(pb, cr));
            }
        }
    }
    // every load of the prologue, the staging of steps k0 .. k0 + 2 included,
    // has landed (the steps' own waits count only their loads)
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);  // vmcnt(0)
    __syncthreads();
    half8_t ar[4];  // A fragments, ring of row tiles
#pragma unroll
    for (int t = 0; t < 2; ++t) ar[t] = __builtin_bit_cast(half8_t, As[afrag + t * 16]);

    // ---- one step ks: buffers (ks - k0) % 4 hold x' of ks, + 1 of ks + 1 (+ 2
    // of ks + 2, landing), + 3 gets ks + 3.  rows[P] hold step ks (finished),
    // rows[P ^ 1] step ks + 1.
    auto step = [&](int ks, auto par) {
        constexpr int P = decltype(par)::value;
        const int b0 = (ks - k0) & 3;
        const u32x4_t* acur = As + b0 * 2048 + afrag;
        const u32x4_t* anext = As + ((b0 + 1) & 3) * 2048 + afrag;
        const int bs = (b0 + 3) & 3;
        uint32_t win[16];
        uint32_t pa = 0, pb = 0, qa = 0, qb = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // half 0 decodes states 8..15 of rows[P] (step ks) into bq[1] and
            // then reloads them with step ks + 2; half 1 finishes rows[P ^ 1]
            // (step ks + 1) and decodes its states 0..7 into bq[0]
            uint32_t (&rr)[4][NB] = h == 0 ? rows[P] : rows[P ^ 1];
#pragma unroll
            for (int rt = 0; rt < 16; ++rt) {
                {  // fragment two row tiles ahead: (rt + 2, h), then (rt - 14, 1), then the next step's (rt - 14, 0)
                    const int t2 = rt + 2;
                    const u32x4_t* src = (h == 1 && t2 >= 16) ? anext : acur;
                    const int hh = t2 >= 16 ? h ^ 1 : h;
                    ar[t2 & 3] = __builtin_bit_cast(half8_t, src[hh * 256 + (t2 & 15) * 16]);
                }
                G4_FENCE;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int idx = 4 * rt + j;
                    const u32x4_t bv = u32x4_t{bq[h][j][0], bq[h][j][1], bq[h][j][2], bq[h][j][3]};
                    g4_mfma(acc[rt][j], ar[rt & 3], bv);
                    // decode unit idx: strip sd, state pair pr, kind
                    const int sd = idx >> 4, pr = (idx >> 2) & 3, kind = idx & 3;
                    const int c0 = (h == 0 ? 8 : 0) + 2 * pr;
                    uint32_t (&b)[NB] = rr[sd];
                    if (kind == 0) {
                        if (h == 1 && pr == 0) finish_row<K>(n, b);
                        pa = g4_mad<K, CB>(c0, b, win, cr);
                    } else if (kind == 1) {
                        pb = g4_mad<K, CB>(c0 + 1, b, win, cr);
                    } else if (kind == 2) {
                        qa = cb_word<CB>(pa, cr);
                        qb = cb_word<CB>(pb, cr);
                        if constexpr (CB == 0) qa = cb_sum(qa);  // first value, high half zero
                    } else {
                        bq[h ^ 1][sd][pr] = g4_pack<CB>(qa, qb);
                        if (h == 0 && pr == 3) load_rows(rr, sd, ks + 2);  // the row is decoded: refill
                    }
                    if (h == 0 && j == 1 && rt < 8) stage_a(rt, ks + 3, bs);
                    G4_FENCE;
                }
            }
        }
        // x' of step ks + 2 (this wave's loads of the previous step) has landed:
        // only the 15 memory loads issued after them (3 row loads of the
        // previous step, the 12 loads of this one) may still be in flight
        __builtin_amdgcn_s_waitcnt(0x0F70 | 15);  // vmcnt(15)
        __builtin_amdgcn_s_barrier();
    };

    int ks = k0;
    for (; ks + 1 < k1; ks += 2) {
        step(ks, std::integral_constant<int, 0>{});
        step(ks + 1, std::integral_constant<int, 1>{});
    }
    if (ks < k1) step(ks, std::integral_constant<int, 0>{});
    // the last MFMAs' results: 8-pass writes need 11 wait states before a read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");

    // D[4g + r][n] of (rt, j): row m0 + 16 rt + 4g + r, output 16 (s0 + j) + n.
    // The results leave through LDS, each wave's tile row by row, in 16-byte
    // runs of rows rather than 2- or 4-byte pieces.  The staging loads of the
    // last steps (past the end) still land in LDS, so every one has to finish
    // first; afterwards a wave reads back only its own tile, and its LDS
    // operations run in order.
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);  // vmcnt(0)
    __syncthreads();
    if (p.zsplit > 1) {  // fp32 partial sums of this split, 128 rows of the tile at a time
        float* part = p.part + (int64_t)blockIdx.z * p.m * p.n_out;
        float* T = reinterpret_cast<float*>(As) + wave * (GEMM_BM / 2) * G4_TLDF;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) T[(16 * i + 4 * g + r) * G4_TLDF + 16 * j + n] = acc[8 * hb + i][j][r];
#pragma unroll 4
            for (int t = 0; t < (GEMM_BM / 2) * 16 / 64; ++t) {
                const int c = lane + 64 * t, row = c >> 4, q = c & 15;  // 16 runs of 4 outputs per row
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(T + row * G4_TLDF + q * 4);
                const int grow = m0 + 128 * hb + row, o = 16 * s0 + 4 * q;
                if (grow < p.m && o < p.n_out) *reinterpret_cast<u32x4_t*>(part + (int64_t)grow * p.n_out + o) = v;
            }
        }
        return;
    }
    // y: fp16, eight outputs per 16-byte run
    uint16_t* T = reinterpret_cast<uint16_t*>(As) + wave * (GEMM_BM * G4_TLD);
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int o = (s0 + j) * 16 + n;
        sc[j] = o < p.n_out ? __half2float(__ushort_as_half(p.out_scale[o])) * 128.0f : 0.0f;
    }
    // lanes n and n ^ 1 hold the same four rows of neighbouring outputs: the
    // even lane writes rows 0 and 1 of the pair of outputs, the odd lane rows
    // 2 and 3, each as fp16 pairs, after trading two values across the pair
    const bool odd = (n & 1) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = sc[j] * acc[i][j][r];
            const float x0 = odd ? v[0] : v[2], x1 = odd ? v[1] : v[3];
            const float t0 = lane_pair_swap(x0), t1 = lane_pair_swap(x1);
            const int row = 16 * i + 4 * g + (odd ? 2 : 0);
            uint32_t* dst = reinterpret_cast<uint32_t*>(T + row * G4_TLD + 16 * j + (n & ~1));
            dst[0] = odd ? pack_h2(t0, v[2]) : pack_h2(v[0], t0);
            dst[G4_TLD / 2] = odd ? pack_h2(t1, v[3]) : pack_h2(v[1], t1);
        }
    // a wave reads back only its own tile, and its LDS operations run in order
#pragma unroll 4
    for (int t = 0; t < GEMM_BM * 8 / 64; ++t) {
        const int c = lane + 64 * t, row = c >> 3, part = c & 7;  // 8 runs of 8 outputs per row
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(T + row * G4_TLD + part * 8);
        const int grow = m0 + row, o = 16 * s0 + 8 * part;
        if (grow < p.m && o < p.n_out) *reinterpret_cast<u32x4_t*>(p.y + (int64_t)grow * p.n_out + o) = v;
    }
}
#undef G4_FENCE


// Split-k reduction: y[r][o] = fp16(out_scale[o] * 128 * sum_z part[z][r][o]),
// the splits added in order.  Four outputs per thread (n_out % 16 == 0).
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part,
                                                          const uint16_t* __restrict__ out_scale,
                                                          uint16_t* __restrict__ y, int m, int n_out, int zsplit) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // group of 4 outputs
    const int64_t total = (int64_t)m * n_out / 4;
    if (q >= total) return;
    const int64_t e = 4 * q;
    const int o = (int)(e % n_out);
    const int64_t plane = (int64_t)m * n_out;
    float4 v = *reinterpret_cast<const float4*>(part + e);
    for (int z = 1; z < zsplit; ++z) {
        const float4 w = *reinterpret_cast<const float4*>(part + z * plane + e);
        v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    const float a[4] = {v.x, v.y, v.z, v.w};
    uint16_t out[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float sc = __half2float(__ushort_as_half(out_scale[o + t])) * 128.0f;
        out[t] = __half_as_ushort(__float2half_rn(sc * a[t]));
    }
    *reinterpret_cast<uint2*>(y + e) = uint2{(uint32_t)out[0] | ((uint32_t)out[1] << 16),
                                           (uint32_t)out[2] | ((uint32_t)out[3] << 16)};
}

template <int K, int CB>
static hipError_t launch_gemm_k(const GemmParams& p, hipStream_t s) {
    if (p.m <= GEMM_BM_SMALL) {
        dim3 grid((p.n_strips + 15) / 16, 1, p.zsplit);
        hipLaunchKernelGGL((gemm_kernel<K, CB, GEMM_BM_SMALL>), grid, dim3(512), 0, s, p);
    } else if (p.m <= 2 * GEMM_BM_SMALL) {
        dim3 grid((p.n_strips + 15) / 16, 1, p.zsplit);
        hipLaunchKernelGGL((gemm_kernel<K, CB, 2 * GEMM_BM_SMALL>), grid, dim3(512), 0, s, p);
    } else {
        if (p.rows < p.m || p.rows % GEMM_BM != 0) return hipErrorInvalidValue;  // group-major x' required
        dim3 grid((p.n_strips + 15) / 16, p.rows / GEMM_BM, p.zsplit);
        hipLaunchKernelGGL((gemm4_kernel<K, CB>), grid, dim3(256), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.zsplit <= 1) return e;
    const int64_t groups = (int64_t)p.m * p.n_out / 4;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, p.part,
                       p.out_scale, p.y, p.m, p.n_out, p.zsplit);
    return hipGetLastError();
}

template <int CB>
static hipError_t launch_gemm_cb(int K, const GemmParams& p, hipStream_t s) {
    switch (K) {
        case 1: return launch_gemm_k<1, CB>(p, s);
        case 2: return launch_gemm_k<2, CB>(p, s);
        case 3: return launch_gemm_k<3, CB>(p, s);
        case 4: return launch_gemm_k<4, CB>(p, s);
        case 5: return launch_gemm_k<5, CB>(p, s);
        case 6: return launch_gemm_k<6, CB>(p, s);
        case 7: return launch_gemm_k<7, CB>(p, s);
        case 8: return launch_gemm_k<8, CB>(p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(int K, int cb, const GemmParams& p, hipStream_t s) {
    return cb == 0 ? launch_gemm_cb<0>(K, p, s) : launch_gemm_cb<1>(K, p, s);
}

}  // namespace exl3
