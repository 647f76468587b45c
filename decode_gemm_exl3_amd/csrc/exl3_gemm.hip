// exl3_gemm.hip - decode-matmul for larger m on the matrix cores (gfx950).
//
// The input is rotated once by a pre-pass (x'/128 in fp16, workspace).  A
// workgroup (4 waves) owns a BM x BN = 128 x 256 block of y; wave w owns all 128
// rows and outputs 64w..64w+63 (4 strips).  The input dimension is walked in
// steps of BK = 64 (4 tile columns):
//   - the x' block [128][64] is staged in LDS (loaded one step ahead into
//     registers) and read as A fragments by all four waves;
//   - each wave decodes its own weights straight into B fragments: lane (n, g)
//     decodes half row g & 1 of row n of tile column g >> 1 (8 states, halves
//     summed to fp16), so decoded weights never touch LDS and are decoded once
//     per workgroup; the trellis rows are loaded one step ahead;
//   - 8 x 4 fragments of v_mfma_f32_16x16x32_f16 per 32 inputs: 64 MFMAs per
//     wave per step.
// Within one wave the vector decode and the matrix core hardly overlap, but the
// matrix core runs one wave's MFMAs while another wave on the same SIMD
// decodes, so the kernel is sized for two workgroups per CU (at most 256
// registers per lane, 128 of them accumulators) and keeps LDS traffic to x'.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

constexpr int GM_BM = 128;
constexpr int GM_BN = 256;            // 16 strips, 64 outputs per wave
constexpr int GM_BK = 64;             // 4 tile columns
constexpr int GM_LD = GM_BK + 8;      // padded LDS row stride in halves (144 bytes)
constexpr int GM_A_HALVES = GM_BM * GM_LD;

template <int K>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmParams p) {
    __shared__ __align__(16) uint16_t As[GM_A_HALVES];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    // XCD-aware block order: consecutive workgroups go to different XCDs (round
    // robin), so hand each XCD a contiguous run of the m-major block order; its
    // L2 then keeps the x' rows of one m-block while it sweeps the outputs.
    const int nbx = gridDim.x, total = gridDim.x * gridDim.y;
    int lin = blockIdx.x + blockIdx.y * nbx;
    if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
    const int m0 = (lin / nbx) * GM_BM;
    const int s0 = (lin % nbx) * (GM_BN / 16) + 4 * wave;  // first strip of this wave
    const CbRegs cr = cb_regs();

    // ---- weights: fragment f = (strip s0 + (f & 3), tile column 2(f >> 2) + (g >> 1), half g & 1).
    // Lane offsets are fixed; strip and step go in the scalar offset.  Strips past
    // the end read as zero (never written out).
    constexpr int KDH = HalfGeom<K>::KDH;
    constexpr uint32_t TILE_B = RowGeom<K>::DW_PER_TILE * 4;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.trellis, (int64_t)p.n_strips * p.tiles_in * TILE_B);
    const int h = g & 1;
    uint32_t voff[KDH];
#pragma unroll
    for (int i = 0; i < KDH; ++i) voff[i] = (uint32_t)(g >> 1) * TILE_B + half_dword<K>(n, h, i) * 4;
    const uint32_t bsh = half_shift<K>(n, h);
    const uint32_t strip_b = (uint32_t)p.tiles_in * TILE_B;
    auto load_frag = [&](uint32_t (&d)[KDH], int f, int tc) {
        const uint32_t so = (uint32_t)(s0 + (f & 3)) * strip_b + (uint32_t)(tc + 2 * (f >> 2)) * TILE_B;
#pragma unroll
        for (int i = 0; i < KDH; ++i) d[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff[i], so, kNT);
    };

    // ---- x' staging: thread t stages half (t & 1) of row t >> 1, 64 bytes per
    // step.  Rows past m read as zero through the buffer range check.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.xr + (int64_t)m0 * p.n_in, ((int64_t)p.m - m0) * p.n_in * 2);
    const int arow = tid >> 1, acol = (tid & 1) * 32;  // in halves
    const uint32_t aoff = (uint32_t)arow * p.n_in * 2 + acol * 2;

    // trellis rows one step in flight: each fragment's registers are refilled
    // with the same fragment of the next step as soon as they are decoded
    uint32_t rows[8][KDH];
#pragma unroll
    for (int f = 0; f < 8; ++f) load_frag(rows[f], f, 0);
    u32x4_t areg[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        areg[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff, (8 * c) * 2, 0));

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int tc = 0; tc < p.tiles_in; tc += 4) {
        {
            __syncthreads();  // the previous step's A fragments have been read
#pragma unroll
            for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4_t*>(As + arow * GM_LD + acol + 8 * c) = areg[c];
#pragma unroll
            for (int c = 0; c < 4; ++c)  // next step (past the end: range check or unused)
                areg[c] = __builtin_bit_cast(u32x4_t,
                                             __builtin_amdgcn_raw_buffer_load_b128(ra, aoff, ((tc + 4) * 16 + 8 * c) * 2, 0));
            __syncthreads();
            const uint16_t* ab = As;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                // decode the 4 B fragments of these 32 inputs, refilling each slot
                // with the same fragment of the next step
                half8_t bf[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int f = 4 * kk + j;
                    uint32_t d[KDH];
                    if constexpr (HalfGeom<K>::ALIGNED) {
#pragma unroll
                        for (int i = 0; i < KDH; ++i) d[i] = rows[f][i];
                    } else {
#pragma unroll
                        for (int i = 0; i < KDH; ++i)
                            d[i] = __builtin_amdgcn_alignbit(rows[f][i + 1 < KDH ? i + 1 : i], rows[f][i], bsh);
                    }
                    load_frag(rows[f], f, tc + 4);
                    uint32_t q[8];
                    decode_half<K>(d, q, cr);
                    uint32_t o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = (uint32_t)cb_sum(q[2 * e]) | ((uint32_t)cb_sum(q[2 * e + 1]) << 16);
                    bf[j] = __builtin_bit_cast(half8_t, u32x4_t{o[0], o[1], o[2], o[3]});
                }
                // A fragments through a ring of 3: reads run two fragments ahead
                // of the 4 MFMAs that use each one
                const uint16_t* abase = ab + n * GM_LD + 32 * kk + 8 * g;
                half8_t af[3];
                af[0] = *reinterpret_cast<const half8_t*>(abase);
                af[1] = *reinterpret_cast<const half8_t*>(abase + 16 * GM_LD);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i + 2 < 8) af[(i + 2) % 3] = *reinterpret_cast<const half8_t*>(abase + (i + 2) * 16 * GM_LD);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i % 3], bf[j], acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    // D[4g + r][n] of fragment (i, j): row 16i + 4g + r, output 16 (s0 + j) + n
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int o = (s0 + j) * 16 + n;
        if (o >= p.n_out) continue;
        const float sc = __half2float(__ushort_as_half(p.out_scale[o])) * 128.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + i * 16 + 4 * g + r;
                if (row < p.m) p.y[(int64_t)row * p.n_out + o] = __half_as_ushort(__float2half_rn(sc * acc[i][j][r]));
            }
    }
}

template <int K>
static hipError_t launch_gemm_k(const GemmParams& p, hipStream_t s) {
    dim3 grid((p.n_strips + 15) / 16, (p.m + GM_BM - 1) / GM_BM);
    hipLaunchKernelGGL(gemm_kernel<K>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm(int K, const GemmParams& p, hipStream_t s) {
    switch (K) {
        case 1: return launch_gemm_k<1>(p, s);
        case 2: return launch_gemm_k<2>(p, s);
        case 3: return launch_gemm_k<3>(p, s);
        case 4: return launch_gemm_k<4>(p, s);
        case 5: return launch_gemm_k<5>(p, s);
        case 6: return launch_gemm_k<6>(p, s);
        case 7: return launch_gemm_k<7>(p, s);
        case 8: return launch_gemm_k<8>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace exl3
