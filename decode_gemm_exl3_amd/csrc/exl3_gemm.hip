// exl3_gemm.hip - decode-matmul for larger m on the matrix cores (gfx950).
//
// The input is rotated once by a pre-pass (x'/128 in fp16, workspace).  Each
// workgroup owns a BM x BN block of y and walks the input dimension in steps of
// 64: it stages the x' block in LDS, decodes the 4 strips x 4 tiles of weights
// it needs into LDS as fp16 (halves summed), and runs v_mfma_f32_16x16x32_f16.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

constexpr int GM_BM = 64;
constexpr int GM_BN = 64;             // 4 strips
constexpr int GM_BK = 64;             // 4 tile columns
constexpr int GM_LDA = GM_BK + 8;     // padded row stride in halves

template <int K>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
    __shared__ __align__(16) uint16_t As[GM_BM * GM_LDA];
    __shared__ __align__(16) uint16_t Bs[GM_BN * GM_LDA];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.y * GM_BM;
    const int s0 = blockIdx.x * (GM_BN / 16);
    const int wm = wave >> 1, wn = wave & 1;
    const CbRegs cr = cb_regs();

    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int strip = s0 + wave;  // strip this wave decodes (past the end: reads zeros)
    constexpr int64_t TILE_B = RowGeom<K>::DW_PER_TILE * 4;
    const int64_t strip_off = (int64_t)strip * p.tiles_in * TILE_B;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const char*>(p.trellis) + strip_off,
                                                (int64_t)p.n_strips * p.tiles_in * TILE_B - strip_off);
    for (int tc = 0; tc < p.tiles_in; tc += 4) {
        // stage x' rows m0..m0+63, inputs 16tc..16tc+63
        for (int e = tid; e < GM_BM * (GM_BK / 8); e += 256) {
            const int r = e / (GM_BK / 8), cc = (e % (GM_BK / 8)) * 8;
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (m0 + r < p.m)
                v = *reinterpret_cast<const u32x4_t*>(p.xr + (int64_t)(m0 + r) * p.n_in + tc * 16 + cc);
            *reinterpret_cast<u32x4_t*>(As + r * GM_LDA + cc) = v;
        }
        // decode strip `wave`, tile column tc + g, row n
        uint32_t b[RowGeom<K>::NB];
        load_row<K>(rs, (uint32_t)((tc + g) * (RowGeom<K>::DW_PER_TILE * 4)) + row_offset<K>(n), 0u, b);
        finish_row<K>(n, b);
        uint32_t q[16];
        decode_row<K>(b, q, cr);
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (uint32_t)cb_sum(q[2 * j]) | ((uint32_t)cb_sum(q[2 * j + 1]) << 16);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(Bs + (wave * 16 + n) * GM_LDA + g * 16);
        dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
        dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GM_BK; kk += 32) {
            half8_t af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const half8_t*>(As + (wm * 32 + i * 16 + n) * GM_LDA + kk + 8 * g);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *reinterpret_cast<const half8_t*>(Bs + (wn * 32 + j * 16 + n) * GM_LDA + kk + 8 * g);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // D[4g + r][n] of fragment (i, j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int o = (s0 * 16) + wn * 32 + j * 16 + n;
            if (o >= p.n_out) continue;
            const float sc = __half2float(__ushort_as_half(p.out_scale[o])) * 128.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 32 + i * 16 + 4 * g + r;
                if (row < p.m) p.y[(int64_t)row * p.n_out + o] = __half_as_ushort(__float2half_rn(sc * acc[i][j][r]));
            }
        }
}

template <int K>
static hipError_t launch_gemm_k(const GemmParams& p, hipStream_t s) {
    dim3 grid((p.n_strips + 3) / 4, (p.m + GM_BM - 1) / GM_BM);
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
