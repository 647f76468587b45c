// exl3_internal.hpp - host/device interface between the C ABI and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exl3 {

constexpr int GEMV_LDS_BUDGET = 160 * 1024;  // bytes of LDS per GEMV workgroup (one per CU)

constexpr int GEMV_MAX_PROJ = 4;  // projections sharing one input in one GEMV launch

// One GEMV launch: up to GEMV_MAX_PROJ projections that share x, sign, n_in
// and the bit width.  Their 16-row strips are numbered one after the other
// (projection 0 first); strip_end[i] is the number of strips in projections
// 0..i, and entries past the last projection hold INT32_MAX.
struct GemvParams {
    const uint16_t* x;
    const uint16_t* sign;
    const uint16_t* xr;  // x'/128 in fp16 [m][n_in] from the rotation pre-pass, or null: rotate in the kernel
    const uint16_t* trellis[GEMV_MAX_PROJ];
    const uint16_t* out_scale[GEMV_MAX_PROJ];
    uint16_t* y[GEMV_MAX_PROJ];
    int n_out[GEMV_MAX_PROJ];
    int strip_end[GEMV_MAX_PROJ];
    int n_proj;
    int m, n_in;
    int tiles_in, n_strips;  // n_strips: all projections together
    int kc;             // tile columns per input chunk (x' of a chunk sits in LDS)
    int n_kchunks;      // input chunks
    int waves;          // waves per workgroup
    int nsw;            // steps (4 tile columns each) per wave per strip, a multiple of pf
    int pf;             // steps in flight per wave
    int grid;           // persistent workgroups; workgroup b owns strips b, b + grid, ...
};

// LDS of a GEMV workgroup: x' rows, a zero block, per-wave partial sums of its nj strips.
constexpr int GEMV_ROW_PAD = 4;  // dwords after each LDS row of x' (bank spread)
__host__ __device__ inline size_t gemv_lds_bytes(int m, int waves, int nsw, int pf, int nj) {
    return ((size_t)m * ((size_t)waves * nsw * 64 + GEMV_ROW_PAD) + (size_t)pf * 64 + (size_t)nj * waves * m * 16) * 4;
}

struct GemmParams {
    const uint16_t* xr;     // rotated input x'/128 in fp16: [m][n_in], or [n_in / 8][rows][8] when rows > 0
    int rows;               // rows of the group-major layout (m rounded up to the row block), or 0
    const uint16_t* trellis;
    const uint16_t* out_scale;
    uint16_t* y;
    int m, n_in, n_out;
    int tiles_in, n_strips;
    // split-k: zsplit workgroups share an output block, each over kz tile
    // columns of the input; with zsplit > 1 they write fp32 partial sums
    // part[z][m][n_out] and a reduction forms y
    int zsplit, kz;
    float* part;
};

constexpr int GEMM_BM = 256, GEMM_BN = 256;  // output block of one GEMM workgroup
constexpr int GEMM_BM_SMALL = 64;            // rows per block when m <= 64
constexpr int GEMM_MAX_SPLIT = 16;
constexpr int GEMM_SIZING_CUS = 256;         // CU count the workspace is sized for (MI355X)

// Split-k plan: split the input dimension while the output blocks alone would
// leave CUs idle (a medium m gives few blocks), in multiples of 4 tile columns.
// One GEMM workgroup fills a CU, so the time goes as (rounds of workgroups) x
// (steps per split + the set-up and write-out of a workgroup, about 3 steps);
// the split count minimises that, the smallest on ties (fewer partial sums).
inline void plan_gemm_split(int m, int n_out, int tiles_in, int cus, int* zsplit, int* kz) {
    const int blocks = ((n_out / 16 + 15) / 16) * ((m + GEMM_BM - 1) / GEMM_BM);
    const int steps = tiles_in / 4 > 0 ? tiles_in / 4 : 1;
    int best_z = 1;
    if (blocks < cus) {
        long best = -1;
        for (int z = 1; z <= GEMM_MAX_SPLIT && z <= steps; ++z) {
            const int kstep = (steps + z - 1) / z;
            const int zz = (steps + kstep - 1) / kstep;  // splits actually used
            const long rounds = ((long)blocks * zz + cus - 1) / cus;
            const long t = rounds * (kstep + 3);
            if (best < 0 || t < best) { best = t; best_z = zz; }
        }
    }
    const int kstep = (steps + best_z - 1) / best_z;
    *kz = 4 * kstep;
    *zsplit = (steps + kstep - 1) / kstep;
}

// The encoder: targets fp32 [n_tiles][256] (trellis order) -> words [n_tiles][16K]
// and the cost of each tile; scratch holds one slot of slot_bytes per workgroup.
struct EncodeParams {
    const float* w;
    int64_t n_tiles;
    uint16_t* words;
    float* costs;  // may be null
    uint8_t* scratch;
    int64_t slot_bytes;
};
inline int64_t encode_slot_bytes(int K) { return (int64_t)256 << (16 - K); }
hipError_t launch_encode(int K, int cb, const EncodeParams& p, int grid, hipStream_t s);

// cb selects the codebook: 0 (multiply, mask-and-plant, half sum) or 1 (byte sum)
hipError_t launch_decode(int K, int cb, const uint16_t* words, int64_t n_tiles, uint16_t* out, hipStream_t s);
// rows == 0: row-major xr[m][n_in]; rows > 0: xr[n_in / 8][rows][8], rows m.. zero
hipError_t launch_rotate(const uint16_t* x, const uint16_t* sign, int m, int n_in, uint16_t* xr,
                         hipStream_t s, int rows = 0);
hipError_t launch_gemv(int K, int cb, const GemvParams& p, hipStream_t s);
hipError_t launch_gemm(int K, int cb, const GemmParams& p, hipStream_t s);

}  // namespace exl3
