// exl3_device.hpp - device building blocks shared by the EXL3 kernels (gfx950).
//
// Trellis rows.  A 16x16 tile is a cyclic stream of 256*K bits (16K uint16
// words, LSB first).  Row n of the tile holds states 16n..16n+15, whose 16-bit
// windows start at stream bits 16nK + cK (c = 0..15) and reach at most 15 bits
// into the next row; row 15 wraps to the start of the tile (tail-biting).  One
// lane owns one row: it loads ceil(K/2) dwords starting at dword floor(nK/2),
// and the one dword it still needs comes from the lane that owns row n+1 (row
// 0 for row 15) through a DPP row rotation inside its 16-lane row, so the
// tile's wrap costs nothing.
//
// Codebooks (table-free; pages: "GEMM kernel" - an index becomes a half through
// one integer multiply and either one three-input bit operation or one dp4a;
// "conclusion first" - three instructions).  Both start with
//   p = s*A + B (mod 2^32)      v_mad_u32_u16, state read from either 16-bit half
// and produce a codebook word: a dword whose two fp16 halves sum to the value.
//   codebook 0:  q = (p & M) | X                    v_and_or_b32
//   codebook 1:  h = 0x6400 + (sum of p's bytes)    v_dot4_u32_u8 = fp16 bits of 1024 + t
//                q = (h * G + C, 0 * G + 0)         v_pk_fma_f16, one rounding; high half +0
// The GEMV leaves the halves' sum to the matrix core (two k slots per weight);
// the GEMM and decode_tile form the fp16 value.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace exl3 {

constexpr uint32_t CB_A = 0xBFD3u;
constexpr uint32_t CB_B = 0x201784FFu;
constexpr uint32_t CB_M = 0x8D7F8DFFu;
constexpr uint32_t CB_X = 0x30003000u;

constexpr uint32_t CB1_A = 0xFEC5u;
constexpr uint32_t CB1_B = 0x77C40AA0u;
constexpr uint32_t CB1_ONES = 0x01010101u;  // dot4 weights: the byte sum
constexpr uint32_t CB1_H = 0x6400u;         // fp16 1024: 0x6400 + t is the fp16 of 1024 + t (t <= 1020)
constexpr uint32_t CB1_G2 = 0x1EED1EEDu;    // (G, G), G = 1773/262144
constexpr uint32_t CB1_C2 = 0x0000C930u;    // (C, +0), C = -10.375

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int K> struct RowGeom {
    static constexpr int KD = (K + 1) / 2;   // dwords a lane loads for its row
    static constexpr int NB = KD + 1;        // plus the neighbour's first dword
    static constexpr int DW_PER_TILE = 8 * K;
};

// Register-held codebook constants.  A VOP3 instruction on gfx9 reads at most
// one SGPR or literal, so the additive constants live in VGPRs and the
// multipliers and masks in SGPRs.  They are produced by opaque moves so the
// compiler cannot fold them back into literals (which would split the
// mask-and-plant into two instructions).
struct CbRegs {
    uint32_t vB, vX, sM;  // codebook 0: B, X, M; codebook 1: B', 0x6400, 0x01010101
    uint32_t vG2, vC2;    // codebook 1: (G, G) and (C, +0)
};

template <int CB>
__device__ __forceinline__ CbRegs cb_regs() {
    CbRegs r;
    uint32_t b = CB == 0 ? CB_B : CB1_B, x = CB == 0 ? CB_X : CB1_H, m = CB == 0 ? CB_M : CB1_ONES;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r.vB) : "s"(b));
    asm volatile("v_mov_b32 %0, %1" : "=v"(r.vX) : "s"(x));
    asm volatile("s_mov_b32 %0, %1" : "=s"(r.sM) : "s"(m));
    r.vG2 = CB1_G2;
    r.vC2 = CB1_C2;
    if (CB == 1) {
        uint32_t g = CB1_G2, c = CB1_C2;
        asm volatile("v_mov_b32 %0, %1" : "=v"(r.vG2) : "s"(g));
        asm volatile("v_mov_b32 %0, %1" : "=v"(r.vC2) : "s"(c));
    }
    return r;
}

// Word from p.  In C so that the compiler sees the VALU write that feeds the
// matrix core and inserts the wait states an MFMA source read requires.
template <int CB>
__device__ __forceinline__ uint32_t cb_word(uint32_t p, const CbRegs& r) {
    if constexpr (CB == 0) {
        return (p & r.sM) | r.vX;
    } else {
        typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
        const uint32_t h = __builtin_amdgcn_udot4(p, r.sM, r.vX, false);
        const h2_t v = __builtin_elementwise_fma(__builtin_bit_cast(h2_t, h), __builtin_bit_cast(h2_t, r.vG2),
                                                 __builtin_bit_cast(h2_t, r.vC2));
        return __builtin_bit_cast(uint32_t, v);
    }
}

// The multiply reads the state from either 16-bit half of a register
// (v_mad_u32_u16 with op_sel), which has no C spelling, so it is inline asm.
// Codebook word for the state held in the low 16 bits of w.
template <int CB>
__device__ __forceinline__ uint32_t cb_lo(uint32_t w, const CbRegs& r) {
    uint32_t p;
    asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(p) : "v"(w), "s"(CB == 0 ? CB_A : CB1_A), "v"(r.vB));
    return cb_word<CB>(p, r);
}

// Codebook word for the state held in the high 16 bits of w.
template <int CB>
__device__ __forceinline__ uint32_t cb_hi(uint32_t w, const CbRegs& r) {
    uint32_t p;
    asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(p) : "v"(w), "s"(CB == 0 ? CB_A : CB1_A), "v"(r.vB));
    return cb_word<CB>(p, r);
}

// fp16 sum of the two halves of a codebook word, round to nearest even.
__device__ __forceinline__ uint16_t cb_sum(uint32_t q) {
    __half lo = __ushort_as_half((unsigned short)(q & 0xFFFFu));
    __half hi = __ushort_as_half((unsigned short)(q >> 16));
    return __half_as_ushort(__hadd(lo, hi));
}

// The fp16 value of a codebook word (bit pattern).
template <int CB>
__device__ __forceinline__ uint16_t cb_value(uint32_t q) {
    if constexpr (CB == 0) return cb_sum(q);
    else return (uint16_t)q;  // the high half is +0
}

// Two values packed as one fp16x2 dword (first in the low half).
template <int CB>
__device__ __forceinline__ uint32_t cb_pack(uint32_t q0, uint32_t q1) {
    if constexpr (CB == 0) return (uint32_t)cb_sum(q0) | ((uint32_t)cb_sum(q1) << 16);
    else return (q0 & 0xFFFFu) | (q1 << 16);
}

// Dword of the lane that owns the next row of the same tile (row 15 -> row 0):
// DPP row_ror:15 inside each 16-lane row.
__device__ __forceinline__ uint32_t next_row_dword(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12F, 0xF, 0xF, false);
}

// Byte offset of row n's first loaded dword (dword floor(nK/2)) inside its tile.
template <int K>
__device__ __forceinline__ uint32_t row_offset(int n) {
    return (uint32_t)(((n * K) >> 1) * 4);
}

// Buffer resource over [base, base + bytes): loads at or past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int nrec = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFF0 ? 0x7FFFFFF0 : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

constexpr int kNT = 2;  // streaming (non-temporal) cache policy for the weight stream

// Load the lane's row: ceil(K/2) dwords at byte voff + soff of the buffer.
// voff is the per-lane offset (row_offset included), soff a wave-uniform step
// offset, so the address costs no vector instruction.
template <int K>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                         uint32_t (&b)[RowGeom<K>::NB]) {
    constexpr int KD = RowGeom<K>::KD;
    if constexpr (KD == 1) {
        b[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, kNT);
    } else if constexpr (KD == 2) {
        u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kNT));
        b[0] = v.x; b[1] = v.y;
    } else if constexpr (KD == 3) {
        typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
        u32x3_t v = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(rs, voff, soff, kNT));
        b[0] = v.x; b[1] = v.y; b[2] = v.z;
    } else {
        u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kNT));
        b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
    }
}

// Complete a loaded row: fetch the neighbour dword and, for odd K on odd rows
// (which start 16 bits into their first dword), shift the row so that state c
// always starts at bit cK of b[].
template <int K>
__device__ __forceinline__ void finish_row(int n, uint32_t (&b)[RowGeom<K>::NB]) {
    constexpr int KD = RowGeom<K>::KD;
    b[KD] = next_row_dword(b[0]);
    if constexpr (K & 1) {
        const uint32_t sh = (uint32_t)((n & 1) << 4);
#pragma unroll
        for (int k = 0; k < KD; ++k) b[k] = __builtin_amdgcn_alignbit(b[k + 1], b[k], sh);
    }
}

// Codebook words of the 16 states of a finished row: q[c] for state c.
// All offsets are compile-time constants; windows at bit 0 or 16 of a dword are
// read in place, and when K divides 16 one funnel shift serves two states.
template <int K, int CB>
__device__ __forceinline__ void decode_row(const uint32_t (&b)[RowGeom<K>::NB], uint32_t (&q)[16],
                                           const CbRegs& r) {
    constexpr int NB = RowGeom<K>::NB;
    constexpr bool pairs = (16 % K) == 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int P = c * K;
        const int dw = P >> 5;
        const int sh = P & 31;
        if (sh == 0) {
            q[c] = cb_lo<CB>(b[dw], r);
        } else if (sh == 16) {
            q[c] = cb_hi<CB>(b[dw], r);
        } else if (pairs && sh > 16) {
            // produced together with state c - 16/K (same funnel shift, high half)
        } else {
            // a window that ends inside b[dw] may take any high operand
            const uint32_t w = __builtin_amdgcn_alignbit(b[(dw + 1 < NB) ? dw + 1 : dw], b[dw],
                                                         (uint32_t)sh);
            q[c] = cb_lo<CB>(w, r);
            if (pairs && c + 16 / K < 16) q[(c + 16 / K) & 15] = cb_hi<CB>(w, r);
        }
    }
}


// ---------------------------------------------------------------------------
// Half rows, for the GEMM's matrix-core B operand (lane (n, g) holds 8
// consecutive k of output n): half row h of row n = states 16n + 8h .. +7, the
// bit window [8K(2n+h), 8K(2n+h) + 8K + 15) of the tile stream.  A lane loads
// KDH dwords starting at the dword holding the window start, each with its own
// (wrapped) offset, then shifts them so that state c starts at bit cK.
// ---------------------------------------------------------------------------
template <int K> struct HalfGeom {
    static constexpr bool ALIGNED = (8 * K) % 32 == 0;  // window starts on a dword boundary
    static constexpr int KDH = ALIGNED ? (8 * K + 15 + 31) / 32 : (24 + 8 * K + 15 + 31) / 32;
};

// Dword index (within the tile) of the i-th dword of half row h of row n, and
// the bit offset of the window inside the first dword.
template <int K>
__device__ __forceinline__ uint32_t half_dword(int n, int h, int i) {
    const int start = 8 * K * (2 * n + h);
    return (uint32_t)(((start >> 5) + i) % (8 * K));
}
template <int K>
__device__ __forceinline__ uint32_t half_shift(int n, int h) {
    return (uint32_t)((8 * K * (2 * n + h)) & 31);
}

// Codebook words of the 8 states of a normalised half row (state c at bit cK).
template <int K, int CB>
__device__ __forceinline__ void decode_half(const uint32_t (&b)[HalfGeom<K>::KDH], uint32_t (&q)[8],
                                            const CbRegs& r) {
    constexpr int NB = HalfGeom<K>::KDH;
    constexpr bool pairs = (16 % K) == 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int P = c * K;
        const int dw = P >> 5;
        const int sh = P & 31;
        if (sh == 0) {
            q[c] = cb_lo<CB>(b[dw], r);
        } else if (sh == 16) {
            q[c] = cb_hi<CB>(b[dw], r);
        } else if (pairs && sh > 16 && c - 16 / K >= 0) {
            // produced together with state c - 16/K
        } else {
            const uint32_t w = __builtin_amdgcn_alignbit(b[(dw + 1 < NB) ? dw + 1 : dw], b[dw], (uint32_t)sh);
            q[c] = cb_lo<CB>(w, r);
            if (pairs && c + 16 / K < 8) q[(c + 16 / K) & 7] = cb_hi<CB>(w, r);
        }
    }
}

}  // namespace exl3
