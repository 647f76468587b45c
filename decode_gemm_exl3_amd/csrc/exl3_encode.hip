// exl3_encode.hip - the tail-biting Viterbi encoder for 16x16 tiles (gfx950).
//
// Pages: "ExLlamaV3 inference speed: EXL3 GEMM kernel and fused Viterbi
// encoding", section "Viterbi encoding kernel": one thread block per 16x16
// block of 256 weights; a forward Viterbi pass over the trellis keeps the
// accumulated cost of every edge and takes the minimum-cost path; the
// tail-biting boundary is closed by enumerating start states so that the
// codeword's head and tail agree; kernels are instantiated per (K, codebook).
//
// Trellis: 65536 states (16-bit windows); state i+1 = (state i >> K) | (b << (16-K)).
// The predecessors of s are the 2^K states (u << K) | j with u = s & (2^(16-K) - 1),
// so one step is a minimum over blocks of 2^K consecutive states,
//     M[u] = min_j cost[(u << K) | j]        (first j on ties)
//     cost'[s] = M[s & (2^(16-K) - 1)] + (w_i - c(s))^2,
// with the subtraction, the square and the sum each rounded in fp32 (no fused
// multiply-add), so the decisions are exactly those of a plain fp32 search.
//
// Tail-biting search, two passes per tile: a free pass over the targets rotated
// by 128 fixes the 16-K overlap bits (the low bits of its state at the original
// position 0); a second pass starts in the states with those low bits and ends
// in the states whose top 16-K bits equal them, which makes the stream cyclic.
//
// Layout: 1024 threads per tile (four waves per SIMD, 128 registers each,
// which hides the LDS and barrier latency better than two waves of 256);
// thread t owns the 64 consecutive states 64t..64t+63 and their costs in
// registers (the codebook values are recomputed each step).  M (2^(16-K)
// floats) is exchanged through LDS.  The choice j of every
// (step, u) goes to the caller's workspace (one slot of 256 * 2^(16-K) bytes
// per tile in flight) and thread 0 walks the path back from it.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

// The search's decisions are defined with the square and the sum rounded
// separately: no multiply-add contraction anywhere in this file.
#pragma clang fp contract(off)

namespace exl3 {

constexpr int ENC_THREADS = 1024;
constexpr int ENC_STATES = 64;  // per thread

template <int K, int CB>
__global__ __launch_bounds__(ENC_THREADS) void encode_kernel(EncodeParams p) {
    constexpr int U = 1 << (16 - K);   // block minima per step
    constexpr int LOW = U - 1;         // overlap mask
    constexpr int BLK = 1 << K;        // states per block
    // block minima, double-buffered where LDS allows (step i writes buffer
    // i & 1, so a step needs one barrier); K = 1 has one buffer and two barriers
    constexpr int NMB = K >= 2 ? 2 : 1;
    // M is stored with four floats of padding after every 64 entries: the cost
    // update has each thread read 64 consecutive entries starting at a multiple
    // of 64, and unpadded every lane of a wave would read the same four banks
    // (a 64-way conflict on every read of every step)
    constexpr int MP = U + 4 * (U / 64);
    auto mpad = [](int u) { return u + 4 * (u >> 6); };
    __shared__ float Mbuf[NMB][MP];
    __shared__ float wt[256];
    __shared__ uint16_t path[256];
    __shared__ float red_c[ENC_THREADS / 64];
    __shared__ int red_s[ENC_THREADS / 64];
    __shared__ int shared_v;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int s0 = ENC_STATES * tid;  // first state of this thread
    uint8_t* back = p.scratch + (int64_t)blockIdx.x * p.slot_bytes;  // [256][U] choices (step 0 unused)

    // Codebook values of the thread's states, recomputed where they are used:
    // registers hold the 128 costs, and a stored copy of the values (or fp32
    // conversions the compiler would hoist out of the step loop) would spill.
    // The product of state s + 1 is that of state s plus A (every state is
    // below 2^16, so the products agree mod 2^32 with the multiply): walking a
    // thread's states costs one add each.  The base passes through an empty
    // asm statement each step so that the compiler cannot hoist the
    // recomputation.
    const CbRegs cr = cb_regs<CB>();
    constexpr uint32_t CA = CB == 0 ? CB_A : CB1_A;
    uint32_t pb = (uint32_t)s0 * CA + (CB == 0 ? CB_B : CB1_B);
    auto launder = [&]() { asm volatile("" : "+v"(pb)); };
    // (w - c(state)) in fp32 from the product of the state: the codebook's
    // fp16 value enters a v_fma_mix_f32 as -h * 1.0 + w, one rounding of the
    // exact difference, the same result as converting h and subtracting
    auto diff = [&](float w, uint32_t pk) -> float {
        const uint32_t h = cb_value<CB>(cb_word<CB>(pk, cr));
        float d;
        asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(w));
        return d;
    };
    const __amdgpu_buffer_rsrc_t rback = make_rsrc(back, p.slot_bytes);

    float cost[ENC_STATES];
    // one pass over the tile's targets starting at `rot`; v < 0: free start and
    // end, else the constrained tail-biting pass.  Returns the end state.
    auto run_pass = [&](int rot, int v) -> int {
        {
            const float w0 = wt[rot & 255];
            uint32_t pk = pb;
#pragma unroll
            for (int k = 0; k < ENC_STATES; ++k, pk += CA) {
                const float d = diff(w0, pk);
                const float e = d * d;
                cost[k] = (v < 0 || ((s0 + k) & LOW) == v) ? e : INFINITY;
                if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bounded live values
            }
        }
        for (int i = 1; i < 256; ++i) {
            launder();
            float* M = Mbuf[i % NMB];
            // ---- block minima of the previous costs (first minimum on ties)
            if constexpr (BLK <= ENC_STATES) {
                // the thread's NBLK blocks are consecutive u: their choices are
                // NBLK consecutive bytes, stored at once
                constexpr int NBLK = ENC_STATES / BLK;
                uint32_t pk[(NBLK + 3) / 4];
#pragma unroll
                for (int q = 0; q < (NBLK + 3) / 4; ++q) pk[q] = 0;
#pragma unroll
                for (int b = 0; b < NBLK; ++b) {
                    float best = cost[b * BLK];
                    int bj = 0;
#pragma unroll
                    for (int j = 1; j < BLK; ++j)
                        if (cost[b * BLK + j] < best) { best = cost[b * BLK + j]; bj = j; }
                    M[mpad((s0 >> K) + b)] = best;
                    pk[b >> 2] |= (uint32_t)bj << (8 * (b & 3));
                    // one block at a time: interleaving the independent chains
                    // would hold one comparison mask per element (a tree of
                    // minima and a scan for the first index measured slower)
                    if ((b & 1) == 1 || BLK >= 16) __builtin_amdgcn_sched_barrier(0);
                }
                const uint32_t off = (uint32_t)(i * U + (s0 >> K));
                if constexpr (NBLK == 64) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]},
                                                               rback, off + 16 * q, 0u, 0);
                } else if constexpr (NBLK == 32) {
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pk[0], pk[1], pk[2], pk[3]}, rback, off, 0u, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pk[4], pk[5], pk[6], pk[7]}, rback, off + 16, 0u, 0);
                } else if constexpr (NBLK == 16) {
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pk[0], pk[1], pk[2], pk[3]}, rback, off, 0u, 0);
                } else if constexpr (NBLK == 8) {
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pk[0], pk[1]}, rback, off, 0u, 0);
                } else if constexpr (NBLK == 4) {
                    __builtin_amdgcn_raw_buffer_store_b32(pk[0], rback, off, 0u, 0);
                } else if constexpr (NBLK == 2) {
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pk[0], rback, off, 0u, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)pk[0], rback, off, 0u, 0);
                }
            } else {
                // a block spans 2^K / 64 neighbouring lanes
                float best = cost[0];
                int bj = 0;
#pragma unroll
                for (int j = 1; j < ENC_STATES; ++j) {
                    if (cost[j] < best) { best = cost[j]; bj = j; }
                    if ((j & 15) == 15) __builtin_amdgcn_sched_barrier(0);
                }
                bj += ENC_STATES * (tid & ((BLK / ENC_STATES) - 1));
#pragma unroll
                for (int x = 1; x < BLK / ENC_STATES; x <<= 1) {
                    const float ob = __shfl_xor(best, x);
                    const int oj = __shfl_xor(bj, x);
                    if (ob < best || (ob == best && oj < bj)) { best = ob; bj = oj; }
                }
                if ((tid & ((BLK / ENC_STATES) - 1)) == 0) {
                    const int u = s0 >> K;
                    M[mpad(u)] = best;
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)bj, rback, (uint32_t)(i * U + u), 0u, 0);
                }
            }
            __syncthreads();
            // ---- new costs: M of each state's predecessor block plus its error
            const float wi = wt[(i + rot) & 255];
            const int u0 = s0 & LOW;  // the thread's 64 states map to u0 .. u0 + 63 (one padded row)
            const float* Mrow = M + mpad(u0);
            uint32_t pk = pb;
#pragma unroll
            for (int k = 0; k < ENC_STATES; k += 4) {
                const float4 m4 = *reinterpret_cast<const float4*>(&Mrow[k]);
                const float mk[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e, pk += CA) {
                    const float d = diff(wi, pk);
                    cost[k + e] = mk[e] + d * d;
                }
                // four states at a time: the scheduler may not compute all 64
                // codebook values ahead of their use
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (NMB == 1) __syncthreads();  // M is rewritten by the next step
        }
        // ---- end state: the lowest-cost state (lowest index on ties), among
        // the states whose top 16-K bits are v for the constrained pass
        float best = INFINITY;
        int bs = 0x7FFFFFFF;
#pragma unroll
        for (int k = 0; k < ENC_STATES; ++k) {
            const int s = s0 + k;
            const bool ok = v < 0 || (s >> K) == v;
            if (ok && (cost[k] < best || (cost[k] == best && s < bs))) { best = cost[k]; bs = s; }
            if ((k & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int x = 32; x >= 1; x >>= 1) {
            const float ob = __shfl_xor(best, x);
            const int os = __shfl_xor(bs, x);
            if (ob < best || (ob == best && os < bs)) { best = ob; bs = os; }
        }
        if (lane == 0) { red_c[wave] = best; red_s[wave] = bs; }
        __syncthreads();
        if (tid == 0) {
            float b = red_c[0];
            int sb = red_s[0];
            for (int w = 1; w < ENC_THREADS / 64; ++w)
                if (red_c[w] < b || (red_c[w] == b && red_s[w] < sb)) { b = red_c[w]; sb = red_s[w]; }
            red_c[0] = b;
            red_s[0] = sb;
        }
        __syncthreads();
        return red_s[0];
    };
    // thread 0: state at step `stop` of the path that ends in `end`.  The
    // choices were stored by other waves of this workgroup; the loads are
    // workgroup-coherent (sc0), so the vector L1 cannot serve a stale line.
    auto walk_back = [&](int end, int stop, bool store) -> int {
        int s = end;
        if (store) path[255] = (uint16_t)s;
        for (int i = 255; i > stop; --i) {
            const int u = s & LOW;
            const int j = __builtin_amdgcn_raw_buffer_load_b8(rback, (uint32_t)(i * U + u), 0u, 1);
            s = (u << K) | j;
            if (store) path[i - 1] = (uint16_t)s;
        }
        return s;
    };

    for (int64_t tile = blockIdx.x; tile < p.n_tiles; tile += gridDim.x) {
        if (tid < 256) wt[tid] = p.w[tile * 256 + tid];
        __syncthreads();
        // pass 1: free search over the targets rotated by 128
        const int end1 = run_pass(128, -1);
        if (tid == 0) shared_v = walk_back(end1, 128, false) & LOW;  // the state at the original position 0
        __syncthreads();
        const int v = shared_v;
        // pass 2: the tail-biting search with those overlap bits
        const int end2 = run_pass(0, v);
        const float c2 = red_c[0];
        if (tid == 0) walk_back(end2, 0, true);
        __syncthreads();
        // pack: stream bits [iK, iK + K) are the low K bits of state i
        if (tid < 16 * K) {
            uint32_t word = 0;
            for (int bit = 0; bit < 16; ++bit) {
                const int pos = 16 * tid + bit;
                word |= (uint32_t)((path[pos / K] >> (pos % K)) & 1) << bit;
            }
            p.words[tile * 16 * K + tid] = (uint16_t)word;
        }
        if (tid == 0 && p.costs) p.costs[tile] = c2;
        __syncthreads();  // LDS (targets, path) is reused by the next tile
    }
}

template <int K, int CB>
static hipError_t launch_encode_k(const EncodeParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((encode_kernel<K, CB>), dim3(grid), dim3(ENC_THREADS), 0, s, p);
    return hipGetLastError();
}

template <int CB>
static hipError_t launch_encode_cb(int K, const EncodeParams& p, int grid, hipStream_t s) {
    switch (K) {
        case 1: return launch_encode_k<1, CB>(p, grid, s);
        case 2: return launch_encode_k<2, CB>(p, grid, s);
        case 3: return launch_encode_k<3, CB>(p, grid, s);
        case 4: return launch_encode_k<4, CB>(p, grid, s);
        case 5: return launch_encode_k<5, CB>(p, grid, s);
        case 6: return launch_encode_k<6, CB>(p, grid, s);
        case 7: return launch_encode_k<7, CB>(p, grid, s);
        case 8: return launch_encode_k<8, CB>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_encode(int K, int cb, const EncodeParams& p, int grid, hipStream_t s) {
    return cb == 0 ? launch_encode_cb<0>(K, p, grid, s) : launch_encode_cb<1>(K, p, grid, s);
}

}  // namespace exl3
