// exl3_api.hip - the C ABI: argument checks, workspace layout, dispatch.
#include <atomic>
#include <climits>
#include <cstdlib>
#include <mutex>

#include "../../include/exl3.h"
#include "exl3_internal.hpp"

// Scratch of exl3_linear_noalloc: one array per GPU, in the library's device
// code, held from the library's load until the process ends.  In host code its
// name is a stand-in, not a device address: host code uses only the per-device
// address that hipGetSymbolAddress returns (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[EXL3_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Integer from the environment, for the tuning overrides (EXL3_GEMV_*, EXL3_GEMM_SPLIT).
int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Device address of `scratch` on the current device, looked up once per device
// with that device current, or null if the lookup fails.
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

void* noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        (void)hipGetLastError();  // the failed lookup must not surface at an unrelated later call
        return nullptr;
    }
    g_scratch[dev].store(ptr, std::memory_order_release);
    return ptr;
}

// Most rows exl3_linear hands to the GEMV.
constexpr int GEMV_LINEAR_MAX_M = 14;

// Largest rotated GEMM input: it is read through one buffer resource (at most
// 2^31 - 16 bytes) with 32-bit offsets.
constexpr int64_t GEMM_MAX_ROT_BYTES = ((int64_t)1 << 31) - ((int64_t)1 << 20);

// exl3_linear's choice of path: the GEMV while m <= 12 and m * n_in <= 2^17,
// or m <= 14 and m * n_in <= 2^16.
bool linear_uses_gemv(int32_t m, int32_t n_in) {
    const int64_t mn = (int64_t)m * n_in;
    return (m <= 12 && mn <= ((int64_t)1 << 17)) || (m <= GEMV_LINEAR_MAX_M && mn <= ((int64_t)1 << 16));
}


// Workspace needs.  Nothing in the workspace survives between calls, so each
// call lays out only what it uses from offset 0:
//   gemv: nothing required (one kernel, partial sums stay in LDS); given
//         m * n_in * 2 bytes it may rotate its input into them once (the
//         pre-pass), which the GEMM sizing below, the rotated input of max_m
//         rows, always covers;
int64_t gemv_ws_bytes(int n_out, int m) { (void)n_out; (void)m; return 0; }
//   gemm: the rotated input in fp16, then for a split input dimension the
//         fp32 partial sums [zsplit][m][n_out].  The rotated input is
//         row-major [m][n_in] for m <= 128; for the 256-row blocks it is
//         group-major [n_in / 8][rows][8] over m rounded up to whole blocks
//         (the padding rows zero).
bool gemm_group_major(int m) { return m > 2 * exl3::GEMM_BM_SMALL; }
int64_t gemm_rows(int m) {
    return gemm_group_major(m) ? ((int64_t)m + exl3::GEMM_BM - 1) / exl3::GEMM_BM * exl3::GEMM_BM : (int64_t)m;
}
int64_t gemm_rot_bytes(int n_in, int m) { return align256(gemm_rows(m) * n_in * 2); }
int64_t gemm_ws_bytes(int n_in, int n_out, int m, int cus) {
    int z = 1, kz = 0;
    exl3::plan_gemm_split(m, n_out, n_in / 16, cus, &z, &kz);
    return gemm_rot_bytes(n_in, m) + (z > 1 ? align256((int64_t)z * m * n_out * 4) : 0);
}
int64_t ws_total(int n_in, int n_out, int max_m) {
    int64_t best = gemv_ws_bytes(n_out, max_m < EXL3_GEMV_MAX_M ? max_m : EXL3_GEMV_MAX_M);
    // the split depends on m through the number of 256-row blocks: the largest
    // m of each block count needs the most; once a block count does not split,
    // no larger one does (more blocks make splitting less useful), and the
    // rotated input of max_m rows is all
    for (int64_t b = 1; b * exl3::GEMM_BM < (int64_t)max_m + exl3::GEMM_BM; ++b) {
        const int m = (int)(b * exl3::GEMM_BM < max_m ? b * exl3::GEMM_BM : max_m);
        const int64_t need = gemm_ws_bytes(n_in, n_out, m, exl3::GEMM_SIZING_CUS);
        if (need > best) best = need;
        int z = 1, kz = 0;
        exl3::plan_gemm_split(m, n_out, n_in / 16, exl3::GEMM_SIZING_CUS, &z, &kz);
        if (z == 1) {
            const int64_t all = gemm_rot_bytes(n_in, max_m);
            return all > best ? all : best;
        }
    }
    return best;
}

// GEMV launch plan.  Persistent workgroups own strips round-robin.  The input
// dimension is cut into as few chunks as the LDS budget allows (x' of a chunk
// lives in LDS).  Within a strip, W waves share the steps (4 tile columns
// each); nsw steps per wave, pf of them in flight (nsw % pf == 0).
//
// The shape of the launch comes from a sweep on MI355X over workgroups per CU
// (1, 2), W (4 .. 16) and pf (2, 4, 8) on the Llama 8B and 70B projections at
// m = 1 and K = 2, 4:
//   - two workgroups of 8 waves per CU beat one of 16 by 5-10 % wherever the
//     strips give each workgroup at least one and both fit in LDS (one
//     workgroup's rotation and final sums overlap the other's stream);
//   - with one workgroup per CU, 16 waves win once a workgroup walks 512 or
//     more steps, 8 waves below that;
//   - pf = 4 is best or within noise of it everywhere (pf = 2 starves the
//     loads, pf = 8 pads short strips).
// Other shapes (m > 1 with long inputs, chunked inputs) fall back to the
// search that wastes the fewest padded steps.
bool plan_chunks(exl3::GemvParams* p, int grid, int nk, int w, int pf, size_t lds_cap) {
    int kc = (p->tiles_in + nk - 1) / nk;
    kc = (kc + 7) & ~7;
    const int steps = (kc + 3) / 4;
    int nsw = (steps + w - 1) / w;
    nsw = (nsw + pf - 1) / pf * pf;
    const int nj = (p->n_strips + grid - 1) / grid;
    if (exl3::gemv_lds_bytes(p->m, w, nsw, pf, nj) > lds_cap) return false;
    p->kc = kc;
    p->n_kchunks = (p->tiles_in + kc - 1) / kc;
    p->waves = w;
    p->nsw = nsw;
    p->pf = pf;
    p->grid = grid;
    return true;
}

bool plan_gemv(exl3::GemvParams* p) {
    static const int nk_force = env_int("EXL3_GEMV_KCHUNKS", 0);
    static const int grid_force = env_int("EXL3_GEMV_GRID_PER_CU", 0);
    static const int pf_force = env_int("EXL3_GEMV_PF", 0);
    static const int w_force = env_int("EXL3_GEMV_WAVES", 0);
    const int cus = cu_count();
    const size_t budget = (size_t)exl3::GEMV_LDS_BUDGET;
    if (nk_force == 0 && grid_force == 0 && pf_force == 0 && w_force == 0) {
        if (p->n_strips >= 2 * cus && plan_chunks(p, 2 * cus, 1, 8, 4, budget / 2)) return true;
        const int grid = p->n_strips < cus ? p->n_strips : cus;
        const int64_t wg_steps = (int64_t)((p->n_strips + grid - 1) / grid) * ((p->tiles_in + 3) / 4);
        if (plan_chunks(p, grid, 1, wg_steps >= 512 ? 16 : 8, 4, budget)) return true;
    }
    int grid = cus * (grid_force > 0 ? grid_force : 1);
    if (grid > p->n_strips) grid = p->n_strips;
    const int nj = (p->n_strips + grid - 1) / grid;
    for (int nk = nk_force > 0 ? nk_force : 1; nk <= p->tiles_in / 8; ++nk) {
        int kc = (p->tiles_in + nk - 1) / nk;
        kc = (kc + 7) & ~7;
        const int steps = (kc + 3) / 4;
        double best = 1e30;
        int bw = 0, bp = 0;
        for (int pf : {4, 8, 2}) {
            if (pf_force > 0 && pf != pf_force) continue;
            for (int w = 16; w >= 4; --w) {
                if (w_force > 0 && w != w_force) continue;
                int nsw = (steps + w - 1) / w;
                nsw = (nsw + pf - 1) / pf * pf;
                const double penalty = pf == 4 ? 1.0 : (pf == 8 ? 1.03 : 1.2);
                const double cost = (double)w * nsw * penalty + 0.01 * (16 - w);
                if (exl3::gemv_lds_bytes(p->m, w, nsw, pf, nj) > budget) continue;
                if (cost < best) { best = cost; bw = w; bp = pf; }
            }
        }
        if (bw > 0 && plan_chunks(p, grid, nk, bw, bp, budget)) return true;
        if (nk_force > 0) return false;
    }
    return false;
}

// Whether a GEMV rotates its input once in a pre-pass (into the workspace)
// rather than in every workgroup.  Each workgroup's rotation costs vector
// issue in proportion to m * n_in; the pre-pass costs one more launch and a
// copy of the rotated rows from L2 into every workgroup's LDS.  Measured on
// MI355X over the 8B and 70B projections at m = 1..16 (us, in-kernel ->
// pre-pass):
//   - m = 1: the pre-pass loses up to 2 us everywhere (the extra launch);
//   - n_in = 4096: it loses at m <= 13 (m = 2, 8, 12: 18.5 -> 20.4,
//     24.3 -> 24.8, 21.0 -> 21.5 on 4096 -> 28672 and 4096 -> 14336) and wins
//     from m = 14 (22.3 -> 22.1, and 32.0 -> 28.4 at m = 16), where the plan
//     drops to 4 waves per workgroup and chunks the input;
//   - n_in = 8192 from m = 4 (16.1 -> 15.9, 20.4 -> 18.9 at m = 8, 32.0 ->
//     28.2 at m = 16 on 8192 -> 8192) and n_in >= 14336 from m = 2 (equal at
//     m = 2, 28.1 -> 23.1 at m = 8, 44.6 -> 36.5 at m = 16 on 14336 -> 4096;
//     57.9 -> 51.8 at m = 4 on 28672 -> 8192): m * n_in >= 28672.
bool gemv_prerotate(int m, int n_in) {
    static const int force = env_int("EXL3_GEMV_PREROT", -1);
    if (force >= 0) return force > 0;
    return m >= 2 && (m >= 14 || (n_in >= 8192 && (int64_t)m * n_in >= 28672));
}

// The bits argument: K in the low byte, the codebook flag above it.
int k_of(int32_t bits) { return bits & 0xFF; }
int cb_of(int32_t bits) { return (bits & EXL3_CODEBOOK_BYTE_SUM) ? 1 : 0; }
bool bad_bits(int32_t bits) {
    return k_of(bits) < 1 || k_of(bits) > 8 || (bits & ~(0xFF | EXL3_CODEBOOK_BYTE_SUM)) != 0;
}

bool bad_shape(int32_t n_in, int32_t n_out, int32_t bits) {
    return n_in <= 0 || n_out <= 0 || (n_in % 128) != 0 || (n_out % 16) != 0 || bad_bits(bits);
}

// Every tensor is read or written in 16-byte pieces somewhere on the path.
bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; }

int common_checks(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
                  const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits, uint16_t* y,
                  void* workspace, size_t workspace_bytes, int64_t need) {
    if (m < 0 || bad_shape(n_in, n_out, bits)) return EXL3_EINVAL;
    if (m == 0) return EXL3_OK;
    if (!x || !trellis || !sign || !out_scale || !y) return EXL3_EINVAL;
    if (misaligned(x) || misaligned(trellis) || misaligned(sign) || misaligned(out_scale) || misaligned(y) ||
        misaligned(workspace))
        return EXL3_EINVAL;
    if ((const void*)x == (const void*)y) return EXL3_EINVAL;
    if (need > 0 && (!workspace || (int64_t)workspace_bytes < need)) return EXL3_EWORKSPACE;
    // weights are read through 32-bit buffer offsets
    if ((int64_t)n_in * n_out * k_of(bits) / 8 >= ((int64_t)1 << 31) - ((int64_t)1 << 20)) return EXL3_EUNSUPPORTED;
    return 1;  // proceed
}

}  // namespace

extern "C" {

int exl3_pack_info(int32_t n_in, int32_t n_out, int32_t bits, int32_t max_m, exl3_pack_info_t* out) {
    if (!out || max_m < 1 || bad_shape(n_in, n_out, bits)) return EXL3_EINVAL;
    out->n_in = n_in;
    out->n_out = n_out;
    out->bits = bits;
    out->max_m = max_m;
    out->tiles_in = n_in / 16;
    out->tiles_out = n_out / 16;
    out->words_per_tile = 16 * k_of(bits);
    out->reserved = 0;
    out->trellis_words = (int64_t)out->tiles_in * out->tiles_out * out->words_per_tile;
    out->trellis_bytes = (int64_t)n_in * n_out * k_of(bits) / 8;
    out->workspace_bytes = ws_total(n_in, n_out, max_m);
    return EXL3_OK;
}

int exl3_decode_tile(const uint16_t* words, int32_t bits, int64_t n_tiles, uint16_t* out, void* stream) {
    if (bad_bits(bits) || n_tiles < 0) return EXL3_EINVAL;
    if (n_tiles == 0) return EXL3_OK;
    if (!words || !out) return EXL3_EINVAL;
    if (misaligned(words) || misaligned(out)) return EXL3_EINVAL;
    if (n_tiles > (int64_t)0xFFFFFFFF * 16) return EXL3_EUNSUPPORTED;
    hipError_t e = exl3::launch_decode(k_of(bits), cb_of(bits), words, n_tiles, out, (hipStream_t)stream);
    return e == hipSuccess ? EXL3_OK : EXL3_EHIP;
}

int exl3_gemv_multi(const uint16_t* x, int32_t m, const uint16_t* sign, int32_t n_in, int32_t bits,
                    const exl3_proj_t* proj, int32_t n_proj, void* workspace, size_t workspace_bytes,
                    void* stream) {
    if (m < 0 || m > EXL3_GEMV_MAX_M || bad_bits(bits) || n_in <= 0 || (n_in % 128) != 0) return EXL3_EINVAL;
    if (!proj || n_proj < 1 || n_proj > EXL3_GEMV_MAX_PROJ) return EXL3_EINVAL;
    for (int i = 0; i < n_proj; ++i) {
        const int32_t n_out = proj[i].n_out;
        if (n_out <= 0 || (n_out % 16) != 0) return EXL3_EINVAL;
    }
    if (m == 0) return EXL3_OK;
    if (!x || !sign) return EXL3_EINVAL;
    if (misaligned(x) || misaligned(sign) || misaligned(workspace)) return EXL3_EINVAL;
    int64_t strips = 0;
    for (int i = 0; i < n_proj; ++i) {
        const exl3_proj_t& q = proj[i];
        if (!q.trellis || !q.out_scale || !q.y) return EXL3_EINVAL;
        if (misaligned(q.trellis) || misaligned(q.out_scale) || misaligned(q.y)) return EXL3_EINVAL;
        if ((const void*)q.y == (const void*)x) return EXL3_EINVAL;
        for (int j = 0; j < i; ++j)
            if (proj[j].y == q.y) return EXL3_EINVAL;
        // weights are read through 32-bit buffer offsets
        if ((int64_t)n_in * q.n_out * k_of(bits) / 8 >= ((int64_t)1 << 31) - ((int64_t)1 << 20)) return EXL3_EUNSUPPORTED;
        strips += q.n_out / 16;
    }
    if (strips > ((int64_t)1 << 30)) return EXL3_EUNSUPPORTED;
    exl3::GemvParams p;
    p.x = x;
    p.sign = sign;
    int end = 0;
    for (int i = 0; i < exl3::GEMV_MAX_PROJ; ++i) {
        const bool used = i < n_proj;
        p.trellis[i] = used ? proj[i].trellis : nullptr;
        p.out_scale[i] = used ? proj[i].out_scale : nullptr;
        p.y[i] = used ? proj[i].y : nullptr;
        p.n_out[i] = used ? proj[i].n_out : 0;
        end += used ? proj[i].n_out / 16 : 0;
        p.strip_end[i] = i < n_proj - 1 ? end : INT32_MAX;
    }
    p.n_proj = n_proj;
    p.m = m;
    p.n_in = n_in;
    p.tiles_in = n_in / 16;
    p.n_strips = (int)strips;
    p.xr = nullptr;
    if (!plan_gemv(&p)) return EXL3_EUNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    if (gemv_prerotate(m, n_in) && workspace && (int64_t)workspace_bytes >= gemm_rot_bytes(n_in, m)) {
        uint16_t* xr = static_cast<uint16_t*>(workspace);
        if (exl3::launch_rotate(x, sign, m, n_in, xr, s) != hipSuccess) return EXL3_EHIP;
        p.xr = xr;
    }
    hipError_t e = exl3::launch_gemv(k_of(bits), cb_of(bits), p, s);
    return e == hipSuccess ? EXL3_OK : EXL3_EHIP;
}

int exl3_gemv(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
              const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits, uint16_t* y,
              void* workspace, size_t workspace_bytes, void* stream) {
    if (m > EXL3_GEMV_MAX_M) return EXL3_EINVAL;
    const int mm = m > 0 ? m : 1;
    int rc = common_checks(x, m, trellis, sign, out_scale, n_in, n_out, bits, y, workspace, workspace_bytes,
                           gemv_ws_bytes(n_out, mm));
    if (rc <= 0) return rc;
    exl3_proj_t one;
    one.trellis = trellis;
    one.out_scale = out_scale;
    one.y = y;
    one.n_out = n_out;
    one.reserved = 0;
    return exl3_gemv_multi(x, m, sign, n_in, bits, &one, 1, workspace, workspace_bytes, stream);
}

int exl3_gemm(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
              const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits, uint16_t* y,
              void* workspace, size_t workspace_bytes, void* stream) {
    int rc = common_checks(x, m, trellis, sign, out_scale, n_in, n_out, bits, y, workspace, workspace_bytes,
                           gemm_rot_bytes(n_in, m > 0 ? m : 1));
    if (rc <= 0) return rc;
    if ((int64_t)m > (int64_t)65535 * 64) return EXL3_EUNSUPPORTED;
    // the rotated input is read through one buffer resource with 32-bit offsets
    if (gemm_rot_bytes(n_in, m) >= GEMM_MAX_ROT_BYTES) return EXL3_EUNSUPPORTED;
    uint16_t* xr = static_cast<uint16_t*>(workspace);
    // split the input dimension while the output blocks leave CUs idle, as far
    // as the workspace holds the partial sums (no split needs none)
    static const int z_force = env_int("EXL3_GEMM_SPLIT", 0);
    int zsplit = 1, kz = n_in / 16;
    exl3::plan_gemm_split(m, n_out, n_in / 16, z_force > 0 ? z_force * 1000000 : cu_count(), &zsplit, &kz);
    if (z_force > 0 && zsplit > z_force) {
        const int steps = n_in / 64, kstep = (steps + z_force - 1) / z_force;
        kz = 4 * kstep;
        zsplit = (steps + kstep - 1) / kstep;
    }
    const int64_t rot = gemm_rot_bytes(n_in, m);
    while (zsplit > 1 && rot + align256((int64_t)zsplit * m * n_out * 4) > (int64_t)workspace_bytes) {
        const int steps = n_in / 64, z = zsplit - 1, kstep = (steps + z - 1) / z;
        kz = 4 * kstep;
        zsplit = (steps + kstep - 1) / kstep;
    }
    if (zsplit <= 1) {
        zsplit = 1;
        kz = n_in / 16;
    }
    hipStream_t s = (hipStream_t)stream;
    const int rows = gemm_group_major(m) ? (int)gemm_rows(m) : 0;
    hipError_t e = exl3::launch_rotate(x, sign, m, n_in, xr, s, rows);
    if (e != hipSuccess) return EXL3_EHIP;
    exl3::GemmParams p;
    p.xr = xr;
    p.rows = rows;
    p.trellis = trellis;
    p.out_scale = out_scale;
    p.y = y;
    p.m = m;
    p.n_in = n_in;
    p.n_out = n_out;
    p.tiles_in = n_in / 16;
    p.n_strips = n_out / 16;
    p.zsplit = zsplit;
    p.kz = kz;
    p.part = zsplit > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + rot) : nullptr;
    e = exl3::launch_gemm(k_of(bits), cb_of(bits), p, s);
    return e == hipSuccess ? EXL3_OK : EXL3_EHIP;
}

int exl3_linear(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
                const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits, uint16_t* y,
                void* workspace, size_t workspace_bytes, void* stream) {
    // Measured crossover (MI355X, K = 4; 4096->14336, 14336->4096 and
    // 8192->8192 for m = 1..16, against the GEMM with 64-row blocks and its
    // split plan, the GEMV with its rotation pre-pass where that applies): the
    // GEMV wins through m = 14 at n_in = 4096 (22.1 against 25.2 us at m = 14,
    // 28.4 against 25.4 at m = 16), through m = 8 at n_in = 8192 (18.9 against
    // 24.6; within 2 % at m = 12) and through m = 9 at n_in = 14336 (even at
    // m = 10), as its x' of the m rows, 4 bytes per input, fills the LDS chunks.
    const bool use_gemv = linear_uses_gemv(m, n_in);
    return use_gemv ? exl3_gemv(x, m, trellis, sign, out_scale, n_in, n_out, bits, y, workspace, workspace_bytes, stream)
                    : exl3_gemm(x, m, trellis, sign, out_scale, n_in, n_out, bits, y, workspace, workspace_bytes, stream);
}

int exl3_linear_noalloc(const uint16_t* x, int32_t m, const uint16_t* trellis, const uint16_t* sign,
                        const uint16_t* out_scale, int32_t n_in, int32_t n_out, int32_t bits, uint16_t* y,
                        void* stream) {
    // every argument check and the size limit come before any HIP call
    const int rc = common_checks(x, m, trellis, sign, out_scale, n_in, n_out, bits, y, nullptr, 0, 0);
    if (rc <= 0) return rc;
    if (m > EXL3_GEMV_MAX_M || !linear_uses_gemv(m, n_in)) {
        // the GEMM's rotated input must fit; its split partial sums take what is
        // left (a smaller split when they do not all fit)
        if (gemm_rot_bytes(n_in, m) > (int64_t)EXL3_NOALLOC_SCRATCH_BYTES) return EXL3_EUNSUPPORTED;
    }
    void* ws = noalloc_scratch();
    if (!ws) return EXL3_EHIP;
    return exl3_linear(x, m, trellis, sign, out_scale, n_in, n_out, bits, y, ws, EXL3_NOALLOC_SCRATCH_BYTES, stream);
}

int64_t exl3_encode_slot_bytes(int32_t bits) {
    if (bad_bits(bits)) return EXL3_EINVAL;
    return exl3::encode_slot_bytes(k_of(bits));
}

int exl3_encode_tiles(const float* w, int64_t n_tiles, int32_t bits, uint16_t* words, float* costs,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (bad_bits(bits) || n_tiles < 0) return EXL3_EINVAL;
    if (n_tiles == 0) return EXL3_OK;
    if (!w || !words) return EXL3_EINVAL;
    if (misaligned(w) || misaligned(words) || misaligned(costs) || misaligned(workspace)) return EXL3_EINVAL;
    const int64_t slot = exl3::encode_slot_bytes(k_of(bits));
    if (!workspace || (int64_t)workspace_bytes < slot) return EXL3_EWORKSPACE;
    int64_t slots = (int64_t)workspace_bytes / slot;
    const int64_t cap = (int64_t)cu_count() * 4;  // tiles in flight: a few per CU
    if (slots > cap) slots = cap;
    if (slots > n_tiles) slots = n_tiles;
    exl3::EncodeParams p;
    p.w = w;
    p.n_tiles = n_tiles;
    p.words = words;
    p.costs = costs;
    p.scratch = static_cast<uint8_t*>(workspace);
    p.slot_bytes = slot;
    const hipError_t e = exl3::launch_encode(k_of(bits), cb_of(bits), p, (int)slots, (hipStream_t)stream);
    return e == hipSuccess ? EXL3_OK : EXL3_EHIP;
}

const char* exl3_status_string(int status) {
    switch (status) {
        case EXL3_OK: return "ok";
        case EXL3_EINVAL: return "invalid argument";
        case EXL3_EUNSUPPORTED: return "unsupported request";
        case EXL3_EWORKSPACE: return "workspace missing or too small";
        case EXL3_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
