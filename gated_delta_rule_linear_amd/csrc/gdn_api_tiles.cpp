// libgdn C-ABI, diagonal-tile comparison: argument validation and dispatch.
// The contract is in include/gdn.h (gdn_prefill_tiles).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <vector>

#include "gdn.h"
#include "gdn_tiles.h"

namespace {

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

// GDN_VALIDATE=1: cu_seqlens, and g in [lo, 0] and finite.
int32_t validate_tiles_inputs(const int32_t* cu_dev, int32_t num_seqs, int64_t T_total, const float* g_dev,
                              int64_t ng, float lo, hipStream_t s) {
    std::vector<int32_t> cu((size_t)num_seqs + 1);
    std::vector<float> g((size_t)ng);
    if (hipMemcpyAsync(cu.data(), cu_dev, sizeof(int32_t) * cu.size(), hipMemcpyDeviceToHost, s) != hipSuccess)
        return GDN_ERR_HIP;
    if (ng > 0 && hipMemcpyAsync(g.data(), g_dev, sizeof(float) * g.size(), hipMemcpyDeviceToHost, s) != hipSuccess)
        return GDN_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_HIP;
    if (cu[0] != 0 || cu[(size_t)num_seqs] != T_total) return GDN_ERR_DOMAIN;
    for (int32_t n = 0; n < num_seqs; ++n)
        if (cu[(size_t)n + 1] < cu[(size_t)n]) return GDN_ERR_DOMAIN;
    for (float x : g)
        if (!(x >= lo && x <= 0.0f) || !std::isfinite(x)) return GDN_ERR_DOMAIN;
    return GDN_OK;
}

}  // namespace

extern "C" {

int32_t gdn_prefill_tiles(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total, const float* initial_state,
                          float* final_state, void* o, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                          int32_t tile_path, void* stream) {
    if (num_seqs < 0 || T_total < 0 || H < 1) return GDN_ERR_INVALID_ARG;
    if (tile_path != GDN_TILES_DENSE && tile_path != GDN_TILES_PAIRS) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (T_total > 0 && num_seqs == 0) return GDN_ERR_INVALID_ARG;
    if (num_seqs == 0) return GDN_OK;
    if (!cu_seqlens || !aligned_to(cu_seqlens, 4)) return GDN_ERR_INVALID_ARG;
    if (T_total > 0) {
        const void* p16[] = {q, k, v, g, o};
        for (const void* p : p16)
            if (!p || !aligned_to(p, 16)) return GDN_ERR_INVALID_ARG;
        if (!beta || !aligned_to(beta, 4)) return GDN_ERR_INVALID_ARG;
    }
    if (initial_state && !aligned_to(initial_state, 16)) return GDN_ERR_INVALID_ARG;
    if (final_state && !aligned_to(final_state, 16)) return GDN_ERR_INVALID_ARG;
    if ((int64_t)num_seqs * H > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (const char* e = std::getenv("GDN_VALIDATE"); e && e[0] == '1') {
        const float lo = tile_path == GDN_TILES_DENSE ? -5.0f : -INFINITY;
        const int32_t st = validate_tiles_inputs(cu_seqlens, num_seqs, T_total, g, T_total * H * d_k, lo, s);
        if (st != GDN_OK) return st;
    }
    gdn::TilesLaunch p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.cu_seqlens = cu_seqlens;
    p.initial_state = initial_state;
    p.final_state = final_state;
    p.o = o;
    p.num_seqs = num_seqs;
    p.H = H;
    p.dk = d_k;
    p.dv = d_v;
    p.bf16 = dtype == GDN_BF16;
    p.pairs = tile_path == GDN_TILES_PAIRS;
    return gdn::launch_tiles(p, s) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
