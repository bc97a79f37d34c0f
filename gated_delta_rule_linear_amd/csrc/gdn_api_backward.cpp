// libgdn C-ABI, backward pass: argument validation and dispatch.  The
// contract of each entry point is in include/gdn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <vector>

#include "gdn.h"
#include "gdn_backward.h"

namespace {

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

// GDN_VALIDATE=1: synchronous host check of cu_seqlens and of g's domain.
int32_t validate_backward_inputs(const int32_t* cu_dev, int32_t num_seqs, int64_t T_total, const float* g_dev,
                                 int64_t ng, hipStream_t s) {
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
        if (!(x >= -5.0f && x <= 0.0f)) return GDN_ERR_DOMAIN;
    return GDN_OK;
}

}  // namespace

namespace gdn {

// The split adds the forward pass's map pass and fold, an adjoint sweep
// without outputs and a reverse fold: on MI355X (bf16, d = 128) the split call
// over 256 (sequence, head) units of 8192 tokens takes 8.05 ms against 6.68
// unsplit, so it pays only when the units leave compute units idle: up to
// 144 units.  Segments (a multiple of 64 tokens, the forward's chunk) are cut
// so that about 512 workgroups run, no shorter than 512 tokens and at least
// three per sequence.  Measured (ms, unsplit -> split): 4 x 8192 tokens x 32
// heads 6.37 -> 4.40 (2048-token segments); 1 x 65536 x 16 heads 49.5 -> 4.85;
// 1 x 262144 x 16 198 -> 17.5; 4 x 2048 x 32 1.60 -> 1.20.
int64_t plan_backward_segment(int64_t T_total, int32_t num_seqs, int32_t H) {
    if (const char* e = std::getenv("GDN_BACKWARD_SEGMENT")) {
        if (*e) {
            const long long v = std::strtoll(e, nullptr, 10);
            return v <= 0 ? 0 : (int64_t)((v + 63) / 64 * 64);
        }
    }
    if (num_seqs <= 0 || T_total <= 0 || H <= 0) return 0;
    const int64_t units = (int64_t)num_seqs * H;
    if (units > 144) {
        // The length-agnostic split, as for the forward pass: with more units
        // than compute units, every sequence longer than T_total / (CUS / H + 1)
        // tokens (a chain at least the batch's work per compute unit) is cut,
        // whatever the lengths are; a batch without such a sequence runs its
        // sweeps as unsplit, one workgroup per (sequence, head).  (Up to CUS
        // units, sequences of similar lengths above that bound would be cut
        // too, and a cut costs the backward more than it gains there.)
        if (num_seqs < 2 || units <= kComputeUnits) return 0;
        const int64_t pmax = kComputeUnits / H + 1;
        const int64_t seg = ((T_total + pmax - 1) / pmax + 63) / 64 * 64;
        return pmax >= 3 && seg >= kSpeculativeMinSegment ? seg : 0;
    }
    const int64_t P = std::max<int64_t>(3, 512 / units), len = (T_total + num_seqs - 1) / num_seqs;
    const int64_t seg = std::max<int64_t>(512, ((len + P - 1) / P + 63) / 64 * 64);
    return (len + seg - 1) / seg >= 3 ? seg : 0;
}

}  // namespace gdn

extern "C" {

size_t gdn_prefill_backward_workspace_bytes(int64_t T_total, int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v,
                                            int32_t dtype) {
    if (T_total < 0 || num_seqs < 0 || H < 1 || d_k < 0 || d_v < 0) return 0;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return 0;
    return gdn::backward_workspace_bytes(T_total, num_seqs, H, d_k, d_v, dtype == GDN_BF16);
}

int32_t gdn_prefill_backward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total,
                             const float* initial_state, const void* d_o, const float* d_final_state, void* dq,
                             void* dk, void* dv, float* dg, float* dbeta, float* d_initial_state, int32_t H,
                             int32_t d_k, int32_t d_v, int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (num_seqs < 0 || T_total < 0 || H < 1) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (T_total > 0 && num_seqs == 0) return GDN_ERR_INVALID_ARG;
    if (num_seqs == 0) return GDN_OK;
    if (!cu_seqlens || !aligned_to(cu_seqlens, 4)) return GDN_ERR_INVALID_ARG;
    if (T_total > 0) {
        const void* p16[] = {q, k, v, g, d_o, dq, dk, dv, dg};
        for (const void* p : p16)
            if (!p || !aligned_to(p, 16)) return GDN_ERR_INVALID_ARG;
        if (!beta || !aligned_to(beta, 4) || !dbeta || !aligned_to(dbeta, 4)) return GDN_ERR_INVALID_ARG;
    }
    const void* st16[] = {initial_state, d_final_state, d_initial_state};
    for (const void* p : st16)
        if (p && !aligned_to(p, 16)) return GDN_ERR_INVALID_ARG;
    const size_t need = gdn::backward_workspace_bytes(T_total, num_seqs, H, d_k, d_v, dtype == GDN_BF16);
    if (!workspace || workspace_bytes < need || !aligned_to(workspace, 16)) return GDN_ERR_INVALID_ARG;
    const int64_t seg = gdn::plan_backward_segment(T_total, num_seqs, H);
    if (((int64_t)num_seqs + (seg > 0 ? T_total / seg : 0)) * H > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (const char* e = std::getenv("GDN_VALIDATE"); e && e[0] == '1') {
        const int32_t st = validate_backward_inputs(cu_seqlens, num_seqs, T_total, g, T_total * H * d_k, s);
        if (st != GDN_OK) return st;
    }
    gdn::BackwardLaunch p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.cu_seqlens = cu_seqlens;
    p.initial_state = initial_state;
    p.d_o = d_o;
    p.d_final_state = d_final_state;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dg = dg;
    p.dbeta = dbeta;
    p.d_initial_state = d_initial_state;
    p.num_seqs = num_seqs;
    p.H = H;
    p.dk_dim = d_k;
    p.dv_dim = d_v;
    p.bf16 = dtype == GDN_BF16;
    p.T_total = T_total;
    p.workspace = workspace;
    p.seg = seg;
    return gdn::launch_backward(p, s) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
