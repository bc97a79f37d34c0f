// libgdn C-ABI: argument validation, status codes and dispatch to the kernels.
// Declarations and the contract of every entry point are in include/gdn.h.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdn_kernels.h"

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool supported_d(int32_t d) { return d == 64 || d == 128; }
bool validate_mode() {
    const char* e = std::getenv("GDN_VALIDATE");
    return e && e[0] == '1';
}

// Host-side check of cu_seqlens and of the log-decay domain (g_dev may be
// null); synchronous.
int32_t validate_inputs(const int32_t* cu_dev, int32_t num_seqs, int64_t T_total, const float* g_dev, int64_t ng,
                        hipStream_t s, int64_t max_seqlen = 0) {
    std::vector<int32_t> cu((size_t)num_seqs + 1);
    if (hipMemcpyAsync(cu.data(), cu_dev, sizeof(int32_t) * cu.size(), hipMemcpyDeviceToHost, s) != hipSuccess)
        return GDN_ERR_HIP;
    std::vector<float> g(g_dev ? (size_t)ng : 0);  // no g (logit gates): cu_seqlens only
    if (g_dev && ng > 0 && hipMemcpyAsync(g.data(), g_dev, sizeof(float) * g.size(), hipMemcpyDeviceToHost, s) != hipSuccess)
        return GDN_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_HIP;
    if (cu[0] != 0 || cu[(size_t)num_seqs] != T_total) return GDN_ERR_DOMAIN;
    for (int32_t n = 0; n < num_seqs; ++n) {
        if (cu[(size_t)n + 1] < cu[(size_t)n]) return GDN_ERR_DOMAIN;
        if (max_seqlen > 0 && cu[(size_t)n + 1] - cu[(size_t)n] > max_seqlen) return GDN_ERR_DOMAIN;
    }
    for (float x : g)
        if (!(x >= -5.0f && x <= 0.0f)) return GDN_ERR_DOMAIN;
    return GDN_OK;
}

}  // namespace

namespace gdn {

// Time split of long sequences.  One workgroup carries one (sequence, head)
// through its chunks in order, so a batch of few long sequences leaves most of
// the 256 compute units idle.  Cutting sequences into segments of Ls tokens
// costs a second pass over the non-last segments (their transitions M and N)
// and a serial fold, and buys parallelism.  The plan compares critical paths
// (SplitCost, in chunk-times of the output pass) for sequences of the mean
// length (the lengths themselves are on the device):
//   whole sequences:  rounds(units) * (chunks + START)
//   split into P:     maps_pass(units (P-1), Ls/64) + fold_pass(P-1, units d_v/16)
//                     + rounds(units P) * (Ls/64 + START)
// where rounds() weights a partly filled round by its occupancy, and splits
// when that saves at least 5%.  The workspace bound, and so the
// plan, depends on the arguments only.
// With a host-side bound max_seqlen on the lengths (a skewed batch: one long
// sequence packed with short ones), the plan assumes the most skewed batch the
// bound allows -- n_long = T_total / max_seqlen sequences of max_seqlen tokens,
// the other tokens spread evenly over the rest -- and compares
//   whole sequences:  max(chain of the longest, total work / CUS)
//   split (length Ls, only the long sequences have more than one segment):
//     phase 1 = max(Ls chain, (long units' first segments + every short unit
//               + the maps of segments 1 .. P-2) / CUS)
//     + fold_pass(P - 2, long units d_v/16) + rounds(long units (P - 1)) (Ls chunks + START)
// in the same chunk-time units, and splits when that saves at least 5%.  When
// every sequence can be of max_seqlen tokens, the mean-length plan is used.
static int64_t plan_prefill_skewed(int64_t T_total, int32_t num_seqs, int32_t H, int32_t d_v, bool share,
                                   int64_t max_len) {
    typedef SplitCost K;
    const double n_long = (double)std::max<int64_t>(1, std::min<int64_t>(num_seqs, T_total / max_len));
    const double n_short = num_seqs - n_long, short_tokens = (double)T_total - n_long * (double)max_len;
    const double len_s = n_short > 0 ? short_tokens / n_short : 0.0;
    const double Ul = n_long * H, Us = n_short * H, chain = std::ceil(max_len / 64.0) + K::START;
    const double short_work = Us * (std::ceil(len_s / 64.0) + K::START);
    const double whole = std::max(chain, (Ul * chain + short_work) / K::CUS);
    double best = whole;
    int64_t best_seg = 0;
    const int64_t step = std::max<int64_t>(64, max_len / 2048 / 64 * 64);
    for (int64_t ls = std::max<int64_t>(1024, (int64_t)std::ceil(len_s / 64.0) * 64); ls < max_len; ls += step) {
        const double P = std::ceil((double)max_len / ls), ch = ls / 64.0;
        bool both = false;
        (void)K::maps_pass(Ul * (P - 2), ch, share, &both);
        const double map_work = (both ? Ul * (P - 2) * (ch * K::MAP_BOTH + K::START)
                                      : 2 * Ul * (P - 2) * (ch * K::MAP_ONE + K::START));
        const double first = std::max(ch + K::START, (Ul * (ch + K::START) + short_work + map_work) / K::CUS);
        const double t = first + K::fold_pass(P - 2, Ul * (d_v / 16)) + K::rounds(Ul * (P - 1)) * (ch + K::START);
        if (t < best) {
            best = t;
            best_seg = ls;
        }
    }
    return best < 0.95 * whole ? best_seg : 0;
}

int64_t plan_prefill_segment(int64_t T_total, int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, bool bf16,
                             int64_t max_seqlen) {
    if (const char* e = std::getenv("GDN_PREFILL_SEGMENT")) {
        if (*e) {
            const long long v = std::strtoll(e, nullptr, 10);
            return v <= 0 ? 0 : (int64_t)((v + 63) / 64 * 64);
        }
    }
    if (num_seqs <= 0 || T_total <= 0 || H <= 0) return 0;
    if (max_seqlen > 0 && max_seqlen < T_total && (int64_t)num_seqs * max_seqlen > T_total)
        return plan_prefill_skewed(T_total, num_seqs, H, d_v, bf16 && d_k == d_v, max_seqlen);
    typedef SplitCost K;
    const bool share = bf16 && d_k == d_v;
    const double units = (double)num_seqs * H;
    const int64_t len = (T_total + num_seqs - 1) / num_seqs;
    const double whole = K::rounds(units) * (std::ceil(len / 64.0) + K::START);
    double best = whole;
    int64_t best_seg = 0;
    // Split of P segments: the output pass of segment 0 beside the maps of
    // segments 1 .. P-2 (one pass: its critical path is the longer of the two,
    // counted as output chunks in rounds of all their workgroups), the fold
    // from segment 1, then the output pass of segments 1 .. P-1.
    const int64_t step = std::max<int64_t>(64, len / 2048 / 64 * 64);
    for (int64_t ls = 1024; ls < len; ls += step) {
        const double P = std::ceil((double)len / ls), ch = ls / 64.0;
        bool both = false;
        const double maps = K::maps_pass(units * (P - 2), ch, share, &both);
        const double first = K::rounds(units + (both ? 1 : 2) * units * (P - 2)) * (ch + K::START);
        const double t = std::max(first, maps) + K::fold_pass(P - 2, units * (d_v / 16)) +
                         K::rounds(units * (P - 1)) * (ch + K::START);
        if (t < best) {
            best = t;
            best_seg = ls;
        }
    }
    if (best < 0.95 * whole) return best_seg;
    // No split for sequences of the mean length.  With more units than compute
    // units the lengths may still be skewed, and one sequence much longer than
    // the rest would then be the critical path of the call.  Split, whatever
    // the lengths turn out to be, every sequence longer than
    //   Ls = T_total / (CUS / H + 1)
    // tokens: a sequence that long has a chain at least the whole batch's work
    // per compute unit, and the later segments of even one sequence of T_total
    // tokens then fill one round of workgroups.  A batch without such a
    // sequence runs as unsplit (its table, empty map and fold passes and an
    // empty pass over later segments cost some tens of microseconds, so the
    // segment must be long enough for that not to matter).
    if (num_seqs > 1 && units > K::CUS) {
        const int64_t pmax = (int64_t)(K::CUS / H) + 1;
        const int64_t ls = ((T_total + pmax - 1) / pmax + 63) / 64 * 64;
        if (pmax >= 3 && ls >= kSpeculativeMinSegment) return ls;
    }
    return 0;
}

}  // namespace gdn

// The logit entry points' gate and parameter; the parameter keeps every
// log-decay in [-5, 0].
static int32_t check_gate(int32_t gate, float p) {
    if (gate == GDN_GATE_SCALED_SIGMOID) return p >= -5.0f && p <= 0.0f ? GDN_OK : GDN_ERR_DOMAIN;
    if (gate == GDN_GATE_ALPHA_MIN) return p >= 0.006737947f && p <= 1.0f ? GDN_OK : GDN_ERR_DOMAIN;  // e^-5 rounded up
    return GDN_ERR_INVALID_ARG;
}

extern "C" {

const char* gdn_status_string(int32_t status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, negative size, short workspace)";
        case GDN_ERR_UNSUPPORTED:
            return "unsupported configuration (d_k and d_v must be 64 or 128; dtype f32 or bf16, bf16 for the logit "
                   "and per-head gate entry points)";
        case GDN_ERR_DOMAIN: return "input outside the domain (g not in [-5, 0] or malformed cu_seqlens)";
        case GDN_ERR_OOM: return "device allocation failed";
        case GDN_ERR_HIP: return "HIP runtime error";
        case GDN_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

size_t gdn_state_bytes(int64_t num_seqs, int32_t H, int32_t d_k, int32_t d_v) {
    if (num_seqs < 0 || H < 0 || d_k < 0 || d_v < 0) return 0;
    size_t b = sizeof(float);
    for (const size_t f : {(size_t)num_seqs, (size_t)H, (size_t)d_k, (size_t)d_v})
        if (__builtin_mul_overflow(b, f, &b)) return SIZE_MAX;  // not addressable: saturate
    return b;
}

int32_t gdn_state_alloc(int64_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, float** out, void* stream) {
    if (!out || num_seqs < 0 || H < 1) return GDN_ERR_INVALID_ARG;
    if (!supported_d(d_k) || !supported_d(d_v)) return GDN_ERR_UNSUPPORTED;
    *out = nullptr;
    const size_t bytes = gdn_state_bytes(num_seqs, H, d_k, d_v);
    if (bytes == 0) return GDN_OK;
    if (bytes == SIZE_MAX) return GDN_ERR_OOM;  // the size does not fit size_t: no device call is made
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* p = nullptr;
    if (hipMallocAsync(&p, bytes, s) != hipSuccess || !p) {
        (void)hipGetLastError();
        return GDN_ERR_OOM;
    }
    if (hipMemsetAsync(p, 0, bytes, s) != hipSuccess) {
        (void)hipFreeAsync(p, s);
        return GDN_ERR_HIP;
    }
    *out = static_cast<float*>(p);
    return GDN_OK;
}

int32_t gdn_state_free(float* state, void* stream) {
    if (!state) return GDN_OK;
    return hipFreeAsync(state, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_prefill_workspace_bytes(int64_t T_total, int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v) {
    return gdn_prefill_workspace_bytes_maxlen(T_total, num_seqs, 0, H, d_k, d_v);
}

size_t gdn_prefill_workspace_bytes_maxlen(int64_t T_total, int32_t num_seqs, int64_t max_seqlen, int32_t H,
                                          int32_t d_k, int32_t d_v) {
    if (T_total < 0 || num_seqs < 0 || max_seqlen < 0 || H < 1 || d_k < 0 || d_v < 0) return 0;
    const int64_t seg = gdn::plan_prefill_segment(T_total, num_seqs, H, d_k, d_v, true, max_seqlen);
    return gdn::prefill_workspace_layout(T_total, num_seqs, H, d_k, d_v, seg).bytes;
}

static int32_t prefill_impl(const void* q, const void* k, const void* v, const float* g, const void* z,
                            int32_t gate, float gate_param, const float* beta, const int32_t* cu_seqlens,
                            int32_t num_seqs, int64_t T_total, const float* initial_state, float* final_state,
                            void* o, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, void* workspace,
                            size_t workspace_bytes, void* stream, int64_t max_seqlen = 0) {
    if (num_seqs < 0 || T_total < 0 || H < 1 || max_seqlen < 0) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!supported_d(d_k) || !supported_d(d_v)) return GDN_ERR_UNSUPPORTED;
    if (T_total > 0 && num_seqs == 0) return GDN_ERR_INVALID_ARG;
    if (num_seqs == 0) return GDN_OK;
    if (!cu_seqlens || !aligned(cu_seqlens, 4)) return GDN_ERR_INVALID_ARG;
    if (T_total > 0) {
        const bool head = gate == gdn::GATE_HEAD;
        const void* ptrs16[] = {q, k, v, gate == GDN_GATE_LOG ? static_cast<const void*>(g) : head ? q : z, o};
        for (const void* p : ptrs16)
            if (!p || !aligned(p, 16)) return GDN_ERR_INVALID_ARG;
        if (!beta || !aligned(beta, 4)) return GDN_ERR_INVALID_ARG;
        if (head && (!g || !aligned(g, 4))) return GDN_ERR_INVALID_ARG;
    }
    if (initial_state && !aligned(initial_state, 16)) return GDN_ERR_INVALID_ARG;
    if (final_state && !aligned(final_state, 16)) return GDN_ERR_INVALID_ARG;
    const int64_t seg = gdn::plan_prefill_segment(T_total, num_seqs, H, d_k, d_v, true, max_seqlen);
    const size_t need = gdn::prefill_workspace_layout(T_total, num_seqs, H, d_k, d_v, seg).bytes;
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16))) return GDN_ERR_INVALID_ARG;
    if (((int64_t)num_seqs + (seg > 0 ? T_total / seg : 0)) * H * (d_v / 16) > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (validate_mode()) {
        // (logits: every finite or infinite z maps into the domain, so only cu_seqlens is checked)
        const bool has_g = gate == GDN_GATE_LOG || gate == gdn::GATE_HEAD;
        const int32_t st = validate_inputs(cu_seqlens, num_seqs, T_total, has_g ? g : nullptr,
                                           T_total * H * (gate == gdn::GATE_HEAD ? 1 : d_k), s, max_seqlen);
        if (st != GDN_OK) return st;
    }
    gdn::PrefillLaunch p;
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
    p.T_total = T_total;
    p.seg = seg;
    p.workspace = workspace;
    p.z = z;
    p.gate = gate;
    p.gate_param = gate_param;
    p.max_seqlen = max_seqlen;
    {
        const char* e = std::getenv("GDN_PREFILL_KERNEL");
        p.legacy = e && std::strcmp(e, "seq") == 0;
    }
    return gdn::launch_prefill(p, s) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int32_t gdn_prefill(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total, const float* initial_state,
                    float* final_state, void* o, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, g, nullptr, GDN_GATE_LOG, 0.f, beta, cu_seqlens, num_seqs, T_total, initial_state,
                        final_state, o, H, d_k, d_v, dtype, workspace, workspace_bytes, stream);
}

int32_t gdn_prefill_maxlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total, int64_t max_seqlen,
                           const float* initial_state, float* final_state, void* o, int32_t H, int32_t d_k,
                           int32_t d_v, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, g, nullptr, GDN_GATE_LOG, 0.f, beta, cu_seqlens, num_seqs, T_total, initial_state,
                        final_state, o, H, d_k, d_v, dtype, workspace, workspace_bytes, stream, max_seqlen);
}

int32_t gdn_prefill_head_gate(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total,
                              const float* initial_state, float* final_state, void* o, int32_t H, int32_t d_k,
                              int32_t d_v, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    return prefill_impl(q, k, v, g, nullptr, gdn::GATE_HEAD, 0.f, beta, cu_seqlens, num_seqs, T_total,
                        initial_state, final_state, o, H, d_k, d_v, dtype, workspace, workspace_bytes, stream);
}

int32_t gdn_prefill_logits(const void* q, const void* k, const void* v, const void* z, int32_t gate,
                           float gate_param, const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                           int64_t T_total, const float* initial_state, float* final_state, void* o, int32_t H,
                           int32_t d_k, int32_t d_v, int32_t dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
    const int32_t st = check_gate(gate, gate_param);
    if (st != GDN_OK) return st;
    if (dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    return prefill_impl(q, k, v, nullptr, z, gate, gate_param, beta, cu_seqlens, num_seqs, T_total, initial_state,
                        final_state, o, H, d_k, d_v, dtype, workspace, workspace_bytes, stream);
}

static int32_t decode_impl(const void* q, const void* k, const void* v, const float* g, const void* z, int32_t gate,
                           float gate_param, const float* beta, float* state, void* o, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, int32_t dtype, void* stream) {
    if (N < 0 || H < 1) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!supported_d(d_k) || !supported_d(d_v)) return GDN_ERR_UNSUPPORTED;
    if (N == 0) return GDN_OK;
    const bool head = gate == gdn::GATE_HEAD;
    const void* ptrs16[] = {q, k, v, gate == GDN_GATE_LOG ? static_cast<const void*>(g) : head ? q : z, o, state};
    for (const void* p : ptrs16)
        if (!p || !aligned(p, 16)) return GDN_ERR_INVALID_ARG;
    if (!beta || !aligned(beta, 4)) return GDN_ERR_INVALID_ARG;
    if (head && (!g || !aligned(g, 4))) return GDN_ERR_INVALID_ARG;
    if ((int64_t)N * H > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (validate_mode() && (gate == GDN_GATE_LOG || head)) {
        std::vector<float> gh((size_t)N * H * (head ? 1 : d_k));
        if (hipMemcpyAsync(gh.data(), g, sizeof(float) * gh.size(), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return GDN_ERR_HIP;
        for (float x : gh)
            if (!(x >= -5.0f && x <= 0.0f)) return GDN_ERR_DOMAIN;
    }
    gdn::DecodeLaunch p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.state = state;
    p.o = o;
    p.N = N;
    p.H = H;
    p.dk = d_k;
    p.dv = d_v;
    p.bf16 = dtype == GDN_BF16;
    p.z = z;
    p.gate = gate;
    p.gate_param = gate_param;
    return gdn::launch_decode(p, s) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int32_t gdn_decode(const void* q, const void* k, const void* v, const float* g, const float* beta, float* state,
                   void* o, int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, void* stream) {
    return decode_impl(q, k, v, g, nullptr, GDN_GATE_LOG, 0.f, beta, state, o, N, H, d_k, d_v, dtype, stream);
}

int32_t gdn_decode_head_gate(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             float* state, void* o, int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                             void* stream) {
    return decode_impl(q, k, v, g, nullptr, gdn::GATE_HEAD, 0.f, beta, state, o, N, H, d_k, d_v, dtype, stream);
}

int32_t gdn_decode_logits(const void* q, const void* k, const void* v, const void* z, int32_t gate, float gate_param,
                          const float* beta, float* state, void* o, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                          int32_t dtype, void* stream) {
    const int32_t st = check_gate(gate, gate_param);
    if (st != GDN_OK) return st;
    if (dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    return decode_impl(q, k, v, nullptr, z, gate, gate_param, beta, state, o, N, H, d_k, d_v, dtype, stream);
}


}  // extern "C"
