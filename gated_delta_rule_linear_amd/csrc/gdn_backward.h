// Host-side launcher of the backward (gradient) kernels in gdn_backward.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct BackwardLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;
    const float* initial_state;  // may be null (zero)
    const void* d_o;
    const float* d_final_state;  // may be null (zero)
    void* dq;
    void* dk;
    void* dv;
    float* dg;
    float* dbeta;
    float* d_initial_state;      // may be null (not wanted)
    int32_t num_seqs;
    int32_t H;
    int32_t dk_dim;
    int32_t dv_dim;
    bool bf16;
    int64_t T_total;
    void* workspace;             // backward_workspace_bytes(...) bytes
};

// Checkpoints of the backward pass: the start state of every 16-token
// sub-chunk, in the input dtype.  Sequence n's sub-chunk c uses slot
// cu[n] / 16 + n + c (slots never overlap: a sequence of len tokens needs
// ceil(len / 16) of them and the next one starts at least that far on), so
// T_total / 16 + num_seqs slots per head suffice.
inline size_t backward_workspace_bytes(int64_t T_total, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                                       bool bf16) {
    return ((size_t)(T_total / 16) + (size_t)num_seqs) * (size_t)H * (size_t)dk * (size_t)dv * (bf16 ? 2 : 4);
}

// Returns hipSuccess or the launch error.  Sizes are validated by the caller.
hipError_t launch_backward(const BackwardLaunch& p, hipStream_t stream);

}  // namespace gdn
