// Host-side launchers of the libgdn kernels (defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct PrefillLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;
    const float* initial_state;  // may be null
    float* final_state;          // may be null
    void* o;
    int32_t num_seqs;
    int32_t H;
    int32_t dk;
    int32_t dv;
    bool bf16;
};

struct DecodeLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* o;
    int32_t N;
    int32_t H;
    int32_t dk;
    int32_t dv;
    bool bf16;
};

// Each returns hipSuccess or the launch error.  Sizes are validated by the caller.
hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& p, hipStream_t stream);

}  // namespace gdn
