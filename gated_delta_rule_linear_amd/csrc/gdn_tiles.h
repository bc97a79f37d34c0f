// Host-side launcher of the diagonal-tile comparison kernels in gdn_tiles.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct TilesLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;
    const float* initial_state;  // may be null (zero)
    float* final_state;          // may be null
    void* o;
    int32_t num_seqs;
    int32_t H;
    int32_t dk;
    int32_t dv;
    bool bf16;
    bool pairs;  // position-pair path (any finite g <= 0) instead of dense window products (g >= -5)
};

// Returns hipSuccess or the launch error.  Sizes are validated by the caller.
hipError_t launch_tiles(const TilesLaunch& p, hipStream_t stream);

}  // namespace gdn
