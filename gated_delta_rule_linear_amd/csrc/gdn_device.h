// Device-side helpers shared by the libgdn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_kernels.h"  // GATE_* values

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }


// sigmoid(z) = 1 / (1 + e^-z) with the hardware base-2 exponential and
// reciprocal; z -> -inf gives 0 (1/inf), z -> +inf gives 1.
__device__ __forceinline__ float sigmoid_hw(float z) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
// Log-decay g of one key channel from its logit z.
__device__ __forceinline__ float gate_log_decay(float z, int gate, float p) {
    const float s = sigmoid_hw(z);
    if (gate == GATE_SCALED_SIGMOID) return p * s;
    return __builtin_amdgcn_logf(p + (1.f - p) * s) * 0.6931471805599453f;  // log2 -> natural log
}
// Decay factor alpha = e^g of one key channel from its logit z.
__device__ __forceinline__ float gate_alpha(float z, int gate, float p) {
    const float s = sigmoid_hw(z);
    if (gate == GATE_SCALED_SIGMOID) return __builtin_amdgcn_exp2f(1.4426950408889634f * p * s);
    return p + (1.f - p) * s;
}

}  // namespace gdn
