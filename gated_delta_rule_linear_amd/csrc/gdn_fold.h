// Column-block fold of the time split's segment maps on the fp32 matrix cores.
//
// A long sequence split into segments is joined by an affine recurrence per
// (sequence, head): x <- A_j x + B_j with A_j = M_j (d_k x d_k) forward, or
// A_j = M_j^T backward, and B_j a d_k x d_v matrix that the result overwrites.
// The columns of x evolve independently, so one workgroup takes 16 of them,
// with one wave per 16-row tile of x: 64 * d_k / 16 threads.
//
// Each step is d_k / 4 products v_mfma_f32_16x16x4_f32 per wave.  The
// contraction index runs in a permuted order: in product (b, s) lane group g
// supplies k = 16b + 4g + s.  A lane's A-operand values for four products are
// then four adjacent entries of one row of A_j (M_j: one 16-byte load from
// memory; M_j^T: four loads that 16 lanes make over 64 contiguous bytes), and
// its B-operand values are the rows 16b + 4g + s of tile b that lane group g
// of that tile's accumulator holds.  x passes between the waves through LDS
// in the accumulator layout (4 KiB per 64 rows); the operands of step
// j + DEPTH are loaded while step j runs (DEPTH 2 for one workgroup per CU,
// DEPTH 1 so that two fit in a CU's registers when there are more
// workgroups than CUs).
#pragma once

#include "gdn_mfma.h"

namespace gdn {

// Runs `steps` steps over columns 16 cb .. 16 cb + 15.  x0: the start value
// (d_k x d_v, row-major; nullptr for zero).  map_at(j): A_j's matrix M
// (d_k x d_k, row-major) for the j-th step taken; add_at(j): B_j (d_k x d_v,
// row-major), read and then overwritten with the step's result.  Every
// thread of the workgroup calls it with the same arguments.
template <int DK, int DV, bool TRANSPOSED, int DEPTH = 2, typename MapAt, typename AddAt>
__device__ __forceinline__ void fold_columns(const float* x0, int steps, int cb, MapAt map_at, AddAt add_at) {
    static_assert(DEPTH == 1 || DEPTH == 2, "prefetch depth");
    constexpr int RT = DK / 16;
    __shared__ floatx4 xs[RT][64];  // xs[t][l] = x[16t + 4g + i][16cb + r], lane l = r + 16g
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, g = l >> 4;
    const size_t my_row = (size_t)(16 * w + 4 * g) * DV + 16 * cb + r;  // element (16w + 4g, 16cb + r)
    {
        floatx4 x = zero4();
        if (x0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = x0[my_row + (size_t)i * DV];
        }
        xs[w][l] = x;
    }
    auto load = [&](int j, floatx4(&m)[RT], floatx4& nn) {
        const float* M = map_at(j);
        if constexpr (!TRANSPOSED) {
            const float* row = M + (size_t)(16 * w + r) * DK + 4 * g;  // A_j[16w + r][16b + 4g + s]
#pragma unroll
            for (int b = 0; b < RT; ++b) m[b] = *reinterpret_cast<const floatx4*>(row + 16 * b);
        } else {
            const float* col = M + (size_t)(4 * g) * DK + 16 * w + r;  // M_j[16b + 4g + s][16w + r]
#pragma unroll
            for (int b = 0; b < RT; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) m[b][s] = col[(size_t)(16 * b + s) * DK];
        }
        const float* B = add_at(j) + my_row;
#pragma unroll
        for (int i = 0; i < 4; ++i) nn[i] = B[(size_t)i * DV];
    };
    // step j with its operands in (m, nn); those of step j + DEPTH go to (m2, n2)
    auto step = [&](int j, const floatx4(&m)[RT], const floatx4& nn, floatx4(&m2)[RT], floatx4& n2) {
        if (j + DEPTH < steps) load(j + DEPTH, m2, n2);
        __syncthreads();  // xs holds the current x
        floatx4 xb[RT];
#pragma unroll
        for (int b = 0; b < RT; ++b) xb[b] = xs[b][l];
        floatx4 acc0 = nn, acc1 = zero4();
#pragma unroll
        for (int b = 0; b < RT; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (b & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[b][s], xb[b][s], acc1, 0, 0, 0);
                else acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(m[b][s], xb[b][s], acc0, 0, 0, 0);
            }
        const floatx4 acc = acc0 + acc1;
        __syncthreads();  // every wave has read x
        xs[w][l] = acc;
        float* B = add_at(j) + my_row;
#pragma unroll
        for (int i = 0; i < 4; ++i) B[(size_t)i * DV] = acc[i];
    };
    if constexpr (DEPTH == 2) {
        floatx4 m0[RT], m1[RT], m2[RT], n0, n1, n2;
        if (steps > 0) load(0, m0, n0);
        if (steps > 1) load(1, m1, n1);
        for (int j = 0; j < steps; j += 3) {
            step(j, m0, n0, m2, n2);
            if (j + 1 < steps) step(j + 1, m1, n1, m0, n0);
            if (j + 2 < steps) step(j + 2, m2, n2, m1, n1);
        }
    } else {
        floatx4 m0[RT], m1[RT], n0, n1;
        if (steps > 0) load(0, m0, n0);
        for (int j = 0; j < steps; j += 2) {
            step(j, m0, n0, m1, n1);
            if (j + 1 < steps) step(j + 1, m1, n1, m0, n0);
        }
    }
}

}  // namespace gdn
