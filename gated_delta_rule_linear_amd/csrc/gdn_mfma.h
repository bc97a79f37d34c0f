// 16x16 matrix-core tiles for gfx950, and the operand layouts the kernels use.
//
// One MFMA multiplies a 16 x K tile of A by a K x 16 tile of B into a 16 x 16
// fp32 accumulator, in one wave of 64 lanes.  With lane l, r = l % 16 and
// g = l / 16 (0..3):
//   accumulator: lane l holds C[4g + i][r], i = 0..3   (a floatx4)
//   A operand:   lane l holds A[r][k] for KW consecutive k starting at g*KW
//   B operand:   lane l holds B[k][r] for the same k
// bf16: K = 32 per instruction, KW = 8 (v_mfma_f32_16x16x32_bf16).
// fp32: K = 4 per instruction,  KW = 1 (v_mfma_f32_16x16x4_f32).
//
// Two ways of walking a contraction of length K are used:
//  * natural:   step m, lane group g holds k = m*K + g*KW + j.  Both operands
//               are read from LDS rows where k is contiguous.
//  * permuted:  the element e = m*KW + j of lane group g stands for
//               k = 16*(e/4) + 4g + e%4.  This is the order in which an
//               accumulator already holds its rows (lane group g owns rows
//               4g..4g+3 of each 16-row tile), so a result tile can be fed
//               back as a B operand straight from registers, and the matching
//               A operand is read from LDS in that order.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
    static constexpr int KW = 8;
    static constexpr int KSTEP = 32;
    typedef bf16x8 frag;
    __device__ __forceinline__ static floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag zero() { return frag{}; }
};

template <>
struct Mma<float> {
    static constexpr int KW = 1;
    static constexpr int KSTEP = 4;
    typedef float frag;
    __device__ __forceinline__ static floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag zero() { return 0.0f; }
};

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// ---- natural order, operand row read from LDS (row-major, k contiguous) ----
__device__ __forceinline__ bf16x8 lds_nat(const bf16* row, int m, int g) {
    return *reinterpret_cast<const bf16x8*>(row + m * 32 + g * 8);
}
__device__ __forceinline__ float lds_nat(const float* row, int m, int g) { return row[m * 4 + g]; }

// ---- permuted order, operand row read from LDS ----
// `kmax` (a multiple of 16): elements with k >= kmax read as zero.
__device__ __forceinline__ bf16x8 lds_perm(const bf16* row, int m, int g, int kmax = 1 << 30) {
    bf16x4 lo = bf16x4{}, hi = bf16x4{};
    if (32 * m < kmax) lo = *reinterpret_cast<const bf16x4*>(row + 32 * m + 4 * g);
    if (32 * m + 16 < kmax) hi = *reinterpret_cast<const bf16x4*>(row + 32 * m + 16 + 4 * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ float lds_perm(const float* row, int m, int g, int kmax = 1 << 30) {
    const int k = 16 * (m >> 2) + 4 * g + (m & 3);
    return k < kmax ? row[k] : 0.0f;
}

// Permuted operand read from an fp32 LDS row and converted to the tile type.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag lds_perm_f32(const float* row, int m, int g, int kmax);
template <>
__device__ __forceinline__ bf16x8 lds_perm_f32<bf16>(const float* row, int m, int g, int kmax) {
    bf16x8 f = bf16x8{};
    if (32 * m < kmax) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(row + 32 * m + 4 * g);
        f[0] = (bf16)a[0]; f[1] = (bf16)a[1]; f[2] = (bf16)a[2]; f[3] = (bf16)a[3];
    }
    if (32 * m + 16 < kmax) {
        const floatx4 b = *reinterpret_cast<const floatx4*>(row + 32 * m + 16 + 4 * g);
        f[4] = (bf16)b[0]; f[5] = (bf16)b[1]; f[6] = (bf16)b[2]; f[7] = (bf16)b[3];
    }
    return f;
}
template <>
__device__ __forceinline__ float lds_perm_f32<float>(const float* row, int m, int g, int kmax) {
    return lds_perm(row, m, g, kmax);
}

// ---- permuted order, B operand taken from accumulator tiles acc[0..] ----
// Tile t of `acc` holds rows 16t..16t+15 of the contraction dimension.
// `ntiles` tiles are valid; later ones read as zero.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag acc_perm(const floatx4* acc, int m, int ntiles);
template <>
__device__ __forceinline__ bf16x8 acc_perm<bf16>(const floatx4* acc, int m, int ntiles) {
    bf16x8 f = bf16x8{};
    if (2 * m < ntiles) {
        const floatx4 a = acc[2 * m];
        f[0] = (bf16)a[0]; f[1] = (bf16)a[1]; f[2] = (bf16)a[2]; f[3] = (bf16)a[3];
    }
    if (2 * m + 1 < ntiles) {
        const floatx4 b = acc[2 * m + 1];
        f[4] = (bf16)b[0]; f[5] = (bf16)b[1]; f[6] = (bf16)b[2]; f[7] = (bf16)b[3];
    }
    return f;
}
template <>
__device__ __forceinline__ float acc_perm<float>(const floatx4* acc, int m, int ntiles) {
    return (m >> 2) < ntiles ? acc[m >> 2][m & 3] : 0.0f;
}

}  // namespace gdn
