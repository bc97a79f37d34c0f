// Helpers for kernels that walk a sequence in 16-token windows (the backward
// pass and the diagonal-tile comparison kernels): 16 x 16 matrix-core tiles
// over the window's tokens, DPP row reductions, LDS-only barriers and
// the LDS copy (DMA) of packed rows.
#pragma once

#include <type_traits>

#include "gdn_mfma.h"

namespace gdn {
namespace t16 {

constexpr int CB = 16;                           // tokens per sub-chunk
constexpr float LOG2E_B = 1.4426950408889634f;   // G is carried in log2 units

// Two fp32 values rounded to bf16 (to nearest even) in one 32-bit word, the
// first in the low half: one v_cvt_pk_bf16_f32.  (A bf16 vector built element
// by element that feeds a 16x16x16 matrix-core operand is compiled as single
// conversions joined by permutes.)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
}
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// Contractions over the 16 tokens of a sub-chunk.  Lane r + 16g supplies
// A[r][4g .. 4g+3] and B[4g .. 4g+3][r]: the register layout of a 16 x 16
// accumulator (lane r + 16g holds C[4g + i][r]) is such a B operand as it is,
// and the A operand of the transposed matrix.
template <typename TI>
struct K16;
template <>
struct K16<bf16> {
    typedef bf16x4 frag;
    __device__ __forceinline__ static frag cvt(floatx4 x) {
        return __builtin_bit_cast(bf16x4, u32x2v{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])});
    }
    __device__ __forceinline__ static frag load(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
    __device__ __forceinline__ static floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <>
struct K16<float> {
    typedef floatx4 frag;
    __device__ __forceinline__ static frag cvt(floatx4 x) { return x; }
    __device__ __forceinline__ static frag load(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
    // four 16x16x4 steps; step e pairs lane group g's element e, i.e. k = 4g + e
    __device__ __forceinline__ static floatx4 mma(frag a, frag b, floatx4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
};

template <typename T>
struct Two;
template <>
struct Two<bf16> {
    typedef bf16x2 type;
    __device__ __forceinline__ static floatx2 f(bf16x2 x) { return floatx2{(float)x[0], (float)x[1]}; }
    __device__ __forceinline__ static bf16x2 t(floatx2 x) { return __builtin_bit_cast(bf16x2, pk_bf16(x[0], x[1])); }
};
template <>
struct Two<float> {
    typedef floatx2 type;
    __device__ __forceinline__ static floatx2 f(floatx2 x) { return x; }
    __device__ __forceinline__ static floatx2 t(floatx2 x) { return x; }
};
template <typename T>
struct Four;
template <>
struct Four<bf16> {
    typedef bf16x4 type;
    __device__ __forceinline__ static floatx4 f(bf16x4 x) { return floatx4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]}; }
    __device__ __forceinline__ static bf16x4 t(floatx4 x) {
        return __builtin_bit_cast(bf16x4, u32x2v{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])});
    }
};
template <>
struct Four<float> {
    typedef floatx4 type;
    __device__ __forceinline__ static floatx4 f(floatx4 x) { return x; }
    __device__ __forceinline__ static floatx4 t(floatx4 x) { return x; }
};


__device__ __forceinline__ floatx4 exp2v(floatx4 x) {
    return floatx4{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]), __builtin_amdgcn_exp2f(x[2]),
                   __builtin_amdgcn_exp2f(x[3])};
}
__device__ __forceinline__ floatx2 exp2v(floatx2 x) {
    return floatx2{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1])};
}

// Cross-lane moves inside a 16-lane row (lanes 16g .. 16g+15) with DPP.
// row_newbcast:J: every lane reads lane J of its row; row_ror:N: lane i reads
// lane (i + N) mod 16; row_shl:N: lane i reads lane i + N, 0 past the row end.
template <int CTRL, bool ZERO>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, ZERO));
}
// Sum over the 16 lanes of a row; every lane of the row gets it.
__device__ __forceinline__ float sum16(float x) {
    x += dpp<0x128, false>(x);
    x += dpp<0x124, false>(x);
    x += dpp<0x122, false>(x);
    x += dpp<0x121, false>(x);
    return x;
}
// Suffix sum inside a row: lane r gets the sum over lanes r .. 15.
__device__ __forceinline__ float suffix16(float x) {
    x += dpp<0x101, true>(x);
    x += dpp<0x102, true>(x);
    x += dpp<0x104, true>(x);
    x += dpp<0x108, true>(x);
    return x;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Workgroup barrier for LDS traffic only: each wave waits for its own LDS
// operations, not for its outstanding global memory operations, so a copy
// into LDS issued earlier (global_load_lds) stays in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ const __attribute__((address_space(1))) void* as_global(const void* p) {
    return (const __attribute__((address_space(1))) void*)p;
}
__device__ __forceinline__ __attribute__((address_space(3))) void* as_lds(void* p) {
    return (__attribute__((address_space(3))) void*)p;
}

// DMA of ROWS rows of RB bytes (row t at src + t * stride, t clamped to
// L - 1) into LDS rows packed back to back at dst; one wave instruction moves
// 1 KiB, and wave w issues instructions w, w + NW, ...
// With SWZ the 16-byte pieces of each row are permuted, piece p of row t landing
// in slot p ^ (t mod LPR) (see swz_off): reads of one column down 16 rows, and
// of the same piece of 16 rows, then fall in different LDS banks.
template <int RB, int ROWS, int NW, bool SWZ = false>
__device__ __forceinline__ void dma_rows(const void* src, size_t stride, int L, char* dst, int w, int lane) {
    constexpr int LPR = RB / 16, RPI = 64 / LPR, NI = ROWS * RB / 1024;
    static_assert(RB % 16 == 0 && RB <= 1024 && (ROWS * RB) % 1024 == 0, "copy shape");
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += NW) {
        const int i = i0 + w;
        if (NI % NW == 0 || i < NI) {
            const int row = i * RPI + lane / LPR, t = min(row, L - 1);
            const int piece = SWZ ? (lane % LPR) ^ (row % LPR) : lane % LPR;
            __builtin_amdgcn_global_load_lds(
                as_global(static_cast<const char*>(src) + (size_t)t * stride + piece * 16),
                as_lds(dst + i * 1024), 16, 0, 0);
        }
    }
}
// Byte offset of element `col` of row `row` in a swizzled copy of rows of RB bytes (elements of ES bytes).
template <int RB, int ES>
__device__ __forceinline__ int swz_off(int row, int col) {
    constexpr int LPR = RB / 16, PER = 16 / ES;
    return row * RB + (((col / PER) ^ (row % LPR)) * 16) + (col % PER) * ES;
}

// Inverse of the unit lower-triangular 16 x 16 matrix I - N (N strictly lower)
// by forward substitution.  Lane r + 16g holds row r of N in nr[0..15] and
// returns M[r][4g .. 4g+3] of M = (I - N)^-1; row j of M is final once rows < j
// are applied, and is read from lane j of the row with a DPP broadcast.
// Step j updates the four columns with one v_fmac_f32 each whose first source
// is lane j of the row (DPP row_newbcast).  A DPP read of a register needs two
// wait states after a VALU write of it: each step starts with s_nop 1, so
// whatever the compiler places between steps (a copy of x included) cannot
// break that, and inside a step the four chains are independent.
template <int J>
__device__ __forceinline__ void fmac4_row_newbcast(float a, float& x0, float& x1, float& x2, float& x3) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
        : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3)
        : "v"(a), "n"(J));
}
__device__ __forceinline__ floatx4 unit_lower_inverse16(const float (&nr)[16], int r, int g) {
    float x0 = r == 4 * g ? 1.f : 0.f, x1 = r == 4 * g + 1 ? 1.f : 0.f;
    float x2 = r == 4 * g + 2 ? 1.f : 0.f, x3 = r == 4 * g + 3 ? 1.f : 0.f;
    static_for<0, 15>([&](auto jc) { fmac4_row_newbcast<decltype(jc)::value>(nr[jc], x0, x1, x2, x3); });
    return floatx4{x0, x1, x2, x3};
}

}  // namespace t16
}  // namespace gdn
