// One decode step of the gated delta rule: one token per sequence, fp32 state
// [N, H, d_k, d_v] updated in place.  Per (sequence, head):
//
//     S' = diag(exp(g)) S           decay first
//     r  = S'^T k                   what the decayed state returns for k
//     u  = beta (v - r)             correct-on-write
//     S  = S' + k u^T
//     o  = S^T q = S'^T q + (k . q) u
//
// (the recurrent form of "How to Think About Trillion-Parameter Sparse
// Multimodal LLMs", section 2.2: a fixed-size state updated token by token).
//
// The step reads and writes the 64 KiB state once and does ~7 d_k d_v flops, so
// it is bound by HBM.  One workgroup of NTHR threads owns one (sequence, head):
// a thread holds 4 adjacent columns (one 16-byte vector per row) of a band of
// rows, so every row of S is read and written as whole 512-byte segments.  The
// two reductions over d_k (S'^T k and S'^T q) are summed in registers over the
// thread's rows and then across row bands through LDS.  The state is touched
// once per step, so it is read and written with non-temporal hints (it does not
// displace the small per-token vectors from the caches); few rows per thread
// and many threads keep more requests in flight per CU.
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

template <typename T>
__device__ __forceinline__ floatx4 load4(const T* p);
template <>
__device__ __forceinline__ floatx4 load4<float>(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
template <>
__device__ __forceinline__ floatx4 load4<bf16>(const bf16* p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return floatx4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
template <typename T>
__device__ __forceinline__ void store4(T* p, floatx4 x);
template <>
__device__ __forceinline__ void store4<float>(float* p, floatx4 x) { *reinterpret_cast<floatx4*>(p) = x; }
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, floatx4 x) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}

constexpr int NTHR = 256;

template <typename TI, int DK, int DV>
__global__ __launch_bounds__(NTHR) void decode_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                                                    const TI* __restrict__ v, const float* __restrict__ g,
                                                    const float* __restrict__ beta, float* __restrict__ state,
                                                    TI* __restrict__ o, const bf16* __restrict__ z, int gate,
                                                    float gate_param) {
    constexpr int CG = DV / 4;     // 4-column groups per row
    constexpr int RG = NTHR / CG;  // row bands
    constexpr int RPB = DK / RG;   // rows per band
    static_assert(RPB >= 1 && RG * CG == NTHR, "unsupported shape");

    __shared__ float s_a[DK], s_k[DK], s_q[DK];
    __shared__ floatx4 s_r[RG][CG], s_p[RG][CG];
    __shared__ float s_kq;

    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;  // sequence * H + head
    if (tid < DK) {
        // decay factor: e^g (per channel or per head), or from the gate logit
        s_a[tid] = gate == GATE_LOG    ? __expf(g[unit * DK + tid])
                   : gate == GATE_HEAD ? __expf(g[unit])  // one gate per (sequence, head)
                                       : gate_alpha((float)z[unit * DK + tid], gate, gate_param);
        s_k[tid] = to_f32(k[unit * DK + tid]);
        s_q[tid] = to_f32(q[unit * DK + tid]);
    }
    __syncthreads();
    if (tid < kWave) {
        float kq = 0.f;
        for (int i = tid; i < DK; i += kWave) kq += s_k[i] * s_q[i];
        for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
        if (tid == 0) s_kq = kq;
    }

    const int cg = tid % CG, rb = tid / CG;
    float* S = state + unit * (int64_t)DK * DV + 4 * cg;
    floatx4 Sv[RPB];
#pragma unroll
    for (int j = 0; j < RPB; ++j)
        Sv[j] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(S + (int64_t)(rb * RPB + j) * DV));
    floatx4 r = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RPB; ++j) {
        const int i = rb * RPB + j;
        Sv[j] *= s_a[i];
        r += Sv[j] * s_k[i];
        p += Sv[j] * s_q[i];
    }
    s_r[rb][cg] = r;
    s_p[rb][cg] = p;
    __syncthreads();
    floatx4 rt = {0.f, 0.f, 0.f, 0.f}, pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < RG; ++b) {
        rt += s_r[b][cg];
        pt += s_p[b][cg];
    }
    const floatx4 vv = load4(v + unit * DV + 4 * cg);
    const floatx4 u = beta[unit] * (vv - rt);
#pragma unroll
    for (int j = 0; j < RPB; ++j) {
        const int i = rb * RPB + j;
        __builtin_nontemporal_store(Sv[j] + s_k[i] * u, reinterpret_cast<floatx4*>(S + (int64_t)i * DV));
    }
    if (rb == 0) store4(o + unit * DV + 4 * cg, pt + s_kq * u);
}

template <typename TI, int DK, int DV>
hipError_t run(const DecodeLaunch& p, hipStream_t s) {
    const int64_t units = (int64_t)p.N * p.H;
    hipLaunchKernelGGL((decode_kernel<TI, DK, DV>), dim3((unsigned)units), dim3(NTHR), 0, s,
                       static_cast<const TI*>(p.q), static_cast<const TI*>(p.k), static_cast<const TI*>(p.v), p.g,
                       p.beta, p.state, static_cast<TI*>(p.o), static_cast<const bf16*>(p.z), p.gate,
                       p.gate_param);
    return hipGetLastError();
}

template <typename TI>
hipError_t run_t(const DecodeLaunch& p, hipStream_t s) {
    if (p.dk == 128 && p.dv == 128) return run<TI, 128, 128>(p, s);
    if (p.dk == 128 && p.dv == 64) return run<TI, 128, 64>(p, s);
    if (p.dk == 64 && p.dv == 128) return run<TI, 64, 128>(p, s);
    if (p.dk == 64 && p.dv == 64) return run<TI, 64, 64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& p, hipStream_t s) {
    if ((int64_t)p.N * p.H == 0) return hipSuccess;
    return p.bf16 ? run_t<bf16>(p, s) : run_t<float>(p, s);
}

}  // namespace gdn
