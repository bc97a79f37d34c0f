// The diagonal-tile comparison: the chunked prefill in 16-token windows with
// the intra-window ("diagonal tile") pair terms formed in one of two ways.
//
// Inside a window with start state S and local cumulative log-decay
// G_t = sum_{r<=t} g_r (per key channel), the outputs and the next state are
//   KK_ts = sum_i k_ti k_si e^{G_ti - G_si}  (s < t),   P_ts = sum_i q_ti k_si e^{G_ti - G_si}  (s <= t)
//   M = (I + diag(b) KK)^-1,   U = M diag(b) (V - K0 S),   O = Q0 S + P U,
//   S <- diag(e^{G_15}) S + Kd^T U
// with K0 = k e^G, Q0 = q e^G, Kd = k e^{G_15 - G}: every factor of those is
// at most 1 for any g <= 0, so the state side is safe whatever the gate.
// The pair terms are where the pages place the difficulty ("How to Think
// About Trillion-Parameter Sparse Multimodal LLMs", section 3; "What a
// Trillion-Parameter MoE Model Reveals About the Next Stage of LLM Scaling",
// section 3.2; "Architecture Evolution and Training Engineering for
// Trillion-Scale Sparse Multimodal Models", section 3.1): written as a dense
// product, e^{G_t - G_s} must be split into a row factor and a column factor,
// one of them a reciprocal of a cumulative decay.
//  - DENSE (PAIRS = false): the split with the window's middle token as
//    reference, k~ = k e^{G-m}, q~ = q e^{G-m}, k^ = k e^{m-G}, and
//    KK = k~ k^T, P = q~ k^T as matrix-core products.  With g >= -5 every factor
//    lies in [e^-40, e^40] (the 16-token bound of "Trillion-Parameter MoE
//    Multimodal LLMs: How to Evaluate the New Generation", section 3.1); with
//    an unbounded gate it overflows.
//  - PAIRS (PAIRS = true): each (t, s) pair's decay e^{G_t - G_s} <= 1 formed
//    channel by channel on the vector units, the explicit position-pair path
//    that an unbounded (negative-softplus) gate forces; valid for any finite
//    g <= 0.
// Everything else is shared, so the time difference between the two is the
// cost of the position-pair path.  One workgroup per (sequence, head), d_v/16
// waves, wave w owning state columns [16w, 16w + 16) in fp32 registers.
#include "gdn_tiles.h"
#include "gdn_tile16.h"

namespace gdn {
namespace {

using namespace t16;

template <typename TI>
struct TArgs {
    const TI* q;
    const TI* k;
    const TI* v;
    const float* g;
    const float* beta;
    const int32_t* cu;
    const float* S0;  // may be null (zero)
    float* Sf;        // may be null
    TI* o;
    int H;
};

constexpr int NPAIR = 136;  // (t, s) with s <= t < 16

template <typename TI, int DK, int DV, bool PAIRS>
struct TCfg {
    typedef Mma<TI> M;
    static constexpr bool STAGE = sizeof(TI) == 2;
    static constexpr int NW = DV / 16, NT = 64 * NW, ES = (int)sizeof(TI);
    static constexpr int KSTEP = M::KSTEP, KW = M::KW, KM = DK / KSTEP, RT = DK / 16;
    static constexpr int SK = DK + 16 / ES;
    static constexpr int B_NK = CB * SK * ES, B_TK = DK * CB * ES;
    static constexpr int NSPLIT = 4, CC = DK / NSPLIT;  // pair path: channel quarters
    static constexpr int OFF_K0 = 0;                        // k e^G natural [16][SK]
    static constexpr int OFF_Q0 = OFF_K0 + B_NK;            // q e^G natural
    static constexpr int OFF_KDT = OFF_Q0 + B_NK;           // (k e^{G_15 - G})^T [DK][16]
    static constexpr int OFF_KW = OFF_KDT + B_TK;           // DENSE: k~ natural;  PAIRS: k natural
    static constexpr int OFF_QW = OFF_KW + B_NK;            // DENSE: q~ natural;  PAIRS: q natural
    static constexpr int OFF_HW = OFF_QW + B_NK;            // DENSE: k^ natural
    static constexpr int OFF_G = OFF_HW + (PAIRS ? 0 : B_NK);  // G (log2) [16][DK] fp32
    static constexpr int OFF_ML = OFF_G + CB * DK * 4;      // m (log2) [DK]
    static constexpr int OFF_GAM = OFF_ML + DK * 4;         // e^{G_15} [DK]
    static constexpr int OFF_BETA = OFF_GAM + DK * 4;       // beta [16]
    static constexpr int OFF_KK = OFF_BETA + CB * 4;        // KK [16][16] (PAIRS), then -diag(b) KK
    static constexpr int OFF_PP = OFF_KK + 256 * 4;         // P [16][16] row-major (PAIRS)
    static constexpr int OFF_PA = OFF_PP + 256 * 4;         // P by lane, A layout (DENSE)
    static constexpr int OFF_MI = OFF_PA + 256 * 4;         // M [16][16]
    static constexpr int OFF_PART = OFF_MI + 256 * 4;       // pair-path partial sums [NSPLIT][NPAIR][2]
    static constexpr int OFF_STG = OFF_PART + (PAIRS ? NSPLIT * NPAIR * 2 * 4 : 0);
    static constexpr int ST_G = OFF_STG;                    // staging: g [16][DK] fp32
    static constexpr int ST_K = ST_G + CB * DK * 4;         // k [16][DK]
    static constexpr int ST_Q = ST_K + CB * DK * ES;        // q [16][DK]
    static constexpr int ST_V = ST_Q + CB * DK * ES;        // v [16][DV]
    static constexpr int ST_B = ST_V + CB * DV * ES;        // beta [64]
    static constexpr int LDS = STAGE ? ST_B + 256 : OFF_STG;
    static_assert(B_NK % 16 == 0 && B_TK % 16 == 0 && LDS <= 160 * 1024, "LDS");
};

template <typename TI, int DK, int DV, bool PAIRS>
__device__ __forceinline__ void dma_window(const TArgs<TI>& a, char* smem, int h, int64_t t0, int L, int w,
                                           int lane) {
    typedef TCfg<TI, DK, DV, PAIRS> P;
    const int H = a.H;
    const size_t row0 = (size_t)t0 * H + h;
    dma_rows<DK * 4, CB, P::NW>(a.g + row0 * DK, (size_t)H * DK * 4, L, smem + P::ST_G, w, lane);
    dma_rows<DK * P::ES, CB, P::NW>(a.k + row0 * DK, (size_t)H * DK * P::ES, L, smem + P::ST_K, w, lane);
    dma_rows<DK * P::ES, CB, P::NW>(a.q + row0 * DK, (size_t)H * DK * P::ES, L, smem + P::ST_Q, w, lane);
    dma_rows<DV * P::ES, CB, P::NW>(a.v + row0 * DV, (size_t)H * DV * P::ES, L, smem + P::ST_V, w, lane);
    if (w == P::NW - 1)
        __builtin_amdgcn_global_load_lds(as_global(a.beta + row0 + (size_t)min(lane, L - 1) * H),
                                         as_lds(smem + P::ST_B), 4, 0, 0);
}

template <typename TI, int DK, int DV, bool PAIRS>
__global__ __launch_bounds__(DV * 4, 1) void tile_prefill_kernel(TArgs<TI> a) {
    typedef TCfg<TI, DK, DV, PAIRS> P;
    typedef Mma<TI> M;
    typedef K16<TI> K;
    typedef typename Two<TI>::type T2;
    typedef typename Four<TI>::type T4;
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    const int tid0 = threadIdx.x, g0 = (tid0 & 63) >> 4, r0 = tid0 & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int H = a.H;
    const int n = blockIdx.x / H, h = blockIdx.x - n * H;
    const int64_t tb = a.cu[n], te = a.cu[n + 1];
    const int col0 = 16 * w;
    TI* sK0 = reinterpret_cast<TI*>(smem + P::OFF_K0);
    TI* sQ0 = reinterpret_cast<TI*>(smem + P::OFF_Q0);
    TI* sKDT = reinterpret_cast<TI*>(smem + P::OFF_KDT);
    TI* sKW = reinterpret_cast<TI*>(smem + P::OFF_KW);
    TI* sQW = reinterpret_cast<TI*>(smem + P::OFF_QW);
    TI* sHW = reinterpret_cast<TI*>(smem + P::OFF_HW);
    float* sG = reinterpret_cast<float*>(smem + P::OFF_G);
    float* sML = reinterpret_cast<float*>(smem + P::OFF_ML);
    float* sGAM = reinterpret_cast<float*>(smem + P::OFF_GAM);
    float* sBETA = reinterpret_cast<float*>(smem + P::OFF_BETA);
    float* sKK = reinterpret_cast<float*>(smem + P::OFF_KK);
    float* sPP = reinterpret_cast<float*>(smem + P::OFF_PP);
    float* sPA = reinterpret_cast<float*>(smem + P::OFF_PA);
    float* sMI = reinterpret_cast<float*>(smem + P::OFF_MI);
    float* sPART = reinterpret_cast<float*>(smem + P::OFF_PART);
    const float* stg_g = reinterpret_cast<const float*>(smem + P::ST_G);
    const TI* stg_k = reinterpret_cast<const TI*>(smem + P::ST_K);
    const TI* stg_q = reinterpret_cast<const TI*>(smem + P::ST_Q);
    const TI* stg_v = reinterpret_cast<const TI*>(smem + P::ST_V);
    const float* stg_b = reinterpret_cast<const float*>(smem + P::ST_B);

    floatx4 S[P::RT];  // S[rt][i] = S[16 rt + 4g + i][col0 + r]
    const float* s0 = a.S0 ? a.S0 + (size_t)blockIdx.x * DK * DV : nullptr;
#pragma unroll
    for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[rt][i] = s0 ? s0[(16 * rt + 4 * g0 + i) * DV + col0 + r0] : 0.f;

    if constexpr (P::STAGE)
        if (te > tb) dma_window<TI, DK, DV, PAIRS>(a, smem, h, tb, (int)(te - tb < CB ? te - tb : CB), w, tid0 & 63);
    for (int64_t t0 = tb; t0 < te; t0 += CB) {
        const int L = (int)(te - t0 < CB ? te - t0 : CB);
        const size_t row0 = (size_t)t0 * H + h;
        // lane-derived values are recomputed every iteration (opaque to the
        // compiler), so addresses built from them are not hoisted out of the
        // loop and held in registers for its whole length
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
        auto clampt = [&](int t) { return t < L ? t : L - 1; };
        if constexpr (P::STAGE) __builtin_amdgcn_s_waitcnt(0);  // this wave's copy of the window has landed
        lds_barrier();  // ... and every wave's; the previous window is done with LDS

        // 1. cumulative log-decay (log2 units), the window reference, beta
        if (tid < DK) {
            float x[CB];
#pragma unroll
            for (int t = 0; t < CB; ++t) {
                if constexpr (P::STAGE) x[t] = stg_g[t * DK + tid];
                else x[t] = a.g[(row0 + (size_t)clampt(t) * H) * DK + tid];
            }
            float G = 0.f, m = 0.f;
#pragma unroll
            for (int t = 0; t < CB; ++t) {
                G = __builtin_fmaf(t < L ? x[t] : 0.f, LOG2E_B, G);
                sG[t * DK + tid] = G;
                if (t == 7) m = G;
            }
            sML[tid] = m;
            sGAM[tid] = __builtin_amdgcn_exp2f(G);
        }
        if (tid >= DK && tid < DK + CB) {
            const int t = tid - DK;
            float b;
            if constexpr (P::STAGE) b = stg_b[t];
            else b = a.beta[row0 + (size_t)clampt(t) * H];
            sBETA[t] = t < L ? b : 0.f;
        }
        floatx4 vv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * g + i;
            float x;
            if constexpr (P::STAGE) x = to_f32(stg_v[t * DV + col0 + r]);
            else x = to_f32(a.v[(row0 + (size_t)clampt(t) * H) * DV + col0 + r]);
            vv[i] = t < L ? x : 0.f;
        }
        lds_barrier();

        // 2. operands, per (token pair, channel pair)
#pragma unroll
        for (int i0 = 0; i0 < 4 * DK; i0 += P::NT) {
            const int i = i0 + tid;
            if ((4 * DK) % P::NT != 0 && i >= 4 * DK) break;
            const int cp = i % (DK / 2), tp = i / (DK / 2), c0 = 2 * cp;
            const floatx2 G15 = *reinterpret_cast<const floatx2*>(sG + 15 * DK + c0);  // rows past L repeat G_{L-1}
            const floatx2 ml = *reinterpret_cast<const floatx2*>(sML + c0);
            floatx2 kd[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = 2 * tp + u;
                floatx2 kk2, qq2;
                if constexpr (P::STAGE) {
                    kk2 = Two<TI>::f(*reinterpret_cast<const T2*>(stg_k + t * DK + c0));
                    qq2 = Two<TI>::f(*reinterpret_cast<const T2*>(stg_q + t * DK + c0));
                } else {
                    const size_t off = (row0 + (size_t)clampt(t) * H) * DK + c0;
                    kk2 = Two<TI>::f(*reinterpret_cast<const T2*>(a.k + off));
                    qq2 = Two<TI>::f(*reinterpret_cast<const T2*>(a.q + off));
                }
                if (t >= L) kk2 = qq2 = floatx2{0.f, 0.f};
                const floatx2 G = *reinterpret_cast<const floatx2*>(sG + t * DK + c0);
                const floatx2 e0 = exp2v(G);
                *reinterpret_cast<T2*>(sK0 + t * P::SK + c0) = Two<TI>::t(kk2 * e0);
                *reinterpret_cast<T2*>(sQ0 + t * P::SK + c0) = Two<TI>::t(qq2 * e0);
                kd[u] = kk2 * exp2v(G15 - G);  // e^{G_15 - G} <= 1
                if constexpr (PAIRS) {
                    *reinterpret_cast<T2*>(sKW + t * P::SK + c0) = Two<TI>::t(kk2);
                    *reinterpret_cast<T2*>(sQW + t * P::SK + c0) = Two<TI>::t(qq2);
                } else {
                    const floatx2 e = exp2v(G - ml), ei = exp2v(ml - G);
                    *reinterpret_cast<T2*>(sKW + t * P::SK + c0) = Two<TI>::t(kk2 * e);
                    *reinterpret_cast<T2*>(sQW + t * P::SK + c0) = Two<TI>::t(qq2 * e);
                    *reinterpret_cast<T2*>(sHW + t * P::SK + c0) = Two<TI>::t(kk2 * ei);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
                *reinterpret_cast<T2*>(sKDT + (c0 + j) * CB + 2 * tp) = Two<TI>::t(floatx2{kd[0][j], kd[1][j]});
        }
        lds_barrier();
        if constexpr (P::STAGE) {
            const int64_t t1 = t0 + CB;
            if (t1 < te) dma_window<TI, DK, DV, PAIRS>(a, smem, h, t1, (int)(te - t1 < CB ? te - t1 : CB), w, lane);
        }

        // 3. the pair terms KK (strictly lower) and P (lower)
        if constexpr (PAIRS) {
            // item (pair p, channel quarter cq): t = the row of p, s its column
            for (int it = tid; it < NPAIR * P::NSPLIT; it += P::NT) {
                const int p = it % NPAIR, cq = it / NPAIR;
                int t = 0;
                while ((t + 1) * (t + 2) / 2 <= p) ++t;
                const int s = p - t * (t + 1) / 2;
                float kk = 0.f, pp = 0.f;
#pragma unroll 2
                for (int c = cq * P::CC; c < (cq + 1) * P::CC; c += 4) {
                    const floatx4 Gt = *reinterpret_cast<const floatx4*>(sG + t * DK + c);
                    const floatx4 Gs = *reinterpret_cast<const floatx4*>(sG + s * DK + c);
                    const floatx4 kt = Four<TI>::f(*reinterpret_cast<const T4*>(sKW + t * P::SK + c));
                    const floatx4 ks = Four<TI>::f(*reinterpret_cast<const T4*>(sKW + s * P::SK + c));
                    const floatx4 qt = Four<TI>::f(*reinterpret_cast<const T4*>(sQW + t * P::SK + c));
                    const floatx4 e = exp2v(Gt - Gs);  // e^{G_t - G_s} <= 1
                    const floatx4 ke = ks * e;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        kk = __builtin_fmaf(kt[j], ke[j], kk);
                        pp = __builtin_fmaf(qt[j], ke[j], pp);
                    }
                }
                sPART[(cq * NPAIR + p) * 2] = kk;
                sPART[(cq * NPAIR + p) * 2 + 1] = pp;
            }
            lds_barrier();
            if (tid < 256) {
                const int t = tid >> 4, s = tid & 15;
                float kk = 0.f, pp = 0.f;
                if (s <= t) {
                    const int p = t * (t + 1) / 2 + s;
#pragma unroll
                    for (int cq = 0; cq < P::NSPLIT; ++cq) {
                        kk += sPART[(cq * NPAIR + p) * 2];
                        pp += sPART[(cq * NPAIR + p) * 2 + 1];
                    }
                }
                sKK[tid] = s < t ? kk : 0.f;
                sPP[tid] = pp;
            }
            lds_barrier();
        }
        if (w == 0) {
            // -diag(b) KK, row r, then M = (I + diag(b) KK)^-1
            floatx4 kk = zero4();
            if constexpr (!PAIRS) {
                // lane r + 16g: KK[t = r][s = 4g + i]
#pragma unroll
                for (int mm = 0; mm < P::KM; ++mm)
                    kk = M::mma(lds_nat(sHW + r * P::SK, mm, g), lds_nat(sKW + r * P::SK, mm, g), kk);
                *reinterpret_cast<floatx4*>(sKK + r * 16 + 4 * g) = kk;
            }
            const float bt = sBETA[r];
            float nr[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const floatx4 x = *reinterpret_cast<const floatx4*>(sKK + r * 16 + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) nr[4 * q4 + e] = 4 * q4 + e < r ? -bt * x[e] : 0.f;
            }
            const floatx4 mi = unit_lower_inverse16(nr, r, g);
            *reinterpret_cast<floatx4*>(sMI + r * 16 + 4 * g) = mi;
        }
        if constexpr (!PAIRS) {
            if (w == 1) {
                // lane r + 16g: P[t = r][s = 4g + i], s <= t
                floatx4 pa = zero4();
#pragma unroll
                for (int mm = 0; mm < P::KM; ++mm)
                    pa = M::mma(lds_nat(sHW + r * P::SK, mm, g), lds_nat(sQW + r * P::SK, mm, g), pa);
#pragma unroll
                for (int e = 0; e < 4; ++e) pa[e] = 4 * g + e <= r ? pa[e] : 0.f;
                *reinterpret_cast<floatx4*>(sPA + 4 * lane) = pa;
            }
        }

        // 4. state side (own columns): K0 S and Q0 S
        floatx4 ks = zero4(), qs = zero4();
#pragma unroll
        for (int mm = 0; mm < P::KM; ++mm) {
            const typename M::frag bs = acc_perm<TI>(S, mm, P::RT);
            ks = M::mma(lds_perm(sK0 + r * P::SK, mm, g), bs, ks);
            qs = M::mma(lds_perm(sQ0 + r * P::SK, mm, g), bs, qs);
        }
        floatx4 br;
#pragma unroll
        for (int i = 0; i < 4; ++i) br[i] = sBETA[4 * g + i] * (vv[i] - ks[i]);
        lds_barrier();  // M and P are ready
        // U = M diag(b) (V - K0 S);  O = Q0 S + P U;  S <- e^{G_15} S + Kd^T U
        const floatx4 U = K::mma(K::cvt(*reinterpret_cast<const floatx4*>(sMI + r * 16 + 4 * g)), K::cvt(br), zero4());
        const typename K::frag bu = K::cvt(U);
        floatx4 pa;
        if constexpr (PAIRS) {
            // lane r + 16g: P[t = r][s = 4g + i]
            pa = *reinterpret_cast<const floatx4*>(sPP + r * 16 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) pa[e] = 4 * g + e <= r ? pa[e] : 0.f;
        } else {
            pa = *reinterpret_cast<const floatx4*>(sPA + 4 * lane);
        }
        const floatx4 O = K::mma(K::cvt(pa), bu, qs);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * g + i;
            if (t < L) a.o[(row0 + (size_t)t * H) * DV + col0 + r] = from_f32<TI>(O[i]);
        }
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt) {
            const floatx4 d = K::mma(K::load(sKDT + (16 * rt + r) * CB + 4 * g), bu, zero4());
            const floatx4 gm = *reinterpret_cast<const floatx4*>(sGAM + 16 * rt + 4 * g);
            S[rt] = gm * S[rt] + d;
        }
    }
    if (a.Sf) {
        float* dst = a.Sf + (size_t)blockIdx.x * DK * DV;
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(16 * rt + 4 * g0 + i) * DV + col0 + r0] = S[rt][i];
    }
}

template <typename TI, int DK, int DV>
hipError_t run_tiles(const TilesLaunch& p, hipStream_t s) {
    TArgs<TI> a;
    a.q = static_cast<const TI*>(p.q);
    a.k = static_cast<const TI*>(p.k);
    a.v = static_cast<const TI*>(p.v);
    a.g = p.g;
    a.beta = p.beta;
    a.cu = p.cu_seqlens;
    a.S0 = p.initial_state;
    a.Sf = p.final_state;
    a.o = static_cast<TI*>(p.o);
    a.H = p.H;
    const unsigned blocks = (unsigned)((int64_t)p.num_seqs * p.H);
    if (p.pairs)
        hipLaunchKernelGGL((tile_prefill_kernel<TI, DK, DV, true>), dim3(blocks), dim3(DV * 4), 0, s, a);
    else
        hipLaunchKernelGGL((tile_prefill_kernel<TI, DK, DV, false>), dim3(blocks), dim3(DV * 4), 0, s, a);
    return hipGetLastError();
}

template <typename TI>
hipError_t run_tiles_t(const TilesLaunch& p, hipStream_t s) {
    if (p.dk == 128 && p.dv == 128) return run_tiles<TI, 128, 128>(p, s);
    if (p.dk == 128 && p.dv == 64) return run_tiles<TI, 128, 64>(p, s);
    if (p.dk == 64 && p.dv == 128) return run_tiles<TI, 64, 128>(p, s);
    return run_tiles<TI, 64, 64>(p, s);
}

}  // namespace

hipError_t launch_tiles(const TilesLaunch& p, hipStream_t s) {
    if (p.num_seqs == 0) return hipSuccess;
    return p.bf16 ? run_tiles_t<bf16>(p, s) : run_tiles_t<float>(p, s);
}

}  // namespace gdn
