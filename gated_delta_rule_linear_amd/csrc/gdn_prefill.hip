// Chunked prefill of the gated delta rule on gfx950.
//
// One workgroup (4 waves) owns one (sequence, head) and walks its 64-token
// chunks in order, carrying the fp32 state S (d_k x d_v) in registers: wave w
// owns state columns [w*dv/4, (w+1)*dv/4).  Per chunk of L <= 64 tokens:
//
//  1. Local cumulative log-decay G_t = sum_{r<=t} g_r (per key channel),
//     restarted at every chunk, so it never drifts towards underflow over a
//     long sequence (the cumulative decay factor of "Architecture Evolution
//     and Training Engineering for Trillion-Scale Sparse Multimodal Models",
//     section 3.2, taken per tile).
//  2. Decay-scaled operands in LDS.  The intra-chunk products need
//     exp(G_t - G_s) split into a row factor and a column factor; a column
//     factor is the reciprocal of a cumulative decay.  The argument of
//     "Trillion-Parameter MoE Multimodal LLMs: How to Evaluate the New
//     Generation", section 3.1, is that with g >= -5 a 16-token window keeps
//     both factors inside the normal fp32/bf16 range (e^-80 .. e^80).  Here:
//       - if every G of the chunk lies in [-40, 40], one reference point (the
//         chunk start) serves all 64 tokens: q~ = q e^G, k~ = k e^G,
//         k^ = k e^-G, and every factor is inside e^-40 .. e^40;
//       - otherwise each 16-token row block I uses its own reference m_I
//         (G at the block's middle row): row factors e^(G_t - m_I) and
//         column factors e^(m_I - G_s) stay inside e^-40 .. e^40 on the
//         diagonal block and are <= 1 off it.
//     Either way every causal tile, the diagonal ones included, is a dense
//     matrix-core product (section 3 of "How to Think About Trillion-Parameter
//     Sparse Multimodal LLMs").
//  3. Gram tiles on MFMA: A = strict_lower(diag(beta) K~ K^T), P = lower(Q~ K^T).
//  4. Unit lower-triangular solve (I + A) X = diag(beta) [K~ | V] by 16-row
//     blocks: the four 16x16 diagonal blocks are inverted by substitution in
//     fp32, the off-diagonal coupling runs on MFMA.  X = [W | Ut].
//  5. State pass on MFMA:  U = Ut - W S,  O = Q~ S + P U,
//     S <- diag(e^{G_L}) S + K_dec^T U  with K_dec = k e^{G_L - G}.
//
// This restates, chunk by chunk, the token recurrence
//   S_t = diag(a_t) S_{t-1} + b_t k_t (v_t - (diag(a_t) S_{t-1})^T k_t)^T, o_t = S_t^T q_t.
#include "gdn_kernels.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int C = 64;  // chunk length (tokens)

template <int A, int B>
struct cmax {
    static constexpr int value = A > B ? A : B;
};

template <typename TI, int DK, int DV>
struct Cfg {
    static constexpr int NT = 256, NW = 4;
    static constexpr int CPR = DK / 2;        // threads per token row in the load step
    static constexpr int NG = NT / CPR;       // token groups
    static constexpr int TPG = C / NG;        // tokens per group
    static constexpr int CW = DV / NW;        // state columns per wave
    static constexpr int NCT = CW / 16;       // 16-wide column tiles per wave
    static constexpr int KWC = DK / NW;       // K~ columns per wave in the solve
    static constexpr int NKT = KWC / 16;
    static constexpr int RT = DK / 16;        // 16-row tiles of the state
    static constexpr int PAD = 16 / (int)sizeof(TI);
    static constexpr int LDK = DK + PAD;      // Qs, Ks, Kh row stride (elements)
    static constexpr int LDV = DV + PAD;      // Vs
    static constexpr int LDT = C + PAD;       // KdT (d_k rows x 64 tokens)
    static constexpr int LDP = C + PAD;       // Ps
    static constexpr int LDA = C + 4;         // An (fp32)
    static constexpr int LDL = 16 + PAD;      // Ls (four 16x16 inverses)
    static constexpr int SZ_Q = C * LDK * (int)sizeof(TI);
    static constexpr int SZ_R3 = cmax<C * LDK * (int)sizeof(TI), C * LDA * 4>::value;
    // bf16 has LDS to spare, so K_dec^T gets its own region and is written while
    // the chunk is loaded; the fp32 variant reuses the v region after the solve.
    static constexpr bool KD_OWN = sizeof(TI) == 2;
    static constexpr int SZ_KD = DK * LDT * (int)sizeof(TI);
    static constexpr int SZ_R4 = KD_OWN ? C * LDV * (int)sizeof(TI) : cmax<C * LDV * (int)sizeof(TI), SZ_KD>::value;
    static constexpr int SZ_P = C * LDP * (int)sizeof(TI);
    static constexpr int SZ_L = 4 * 16 * LDL * (int)sizeof(TI);
    static constexpr int NF = C + DK + NG * DK + 4 * DK + 8;
    static constexpr int LDS = 2 * SZ_Q + SZ_R3 + SZ_R4 + (KD_OWN ? SZ_KD : 0) + SZ_P + SZ_L + NF * 4;
    static_assert(NCT >= 1 && NKT >= 1 && TPG >= 1, "unsupported shape");
};

template <typename TI>
struct Args {
    const TI* q;
    const TI* k;
    const TI* v;
    const float* g;
    const float* beta;
    const int32_t* cu;
    const float* S0;
    float* Sf;
    TI* o;
    int H;
};

template <typename T>
__device__ __forceinline__ floatx2 load2(const T* p);
template <>
__device__ __forceinline__ floatx2 load2<float>(const float* p) { return *reinterpret_cast<const floatx2*>(p); }
template <>
__device__ __forceinline__ floatx2 load2<bf16>(const bf16* p) {
    const bf16x2 x = *reinterpret_cast<const bf16x2*>(p);
    return floatx2{(float)x[0], (float)x[1]};
}
template <typename T>
__device__ __forceinline__ void store2(T* p, floatx2 x) {
    p[0] = from_f32<T>(x[0]);
    p[1] = from_f32<T>(x[1]);
}

__device__ __forceinline__ floatx2 exp2v(floatx2 x) { return floatx2{fast_exp(x[0]), fast_exp(x[1])}; }

__device__ __forceinline__ float wave_min(float x) {
    for (int off = 32; off > 0; off >>= 1) x = fminf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Row block I and column block J of the p-th tile of the lower triangle
// (0,0),(1,0),(1,1),(2,0),(2,1),(2,2),(3,0),(3,1),(3,2),(3,3).
__device__ __forceinline__ void tri_pair(int p, int& I, int& J) {
    I = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
    J = p - I * (I + 1) / 2;
}

template <typename TI, int DK, int DV>
__global__ __launch_bounds__(256, 1) void prefill_seq_kernel(Args<TI> a) {
    typedef Cfg<TI, DK, DV> P;
    typedef Mma<TI> M;
    typedef typename M::frag frag;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    TI* Qs = reinterpret_cast<TI*>(smem);
    TI* Ks = reinterpret_cast<TI*>(smem + P::SZ_Q);
    char* r3 = smem + 2 * P::SZ_Q;
    char* r4 = r3 + P::SZ_R3;
    char* r5 = r4 + P::SZ_R4;
    TI* Ps = reinterpret_cast<TI*>(r5 + (P::KD_OWN ? P::SZ_KD : 0));
    TI* Ls = reinterpret_cast<TI*>(reinterpret_cast<char*>(Ps) + P::SZ_P);
    float* fs = reinterpret_cast<float*>(reinterpret_cast<char*>(Ls) + P::SZ_L);
    TI* Kh = reinterpret_cast<TI*>(r3);      // k^ (Gram column operand) ...
    float* An = reinterpret_cast<float*>(r3);  // ... then -A (fp32)
    TI* Vs = reinterpret_cast<TI*>(r4);
    TI* KdT = reinterpret_cast<TI*>(P::KD_OWN ? r5 : r4);
    float* s_beta = fs;
    float* s_gam = s_beta + C;
    float* s_gtot = s_gam + DK;
    float* s_mid = s_gtot + P::NG * DK;
    float* s_red = s_mid + 4 * DK;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
    const int H = a.H;
    const int unit = blockIdx.x;
    const int n = unit / H, h = unit - n * H;
    const int64_t tb = a.cu[n], te = a.cu[n + 1];
    const int col0 = w * P::CW;
    const int kcol0 = w * P::KWC;
    const size_t sbase = (size_t)unit * DK * DV;

    // fp32 state: S[ct][rt][i] = S[16 rt + 4g + i][col0 + 16 ct + r]
    floatx4 S[P::NCT][P::RT];
#pragma unroll
    for (int ct = 0; ct < P::NCT; ++ct)
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[ct][rt][i] = a.S0 ? a.S0[sbase + (size_t)(16 * rt + 4 * g + i) * DV + col0 + 16 * ct + r] : 0.f;

    const int cp = tid % P::CPR, grp = tid / P::CPR, ch = 2 * cp;

    for (int64_t c0 = tb; c0 < te; c0 += C) {
        const int L = (int)(te - c0 < C ? te - c0 : C);

        // ---- 1. raw loads and the local cumulative log-decay ------------------
        floatx2 G[P::TPG], qv[P::TPG], kv[P::TPG];
#pragma unroll
        for (int tt = 0; tt < P::TPG; ++tt) {
            const int t = grp * P::TPG + tt;
            if (t < L) {
                const size_t off = ((size_t)(c0 + t) * H + h) * DK + ch;
                G[tt] = *reinterpret_cast<const floatx2*>(a.g + off);
                qv[tt] = load2(a.q + off);
                kv[tt] = load2(a.k + off);
            } else {
                G[tt] = floatx2{0.f, 0.f};
                qv[tt] = floatx2{0.f, 0.f};
                kv[tt] = floatx2{0.f, 0.f};
            }
        }
        {
            constexpr int per_row = DV * (int)sizeof(TI) / 16;
            for (int e = tid; e < C * per_row; e += P::NT) {
                const int t = e / per_row, part = e - t * per_row;
                floatx4 x = floatx4{0.f, 0.f, 0.f, 0.f};
                if (t < L)
                    x = *reinterpret_cast<const floatx4*>(a.v + ((size_t)(c0 + t) * H + h) * DV + part * (16 / sizeof(TI)));
                *reinterpret_cast<floatx4*>(Vs + t * P::LDV + part * (16 / sizeof(TI))) = x;
            }
        }
        if (tid < C) s_beta[tid] = tid < L ? a.beta[(size_t)(c0 + tid) * H + h] : 0.f;
        floatx2 run = floatx2{0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < P::TPG; ++tt) {
            run += G[tt];
            G[tt] = run;
        }
        s_gtot[grp * DK + ch] = run[0];
        s_gtot[grp * DK + ch + 1] = run[1];
        __syncthreads();
        floatx2 off = floatx2{0.f, 0.f}, tot = floatx2{0.f, 0.f};
#pragma unroll
        for (int gg = 0; gg < P::NG; ++gg) {
            const floatx2 x = floatx2{s_gtot[gg * DK + ch], s_gtot[gg * DK + ch + 1]};
            tot += x;
            if (gg < grp) off += x;
        }
        float gmin = 0.f, gmax = 0.f;
#pragma unroll
        for (int tt = 0; tt < P::TPG; ++tt) {
            G[tt] += off;
            gmin = fminf(gmin, fminf(G[tt][0], G[tt][1]));
            gmax = fmaxf(gmax, fmaxf(G[tt][0], G[tt][1]));
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if ((16 * I + 7) / P::TPG == grp) {
                s_mid[I * DK + ch] = G[(16 * I + 7) % P::TPG][0];
                s_mid[I * DK + ch + 1] = G[(16 * I + 7) % P::TPG][1];
            }
        }
        gmin = wave_min(gmin);
        gmax = wave_max(gmax);
        if (lane == 0) {
            s_red[w] = gmin;
            s_red[4 + w] = gmax;
        }
        const floatx2 gam = exp2v(tot);
        if (grp == 0) {
            s_gam[ch] = gam[0];
            s_gam[ch + 1] = gam[1];
        }
        __syncthreads();  // s_red, s_mid visible
        const bool fast = fminf(fminf(s_red[0], s_red[1]), fminf(s_red[2], s_red[3])) >= -40.f &&
                          fmaxf(fmaxf(s_red[4], s_red[5]), fmaxf(s_red[6], s_red[7])) <= 40.f;

        // ---- 2. decay-scaled operands --------------------------------------
        floatx2 kd[P::TPG];  // K_dec = k e^{G_L - G}, stored transposed
        if (fast) {
#pragma unroll
            for (int tt = 0; tt < P::TPG; ++tt) {
                const int t = grp * P::TPG + tt;
                const floatx2 e = exp2v(G[tt]), ei = exp2v(-G[tt]);
                store2(Qs + t * P::LDK + ch, qv[tt] * e);
                store2(Ks + t * P::LDK + ch, kv[tt] * e);
                store2(Kh + t * P::LDK + ch, kv[tt] * ei);
                kd[tt] = kv[tt] * ei * gam;
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < P::TPG; ++tt) {
                const int t = grp * P::TPG + tt;
                const floatx2 m = floatx2{s_mid[(t >> 4) * DK + ch], s_mid[(t >> 4) * DK + ch + 1]};
                const floatx2 e = exp2v(G[tt] - m);
                store2(Qs + t * P::LDK + ch, qv[tt] * e);
                store2(Ks + t * P::LDK + ch, kv[tt] * e);
                kd[tt] = kv[tt] * exp2v(tot - G[tt]);
            }
        }
        auto store_kd = [&]() {
#pragma unroll
            for (int tt = 0; tt < P::TPG; ++tt) {
                const int t = grp * P::TPG + tt;
                KdT[ch * P::LDT + t] = from_f32<TI>(kd[tt][0]);
                KdT[(ch + 1) * P::LDT + t] = from_f32<TI>(kd[tt][1]);
            }
        };
        if (P::KD_OWN) store_kd();

        // ---- 3. Gram tiles ---------------------------------------------------
        floatx4 accA[5];
        int aI[5], aJ[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            accA[j] = zero4();
            aI[j] = -1;
            aJ[j] = 0;
        }
        auto gram = [&](const TI* rows, int I, int J) {
            floatx4 acc = zero4();
            const TI* ra = rows + (16 * I + r) * P::LDK;
            const TI* rb = Kh + (16 * J + r) * P::LDK;
#pragma unroll
            for (int m = 0; m < DK / M::KSTEP; ++m) acc = M::mma(lds_nat(ra, m, g), lds_nat(rb, m, g), acc);
            return acc;
        };
        auto store_p = [&](const floatx4& acc, int I, int J) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * I + 4 * g + i, s = 16 * J + r;
                Ps[t * P::LDP + s] = from_f32<TI>(s <= t ? acc[i] : 0.f);
            }
        };
        if (fast) {
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const int p = w + 4 * j;
                int I, J;
                tri_pair(p % 10, I, J);
                if (p < 10) {
                    accA[j] = gram(Ks, I, J);
                    aI[j] = I;
                    aJ[j] = J;
                } else {
                    store_p(gram(Qs, I, J), I, J);
                }
            }
            __syncthreads();  // all Gram reads of Kh done
        } else {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                __syncthreads();  // readers of the previous Kh are done
#pragma unroll
                for (int tt = 0; tt < P::TPG; ++tt) {
                    const int t = grp * P::TPG + tt;
                    if (t < 16 * (I + 1)) {
                        const floatx2 m = floatx2{s_mid[I * DK + ch], s_mid[I * DK + ch + 1]};
                        store2(Kh + t * P::LDK + ch, kv[tt] * exp2v(m - G[tt]));
                    }
                }
                __syncthreads();
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int qq = w + 4 * jj;
                    if (qq < 2 * (I + 1)) {
                        if (qq < I + 1) {
                            accA[I] = gram(Ks, I, qq);
                            aI[I] = I;
                            aJ[I] = qq;
                        } else {
                            store_p(gram(Qs, I, qq - I - 1), I, qq - I - 1);
                        }
                    }
                }
            }
            __syncthreads();  // all Gram reads of Qs/Ks/Kh done
            // the inter-chunk products use the chunk start as reference
#pragma unroll
            for (int tt = 0; tt < P::TPG; ++tt) {
                const int t = grp * P::TPG + tt;
                const floatx2 e = exp2v(G[tt]);
                store2(Qs + t * P::LDK + ch, qv[tt] * e);
                store2(Ks + t * P::LDK + ch, kv[tt] * e);
            }
        }
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            if (aI[j] >= 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * aI[j] + 4 * g + i, s = 16 * aJ[j] + r;
                    An[t * P::LDA + s] = s < t ? -s_beta[t] * accA[j][i] : 0.f;
                }
            }
        }
        __syncthreads();

        // ---- 4a. inverses of the four 16x16 diagonal blocks of (I + A) --------
        if (lane < 16) {
            const int c = lane;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = i == c ? 1.f : 0.f;
            const float* blk = An + (16 * w) * P::LDA + 16 * w;
#pragma unroll
            for (int j = 0; j < 16; ++j)
#pragma unroll
                for (int i = j + 1; i < 16; ++i) x[i] += blk[i * P::LDA + j] * x[j];
#pragma unroll
            for (int i = 0; i < 16; ++i) Ls[(16 * w + i) * P::LDL + c] = from_f32<TI>(x[i]);
        }
        __syncthreads();

        // ---- 4b. block forward substitution for X = [W | Ut] (own columns) ----
        constexpr int NX = P::NKT + P::NCT;
        floatx4 X[NX][4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int tile = 0; tile < NX; ++tile) {
                const bool isK = tile < P::NKT;
                const int cc = isK ? kcol0 + 16 * tile : col0 + 16 * (tile - P::NKT);
                floatx4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * I + 4 * g + i;
                    const TI x = isK ? Ks[t * P::LDK + cc + r] : Vs[t * P::LDV + cc + r];
                    acc[i] = s_beta[t] * to_f32(x);
                }
                if (I > 0) {
                    const float* arow = An + (16 * I + r) * P::LDA;
#pragma unroll
                    for (int m = 0; m < (16 * I + M::KSTEP - 1) / M::KSTEP; ++m)
                        acc = M::mma(lds_perm_f32<TI>(arow, m, g, 16 * I), acc_perm<TI>(X[tile], m, I), acc);
                }
                floatx4 xi = zero4();
                const TI* lrow = Ls + (16 * I + r) * P::LDL;
#pragma unroll
                for (int m = 0; m < (16 + M::KSTEP - 1) / M::KSTEP; ++m)
                    xi = M::mma(lds_perm(lrow, m, g, 16), acc_perm<TI>(&acc, m, 1), xi);
                X[tile][I] = xi;
            }
        }
        // -W into the own K~ columns of Ks (each wave only ever read its own)
#pragma unroll
        for (int tile = 0; tile < P::NKT; ++tile)
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Ks[(16 * I + 4 * g + i) * P::LDK + kcol0 + 16 * tile + r] = from_f32<TI>(-X[tile][I][i]);
        __syncthreads();  // Vs is free, -W complete
        if (!P::KD_OWN) {
            store_kd();
            __syncthreads();
        }

        // ---- 5. state pass (own columns) --------------------------------------
        floatx4 U[P::NCT][4], O[P::NCT][4];
#pragma unroll
        for (int ct = 0; ct < P::NCT; ++ct)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                U[ct][rb] = X[P::NKT + ct][rb];
                O[ct][rb] = zero4();
            }
        // U += (-W) S ; O += Q~ S
#pragma unroll
        for (int m = 0; m < DK / M::KSTEP; ++m) {
            frag bS[P::NCT];
#pragma unroll
            for (int ct = 0; ct < P::NCT; ++ct) bS[ct] = acc_perm<TI>(S[ct], m, P::RT);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const frag aw = lds_perm(Ks + (16 * rb + r) * P::LDK, m, g);
                const frag aq = lds_perm(Qs + (16 * rb + r) * P::LDK, m, g);
#pragma unroll
                for (int ct = 0; ct < P::NCT; ++ct) {
                    U[ct][rb] = M::mma(aw, bS[ct], U[ct][rb]);
                    O[ct][rb] = M::mma(aq, bS[ct], O[ct][rb]);
                }
            }
        }
        // S <- diag(e^{G_L}) S before the chunk's writes are added
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float d = s_gam[16 * rt + 4 * g + i];
#pragma unroll
                for (int ct = 0; ct < P::NCT; ++ct) S[ct][rt][i] *= d;
            }
        // O += P U ; S += K_dec^T U
#pragma unroll
        for (int m = 0; m < C / M::KSTEP; ++m) {
            frag bU[P::NCT];
#pragma unroll
            for (int ct = 0; ct < P::NCT; ++ct) bU[ct] = acc_perm<TI>(U[ct], m, 4);
            const int first_tile = (m * M::KW) / 4;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                if (first_tile <= rb) {
                    // blocks above the diagonal of P are never written: mask them
                    const frag ap = lds_perm(Ps + (16 * rb + r) * P::LDP, m, g, 16 * (rb + 1));
#pragma unroll
                    for (int ct = 0; ct < P::NCT; ++ct) O[ct][rb] = M::mma(ap, bU[ct], O[ct][rb]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < P::RT; ++rt) {
                const frag ak = lds_perm(KdT + (16 * rt + r) * P::LDT, m, g);
#pragma unroll
                for (int ct = 0; ct < P::NCT; ++ct) S[ct][rt] = M::mma(ak, bU[ct], S[ct][rt]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < P::NCT; ++ct)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * rb + 4 * g + i;
                    if (t < L) a.o[((size_t)(c0 + t) * H + h) * DV + col0 + 16 * ct + r] = from_f32<TI>(O[ct][rb][i]);
                }
        __syncthreads();  // LDS is rewritten by the next chunk
    }

    if (a.Sf) {
#pragma unroll
        for (int ct = 0; ct < P::NCT; ++ct)
#pragma unroll
            for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.Sf[sbase + (size_t)(16 * rt + 4 * g + i) * DV + col0 + 16 * ct + r] = S[ct][rt][i];
    }
}

template <typename TI, int DK, int DV>
hipError_t run(const PrefillLaunch& p, hipStream_t s) {
    typedef Cfg<TI, DK, DV> P;
    static_assert(P::LDS <= 160 * 1024, "LDS budget");
    auto kern = prefill_seq_kernel<TI, DK, DV>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, P::LDS);
    if (e != hipSuccess) return e;
    Args<TI> a;
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
    const int64_t units = (int64_t)p.num_seqs * p.H;
    hipLaunchKernelGGL(kern, dim3((unsigned)units), dim3(P::NT), P::LDS, s, a);
    return hipGetLastError();
}

template <typename TI>
hipError_t run_t(const PrefillLaunch& p, hipStream_t s) {
    if (p.dk == 128 && p.dv == 128) return run<TI, 128, 128>(p, s);
    if (p.dk == 128 && p.dv == 64) return run<TI, 128, 64>(p, s);
    if (p.dk == 64 && p.dv == 128) return run<TI, 64, 128>(p, s);
    if (p.dk == 64 && p.dv == 64) return run<TI, 64, 64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t s) {
    if ((int64_t)p.num_seqs * p.H == 0) return hipSuccess;
    return p.bf16 ? run_t<bf16>(p, s) : run_t<float>(p, s);
}

}  // namespace gdn
