// Chunked prefill of the gated delta rule on gfx950.
//
// One workgroup owns one (sequence, head) and walks its 64-token chunks in
// order, carrying the fp32 state S (d_k x d_v) in registers.  The workgroup has
// d_v / 16 waves; wave w owns the 16 state columns [16w, 16w + 16).
// Per chunk of L <= 64 tokens:
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
//       - if the chunk's total log-decay is >= -40 on every channel, one
//         reference point (the chunk start) serves all 64 tokens:
//         q~ = q e^G, k~ = k e^G, k^ = k e^-G, all factors within e^+-40;
//       - otherwise each 16-token row block I uses its own reference m_I
//         (G at the block's middle row): row factors e^(G_t - m_I) and column
//         factors e^(m_I - G_s) stay within e^+-40 on the diagonal block and
//         are <= 1 off it.
//     Either way every causal tile, the diagonal ones included, is a dense
//     matrix-core product (section 3 of "How to Think About Trillion-Parameter
//     Sparse Multimodal LLMs").
//  3. Gram tiles on MFMA, computed transposed so that each result lands in
//     the register layout of the operand that consumes it:
//     A = strict_lower(diag(beta) K~ K^T) and P = lower(Q~ K^T).
//  4. Unit lower-triangular solve (I + A) X = diag(beta) [K~ | V] by 16-row
//     blocks.  Every wave inverts the four 16x16 diagonal blocks in registers
//     (forward substitution; row j is broadcast along each 16-lane row with
//     DPP), the off-diagonal coupling runs on MFMA.  X = [W | Ut].
//  5. State pass on MFMA:  U = Ut - W S,  O = Q~ S + P U,
//     S <- diag(e^{G_L}) S + K_dec^T U  with K_dec = k e^{G_L - G}.
//  With bf16 inputs the next chunk's raw inputs are copied by DMA
//  (global_load_lds, 16 bytes per lane) into an LDS staging area while steps
//  3-5 of the current chunk run, so the prefetch holds no registers.
//
// LDS holds every MFMA operand in "operand layout": for a matrix with rows in
// 16-row blocks and a contraction index k, the fragment (block, step m) is 64
// lanes x KW contiguous elements, lane r + 16g holding row r and the k values
// 16*(e/4) + 4g + e%4 for e = m*KW .. m*KW + KW-1 (see gdn_mfma.h).  Reading a
// fragment is one contiguous vector load per lane.
//
// Global memory is addressed from wave-uniform per-chunk bases with 32-bit
// byte offsets, so each access costs one VGPR.
//
// This restates, chunk by chunk, the token recurrence
//   S_t = diag(a_t) S_{t-1} + b_t k_t (v_t - (diag(a_t) S_{t-1})^T k_t)^T, o_t = S_t^T q_t.
#include <algorithm>
#include <memory>
#include <mutex>
#include <type_traits>
#include <vector>

#include "gdn_fold.h"
#include "gdn_kernels.h"
#include "gdn_mfma.h"
#include "gdn_segunit.h"

namespace gdn {
namespace {

constexpr int C = 64;  // chunk length (tokens)

template <int A, int B>
struct cmax {
    static constexpr int value = A > B ? A : B;
};

template <typename TI, int DK, int DV>
struct Cfg {
    typedef Mma<TI> M;
    static constexpr int NW = DV / 16;        // waves; wave w owns state columns 16w .. 16w+15
    static constexpr int NT = 64 * NW;
    static constexpr int KW = M::KW, KSTEP = M::KSTEP;
    static constexpr int CPR = DK / 2;        // threads per token row in the load step
    static constexpr int NG = NT / CPR;       // token groups
    static constexpr int TPG = C / NG;        // tokens per group
    static constexpr bool UG = CPR == 64;     // one token group per wave: token indices are wave-uniform
    static constexpr int RT = DK / 16;        // 16-row tiles of the state
    static constexpr int KM = DK / KSTEP;     // MFMA steps over d_k
    static constexpr int TM = C / KSTEP;      // MFMA steps over the chunk's tokens
    static constexpr int NPT = (20 + NW - 1) / NW;  // Gram tiles per wave (fast path)
    static constexpr int NQS = (8 + NW - 1) / NW;   // Gram tiles per wave and row block (sub-tile path)
    static constexpr bool STAGE = sizeof(TI) == 2;  // next chunk prefetched into LDS by DMA
    static constexpr int SG_G = C * DK * 4;                // staging: g [C][DK] fp32
    static constexpr int SG_Q = C * DK * (int)sizeof(TI);  // q, k [C][DK]
    static constexpr int SG_V = C * DV * (int)sizeof(TI);  // v [C][DV]
    static constexpr int SG_B = C * 4;                     // beta [C]
    static constexpr int SZ_STG = STAGE ? SG_G + 2 * SG_Q + SG_V + SG_B : 0;
    static constexpr int SZ_OPK = C * DK * (int)sizeof(TI);
    static constexpr int SZ_AN = 14 * 64 * 16;  // ten 16x16 fp32 blocks of -A, then the four diagonal inverses
    static constexpr int SZ_R3 = cmax<SZ_OPK, SZ_AN>::value;
    static constexpr int SZ_KD = DK * C * (int)sizeof(TI);
    static constexpr int SZ_P = C * C * (int)sizeof(TI);
    static constexpr int NF = C + DK + NG * DK + 4 * DK;
    // LDS layout: the MFMA operands first (inside the 64 KiB reach of a
    // ds_read/ds_write immediate offset from one base), then the small
    // per-chunk vectors, then the staging area.
    static constexpr int OFF_QO = 0, OFF_KO = SZ_OPK, OFF_R3 = 2 * SZ_OPK, OFF_KD = OFF_R3 + SZ_R3;
    static constexpr int OFF_P = OFF_KD + SZ_KD, OFF_F = OFF_P + SZ_P;
    static constexpr int OFF_STG = (OFF_F + NF * 4 + 1023) / 1024 * 1024;
    static constexpr int LDS = OFF_STG + SZ_STG;
    static_assert(TPG >= 1 && NT <= 1024, "unsupported shape");
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
    // Time split of long sequences (seg > 0): sequence n is cut into segments of
    // `seg` tokens (the last one shorter); nl[n] counts the non-last segments of
    // sequences 0 .. n-1.  Non-last segment k (head h) owns slot k*H + h of the
    // map areas: wsM holds its d_k x d_k transition M, wsN its offset N, which
    // the fold step then replaces by the state at the start of segment k+1.
    int num_seqs;
    int seg;
    const int32_t* nl;
    const int32_t* spl;  // the sequences with more than one segment (see seg_table_kernel)
    float* wsM;
    float* wsN;
    int m_blocks;       // map launches: blocks [0, m_blocks) compute M, the rest N
    int map_from;       // map launches: first segment of a sequence that gets a map (0 or 1)
    int phase;          // split output launches: 1 segment 0 only (one workgroup per (sequence, head),
                        // its end state to slot nl[n] when more segments follow); 2 the later segments (one
                        // workgroup per (non-last segment, head): the segment after it)
    int legacy;         // bf16: use the single-role kernel instead of the warp-specialised one
    // gate != GATE_LOG: g is not read; the log-decay comes from the bf16 logits
    // z in the same layout (warp-specialised kernel only)
    const bf16* z;
    int gate;
    float gate_param;
    // passes over whole sequences (seg == 0) and over first segments (phase 1):
    // workgroup b takes head b % H of sequence ord[b / H] (longest first), or
    // of sequence b / H when ord is null
    const int32_t* ord;
    // Transition pass for the backward (QH): q^_t = M_t^T q_t of the tokens of
    // every segment it takes goes to qh ([T, H, d_k]; M_t: the transition from
    // the segment's start through token t; the backward reads those of the
    // segments after the first), and workgroups from m_blocks on take the last
    // segment of the split sequences in spl, whose M goes to wsML (slot kk for
    // spl[kk])
    TI* qh;
    float* wsML;
    // Checkpoint pass for the backward (CKP): the units of seg_unit (ord, and
    // with the split pfx; seg as above), each started from S0 (its sequence's
    // initial state, or zero) or, for segment j >= 1 of sequence n, from slot
    // nl[n] + j - 1 of wsN; the start state of the unit's 16-token window c goes
    // to ck slot (cu[n] / 16 + n + (sb - cu[n]) / 16 + c, h) ([slot][H][d_k * d_v],
    // in column blocks: element (i, c) at ((c / 16) d_k + i) 16 + c % 16).
    const int32_t* pfx;
    TI* ck;
};

template <typename T>
struct Pair;
template <>
struct Pair<bf16> {
    typedef bf16x2 type;
};
template <>
struct Pair<float> {
    typedef floatx2 type;
};

__device__ __forceinline__ floatx2 to_f2(bf16x2 x) { return floatx2{(float)x[0], (float)x[1]}; }
__device__ __forceinline__ floatx2 to_f2(floatx2 x) { return x; }
// Cumulative log-decays are carried in log2 units (g * log2(e)), so every
// decay factor is one v_exp_f32 (2^x), negated arguments included.
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ floatx2 pow2v(floatx2 x) {
    return floatx2{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1])};
}
__device__ __forceinline__ floatx2 fma2(floatx2 a, float b, floatx2 c) {
    return floatx2{__builtin_fmaf(a[0], b, c[0]), __builtin_fmaf(a[1], b, c[1])};
}

// Element at a 32-bit byte offset from a wave-uniform base (one VGPR per access).
template <typename T>
__device__ __forceinline__ const T& at(const void* base, uint32_t byte_off) {
    return *reinterpret_cast<const T*>(static_cast<const char*>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ T& at_mut(void* base, uint32_t byte_off) {
    return *reinterpret_cast<T*>(static_cast<char*>(base) + byte_off);
}

// Operand layout with a bank swizzle: inside fragment (blk, m) the 16 slots of
// lane group g are permuted by r -> r ^ ((4g + m + blk) & 15).  A fragment read
// is still one slot per lane (a permutation), and the 16 slots that one token
// row occupies across the fragments of its block land in 16 different bank
// groups, so a wave storing a whole row does not conflict.
__device__ __forceinline__ int op_slot(int blk, int m, int r, int g) { return 16 * g + ((r ^ (4 * g + m + blk)) & 15); }
// Element offset of (row, k) in an operand-layout matrix with KM steps per 16-row block.
template <typename TI, int KM>
__device__ __forceinline__ int op_idx(int row, int k) {
    constexpr int KW = Mma<TI>::KW;
    const int ef = 4 * (k >> 4) + (k & 3);
    const int m = ef / KW, e = ef % KW, blk = row >> 4;
    return ((blk * KM + m) * 64 + op_slot(blk, m, row & 15, (k >> 2) & 3)) * KW + e;
}
// Stores columns (c, c+1) of one row (c even).
template <typename TI, int KM>
__device__ __forceinline__ void op_store2(TI* base, int row, int c, floatx2 x) {
    if constexpr (sizeof(TI) == 2) {
        *reinterpret_cast<bf16x2*>(base + op_idx<TI, KM>(row, c)) = bf16x2{(bf16)x[0], (bf16)x[1]};
    } else {
        base[op_idx<TI, KM>(row, c)] = x[0];
        base[op_idx<TI, KM>(row, c + 1)] = x[1];
    }
}
template <typename TI, int KM>
__device__ __forceinline__ typename Mma<TI>::frag op_frag(const TI* base, int blk, int m, int lane) {
    return reinterpret_cast<const typename Mma<TI>::frag*>(base)[(blk * KM + m) * 64 + op_slot(blk, m, lane & 15, lane >> 4)];
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Fourth word of a raw buffer resource on gfx9-family parts (32-bit data
// format, no swizzle); with stride 0, accesses at or past num_records bytes
// are dropped (stores) or return 0 (loads).
constexpr uint32_t BUFFER_RSRC_WORD3 = 0x00020000u;
typedef unsigned int u32x2 __attribute__((__vector_size__(8)));
typedef unsigned int u32x4 __attribute__((__vector_size__(16)));

// x[e] += a * x[e][lane J of this lane's 16-lane row], e = 0..3: four
// v_fmac_f32 whose first source is read through the DPP row_newbcast
// modifier.  A broadcast read needs two wait states after the VALU write of
// its register: consecutive calls leave three instructions between them, and
// row_inverse puts them before the first call.
template <int J>
__device__ __forceinline__ void fma4_row_bcast(float a, float& x0, float& x1, float& x2, float& x3) {
    asm volatile(
        "v_fmac_f32_dpp %0, %0, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
        : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3)
        : "v"(a), "n"(J));
}

// Inverse of the unit lower-triangular 16 x 16 matrix I - N, N strictly lower,
// by forward substitution.  Lane r + 16g holds row r of N in arow[0..15] and
// returns entries (r, 4g + e) of the inverse.  Row j of the inverse is final
// once rows < j have been applied, so step j broadcasts row j along the
// 16-lane row.
__device__ __forceinline__ floatx4 row_inverse(const float (&arow)[16], int r, int g) {
    float x0 = r == 4 * g ? 1.f : 0.f, x1 = r == 4 * g + 1 ? 1.f : 0.f;
    float x2 = r == 4 * g + 2 ? 1.f : 0.f, x3 = r == 4 * g + 3 ? 1.f : 0.f;
    asm volatile("s_nop 4" ::: "memory");  // wait states before the first broadcast read (and an EXEC write)
    static_for<0, 15>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        fma4_row_bcast<j>(arow[j], x0, x1, x2, x3);
    });
    return floatx4{x0, x1, x2, x3};
}

// Index of the lower-triangle block (I, J), J <= I, in row-major order.
__device__ __forceinline__ constexpr int tri_id(int I, int J) { return I * (I + 1) / 2 + J; }
__device__ __forceinline__ void tri_pair(int p, int& I, int& J) {
    I = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
    J = p - I * (I + 1) / 2;
}

__device__ __forceinline__ const __attribute__((address_space(1))) void* gptr(const void* p) {
    return (const __attribute__((address_space(1))) void*)p;
}
__device__ __forceinline__ __attribute__((address_space(3))) void* lptr(void* p) {
    return (__attribute__((address_space(3))) void*)p;
}

// DMA of one chunk's raw inputs into the staging area: rows of g, q, k, v land
// row-major and beta contiguous; one wave instruction moves 1 KiB (64 lanes x
// 16 bytes).  Rows at or past the chunk's end fetch a copy of its last row
// (no branches); the chunk zeroes them after the wait.
// The copy is a list of 1-KiB wave instructions, NI_* per input; wave w takes
// instructions w, w + NW, ... of each, so its own list has N entries (g, q, k,
// v in that order; beta goes with the last).  A wave that issues many of them
// at once stalls until the memory pipeline has accepted them, so the list is
// cut into NS slots placed between the chunk's compute steps.
template <typename TI, int DK, int DV>
struct Dma {
    typedef Cfg<TI, DK, DV> P;
    static constexpr int RB_G = DK * 4, RB_Q = DK * (int)sizeof(TI), RB_V = DV * (int)sizeof(TI);
    static constexpr int NI_G = C * RB_G / 1024, NI_Q = C * RB_Q / 1024, NI_V = C * RB_V / 1024;
    static_assert(NI_G % P::NW == 0 && NI_Q % P::NW == 0 && NI_V % P::NW == 0, "copy list does not split");
    static constexpr int PG = NI_G / P::NW, PQ = NI_Q / P::NW, PV = NI_V / P::NW;
    static constexpr int N = PG + 2 * PQ + PV;
    static constexpr int NS = 6;
};

// Entry J of wave wv's copy list for the chunk whose first (token, head) row is
// tok0 and which holds L1 > 0 tokens.
template <int J, typename TI, int DK, int DV>
__device__ __forceinline__ void dma_one(const Args<TI>& a, char* stg, size_t tok0, int L1, int wv, int lane, bool withq,
                                        bool withv) {
    typedef Dma<TI, DK, DV> D;
    typedef Cfg<TI, DK, DV> P;
    auto row = [&](const void* src, int RB, char* dst, int i) {
        const int lpr = RB / 16, rpi = 64 / lpr;
        const int t = min(i * rpi + lane / lpr, L1 - 1);
        const char* base = static_cast<const char*>(src) + tok0 * RB;
        __builtin_amdgcn_global_load_lds(gptr(base + (uint32_t)(t * a.H * RB + (lane % lpr) * 16)), lptr(dst + i * 1024),
                                         16, 0, 0);
    };
    if constexpr (J < D::PG) {
        row(a.g, D::RB_G, stg, wv + P::NW * J);
    } else if constexpr (J < D::PG + D::PQ) {
        if (withq) row(a.q, D::RB_Q, stg + P::SG_G, wv + P::NW * (J - D::PG));
    } else if constexpr (J < D::PG + 2 * D::PQ) {
        row(a.k, D::RB_Q, stg + P::SG_G + P::SG_Q, wv + P::NW * (J - D::PG - D::PQ));
    } else {
        if (withv) row(a.v, D::RB_V, stg + P::SG_G + 2 * P::SG_Q, wv + P::NW * (J - D::PG - 2 * D::PQ));
    }
}

// Slot S of the copy of the chunk starting at token c1 (L1 tokens; none if <= 0).
template <int S, typename TI, int DK, int DV>
__device__ __forceinline__ void dma_slot(const Args<TI>& a, char* stg, int64_t c1, int L1, int h, int wv, int lane,
                                         bool withq, bool withv) {
    typedef Dma<TI, DK, DV> D;
    typedef Cfg<TI, DK, DV> P;
    if (L1 <= 0) return;
    const size_t tok0 = (size_t)c1 * a.H + h;
    static_for<S * D::N / D::NS, (S + 1) * D::N / D::NS>(
        [&](auto jc) { dma_one<decltype(jc)::value, TI, DK, DV>(a, stg, tok0, L1, wv, lane, withq, withv); });
    if constexpr (S == D::NS - 1) {
        if (wv == 0)
            __builtin_amdgcn_global_load_lds(gptr(a.beta + tok0 + (size_t)min(lane, L1 - 1) * a.H),
                                             lptr(stg + P::SG_G + 2 * P::SG_Q + P::SG_V), 4, 0, 0);
    }
}

template <typename TI, int DK, int DV>
__device__ __forceinline__ void dma_all(const Args<TI>& a, char* stg, int64_t c1, int L1, int h, int wv, int lane,
                                        bool withq, bool withv) {
    static_for<0, Dma<TI, DK, DV>::NS>(
        [&](auto sc) { dma_slot<decltype(sc)::value, TI, DK, DV>(a, stg, c1, L1, h, wv, lane, withq, withv); });
}

// Workgroup barrier for LDS traffic only: each wave waits for its own LDS
// operations (lgkmcnt), not for its outstanding global loads and stores.  The
// prefetch copy writes LDS through the vector-memory path, so a memory-model
// fence on LDS (as in __syncthreads) would wait for it to land at every
// barrier; the copy's destination is only read after the explicit wait at the
// next chunk's start.  The "memory" clobber keeps the compiler from moving
// memory operations across.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// First sequence n in [0, num_seqs) with nl[n + 1] + bias * (n + 1) > key.
__device__ __forceinline__ int seq_of(const int32_t* nl, int num_seqs, int key, int bias) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (nl[mid + 1] + bias * (mid + 1) > key) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

// What one workgroup works on: the token range [tb, te) of head h, its start
// state (s0, or the identity (eye), or zero) and where its end state goes
// (sf; with NCB = 2 the N part goes to sf2).  See the kernels below for the
// three modes; `valid` is false for the surplus workgroups of a grid sized for
// a bound.
struct Unit {
    int h;
    int64_t tb, te;
    const float* s0;
    float* sf;
    float* sf2;
    void* ck;  // CKP: the checkpoint slot of the unit's first 16-token window
    bool eye, vzero, valid;
};
template <typename TI, int DK, int DV, bool MAP, int NCB, bool QH = false, bool CKP = false>
__device__ __forceinline__ Unit resolve_unit(const Args<TI>& a, int b) {
    const int H = a.H;
    Unit u;
    u.s0 = nullptr;
    u.sf = u.sf2 = nullptr;
    u.ck = nullptr;
    u.eye = u.vzero = false;
    u.valid = true;
    if constexpr (CKP) {
        const SegUnit su = seg_unit(a, b);
        u.valid = su.valid;
        if (!su.valid) return u;
        u.h = su.h;
        u.tb = su.sb;
        u.te = su.se;
        if (su.j == 0) u.s0 = a.S0 ? a.S0 + ((size_t)su.n * H + su.h) * DK * DV : nullptr;
        else u.s0 = a.wsN + ((size_t)(a.nl[su.n] + su.j - 1) * H + su.h) * DK * DV;
        u.ck = a.ck + (((size_t)(su.tb >> 4) + su.n + (size_t)((su.sb - su.tb) >> 4)) * H + su.h) * DK * DV;
    } else if constexpr (MAP && NCB == 2) {
        if (QH && b >= a.m_blocks) {
            // the last segment of split sequence spl[kk]: its M (to wsML) and q^; N is not kept
            const int kk = (b - a.m_blocks) / H;
            u.h = b - a.m_blocks - kk * H;
            const int n = a.spl[kk];
            if (n < 0) {
                u.valid = false;
                return u;
            }
            u.tb = a.cu[n] + (int64_t)(a.nl[n + 1] - a.nl[n]) * a.seg;
            u.te = a.cu[n + 1];
            u.eye = true;
            u.sf = a.wsML + ((size_t)kk * H + u.h) * DK * DK;
            return u;
        }
        const int k = b / H;
        u.h = b - k * H;
        if (k >= a.nl[a.num_seqs]) {
            u.valid = false;
            return u;
        }
        const int n = seq_of(a.nl, a.num_seqs, k, 0);
        if (k - a.nl[n] < a.map_from) {
            u.valid = false;
            return u;
        }
        u.tb = a.cu[n] + (int64_t)(k - a.nl[n]) * a.seg;
        u.te = u.tb + a.seg;
        u.eye = true;
        u.sf = a.wsM + ((size_t)k * H + u.h) * DK * DK;
        u.sf2 = a.wsN + ((size_t)k * H + u.h) * DK * DV;
    } else if constexpr (MAP) {
        const bool kindM = b < a.m_blocks;
        const int idx = kindM ? b : b - a.m_blocks;
        const int k = idx / H;
        u.h = idx - k * H;
        if (k >= a.nl[a.num_seqs]) {  // fewer non-last segments than the bound the grid was sized for
            u.valid = false;
            return u;
        }
        const int n = seq_of(a.nl, a.num_seqs, k, 0);
        if (k - a.nl[n] < a.map_from) {
            u.valid = false;
            return u;
        }
        u.tb = a.cu[n] + (int64_t)(k - a.nl[n]) * a.seg;
        u.te = u.tb + a.seg;
        u.eye = u.vzero = kindM;
        u.sf = kindM ? a.wsM + ((size_t)k * H + u.h) * DK * DK : a.wsN + ((size_t)k * H + u.h) * DK * DV;
    } else if (a.seg > 0 && a.phase == 1) {
        const int nb = b / H;
        u.h = b - nb * H;
        const int n = a.ord ? a.ord[nb] : nb;
        const size_t unit = (size_t)n * H + u.h;
        u.tb = a.cu[n];
        u.te = u.tb + a.seg < a.cu[n + 1] ? u.tb + a.seg : a.cu[n + 1];
        u.s0 = a.S0 ? a.S0 + unit * DK * DV : nullptr;
        if (a.nl[n + 1] > a.nl[n]) u.sf = a.wsN + ((size_t)a.nl[n] * H + u.h) * DK * DV;
        else u.sf = a.Sf ? a.Sf + unit * DK * DV : nullptr;
    } else if (a.seg > 0) {  // phase 2
        // non-last segment k of the batch (sequence n, its segment k - nl[n]) is
        // followed by segment j = k - nl[n] + 1, which this workgroup runs
        const int k = b / H;
        u.h = b - k * H;
        if (k >= a.nl[a.num_seqs]) {
            u.valid = false;
            return u;
        }
        const int n = seq_of(a.nl, a.num_seqs, k, 0);
        const int j = k - a.nl[n] + 1, last = a.nl[n + 1] - a.nl[n];
        const size_t unit = (size_t)n * H + u.h;
        u.tb = a.cu[n] + (int64_t)j * a.seg;
        u.te = u.tb + a.seg < a.cu[n + 1] ? u.tb + a.seg : a.cu[n + 1];
        u.s0 = a.wsN + ((size_t)(k) * H + u.h) * DK * DV;
        if (j == last && a.Sf) u.sf = a.Sf + unit * DK * DV;
    } else {
        const int nb = b / H;
        u.h = b - nb * H;
        const int n = a.ord ? a.ord[nb] : nb;
        const size_t unit = (size_t)n * H + u.h;
        u.tb = a.cu[n];
        u.te = a.cu[n + 1];
        u.s0 = a.S0 ? a.S0 + unit * DK * DV : nullptr;
        u.sf = a.Sf ? a.Sf + unit * DK * DV : nullptr;
    }
    return u;
}

// MAP = false: outputs o for a token range and carries the state from S0 to Sf
// (a whole sequence, or one segment of a split one).
// MAP = true: the transition of one full non-last segment.  The recurrence is
// affine in the state, S_end = M S_start + N, so M is the end state reached from
// S_start = I with v = 0 (a d_k-column state) and N the one reached from
// S_start = 0 with the real v; no q, P or o is formed.  With NCB = 1 a
// workgroup computes one of them (blocks below m_blocks: M); with NCB = 2
// (d_k = d_v) it computes both, wave w carrying columns 16w .. 16w+15 of each,
// so the key-side work of the chunk is done once for the two.
template <typename TI, int DK, int DV, bool MAP, int NCB = 1>
__global__ __launch_bounds__((Cfg<TI, DK, DV>::NT), 1) void prefill_seq_kernel(Args<TI> a) {
    typedef Cfg<TI, DK, DV> P;
    constexpr bool OUT = !MAP;
    static_assert(NCB == 1 || (MAP && DK == DV), "two column blocks only for transitions with d_k = d_v");
    typedef Mma<TI> M;
    typedef typename M::frag frag;
    typedef typename Pair<TI>::type T2;
    constexpr int KW = P::KW;
    // static, so that every LDS address is a compile-time offset that folds
    // into the instruction's immediate
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    char* stg = smem + P::OFF_STG;  // next chunk's raw inputs (bf16 only)
    const float* stg_g = reinterpret_cast<const float*>(stg);
    const TI* stg_q = reinterpret_cast<const TI*>(stg + P::SG_G);
    const TI* stg_k = reinterpret_cast<const TI*>(stg + P::SG_G + P::SG_Q);
    const TI* stg_v = reinterpret_cast<const TI*>(stg + P::SG_G + 2 * P::SG_Q);
    const float* stg_b = reinterpret_cast<const float*>(stg + P::SG_G + 2 * P::SG_Q + P::SG_V);
    TI* Qo = reinterpret_cast<TI*>(smem + P::OFF_QO);          // q~ (operand layout over d_k)
    TI* Ko = reinterpret_cast<TI*>(smem + P::OFF_KO);          // k~
    char* r3 = smem + P::OFF_R3;
    TI* Kh = reinterpret_cast<TI*>(r3);                        // k^ (Gram operand) ...
    floatx4* An = reinterpret_cast<floatx4*>(r3);              // ... then the blocks of -A
    TI* KdT = reinterpret_cast<TI*>(smem + P::OFF_KD);         // K_dec^T (operand layout over tokens)
    TI* Po = reinterpret_cast<TI*>(smem + P::OFF_P);           // P (operand layout over tokens)
    float* s_beta = reinterpret_cast<float*>(smem + P::OFF_F);
    float* s_gam = s_beta + C;
    float* s_gtot = s_gam + DK;
    float* s_mid = s_gtot + P::NG * DK;

    const int tid0 = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int H = a.H;
    const Unit u = resolve_unit<TI, DK, DV, MAP, NCB>(a, blockIdx.x);
    if (!u.valid) return;
    const int h = u.h;
    const int64_t tb = u.tb, te = u.te;
    const float* s0 = u.s0;
    float* sf = u.sf;
    float* sf2 = u.sf2;
    const bool eye = u.eye, vzero = u.vzero;
    const int col0 = 16 * w;  // this wave's state columns
    const uint32_t krow = (uint32_t)H * DK;  // elements between consecutive tokens of q, k, g
    const uint32_t vrow = (uint32_t)H * DV;  // ... of v, o

    // fp32 state: S[rt][i] = S[16 rt + 4g + i][col0 + r]
    const int r0 = tid0 & 15, g0 = (tid0 & 63) >> 4;
    // (NCB = 2: S[0] is the M part, started at the identity, S[1] the N part)
    floatx4 S[NCB][P::RT];
#pragma unroll
    for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * g0 + i;
            S[0][rt][i] = s0 ? at<float>(s0, (row * DV + col0 + r0) * 4) : (eye && row == col0 + r0) ? 1.f : 0.f;
            if constexpr (NCB == 2) S[1][rt][i] = 0.f;
        }

    if constexpr (P::STAGE) dma_all<TI, DK, DV>(a, stg, tb, (int)(te - tb < C ? te - tb : C), h, w, tid0 & 63, OUT, !vzero);

    // A chunk's outputs are stored at the start of the next chunk, after its
    // wait for the prefetch: vmcnt also counts stores, so storing them at the
    // end of the chunk would make that wait a full store round trip.
    // opend[rb] holds o[16 rb + r][col0 + 4g .. col0 + 4g + 3] (lane r + 16g).
    typedef typename std::conditional<sizeof(TI) == 2, bf16x4, floatx4>::type OV;
    OV opend[4];
    TI* opend_base = nullptr;
    int opend_L = 0;
    // Row block rb of the pending outputs; the four stores are spread over the
    // next chunk's first steps (a wave that issues several vector-memory
    // instructions at once waits for the pipeline to take them).
    auto flush_o = [&](int rb, int gl, int rl) {
        const int t = 16 * rb + rl;
        if (opend_base && t < opend_L)
            at_mut<OV>(opend_base, (t * vrow + col0 + 4 * gl) * (uint32_t)sizeof(TI)) = opend[rb];
    };

    for (int64_t c0 = tb; c0 < te; c0 += C) {
        // Lane-derived values are recomputed every chunk: kept opaque to the
        // compiler, so that addresses built from them are not hoisted out of
        // the loop and held in registers for its whole length.
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
        const int cp = tid % P::CPR, grp = P::UG ? w : tid / P::CPR, ch = 2 * cp;
        const int L = (int)(te - c0 < C ? te - c0 : C);
        const int64_t c1 = c0 + C;
        const int L1 = (int)(te - c1 < C ? te - c1 : C);  // valid tokens of the next chunk (<= 0: none)
        const size_t tok0 = (size_t)c0 * H + h;            // (token, head) row of the chunk's first token
        const float* gbase = a.g + tok0 * DK;
        const TI* qbase = a.q + tok0 * DK;
        const TI* kbase = a.k + tok0 * DK;
        const TI* vbase = a.v + tok0 * DV;
        TI* obase = a.o + tok0 * DV;

        // ---- 1. local cumulative log-decay ------------------------------------
        // Thread (cp, grp) owns key channels (ch, ch+1) of the tokens
        // grp*TPG .. grp*TPG+TPG-1 (at d_k = 128 a wave is one token group, so
        // token indices are wave-uniform).  Its inputs are read twice (from the
        // staging area, or from global memory where the second read hits the
        // cache): once to sum the group's log-decays, once to build the
        // operands, so few registers stay live.  G is kept in log2 units.
        // Staged rows at or past L are zero; global reads clamp the row and
        // select zero, so the loads carry no branches.
        auto rd_g = [&](int t) -> floatx2 {
            if constexpr (P::STAGE) return *reinterpret_cast<const floatx2*>(stg_g + t * DK + ch);
            const floatx2 x = at<floatx2>(gbase, ((t < L ? t : L - 1) * krow + ch) * 4);
            return t < L ? x : floatx2{0.f, 0.f};
        };
        auto rd_qk = [&](const TI* sp, const TI* gp, int t) -> floatx2 {
            if constexpr (P::STAGE) return to_f2(*reinterpret_cast<const T2*>(sp + t * DK + ch));
            const floatx2 x = to_f2(at<T2>(gp, ((t < L ? t : L - 1) * krow + ch) * (uint32_t)sizeof(TI)));
            return t < L ? x : floatx2{0.f, 0.f};
        };
        if constexpr (P::STAGE) {
            __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA has landed
            lds_barrier();                // ... and every other wave's; the previous chunk is done with LDS
            if (L < C) {
                // a partial chunk: zero the staging rows L .. C-1
                auto zero = [&](char* base, int row_bytes) {
                    floatx4* p = reinterpret_cast<floatx4*>(base + L * row_bytes);
                    const int n = (C - L) * row_bytes / 16;
                    for (int i = tid; i < n; i += P::NT) p[i] = zero4();
                };
                zero(stg, DK * 4);
                zero(stg + P::SG_G, DK * (int)sizeof(TI));
                zero(stg + P::SG_G + P::SG_Q, DK * (int)sizeof(TI));
                zero(stg + P::SG_G + 2 * P::SG_Q, DV * (int)sizeof(TI));
                if (tid >= L && tid < C) const_cast<float*>(stg_b)[tid] = 0.f;
                lds_barrier();
            }
        } else {
            lds_barrier();  // the previous chunk is done with LDS
        }
        if constexpr (OUT)
            for (int rb = 0; rb < 4; ++rb) flush_o(rb, g, r);  // the previous chunk's outputs
        // the solve's v right-hand side in accumulator layout: vr[I][i] = v[16I + 4g + i][col0 + r]
        typedef typename std::conditional<sizeof(TI) == 2, bf16x4, floatx4>::type VR;
        VR vr[4];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * I + 4 * g + i;
                if constexpr (P::STAGE) {
                    vr[I][i] = vzero ? TI(0.f) : stg_v[t * DV + col0 + r];
                } else {
                    const TI x = at<TI>(vbase, ((t < L ? t : L - 1) * vrow + col0 + r) * (uint32_t)sizeof(TI));
                    vr[I][i] = (t < L && !vzero) ? x : TI(0.f);
                }
            }
        if (tid < C) {
            float b;
            if constexpr (P::STAGE) {
                b = stg_b[tid];
            } else {
                b = at<float>(a.beta + tok0, (tid < L ? tid : L - 1) * H * 4);
                b = tid < L ? b : 0.f;
            }
            s_beta[tid] = b;
        }
        const int t0 = grp * P::TPG;
        {
            floatx2 sum = floatx2{0.f, 0.f};
#pragma unroll 4
            for (int tt = 0; tt < P::TPG; ++tt) sum = fma2(rd_g(t0 + tt), LOG2E, sum);
            *reinterpret_cast<floatx2*>(s_gtot + grp * DK + ch) = sum;
        }
        lds_barrier();
        floatx2 off = floatx2{0.f, 0.f}, tot = floatx2{0.f, 0.f};
#pragma unroll
        for (int gg = 0; gg < P::NG; ++gg) {
            if (gg == grp) off = tot;
            tot += *reinterpret_cast<const floatx2*>(s_gtot + gg * DK + ch);
        }
        // With g <= 0 the cumulative log-decay is non-increasing, so its most
        // negative value on a channel is the chunk total; every wave sees all
        // channels, so the decision is uniform over the workgroup.
        constexpr float BUDGET = -40.f * LOG2E;  // e^-40, in log2 units
        const bool fast = __all(tot[0] >= BUDGET && tot[1] >= BUDGET);
        const floatx2 gam = pow2v(tot);
        if (grp == 0) *reinterpret_cast<floatx2*>(s_gam + ch) = gam;

        // ---- 2. decay-scaled operands --------------------------------------
        // K_dec^T is stored four tokens at a time (one 8-byte store per channel).
        auto store_kd4 = [&](int t, const floatx2* kd) {
            if constexpr (sizeof(TI) == 2) {
                *reinterpret_cast<bf16x4*>(KdT + op_idx<TI, P::TM>(ch, t)) =
                    bf16x4{(bf16)kd[0][0], (bf16)kd[1][0], (bf16)kd[2][0], (bf16)kd[3][0]};
                *reinterpret_cast<bf16x4*>(KdT + op_idx<TI, P::TM>(ch + 1, t)) =
                    bf16x4{(bf16)kd[0][1], (bf16)kd[1][1], (bf16)kd[2][1], (bf16)kd[3][1]};
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    KdT[op_idx<TI, P::TM>(ch, t + j)] = kd[j][0];
                    KdT[op_idx<TI, P::TM>(ch + 1, t + j)] = kd[j][1];
                }
            }
        };
        if (fast) {
            floatx2 G = off;
            // In the bf16 operand layout the byte offset of (t0 + tt, ch) is
            // that of (t0, ch) with tt XORed into bits 4.. (t0 is a multiple of
            // TPG, a power of two, and a token group stays in one 16-row block),
            // and Qo, Ko, Kh share it.
            const uint32_t a0 = op_idx<TI, P::KM>(t0, ch) * (uint32_t)sizeof(TI);
            auto put = [&](TI* mat, int tt, int t, floatx2 x) {
                if constexpr (KW == 8) {
                    *reinterpret_cast<bf16x2*>(reinterpret_cast<char*>(mat) + (a0 ^ (uint32_t)(tt << 4))) =
                        bf16x2{(bf16)x[0], (bf16)x[1]};
                } else {
                    op_store2<TI, P::KM>(mat, t, ch, x);
                }
            };
#pragma unroll 1
            for (int tq = 0; tq < P::TPG; tq += 4) {
                floatx2 kd[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int tt = tq + j, t = t0 + tt;
                    G = fma2(rd_g(t), LOG2E, G);
                    const floatx2 e = pow2v(G), ei = pow2v(-G);
                    const floatx2 kk = rd_qk(stg_k, kbase, t);
                    const floatx2 kh = kk * ei;
                    if constexpr (OUT) put(Qo, tt, t, rd_qk(stg_q, qbase, t) * e);
                    put(Ko, tt, t, kk * e);
                    put(Kh, tt, t, kh);
                    kd[j] = kh * gam;  // K_dec = k e^{G_L - G}
                }
                store_kd4(t0 + tq, kd);
            }
        } else {
            // reference of row block I: G at its middle row 16I + 7
            {
                floatx2 G = off;
                for (int tt = 0; tt < P::TPG; ++tt) {
                    const int t = t0 + tt;
                    G = fma2(rd_g(t), LOG2E, G);
                    if ((t & 15) == 7) *reinterpret_cast<floatx2*>(s_mid + (t >> 4) * DK + ch) = G;
                }
            }
            lds_barrier();  // s_mid visible
            floatx2 G = off;
#pragma unroll 1
            for (int tq = 0; tq < P::TPG; tq += 4) {
                floatx2 kd[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = t0 + tq + j;
                    G = fma2(rd_g(t), LOG2E, G);
                    const floatx2 m = *reinterpret_cast<const floatx2*>(s_mid + (t >> 4) * DK + ch);
                    const floatx2 e = pow2v(G - m);
                    const floatx2 kk = rd_qk(stg_k, kbase, t);
                    if constexpr (OUT) op_store2<TI, P::KM>(Qo, t, ch, rd_qk(stg_q, qbase, t) * e);
                    op_store2<TI, P::KM>(Ko, t, ch, kk * e);
                    kd[j] = kk * pow2v(tot - G);
                }
                store_kd4(t0 + tq, kd);
            }
        }

        // ---- 3. Gram tiles (transposed) -------------------------------------
        // tile (I, J): C[s][t] = sum_c k^[s][c] x[t][c], s in block J, t in block I;
        // lane r + 16g ends with x-row t = 16I + r against columns s = 16J + 4g + i.
        auto gram = [&](const TI* rows, int I, int J) {
            frag fa[P::KM], fb[P::KM];
#pragma unroll
            for (int m = 0; m < P::KM; ++m) {
                fa[m] = op_frag<TI, P::KM>(Kh, J, m, lane);
                fb[m] = op_frag<TI, P::KM>(rows, I, m, lane);
            }
            floatx4 acc = zero4();
#pragma unroll
            for (int m = 0; m < P::KM; ++m) acc = M::mma(fa[m], fb[m], acc);
            return acc;
        };
        // P tile (I, J) into the operand layout of P over tokens (rows t, k = s).
        auto store_p = [&](const floatx4& acc, int I, int J) {
            const int t = 16 * I + r;
            floatx4 p;
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = (16 * J + 4 * g + i <= t) ? acc[i] : 0.f;
            if constexpr (KW == 8) {
                const bf16x4 pb = bf16x4{(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3]};
                bf16* dst = reinterpret_cast<bf16*>(Po) + ((I * P::TM + J / 2) * 64 + op_slot(I, J / 2, r, g)) * 8 + 4 * (J & 1);
                *reinterpret_cast<bf16x4*>(dst) = pb;
                if (J == I && (I & 1) == 0) *reinterpret_cast<bf16x4*>(dst + 4) = bf16x4{};  // block above the diagonal
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    reinterpret_cast<float*>(Po)[(I * P::TM + 4 * J + i) * 64 + op_slot(I, 4 * J + i, r, g)] = p[i];
            }
        };
        constexpr int NACC = P::NPT > 4 ? P::NPT : 4;
        floatx4 accA[NACC];
        int aP[NACC];
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
            accA[j] = zero4();
            aP[j] = -1;
        }
        if (fast) {
            lds_barrier();
            // the staging area is free from here on: the next chunk's copy is
            // issued in slots over steps 3-4b
            if constexpr (P::STAGE) dma_slot<0, TI, DK, DV>(a, stg, c1, L1, h, w, lane, OUT, !vzero);
            // 20 tiles (10 of A, 10 of P); wave w takes tiles w, w+NW, ...
#pragma unroll
            for (int j = 0; j < P::NPT; ++j) {
                const int q = w + P::NW * j;
                if (q < (OUT ? 20 : 10)) {
                    int I, J;
                    tri_pair(q % 10, I, J);
                    const floatx4 acc = gram(q < 10 ? Ko : Qo, I, J);
                    if (q < 10) {
                        accA[j] = acc;
                        aP[j] = q;
                    } else if constexpr (OUT) {
                        store_p(acc, I, J);
                    }
                }
            }
            if constexpr (P::STAGE) dma_slot<1, TI, DK, DV>(a, stg, c1, L1, h, w, lane, OUT, !vzero);
            lds_barrier();  // every read of Kh is done
        } else {
            for (int I = 0; I < 4; ++I) {
                lds_barrier();  // readers of the previous Kh are done
                {
                    const floatx2 m = *reinterpret_cast<const floatx2*>(s_mid + I * DK + ch);
                    floatx2 G = off;
                    for (int tt = 0; tt < P::TPG; ++tt) {
                        const int t = t0 + tt;
                        G = fma2(rd_g(t), LOG2E, G);
                        if (t < 16 * (I + 1))
                            op_store2<TI, P::KM>(Kh, t, ch, rd_qk(stg_k, kbase, t) * pow2v(m - G));
                    }
                }
                lds_barrier();
#pragma unroll
                for (int jj = 0; jj < P::NQS; ++jj) {
                    const int qq = w + P::NW * jj;
                    if (qq < (OUT ? 2 : 1) * (I + 1)) {
                        if (qq < I + 1) {
                            // at most one A tile per wave and row block: slot I
#pragma unroll
                            for (int sI = 0; sI < 4; ++sI)
                                if (sI == I) {
                                    accA[sI] = gram(Ko, I, qq);
                                    aP[sI] = tri_id(I, qq);
                                }
                        } else if constexpr (OUT) {
                            store_p(gram(Qo, I, qq - I - 1), I, qq - I - 1);
                        }
                    }
                }
            }
            lds_barrier();  // every read of Qo/Ko/Kh is done
            // the inter-chunk products use the chunk start as reference
            {
                floatx2 G = off;
                for (int tt = 0; tt < P::TPG; ++tt) {
                    const int t = t0 + tt;
                    G = fma2(rd_g(t), LOG2E, G);
                    const floatx2 e = pow2v(G);
                    if constexpr (OUT) op_store2<TI, P::KM>(Qo, t, ch, rd_qk(stg_q, qbase, t) * e);
                    op_store2<TI, P::KM>(Ko, t, ch, rd_qk(stg_k, kbase, t) * e);
                }
            }
            if constexpr (P::STAGE) dma_all<TI, DK, DV>(a, stg, c1, L1, h, w, lane, OUT, !vzero);
        }
        // -A tiles: lane r + 16g holds -beta_t A[t][s], t = 16I + r, s = 16J + 4g + i
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
            if (aP[j] >= 0) {
                int I, J;
                tri_pair(aP[j], I, J);
                const int t = 16 * I + r;
                const float bt = s_beta[t];
                floatx4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (16 * J + 4 * g + i < t) ? -bt * accA[j][i] : 0.f;
                An[aP[j] * 64 + lane] = x;
            }
        }
        if constexpr (P::STAGE)
            if (fast) dma_slot<2, TI, DK, DV>(a, stg, c1, L1, h, w, lane, OUT, !vzero);
        lds_barrier();

        // ---- 4a. inverses of the diagonal blocks of (I + A) -------------------
        // Wave I < 4 inverts block I by forward substitution (row j of the
        // inverse is final once rows < j have been applied, and is broadcast
        // along each 16-lane row) and publishes it after the blocks of -A;
        // lane r + 16g holds Linv_I[r][4g .. 4g+3].
        if (w < 4) {
            const int I = w;
            float arow[16];
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const floatx4 x = An[tri_id(I, I) * 64 + r + 16 * gg];
#pragma unroll
                for (int i = 0; i < 4; ++i) arow[4 * gg + i] = x[i];
            }
            const floatx4 x = row_inverse(arow, r, g);
            An[(10 + I) * 64 + lane] = x;
        }
        lds_barrier();
        // (each consumer reads Linv_I from LDS where it needs it)
        if constexpr (P::STAGE)
            if (fast) dma_slot<3, TI, DK, DV>(a, stg, c1, L1, h, w, lane, OUT, !vzero);

        // ---- 4b. U = (I + A)^-1 diag(beta) (V - K~ S), own columns -----------
        // This is U = Ut - W S with W = (I + A)^-1 diag(beta) K~ never formed:
        // the right-hand side takes K~ S first, then the block forward
        // substitution runs on the wave's 16 columns only.
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
        // column block cb of the wave (NCB = 2: the M part has v = 0)
        const bool vblock = NCB == 1 || cb == 1;
        frag bS[P::KM];
#pragma unroll
        for (int m = 0; m < P::KM; ++m) bS[m] = acc_perm<TI>(S[cb], m, P::RT);
        floatx4 U[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            frag ak[P::KM];
#pragma unroll
            for (int m = 0; m < P::KM; ++m) ak[m] = op_frag<TI, P::KM>(Ko, I, m, lane);
            floatx4 ks = zero4();
#pragma unroll
            for (int m = 0; m < P::KM; ++m) ks = M::mma(ak[m], bS[m], ks);
            floatx4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = s_beta[16 * I + 4 * g + i] * ((vblock ? (float)vr[I][i] : 0.f) - ks[i]);
            if constexpr (KW == 8) {
#pragma unroll
                for (int m = 0; 2 * m < I; ++m) {
                    const floatx4 lo = An[tri_id(I, 2 * m) * 64 + lane];
                    const floatx4 hi = (2 * m + 1 < I) ? An[tri_id(I, 2 * m + 1) * 64 + lane] : zero4();
                    const bf16x8 af = bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
                                             (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
                    acc = M::mma(af, acc_perm<TI>(U, m, I), acc);
                }
                const floatx4 li = An[(10 + I) * 64 + lane];
                const bf16x8 lf = bf16x8{(bf16)li[0], (bf16)li[1], (bf16)li[2], (bf16)li[3],
                                         (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
                U[I] = M::mma(lf, acc_perm<TI>(&acc, 0, 1), zero4());
            } else {
#pragma unroll
                for (int J = 0; J < I; ++J) {
                    const floatx4 an = An[tri_id(I, J) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = M::mma(an[e], U[J][e], acc);
                }
                floatx4 ui = zero4();
                const floatx4 li = An[(10 + I) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) ui = M::mma(li[e], acc[e], ui);
                U[I] = ui;
            }
            if constexpr (P::STAGE)
                if (I == 1 && cb == 0 && fast) dma_slot<4, TI, DK, DV>(a, stg, c1, L1, h, w, lane, OUT, !vzero);
        }
        if constexpr (P::STAGE)
            if (cb == 0 && fast) dma_slot<5, TI, DK, DV>(a, stg, c1, L1, h, w, lane, OUT, !vzero);

        // ---- 5. outputs and state (own columns) -------------------------------
        // O = Q~ S + P U one row block at a time, then S <- diag(e^{G_L}) S + K_dec^T U.
        // O is formed transposed, O^T = S^T Q~^T + U^T P^T: the operand layouts
        // of MFMA's two inputs coincide, so the same fragments serve with their
        // roles swapped, and each lane ends with four adjacent columns of one
        // token row (one 8- or 16-byte store).
        frag bU[P::TM];
#pragma unroll
        for (int m = 0; m < P::TM; ++m) bU[m] = acc_perm<TI>(U, m, 4);
#pragma unroll
        for (int rb = 0; rb < (OUT ? 4 : 0); ++rb) {
            frag aq[P::KM];
#pragma unroll
            for (int m = 0; m < P::KM; ++m) aq[m] = op_frag<TI, P::KM>(Qo, rb, m, lane);
            floatx4 O = zero4();
#pragma unroll
            for (int m = 0; m < P::KM; ++m) O = M::mma(bS[m], aq[m], O);
#pragma unroll
            for (int m = 0; m < P::TM; ++m)
                if ((m * KW) / 4 <= rb) O = M::mma(bU[m], op_frag<TI, P::TM>(Po, rb, m, lane), O);
#pragma unroll
            for (int i = 0; i < 4; ++i) opend[rb][i] = from_f32<TI>(O[i]);
        }
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt) {
            const floatx4 d = *reinterpret_cast<const floatx4*>(s_gam + 16 * rt + 4 * g);
            S[cb][rt] *= d;
        }
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt) {
            frag ak[P::TM];
#pragma unroll
            for (int m = 0; m < P::TM; ++m) ak[m] = op_frag<TI, P::TM>(KdT, rt, m, lane);
#pragma unroll
            for (int m = 0; m < P::TM; ++m) S[cb][rt] = M::mma(ak[m], bU[m], S[cb][rt]);
        }
        if constexpr (NCB > 1) __builtin_amdgcn_sched_barrier(0);  // keep the blocks' live ranges apart
        }  // column blocks
        if constexpr (OUT) {
            opend_base = obase;
            opend_L = L;
        }
        // The next chunk writes LDS only after its first barrier, which every
        // wave reaches after finishing this state pass.
    }
    if constexpr (OUT)
        for (int rb = 0; rb < 4; ++rb) flush_o(rb, g0, r0);

#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        float* dst = cb == 0 ? sf : sf2;
        if (dst) {
#pragma unroll
            for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    at_mut<float>(dst, ((16 * rt + 4 * g0 + i) * DV + col0 + r0) * 4) = S[cb][rt][i];
        }
    }
}

// ============================================================================
// Warp-specialised prefill (bf16 inputs).
//
// The per-chunk work splits into a key side that does not touch the state
// (local decay, decay-scaled operands, Gram tiles, inverses of the diagonal
// blocks) and a state side (K~S, the solve for U, outputs, state update).  A
// workgroup has NK = 4 key waves and d_v/16 state waves: while the state waves
// run chunk j, the key waves prepare chunk j+1 into the other half of a
// double-buffered LDS area, so the two instruction mixes (exponentials and
// vector ALU on one side, matrix cores on the other) overlap on every SIMD,
// and a chunk costs three workgroup barriers.
//
// Chunks are 32 tokens.  With g >= -5 a 32-token chunk spans at most -160,
// so a reference at its 16th token keeps every factor inside e^+-80 (the
// 16-token window of "Trillion-Parameter MoE Multimodal LLMs: How to Evaluate
// the New Generation", section 3.1, taken on both sides of the reference):
//   - if the chunk total is >= -64 on every channel, the chunk start is the
//     reference for everything (q~ = q e^G, k~ = k e^G, k^ = k e^-G);
//   - otherwise the Gram operands use the middle reference m (q e^(G-m),
//     k e^(G-m), k e^(m-G)) while the inter-chunk operands keep the chunk
//     start (q e^G, k e^G <= 1, which may underflow harmlessly).
// No sub-tile path is needed.
//
// Per chunk (2 row blocks of 16 tokens):
//   key:   G (log2 units) -> group sums | operands QO, KO, KH, KD, gamma, beta
//          | Gram A, P tiles; -beta A masked; Linv_0, Linv_1 by forward
//          substitution; An_10
//   state: KS = K~ S; R = beta (V - KS) | U_0 = Linv_0 R_0,
//          U_1 = Linv_1 (R_1 + An_10 U_0); O = Q~ S + P U (stored) |
//          S <- diag(gamma) S + K_dec^T U
// ============================================================================

template <int DK, int DV, int NCB = 1>
struct CfgW {
    static constexpr int CW = 32;             // chunk length (tokens)
    static constexpr int NK = 4;              // key waves
    static constexpr int NS = DV / 16;        // state waves; state wave s owns columns 16s .. 16s+15
    static constexpr int NT = 64 * (NK + NS);
    static constexpr int KM = DK / 32;        // MFMA k-steps over d_k
    static constexpr int RT = DK / 16;        // 16-row tiles of the state
    static constexpr int CPR = DK / 2;        // key lanes per token row (two channels per lane)
    static constexpr int NG = NK * 64 / CPR;  // token groups of the key side
    static constexpr int TPL = CW / NG;       // tokens per group (8 at d_k = 128, 4 at 64)
    static constexpr int TPW = CW / NK;       // tokens whose inputs one key wave copies (8)
    static constexpr int SZ_OP = CW * DK * 2;
    static constexpr int SZ_PO = CW * CW * 2;
    // one half of the double buffer: written by the key side for chunk j,
    // read by the state side one chunk later
    static constexpr int B_QO = 0, B_KO = SZ_OP, B_KD = 2 * SZ_OP, B_PO = 3 * SZ_OP;
    static constexpr int B_TB = B_PO + SZ_PO;  // Linv_0, Linv_1, An_10 as A-operand fragments, 1 KiB each
    static constexpr int B_BETA = B_TB + 3 * 1024, B_GM = B_BETA + CW * 4;
    // per-head gates: e^{G_t} [CW], e^{G_L - G_t} [CW], e^{G_L} in place of
    // the per-channel gamma (a kernel uses one or the other)
    static constexpr int B_EG = B_GM;
    static constexpr int SZ_GM = DK * 4 > (2 * CW + 1) * 4 ? DK * 4 : (2 * CW + 1) * 4;
    static constexpr int SZ_BUF = (B_GM + SZ_GM + 255) / 256 * 256;
    // key-side scratch
    static constexpr int OFF_KH = 2 * SZ_BUF, OFF_QM = OFF_KH + SZ_OP, OFF_KM = OFF_QM + SZ_OP;
    static constexpr int OFF_AN = OFF_KM + SZ_OP, OFF_GT = OFF_AN + 2 * 1024;
    static constexpr int OFF_STG = (OFF_GT + NG * DK * 4 + 1023) / 1024 * 1024;
    static constexpr int SG_G = CW * DK * 4, SG_Q = CW * DK * 2;
    static constexpr int LDS = OFF_STG + SG_G + 2 * SG_Q + 64 * 4;
    static_assert(TPL >= 4 && (TPL & (TPL - 1)) == 0, "token groups");
};

// Slot of (row r, tokens 4g .. 4g+3) inside 16-row tile rt of the checkpoint
// pass's K_dec_mid operand (16 x 16 A-operand fragments of 64 slots of 4 bf16).
// The XOR spreads a key wave's store of one token quad over 64 channels across
// all the LDS banks; a fragment read is still one slot per lane.
__device__ __forceinline__ int kdm_slot(int rt, int r, int g) { return (16 * g + r) ^ (rt & 1) ^ ((rt & 2) << 3); }

// Key side: waves 0 .. NK-1.  Prepares chunk i in iteration i.
// CKP (with MAP): the backward's checkpoint pass; besides the transition's
// operands, K_dec_mid = k e^{G_15 - G} of the first 16 tokens (in the unused
// q-operand area) and e^{G_15} (in the unused P area), from which the state
// side forms the state after token 15.
template <int DK, int DV, bool MAP, int NCB, bool ZG, bool QH = false, bool CKP = false>
__device__ __forceinline__ void ws_key(const Args<bf16>& a, char* smem, int kw, int h, int64_t tb, int64_t te,
                                       int nch) {
    typedef CfgW<DK, DV, NCB> P;
    typedef bf16 TI;
    typedef Mma<bf16> M;
    typedef bf16x8 frag;
    // the q operands and P are formed for outputs: those of the output pass,
    // and q^ of a transition pass for the backward (QH)
    constexpr bool OUT = !MAP || QH;
    constexpr int CW = P::CW, KM = P::KM;
    const int H = a.H;
    char* stg = smem + P::OFF_STG;
    const float* stg_g = reinterpret_cast<const float*>(stg);
    const TI* stg_q = reinterpret_cast<const TI*>(stg + P::SG_G);
    const TI* stg_k = reinterpret_cast<const TI*>(stg + P::SG_G + P::SG_Q);
    float* stg_b = reinterpret_cast<float*>(stg + P::SG_G + 2 * P::SG_Q);
    TI* KH = reinterpret_cast<TI*>(smem + P::OFF_KH);
    TI* QM = reinterpret_cast<TI*>(smem + P::OFF_QM);
    TI* KMm = reinterpret_cast<TI*>(smem + P::OFF_KM);
    floatx4* AN = reinterpret_cast<floatx4*>(smem + P::OFF_AN);
    float* s_gt = reinterpret_cast<float*>(smem + P::OFF_GT);

    // waves 0, 1: inverse of the diagonal block kw of (I + beta A), whose
    // strictly lower part -beta A is in this wave's AN area, as an A-operand
    // fragment (each lane gathers its row of the block from LDS)
    auto inverse_to = [&](frag* tb) {
        const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
        float arow[16];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const floatx4 y = AN[kw * 64 + r + 16 * gg];
#pragma unroll
            for (int e = 0; e < 4; ++e) arow[4 * gg + e] = y[e];
        }
        const floatx4 li = row_inverse(arow, r, g);
        tb[kw * 64 + lane] =
            frag{(bf16)li[0], (bf16)li[1], (bf16)li[2], (bf16)li[3], (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    };

    // copy of chunk j's g, q, k rows TPW*kw .. TPW*kw+TPW-1 (and, wave 0, beta)
    auto dma = [&](int j, int lane) {
        const int64_t c0 = tb + (int64_t)j * CW;
        const int L = (int)(te - c0 < CW ? te - c0 : CW);
        const size_t tok0 = (size_t)c0 * H + h;
        auto rows = [&](const void* src, int RB, char* dst) {
            const int lpr = RB / 16, rpi = 64 / lpr;
            const char* base = static_cast<const char*>(src) + tok0 * RB;
#pragma unroll
            for (int i = 0; i < P::TPW / rpi; ++i) {
                const int r0 = P::TPW * kw + rpi * i;
                const int t = min(r0 + lane / lpr, L - 1);
                __builtin_amdgcn_global_load_lds(gptr(base + (uint32_t)(t * H * RB + (lane % lpr) * 16)),
                                                 lptr(dst + r0 * RB), 16, 0, 0);
            }
        };
        if constexpr (ZG) rows(a.z, DK * 2, stg);  // logits: bf16 rows
        else rows(a.g, DK * 4, stg);
        if (OUT) rows(a.q, DK * 2, stg + P::SG_G);
        rows(a.k, DK * 2, stg + P::SG_G + P::SG_Q);
        if (kw == 0)
            __builtin_amdgcn_global_load_lds(gptr(a.beta + tok0 + (size_t)min(lane, L - 1) * H), lptr(stg_b), 4, 0, 0);
    };
    if (nch > 0) dma(0, threadIdx.x & 63);

    for (int i = 0; i <= nch; ++i) {
        int tid = kw * 64 + (threadIdx.x & 63);
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
        const int cp = tid % P::CPR, grp = tid / P::CPR, ch = 2 * cp, t0 = grp * P::TPL;
        const bool act = i < nch;
        char* buf = smem + (i & 1) * P::SZ_BUF;
        TI* QO = reinterpret_cast<TI*>(buf + P::B_QO);
        TI* KO = reinterpret_cast<TI*>(buf + P::B_KO);
        TI* KD = reinterpret_cast<TI*>(buf + P::B_KD);
        TI* PO = reinterpret_cast<TI*>(buf + P::B_PO);
        frag* TB = reinterpret_cast<frag*>(buf + P::B_TB);
        float* BETA = reinterpret_cast<float*>(buf + P::B_BETA);
        float* GM = reinterpret_cast<float*>(buf + P::B_GM);
        const int64_t c0 = tb + (int64_t)i * CW;
        const int L = (int)(te - c0 < CW ? te - c0 : CW);

        // ---- K1: this wave's copy has landed; its rows go to registers (their
        // latency hides behind the barrier) and the group sums of g (log2 units)
        // to LDS
        floatx2 gv[P::TPL];
        bf16x2 kv[P::TPL], qv[P::TPL], zv[P::TPL];
        if (act) {
            __builtin_amdgcn_s_waitcnt(0);
            if (L < CW) {
                // rows L .. CW-1 of this wave's part hold copies of row L-1: zero them
                for (int t = P::TPW * kw; t < P::TPW * (kw + 1); ++t)
                    if (t >= L) {
                        if (!ZG && lane < DK / 4)
                            reinterpret_cast<floatx4*>(const_cast<float*>(stg_g) + t * DK)[lane] = zero4();
                        if (lane < DK / 8) {
                            reinterpret_cast<floatx4*>(const_cast<TI*>(stg_q) + t * DK)[lane] = zero4();
                            reinterpret_cast<floatx4*>(const_cast<TI*>(stg_k) + t * DK)[lane] = zero4();
                        }
                    }
                if (kw == 0 && lane >= L && lane < CW) stg_b[lane] = 0.f;
            }
            if constexpr (!ZG) {
#pragma unroll
                for (int tt = 0; tt < P::TPL; ++tt)
                    gv[tt] = *reinterpret_cast<const floatx2*>(stg_g + (t0 + tt) * DK + ch);
            } else {
                const TI* stg_z = reinterpret_cast<const TI*>(stg);
#pragma unroll
                for (int tt = 0; tt < P::TPL; ++tt) zv[tt] = *reinterpret_cast<const bf16x2*>(stg_z + (t0 + tt) * DK + ch);
            }
#pragma unroll
            for (int tt = 0; tt < P::TPL; ++tt) {
                kv[tt] = *reinterpret_cast<const bf16x2*>(stg_k + (t0 + tt) * DK + ch);
                if constexpr (OUT) qv[tt] = *reinterpret_cast<const bf16x2*>(stg_q + (t0 + tt) * DK + ch);
            }
        }
        if constexpr (MAP && !QH)
            if (i >= 1 && kw < 2) inverse_to(reinterpret_cast<frag*>(smem + ((i - 1) & 1) * P::SZ_BUF + P::B_TB));
        if (act) {
            auto group_sum = [&]() {
                floatx2 sum = floatx2{0.f, 0.f};
#pragma unroll
                for (int tt = 0; tt < P::TPL; ++tt) sum = fma2(gv[tt], LOG2E, sum);
                *reinterpret_cast<floatx2*>(s_gt + grp * DK + ch) = sum;
            };
            if constexpr (!ZG) group_sum();
            if (kw == 0 && lane < CW) BETA[lane] = stg_b[lane];
            // this wave's staging rows are in registers: copy the next chunk
            // (it lands during the rest of this iteration and is waited for
            // at the start of the next)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (i + 1 < nch) dma(i + 1, lane);
            if constexpr (ZG) {
                // the gate parameterisation, after the copy is under way; rows
                // past the end then get g = 0 (their logits are copies of the
                // last row's).  One branch-free loop per parameterisation, so
                // that the 2 TPL independent exp -> rcp (-> log) chains
                // interleave.
                const float p = a.gate_param;
                auto from_logits = [&](auto fn) {
#pragma unroll
                    for (int tt = 0; tt < P::TPL; ++tt) gv[tt] = floatx2{fn((float)zv[tt][0]), fn((float)zv[tt][1])};
                };
                if (a.gate == GATE_SCALED_SIGMOID) from_logits([&](float x) { return p * sigmoid_hw(x); });
                else from_logits([&](float x) { return gate_log_decay(x, GATE_ALPHA_MIN, p); });
                if (L < CW) {
#pragma unroll
                    for (int tt = 0; tt < P::TPL; ++tt)
                        if (t0 + tt >= L) gv[tt] = floatx2{0.f, 0.f};
                }
                group_sum();
            }
        }
        lds_barrier();  // B1

        // ---- K2: decay-scaled operands
        bool fast = true;
        if (act) {
            floatx2 off = floatx2{0.f, 0.f}, tot = floatx2{0.f, 0.f}, mid = floatx2{0.f, 0.f};
#pragma unroll
            for (int gg = 0; gg < P::NG; ++gg) {
                if (gg == grp) off = tot;
                if (gg == 16 / P::TPL) mid = tot;  // G after token 15
                tot += *reinterpret_cast<const floatx2*>(s_gt + gg * DK + ch);
            }
            constexpr float BUDGET = -64.f * LOG2E;  // e^-64, in log2 units
            fast = __all(tot[0] >= BUDGET && tot[1] >= BUDGET);
            const floatx2 gam = pow2v(tot);
            if (grp == 0) *reinterpret_cast<floatx2*>(GM + ch) = gam;
            floatx2 emid = floatx2{0.f, 0.f};  // CKP: e^{G_15}
            if constexpr (CKP) {
                emid = pow2v(mid);
                if (grp == 0) *reinterpret_cast<floatx2*>(reinterpret_cast<float*>(buf + P::B_PO) + ch) = emid;
            }
            // CKP: K_dec_mid of tokens t .. t+3 (t < 16, a multiple of 4), channels ch, ch + 1
            auto store_kdm4 = [&](int t, const floatx2* km) {
                TI* KDM = reinterpret_cast<TI*>(buf + P::B_QO);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int c = ch + e, rt = c >> 4;
                    *reinterpret_cast<bf16x4*>(KDM + (rt * 64 + kdm_slot(rt, c & 15, t >> 2)) * 4) =
                        bf16x4{(bf16)km[0][e], (bf16)km[1][e], (bf16)km[2][e], (bf16)km[3][e]};
                }
            };
            // byte offset of (t0 + tt, ch) in the bf16 operand layout: that of
            // (t0, ch) with tt XORed into bits 4.. (t0 is a multiple of TPL, a
            // power of two, and a group stays in one 16-row block)
            const uint32_t a0 = op_idx<TI, KM>(t0, ch) * 2u;
            auto put = [&](TI* mat, int tt, floatx2 x) {
                *reinterpret_cast<bf16x2*>(reinterpret_cast<char*>(mat) + (a0 ^ (uint32_t)(tt << 4))) =
                    bf16x2{(bf16)x[0], (bf16)x[1]};
            };
            auto store_kd4 = [&](int t, const floatx2* kd) {
                *reinterpret_cast<bf16x4*>(KD + op_idx<TI, 1>(ch, t)) =
                    bf16x4{(bf16)kd[0][0], (bf16)kd[1][0], (bf16)kd[2][0], (bf16)kd[3][0]};
                *reinterpret_cast<bf16x4*>(KD + op_idx<TI, 1>(ch + 1, t)) =
                    bf16x4{(bf16)kd[0][1], (bf16)kd[1][1], (bf16)kd[2][1], (bf16)kd[3][1]};
            };
            // one loop per case (the choice is uniform), so that the loads of
            // all TPL tokens can be issued together
            auto ld_g = [&](int t) { return gv[t - t0]; };
            auto ld_k = [&](int t) { return to_f2(kv[t - t0]); };
            auto ld_q = [&](int t) {
                if constexpr (OUT) return to_f2(qv[t - t0]);
                return floatx2{0.f, 0.f};
            };
            floatx2 G = off;
            if (fast) {
#pragma unroll
                for (int tq = 0; tq < P::TPL; tq += 4) {
                    floatx2 kd[4], km[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int tt = tq + j, t = t0 + tt;
                        G = fma2(ld_g(t), LOG2E, G);
                        const floatx2 kk = ld_k(t), e = pow2v(G), ei = pow2v(-G);
                        const floatx2 kh = kk * ei;
                        if constexpr (OUT) put(QO, tt, ld_q(t) * e);
                        put(KO, tt, kk * e);
                        put(KH, tt, kh);
                        kd[j] = kh * gam;  // K_dec = k e^(G_L - G)
                        km[j] = kh * emid;  // K_dec_mid = k e^(G_15 - G), t <= 15
                    }
                    store_kd4(t0 + tq, kd);
                    if constexpr (CKP)
                        if (t0 < 16) store_kdm4(t0 + tq, km);
                }
            } else {
#pragma unroll
                for (int tq = 0; tq < P::TPL; tq += 4) {
                    floatx2 kd[4], km[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int tt = tq + j, t = t0 + tt;
                        G = fma2(ld_g(t), LOG2E, G);
                        const floatx2 kk = ld_k(t);
                        const floatx2 e0 = pow2v(G), em = pow2v(G - mid), eim = pow2v(mid - G);
                        km[j] = kk * eim;  // K_dec_mid = k e^(G_15 - G), t <= 15
                        if constexpr (OUT) {
                            const floatx2 qq = ld_q(t);
                            put(QO, tt, qq * e0);
                            put(QM, tt, qq * em);
                        }
                        put(KO, tt, kk * e0);
                        put(KMm, tt, kk * em);
                        put(KH, tt, kk * eim);
                        kd[j] = kk * pow2v(tot - G);
                    }
                    store_kd4(t0 + tq, kd);
                    if constexpr (CKP)
                        if (t0 < 16) store_kdm4(t0 + tq, km);
                }
            }
        }
        lds_barrier();  // B2

        // ---- K3: Gram tiles.  Waves 0, 1: block (I, I) of -beta A and its
        // inverse; wave 2: block (1, 0) of -beta A and of P; wave 3: the
        // diagonal blocks of P
        if (act) {
            const TI* rk = fast ? KO : KMm;
            const TI* rq = fast ? QO : QM;
            // block (I, J) of Q~ K^^T, masked to s <= t, to PO
            auto p_tile = [&](int I, int J, const frag (&fa)[KM]) {
                frag fq[KM];
#pragma unroll
                for (int m = 0; m < KM; ++m) fq[m] = op_frag<TI, KM>(rq, I, m, lane);
                floatx4 accP = zero4();
#pragma unroll
                for (int m = 0; m < KM; ++m) accP = M::mma(fa[m], fq[m], accP);
                const int t = 16 * I + r;
                floatx4 p;
#pragma unroll
                for (int e = 0; e < 4; ++e) p[e] = (16 * J + 4 * g + e <= t) ? accP[e] : 0.f;
                bf16* dst = reinterpret_cast<bf16*>(PO) + (I * 64 + op_slot(I, 0, r, g)) * 8 + 4 * J;
                *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3]};
                if (I == 0) *reinterpret_cast<bf16x4*>(dst + 4) = bf16x4{};  // block above the diagonal
            };
            // block (I, J) of -beta_t A[t][s], s < t; lane r + 16g: row t, columns 16J + 4g + e
            auto a_tile = [&](int I, int J, const frag (&fa)[KM]) {
                frag fk[KM];
#pragma unroll
                for (int m = 0; m < KM; ++m) fk[m] = op_frag<TI, KM>(rk, I, m, lane);
                floatx4 accA = zero4();
#pragma unroll
                for (int m = 0; m < KM; ++m) accA = M::mma(fa[m], fk[m], accA);
                const int t = 16 * I + r;
                const float bt = BETA[t];
                floatx4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (16 * J + 4 * g + e < t) ? -bt * accA[e] : 0.f;
                return x;
            };
            auto kh = [&](int J, frag (&fa)[KM]) {
#pragma unroll
                for (int m = 0; m < KM; ++m) fa[m] = op_frag<TI, KM>(KH, J, m, lane);
            };
            frag fa[KM];
            if (kw < 2) {
                kh(kw, fa);
                AN[kw * 64 + lane] = a_tile(kw, kw, fa);
                // (transition maps: inverted at the start of the next iteration,
                // where the key side has more slack)
                if constexpr (OUT) {
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS operations of a wave complete in order
                    inverse_to(TB);
                }
            } else if (kw == 2) {
                kh(0, fa);
                const floatx4 x = a_tile(1, 0, fa);
                TB[2 * 64 + lane] = frag{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3], (bf16)0.f, (bf16)0.f,
                                         (bf16)0.f, (bf16)0.f};
                if constexpr (OUT) p_tile(1, 0, fa);
            } else if constexpr (OUT) {
                kh(0, fa);
                p_tile(0, 0, fa);
                kh(1, fa);
                p_tile(1, 1, fa);
            }
        }
        lds_barrier();  // B3
    }
}

// Key side with one gate per (token, head): the decay of a pair (t, s) is the
// scalar e^{G_t - G_s}, so it multiplies the products instead of the operands.
// The chunk's q and k go to the operand layouts unscaled (no exponential per
// element); the Gram blocks are scaled by the 32 x 32 decay matrix; the state
// side scales rows by e^{G_t} and e^{G_L - G_t} (exponentials of non-positive
// numbers only, so there is no exponent budget to keep).
template <int DK, int DV, bool MAP, int NCB>
__device__ __forceinline__ void ws_key_head(const Args<bf16>& a, char* smem, int kw, int h, int64_t tb, int64_t te,
                                            int nch) {
    typedef CfgW<DK, DV, NCB> P;
    typedef bf16 TI;
    typedef Mma<bf16> M;
    typedef bf16x8 frag;
    constexpr bool OUT = !MAP;
    constexpr int CW = P::CW, KM = P::KM;
    const int H = a.H;
    char* stg = smem + P::OFF_STG;
    float* stg_gs = reinterpret_cast<float*>(stg);  // the chunk's gates (the per-channel g area is not used)
    const TI* stg_q = reinterpret_cast<const TI*>(stg + P::SG_G);
    const TI* stg_k = reinterpret_cast<const TI*>(stg + P::SG_G + P::SG_Q);
    float* stg_b = reinterpret_cast<float*>(stg + P::SG_G + 2 * P::SG_Q);
    floatx4* AN = reinterpret_cast<floatx4*>(smem + P::OFF_AN);
    float* s_gs = reinterpret_cast<float*>(smem + P::OFF_GT);  // gates of chunk i [CW]
    float* s_G = s_gs + CW;                                     // G_t of chunk i [CW]

    auto inverse_to = [&](frag* tb) {
        const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
        float arow[16];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const floatx4 y = AN[kw * 64 + r + 16 * gg];
#pragma unroll
            for (int e = 0; e < 4; ++e) arow[4 * gg + e] = y[e];
        }
        const floatx4 li = row_inverse(arow, r, g);
        tb[kw * 64 + lane] =
            frag{(bf16)li[0], (bf16)li[1], (bf16)li[2], (bf16)li[3], (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    };

    // copy of chunk j's q, k rows TPW*kw .. TPW*kw+TPW-1; wave 0 beta, wave 1 the gates
    auto dma = [&](int j, int lane) {
        const int64_t c0 = tb + (int64_t)j * CW;
        const int L = (int)(te - c0 < CW ? te - c0 : CW);
        const size_t tok0 = (size_t)c0 * H + h;
        auto rows = [&](const void* src, int RB, char* dst) {
            const int lpr = RB / 16, rpi = 64 / lpr;
            const char* base = static_cast<const char*>(src) + tok0 * RB;
#pragma unroll
            for (int i = 0; i < P::TPW / rpi; ++i) {
                const int r0 = P::TPW * kw + rpi * i;
                const int t = min(r0 + lane / lpr, L - 1);
                __builtin_amdgcn_global_load_lds(gptr(base + (uint32_t)(t * H * RB + (lane % lpr) * 16)),
                                                 lptr(dst + r0 * RB), 16, 0, 0);
            }
        };
        if (OUT) rows(a.q, DK * 2, stg + P::SG_G);
        rows(a.k, DK * 2, stg + P::SG_G + P::SG_Q);
        if (kw < 2)
            __builtin_amdgcn_global_load_lds(gptr((kw == 0 ? a.beta : a.g) + tok0 + (size_t)min(lane, L - 1) * H),
                                             lptr(kw == 0 ? stg_b : stg_gs), 4, 0, 0);
    };
    if (nch > 0) dma(0, threadIdx.x & 63);

    for (int i = 0; i <= nch; ++i) {
        int tid = kw * 64 + (threadIdx.x & 63);
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
        const int cp = tid % P::CPR, grp = tid / P::CPR, ch = 2 * cp, t0 = grp * P::TPL;
        const bool act = i < nch;
        char* buf = smem + (i & 1) * P::SZ_BUF;
        TI* QO = reinterpret_cast<TI*>(buf + P::B_QO);
        TI* KO = reinterpret_cast<TI*>(buf + P::B_KO);
        TI* KD = reinterpret_cast<TI*>(buf + P::B_KD);
        TI* PO = reinterpret_cast<TI*>(buf + P::B_PO);
        frag* TB = reinterpret_cast<frag*>(buf + P::B_TB);
        float* BETA = reinterpret_cast<float*>(buf + P::B_BETA);
        float* EG = reinterpret_cast<float*>(buf + P::B_EG);
        const int64_t c0 = tb + (int64_t)i * CW;
        const int L = (int)(te - c0 < CW ? te - c0 : CW);

        // ---- K1: this wave's rows to registers; beta and the gates (zero past
        // the end) out of the staging area; the next chunk's copy
        bf16x2 kv[P::TPL], qv[P::TPL];
        if (act) {
            __builtin_amdgcn_s_waitcnt(0);
            if (L < CW) {
                for (int t = P::TPW * kw; t < P::TPW * (kw + 1); ++t)
                    if (t >= L && lane < DK / 8) {
                        reinterpret_cast<floatx4*>(const_cast<TI*>(stg_q) + t * DK)[lane] = zero4();
                        reinterpret_cast<floatx4*>(const_cast<TI*>(stg_k) + t * DK)[lane] = zero4();
                    }
            }
#pragma unroll
            for (int tt = 0; tt < P::TPL; ++tt) {
                kv[tt] = *reinterpret_cast<const bf16x2*>(stg_k + (t0 + tt) * DK + ch);
                if constexpr (OUT) qv[tt] = *reinterpret_cast<const bf16x2*>(stg_q + (t0 + tt) * DK + ch);
            }
            if (kw == 0 && lane < CW) BETA[lane] = lane < L ? stg_b[lane] : 0.f;
            if (kw == 1 && lane < CW) s_gs[lane] = lane < L ? stg_gs[lane] : 0.f;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (i + 1 < nch) dma(i + 1, lane);
        }
        if constexpr (MAP)
            if (i >= 1 && kw < 2) inverse_to(reinterpret_cast<frag*>(smem + ((i - 1) & 1) * P::SZ_BUF + P::B_TB));
        lds_barrier();  // B1

        // ---- K2: q, k unscaled into the operand layouts; wave 3: G_t and the
        // decay vectors of the state side
        if (act) {
            const uint32_t a0 = op_idx<TI, KM>(t0, ch) * 2u;
            auto put = [&](TI* mat, int tt, bf16x2 x) {
                *reinterpret_cast<bf16x2*>(reinterpret_cast<char*>(mat) + (a0 ^ (uint32_t)(tt << 4))) = x;
            };
#pragma unroll
            for (int tt = 0; tt < P::TPL; ++tt) {
                if constexpr (OUT) put(QO, tt, qv[tt]);
                put(KO, tt, kv[tt]);
            }
#pragma unroll
            for (int tq = 0; tq < P::TPL; tq += 4) {
                *reinterpret_cast<bf16x4*>(KD + op_idx<TI, 1>(ch, t0 + tq)) =
                    bf16x4{kv[tq][0], kv[tq + 1][0], kv[tq + 2][0], kv[tq + 3][0]};
                *reinterpret_cast<bf16x4*>(KD + op_idx<TI, 1>(ch + 1, t0 + tq)) =
                    bf16x4{kv[tq][1], kv[tq + 1][1], kv[tq + 2][1], kv[tq + 3][1]};
            }
            if (kw == 3) {
                // inclusive prefix of the gates over lanes 0 .. CW-1 (rows past
                // the end hold 0): log-step scan through lane shuffles
                float G = lane < CW ? s_gs[lane] : 0.f;
#pragma unroll
                for (int off = 1; off < CW; off <<= 1) {
                    const float y = __shfl_up(G, off, 64);
                    if (lane >= off) G += y;
                }
                const float GL = __shfl(G, CW - 1, 64);
                if (lane < CW) {
                    s_G[lane] = G;
                    EG[lane] = __expf(G);
                    EG[CW + lane] = __expf(GL - G);
                }
                if (lane == 0) EG[2 * CW] = __expf(GL);
            }
        }
        lds_barrier();  // B2

        // ---- K3: Gram blocks of the unscaled q, k, times the decay e^{G_t - G_s}
        if (act) {
            // lane r + 16g of block (I, J): row t = 16I + r, columns s = 16J + 4g + e
            auto decay = [&](int I, int J) {
                const float Gt = s_G[16 * I + r];
                const floatx4 Gs = *reinterpret_cast<const floatx4*>(s_G + 16 * J + 4 * g);
                floatx4 d;
#pragma unroll
                for (int e = 0; e < 4; ++e) d[e] = __expf(Gt - Gs[e]);
                return d;
            };
            auto p_tile = [&](int I, int J, const frag (&fa)[KM]) {
                frag fq[KM];
#pragma unroll
                for (int m = 0; m < KM; ++m) fq[m] = op_frag<TI, KM>(QO, I, m, lane);
                floatx4 accP = zero4();
#pragma unroll
                for (int m = 0; m < KM; ++m) accP = M::mma(fa[m], fq[m], accP);
                const int t = 16 * I + r;
                const floatx4 d = decay(I, J);
                floatx4 p;
#pragma unroll
                for (int e = 0; e < 4; ++e) p[e] = (16 * J + 4 * g + e <= t) ? d[e] * accP[e] : 0.f;
                bf16* dst = reinterpret_cast<bf16*>(PO) + (I * 64 + op_slot(I, 0, r, g)) * 8 + 4 * J;
                *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3]};
                if (I == 0) *reinterpret_cast<bf16x4*>(dst + 4) = bf16x4{};  // block above the diagonal
            };
            auto a_tile = [&](int I, int J, const frag (&fa)[KM]) {
                frag fk[KM];
#pragma unroll
                for (int m = 0; m < KM; ++m) fk[m] = op_frag<TI, KM>(KO, I, m, lane);
                floatx4 accA = zero4();
#pragma unroll
                for (int m = 0; m < KM; ++m) accA = M::mma(fa[m], fk[m], accA);
                const int t = 16 * I + r;
                const float bt = BETA[t];
                const floatx4 d = decay(I, J);
                floatx4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (16 * J + 4 * g + e < t) ? -bt * d[e] * accA[e] : 0.f;
                return x;
            };
            auto kf = [&](int J, frag (&fa)[KM]) {
#pragma unroll
                for (int m = 0; m < KM; ++m) fa[m] = op_frag<TI, KM>(KO, J, m, lane);
            };
            frag fa[KM];
            if (kw < 2) {
                kf(kw, fa);
                AN[kw * 64 + lane] = a_tile(kw, kw, fa);
                if constexpr (OUT) {
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS operations of a wave complete in order
                    inverse_to(TB);
                }
            } else if (kw == 2) {
                kf(0, fa);
                const floatx4 x = a_tile(1, 0, fa);
                TB[2 * 64 + lane] = frag{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3], (bf16)0.f, (bf16)0.f,
                                         (bf16)0.f, (bf16)0.f};
                if constexpr (OUT) p_tile(1, 0, fa);
            } else if constexpr (OUT) {
                kf(0, fa);
                p_tile(0, 0, fa);
                kf(1, fa);
                p_tile(1, 1, fa);
            }
        }
        lds_barrier();  // B3
    }
}

// State side: waves NK .. NK+NS-1.  Runs chunk i-1 in iteration i.
// CKP: stores the state at the start of each 16-token window of the chunk in
// bf16 (checkpoints for the backward): the chunk's start state, and the state
// after token 15, diag(e^{G_15}) S + K_dec_mid^T U_0 (U_0: rows 0 .. 15 of U).
template <int DK, int DV, bool MAP, int NCB, bool HG, bool QH = false, bool CKP = false>
__device__ __forceinline__ void ws_state(const Args<bf16>& a, char* smem, int sw, const Unit& u, int nch) {
    typedef CfgW<DK, DV, NCB> P;
    typedef bf16 TI;
    typedef Mma<bf16> M;
    typedef bf16x8 frag;
    constexpr bool OUT = !MAP || QH;
    static_assert(!QH || (MAP && NCB == 2 && DK == DV), "q^ from the M block of a two-block transition pass");
    static_assert(!CKP || (MAP && NCB == 1 && !HG && !QH), "checkpoints: one state block, per-channel gates");
    constexpr int CW = P::CW, KM = P::KM, RT = P::RT;
    const int H = a.H, h = u.h;
    const int64_t tb = u.tb, te = u.te;
    const int col0 = 16 * sw;
    const uint32_t vrow = (uint32_t)H * DV;
    const int r0 = threadIdx.x & 15, g0 = (threadIdx.x & 63) >> 4;

    // fp32 state: S[cb][rt][i] = S[16 rt + 4g + i][col0 + r] (NCB = 2: [0] the M part from I, [1] the N part)
    floatx4 S[NCB][RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * g0 + i;
            S[0][rt][i] = u.s0 ? at<float>(u.s0, (row * DV + col0 + r0) * 4) : (u.eye && row == col0 + r0) ? 1.f : 0.f;
            if constexpr (NCB == 2) S[1][rt][i] = 0.f;
        }
    const bool vuse = !u.vzero;
    // v of chunk j in accumulator layout: vr[I][i] = v[16I + 4g + i][col0 + r] (rows clamped to the chunk)
    TI vnext[2][4];
    auto load_v = [&](int j, int g, int r) {
        const int64_t c0 = tb + (int64_t)j * CW;
        const int L = (int)(te - c0 < CW ? te - c0 : CW);
        const TI* vb = a.v + ((size_t)c0 * H + h) * DV;
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = min(16 * I + 4 * g + i, L - 1);
                vnext[I][i] = vuse ? at<TI>(vb, (t * vrow + col0 + r) * 2u) : TI(0.f);
            }
    };
    if (nch > 0) load_v(0, g0, r0);

    // CKP: a checkpoint slot holds the state in column blocks: the 16 columns of
    // state wave s are block s, d_k rows of 32 bytes (element (i, c) at
    // ((c / 16) d_k + i) 16 + c % 16), so each wave's part is one contiguous
    // 4 KiB.  The wave assembles it in its own LDS area, in the same layout, and
    // copies it out with 16-byte stores (whole cache lines).
    char* ckst = smem + P::LDS + sw * DK * 32;
    // rows of 16-row tile rt from this lane's rows as bf16 pairs (p01: rows 4g,
    // 4g+1 of column col0 + r; p23: rows 4g+2, 4g+3) into the wave's area.  A
    // lane and its neighbour r ^ 1 swap one pair (DPP quad_perm [1, 0, 3, 2]),
    // so each writes two whole 4-byte words: the even lane rows 4g, 4g+1 and
    // the odd lane rows 4g+2, 4g+3 of columns (r & ~1, r | 1).
    auto ck_put = [&](int rt, uint32_t p01, uint32_t p23, int r, int g) {
        const bool odd = (r & 1) != 0;
        const uint32_t send = odd ? p01 : p23, own = odd ? p23 : p01;
        const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xf, 0xf, false);
        const uint32_t lo = odd ? recv : own, hi = odd ? own : recv;
        char* dst = ckst + (16 * rt + 4 * g + (odd ? 2 : 0)) * 32 + (r & ~1) * 2;
        *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        *reinterpret_cast<uint32_t*>(dst + 32) = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
    };
    // the wave's assembled block to its place in the slot (LDS operations of a
    // wave complete in order, so the reads see this wave's writes)
    auto ck_flush = [&](__amdgpu_buffer_rsrc_t rs, int lane) {
#pragma unroll
        for (int k = 0; k < DK * 32 / 1024; ++k) {
            const uint32_t off = (uint32_t)(k * 1024 + lane * 16);
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(ckst + off), rs,
                                                   (uint32_t)(sw * DK * 32) + off, 0, 0);
        }
    };
    auto pack2 = [](float x, float y) { return __builtin_bit_cast(uint32_t, bf16x2{(bf16)x, (bf16)y}); };

    for (int i = 0; i <= nch; ++i) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
        const bool act = i >= 1;
        const int j = i - 1;
        const char* buf = smem + (j & 1) * P::SZ_BUF;
        const TI* QO = reinterpret_cast<const TI*>(buf + P::B_QO);
        const TI* KO = reinterpret_cast<const TI*>(buf + P::B_KO);
        const TI* KD = reinterpret_cast<const TI*>(buf + P::B_KD);
        const TI* PO = reinterpret_cast<const TI*>(buf + P::B_PO);
        const frag* TB = reinterpret_cast<const frag*>(buf + P::B_TB);
        const float* BETA = reinterpret_cast<const float*>(buf + P::B_BETA);
        const float* GM = reinterpret_cast<const float*>(buf + P::B_GM);
        const float* EG = reinterpret_cast<const float*>(buf + P::B_EG);  // per-head gates
        const int64_t c0 = tb + (int64_t)j * CW;
        const int L = (int)(te - c0 < CW ? te - c0 : CW);

        TI vr[2][4];
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
            for (int e = 0; e < 4; ++e) vr[I][e] = vnext[I][e];
        if (i < nch) load_v(i, g, r);
        // CKP: the slot of the chunk's window w (0, 1); the second one's extent is
        // zero when the chunk has no second window, so its stores are dropped
        // (the count of stores per iteration is fixed)
        auto ck_slot = [&](int w) {
            TI* p = static_cast<TI*>(u.ck) + (size_t)(2 * (act ? j : 0) + w) * H * DK * DV;
            return __builtin_amdgcn_make_buffer_rsrc(p, 0, w == 0 || L > 16 ? DK * DV * 2 : 0, BUFFER_RSRC_WORD3);
        };

        // ---- S1: K~ S and the right-hand side beta (V - K~ S)
        frag bS[NCB][KM];
        floatx4 R[NCB][2];
        if (act) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const bool vblock = NCB == 1 || cb == 1;
#pragma unroll
                for (int m = 0; m < KM; ++m) bS[cb][m] = acc_perm<TI>(S[cb], m, RT);
                if constexpr (CKP) {
                    // bS[m] holds rows 4g .. 4g+3 of tiles 2m and 2m + 1 in bf16
#pragma unroll
                    for (int m = 0; m < KM; ++m) {
                        const u32x4 w = __builtin_bit_cast(u32x4, bS[cb][m]);
                        ck_put(2 * m, w[0], w[1], r, g);
                        ck_put(2 * m + 1, w[2], w[3], r, g);
                    }
                    ck_flush(ck_slot(0), lane);
                }
#pragma unroll
                for (int I = 0; I < 2; ++I) {
                    floatx4 ks = zero4();
#pragma unroll
                    for (int m = 0; m < KM; ++m) ks = M::mma(op_frag<TI, KM>(KO, I, m, lane), bS[cb][m], ks);
                    if constexpr (HG) ks *= *reinterpret_cast<const floatx4*>(EG + 16 * I + 4 * g);  // rows t: e^{G_t}
                    const floatx4 bt = *reinterpret_cast<const floatx4*>(BETA + 16 * I + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) R[cb][I][e] = bt[e] * ((vblock ? (float)vr[I][e] : 0.f) - ks[e]);
                }
            }
        }
        lds_barrier();  // B1

        // ---- S2: U by block forward substitution; outputs
        frag bU[NCB], bUs[NCB];  // bUs: rows t scaled by e^{G_L - G_t} (per-head gates)
        if (act) {
            const frag l0 = TB[lane], l1 = TB[64 + lane], an = TB[128 + lane];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                floatx4 U[2];
                U[0] = M::mma(l0, acc_perm<TI>(&R[cb][0], 0, 1), zero4());
                const floatx4 r1 = M::mma(an, acc_perm<TI>(U, 0, 1), R[cb][1]);
                U[1] = M::mma(l1, acc_perm<TI>(&r1, 0, 1), zero4());
                bU[cb] = acc_perm<TI>(U, 0, 2);
                if constexpr (CKP) {
                    // the state after token 15: U_0 in accumulator layout is the B
                    // operand of a 16-token product as it is
                    const TI* KDM = reinterpret_cast<const TI*>(buf + P::B_QO);
                    const float* GMM = reinterpret_cast<const float*>(buf + P::B_PO);
                    const bf16x4 bu0 = bf16x4{(bf16)U[0][0], (bf16)U[0][1], (bf16)U[0][2], (bf16)U[0][3]};
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        floatx4 sm = S[cb][rt] * *reinterpret_cast<const floatx4*>(GMM + 16 * rt + 4 * g);
                        sm = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                            *reinterpret_cast<const bf16x4*>(KDM + (rt * 64 + kdm_slot(rt, r, g)) * 4), bu0, sm, 0, 0, 0);
                        ck_put(rt, pack2(sm[0], sm[1]), pack2(sm[2], sm[3]), r, g);
                    }
                    ck_flush(ck_slot(1), lane);
                }
                if constexpr (HG) {
#pragma unroll
                    for (int I = 0; I < 2; ++I) U[I] *= *reinterpret_cast<const floatx4*>(EG + CW + 16 * I + 4 * g);
                    bUs[cb] = acc_perm<TI>(U, 0, 2);
                }
            }
            if constexpr (OUT) {
                // O = Q~ S + P U from the state at the chunk start (bS) and U,
                // with buffer stores: rows t >= L lie past the extent of the
                // resource and the hardware drops them, so every lane stores
                // (no branch, and the count of stores in flight is fixed).
                // QH: the same product of the M block (block 0) is q^ (d_k = d_v,
                // so its rows have vrow elements too), stored for every segment
                // (the first segment's is not used; skipping it costs registers).
                const __amdgpu_buffer_rsrc_t ob = __builtin_amdgcn_make_buffer_rsrc(
                    (QH ? a.qh : a.o) + ((size_t)c0 * H + h) * DV, 0, L * vrow * 2, BUFFER_RSRC_WORD3);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    floatx4 O = zero4();
#pragma unroll
                    for (int m = 0; m < KM; ++m) O = M::mma(bS[0][m], op_frag<TI, KM>(QO, rb, m, lane), O);
                    if constexpr (HG) O *= EG[16 * rb + r];  // this lane's token: e^{G_t}
                    O = M::mma(bU[0], op_frag<TI, 1>(PO, rb, 0, lane), O);
                    const int t = 16 * rb + r;
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(u32x2, bf16x4{(bf16)O[0], (bf16)O[1], (bf16)O[2], (bf16)O[3]}), ob,
                        (t * vrow + col0 + 4 * g) * 2u, 0, 0);
                }
            }
        }
        lds_barrier();  // B2

        // ---- S3: S <- diag(gamma) S + K_dec^T U
        if (act) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    if constexpr (HG) {
                        S[cb][rt] *= EG[2 * CW];  // e^{G_L}
                        S[cb][rt] = M::mma(op_frag<TI, 1>(KD, rt, 0, lane), bUs[cb], S[cb][rt]);
                    } else {
                        const floatx4 d = *reinterpret_cast<const floatx4*>(GM + 16 * rt + 4 * g);
                        S[cb][rt] *= d;
                        S[cb][rt] = M::mma(op_frag<TI, 1>(KD, rt, 0, lane), bU[cb], S[cb][rt]);
                    }
                }
            }
        }
        lds_barrier();  // B3
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        float* dst = cb == 0 ? u.sf : u.sf2;
        if (dst) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    at_mut<float>(dst, ((16 * rt + 4 * g0 + i) * DV + col0 + r0) * 4) = S[cb][rt][i];
        }
    }
}

// GMODE 0: per-channel g; 1: per-channel g from bf16 logits (Args::z, gate,
// gate_param); 2: one g per (token, head) (Args::g is [T, H])
// QH (MAP, NCB = 2, per-channel gates): the transition pass of the
// backward's time split, which also forms q^ and takes the split sequences'
// last segments.
template <int DK, int DV, bool MAP, int NCB, int GMODE, bool QH = false, bool CKP = false>
__global__ __launch_bounds__((CfgW<DK, DV, NCB>::NT), 1) void prefill_ws_kernel(Args<bf16> a) {
    typedef CfgW<DK, DV, NCB> P;
    static_assert(NCB == 1 || (MAP && DK == DV), "two column blocks only for transitions with d_k = d_v");
    static_assert(!QH || GMODE == 0, "q^ transition pass: per-channel gates");
    static_assert(!CKP || (MAP && NCB == 1 && GMODE == 0 && !QH), "checkpoint pass");
    // (CKP: after the layout, each state wave's area for assembling checkpoints)
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS + (CKP ? P::NS * DK * 32 : 0)];
    const Unit u = resolve_unit<bf16, DK, DV, MAP, NCB, QH, CKP>(a, blockIdx.x);
    if (!u.valid) return;
    const int nch = (int)((u.te - u.tb + P::CW - 1) / P::CW);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w < P::NK) {
        if constexpr (GMODE == 2) ws_key_head<DK, DV, MAP, NCB>(a, smem, w, u.h, u.tb, u.te, nch);
        else ws_key<DK, DV, MAP, NCB, GMODE == 1, QH, CKP>(a, smem, w, u.h, u.tb, u.te, nch);
    } else {
        ws_state<DK, DV, MAP, NCB, GMODE == 2, QH, CKP>(a, smem, w - P::NK, u, nch);
    }
}

// nl[0] = 0, nl[n + 1] = nl[n] + (number of non-last segments of sequence n):
// a sequence of len > 0 tokens has ceil(len / seg) segments, an empty one has
// one (of zero tokens).  spl[0 .. splits): the sequences with more than one
// segment in increasing order, then -1 (a list longer than `splits`, which
// well-formed lengths cannot give, is cut there).  One workgroup, block-wide
// scans per 256 sequences.
__global__ __launch_bounds__(256) void seg_table_kernel(const int32_t* __restrict__ cu, int num_seqs, int seg,
                                                        int32_t* __restrict__ nl, int32_t* __restrict__ spl,
                                                        int splits) {
    __shared__ int part[256], pf[256];
    const int t = threadIdx.x;
    int carry = 0, carryf = 0;
    if (t == 0) nl[0] = 0;
    for (int base = 0; base < num_seqs; base += 256) {
        const int n = base + t;
        int c = 0;
        if (n < num_seqs) {
            const int len = cu[n + 1] - cu[n];
            c = len > 0 ? (len - 1) / seg : 0;
        }
        part[t] = c;
        pf[t] = c > 0;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int x = t >= off ? part[t - off] : 0, y = t >= off ? pf[t - off] : 0;
            __syncthreads();
            part[t] += x;
            pf[t] += y;
            __syncthreads();
        }
        if (n < num_seqs) {
            nl[n + 1] = carry + part[t];
            const int pos = carryf + pf[t] - 1;
            if (c > 0 && pos < splits) spl[pos] = n;
        }
        carry += part[255];
        carryf += pf[255];
        __syncthreads();
    }
    for (int k = carryf + t; k < splits; k += 256) spl[k] = -1;
}

// Order of the sequences for a pass with one workgroup per (sequence, head):
// longest first, so that the longest chains are dispatched first (a pass over
// many units of mixed lengths otherwise ends on a long unit that started
// late).  The key of a sequence is the bucket of its length in 64-token chunks
// (capped at `cap` tokens when cap > 0: a first segment is at most one
// segment long), four buckets per octave, 0 for an empty sequence; ord lists
// the buckets from the highest down, each in increasing sequence index, so the
// order is deterministic.  One workgroup: a histogram of the keys, a scan over
// the buckets, then the placement, 1024 sequences per step (the lanes of a wave
// that share a key are found with one ballot per key bit; the waves' counts
// per key are summed in LDS).
constexpr int kOrderBuckets = 128;  // keys 0 .. 104 (and one value for idle lanes)
__device__ __forceinline__ int order_key(int len, int cap) {
    if (cap > 0 && len > cap) len = cap;
    if (len <= 0) return 0;
    const unsigned c = ((unsigned)len + 63u) / 64u;
    const int e = 31 - __builtin_clz(c);
    const int sub = e >= 2 ? (int)(c >> (e - 2)) & 3 : (int)(c << (2 - e)) & 3;
    return 1 + 4 * e + sub;
}
__global__ __launch_bounds__(1024) void seq_order_kernel(const int32_t* __restrict__ cu, int num_seqs, int cap,
                                                         int32_t* __restrict__ ord, int seg,
                                                         int32_t* __restrict__ pfx) {
    constexpr int NB = kOrderBuckets, NWV = 16;
    __shared__ int hist[NB], start[NB], done[NB];
    __shared__ int cnt[NWV][NB];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    if (t < NB) {
        hist[t] = 0;
        done[t] = 0;
    }
    for (int i = t; i < NWV * NB; i += 1024) (&cnt[0][0])[i] = 0;
    __syncthreads();
    for (int n = t; n < num_seqs; n += 1024) atomicAdd(&hist[order_key(cu[n + 1] - cu[n], cap)], 1);
    __syncthreads();
    if (t == 0) {
        int acc = 0;
        for (int k = NB - 1; k >= 0; --k) {
            start[k] = acc;
            acc += hist[k];
        }
    }
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int base = 0; base < num_seqs; base += 1024) {
        const int n = base + t;
        const bool valid = n < num_seqs;
        const int key = valid ? order_key(cu[n + 1] - cu[n], cap) : NB;  // NB: idle lanes, a key of their own
        unsigned long long same = ~0ull;
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (key >> bit) & 1;
            const unsigned long long m = __ballot(on);
            same &= on ? m : ~m;
        }
        const int rank = __popcll(same & below);
        if (valid && rank == 0) cnt[w][key] = __popcll(same);
        __syncthreads();
        if (valid) {
            int pos = start[key] + done[key] + rank;
            for (int v = 0; v < w; ++v) pos += cnt[v][key];
            ord[pos] = n;
        }
        __syncthreads();
        if (t < NB) {
            int sum = 0;
            for (int v = 0; v < NWV; ++v) {
                sum += cnt[v][t];
                cnt[v][t] = 0;
            }
            done[t] += sum;
        }
        __syncthreads();
    }
    if (!pfx) return;
    // pfx[i] = segments (of seg tokens; an empty sequence has one) of the
    // sequences ord[0 .. i-1]: the workgroups of a pass over every segment
    // take the sequences in this order (ord, written above by other threads
    // of this workgroup, is read back after the barrier)
    __syncthreads();
    __shared__ int part[1024];
    int carry = 0;
    if (t == 0) pfx[0] = 0;
    for (int base = 0; base < num_seqs; base += 1024) {
        const int i = base + t;
        int c = 0;
        if (i < num_seqs) {
            const int m = ord[i], len = cu[m + 1] - cu[m];
            c = len > 0 ? (len - 1) / seg + 1 : 1;
        }
        part[t] = c;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int x = t >= off ? part[t - off] : 0;
            __syncthreads();
            part[t] += x;
            __syncthreads();
        }
        if (i < num_seqs) pfx[i + 1] = carry + part[t];
        carry += part[1023];
        __syncthreads();
    }
}

// Serial fold over the segments of one (sequence, head), 16 state columns per
// workgroup (columns of the state evolve independently):
//   S_start(j + 1) = M_j S_start(j) + N_j,  j >= first,
// written over N_j, from S_start(0) = S0 (or zero) when first = 0, or from
// S_start(1) already in slot N_0 (segment 0's own end state) when first = 1;
// fp32 matrix-core steps (fold_columns), one wave per 16-row tile.
template <int DK, int DV, int DEPTH = 2>
__global__ __launch_bounds__(64 * (DK / 16), DEPTH == 1 ? 2 : 1) void seg_fold_kernel(
    const int32_t* __restrict__ nl, const int32_t* __restrict__ spl, int H, const float* __restrict__ S0,
    const float* __restrict__ wsM, float* __restrict__ wsN, int first) {
    // one workgroup per (split sequence, head, 16 columns): workgroup slot
    // `us` = k H + h is head h of the k-th sequence in spl
    constexpr int NCB = DV / 16;
    int bid = blockIdx.x, cb, us;
    if ((gridDim.x / NCB) % 8 == 0) {
        // workgroups go to the eight XCDs in turn: keep the NCB column blocks
        // of a unit on one XCD, so that its L2 fetches each map once
        const int x = bid % 8, q = bid / 8;
        cb = q % NCB;
        us = (q / NCB) * 8 + x;
    } else {
        cb = bid % NCB;
        us = bid / NCB;
    }
    const int kk = us / H, h = us - kk * H, n = spl[kk];
    if (n < 0) return;
    const int unit = n * H + h;
    const int k0 = nl[n], cnt = nl[n + 1] - k0;
    if (cnt <= first) return;
    const float* x0 = first ? wsN + ((size_t)k0 * H + h) * DK * DV : S0 ? S0 + (size_t)unit * DK * DV : nullptr;
    fold_columns<DK, DV, false, DEPTH>(
        x0, cnt - first, cb, [&](int j) { return wsM + ((size_t)(k0 + first + j) * H + h) * DK * DK; },
        [&](int j) { return wsN + ((size_t)(k0 + first + j) * H + h) * DK * DV; });
}

template <int DK, int DV, bool MAP, int NCB = 1>
hipError_t launch_ws(const Args<bf16>& a, int64_t blocks, hipStream_t s) {
    typedef CfgW<DK, DV, NCB> P;
    static_assert(P::LDS <= 160 * 1024, "LDS budget");
    if (blocks <= 0) return hipSuccess;
    if (a.gate == GATE_HEAD)
        hipLaunchKernelGGL((prefill_ws_kernel<DK, DV, MAP, NCB, 2>), dim3((unsigned)blocks), dim3(P::NT), 0, s, a);
    else if (a.gate != GATE_LOG)
        hipLaunchKernelGGL((prefill_ws_kernel<DK, DV, MAP, NCB, 1>), dim3((unsigned)blocks), dim3(P::NT), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_ws_kernel<DK, DV, MAP, NCB, 0>), dim3((unsigned)blocks), dim3(P::NT), 0, s, a);
    return hipGetLastError();
}

template <typename TI, int DK, int DV, bool MAP, int NCB = 1>
hipError_t launch_seq(const Args<TI>& a, int64_t blocks, hipStream_t s) {
    typedef Cfg<TI, DK, DV> P;
    static_assert(P::LDS <= 160 * 1024, "LDS budget");
    if (blocks <= 0) return hipSuccess;
    if constexpr (sizeof(TI) == 2) {
        if (!a.legacy || a.gate != GATE_LOG) return launch_ws<DK, DV, MAP, NCB>(a, blocks, s);
    }
    auto kern = prefill_seq_kernel<TI, DK, DV, MAP, NCB>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(P::NT), 0, s, a);
    return hipGetLastError();
}

template <typename TI>
Args<TI> make_args(const PrefillLaunch& p) {
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
    a.num_seqs = p.num_seqs;
    a.seg = 0;
    a.nl = nullptr;
    a.spl = nullptr;
    a.wsM = a.wsN = nullptr;
    a.m_blocks = 0;
    a.map_from = 0;
    a.phase = 0;
    a.legacy = p.legacy;
    a.z = static_cast<const bf16*>(p.z);
    a.gate = p.gate;
    a.gate_param = p.gate_param;
    a.ord = nullptr;
    a.qh = nullptr;
    a.wsML = nullptr;
    a.pfx = nullptr;
    a.ck = nullptr;
    return a;
}

// Time split: the workspace pointers and the segment table.
template <typename TI, int DK, int DV>
hipError_t run_table(const PrefillLaunch& p, Args<TI>& a, hipStream_t s) {
    const PrefillWorkspace ws = prefill_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DV, p.seg);
    char* w = static_cast<char*>(p.workspace);
    a.seg = p.seg;
    a.nl = reinterpret_cast<int32_t*>(w + ws.nl_off);
    a.wsM = reinterpret_cast<float*>(w + ws.m_off);
    a.wsN = reinterpret_cast<float*>(w + ws.n_off);
    a.spl = reinterpret_cast<int32_t*>(w + ws.spl_off);
    hipLaunchKernelGGL(seg_table_kernel, dim3(1), dim3(256), 0, s, p.cu_seqlens, p.num_seqs, p.seg,
                       const_cast<int32_t*>(a.nl), const_cast<int32_t*>(a.spl), (int)ws.splits);
    return hipGetLastError();
}

// Time split: the maps of the non-last segments from segment a.map_from on
// (after run_table).
template <typename TI, int DK, int DV>
hipError_t run_map_pass(const PrefillLaunch& p, Args<TI>& a, hipStream_t s) {
    const PrefillWorkspace ws = prefill_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DV, p.seg);
    const int64_t map_blocks = ws.slots * p.H;
    if (map_blocks <= 0) return hipSuccess;
    // M and N in one workgroup or in two: decided for the number of transitions
    // that sequences of the mean length would have; with a bound on the lengths,
    // for the long sequences of the most skewed batch it allows; and when a
    // sequence of the mean length is not split at all (the length-agnostic
    // plan), for one sequence of all the tokens.  (The grid is sized for the
    // bound; surplus workgroups exit at once.)
    int64_t len = (p.T_total + p.num_seqs - 1) / p.num_seqs, nlen = p.num_seqs;
    if (p.max_seqlen > len) {
        len = p.max_seqlen;
        nlen = std::max<int64_t>(1, std::min<int64_t>(p.num_seqs, p.T_total / p.max_seqlen));
    } else if (len <= p.seg) {
        len = p.T_total;
        nlen = 1;
    }
    const double maps = (double)nlen * p.H * (len > 0 ? std::max<int64_t>(0, (len - 1) / p.seg - a.map_from) : 0);
    bool both = false;
    SplitCost::maps_pass(maps, p.seg / 64.0, DK == DV && sizeof(TI) == 2, &both);
    hipError_t e;
    if constexpr (DK == DV && sizeof(TI) == 2) {
        if (both) {
            e = launch_seq<TI, DK, DV, true, 2>(a, map_blocks, s);
        } else {
            a.m_blocks = (int)map_blocks;
            e = launch_seq<TI, DK, DV, true>(a, 2 * map_blocks, s);
        }
    } else {
        a.m_blocks = (int)map_blocks;
        e = launch_seq<TI, DK, DK, true>(a, map_blocks, s);
        a.m_blocks = 0;
        if (e == hipSuccess) e = launch_seq<TI, DK, DV, true>(a, map_blocks, s);
    }
    return e;
}

// Time split: the fold from segment a.map_from on, after the maps (and, when
// given, after the event before_fold).
template <typename TI, int DK, int DV>
hipError_t run_fold_pass(const PrefillLaunch& p, Args<TI>& a, hipStream_t s, hipEvent_t before_fold) {
    const PrefillWorkspace ws = prefill_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DV, p.seg);
    hipError_t e = hipSuccess;
    if (before_fold && (e = hipStreamWaitEvent(s, before_fold, 0)) != hipSuccess) return e;
    if (ws.slots > 0 && ws.splits > 0) {
        // more workgroups than CUs: the shallower prefetch, two workgroups per CU
        const int64_t wgs = ws.splits * p.H * (DV / 16);
        if (wgs > kComputeUnits)
            hipLaunchKernelGGL((seg_fold_kernel<DK, DV, 1>), dim3((unsigned)wgs), dim3(64 * (DK / 16)), 0, s, a.nl,
                               a.spl, p.H, p.initial_state, a.wsM, a.wsN, a.map_from);
        else
            hipLaunchKernelGGL((seg_fold_kernel<DK, DV, 2>), dim3((unsigned)wgs), dim3(64 * (DK / 16)), 0, s, a.nl,
                               a.spl, p.H, p.initial_state, a.wsM, a.wsN, a.map_from);
        e = hipGetLastError();
    }
    return e;
}

// Side lanes of the time split.  The output pass of every sequence's first
// segment runs on a second stream beside the maps of the later segments.  Each
// caller stream gets its own lane: a side stream (default priority) and the
// two events that fork it from and join it back into the caller's stream, all
// kept for the life of the process.  A lane is held by one call while that call
// enqueues; a call takes the idle lane already keyed to its stream, else a new
// lane while a device has fewer than kLanesKept, else the idle lane used least
// recently whose side stream is not inside a graph capture, else a new lane.
// Calls on different caller streams therefore do not share a side stream unless
// more than kLanesKept caller streams are in use, and a side stream that joined
// one thread's capture is never handed to another call until that capture ends.
struct SideLane {
    int dev = 0;
    hipStream_t caller = nullptr;
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool busy = false;
    uint64_t last_use = 0;
};

constexpr int kLanesKept = 16;

class SideLanes {
  public:
    hipError_t acquire(hipStream_t caller, SideLane** out) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        std::lock_guard<std::mutex> lock(mu_);
        SideLane* pick = nullptr;
        int on_dev = 0;
        for (auto& l : lanes_) {
            if (l->dev != dev) continue;
            ++on_dev;
            if (!l->busy && l->caller == caller) { pick = l.get(); break; }
        }
        if (!pick && on_dev >= kLanesKept) {
            for (auto& l : lanes_) {
                if (l->dev != dev || l->busy || (pick && l->last_use >= pick->last_use)) continue;
                hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
                if (hipStreamIsCapturing(l->side, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) pick = l.get();
            }
        }
        if (!pick) {
            auto l = std::make_unique<SideLane>();
            l->dev = dev;
            if ((e = hipStreamCreateWithFlags(&l->side, hipStreamNonBlocking)) != hipSuccess) return e;
            if ((e = hipEventCreateWithFlags(&l->fork, hipEventDisableTiming)) != hipSuccess ||
                (e = hipEventCreateWithFlags(&l->join, hipEventDisableTiming)) != hipSuccess) {
                if (l->fork) (void)hipEventDestroy(l->fork);
                (void)hipStreamDestroy(l->side);
                return e;
            }
            pick = l.get();
            lanes_.push_back(std::move(l));
        }
        pick->caller = caller;
        pick->busy = true;
        pick->last_use = ++clock_;
        *out = pick;
        return hipSuccess;
    }
    void release(SideLane* l) {
        std::lock_guard<std::mutex> lock(mu_);
        l->busy = false;
    }

  private:
    std::mutex mu_;
    std::vector<std::unique_ptr<SideLane>> lanes_;
    uint64_t clock_ = 0;
};

SideLanes& side_lanes() {
    static SideLanes* lanes = new SideLanes();  // never destroyed: streams may still run at exit
    return *lanes;
}

template <typename TI, int DK, int DV>
hipError_t run(const PrefillLaunch& p, hipStream_t s) {
    Args<TI> a = make_args<TI>(p);
    const int64_t units = (int64_t)p.num_seqs * p.H;
    const PrefillWorkspace wl = prefill_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DV, p.seg);
    if (wl.ord) {
        // longest sequences first (for the pass over whole sequences, or over first segments)
        int32_t* ord = reinterpret_cast<int32_t*>(static_cast<char*>(p.workspace) + wl.ord_off);
        const hipError_t e = launch_seq_order(p.cu_seqlens, p.num_seqs, p.seg, ord, s);
        if (e != hipSuccess) return e;
        a.ord = ord;
    }
    if (p.seg <= 0) return launch_seq<TI, DK, DV, false>(a, units, s);

    // Time split.  Segment 0 of every sequence needs no map: its own output
    // pass (on the side stream, after the table) gives the start state of
    // segment 1 while the maps of segments 1 .. last-1 run on the caller's
    // stream; the fold then starts at segment 1 and the output pass of the
    // remaining segments follows.  Segment 0 is done before any later segment
    // writes a final state, so a final state that aliases the initial state
    // needs no copy.
    SideLane* lane = nullptr;
    hipError_t e = side_lanes().acquire(s, &lane);
    if (e != hipSuccess) return e;
    hipStream_t s2 = lane->side;
    bool forked = false, joined = false;
    auto body = [&]() -> hipError_t {
        hipError_t r = run_table<TI, DK, DV>(p, a, s);
        if (r != hipSuccess) return r;
        if ((r = hipEventRecord(lane->fork, s)) != hipSuccess) return r;
        // the maps are enqueued first, so that their long chains start as soon
        // as the pass over first segments, whose units may be many and short,
        // begins beside them
        a.map_from = 1;
        if ((r = run_map_pass<TI, DK, DV>(p, a, s)) != hipSuccess) return r;
        if ((r = hipStreamWaitEvent(s2, lane->fork, 0)) != hipSuccess) return r;
        forked = true;
        a.phase = 1;
        if ((r = launch_seq<TI, DK, DV, false>(a, units, s2)) != hipSuccess) return r;
        if ((r = hipEventRecord(lane->join, s2)) != hipSuccess) return r;
        r = run_fold_pass<TI, DK, DV>(p, a, s, lane->join);
        joined = r == hipSuccess;  // the fold (or its absence) waited for the join event
        if (r != hipSuccess) return r;
        a.phase = 2;
        const int64_t slots = prefill_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DV, p.seg).slots;
        return launch_seq<TI, DK, DV, false>(a, slots * p.H, s);
    };
    e = body();
    if (forked && !joined) {
        // A step after the fork failed: join the side stream back into the
        // caller's stream all the same, so that nothing enqueued on it can
        // outlive the call's buffers in the caller's stream order (and a
        // capture is not left with an unjoined fork).  Should the event path
        // fail too, wait for the side stream on the host, unless it is being
        // captured (the capture is then invalid anyway).
        if (hipEventRecord(lane->join, s2) != hipSuccess || hipStreamWaitEvent(s, lane->join, 0) != hipSuccess) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(s2, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
                (void)hipStreamSynchronize(s2);
        }
    }
    side_lanes().release(lane);
    return e;
}

template <typename TI>
hipError_t run_t(const PrefillLaunch& p, hipStream_t s) {
    if (p.dk == 128 && p.dv == 128) return run<TI, 128, 128>(p, s);
    if (p.dk == 128 && p.dv == 64) return run<TI, 128, 64>(p, s);
    if (p.dk == 64 && p.dv == 128) return run<TI, 64, 128>(p, s);
    if (p.dk == 64 && p.dv == 64) return run<TI, 64, 64>(p, s);
    return hipErrorInvalidValue;
}

template <typename TI, int DK, int DV>
hipError_t run_maps(const PrefillLaunch& p, hipStream_t s) {
    Args<TI> a = make_args<TI>(p);
    hipError_t e = run_table<TI, DK, DV>(p, a, s);
    if (e == hipSuccess) e = run_map_pass<TI, DK, DV>(p, a, s);
    return e != hipSuccess ? e : run_fold_pass<TI, DK, DV>(p, a, s, nullptr);
}

// The backward's forward half with q^ (bf16, d_k = d_v, per-channel gates):
// the table, one transition pass over the non-last segments (slots
// 0 .. slots-1) and the split sequences' last segments (the `splits` list
// after them), then the fold from segment 0.
template <int DK>
hipError_t run_maps_q(const PrefillLaunch& p, bf16* qh, float* wsML, hipStream_t s) {
    Args<bf16> a = make_args<bf16>(p);
    hipError_t e = run_table<bf16, DK, DK>(p, a, s);
    if (e != hipSuccess) return e;
    const PrefillWorkspace ws = prefill_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DK, p.seg);
    a.qh = qh;
    a.wsML = wsML;
    a.m_blocks = (int)(ws.slots * p.H);
    if ((ws.slots + ws.splits) * p.H > 0)
        hipLaunchKernelGGL((prefill_ws_kernel<DK, DK, true, 2, 0, true>),
                           dim3((unsigned)((ws.slots + ws.splits) * p.H)), dim3(CfgW<DK, DK, 2>::NT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    a.m_blocks = 0;
    return run_fold_pass<bf16, DK, DK>(p, a, s, nullptr);
}

template <typename TI>
hipError_t run_maps_t(const PrefillLaunch& p, hipStream_t s) {
    if (p.dk == 128 && p.dv == 128) return run_maps<TI, 128, 128>(p, s);
    if (p.dk == 128 && p.dv == 64) return run_maps<TI, 128, 64>(p, s);
    if (p.dk == 64 && p.dv == 128) return run_maps<TI, 64, 128>(p, s);
    if (p.dk == 64 && p.dv == 64) return run_maps<TI, 64, 64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t s) {
    if ((int64_t)p.num_seqs * p.H == 0) return hipSuccess;
    return p.bf16 ? run_t<bf16>(p, s) : run_t<float>(p, s);
}

hipError_t launch_seq_order(const int32_t* cu_seqlens, int32_t num_seqs, int64_t cap, int32_t* ord, hipStream_t s,
                            int64_t seg, int32_t* pfx) {
    if (num_seqs <= 0) return hipSuccess;
    hipLaunchKernelGGL(seq_order_kernel, dim3(1), dim3(1024), 0, s, cu_seqlens, num_seqs,
                       (int)std::min<int64_t>(std::max<int64_t>(cap, 0), 0x7fffffff), ord,
                       (int)std::min<int64_t>(std::max<int64_t>(seg, 1), 0x7fffffff), pfx);
    return hipGetLastError();
}

hipError_t launch_prefill_maps(const PrefillLaunch& p, hipStream_t s) {
    if ((int64_t)p.num_seqs * p.H == 0 || p.seg <= 0) return hipSuccess;
    return p.bf16 ? run_maps_t<bf16>(p, s) : run_maps_t<float>(p, s);
}

namespace {

template <int DK, int DV>
hipError_t run_checkpoints(const CheckpointLaunch& c, hipStream_t s) {
    typedef CfgW<DK, DV, 1> P;
    static_assert(P::LDS + P::NS * DK * 32 <= 160 * 1024, "LDS budget");
    Args<bf16> a = {};
    a.k = static_cast<const bf16*>(c.k);
    a.v = static_cast<const bf16*>(c.v);
    a.g = c.g;
    a.beta = c.beta;
    a.cu = c.cu_seqlens;
    a.S0 = c.initial_state;
    a.H = c.H;
    a.num_seqs = c.num_seqs;
    a.seg = (int)c.seg;
    a.nl = c.nl;
    a.wsN = const_cast<float*>(c.seg_start);
    a.gate = GATE_LOG;
    a.ord = c.ord;
    a.pfx = c.pfx;
    a.ck = static_cast<bf16*>(c.ck);
    hipLaunchKernelGGL((prefill_ws_kernel<DK, DV, true, 1, 0, false, true>), dim3((unsigned)c.blocks), dim3(P::NT), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_checkpoints(const CheckpointLaunch& c, hipStream_t s) {
    if ((c.dk != 64 && c.dk != 128) || (c.dv != 64 && c.dv != 128) || c.seg < 0 || c.seg > INT32_MAX ||
        c.blocks > UINT32_MAX)
        return hipErrorInvalidValue;
    if (c.blocks <= 0) return hipSuccess;
    if (c.dk == 128) return c.dv == 128 ? run_checkpoints<128, 128>(c, s) : run_checkpoints<128, 64>(c, s);
    return c.dv == 128 ? run_checkpoints<64, 128>(c, s) : run_checkpoints<64, 64>(c, s);
}

hipError_t launch_prefill_maps_q(const PrefillLaunch& p, void* qh, float* wsML, hipStream_t s) {
    if (!p.bf16 || p.dk != p.dv || p.seg <= 0 || p.gate != GATE_LOG || (p.dk != 64 && p.dk != 128))
        return hipErrorInvalidValue;
    if ((int64_t)p.num_seqs * p.H == 0) return hipSuccess;
    return p.dk == 128 ? run_maps_q<128>(p, static_cast<bf16*>(qh), wsML, s)
                       : run_maps_q<64>(p, static_cast<bf16*>(qh), wsML, s);
}

}  // namespace gdn
