// Gradients of the chunked gated delta rule on gfx950 (reverse mode).
//
// The forward map per (sequence, head), token by token, is
//   X_t = diag(a_t) S_{t-1},  a_t = e^{g_t},  u_t = b_t (v_t - X_t^T k_t),
//   S_t = X_t + k_t u_t^T,    o_t = S_t^T q_t,
// the fixed-size state with correct-on-write updates and a position-dependent
// decay of "How to Think About Trillion-Parameter Sparse Multimodal LLMs",
// section 2.2, with the lower-bounded log-decay g in [-5, 0] of
// "Trillion-Parameter MoE Multimodal LLMs: How to Evaluate the New
// Generation", section 3.1.  The method is trained by back-propagation
// ("Architecture Evolution and Training Engineering for Trillion-Scale Sparse
// Multimodal Models", section 3.3); the pages do not write the backward pass
// out, so this file computes the plain adjoint of the forward map, organised
// in chunks of 16 tokens:
//
// Inside a 16-token sub-chunk with start state S0 and local cumulative
// log-decay G_t = sum_{r<=t} g_r (per key channel), and with m = G_7 the
// reference point of the window (the 16-token tile of the pages' bound keeps
// every factor e^{+-(G_t - m)} inside e^{+-40}):
//   q~ = q e^{G-m},  k~ = k e^{G-m},  k^ = k e^{m-G},  E = diag(e^m),
//   F = diag(e^{G_15 - m}),  gamma = e^{G_15}
//   P  = lower(q~ k^T)             KK = strict_lower(k~ k^T)
//   M  = (I + diag(b) KK)^-1
//   R  = V - k~ (E S0),  U = M diag(b) R
//   O  = q~ (E S0) + P U,  S_end = gamma S0 + F k^T U
// Given dO and dS = dL/dS_end, the adjoint of the sub-chunk is
//   dU  = P^T dO + k^ (F dS)           dRm = M^T dU,  dR = diag(b) dRm,  dv = dR
//   dA  = -strict_lower(dRm U^T)      dKK = diag(b) dA     dP = lower(dO U^T)
//   db_t = R_t . dRm_t + sum_s dA_ts KK_ts
//   dS0 = gamma dS + E (q~^T dO - k~^T dR)
//   Z = dO (E S0)^T + dP k^,  X = -dR (E S0)^T + dKK k^,
//   Y = dKK^T k~ + dP^T q~ + U (F dS)^T
//   dq = e^{G-m} Z,  dk = e^{G-m} X + e^{m-G} Y
//   dG = q~ Z + k~ X - k^ Y  (elementwise), plus on the last row
//   dG_15 += rowsum(dS * S_end) = rowsum((F dS) * (E S0)) + colsum(k^ * U (F dS)^T)
//   dg_t = sum_{t' >= t} dG_t'
// Every product is a 16 x 16 matrix-core tile (bf16 operands and fp32
// accumulation for bf16 inputs, fp32 throughout for fp32 inputs).
//
// Two sweeps per call, one workgroup per (sequence, head) each:
//  1. a forward sweep stores every sub-chunk's start state (a checkpoint, in
//     the input dtype) in the caller's workspace: for bf16 the prefill's
//     warp-specialised kernel in its checkpoint form, which walks 32-token
//     chunks and stores the state at each chunk's start and after its 16th
//     token (launch_backward_checkpoints); for fp32 bwd_states_kernel;
//  2. bwd_grad_kernel walks them backward, carrying dS in registers, and
//     writes dq, dk, dv, dg, dbeta and the initial state's gradient.
// The workgroup has d_v / 16 waves; for state-shaped quantities wave w owns
// the 16 value columns [16w, 16w + 16), for the key-channel outputs the
// 16-channel tiles w, w + d_v/16, ...
//
// Time split (few (sequence, head) pairs, long sequences): each sequence is
// cut into segments of seg tokens and every sweep runs one workgroup per
// (segment, head).  The forward map of a segment is affine in its start
// state, S_end = M S_start + N, and the reverse map of its state gradient is
// dS_start = M^T dS_end + D.  D, the state gradient at the segment's start for
// dS_end = 0, is the gradient of the segment's outputs o_t = S_t^T q_t with
// S_t = M_t S_start + N_t (M_t: the transition from the segment's start
// through token t):
//   D = sum over the segment's tokens of q^_t dO_t^T,  q^_t = M_t^T q_t.
// bf16 with d_k = d_v:
//  a. the forward pass's transition pass in its q^ form
//     (launch_prefill_maps_q): M_j and N_j of every non-last segment, M of
//     every split sequence's last segment, q^ of every segment j >= 1, and the
//     fold S_start(j + 1) = M_j S_start(j) + N_j;
//  b. bwd_dpass_kernel: D_j of every segment j >= 1 from q^ and dO;
//  c. bwd_fold_rev_q_kernel: from dS_end of the last segment (dL/d(final
//     state)), dS_end(j - 1) = M_j^T dS_end(j) + D_j in reverse;
//  d. sweeps 1 and 2 per segment, from S_start(j) and dS_end(j).
// Otherwise D_j comes from a reverse sweep of the dS recurrence alone
// (bwd_grad_kernel<DONLY>, every segment but the first, the last one started
// from dL/d(final state), which makes it dS_end of the one before), after the
// forward pass's maps and fold (launch_prefill_maps), and bwd_fold_rev_kernel
// composes the maps of the non-last segments.
#include <type_traits>

#include "gdn_backward.h"
#include "gdn_fold.h"
#include "gdn_segunit.h"
#include "gdn_tile16.h"

namespace gdn {
namespace {

using namespace t16;

// Fourth word of a raw buffer resource on gfx9-family parts (32-bit data
// format, no swizzle); with stride 0, stores at or past num_records bytes are
// dropped.
constexpr uint32_t kBufWord3 = 0x00020000u;
typedef unsigned int u32x2b __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4b __attribute__((ext_vector_type(4)));

template <typename TI>
struct BArgs {
    const TI* q;
    const TI* k;
    const TI* v;
    const float* g;
    const float* beta;
    const int32_t* cu;
    const float* S0;   // [num_seqs, H, DK, DV] or null (zero)
    const TI* dO;      // [T, H, DV]
    const float* dSf;  // [num_seqs, H, DK, DV] or null (zero)
    TI* dq;
    TI* dk;
    TI* dv;
    float* dg;
    float* dbeta;
    float* dS0;        // [num_seqs, H, DK, DV] or null (not wanted)
    TI* ck;            // checkpoints: slot (cu[n] / 16 + n + c, h) is the start state of sub-chunk c of sequence n
                       // (fp32: row-major; bf16: in column blocks of 16, see dma_ck_blocks)
    int H;
    // Time split (seg > 0, a multiple of 64): sequence n is cut into segments of
    // seg tokens.  From the forward pass's split, for segment j < last of
    // sequence n, slot nl[n] + j of
    //   fM  its transition M_j (d_k x d_k fp32; S_end = M_j S_start + N_j)
    //   fN  the start state of segment j + 1 (d_k x d_v fp32)
    // and segment j's slot cu[n] / seg + n + j of
    //   wsD  D_j, the state gradient at its start for a zero end gradient (the
    //        last segment's from dL/d(final state)), replaced by the previous
    //        segment's end gradient in the reverse fold (d_k x d_v fp32)
    int num_seqs;
    int64_t seg;
    const int32_t* nl;
    const float* fM;
    const float* fN;
    float* wsD;
    // without the split: workgroup b takes head b % H of sequence ord[b / H]
    // (longest first), or of sequence b / H when ord is null.  With the split
    // and pfx: workgroup b takes head b % H of segment b / H - pfx[i] of
    // sequence ord[i], pfx[i] <= b / H < pfx[i + 1] (the long sequences'
    // segments first); without pfx, segment slot b / H.
    const int32_t* ord;
    const int32_t* pfx;
};

// What one workgroup of a sweep works on (gdn_segunit.h).
typedef SegUnit BUnit;
template <typename TI>
__device__ __forceinline__ BUnit bwd_unit(const BArgs<TI>& a, int b) {
    return seg_unit(a, b);
}

// LDS layout.  "Natural" matrices are row-major over the contraction index
// with one 16-byte pad per row; "transposed" ones hold 16 tokens per key
// channel.  FULL: the gradient kernel's buffers; otherwise the forward one's.
// With bf16 inputs (STAGE) the next sub-chunk's raw inputs, and in the
// gradient kernel its checkpoint, are copied into a staging area by DMA
// while the current one is processed.  LITE (FULL only): without what only
// the outputs need (U, dRm, F dS, the staged v and checkpoint), so that two
// workgroups share a compute unit.
template <typename TI, int DK, int DV, bool FULL, int NWX = DV / 16, bool LITE = false>
struct BCfg {
    typedef Mma<TI> M;
    static constexpr bool STAGE = sizeof(TI) == 2;
    static constexpr int NW = NWX, NT = 64 * NW;
    static constexpr int ES = (int)sizeof(TI);
    static constexpr int KSTEP = M::KSTEP, KW = M::KW;
    static constexpr int KM = DK / KSTEP, KV = DV / KSTEP;  // MFMA steps over d_k, d_v
    static constexpr int RT = DK / 16;                      // 16-row tiles of d_k
    static constexpr int TPW = (RT + NW - 1) / NW;          // key-channel tiles per wave
    static constexpr int UNR = KW == 8 ? 8 : 4;             // unroll of the contraction loops
    static constexpr int UNR4 = 4;                          // ... of the key-channel outputs' pass over d_v
    static constexpr int SK = DK + 16 / ES, SV = DV + 16 / ES;
    static constexpr int B_NK = CB * SK * ES, B_TK = DK * CB * ES, B_NV = CB * SV * ES, B_FS = DK * SV * ES;
    static constexpr int OFF_KN = 0;                                   // k~ natural [16][SK]
    static constexpr int OFF_HN = OFF_KN + B_NK;                       // k^ natural
    static constexpr int OFF_HT = OFF_HN + B_NK;                       // k^ transposed [DK][16]
    static constexpr int OFF_QN = OFF_HT + B_TK;                       // q~ natural      (FULL)
    static constexpr int OFF_KT = OFF_QN + (FULL ? B_NK : 0);          // k~ transposed   (FULL)
    static constexpr int OFF_QT = OFF_KT + (FULL ? B_TK : 0);          // q~ transposed   (FULL)
    static constexpr int OFF_DO = OFF_QT + (FULL ? B_TK : 0);          // dO natural [16][SV]   (FULL)
    static constexpr bool GX = FULL && !LITE;                          // the outputs' buffers
    static constexpr int OFF_U = OFF_DO + (FULL ? B_NV : 0);           // U natural       (GX)
    static constexpr int OFF_DR = OFF_U + (GX ? B_NV : 0);             // dRm natural     (GX)
    static constexpr int OFF_FS = OFF_DR + (GX ? B_NV : 0);            // F dS [DK][SV]   (GX)
    static constexpr int OFF_G = OFF_FS + (GX ? B_FS : 0);             // G (log2) [16][DK] fp32
    static constexpr int OFF_ML = OFF_G + CB * DK * 4;                 // m (log2) [DK]
    static constexpr int OFF_EM = OFF_ML + DK * 4;                     // e^m [DK]
    static constexpr int OFF_FF = OFF_EM + DK * 4;                     // e^{G_15 - m} [DK]
    static constexpr int OFF_GAM = OFF_FF + DK * 4;                    // e^{G_15} [DK]
    static constexpr int OFF_DG15 = OFF_GAM + DK * 4;                  // dG_15 part [DK]  (FULL)
    static constexpr int OFF_BETA = OFF_DG15 + DK * 4;                 // beta [16]
    static constexpr int OFF_DB = OFF_BETA + CB * 4;                   // R . dRm per wave [NW][16]  (FULL)
    static constexpr int OFF_N = OFF_DB + NW * CB * 4;                 // -diag(b) KK [16][16]
    static constexpr int OFF_MI = OFF_N + 256 * 4;                     // M [16][16]
    static constexpr int OFF_MT = OFF_MI + 256 * 4;                    // M^T [16][16]
    static constexpr int OFF_P = OFF_MT + 256 * 4;                     // P, accumulator layout by lane (FULL)
    static constexpr bool KE = GX && STAGE;
    static constexpr int OFF_KE = OFF_P + (FULL ? 256 * 4 : 0);        // k e^G = k~ E natural   (KE)
    // dq, dk of a sub-chunk [16][DK] in the input dtype, rows padded by 16 bytes (KE): the
    // key-channel tiles of every wave, stored to HBM as whole rows
    static constexpr int SO = DK * ES + 16;
    static constexpr int OFF_OQ = OFF_KE + (KE ? B_NK : 0);
    static constexpr int OFF_OK = OFF_OQ + (KE ? CB * SO : 0);
    // staging (rows packed back to back, as the DMA writes them)
    static constexpr int OFF_STG = OFF_OK + (KE ? CB * SO : 0);
    static constexpr int ST_G = OFF_STG;                               // g [16][DK] fp32
    static constexpr int ST_K = ST_G + CB * DK * 4;                    // k [16][DK]
    static constexpr int ST_Q = ST_K + CB * DK * ES;                   // q [16][DK]   (FULL)
    static constexpr int ST_O = ST_Q + (FULL ? CB * DK * ES : 0);      // dO [16][DV]  (FULL)
    static constexpr int ST_V = ST_O + (FULL ? CB * DV * ES : 0);      // v [16][DV]   (not FULL && LITE)
    static constexpr int ST_B = ST_V + (FULL && LITE ? 0 : CB * DV * ES);  // beta [64] (lanes past 16 repeat the last row)
    static constexpr int ST_C = ST_B + 256;                            // checkpoint [DK][DV]  (GX)
    static constexpr int STG_END = STAGE ? ST_C + (GX ? DK * DV * ES : 0) : OFF_STG;
    // forward kernel: the state in the input dtype, rows padded, for coalesced checkpoint stores
    static constexpr int OFF_CK = STG_END;
    static constexpr int LDS = OFF_CK + (FULL ? 0 : DK * SV * ES);
    static_assert(B_NK % 16 == 0 && B_TK % 16 == 0 && B_NV % 16 == 0 && B_FS % 16 == 0, "alignment");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Element offset of (key channel c, token t) in a transposed [DK][16] operand.
// The 4-token group of t is XORed with bits 3-4 of c: the stores of one token
// pair by a wave (64 channel pairs) then spread over 16 LDS banks instead of 4,
// and a read of 4 tokens of one channel is still one aligned group (a wave's
// read of 16 channels covers every bank twice, as without the XOR).
__device__ __forceinline__ int tr_idx(int c, int t) { return c * CB + (t ^ (((c >> 3) & 3) << 2)); }

// Stores x[i] = X[row0 + 4g + i][col0 + r] (i = 0..3) of this lane into a
// row-major bf16 LDS matrix with an even row stride ld, as whole 4-byte words:
// a lane and its neighbour r ^ 1 swap one pair of rows (DPP quad_perm
// [1, 0, 3, 2]), then the even lane stores rows 4g, 4g+1 and the odd lane rows
// 4g+2, 4g+3 of columns (r & ~1, r | 1).  (Two lanes storing the two halves of
// one word conflict in the LDS banks.)
__device__ __forceinline__ void pair_store(bf16* base, int ld, int row0, int col0, floatx4 x, int r, int g) {
    const uint32_t p01 = pk_bf16(x[0], x[1]), p23 = pk_bf16(x[2], x[3]);
    const bool odd = (r & 1) != 0;
    const uint32_t send = odd ? p01 : p23, own = odd ? p23 : p01;
    const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xf, 0xf, false);
    const uint32_t lo = odd ? recv : own, hi = odd ? own : recv;
    uint32_t* dst = reinterpret_cast<uint32_t*>(base + (row0 + 4 * g + (odd ? 2 : 0)) * ld + col0 + (r & ~1));
    dst[0] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    dst[ld / 2] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Copy of a bf16 checkpoint into the staging area as DK rows of DV elements,
// each row's 16-byte pieces permuted as dma_rows<..., SWZ = true> permutes them
// (piece p of row i to slot p ^ (i mod (DV / 8))).  The checkpoint pass stores
// a slot in column blocks of 16 (element (i, c) at ((c / 16) DK + i) 16 + c % 16),
// so piece p of row i is the (p mod 2)-th half of row i of block p / 2; the
// rows that one copy instruction takes are consecutive, so it reads whole
// 128-byte lines of each block.
template <int DK, int DV, int NW>
__device__ __forceinline__ void dma_ck_blocks(const bf16* ck, char* dst, int w, int lane) {
    constexpr int LPR = DV * 2 / 16, RPI = 64 / LPR, NI = DK * DV * 2 / 1024;
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += NW) {
        const int i = i0 + w;
        if (NI % NW == 0 || i < NI) {
            const int row = i * RPI + lane / LPR;
            const int piece = (lane % LPR) ^ (row % LPR);
            __builtin_amdgcn_global_load_lds(
                as_global(reinterpret_cast<const char*>(ck) + ((piece >> 1) * DK + row) * 32 + (piece & 1) * 16),
                as_lds(dst + i * 1024), 16, 0, 0);
        }
    }
}

// Copy of one sub-chunk's raw inputs (t0: first token, L tokens) into the staging area.
template <typename TI, int DK, int DV, bool FULL, int NWX = DV / 16, bool LITE = false>
__device__ __forceinline__ void dma_inputs(const BArgs<TI>& a, char* smem, int h, int64_t t0, int L, int w,
                                           int lane) {
    typedef BCfg<TI, DK, DV, FULL, NWX, LITE> P;
    const int H = a.H;
    const size_t row0 = (size_t)t0 * H + h;
    dma_rows<DK * 4, CB, P::NW>(a.g + row0 * DK, (size_t)H * DK * 4, L, smem + P::ST_G, w, lane);
    dma_rows<DK * P::ES, CB, P::NW>(a.k + row0 * DK, (size_t)H * DK * P::ES, L, smem + P::ST_K, w, lane);
    if constexpr (FULL) {
        dma_rows<DK * P::ES, CB, P::NW>(a.q + row0 * DK, (size_t)H * DK * P::ES, L, smem + P::ST_Q, w, lane);
        dma_rows<DV * P::ES, CB, P::NW>(a.dO + row0 * DV, (size_t)H * DV * P::ES, L, smem + P::ST_O, w, lane);
    }
    if constexpr (!(FULL && LITE))
        dma_rows<DV * P::ES, CB, P::NW>(a.v + row0 * DV, (size_t)H * DV * P::ES, L, smem + P::ST_V, w, lane);
    if (w == P::NW - 1)
        __builtin_amdgcn_global_load_lds(as_global(a.beta + row0 + (size_t)min(lane, L - 1) * H),
                                         as_lds(smem + P::ST_B), 4, 0, 0);
}

// Steps 1 and 2 of a sub-chunk (both kernels): cumulative log-decay, the
// per-channel vectors, beta, the operands; dO into its padded layout (FULL);
// this lane's 4 values of v (rows 4g + i, column col0 + r; zero for a FULL
// LITE layout, which has no v).  Ends with an LDS barrier after the operands.
template <typename TI, int DK, int DV, bool FULL, int NWX = DV / 16, bool LITE = false>
__device__ __forceinline__ floatx4 prep(const BArgs<TI>& a, char* smem, int h, int64_t t0, int L, int tid, int col0) {
    typedef BCfg<TI, DK, DV, FULL, NWX, LITE> P;
    typedef typename Two<TI>::type T2;
    const int H = a.H;
    const int lane = tid & 63, r = lane & 15, g = lane >> 4;
    float* sG = reinterpret_cast<float*>(smem + P::OFF_G);
    float* sML = reinterpret_cast<float*>(smem + P::OFF_ML);
    float* sEM = reinterpret_cast<float*>(smem + P::OFF_EM);
    float* sFF = reinterpret_cast<float*>(smem + P::OFF_FF);
    float* sGAM = reinterpret_cast<float*>(smem + P::OFF_GAM);
    float* sBETA = reinterpret_cast<float*>(smem + P::OFF_BETA);
    TI* sKN = reinterpret_cast<TI*>(smem + P::OFF_KN);
    TI* sHN = reinterpret_cast<TI*>(smem + P::OFF_HN);
    TI* sHT = reinterpret_cast<TI*>(smem + P::OFF_HT);
    TI* sQN = reinterpret_cast<TI*>(smem + P::OFF_QN);
    TI* sKT = reinterpret_cast<TI*>(smem + P::OFF_KT);
    TI* sQT = reinterpret_cast<TI*>(smem + P::OFF_QT);
    TI* sDO = reinterpret_cast<TI*>(smem + P::OFF_DO);
    TI* sKE = reinterpret_cast<TI*>(smem + P::OFF_KE);
    const float* stg_g = reinterpret_cast<const float*>(smem + P::ST_G);
    const TI* stg_k = reinterpret_cast<const TI*>(smem + P::ST_K);
    const TI* stg_q = reinterpret_cast<const TI*>(smem + P::ST_Q);
    const TI* stg_o = reinterpret_cast<const TI*>(smem + P::ST_O);
    const TI* stg_v = reinterpret_cast<const TI*>(smem + P::ST_V);
    const float* stg_b = reinterpret_cast<const float*>(smem + P::ST_B);
    const size_t row0 = (size_t)t0 * H + h;  // (token, head) row of the sub-chunk's first token
    auto clampt = [&](int t) { return t < L ? t : L - 1; };

    // 1. cumulative log-decay of each key channel (rows past L count as g = 0)
    if constexpr (P::STAGE && P::NT >= 4 * DK) {
        // four lanes per channel, one per group of four tokens: wave w takes
        // channels 16w + r (r = lane mod 16), its lane group q tokens 4q .. 4q+3.
        // Each lane writes the sums over its group's prefix, then reads the four
        // group totals (written by lanes of the same wave: LDS operations of a
        // wave complete in order) and adds the totals before its group.
        if (tid < 4 * DK) {
            const int ch = 16 * (tid >> 6) + (tid & 15), qd = (tid >> 4) & 3;
            float Gq[4], acc = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * qd + i;
                acc = __builtin_fmaf(t < L ? stg_g[t * DK + ch] : 0.f, LOG2E_B, acc);
                Gq[i] = acc;
            }
            sG[(4 * qd + 3) * DK + ch] = acc;
            asm volatile("" ::: "memory");
            float tot[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) tot[q] = sG[(4 * q + 3) * DK + ch];
            asm volatile("" ::: "memory");
            const float off = (qd > 0 ? tot[0] : 0.f) + (qd > 1 ? tot[1] : 0.f) + (qd > 2 ? tot[2] : 0.f);
#pragma unroll
            for (int i = 0; i < 4; ++i) sG[(4 * qd + i) * DK + ch] = Gq[i] + off;
            if (qd == 0) {
                const float m = tot[0] + tot[1], G = m + tot[2] + tot[3];
                sML[ch] = m;
                sEM[ch] = __builtin_amdgcn_exp2f(m);
                sFF[ch] = __builtin_amdgcn_exp2f(G - m);
                sGAM[ch] = __builtin_amdgcn_exp2f(G);
            }
        }
        if (tid < CB) sBETA[tid] = tid < L ? stg_b[tid] : 0.f;
    } else {
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
        sEM[tid] = __builtin_amdgcn_exp2f(m);
        sFF[tid] = __builtin_amdgcn_exp2f(G - m);
        sGAM[tid] = __builtin_amdgcn_exp2f(G);
    }
    if (tid >= DK && tid < DK + CB) {
        const int t = tid - DK;
        float b;
        if constexpr (P::STAGE) b = stg_b[t];
        else b = a.beta[row0 + (size_t)clampt(t) * H];
        sBETA[t] = t < L ? b : 0.f;
    }
    }
    if constexpr (FULL) {
        // dO rows into the padded layout (16-byte pieces; rows past L are zero)
        constexpr int PER = 16 / P::ES, NPR = DV / PER;
#pragma unroll
        for (int i0 = 0; i0 < CB * NPR; i0 += P::NT) {
            const int i = i0 + tid;
            if ((CB * NPR) % P::NT == 0 || i < CB * NPR) {
                const int t = i / NPR, c = (i % NPR) * PER;
                floatx4 x;
                if constexpr (P::STAGE) x = *reinterpret_cast<const floatx4*>(stg_o + t * DV + c);
                else x = *reinterpret_cast<const floatx4*>(a.dO + (row0 + (size_t)clampt(t) * H) * DV + c);
                *reinterpret_cast<floatx4*>(sDO + t * P::SV + c) = t < L ? x : zero4();
            }
        }
    }
    floatx4 vv = zero4();
#pragma unroll
    for (int i = 0; i < 4 && !(FULL && LITE); ++i) {
        const int t = 4 * g + i;
        float x;
        if constexpr (P::STAGE) x = to_f32(stg_v[t * DV + col0 + r]);
        else x = to_f32(a.v[(row0 + (size_t)clampt(t) * H) * DV + col0 + r]);
        vv[i] = t < L ? x : 0.f;
    }
    lds_barrier();

    // 2. operands: (token pair tp, channel pair cp) per item
#pragma unroll
    for (int i0 = 0; i0 < 4 * DK; i0 += P::NT) {
        const int i = i0 + tid;
        if ((4 * DK) % P::NT != 0 && i >= 4 * DK) break;
        const int cp = i % (DK / 2), tp = i / (DK / 2), c0 = 2 * cp;
        const floatx2 ml = *reinterpret_cast<const floatx2*>(sML + c0);
        floatx2 em2 = floatx2{0.f, 0.f};
        if constexpr (P::KE) em2 = *reinterpret_cast<const floatx2*>(sEM + c0);
        floatx2 kt[2], kh[2], qt[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = 2 * tp + u;
            floatx2 kk2, qq2 = floatx2{0.f, 0.f};
            if constexpr (P::STAGE) {
                kk2 = Two<TI>::f(*reinterpret_cast<const T2*>(stg_k + t * DK + c0));
                if constexpr (FULL) qq2 = Two<TI>::f(*reinterpret_cast<const T2*>(stg_q + t * DK + c0));
            } else {
                const size_t off = (row0 + (size_t)clampt(t) * H) * DK + c0;
                kk2 = Two<TI>::f(*reinterpret_cast<const T2*>(a.k + off));
                if constexpr (FULL) qq2 = Two<TI>::f(*reinterpret_cast<const T2*>(a.q + off));
            }
            if (t >= L) kk2 = qq2 = floatx2{0.f, 0.f};
            const floatx2 G = *reinterpret_cast<const floatx2*>(sG + t * DK + c0);
            const floatx2 e = exp2v(G - ml), ei = exp2v(ml - G);
            kt[u] = kk2 * e;
            kh[u] = kk2 * ei;
            *reinterpret_cast<T2*>(sKN + t * P::SK + c0) = Two<TI>::t(kt[u]);
            *reinterpret_cast<T2*>(sHN + t * P::SK + c0) = Two<TI>::t(kh[u]);
            if constexpr (P::KE) *reinterpret_cast<T2*>(sKE + t * P::SK + c0) = Two<TI>::t(kt[u] * em2);
            if constexpr (FULL) {
                qt[u] = qq2 * e;
                *reinterpret_cast<T2*>(sQN + t * P::SK + c0) = Two<TI>::t(qt[u]);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = c0 + j;
            *reinterpret_cast<T2*>(sHT + tr_idx(c, 2 * tp)) = Two<TI>::t(floatx2{kh[0][j], kh[1][j]});
            if constexpr (FULL) {
                *reinterpret_cast<T2*>(sKT + tr_idx(c, 2 * tp)) = Two<TI>::t(floatx2{kt[0][j], kt[1][j]});
                *reinterpret_cast<T2*>(sQT + tr_idx(c, 2 * tp)) = Two<TI>::t(floatx2{qt[0][j], qt[1][j]});
            }
        }
    }
    // (gradient kernel, bf16: the checkpoint's copy, issued at the top of the
    // iteration, has landed in every wave before the value-column steps read it)
    if constexpr (P::GX && P::STAGE) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    return vv;
}

// Step 3 of a sub-chunk (one wave): KK = k~ k^T (returned in accumulator
// layout, lane r + 16g holding KK[4g + i][r], strictly lower part), the unit
// lower-triangular I + diag(b) KK and its inverse M by forward substitution
// (lane r + 16g carries M[r][4g .. 4g+3]; row j of M is final once rows < j
// are applied, and is read from lane j of the row with a DPP broadcast), then
// M and M^T into LDS.
template <typename TI, int DK, int DV, bool FULL, int NWX = DV / 16, bool LITE = false>
__device__ __forceinline__ floatx4 gram_inverse(char* smem, int lane) {
    typedef BCfg<TI, DK, DV, FULL, NWX, LITE> P;
    typedef Mma<TI> M;
    const int r = lane & 15, g = lane >> 4;
    const TI* sKN = reinterpret_cast<const TI*>(smem + P::OFF_KN);
    const TI* sHN = reinterpret_cast<const TI*>(smem + P::OFF_HN);
    const float* sBETA = reinterpret_cast<const float*>(smem + P::OFF_BETA);
    float* sN = reinterpret_cast<float*>(smem + P::OFF_N);
    float* sMI = reinterpret_cast<float*>(smem + P::OFF_MI);
    float* sMT = reinterpret_cast<float*>(smem + P::OFF_MT);
    floatx4 kk = zero4();
#pragma unroll(P::UNR)
    for (int mm = 0; mm < P::KM; ++mm) kk = M::mma(lds_nat(sKN + r * P::SK, mm, g), lds_nat(sHN + r * P::SK, mm, g), kk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * g + i;
        kk[i] = r < t ? kk[i] : 0.f;
        sN[t * 16 + r] = -sBETA[t] * kk[i];
    }
    // (lanes of this wave read what other lanes wrote: LDS operations of one wave complete in order)
    const floatx4 n0 = *reinterpret_cast<const floatx4*>(sN + r * 16);
    const floatx4 n1 = *reinterpret_cast<const floatx4*>(sN + r * 16 + 4);
    const floatx4 n2 = *reinterpret_cast<const floatx4*>(sN + r * 16 + 8);
    const floatx4 n3 = *reinterpret_cast<const floatx4*>(sN + r * 16 + 12);
    const float nr[16] = {n0[0], n0[1], n0[2], n0[3], n1[0], n1[1], n1[2], n1[3],
                          n2[0], n2[1], n2[2], n2[3], n3[0], n3[1], n3[2], n3[3]};
    const floatx4 x = unit_lower_inverse16(nr, r, g);
    *reinterpret_cast<floatx4*>(sMI + r * 16 + 4 * g) = x;
#pragma unroll
    for (int e = 0; e < 4; ++e) sMT[(4 * g + e) * 16 + r] = x[e];
    return kk;
}

// Forward sweep over the sub-chunks of one (sequence, head), or with a time
// split of one (segment, head), storing every sub-chunk's start state (its
// checkpoint), from the initial state or from the segment's start state left
// by the forward fold.  Used for fp32 inputs (bf16 checkpoints come from the
// prefill kernel's checkpoint pass).
template <typename TI, int DK, int DV>
__global__ __launch_bounds__(DV * 4, 1) void bwd_states_kernel(BArgs<TI> a) {
    typedef BCfg<TI, DK, DV, false> P;
    typedef Mma<TI> M;
    typedef K16<TI> K;
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    const int tid0 = threadIdx.x, g0 = (tid0 & 63) >> 4, r0 = tid0 & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int H = a.H;
    const BUnit u = bwd_unit(a, blockIdx.x);
    if (!u.valid) return;
    const int n = u.n, h = u.h;
    const int64_t sb = u.sb, se = u.se;
    const int col0 = 16 * w;
    const float* sEM = reinterpret_cast<const float*>(smem + P::OFF_EM);
    const float* sFF = reinterpret_cast<const float*>(smem + P::OFF_FF);
    const float* sGAM = reinterpret_cast<const float*>(smem + P::OFF_GAM);
    const float* sBETA = reinterpret_cast<const float*>(smem + P::OFF_BETA);
    const TI* sKN = reinterpret_cast<const TI*>(smem + P::OFF_KN);
    const TI* sHT = reinterpret_cast<const TI*>(smem + P::OFF_HT);
    const float* sMI = reinterpret_cast<const float*>(smem + P::OFF_MI);
    TI* sCK = reinterpret_cast<TI*>(smem + P::OFF_CK);

    // state, own columns: S[rt][i] = S[16 rt + 4g + i][col0 + r]
    floatx4 S[P::RT];
    const float* s0;
    if (u.j == 0) s0 = a.S0 ? a.S0 + ((size_t)n * H + h) * DK * DV : nullptr;
    else s0 = a.fN + ((size_t)(a.nl[n] + u.j - 1) * H + h) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[rt][i] = s0 ? s0[(16 * rt + 4 * g0 + i) * DV + col0 + r0] : 0.f;

    if constexpr (P::STAGE)
        if (se > sb) dma_inputs<TI, DK, DV, false>(a, smem, h, sb, (int)(se - sb < CB ? se - sb : CB), w, tid0 & 63);
    TI* ck = a.ck + (((size_t)(u.tb >> 4) + n + (size_t)((sb - u.tb) >> 4)) * H + h) * DK * DV;
    for (int64_t t0 = sb; t0 < se; t0 += CB, ck += (size_t)H * DK * DV) {
        const int L = (int)(se - t0 < CB ? se - t0 : CB);
        // lane-derived values are recomputed every iteration (opaque to the
        // compiler), so addresses built from them are not hoisted out of the
        // loop and held in registers for its whole length
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
        if constexpr (P::STAGE) __builtin_amdgcn_s_waitcnt(0);  // this wave's copy of the sub-chunk has landed
        lds_barrier();  // ... and every wave's; the previous sub-chunk is done with LDS
        // the checkpoint: own columns into LDS, then whole rows out in 16-byte pieces
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sCK[(16 * rt + 4 * g + i) * P::SV + col0 + r] = from_f32<TI>(S[rt][i]);
        const floatx4 vv = prep<TI, DK, DV, false>(a, smem, h, t0, L, tid, col0);
        if constexpr (P::STAGE) {
            const int64_t t1 = t0 + CB;
            if (t1 < se) dma_inputs<TI, DK, DV, false>(a, smem, h, t1, (int)(se - t1 < CB ? se - t1 : CB), w, lane);
        }
        {
            constexpr int PER = 16 / P::ES, NPR = DV / PER;
#pragma unroll
            for (int k = 0; k < DK * NPR / P::NT; ++k) {
                const int id = tid + P::NT * k, row = id / NPR, pc = id % NPR;
                *reinterpret_cast<floatx4*>(ck + row * DV + pc * PER) =
                    *reinterpret_cast<const floatx4*>(sCK + row * P::SV + pc * PER);
            }
        }
        if (w == 0) (void)gram_inverse<TI, DK, DV, false>(smem, lane);
        // R = V - k~ (E S), own columns
        floatx4 acc = zero4();
#pragma unroll(P::UNR)
        for (int mm = 0; mm < P::KM; ++mm) {
            floatx4 es[P::RT];
#pragma unroll
            for (int rt = 0; rt < P::RT; ++rt) es[rt] = S[rt] * *reinterpret_cast<const floatx4*>(sEM + 16 * rt + 4 * g);
            acc = M::mma(lds_perm(sKN + r * P::SK, mm, g), acc_perm<TI>(es, mm, P::RT), acc);
        }
        floatx4 br;
#pragma unroll
        for (int i = 0; i < 4; ++i) br[i] = sBETA[4 * g + i] * (vv[i] - acc[i]);
        lds_barrier();  // M is ready
        // U = M diag(b) R
        const floatx4 U = K::mma(K::cvt(*reinterpret_cast<const floatx4*>(sMI + r * 16 + 4 * g)), K::cvt(br), zero4());
        const typename K::frag bu = K::cvt(U);
        // S <- gamma S + F (k^T U)
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt) {
            const floatx4 d = K::mma(K::load(sHT + tr_idx(16 * rt + r, 4 * g)), bu, zero4());
            const floatx4 gm = *reinterpret_cast<const floatx4*>(sGAM + 16 * rt + 4 * g);
            const floatx4 ff = *reinterpret_cast<const floatx4*>(sFF + 16 * rt + 4 * g);
            S[rt] = gm * S[rt] + ff * d;
        }
    }
}

// Time split, reverse fold, per (sequence, head) and 16 state columns: from
// x = dS_end of the second-to-last segment (the last segment's adjoint-only
// sweep, started from dL/d(final state)), for j = P-2 down to 1,
// x <- M_j^T x + D_j, the gradient at the end of segment j - 1, written over D_j.
template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void bwd_fold_rev_kernel(const int32_t* cu, const int32_t* nl, int H,
                                                                      int64_t seg, const float* fM, float* wsD) {
    // grid (units, DV / 16): the column blocks of a unit are launched one grid
    // row apart, on one XCD when the number of units is a multiple of 8
    const int unit = blockIdx.x, n = unit / H, h = unit - n * H;
    const int64_t tb = cu[n], len = cu[n + 1] - tb;
    const int P = (int)((len + seg - 1) / seg);
    if (P < 3) return;
    const int64_t base = tb / seg + n;
    const float* x0 = wsD + ((size_t)(base + P - 1) * H + h) * DK * DV;
    // step i takes segment j = P - 2 - i
    fold_columns<DK, DV, true>(
        x0, P - 2, blockIdx.y, [&](int i) { return fM + ((size_t)(nl[n] + P - 2 - i) * H + h) * DK * DK; },
        [&](int i) { return wsD + ((size_t)(base + P - 2 - i) * H + h) * DK * DV; });
}

// Time split, bf16 with d_k = d_v: the offset of the reverse map of segment
// j >= 1 of a split sequence, D_j = sum over its tokens t of q^_t dO_t^T.  One
// workgroup per (non-last slot k, head): the segment after non-last segment k,
// i.e. j = k - nl[n] + 1 of sequence n.  Wave w accumulates rows
// [16w, 16w + 16) of D over all d_k columns (d_v = d_k).  Tiles of 64 tokens of
// q^ and dO are copied into LDS transposed, tokens contiguous per channel:
// each lane loads 8 channels of two adjacent tokens and writes them as 8
// two-token words (the 32 lanes of a token pair range write 32 consecutive
// words, so the stores of a wave spread over the banks); the next tile's loads
// are in flight while the current one is contracted with 16x16x32 bf16
// products.
template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void bwd_dpass_kernel(const int32_t* __restrict__ cu,
                                                                   const int32_t* __restrict__ nl, int num_seqs,
                                                                   int H, int64_t seg, const bf16* __restrict__ qh,
                                                                   const bf16* __restrict__ dO,
                                                                   float* __restrict__ wsD) {
    static_assert(DK == DV, "square state");
    constexpr int NW = DK / 16, NT = 64 * NW, TT = 64, SP = TT + 8, CT = DV / 16;
    constexpr int NCG = DK / 8;            // 8-channel groups of a row
    static_assert((TT / 2) * NCG == NT, "one (token pair, channel group) per thread");
    __shared__ __attribute__((aligned(16))) bf16 qT[DK * SP];
    __shared__ __attribute__((aligned(16))) bf16 oT[DV * SP];
    const int k = blockIdx.x / H, h = blockIdx.x - k * H;
    if (k >= nl[num_seqs]) return;
    int lo = 0, hi = num_seqs - 1;  // the sequence n with nl[n] <= k < nl[n + 1]
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (nl[mid + 1] > k) hi = mid;
        else lo = mid + 1;
    }
    const int n = lo, j = k - nl[n] + 1;
    const int64_t tb = cu[n] + (int64_t)j * seg, te = tb + seg < cu[n + 1] ? tb + seg : cu[n + 1];
    const int L = (int)(te - tb);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int tp = tid % (TT / 2), cg = tid / (TT / 2);  // this thread's token pair and channel group
    bf16x8 xq[2], xo[2];
    auto load = [&](int t0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = t0 + 2 * tp + u;
            const size_t off = ((size_t)(tb + t) * H + h) * DK + 8 * cg;
            xq[u] = t < L ? *reinterpret_cast<const bf16x8*>(qh + off) : bf16x8{};
            xo[u] = t < L ? *reinterpret_cast<const bf16x8*>(dO + off) : bf16x8{};
        }
    };
    floatx4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = zero4();
    if (L > 0) load(0);
    for (int t0 = 0; t0 < L; t0 += TT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            *reinterpret_cast<bf16x2*>(qT + (8 * cg + e) * SP + 2 * tp) = bf16x2{xq[0][e], xq[1][e]};
            *reinterpret_cast<bf16x2*>(oT + (8 * cg + e) * SP + 2 * tp) = bf16x2{xo[0][e], xo[1][e]};
        }
        __syncthreads();
        if (t0 + TT < L) load(t0 + TT);
#pragma unroll
        for (int kk = 0; kk < TT / 32; ++kk) {
            // A[c][t] = q^[t][c], B[t][v] = dO[t][v]: lane r + 16g supplies tokens 32kk + 8g .. +7
            const bf16x8 fa = *reinterpret_cast<const bf16x8*>(qT + (16 * w + r) * SP + 32 * kk + 8 * g);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                acc[ct] = Mma<bf16>::mma(fa, *reinterpret_cast<const bf16x8*>(oT + (16 * ct + r) * SP + 32 * kk + 8 * g),
                                         acc[ct]);
        }
        __syncthreads();
    }
    // lane r + 16g holds D[16w + 4g + i][16ct + r]
    float* D = wsD + (((size_t)(cu[n] / seg) + n + j) * H + h) * DK * DV;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) D[(size_t)(16 * w + 4 * g + i) * DV + 16 * ct + r] = acc[ct][i];
}

// Time split, bf16 with d_k = d_v: the reverse fold, per (split-list entry kk,
// head) and 16 state columns, from x = dL/d(final state) (or zero): for
// j = P-1 down to 1, x <- M_j^T x + D_j, the gradient at the end of segment
// j - 1, written over D_j (M_{P-1} from wsML slot kk, M_j for j < P-1 from
// slot nl[n] + j of the forward maps).
template <int DK, int DV, int DEPTH = 2>
__global__ __launch_bounds__(64 * (DK / 16), DEPTH == 1 ? 2 : 1) void bwd_fold_rev_q_kernel(
    const int32_t* cu, const int32_t* nl, const int32_t* spl, int H, int64_t seg, const float* fM,
    const float* wsML, const float* dSf, float* wsD) {
    const int unit = blockIdx.x, kk = unit / H, h = unit - kk * H;
    const int n = spl[kk];
    if (n < 0) return;
    const int P = nl[n + 1] - nl[n] + 1;
    const int64_t base = cu[n] / seg + n;
    const float* x0 = dSf ? dSf + ((size_t)n * H + h) * DK * DV : nullptr;
    // step i takes segment j = P - 1 - i
    auto d_at = [&](int i) { return wsD + ((size_t)(base + P - 1 - i) * H + h) * DK * DV; };
    fold_columns<DK, DV, true, DEPTH>(
        x0, P - 1, blockIdx.y,
        [&](int i) {
            return i == 0 ? wsML + ((size_t)kk * H + h) * DK * DK : fM + ((size_t)(nl[n] + P - 1 - i) * H + h) * DK * DK;
        },
        d_at);
}

// Reverse sweep over the sub-chunks of one (sequence, head), or with a time
// split of one (segment, head), last to first, from the gradient of the state
// at its end: that of the final state, or for a non-last segment the one the
// reverse fold left.  A sub-chunk's outputs are stored in the next iteration,
// after its waits for the copies in flight (the inputs, then the checkpoint), so
// those waits do not include them.
// DONLY (time split, segments after the first): only the state-gradient
// recursion, from a zero end gradient (the last segment: from dL/d(final
// state)); its result is written to the segment's slot for the reverse fold.
// It needs neither the checkpoints nor v.
// (DONLY: two workgroups per compute unit, i.e. d_v / 32 waves per SIMD.)
template <typename TI, int DK, int DV, bool DONLY>
__global__ __launch_bounds__(DV * 4, DONLY ? DV / 32 : 1) void bwd_grad_kernel(BArgs<TI> a) {
    typedef BCfg<TI, DK, DV, true, DV / 16, DONLY> P;
    typedef Mma<TI> M;
    typedef typename M::frag frag;
    typedef K16<TI> K;
    typedef Four<TI> F4;
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    const int tid0 = threadIdx.x, g0 = (tid0 & 63) >> 4, r0 = tid0 & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int H = a.H;
    const BUnit u = bwd_unit(a, blockIdx.x);
    if (!u.valid || (DONLY && u.j == 0)) return;
    const int n = u.n, h = u.h;
    const int64_t tb = u.tb, sb = u.sb, se = u.se;
    const int col0 = 16 * w;
    const float* sG = reinterpret_cast<const float*>(smem + P::OFF_G);
    const float* sML = reinterpret_cast<const float*>(smem + P::OFF_ML);
    const float* sEM = reinterpret_cast<const float*>(smem + P::OFF_EM);
    const float* sFF = reinterpret_cast<const float*>(smem + P::OFF_FF);
    float* sDG15 = reinterpret_cast<float*>(smem + P::OFF_DG15);
    const float* sBETA = reinterpret_cast<const float*>(smem + P::OFF_BETA);
    float* sDB = reinterpret_cast<float*>(smem + P::OFF_DB);
    const TI* sKN = reinterpret_cast<const TI*>(smem + P::OFF_KN);
    const TI* sHN = reinterpret_cast<const TI*>(smem + P::OFF_HN);
    const TI* sQN = reinterpret_cast<const TI*>(smem + P::OFF_QN);
    const TI* sKT = reinterpret_cast<const TI*>(smem + P::OFF_KT);
    const TI* sHT = reinterpret_cast<const TI*>(smem + P::OFF_HT);
    const TI* sQT = reinterpret_cast<const TI*>(smem + P::OFF_QT);
    const TI* sDO = reinterpret_cast<const TI*>(smem + P::OFF_DO);
    TI* sU = reinterpret_cast<TI*>(smem + P::OFF_U);
    TI* sDR = reinterpret_cast<TI*>(smem + P::OFF_DR);
    TI* sFS = reinterpret_cast<TI*>(smem + P::OFF_FS);
    const float* sMI = reinterpret_cast<const float*>(smem + P::OFF_MI);
    const float* sMT = reinterpret_cast<const float*>(smem + P::OFF_MT);
    float* sP = reinterpret_cast<float*>(smem + P::OFF_P);
    const TI* stg_c = reinterpret_cast<const TI*>(smem + P::ST_C);
    const TI* sKE = reinterpret_cast<const TI*>(smem + P::OFF_KE);

    // dS = dL/d(state at the end of the current sub-chunk), own columns.  Inside
    // an iteration it holds F dS from the operand preparation on, and the dS
    // update leaves dS of the sub-chunk before: gamma dS + E x = E (F dS + x).
    floatx4 dS[P::RT];
    const float* dsf;
    if (u.j == u.P - 1) dsf = a.dSf ? a.dSf + ((size_t)n * H + h) * DK * DV : nullptr;
    else dsf = DONLY ? nullptr : a.wsD + ((size_t)(u.slot + 1) * H + h) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[rt][i] = dsf ? dsf[(16 * rt + 4 * g0 + i) * DV + col0 + r0] : 0.f;

    // outputs of the previous iteration, stored at the start of the next one
    floatx4 o_dv = zero4(), o_db = zero4();
    floatx4 o_dq[P::TPW], o_dk[P::TPW], o_dg[P::TPW];
#pragma unroll
    for (int j = 0; j < P::TPW; ++j) o_dq[j] = o_dk[j] = o_dg[j] = zero4();
    size_t o_row0 = 0;
    int o_L = 0;  // 0: nothing pending
    // The stores go through buffer resources that end at the sub-chunk's last
    // (token, head) row: the hardware drops rows past it (a shorter last
    // sub-chunk), so no store needs a branch.
    auto flush = [&](int r, int g) {
        if (o_L == 0) return;
        const uint32_t rows = (uint32_t)o_L * (uint32_t)H;  // rows o_row0 .. o_row0 + rows - 1 of [T, H]
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc(a.dv + o_row0 * DV, 0, rows * DV * P::ES, kBufWord3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = ((uint32_t)(4 * g + i) * H * DV + col0 + r) * P::ES;
            if constexpr (P::ES == 2)
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f32<TI>(o_dv[i])), rv,
                                                      off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((float)o_dv[i]), rv, off, 0, 0);
        }
        if (w == 0 && r == 0) {
            const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(a.dbeta + o_row0, 0, rows * 4, kBufWord3);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((float)o_db[i]), rb,
                                                      (uint32_t)(4 * g + i) * H * 4, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t rq =
            __builtin_amdgcn_make_buffer_rsrc(a.dq + o_row0 * DK, 0, rows * DK * P::ES, kBufWord3);
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc(a.dk + o_row0 * DK, 0, rows * DK * P::ES, kBufWord3);
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(a.dg + o_row0 * DK, 0, rows * DK * 4, kBufWord3);
        if constexpr (P::KE) {
            // dq and dk from their staged rows: 16-byte pieces, 16 lanes per 256-byte
            // row, so each store covers whole cache lines (waves of the first half
            // take dq, the others dk, at d = 128)
            constexpr int PR = DK * P::ES / 16, NPC = CB * PR;
            static_assert(NPC % 64 == 0, "a wave's pieces lie in one matrix");
#pragma unroll
            for (int p0 = 0; p0 < 2 * NPC; p0 += P::NT) {
                const int pw = p0 + 64 * w;  // the wave's first piece (uniform)
                if ((2 * NPC) % P::NT == 0 || pw < 2 * NPC) {
                    const int mk = pw / NPC, q = pw % NPC + 16 * g + r, row = q / PR, cp = q % PR;
                    const u32x4b x =
                        *reinterpret_cast<const u32x4b*>(smem + (mk ? P::OFF_OK : P::OFF_OQ) + row * P::SO + cp * 16);
                    __builtin_amdgcn_raw_buffer_store_b128(x, mk ? rk : rq, (uint32_t)row * H * DK * P::ES + cp * 16,
                                                           0, 0);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < P::TPW; ++j) {
            const int it = w + P::NW * j;
            if (P::RT % P::NW != 0 && it >= P::RT) break;
            const uint32_t e = (uint32_t)r * H * DK + 16 * it + 4 * g;  // element offset of (token r, channel)
            if constexpr (P::KE) {
                // (dq and dk: stored as whole rows above)
            } else if constexpr (P::ES == 2) {
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2b, F4::t(o_dq[j])), rq, e * 2, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2b, F4::t(o_dk[j])), rk, e * 2, 0, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4b, o_dq[j]), rq, e * 4, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4b, o_dk[j]), rk, e * 4, 0, 0);
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4b, o_dg[j]), rg, e * 4, 0, 0);
        }
    };
    // sub-chunk c of the segment: checkpoint slot and length
    const size_t cbase = (size_t)(tb >> 4) + n + (size_t)((sb - tb) >> 4);
    auto slot = [&](int64_t c) { return a.ck + (((cbase + (size_t)c) * H + h) * DK * DV); };
    auto sub_len = [&](int64_t c) { return (int)(se - (sb + CB * c) < CB ? se - (sb + CB * c) : CB); };

    const int64_t nsub = (se - sb + CB - 1) / CB;
    if constexpr (P::STAGE) {
        if (nsub > 0) {
            dma_inputs<TI, DK, DV, true, DV / 16, DONLY>(a, smem, h, sb + CB * (nsub - 1), sub_len(nsub - 1), w,
                                                         tid0 & 63);
        }
    }
    for (int64_t c = nsub - 1; c >= 0; --c) {
        const int64_t t0 = sb + CB * c;
        const int L = sub_len(c);
        const size_t row0 = (size_t)t0 * H + h;
        const TI* ck = slot(c);
        // lane-derived values are recomputed every iteration (opaque to the
        // compiler), so addresses built from them are not hoisted out of the
        // loop and held in registers for its whole length; the copies and the
        // deferred output stores take the plain lane values instead, so their
        // per-lane offsets are formed once (32 more VGPRs, 80 fewer VALU
        // instructions per iteration)
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
        if constexpr (P::STAGE) __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
        lds_barrier();  // ... and every wave's; the previous sub-chunk is done with LDS
        // bf16: this sub-chunk's checkpoint into the staging area.  It stays there
        // through the key-channel outputs, which read its rows from LDS; its copy
        // is waited for at the end of prep.
        if constexpr (P::STAGE && !DONLY)
            dma_ck_blocks<DK, DV, P::NW>(ck, smem + P::ST_C, w, tid0 & 63);
        const floatx4 vv = prep<TI, DK, DV, true, DV / 16, DONLY>(a, smem, h, t0, L, tid, col0);
        // (the previous sub-chunk's outputs are stored in the value-column steps
        // and the next sub-chunk's inputs copied after the dS update, both after
        // prep's wait for the checkpoint: vector-memory counts complete in issue
        // order, so anything issued before that wait would have been waited for
        // with it; spread over the iteration, the stores and copies do not queue
        // behind one another)
        floatx4 kk = zero4();
        if (w == 0) kk = gram_inverse<TI, DK, DV, true, DV / 16, DONLY>(smem, lane);

        // ---- 3. value-column steps (own columns) -------------------------------
        // (wave 1) P = lower(q~ k^T): lane r + 16g holds P[t = 4g + i][s = r]; shared through LDS
        if (w == 1) {
            floatx4 Pa = zero4();
#pragma unroll(P::UNR)
            for (int mm = 0; mm < P::KM; ++mm)
                Pa = M::mma(lds_nat(sQN + r * P::SK, mm, g), lds_nat(sHN + r * P::SK, mm, g), Pa);
#pragma unroll
            for (int i = 0; i < 4; ++i) Pa[i] = r <= 4 * g + i ? Pa[i] : 0.f;
            *reinterpret_cast<floatx4*>(sP + 4 * lane) = Pa;
        }
        // R = V - k~ (E S0), S0 from the checkpoint: the B operand's element e of
        // step mm is S0[k][col0 + r] with k in the permuted order.  bf16: as the
        // staged copy holds it (k = 32 mm + 16 (e / 4) + 4g + e % 4), with E moved
        // to the other operand, k~ E = k e^G; fp32: E S0 from global memory
        // (k = 16 (mm / 4) + 4g + mm % 4).
        floatx4 acc = zero4();
        if constexpr (!DONLY) {
            // bf16: byte address of (row 4g + i, column col0 + r) in the staged
            // copy (swz_off), i = 0..3; rows 16 past it are 16 row strides
            // further (a row's swizzle depends on the row mod 16 only), an
            // offset the loads take as an immediate
            const char* cbi[4];
            if constexpr (P::KE) {
                constexpr int LPR = DV * P::ES / 16, PER = 16 / P::ES;
                const int c = col0 + r;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    cbi[i] = reinterpret_cast<const char*>(stg_c) + (4 * g + i) * (DV * P::ES) +
                             ((c / PER) ^ ((4 * g + i) % LPR)) * 16 + (c % PER) * P::ES;
            }
#pragma unroll(P::UNR)
            for (int mm = 0; mm < P::KM; ++mm) {
                frag fb;
                if constexpr (P::KE) {
                    static_assert(DV * P::ES / 16 == 16 || DV * P::ES / 16 == 8, "row swizzle period divides 16");
#pragma unroll
                    for (int e = 0; e < P::KW; ++e)
                        fb[e] = *reinterpret_cast<const TI*>(cbi[e & 3] + (32 * mm + 16 * (e >> 2)) * (DV * P::ES));
                    acc = M::mma(lds_perm(sKE + r * P::SK, mm, g), fb, acc);
                } else {
                    const int row = 16 * (mm >> 2) + 4 * g + (mm & 3);
                    fb = sEM[row] * to_f32(ck[row * DV + col0 + r]);
                    acc = M::mma(lds_perm(sKN + r * P::SK, mm, g), fb, acc);
                }
            }
        }
        floatx4 R, br;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            R[i] = vv[i] - acc[i];
            br[i] = sBETA[4 * g + i] * R[i];
        }
        // own columns of dO
        floatx4 dOc;
#pragma unroll
        for (int i = 0; i < 4; ++i) dOc[i] = to_f32(sDO[(4 * g + i) * P::SV + col0 + r]);
        // dS -> F dS
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt) dS[rt] = dS[rt] * *reinterpret_cast<const floatx4*>(sFF + 16 * rt + 4 * g);
        // dU = k^ (F dS) + P^T dO (the second term once P is shared)
        floatx4 dU = zero4();
#pragma unroll(P::UNR)
        for (int mm = 0; mm < P::KM; ++mm) dU = M::mma(lds_perm(sHN + r * P::SK, mm, g), acc_perm<TI>(dS, mm, P::RT), dU);
        lds_barrier();  // M is ready
        const floatx4 U = K::mma(K::cvt(*reinterpret_cast<const floatx4*>(sMI + r * 16 + 4 * g)), K::cvt(br), zero4());
        dU = K::mma(K::cvt(*reinterpret_cast<const floatx4*>(sP + 4 * lane)), K::cvt(dOc), dU);
        // dRm = M^T dU, dR = diag(b) dRm = dv
        const floatx4 dRm = K::mma(K::cvt(*reinterpret_cast<const floatx4*>(sMT + r * 16 + 4 * g)), K::cvt(dU), zero4());
        floatx4 dR, ndR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * g + i;
            dR[i] = sBETA[t] * dRm[i];
            ndR[i] = -dR[i];
            if constexpr (!DONLY) {
                const float p = sum16(R[i] * dRm[i]);
                if (r == 0) sDB[w * CB + t] = p;
            }
        }
        if constexpr (!DONLY) flush(r0, g0);  // the previous sub-chunk's outputs, before o_dv is replaced
        o_dv = dR;
        // exchange: F dS, U, dRm (natural layouts) for the key-channel products
        if constexpr (!DONLY && P::ES == 2) {
#pragma unroll
            for (int rt = 0; rt < P::RT; ++rt) pair_store(sFS, P::SV, 16 * rt, col0, dS[rt], r, g);
            pair_store(sU, P::SV, 0, col0, U, r, g);
            pair_store(sDR, P::SV, 0, col0, dRm, r, g);
        } else if constexpr (!DONLY) {
#pragma unroll
            for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sFS[(16 * rt + 4 * g + i) * P::SV + col0 + r] = from_f32<TI>(dS[rt][i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sU[(4 * g + i) * P::SV + col0 + r] = from_f32<TI>(U[i]);
                sDR[(4 * g + i) * P::SV + col0 + r] = from_f32<TI>(dRm[i]);
            }
        }
        // dS <- gamma dS + E (q~^T dO - k~^T dR) = E (F dS + q~^T dO - k~^T dR)
        {
            const typename K::frag bo = K::cvt(dOc), br2 = K::cvt(ndR);
#pragma unroll
            for (int rt = 0; rt < P::RT; ++rt) {
                floatx4 x = K::mma(K::load(sQT + tr_idx(16 * rt + r, 4 * g)), bo, dS[rt]);
                x = K::mma(K::load(sKT + tr_idx(16 * rt + r, 4 * g)), br2, x);
                dS[rt] = *reinterpret_cast<const floatx4*>(sEM + 16 * rt + 4 * g) * x;
            }
        }
        // the next sub-chunk's inputs (every staged row was read by prep)
        if constexpr (P::STAGE)
            if (c > 0) dma_inputs<TI, DK, DV, true, DV / 16, DONLY>(a, smem, h, t0 - CB, sub_len(c - 1), w, tid0 & 63);
        if constexpr (DONLY) continue;
        lds_barrier();

        // ---- 4. key-channel outputs ------------------------------------------
        // Contractions over d_v, one pass over the value rows: the token-pair
        // matrices (the same in every wave) and, for each of this wave's
        // key-channel tiles i0 = 16 it, the products with state rows i0 + r (the
        // checkpoint: its staged copy in LDS for bf16, global memory for fp32;
        // and F dS).
        floatx4 dPT = zero4(), dPa = zero4(), dAa = zero4(), dAT = zero4();
        floatx4 z1[P::TPW], x1[P::TPW], y1[P::TPW];
        // (F dS) S0^T over the tile's rows: its diagonal is rowsum((F dS) * S0)
        floatx4 d1[P::TPW];
#pragma unroll
        for (int j = 0; j < P::TPW; ++j) z1[j] = x1[j] = y1[j] = d1[j] = zero4();
#pragma unroll(P::UNR4)
        for (int mm = 0; mm < P::KV; ++mm) {
            const frag fo = lds_nat(sDO + r * P::SV, mm, g);
            const frag fu = lds_nat(sU + r * P::SV, mm, g);
            const frag fr = lds_nat(sDR + r * P::SV, mm, g);
            dPT = M::mma(fu, fo, dPT);  // dP[t = r][s = 4g + i]
            dPa = M::mma(fo, fu, dPa);  // dP[t = 4g + i][s = r]
            dAa = M::mma(fr, fu, dAa);  // -dA[t = 4g + i][s = r]
            dAT = M::mma(fu, fr, dAT);  // -dA[t = r][s = 4g + i]
#pragma unroll
            for (int j = 0; j < P::TPW; ++j) {
                const int it = w + P::NW * j;
                if (P::RT % P::NW != 0 && it >= P::RT) break;
                const int i0 = 16 * it;
                frag fs0;
                if constexpr (P::STAGE)  // the staged copy (16-byte pieces permuted per row)
                    fs0 = *reinterpret_cast<const frag*>(reinterpret_cast<const char*>(stg_c) +
                                                         swz_off<DV * P::ES, P::ES>(i0 + r, mm * P::KSTEP + g * P::KW));
                else
                    fs0 = *reinterpret_cast<const frag*>(ck + (size_t)(i0 + r) * DV + mm * P::KSTEP + g * P::KW);
                const frag ffs = lds_nat(sFS + (i0 + r) * P::SV, mm, g);
                z1[j] = M::mma(fs0, fo, z1[j]);
                x1[j] = M::mma(fs0, fr, x1[j]);
                y1[j] = M::mma(ffs, fu, y1[j]);
                d1[j] = M::mma(ffs, fs0, d1[j]);
            }
        }
        floatx4 dKKa, dKKT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ti = 4 * g + i;
            dPT[i] = ti <= r ? dPT[i] : 0.f;
            dPa[i] = r <= ti ? dPa[i] : 0.f;
            dAa[i] = r < ti ? -dAa[i] : 0.f;
            dAT[i] = ti < r ? -dAT[i] : 0.f;
            dKKa[i] = sBETA[ti] * dAa[i];
            dKKT[i] = sBETA[r] * dAT[i];
        }
        if (w == 0) {
            // dbeta_t = R_t . dRm_t + sum_s dA_ts KK_ts,  t = 4g + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * g + i;
                float p = sum16(dAa[i] * kk[i]);
#pragma unroll
                for (int ww = 0; ww < P::NW; ++ww) p += sDB[ww * CB + t];
                o_db[i] = p;
            }
        }
        const typename K::frag bPT = K::cvt(dPT), bKKT = K::cvt(dKKT), bKKa = K::cvt(dKKa), bPa = K::cvt(dPa);
#pragma unroll
        for (int j = 0; j < P::TPW; ++j) {
            const int it = w + P::NW * j;
            if (P::RT % P::NW != 0 && it >= P::RT) break;
            const int i0 = 16 * it;
            // diagonal element (r, r) sits in lane r of lane group r / 4, entry r % 4
            if (g == (r >> 2)) {
                const int e = r & 3;
                const float dd = e == 0 ? d1[j][0] : e == 1 ? d1[j][1] : e == 2 ? d1[j][2] : d1[j][3];
                sDG15[i0 + r] = dd * sEM[i0 + r];
            }
            // lane r + 16g: key channel i = i0 + 4g + e, token t = r
            const floatx4 em = *reinterpret_cast<const floatx4*>(sEM + i0 + 4 * g);
            const float bt = sBETA[r];
            floatx4 Z = em * z1[j], X = -(bt * em) * x1[j];
            Z = K::mma(K::load(sHT + tr_idx(i0 + r, 4 * g)), bPT, Z);
            X = K::mma(K::load(sHT + tr_idx(i0 + r, 4 * g)), bKKT, X);
            floatx4 Y = K::mma(K::load(sKT + tr_idx(i0 + r, 4 * g)), bKKa, y1[j]);
            Y = K::mma(K::load(sQT + tr_idx(i0 + r, 4 * g)), bPa, Y);
            const floatx4 khat = F4::f(*reinterpret_cast<const typename F4::type*>(sHN + r * P::SK + i0 + 4 * g));
            const floatx4 ktil = F4::f(*reinterpret_cast<const typename F4::type*>(sKN + r * P::SK + i0 + 4 * g));
            const floatx4 qtil = F4::f(*reinterpret_cast<const typename F4::type*>(sQN + r * P::SK + i0 + 4 * g));
            const floatx4 Gl = *reinterpret_cast<const floatx4*>(sG + r * DK + i0 + 4 * g);
            const floatx4 ml = *reinterpret_cast<const floatx4*>(sML + i0 + 4 * g);
            const floatx4 ef = exp2v(Gl - ml), eb = exp2v(ml - Gl);
            if constexpr (P::KE) {
                // lane r + 16g: token r, channels i0 + 4g .. i0 + 4g + 3
                char* rowq = smem + P::OFF_OQ + r * P::SO + (i0 + 4 * g) * P::ES;
                *reinterpret_cast<u32x2b*>(rowq) = __builtin_bit_cast(u32x2b, F4::t(ef * Z));
                *reinterpret_cast<u32x2b*>(rowq + (P::OFF_OK - P::OFF_OQ)) = __builtin_bit_cast(u32x2b, F4::t(ef * X + eb * Y));
            } else {
                o_dq[j] = ef * Z;
                o_dk[j] = ef * X + eb * Y;
            }
            floatx4 dG = qtil * Z + ktil * X - khat * Y;
            floatx4 d2;
#pragma unroll
            for (int e = 0; e < 4; ++e) d2[e] = sum16(khat[e] * y1[j][e]);
            const floatx4 d15 = *reinterpret_cast<const floatx4*>(sDG15 + i0 + 4 * g) + d2;
#pragma unroll
            for (int e = 0; e < 4; ++e) dG[e] = suffix16(dG[e]) + d15[e];
            o_dg[j] = dG;
        }
        o_row0 = row0;
        o_L = L;
    }
    if constexpr (DONLY) {
        // lane indices recomputed here, so that nothing lane-derived stays live across the loop
        int te = threadIdx.x;
        asm volatile("" : "+v"(te));
        const int ge = (te & 63) >> 4, re = te & 15;
        float* dst = a.wsD + ((size_t)u.slot * H + h) * DK * DV;
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(16 * rt + 4 * ge + i) * DV + col0 + re] = dS[rt][i];
        return;
    }
    if constexpr (P::KE) lds_barrier();  // every wave's staged dq, dk rows of the last sub-chunk
    flush(r0, g0);
    if (u.j == 0 && a.dS0) {
        float* dst = a.dS0 + ((size_t)n * H + h) * DK * DV;
#pragma unroll
        for (int rt = 0; rt < P::RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(16 * rt + 4 * g0 + i) * DV + col0 + r0] = dS[rt][i];
    }
}

// The checkpoint sweep over `blocks` units: bf16 on the prefill's kernel in
// 32-token chunks (launch_backward_checkpoints, the same slots), fp32 on
// bwd_states_kernel.
template <typename TI, int DK, int DV>
hipError_t run_states(const BArgs<TI>& a, int64_t blocks, hipStream_t s) {
    if constexpr (sizeof(TI) == 2) {
        CheckpointLaunch c;
        c.k = a.k;
        c.v = a.v;
        c.g = a.g;
        c.beta = a.beta;
        c.cu_seqlens = a.cu;
        c.initial_state = a.S0;
        c.num_seqs = a.num_seqs;
        c.H = a.H;
        c.dk = DK;
        c.dv = DV;
        c.seg = a.seg;
        c.nl = a.nl;
        c.seg_start = a.fN;
        c.ord = a.ord;
        c.pfx = a.pfx;
        c.ck = a.ck;
        c.blocks = blocks;
        return launch_backward_checkpoints(c, s);
    } else {
        hipLaunchKernelGGL((bwd_states_kernel<TI, DK, DV>), dim3((unsigned)blocks), dim3(DV * 4), 0, s, a);
        return hipGetLastError();
    }
}

template <typename TI, int DK, int DV>
hipError_t run_bwd(const BackwardLaunch& p, hipStream_t s) {
    BArgs<TI> a;
    a.q = static_cast<const TI*>(p.q);
    a.k = static_cast<const TI*>(p.k);
    a.v = static_cast<const TI*>(p.v);
    a.g = p.g;
    a.beta = p.beta;
    a.cu = p.cu_seqlens;
    a.S0 = p.initial_state;
    a.dO = static_cast<const TI*>(p.d_o);
    a.dSf = p.d_final_state;
    a.dq = static_cast<TI*>(p.dq);
    a.dk = static_cast<TI*>(p.dk);
    a.dv = static_cast<TI*>(p.dv);
    a.dg = p.dg;
    a.dbeta = p.dbeta;
    a.dS0 = p.d_initial_state;
    a.ck = static_cast<TI*>(p.workspace);
    a.H = p.H;
    a.num_seqs = p.num_seqs;
    a.seg = p.seg;
    a.nl = nullptr;
    a.fM = a.fN = nullptr;
    a.wsD = nullptr;
    a.ord = nullptr;
    a.pfx = nullptr;
    if (p.seg <= 0) {
        const unsigned blocks = (unsigned)((int64_t)p.num_seqs * p.H);
        const BackwardWorkspace wl = backward_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DV, p.bf16, 0);
        if (wl.ord) {
            // longest sequences first, the same order in both sweeps
            int32_t* ord = reinterpret_cast<int32_t*>(static_cast<char*>(p.workspace) + wl.ord_off);
            const hipError_t e = launch_seq_order(p.cu_seqlens, p.num_seqs, 0, ord, s);
            if (e != hipSuccess) return e;
            a.ord = ord;
        }
        hipError_t e = run_states<TI, DK, DV>(a, blocks, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_grad_kernel<TI, DK, DV, false>), dim3(blocks), dim3(DV * 4), 0, s, a);
        return hipGetLastError();
    }
    // time split: the forward's maps and fold, the adjoint-only sweeps, the
    // reverse fold, then both sweeps per segment from the folded boundary values
    const BackwardWorkspace ws = backward_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DV, p.bf16, p.seg);
    char* base = static_cast<char*>(p.workspace);
    const PrefillWorkspace pw = prefill_workspace_layout(p.T_total, p.num_seqs, p.H, DK, DV, p.seg, false);
    a.nl = reinterpret_cast<const int32_t*>(base + ws.pre_off + pw.nl_off);
    a.fM = reinterpret_cast<const float*>(base + ws.pre_off + pw.m_off);
    a.fN = reinterpret_cast<const float*>(base + ws.pre_off + pw.n_off);
    a.wsD = reinterpret_cast<float*>(base + ws.d_off);
    PrefillLaunch f;
    f.q = p.q;
    f.k = p.k;
    f.v = p.v;
    f.g = p.g;
    f.beta = p.beta;
    f.cu_seqlens = p.cu_seqlens;
    f.initial_state = p.initial_state;
    f.final_state = nullptr;
    f.o = nullptr;
    f.num_seqs = p.num_seqs;
    f.H = p.H;
    f.dk = DK;
    f.dv = DV;
    f.bf16 = p.bf16;
    f.T_total = p.T_total;
    f.seg = p.seg;
    f.workspace = base + ws.pre_off;
    f.legacy = false;
    hipError_t e;
    if constexpr (DK == DV && sizeof(TI) == 2) {
        // D from the transition pass's q^: no adjoint-only sweep
        bf16* qh = reinterpret_cast<bf16*>(base + ws.qh_off);
        const float* wsML = reinterpret_cast<const float*>(base + ws.ml_off);
        const int32_t* spl = reinterpret_cast<const int32_t*>(base + ws.pre_off + pw.spl_off);
        if ((e = launch_prefill_maps_q(f, qh, const_cast<float*>(wsML), s)) != hipSuccess) return e;
        if (ws.ord) {
            int32_t* ord = reinterpret_cast<int32_t*>(base + ws.ord_off);
            int32_t* pfx = reinterpret_cast<int32_t*>(base + ws.pfx_off);
            if ((e = launch_seq_order(p.cu_seqlens, p.num_seqs, 0, ord, s, p.seg, pfx)) != hipSuccess) return e;
            a.ord = ord;
            a.pfx = pfx;
        }
        if (pw.slots > 0) {
            hipLaunchKernelGGL((bwd_dpass_kernel<DK, DV>), dim3((unsigned)(pw.slots * p.H)), dim3(64 * (DK / 16)), 0,
                               s, a.cu, a.nl, p.num_seqs, p.H, p.seg, qh, a.dO, a.wsD);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (pw.splits > 0) {
            // more workgroups than CUs: the shallower prefetch, two workgroups per CU
            if (pw.splits * p.H * (DV / 16) > kComputeUnits)
                hipLaunchKernelGGL((bwd_fold_rev_q_kernel<DK, DV, 1>), dim3((unsigned)(pw.splits * p.H), DV / 16),
                                   dim3(64 * (DK / 16)), 0, s, a.cu, a.nl, spl, p.H, p.seg, a.fM, wsML, a.dSf, a.wsD);
            else
                hipLaunchKernelGGL((bwd_fold_rev_q_kernel<DK, DV, 2>), dim3((unsigned)(pw.splits * p.H), DV / 16),
                                   dim3(64 * (DK / 16)), 0, s, a.cu, a.nl, spl, p.H, p.seg, a.fM, wsML, a.dSf, a.wsD);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const unsigned blocks = (unsigned)(ws.slots * p.H);
        if ((e = run_states<TI, DK, DV>(a, blocks, s)) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_grad_kernel<TI, DK, DV, false>), dim3(blocks), dim3(DV * 4), 0, s, a);
        return hipGetLastError();
    }
    e = launch_prefill_maps(f, s);
    if (e != hipSuccess) return e;
    if (ws.ord) {
        // the sweeps over segments take the longest sequences' segments first
        int32_t* ord = reinterpret_cast<int32_t*>(base + ws.ord_off);
        int32_t* pfx = reinterpret_cast<int32_t*>(base + ws.pfx_off);
        if ((e = launch_seq_order(p.cu_seqlens, p.num_seqs, 0, ord, s, p.seg, pfx)) != hipSuccess) return e;
        a.ord = ord;
        a.pfx = pfx;
    }
    const unsigned blocks = (unsigned)(ws.slots * p.H);
    hipLaunchKernelGGL((bwd_grad_kernel<TI, DK, DV, true>), dim3(blocks), dim3(DV * 4), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_fold_rev_kernel<DK, DV>), dim3((unsigned)((int64_t)p.num_seqs * p.H), DV / 16),
                       dim3(64 * (DK / 16)), 0, s, a.cu, a.nl, p.H, p.seg, a.fM, a.wsD);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = run_states<TI, DK, DV>(a, blocks, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_grad_kernel<TI, DK, DV, false>), dim3(blocks), dim3(DV * 4), 0, s, a);
    return hipGetLastError();
}

template <typename TI>
hipError_t run_bwd_t(const BackwardLaunch& p, hipStream_t s) {
    if (p.dk_dim == 128 && p.dv_dim == 128) return run_bwd<TI, 128, 128>(p, s);
    if (p.dk_dim == 128 && p.dv_dim == 64) return run_bwd<TI, 128, 64>(p, s);
    if (p.dk_dim == 64 && p.dv_dim == 128) return run_bwd<TI, 64, 128>(p, s);
    return run_bwd<TI, 64, 64>(p, s);
}

}  // namespace

hipError_t launch_backward(const BackwardLaunch& p, hipStream_t s) {
    if (p.num_seqs == 0) return hipSuccess;
    return p.bf16 ? run_bwd_t<bf16>(p, s) : run_bwd_t<float>(p, s);
}

}  // namespace gdn
