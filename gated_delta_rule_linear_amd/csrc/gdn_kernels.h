// Host-side launchers of the libgdn kernels (defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Gate of a call: GATE_LOG, GATE_SCALED_SIGMOID and GATE_ALPHA_MIN are the
// values of gdn_gate; GATE_HEAD is the one-gate-per-(token, head) entry points.
constexpr int GATE_LOG = 0;             // g given per key channel
constexpr int GATE_SCALED_SIGMOID = 1;  // g = p sigmoid(z), p = g_min
constexpr int GATE_ALPHA_MIN = 2;       // g = log(p + (1 - p) sigmoid(z)), p = a_min
constexpr int GATE_HEAD = 3;            // one g per (token, head), shared by the key channels

struct PrefillLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;
    const float* initial_state;  // may be null
    float* final_state;          // may be null
    void* o;
    int32_t num_seqs;
    int32_t H;
    int32_t dk;
    int32_t dv;
    bool bf16;
    int64_t T_total;
    int64_t seg;      // segment length of the time split (tokens, multiple of 64); 0: none
    void* workspace;  // prefill_workspace_layout(...).bytes bytes (none when that is 0)
    bool legacy;      // bf16: single-role kernel (GDN_PREFILL_KERNEL=seq) instead of the warp-specialised one
    const void* z = nullptr;  // bf16 gate logits [T_total, H, d_k] (gate != 0; g unused)
    int32_t gate = 0;         // 0: g given; 1, 2: gdn_gate parameterisation of z
    float gate_param = 0.f;
    int64_t max_seqlen = 0;   // host-side bound on the sequence lengths (0: unknown)
};

// Compute units of the device the plans are made for (MI355X).
constexpr int64_t kComputeUnits = 256;
// Shortest segment of the length-agnostic split of a batch that the
// mean-length plan does not split (a segment of 512 chunks of 32 tokens).
constexpr int64_t kSpeculativeMinSegment = 16384;

// Workspace of the prefill.
// Time split, for segments of `seg` tokens: a sequence's non-last segments
// hold exactly seg tokens, so there are at most T_total / seg of them over the
// batch; each (non-last segment, head) owns an M slot (d_k x d_k fp32) and an
// N slot (d_k x d_v fp32).  nl is the int32 table of non-last segment counts
// [num_seqs + 1]; spl lists the sequences that have more than one segment (a
// sequence longer than seg tokens: at most min(num_seqs, T_total / (seg + 1))
// of them, the `splits` entries of the list, unused ones -1), so that the fold
// runs one workgroup per split (sequence, head) only.
// Unit order: with more than one sequence, the workgroups of a pass over
// whole sequences (or over every sequence's first segment) take the sequences
// longest first, from the int32 table ord [num_seqs] (a permutation of the
// sequence indices that the order kernel writes at the start of the call), so
// that the long chains start first.  It is kept when the split runs, or when
// there are more (sequence, head) units than compute units; otherwise every
// unit starts at once and the order changes nothing.  (with_order = false: the
// maps and fold alone, which need no order.)
struct PrefillWorkspace {
    int64_t slots = 0, splits = 0;
    size_t m_off = 0, n_off = 0, nl_off = 0, spl_off = 0, ord_off = 0, bytes = 0;
    bool ord = false;
};
inline PrefillWorkspace prefill_workspace_layout(int64_t T_total, int32_t num_seqs, int32_t H, int32_t dk,
                                                 int32_t dv, int64_t seg, bool with_order = true) {
    PrefillWorkspace w;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    if (seg > 0) {
        w.slots = T_total / seg;
        w.m_off = 0;
        w.n_off = al((size_t)w.slots * H * dk * dk * sizeof(float));
        w.nl_off = w.n_off + al((size_t)w.slots * H * dk * dv * sizeof(float));
        w.splits = std::min<int64_t>(num_seqs, T_total / (seg + 1));
        w.spl_off = w.nl_off + al(((size_t)num_seqs + 1) * sizeof(int32_t));
        w.bytes = w.spl_off + al((size_t)std::max<int64_t>(w.splits, 1) * sizeof(int32_t));
    }
    if (with_order && num_seqs > 1 && (seg > 0 || (int64_t)num_seqs * H > kComputeUnits)) {
        w.ord = true;
        w.ord_off = w.bytes;
        w.bytes += al((size_t)num_seqs * sizeof(int32_t));
    }
    return w;
}

// Cost model of the time split, in chunk-times of the output pass, fitted to
// measured kernel times on MI355X (one workgroup per CU at a time).
struct SplitCost {
    // Costs in units of one 64-token chunk of the output pass with every CU busy
    // (fitted to kernel traces of the bf16 kernels at d = 128 on MI355X).
    static constexpr double CUS = (double)kComputeUnits;
    static constexpr double MAP_ONE = 0.76;  // a transition workgroup computing M or N
    static constexpr double MAP_BOTH = 0.87; // one computing M and N together (bf16, d_k = d_v)
    static constexpr double START = 0.7;     // fixed cost per workgroup
    static constexpr double FOLD = 0.6;      // per fold step and round of 256 fold workgroups
    // Relative time of a round in which a fraction `occ` of the CUs is busy: a
    // chunk runs faster when fewer workgroups share HBM and the power budget
    // (measured 0.79 with 1/8 of the CUs busy, 0.80 at 1/4, 0.85 at 1/2).
    static double occ_factor(double occ) {
        static const double X[5] = {0.0, 0.125, 0.25, 0.5, 1.0}, Y[5] = {0.79, 0.791, 0.801, 0.845, 1.0};
        if (occ >= 1.0) return 1.0;
        int i = 0;
        while (occ > X[i + 1]) ++i;
        return Y[i] + (Y[i + 1] - Y[i]) * (occ - X[i]) / (X[i + 1] - X[i]);
    }
    // Critical path of `wgs` workgroups in rounds of CUS, the last round weighted by its occupancy.
    static double rounds(double wgs) {
        if (wgs <= 0) return 0;
        const double full = (double)(int64_t)(wgs / CUS), rem = wgs - full * CUS;
        return full + (rem > 0 ? occ_factor(rem / CUS) : 0.0);
    }
    // Critical path of the transition pass over `maps` (segment, head) pairs of
    // `chunks` chunks; *both says whether M and N share a workgroup.
    static double maps_pass(double maps, double chunks, bool can_share, bool* both) {
        const double one = rounds(2 * maps) * (chunks * MAP_ONE + START);
        const double two = can_share ? rounds(maps) * (chunks * MAP_BOTH + START) : one + 1;
        if (both) *both = two < one;
        return two < one ? two : one;
    }
    // The fold: `steps` sequential steps, each over (sequence, head, 16 columns) workgroups.
    static double fold_pass(double steps, double fold_wgs) {
        return steps * FOLD * (double)(int64_t)((fold_wgs + CUS - 1) / CUS);
    }
};

// Segment length chosen for a batch of these sizes (0: one workgroup per whole
// sequence and head).  Depends on the arguments only (max_seqlen: a host-side
// bound on the lengths, 0 when unknown), and on the environment variable
// GDN_PREFILL_SEGMENT, which forces a length (0 = never split).
int64_t plan_prefill_segment(int64_t T_total, int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, bool bf16,
                             int64_t max_seqlen = 0);

struct DecodeLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* o;
    int32_t N;
    int32_t H;
    int32_t dk;
    int32_t dv;
    bool bf16;
    const void* z = nullptr;  // bf16 gate logits [N, H, d_k] (gate != 0; g unused)
    int32_t gate = 0;
    float gate_param = 0.f;
};

// Each returns hipSuccess or the launch error.  Sizes are validated by the caller.
hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream);
// The first half of the time split alone (p.seg > 0, workspace laid out by
// prefill_workspace_layout): the segment table nl, the maps of every non-last
// segment and the fold.  On return, for segment j of sequence n that is not
// its last, slot nl[n] + j of wsM holds its transition M_j and slot
// nl[n] + j of wsN the start state of segment j + 1.  o and final_state are
// not used.
hipError_t launch_prefill_maps(const PrefillLaunch& p, hipStream_t stream);
// The same for the backward's time split with q^ (bf16, d_k = d_v, per-channel
// gates; M and N in one workgroup): besides the above, for every segment j >= 1
// of a split sequence, q^_t = M_{j,t}^T q_t for its tokens t into qh (bf16
// [T_total, H, d_k]; M_{j,t}: the transition from the segment's start through
// token t), and the last segment's transition M into slot kk of wsML
// (d_k x d_k fp32 per (split-list entry, head), the sequence in entry kk of the
// split list).
hipError_t launch_prefill_maps_q(const PrefillLaunch& p, void* qh, float* wsML, hipStream_t stream);
// The backward's checkpoint pass on the prefill's bf16 kernel: the state at
// the start of every 16-token window of each unit (one (sequence, head), or
// with the time split one (segment, head); the units and their order are those
// of the backward's sweeps) in bf16 to slot (cu[n] / 16 + n + c, h) of ck
// ([slot][H][d_k][d_v]; c: the window's index in sequence n).  A unit starts
// from initial_state (or zero) or, for segment j >= 1 of sequence n, from slot
// nl[n] + j - 1 of seg_start (launch_prefill_maps' wsN).
struct CheckpointLaunch {
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;
    const float* initial_state;  // may be null
    int32_t num_seqs;
    int32_t H;
    int32_t dk;
    int32_t dv;
    int64_t seg;                 // 0: no split
    const int32_t* nl;           // time split only
    const float* seg_start;      // time split only
    const int32_t* ord;          // may be null
    const int32_t* pfx;          // time split: may be null
    void* ck;
    int64_t blocks;              // grid: the backward's sweeps' grid
};
hipError_t launch_backward_checkpoints(const CheckpointLaunch& c, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& p, hipStream_t stream);
// The unit order (see PrefillWorkspace): ord[0 .. num_seqs) receives the
// sequence indices, longest first, lengths capped at cap tokens when cap > 0;
// with pfx, also pfx[0 .. num_seqs]: pfx[i] is the number of segments of seg
// tokens (one for an empty sequence) of the sequences ord[0 .. i-1].
hipError_t launch_seq_order(const int32_t* cu_seqlens, int32_t num_seqs, int64_t cap, int32_t* ord,
                            hipStream_t stream, int64_t seg = 1, int32_t* pfx = nullptr);

}  // namespace gdn
