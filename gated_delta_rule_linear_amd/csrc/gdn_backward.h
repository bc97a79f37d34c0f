// Host-side launcher of the backward (gradient) kernels in gdn_backward.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_kernels.h"

namespace gdn {

struct BackwardLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;
    const float* initial_state;  // may be null (zero)
    const void* d_o;
    const float* d_final_state;  // may be null (zero)
    void* dq;
    void* dk;
    void* dv;
    float* dg;
    float* dbeta;
    float* d_initial_state;      // may be null (not wanted)
    int32_t num_seqs;
    int32_t H;
    int32_t dk_dim;
    int32_t dv_dim;
    bool bf16;
    int64_t T_total;
    void* workspace;             // backward_workspace_bytes(...) bytes
    int64_t seg = 0;             // time split segment length (tokens, multiple of 64); 0: none
};

// Segment length of the backward's time split for these sizes (tokens, a
// multiple of 64; 0: every (sequence, head) walked by one workgroup).  Depends
// on the arguments only, and on the environment variable GDN_BACKWARD_SEGMENT,
// which forces a length (0 = never split).
int64_t plan_backward_segment(int64_t T_total, int32_t num_seqs, int32_t H);

// Workspace of the backward pass.
//  - Checkpoints: the start state of every 16-token sub-chunk, in the input
//    dtype.  Sequence n's sub-chunk c uses slot cu[n] / 16 + n + c (slots never
//    overlap: a sequence of len tokens needs ceil(len / 16) of them and the next
//    one starts at least that far on), so T_total / 16 + num_seqs slots per head.
//  - With a time split of segment length seg: at pre_off, the forward pass's
//    split workspace (prefill_workspace_layout: the maps M, N of the non-last
//    segments and the segment table); at d_off, per segment slot and head (slot
//    cu[n] / seg + n + j for segment j of sequence n, T_total / seg + num_seqs
//    slots) the d_k x d_v fp32 state gradient D of the reverse fold.
//    For bf16 with d_k = d_v (D from the transition pass, see launch_backward)
//    also, at ml_off, the last segment's transition M of every split sequence
//    (d_k x d_k fp32 per split-list entry and head, min(num_seqs,
//    T_total / (seg + 1)) entries), and at qh_off the bf16 q^ buffer
//    [T_total, H, d_k].
//  - Without the split, when (sequence, head) units outnumber the compute
//    units and there is more than one sequence: at ord_off the int32 order of
//    the sequences, longest first (launch_seq_order), which both sweeps follow.
//    With the split and more than one sequence: that order and, at pfx_off,
//    the int32 segment prefix table [num_seqs + 1] of the sequences in that
//    order, through which the sweeps over segments take the long sequences'
//    segments first.
struct BackwardWorkspace {
    int64_t slots = 0, splits = 0;
    size_t pre_off = 0, d_off = 0, ml_off = 0, qh_off = 0, ord_off = 0, pfx_off = 0, bytes = 0;
    bool ord = false, qmaps = false;
};
inline BackwardWorkspace backward_workspace_layout(int64_t T_total, int32_t num_seqs, int32_t H, int32_t dk,
                                                   int32_t dv, bool bf16, int64_t seg) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BackwardWorkspace w;
    w.pre_off = al(((size_t)(T_total / 16) + (size_t)num_seqs) * (size_t)H * (size_t)dk * (size_t)dv * (bf16 ? 2 : 4));
    w.bytes = w.pre_off;
    if (seg > 0) {
        w.slots = T_total / seg + num_seqs;
        w.d_off = w.pre_off + al(prefill_workspace_layout(T_total, num_seqs, H, dk, dv, seg, false).bytes);
        w.bytes = w.d_off + al((size_t)w.slots * H * dk * dv * sizeof(float));
        if (bf16 && dk == dv) {
            w.qmaps = true;
            w.splits = std::min<int64_t>(num_seqs, T_total / (seg + 1));
            w.ml_off = w.bytes;
            w.qh_off = w.ml_off + al((size_t)w.splits * H * dk * dk * sizeof(float));
            w.bytes = w.qh_off + al((size_t)T_total * H * dk * 2);
        }
        if (num_seqs > 1) {
            w.ord = true;
            w.ord_off = w.bytes;
            w.pfx_off = w.ord_off + al((size_t)num_seqs * sizeof(int32_t));
            w.bytes = w.pfx_off + al(((size_t)num_seqs + 1) * sizeof(int32_t));
        }
    } else if (num_seqs > 1 && (int64_t)num_seqs * H > kComputeUnits) {
        w.ord = true;
        w.ord_off = w.bytes;
        w.bytes += al((size_t)num_seqs * sizeof(int32_t));
    }
    return w;
}
inline size_t backward_workspace_bytes(int64_t T_total, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                                       bool bf16) {
    return backward_workspace_layout(T_total, num_seqs, H, dk, dv, bf16,
                                     plan_backward_segment(T_total, num_seqs, H)).bytes;
}

// Returns hipSuccess or the launch error.  Sizes are validated by the caller.
hipError_t launch_backward(const BackwardLaunch& p, hipStream_t stream);

}  // namespace gdn
