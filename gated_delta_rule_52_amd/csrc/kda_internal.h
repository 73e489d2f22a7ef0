// kda_internal.h - launch descriptors shared by the host entry points
// (kda_api.cpp) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Optional per-token input transforms (KDA_FLAG_* in kda.h), handed to the
// kernels by value.
constexpr float kL2Eps = 1e-6f;  // the L2 norm's epsilon, KDA_L2NORM_EPS
struct InputXform {
    bool qk_l2norm;      // q, k divided by sqrt(sum x^2 + kL2Eps) over dk
    bool gate_softplus;  // g holds logits z; log-gate = -gate_scale softplus(z)
    float gate_scale;
    bool scalar_gate;    // g is [tokens, H]: one gate per token and head for every key channel
    bool any() const { return qk_l2norm || gate_softplus || scalar_gate; }
    // The log-gate for input value g.  softplus(z) = log(1 + e^z) is taken as
    // max(z, log(1 + e^min(z, 15))): above 15 softplus(z) - z < 3.1e-7, and
    // below it the only loss is 1 + e^z rounding, an absolute error under
    // 6e-8 in the log-gate, i.e. a relative error of that size in alpha.
    __device__ __forceinline__ float log_gate(float g) const {
        return gate_softplus ? -gate_scale * fmaxf(g, __logf(1.f + __expf(fminf(g, 15.f)))) : g;
    }
};

// Token-by-token kernel: decode step (T = 1, N = number of sequences) or a
// loop over the tokens of each sequence.
struct RecurrentLaunch {
    const void *q, *k, *v;
    const float *g;
    const void *beta;
    const float *h0;
    float *hT;
    void *o;
    const int32_t *cu_seqlens;  // device, or nullptr: N sequences of T tokens
    int N, T, H, dk, dv;
    float scale;
    bool in_bf16, out_bf16;
    bool multi_token;           // split dv into narrow slices for long loops
    InputXform xf;
    hipStream_t stream;
};

hipError_t launch_recurrent(const RecurrentLaunch &L);

// The general DPLR recurrence, token by token (kda_dplr.hip).
struct DplrLaunch {
    const void *q, *k, *v, *a, *b;
    const float *g;
    const float *h0;
    float *hT;
    void *o;
    const int32_t *cu_seqlens;  // device, or nullptr: N sequences of T tokens
    int N, T, H, dk, dv;
    float scale;
    bool in_bf16, out_bf16;
    hipStream_t stream;
};

hipError_t launch_dplr(const DplrLaunch &L);

// Gradients of the recurrence, token by token (kda_backward.hip).
struct BackwardLaunch {
    const void *q, *k, *v;
    const float *g;
    const void *beta;
    const void *d_o;            // output gradient, dtype of q
    const float *h0, *dhT;      // initial state and final-state gradient (null: zero)
    float *dq, *dk, *dv, *dg, *dbeta, *dh0;  // fp32; dh0 may be null
    const int32_t *cu_seqlens;  // device, or nullptr: B sequences of T tokens
    int B, N, T, H, dk_dim, dv_dim;
    float scale;
    bool in_bf16;
    bool scalar_gate;           // g and dg are [tokens, H]: one gate per token and head
    InputXform xf;              // Q/K L2 norm and softplus gate: gradients of the raw inputs
    void *workspace;            // backward_workspace_bytes()
    float *ckpt;                // stored forward states (set by launch_backward inside the workspace)
    hipStream_t stream;
};

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int N, bool varlen, bool transforms,
                                bool scalar_gate);
hipError_t launch_backward(const BackwardLaunch &L);

// Chunkwise prefill.
struct ChunkLaunch {
    const void *q, *k, *v;
    const float *g;
    const void *beta;
    const float *h0;
    float *hT;
    void *o;
    const int32_t *cu_seqlens;  // device, or nullptr
    int B, T, H, dk, dv, N;
    int chunk;
    float scale;
    bool in_bf16, out_bf16;
    InputXform xf;
    void *workspace;
    size_t workspace_bytes;
    hipStream_t stream;
};

size_t chunk_workspace_bytes(int B, int T, int H, int dk, int dv, int N, int chunk, bool varlen, bool in_bf16);
hipError_t launch_chunk(const ChunkLaunch &L);

// ---- segmented prefill (kda_segments.hip)
//
// Sequences are cut into segments of whole chunks.  Pass 1 (kLocal) gives
// every segment but the last of each sequence its local state H (zero start)
// and transition P (identity start, v = 0), so that leaving state =
// P * entering state + H.  The combine pass chains these per sequence from
// the initial state and stores each segment's entering state; pass 2 (kOut)
// replays every segment from its entering state and writes o (and, for the
// last segment, the final state).
constexpr int kLocal = 0;
constexpr int kOut = 1;
constexpr int kSegLast = 1;
constexpr int kSegFirst = 2;

struct SegmentView {
    const int4 *table;      // [max_segs] {sequence, first token, end token, flags}
    const int32_t *seq_seg; // [N + 1] first segment of each sequence; [N] = count
    int N;
    float *P;               // [max_segs, H, dk, dk] fp32; on the matrix-core path two bf16 planes in the same
                            // bytes per (segment, head): high parts [dk][dk], then low parts [dk][dk]
    float *Hs;              // [max_segs, H, dk, dv]
    float *sin;             // [max_segs, H, dk, dv] entering states (not filled for one-segment sequences)
    const float *h0;        // [N, H, dk, dv] initial states (null: zero)
    int *xlist;             // chunks (pack numbers) the matrix-core prep hands to its exact path
    int *xcount;            // their count (zeroed by the segment-table kernel)
    __device__ __forceinline__ int count() const { return seq_seg[N]; }
    // the entering state of segment seg = {sequence, first token, end token, flags} at head h, row-major
    // dk x dv; null stands for the zero state.  A sequence of one segment enters with its initial state,
    // read in place: the workgroup that reads it is the one that later writes the final state, which may
    // alias it.  Longer sequences read a copy, because their last segment may finish before the first
    // has read its entering state.
    __device__ __forceinline__ const float *entering(int seg, int4 sd, int h, int H, int DK, int DV) const {
        if ((sd.w & (kSegFirst | kSegLast)) == (kSegFirst | kSegLast))
            return h0 ? h0 + (static_cast<int64_t>(sd.x) * H + h) * DK * DV : nullptr;
        return sin + (static_cast<int64_t>(seg) * H + h) * DK * DV;
    }
};

template <int MODE>
void launch_fp32_pass(const ChunkLaunch &L, const SegmentView &sv, int max_segs);

// Pieces of the segmented forward for the gradients: the segment table of a
// plan without operand packs (chunk 64), and the combine that turns P and H
// of every segment (written by the caller's own local pass into sv.P, sv.Hs)
// into entering states.  L.workspace must hold segment_states_bytes(); o and
// hT are not touched.
struct SegmentStates {
    SegmentView sv;
    int max_segs;  // bound on the number of segments (grid size)
};
size_t segment_states_bytes(int B, int T, int H, int dk, int dv, int N, bool varlen);
SegmentStates launch_segment_table(const ChunkLaunch &L);
void launch_segment_combine(const ChunkLaunch &L, const SegmentStates &s);

// fp16/bf16 matrix-core path (bf16 inputs, dk = dv = 128, chunk 64): a
// parallel prep kernel writes one operand pack per chunk and head
// (kda_prep.hip); the local and output passes stream them (kda_scan.hip).
bool f16_path_supported(bool in_bf16, int dk, int dv, int chunk);
size_t pack_bytes();  // bytes of one operand pack
void launch_prep(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, void *packs);
template <int MODE>
void launch_scan(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, const void *packs);

}  // namespace kda
