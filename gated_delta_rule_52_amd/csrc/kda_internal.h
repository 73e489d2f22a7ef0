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
// false when one of the prefill's launches would exceed a grid dimension's 32-bit thread count
bool chunk_grids_fit(int B, int T, int H, int dk, int dv, int N, int chunk, bool varlen, bool in_bf16);
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
// passes of the chunkwise gradients on the matrix-core path (kda_scan.hip): a forward replay that keeps
// every chunk's entering state and V_new, and the two reverse walks that carry the state gradient
constexpr int kStates = 2;
constexpr int kRevLocal = 3;
constexpr int kRevOut = 4;
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
    int fixed_T = -1;       // >= 0: fixed-length batch of N sequences of fixed_T tokens, cut into segments of
    int seg_len = 0;        // seg_len tokens; the table is then computed where needed instead of read
    uint8_t *pz = nullptr;  // [max_segs, H, 8] matrix-core path: byte w is 1 when column tile w (16 columns) of
                            // the segment's P is exactly zero; the local pass writes it for every P it builds
    // segments per sequence of a fixed-length batch
    __device__ __forceinline__ int fixed_segs() const { return (fixed_T + seg_len - 1) / seg_len; }
    __device__ __forceinline__ int count() const { return fixed_T >= 0 ? N * fixed_segs() : seq_seg[N]; }
    // first segment of sequence n (n = N: the count)
    __device__ __forceinline__ int first_seg(int n) const { return fixed_T >= 0 ? n * fixed_segs() : seq_seg[n]; }
    // {sequence, first token, end token, flags} of segment seg
    __device__ __forceinline__ int4 desc(int seg) const {
        if (fixed_T < 0) return table[seg];
        const int ns = fixed_segs(), n = seg / ns, s = seg - n * ns;
        const int t0 = n * fixed_T + s * seg_len, end = (n + 1) * fixed_T;
        return make_int4(n, t0, t0 + seg_len < end ? t0 + seg_len : end,
                         (s == ns - 1 ? kSegLast : 0) | (s == 0 ? kSegFirst : 0));
    }
    // the entering state of segment seg = {sequence, first token, end token, flags} at head h, row-major
    // dk x dv; null stands for the zero state.  A sequence of one segment enters with its initial state,
    // read in place: the workgroup that reads it is the one that later writes the final state, which may
    // alias it.  Longer sequences read a copy, because their last segment may finish before the first
    // has read its entering state.
    // A later segment whose predecessor's P is exactly zero enters with that predecessor's H (the combine
    // leaves such states unwritten when a sequence has no nonzero P).
    __device__ __forceinline__ const float *entering(int seg, int4 sd, int h, int H, int DK, int DV) const {
        if ((sd.w & (kSegFirst | kSegLast)) == (kSegFirst | kSegLast))
            return h0 ? h0 + (static_cast<int64_t>(sd.x) * H + h) * DK * DV : nullptr;
        if (!(sd.w & kSegFirst) && pz_all(seg - 1, h, H)) return Hs + (static_cast<int64_t>(seg - 1) * H + h) * DK * DV;
        return sin + (static_cast<int64_t>(seg) * H + h) * DK * DV;
    }
    // every column tile of segment seg's P at head h is exactly zero (false without flags)
    __device__ __forceinline__ bool pz_all(int seg, int h, int H) const {
        return pz && *reinterpret_cast<const uint64_t *>(pz + (static_cast<int64_t>(seg) * H + h) * 8) ==
                         0x0101010101010101ull;
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
    int seg_len;   // tokens per segment
};
size_t segment_states_bytes(int B, int T, int H, int dk, int dv, int N, bool varlen, int chunk);
// the segment table of a plan at chunk size L.chunk, without operand packs
SegmentStates launch_segment_table(const ChunkLaunch &L);
// the combine into entering states; sequences without tokens get final = initial in L.hT (when given)
void launch_segment_combine(const ChunkLaunch &L, const SegmentStates &s);

// fp16/bf16 matrix-core path (bf16 inputs, dk = dv = 128, chunk 64): a
// parallel prep kernel writes one operand pack per chunk and head
// (kda_prep.hip); the local and output passes stream them (kda_scan.hip).
bool f16_path_supported(bool in_bf16, int dk, int dv, int chunk);
size_t pack_bytes();  // bytes of one operand pack
// rpacks (the gradients only): also the reverse packs' -Kd, -W^T and Q^T slots (kda_mfma.h)
void launch_prep(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, void *packs,
                 void *rpacks = nullptr);
template <int MODE>
void launch_scan(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, const void *packs);

// Buffers of the gradient passes of the scan.  Per chunk (pack slot s = segment * per + chunk, head h,
// index s * H + h) the states and V_new are kept in accumulator order: 16-byte unit (w * R + t) * 64 + l
// holds rows 16 t + 4 (l / 16) .. + 3 of column 16 w + l % 16, R = 8 row tiles for a state (dk x dv),
// R = 4 for V_new (C x dv).
struct ScanGrad {
    float *st;            // kStates: the state entering each chunk (fp16 in the walk's frame, accumulator order)
    int *stf;             // kStates: that frame's exponent per chunk and 16-column tile ([chunk slot * H + h][8])
    int *dstf;            // kRevOut: the same for dst
    float *vn;            // kStates: V_new of each chunk; kRevOut: dV_new of each chunk
    float *dst;           // kRevOut: the gradient of the state each chunk leaves (stored as st)
    const float *dleave;  // kRevOut: [segment * H + h] gradient of the state each segment leaves (row-major)
    const float *dhT;     // kRevOut: [sequence * H + h] final-state gradient (null: zero)
    float *dh0;           // kRevOut: [sequence * H + h] initial-state gradient (null: not written)
    float *hb;            // kRevLocal: [segment * H + h] state gradient at the segment start from zero at its end
    bool keep_last;       // kLocal: P and H of every segment but a one-segment sequence's (the reverse combine
                          // needs P of last segments)
    char *pt;             // kLocal: also P^T as bf16 high and low planes, [segment * H + h] 64 KiB each
    uint8_t *pzh;         // kLocal writes (its second grid layer), kRevLocal reads: [segment * H + h] 8 bytes,
                          // byte w 1 where column tile w of the transition over the segment's first 4 chunks
                          // is exactly zero (not written for segments of at most 4 chunks)
};
template <int MODE>
void launch_scan_grad(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, const void *packs,
                      const ScanGrad &gr);

// The chunkwise gradients (kda_chunk_bwd.hip) on the matrix-core path: the forward part of the segmented
// prefill (segment table, prep, local pass keeping last segments, combine, kStates replay) in the layout
// of the forward plan, then the reverse passes.
struct ChunkGradLayout {
    size_t bytes;  // workspace of the forward part (segment table, states, packs)
    int per;       // chunks per segment
    int max_segs;  // bound on the number of segments
    bool packs;    // the matrix-core path applies
};
ChunkGradLayout chunk_grad_layout(int B, int T, int H, int N, bool varlen);
// Runs the forward part into L.workspace (chunk_grad_layout().bytes), the reverse packs' transposed slots
// into rpacks, and the kStates replay into gr.st and gr.vn; *chained tells whether any sequence has more than one segment (else the local pass, the combines
// and kRevLocal have nothing to do), *packs where the operand packs are.
SegmentView launch_chunk_grad_forward(const ChunkLaunch &L, const ScanGrad &gr, void *rpacks, bool *chained,
                                      void **packs);
// The gradients' reverse combine on bf16 matrix cores for the matrix-core path (dk = dv = 128, kda_segments.hip):
// dleave(s - 1) = P_s^T dleave(s) + Hb_s over the P^T planes in pt (ScanGrad::pt).
void launch_reverse_combine_bf16(const SegmentView &sv, const char *pt, const float *hb, const float *dhT, float *dl,
                                 float *dh0, int H, int N, hipStream_t stream);
bool chunk_bwd_supported(bool in_bf16, int dk, int dv);
size_t chunk_bwd_workspace_bytes(int B, int T, int H, int N, bool varlen);
// false when a launch would exceed a grid dimension's 32-bit thread count or the matrix-core path's
// 32-bit offsets
bool chunk_bwd_grids_fit(int B, int T, int H, int N, bool varlen);
hipError_t launch_chunk_bwd(const BackwardLaunch &L);

// The general DPLR recurrence in chunkwise form (kda_dplr_chunk.hip), on the segment machinery above.
struct DplrChunkLaunch {
    const void *q, *k, *v, *a, *b;
    const float *g;
    const float *h0;
    float *hT;
    void *o;
    const int32_t *cu_seqlens;  // device, or nullptr: B sequences of T tokens
    int B, T, H, dk, dv, N;
    float scale;
    bool in_bf16, out_bf16;
    void *workspace;            // dplr_chunk_workspace_bytes()
    hipStream_t stream;
};
int dplr_chunk_size();
size_t dplr_chunk_workspace_bytes(int B, int T, int H, int dk, int dv, int N, bool varlen);
hipError_t launch_dplr_chunk(const DplrChunkLaunch &L);

// Sets the thread-local text that kda_last_error() returns (kda_api.cpp).
void set_last_error(const char *text);

}  // namespace kda
