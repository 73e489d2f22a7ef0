// kda_segments.hip - segmented chunkwise prefill: the chunk table, the
// combine pass, and the host orchestration of the passes.
//
// Only the fp32 state crosses chunk boundaries (Kimi Linear review notes,
// section "Chunkwise Algorithm"), and the state map of a run of chunks is
// affine: leaving = P * entering + H, with P the product of the chunks'
// transitions (dk x dk) and H the state reached from zero.  This lets the
// long, serial chunk chain of a sequence be cut into segments that run in
// parallel on all compute units:
//
//   table   : cut every sequence into segments of whole chunks, chunks never
//             straddling two sequences (packed variable length);
//   prep    : (matrix-core path) per (chunk, head), in parallel: everything
//             in a chunk that does not depend on the entering state;
//   pass 1  : per (segment, head), in parallel: H and P of the segment;
//   combine : per (sequence, head, dv slice), serial over its segments:
//             entering(s+1) = P_s entering(s) + H_s, from the initial state;
//   pass 2  : per (segment, head), in parallel: replay from the entering
//             state, write o and (last segment) the final state.
//
// All passes run on the caller's stream; nothing is allocated.
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {

namespace {

// segments x heads: one long segment per compute unit and pass; for short problems (at most 1,024
// chunk-heads) half that, where the combine's serial chain would cost more than the extra parallelism saves
// (measured: 2K tokens x 16 heads 90 -> 79 us), unless segments of kTail chunks give more (4K tokens x 16
// heads: 16 segments of 4 chunks per head, 93.5 -> 85.6 us)
constexpr int kTargetUnits = 256, kTargetUnitsShort = 128, kShortChunkHeads = 1024;
constexpr int kTail = 4;  // chunks the local pass walks first at a segment's end (kda_scan.hip)

struct Plan {
    int per;        // chunks per segment
    int seg_len;    // tokens per segment (per * chunk)
    int max_segs;   // bound on the number of segments
    bool packs;     // matrix-core path: one operand pack per chunk and head
    size_t off_table, off_seq, off_P, off_H, off_S, off_pack, off_pz, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~size_t{255}; }

Plan make_plan(int B, int T, int H, int dk, int dv, int N, int chunk, bool varlen, bool in_bf16) {
    Plan p{};
    const int64_t tokens = varlen ? T : static_cast<int64_t>(B) * T;
    const int64_t chunks = varlen ? (tokens + chunk - 1) / chunk + N
                                  : static_cast<int64_t>(B) * ((T + chunk - 1) / chunk);
    // short problems: segments of at least kTail chunks (the local pass walks such a segment whole, and its
    // transition is then zero under strong gates, which empties the combine), at most 256 of them
    const int64_t units = chunks * H <= kShortChunkHeads
                              ? std::max<int64_t>(kTargetUnitsShort, std::min<int64_t>(kTargetUnits, chunks * H / kTail))
                              : kTargetUnits;
    int64_t per = (chunks * H + units - 1) / units;
    if (per > 64) per = 64;
    // Segments never span two sequences, so a segment longer than the
    // sequences only pads the pack array (and the prep grid) with empty
    // slots: cap it at the sequence length, or for packed input at the
    // average sequence length (the lengths themselves live on the device).
    const int64_t seq_chunks = varlen ? (tokens + static_cast<int64_t>(chunk) * N - 1) / (static_cast<int64_t>(chunk) * (N > 0 ? N : 1))
                                      : (T + chunk - 1) / chunk;
    if (per > seq_chunks) per = seq_chunks;
    if (per < 1) per = 1;
    p.per = static_cast<int>(per);
    p.seg_len = p.per * chunk;
    p.max_segs = varlen ? static_cast<int>((tokens + p.seg_len - 1) / p.seg_len + N)
                        : B * ((T + p.seg_len - 1) / p.seg_len);
    if (p.max_segs < 1) p.max_segs = 1;
    // the matrix-core kernels address a segment's tokens with 32-bit byte offsets
    p.packs = f16_path_supported(in_bf16, dk, dv, chunk) &&
              static_cast<int64_t>(p.seg_len) * H * dk * sizeof(float) < (int64_t{1} << 31);
    const size_t ms = static_cast<size_t>(p.max_segs);
    size_t o = 0;
    p.off_table = o; o = align256(o + ms * sizeof(int4));
    p.off_seq = o;   o = align256(o + (static_cast<size_t>(N) + 1) * sizeof(int32_t));
    p.off_P = o;     o = align256(o + ms * H * dk * dk * sizeof(float));
    p.off_H = o;     o = align256(o + ms * H * dk * dv * sizeof(float));
    p.off_S = o;     o = align256(o + ms * H * dk * dv * sizeof(float));
    p.off_pack = o;  o = align256(o + (p.packs ? ms * p.per * H * pack_bytes() : 0));
    p.off_pz = o;    o = align256(o + (p.packs ? ms * H * 8 : 0));
    p.bytes = o;
    return p;
}

// a7: the segment table.  Each thread owns a contiguous range of sequences;
// one block-wide exclusive scan of the per-thread segment counts (shuffles
// within each wave, then the four wave totals) gives every sequence its first
// segment.
__global__ void __launch_bounds__(256)
build_segments_kernel(const int32_t *__restrict__ cu_seqlens, int T, int N, int seg_len,
                      int4 *__restrict__ table, int32_t *__restrict__ seq_seg) {
    __shared__ int s_cnt[4];
    const int tid = threadIdx.x;
    const int per = (N + 255) / 256;
    const int n0 = tid * per, n1 = min(N, n0 + per);
    auto bounds = [&](int n, int64_t &a, int64_t &b) {
        if (cu_seqlens) {
            a = cu_seqlens[n];
            b = cu_seqlens[n + 1];
            if (b < a) b = a;
        } else {
            a = static_cast<int64_t>(n) * T;
            b = a + T;
        }
    };
    int cnt = 0;
    for (int n = n0; n < n1; ++n) {
        int64_t a, b;
        bounds(n, a, b);
        cnt += static_cast<int>((b - a + seg_len - 1) / seg_len);
    }
    // exclusive scan of the counts: inclusive within each wave by shuffles, then the wave totals
    const int lane = tid & 63, wave = tid >> 6;
    int inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
    }
    if (lane == 63) s_cnt[wave] = inc;
    __syncthreads();
    int idx = inc - cnt;
    for (int w = 0; w < wave; ++w) idx += s_cnt[w];
    if (tid == 255) seq_seg[N] = idx + cnt;
    for (int n = n0; n < n1; ++n) {
        int64_t a, b;
        bounds(n, a, b);
        seq_seg[n] = idx;
        const int ns = static_cast<int>((b - a + seg_len - 1) / seg_len);
        for (int s = 0; s < ns; ++s) {
            const int64_t t0 = a + static_cast<int64_t>(s) * seg_len;
            const int64_t t1 = t0 + seg_len < b ? t0 + seg_len : b;
            const int flags = (s == ns - 1 ? kSegLast : 0) | (s == 0 ? kSegFirst : 0);
            table[idx++] = make_int4(n, static_cast<int>(t0), static_cast<int>(t1), flags);
        }
    }
}

// Combine: per (sequence, head, 16-column slice of dv), walk the segments in
// order, store each entering state and advance it by  S <- P_s S + H_s.
// Sequences of one segment are skipped: their output pass reads the initial
// state itself.
// P_s (dk x dk fp32) is staged in LDS; the next one is fetched into registers
// while the current product runs.  fp32 FMA throughout.
template <int DK>
__global__ void __launch_bounds__(256, 1)
combine_kernel(SegmentView sv, const float *h0, float *hT, int H, int DV) {
    constexpr int BV = 16, DKP = DK + 1, RG = 256 / BV, ROWS = DK / RG;
    constexpr int PV4 = DK * DK / 4 / 256;   // float4 loads per thread for one P
    __shared__ float sP[DK * DKP];
    __shared__ float sS[DK * BV];
    const int slice = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
    const int tid = threadIdx.x, j = tid % BV, ig = tid / BV;
    const int j0 = slice * BV;
    const int first = sv.first_seg(n), end = sv.first_seg(n + 1);
    if (end - first == 1) return;  // one segment: nothing to carry
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;

    float s[ROWS];
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
        const int i = ig + RG * u;
        s[u] = h0 ? h0[sbase + static_cast<int64_t>(i) * DV + j0 + j] : 0.f;
    }
    if (first == end) {  // empty sequence: the final state is the initial state
        if (hT)
#pragma unroll
            for (int u = 0; u < ROWS; ++u) hT[sbase + static_cast<int64_t>(ig + RG * u) * DV + j0 + j] = s[u];
        return;
    }
    float4 pn[PV4];
    auto fetch = [&](int seg) {
        const float4 *src = reinterpret_cast<const float4 *>(sv.P + (static_cast<int64_t>(seg) * H + h) * DK * DK);
#pragma unroll
        for (int m = 0; m < PV4; ++m) pn[m] = src[tid + 256 * m];
    };
    if (first + 1 < end) fetch(first);
    for (int seg = first; seg < end; ++seg) {
        float *sin = sv.sin + (static_cast<int64_t>(seg) * H + h) * DK * DV;
#pragma unroll
        for (int u = 0; u < ROWS; ++u) sin[static_cast<int64_t>(ig + RG * u) * DV + j0 + j] = s[u];
        if (seg + 1 == end) break;
        __syncthreads();  // previous product finished with sP and sS
#pragma unroll
        for (int m = 0; m < PV4; ++m) {
            const int e = 4 * (tid + 256 * m), r = e / DK, c = e % DK;
            sP[r * DKP + c] = pn[m].x;
            sP[r * DKP + c + 1] = pn[m].y;
            sP[r * DKP + c + 2] = pn[m].z;
            sP[r * DKP + c + 3] = pn[m].w;
        }
#pragma unroll
        for (int u = 0; u < ROWS; ++u) sS[(ig + RG * u) * BV + j] = s[u];
        __syncthreads();
        if (seg + 2 < end) fetch(seg + 1);
        const float *hs = sv.Hs + (static_cast<int64_t>(seg) * H + h) * DK * DV;
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int i = ig + RG * u;
            float a0 = 0.f, a1 = 0.f;
            for (int m = 0; m < DK; m += 2) {
                a0 += sP[i * DKP + m] * sS[m * BV + j];
                a1 += sP[i * DKP + m + 1] * sS[(m + 1) * BV + j];
            }
            s[u] = (a0 + a1) + hs[static_cast<int64_t>(i) * DV + j0 + j];
        }
    }
}

// Combine on fp32 matrix cores (dk = 128): per (sequence, head, 16-column
// slice of dv), entering(s+1) = P_s entering(s) + H_s, serial over the
// sequence's segments.  Wave w produces row tiles 2w and 2w + 1 with
// v_mfma_f32_16x16x4f32.  The contraction index of a product runs over
// (tile t, lane group g, jj) as k = 16 t + 4 g + jj, so that
// * lane (m, g) takes its A operands for row r straight from HBM as eight
//   16-byte pieces P[r][16 t + 4 g .. + 3] (no LDS), fetched two segments
//   ahead into a register ring;
// * the B operand, the state slice, is read from LDS kept transposed
//   ([column][row]), and the accumulator layout of a result is exactly that
//   layout, so each step writes its result back without reshuffling.
// The state slice alternates between two LDS buffers: one barrier per step.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kCP = 132;  // padded row stride of the transposed state (floats)

__global__ void __launch_bounds__(256, 1)
combine_mfma_kernel(SegmentView sv, const float *h0, float *hT, int H, int DV) {
    constexpr int DK = 128;
    __shared__ __attribute__((aligned(16))) float sS[2][16 * kCP];
    // grid (H, dv / 16, N): the eight slices of head h are workgroups h + H i, all on XCD h mod 8
    // when H is a multiple of 8, so P_s is read from HBM once per head and then hits in that L2
    const int h = blockIdx.x, slice = blockIdx.y, n = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, m = lane & 15;
    const int j0 = 16 * slice;
    const int first = sv.first_seg(n), end = sv.first_seg(n + 1);
    const int nsteps = end - first - 1;  // segments whose leaving state is some segment's entering state
    if (nsteps == 0) return;             // one segment: nothing to carry
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;

    // entering state of the first segment: thread (row tid / 2, 8 columns)
    {
        const int r = tid >> 1, c8 = 8 * (tid & 1);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = h0 ? h0[sbase + static_cast<int64_t>(r) * DV + j0 + c8 + e] : 0.f;
        if (first == end) {  // empty sequence: the final state is the initial state
            if (hT)
#pragma unroll
                for (int e = 0; e < 8; ++e) hT[sbase + static_cast<int64_t>(r) * DV + j0 + c8 + e] = x[e];
            return;
        }
        float *sin = sv.sin + (static_cast<int64_t>(first) * H + h) * DK * DV;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sin[static_cast<int64_t>(r) * DV + j0 + c8 + e] = x[e];
            sS[0][(c8 + e) * kCP + r] = x[e];
        }
    }

    // operands of one step: P rows 16 (2 wave + ii) + m at columns 16 t + 4 g, and H at the accumulator positions
    auto fetch = [&](int seg, f32x4 (&pa)[2][8], f32x4 (&hb)[2]) {
        const float *src = sv.P + (static_cast<int64_t>(seg) * H + h) * DK * DK;
        const float *hs = sv.Hs + (static_cast<int64_t>(seg) * H + h) * DK * DV;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int r = 16 * (2 * wave + ii) + m;
#pragma unroll
            for (int t = 0; t < 8; ++t) pa[ii][t] = *reinterpret_cast<const f32x4 *>(src + r * DK + 16 * t + 4 * g);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                hb[ii][jj] = hs[static_cast<int64_t>(16 * (2 * wave + ii) + 4 * g + jj) * DV + j0 + m];
        }
    };
    // one step: entering(seg + 1) from entering(seg) in sS[b], into sS[b ^ 1]
    auto step = [&](int seg, int b, const f32x4 (&pa)[2][8], const f32x4 (&hb)[2]) {
        __syncthreads();  // entering(seg) complete in sS[b]; sS[b ^ 1] no longer read
        f32x4 acc[2] = {hb[0], hb[1]};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(&sS[b][m * kCP + 16 * t + 4 * g]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
                    acc[ii] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[ii][t][jj], bv[jj], acc[ii], 0, 0, 0);
        }
        float *sin = sv.sin + (static_cast<int64_t>(seg + 1) * H + h) * DK * DV;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int r0 = 16 * (2 * wave + ii) + 4 * g;
            *reinterpret_cast<f32x4 *>(&sS[b ^ 1][m * kCP + r0]) = acc[ii];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sin[static_cast<int64_t>(r0 + jj) * DV + j0 + m] = acc[ii][jj];
        }
    };
    // Two segments' operands in flight.  The fetches are unconditional (past the
    // last step they repeat its segment) so that every path through the loop
    // has the same memory operations and the wait for a buffer leaves the
    // other one in flight.
    const int last_seg = end - 2;
    f32x4 pA[2][8], pB[2][8], hA[2], hB[2];
    fetch(first, pA, hA);
    fetch(min(first + 1, last_seg), pB, hB);
    int i = 0;
    for (; i + 1 < nsteps; i += 2) {
        step(first + i, 0, pA, hA);
        fetch(min(first + i + 2, last_seg), pA, hA);
        step(first + i + 1, 1, pB, hB);
        fetch(min(first + i + 3, last_seg), pB, hB);
    }
    if (i < nsteps) step(first + i, 0, pA, hA);
}

// Combine on bf16 matrix cores for the matrix-core prefill (dk = dv = 128):
// per (sequence, head, 16-column slice of dv) one workgroup of 8 waves walks
// the chain entering(s+1) = P_s entering(s) + H_s on its 16 columns of the
// state (columns evolve independently).  P_s arrives from the local pass as
// bf16 high and low planes (P = hi + lo to about 16 significant bits); the
// state slice is split the same way at every step.  Each product is
// hi.hi + hi.lo + lo.hi on v_mfma_f32_16x16x32_bf16 with fp32 accumulation,
// about 2^-16 relative error per step, well inside the bf16 path's budget.
//
// The chain is bound by memory latency, not arithmetic (a step is 3 x 4
// products per wave).  Wave w owns row tile w; its P operands (rows 16 w + m,
// k = 32 t + 8 g .. + 7 for lane (m, g): 16 contiguous bytes of a row of each
// plane) and H addends go through a ring of four register stages, fetched
// three steps before their step.  A head's eight slices sit on one XCD (heads
// fastest in the grid), where P_s is read from HBM once.  The state slice
// lives in LDS transposed ([column][row]) in hi and lo planes, double
// buffered: the B operand of block t is 16 contiguous bytes of a column, and
// the accumulator (rows 16 w + 4 g .. + 3 of column m) goes back as 8
// contiguous bytes per plane.  One barrier per step.
//
// REV runs the gradients' reverse chain the same way: from the final-state
// gradient (h0 here), dleave(s - 1) = P_s^T dleave(s) + Hb_s from the last
// segment down to the first, over P^T planes (pt, written by the local pass
// beside P) and Hb (hb), storing every segment's leaving gradient in dl; an
// empty sequence's initial-state gradient (hT here) is the final-state one.
constexpr int kSP = 128 + 8;  // padded row stride (bf16) of the transposed state planes

template <bool REV>
__global__ void __launch_bounds__(512, 1)
combine_bf16x3_kernel(SegmentView sv, const float *h0, float *hT, int H, const char *pt, const float *hb, float *dl) {
    constexpr int DK = 128, DV = 128, NC = 16;  // columns per workgroup
    typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
    typedef unsigned u4v __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) uint16_t sS[2][2][NC * kSP];  // [buffer][hi, lo][column * kSP + row]
    const int h = blockIdx.x, slice = blockIdx.y, n = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, m = lane & 15;
    const int j0 = NC * slice;
    const int first = sv.first_seg(n), end = sv.first_seg(n + 1);
    const int nsteps = end - first - 1;
    if (nsteps == 0) return;  // one segment: nothing to carry
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;

    {   // entering state of the first segment: thread (row tid / 4, 4 columns of the slice)
        const int r = tid >> 2, cl = 4 * (tid & 3);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = h0 ? h0[sbase + static_cast<int64_t>(r) * DV + j0 + cl + e] : 0.f;
        if (first == end) {  // empty sequence: the final state is the initial state
            if (hT)
#pragma unroll
                for (int e = 0; e < 4; ++e) hT[sbase + static_cast<int64_t>(r) * DV + j0 + cl + e] = x[e];
            return;
        }
        float *sin = REV ? dl + (static_cast<int64_t>(end - 1) * H + h) * DK * DV
                         : sv.sin + (static_cast<int64_t>(first) * H + h) * DK * DV;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sin[static_cast<int64_t>(r) * DV + j0 + cl + e] = x[e];
            const __bf16 hi = static_cast<__bf16>(x[e]);
            sS[0][0][(cl + e) * kSP + r] = __builtin_bit_cast(uint16_t, hi);
            sS[0][1][(cl + e) * kSP + r] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[e] - static_cast<float>(hi)));
        }
    }

    // segments the chain reads: first .. end - 2 forward, end - 1 .. first + 1 reversed
    auto seg_of = [&](int i) { return REV ? end - 1 - i : first + i; };
    // steps whose P is exactly zero (all eight column tiles flagged by the local pass) reduce to
    // entering(s + 1) = H_s: their P operands come from an empty buffer range, which reads zeros
    // without a memory access (the same instructions run, so the step's result is the same bits)
    constexpr int kZCap = 1024;  // steps past this many fetch P as usual
    __shared__ uint8_t pzs[kZCap];
    bool live = nsteps > kZCap;  // some step's P is not known to be zero
    for (int i = tid; i < min(nsteps, kZCap); i += 512) {
        pzs[i] = sv.pz_all(seg_of(i), h, H);
        live |= !pzs[i];
    }
    // A chain of zero transitions only: entering(s + 1) = H_s throughout (reversed: dleave(s - 1) = Hb_s), and
    // the output pass (the reverse replay) reads those states where the local pass left them
    // (SegmentView::entering, and the reverse replay's own choice), so only the first state's copy (written
    // above) is needed.
    if (!__syncthreads_or(live)) return;
    struct Stage {
        u4v pa[2][4];  // P operands, [plane][block]
        f32x4 hb;      // H addends
    };
    // unconditional (past the last step it repeats that step's segment), so
    // that every path through the loop has the same memory operations
    auto fetch = [&](int i, Stage &st) {
        const int ic = min(i, nsteps - 1), seg = seg_of(ic);
        const char *src = REV ? pt + (static_cast<int64_t>(seg) * H + h) * DK * DK * 4
                              : reinterpret_cast<const char *>(sv.P + (static_cast<int64_t>(seg) * H + h) * DK * DK);
        const float *hs = (REV ? hb : sv.Hs) + (static_cast<int64_t>(seg) * H + h) * DK * DV;
        const int r = 16 * wave + m;
        const bool pzero = ic < kZCap && __builtin_amdgcn_readfirstlane(pzs[ic]);
        const mc::rsrc_t rp = mc::make_rsrc(src, pzero ? 0u : 4u * DK * DK);
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                st.pa[pl][t] = __builtin_amdgcn_raw_buffer_load_b128(rp, pl * 2 * DK * DK + 2 * (r * DK + 32 * t + 8 * g),
                                                                      0, 0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) st.hb[jj] = hs[(16 * wave + 4 * g + jj) * DV + j0 + m];
    };
    auto step = [&](int i, int b, const Stage &st) {
        const int seg = seg_of(i);
        __syncthreads();  // entering(seg) complete in sS[b]; sS[b ^ 1] no longer read
        f32x4 acc = st.hb;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int o = m * kSP + 32 * t + 8 * g;
            const bf8 sh = __builtin_bit_cast(bf8, *reinterpret_cast<const u4v *>(&sS[b][0][o]));
            const bf8 sl = __builtin_bit_cast(bf8, *reinterpret_cast<const u4v *>(&sS[b][1][o]));
            const bf8 ph = __builtin_bit_cast(bf8, st.pa[0][t]), pl = __builtin_bit_cast(bf8, st.pa[1][t]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, sh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, sl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, sh, acc, 0, 0, 0);
        }
        float *sin = REV ? dl + (static_cast<int64_t>(seg - 1) * H + h) * DK * DV
                         : sv.sin + (static_cast<int64_t>(seg + 1) * H + h) * DK * DV;
        const int r0 = 16 * wave + 4 * g;
        unsigned hw[2], lw[2];
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
            const __bf16 a0 = static_cast<__bf16>(acc[2 * p2]), a1 = static_cast<__bf16>(acc[2 * p2 + 1]);
            const __bf16 l0 = static_cast<__bf16>(acc[2 * p2] - static_cast<float>(a0));
            const __bf16 l1 = static_cast<__bf16>(acc[2 * p2 + 1] - static_cast<float>(a1));
            hw[p2] = __builtin_bit_cast(uint16_t, a0) | (static_cast<unsigned>(__builtin_bit_cast(uint16_t, a1)) << 16);
            lw[p2] = __builtin_bit_cast(uint16_t, l0) | (static_cast<unsigned>(__builtin_bit_cast(uint16_t, l1)) << 16);
        }
        *reinterpret_cast<uint2 *>(&sS[b ^ 1][0][m * kSP + r0]) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2 *>(&sS[b ^ 1][1][m * kSP + r0]) = make_uint2(lw[0], lw[1]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sin[(r0 + jj) * DV + j0 + m] = acc[jj];
    };
    // the ring: step j uses stage j mod 4, refilled for step j + 4 right after
    Stage s0, s1, s2, s3;
    fetch(0, s0);
    fetch(1, s1);
    fetch(2, s2);
    fetch(3, s3);
    int i = 0;
    for (; i + 4 <= nsteps; i += 4) {
        step(i, 0, s0);
        fetch(i + 4, s0);
        step(i + 1, 1, s1);
        fetch(i + 5, s1);
        step(i + 2, 0, s2);
        fetch(i + 6, s2);
        step(i + 3, 1, s3);
        fetch(i + 7, s3);
    }
    if (i < nsteps) step(i, 0, s0);
    if (i + 1 < nsteps) step(i + 1, 1, s1);
    if (i + 2 < nsteps) step(i + 2, 0, s2);
}

}  // namespace

size_t chunk_workspace_bytes(int B, int T, int H, int dk, int dv, int N, int chunk, bool varlen, bool in_bf16) {
    return make_plan(B, T, H, dk, dv, N, chunk, varlen, in_bf16).bytes;
}

bool chunk_grids_fit(int B, int T, int H, int dk, int dv, int N, int chunk, bool varlen, bool in_bf16) {
    const Plan p = make_plan(B, T, H, dk, dv, N, chunk, varlen, in_bf16);
    // a dispatch's grid size is a 32-bit count of threads per dimension; the largest 1-D grids are the
    // prep's (chunk slots x heads workgroups of 256) and the fp32 local pass's (slices x segments of 256)
    const uint64_t prep = static_cast<uint64_t>(p.max_segs) * p.per * H * 256;
    const uint64_t fp32 = static_cast<uint64_t>(p.max_segs) * ((dv + dk) / 32) * 256;
    return prep < (uint64_t{1} << 32) && fp32 < (uint64_t{1} << 32);
}

// The segment table of a packed batch; a fixed-length batch's segments are computed where they are needed
// (SegmentView::desc), which saves a launch.
void launch_table(const ChunkLaunch &L, const Plan &p, char *ws, SegmentView &sv) {
    if (L.cu_seqlens) {
        hipLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(256), 0, L.stream, L.cu_seqlens, L.T, L.N, p.seg_len,
                           reinterpret_cast<int4 *>(ws + p.off_table), reinterpret_cast<int32_t *>(ws + p.off_seq));
    } else {
        sv.fixed_T = L.T;
        sv.seg_len = p.seg_len;
    }
}

hipError_t launch_chunk(const ChunkLaunch &L) {
    const bool varlen = L.cu_seqlens != nullptr;
    const Plan p = make_plan(L.B, L.T, L.H, L.dk, L.dv, L.N, L.chunk, varlen, L.in_bf16);
    char *ws = static_cast<char *>(L.workspace);
    SegmentView sv;
    sv.table = reinterpret_cast<const int4 *>(ws + p.off_table);
    sv.seq_seg = reinterpret_cast<const int32_t *>(ws + p.off_seq);
    sv.N = L.N;
    sv.P = reinterpret_cast<float *>(ws + p.off_P);
    sv.Hs = reinterpret_cast<float *>(ws + p.off_H);
    sv.sin = reinterpret_cast<float *>(ws + p.off_S);
    sv.h0 = L.h0;
    sv.pz = p.packs ? reinterpret_cast<uint8_t *>(ws + p.off_pz) : nullptr;
    launch_table(L, p, ws, sv);
    void *packs = ws + p.off_pack;
    // fixed-length sequences no longer than a segment are one segment each: the local pass and the
    // combine would only return (their launches alone cost tens of microseconds on many short sequences)
    const bool chained = varlen || L.T == 0 || L.T > p.seg_len;
    if (p.packs) {
        launch_prep(L, sv, p.max_segs, p.per, packs);
        if (chained) launch_scan<kLocal>(L, sv, p.max_segs, p.per, packs);
    } else if (chained) {
        launch_fp32_pass<kLocal>(L, sv, p.max_segs);
    }
    if (chained) {
        if (p.packs)  // P in bf16 planes; one workgroup per (head, 16-column slice, sequence), heads fastest
            hipLaunchKernelGGL(combine_bf16x3_kernel<false>, dim3(L.H, L.dv / 16, L.N), dim3(512), 0, L.stream, sv,
                               L.h0, L.hT, L.H, static_cast<const char *>(nullptr), static_cast<const float *>(nullptr),
                               static_cast<float *>(nullptr));
        else if (L.dk == 128)  // heads fastest: a head's slices share one XCD (workgroups go round-robin over XCDs)
            hipLaunchKernelGGL(combine_mfma_kernel, dim3(L.H, L.dv / 16, L.N), dim3(256), 0, L.stream, sv, L.h0,
                               L.hT, L.H, L.dv);
        else
            hipLaunchKernelGGL(combine_kernel<64>, dim3(L.dv / 16, L.H, L.N), dim3(256), 0, L.stream, sv, L.h0,
                               L.hT, L.H, L.dv);
    }
    if (p.packs) launch_scan<kOut>(L, sv, p.max_segs, p.per, packs);
    else launch_fp32_pass<kOut>(L, sv, p.max_segs);
    return hipGetLastError();
}

ChunkGradLayout chunk_grad_layout(int B, int T, int H, int N, bool varlen) {
    const Plan p = make_plan(B, T, H, 128, 128, N, 64, varlen, true);
    return ChunkGradLayout{p.bytes, p.per, p.max_segs, p.packs};
}

SegmentView launch_chunk_grad_forward(const ChunkLaunch &L, const ScanGrad &gr, void *rpacks, bool *chained,
                                      void **packs) {
    const bool varlen = L.cu_seqlens != nullptr;
    const Plan p = make_plan(L.B, L.T, L.H, L.dk, L.dv, L.N, L.chunk, varlen, L.in_bf16);
    char *ws = static_cast<char *>(L.workspace);
    SegmentView sv;
    sv.table = reinterpret_cast<const int4 *>(ws + p.off_table);
    sv.seq_seg = reinterpret_cast<const int32_t *>(ws + p.off_seq);
    sv.N = L.N;
    sv.P = reinterpret_cast<float *>(ws + p.off_P);
    sv.Hs = reinterpret_cast<float *>(ws + p.off_H);
    sv.sin = reinterpret_cast<float *>(ws + p.off_S);
    sv.h0 = L.h0;
    sv.pz = p.packs ? reinterpret_cast<uint8_t *>(ws + p.off_pz) : nullptr;
    launch_table(L, p, ws, sv);
    *packs = ws + p.off_pack;
    *chained = varlen || L.T == 0 || L.T > p.seg_len;
    launch_prep(L, sv, p.max_segs, p.per, *packs, rpacks);
    if (*chained) {
        launch_scan_grad<kLocal>(L, sv, p.max_segs, p.per, *packs, gr);
        hipLaunchKernelGGL(combine_bf16x3_kernel<false>, dim3(L.H, L.dv / 16, L.N), dim3(512), 0, L.stream, sv,
                           L.h0, static_cast<float *>(nullptr), L.H, static_cast<const char *>(nullptr),
                           static_cast<const float *>(nullptr), static_cast<float *>(nullptr));
    }
    launch_scan_grad<kStates>(L, sv, p.max_segs, p.per, *packs, gr);
    return sv;
}

void launch_reverse_combine_bf16(const SegmentView &sv, const char *pt, const float *hb, const float *dhT, float *dl,
                                 float *dh0, int H, int N, hipStream_t stream) {
    hipLaunchKernelGGL(combine_bf16x3_kernel<true>, dim3(H, 128 / 16, N), dim3(512), 0, stream, sv, dhT, dh0, H, pt, hb,
                       dl);
}

size_t segment_states_bytes(int B, int T, int H, int dk, int dv, int N, bool varlen, int chunk) {
    return make_plan(B, T, H, dk, dv, N, chunk, varlen, false).bytes;
}

SegmentStates launch_segment_table(const ChunkLaunch &L) {
    const bool varlen = L.cu_seqlens != nullptr;
    const Plan p = make_plan(L.B, L.T, L.H, L.dk, L.dv, L.N, L.chunk, varlen, false);
    char *ws = static_cast<char *>(L.workspace);
    SegmentStates r{};
    SegmentView &sv = r.sv;
    sv.table = reinterpret_cast<const int4 *>(ws + p.off_table);
    sv.seq_seg = reinterpret_cast<const int32_t *>(ws + p.off_seq);
    sv.N = L.N;
    sv.P = reinterpret_cast<float *>(ws + p.off_P);
    sv.Hs = reinterpret_cast<float *>(ws + p.off_H);
    sv.sin = reinterpret_cast<float *>(ws + p.off_S);
    sv.h0 = L.h0;
    r.max_segs = p.max_segs;
    r.seg_len = p.seg_len;
    hipLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(256), 0, L.stream, L.cu_seqlens, L.T, L.N,
                       p.seg_len, reinterpret_cast<int4 *>(ws + p.off_table),
                       reinterpret_cast<int32_t *>(ws + p.off_seq));
    return r;
}

void launch_segment_combine(const ChunkLaunch &L, const SegmentStates &s) {
    if (L.dk == 128)
        hipLaunchKernelGGL(combine_mfma_kernel, dim3(L.H, L.dv / 16, L.N), dim3(256), 0, L.stream, s.sv, L.h0,
                           L.hT, L.H, L.dv);
    else
        hipLaunchKernelGGL(combine_kernel<64>, dim3(L.dv / 16, L.H, L.N), dim3(256), 0, L.stream, s.sv, L.h0,
                           L.hT, L.H, L.dv);
}

}  // namespace kda
