// kda_dplr_chunk.hip - chunkwise-parallel form of the general diagonal-plus-low-rank (DPLR) recurrence
// for gfx950, on fp32 matrix cores, in the harness of the fp32 KDA chunk kernel (kda_chunk.hip): the
// same work split, segment table, local/output passes and combine.
//
// The recurrence (KDA's transition is the member a = beta k, b = alpha .* k with write key beta k:
// Kimi Linear review notes, section "Chunkwise Algorithm"):
//
//     x_t = S_{t-1}^T b_t,   S_t = Diag(alpha_t) S_{t-1} - a_t x_t^T + k_t v_t^T,   o_t = scale S_t^T q_t.
//
// Inside a chunk with rows r = 0..L-1, entering state S, G_r the inclusive chunk-local cumulative log
// decay and G_{-1} = 0 (derived from the recurrence by induction; the jxzklqfsx.com article's efficiency
// section counts four secondary-chunk products for the general form against KDA's two, and three more
// matrix products):
//
//   B_k[r,i] = sum_c b_r k_i exp(G_{r-1} - G_i),  B_a[r,i] = sum_c b_r a_i exp(G_{r-1} - G_i),  i <  r
//   A_qk[r,i]= sum_c q_r k_i exp(G_r - G_i),      A_qa[r,i]= sum_c q_r a_i exp(G_r - G_i),      i <= r
//   T        = (I + B_a)^{-1}                                  (UT transform, forward substitution)
//   X        = T ((b e^{G_{r-1}}) S + B_k V)                   (the low-rank reads x_r of the chunk)
//   O        = scale ((q e^G) S + A_qk V - A_qa X)
//   S       <- e^{G_L} * S + (e^{G_L - G} k)^T V - (e^{G_L - G} a)^T X
//
// Per chunk and 32-column slice that is eight products (KDA's kernel: five) after four Gram blocks
// (KDA's: two).  The Gram blocks use the KDA kernel's factoring per 16-row block a, reference row
// ref = 16a - 1: row factors exp(G_r - G_ref) and exp(G_{r-1} - G_ref) are <= 1, column factors
// exp(G_ref - G_i) are <= 1 left of the block and at most exp(range of 16 rows) inside it; a diagonal
// block whose range exceeds 80 in some channel is recomputed pair by pair.
//
// Five [C][dk] fp32 operands (G, k, q, a, b) must sit in LDS beside four C x C blocks and the state
// slice, which at dk = 128 fits 160 KiB for C = 32 (C = 64 would need 265 KiB): the kernel runs C = 32.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr float kMaxBlockDecay = 80.0f;

template <int DK, int C, int BV, bool InBf16, bool OutBf16, int MODE>
__global__ void __launch_bounds__(256, 1)
dplr_chunk_kernel(DplrChunkLaunch Lp, SegmentView sv) {
    using In = Elem<InBf16>;
    using Out = Elem<OutBf16>;
    using IT = typename In::T;
    const IT *q = static_cast<const IT *>(Lp.q), *k = static_cast<const IT *>(Lp.k);
    const IT *v = static_cast<const IT *>(Lp.v), *av = static_cast<const IT *>(Lp.a);
    const IT *bv = static_cast<const IT *>(Lp.b);
    const float *g = Lp.g;
    typename Out::T *o = static_cast<typename Out::T *>(Lp.o);
    const int H = Lp.H, DV = Lp.dv;
    const float scale = Lp.scale;

    constexpr int NB = C / 16;        // 16-row blocks per chunk
    constexpr int DKP = DK + 1;       // padded row strides (bank spread)
    constexpr int CP = C + 1;
    constexpr int BVP = BV + 1;
    constexpr int NCT = BV / 16;      // 16-column tiles in the slice
    static_assert(C % 16 == 0 && NB <= 4 && BV % 16 == 0 && DK % 16 == 0, "tiling");

    __shared__ float sG[C * DKP];     // G (cumulative log decay)
    __shared__ float sK[C * DKP];
    __shared__ float sQ[C * DKP];
    __shared__ float sA[C * DKP];     // a
    __shared__ float sB[C * DKP];     // b
    __shared__ float sT[C * CP];      // B_a (strictly lower), then T in place
    __shared__ float sBk[C * CP];     // B_k (strictly lower)
    __shared__ float sAq[C * CP];     // A_qk (lower incl. diagonal)
    __shared__ float sAa[C * CP];     // A_qa (lower incl. diagonal)
    __shared__ float sS[DK * BVP];    // state slice, [dk][dv]
    __shared__ float sV[C * BVP];     // v slice of the chunk (zero for P columns)
    __shared__ float sX[C * BVP];     // B^ S + B_k V, then X
    __shared__ int sRange[NB];        // float bits of each block's largest decay

    // grid.x = segment * slices + slice, grid.y = head
    const int slices = MODE == kOut ? DV / BV : (DV + DK) / BV;
    const int slice = static_cast<int>(blockIdx.x % slices), seg = static_cast<int>(blockIdx.x / slices);
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    if (seg >= sv.count()) return;
    const int4 sd = sv.desc(seg);
    const int n = sd.x;
    const bool last = sd.w & kSegLast;
    if (MODE == kLocal && last) return;
    const int64_t t0 = sd.y, t1 = sd.z;
    // kLocal: slices [0, DV/BV) are columns of H (zero start), the rest columns of P (identity start, v = 0)
    const bool pcols = MODE == kLocal && slice >= DV / BV;
    const int j0 = (pcols ? slice - DV / BV : slice) * BV;
    const int ld = pcols ? DK : DV;

    if (MODE == kOut) {
        const float *src = sv.entering(seg, sd, h, H, DK, DV);
        for (int e = tid; e < DK * BV; e += 256) {
            const int i = e / BV, j = e % BV;
            sS[i * BVP + j] = src ? src[static_cast<int64_t>(i) * DV + j0 + j] : 0.f;
        }
    } else {
        for (int e = tid; e < DK * BV; e += 256) {
            const int i = e / BV, j = e % BV;
            sS[i * BVP + j] = (pcols && i == j0 + j) ? 1.f : 0.f;
        }
    }

    for (int64_t c0 = t0; c0 < t1; c0 += C) {
        const int L = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);
        // ---- load the chunk; chunk-local cumulative log decay
        if (tid < NB) sRange[tid] = 0;
        for (int e = tid; e < C * DK; e += 256) {
            const int r = e / DK, c = e % DK;
            const int64_t gi = ((c0 + r) * H + h) * DK + c;
            const bool ok = r < L;
            sK[r * DKP + c] = ok ? In::load(k, gi) : 0.f;
            sQ[r * DKP + c] = ok ? In::load(q, gi) : 0.f;
            sA[r * DKP + c] = ok ? In::load(av, gi) : 0.f;
            sB[r * DKP + c] = ok ? In::load(bv, gi) : 0.f;
        }
        for (int e = tid; e < C * BV; e += 256) {
            const int r = e / BV, j = e % BV;
            sV[r * BVP + j] = (r < L && !pcols) ? In::load(v, ((c0 + r) * H + h) * static_cast<int64_t>(DV) + j0 + j)
                                                : 0.f;
        }
        {   // per channel, 256/DK threads each scan C*DK/256 consecutive rows
            constexpr int PARTS = 256 / DK, RP = C / PARTS;
            const int c = tid % DK, part = tid / DK;
            float gv[RP];
#pragma unroll
            for (int m = 0; m < RP; ++m) {
                const int r = part * RP + m;
                gv[m] = r < L ? g[((c0 + r) * H + h) * DK + c] : 0.f;
            }
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < RP; ++m) {
                acc += gv[m];
                sG[(part * RP + m) * DKP + c] = acc;
            }
            __syncthreads();
            float off = 0.f;
            for (int pp = 0; pp < part; ++pp) off += sG[((pp + 1) * RP - 1) * DKP + c];
            __syncthreads();
            if (part > 0) {
#pragma unroll
                for (int m = 0; m < RP; ++m) sG[(part * RP + m) * DKP + c] += off;
            }
        }
        __syncthreads();
        for (int c = tid; c < DK; c += 256) {
#pragma unroll
            for (int a = 0; a < NB; ++a) {
                const float gref = a ? sG[(16 * a - 1) * DKP + c] : 0.f;
                const float rng = gref - sG[(16 * a + 15) * DKP + c];
                atomicMax(&sRange[a], __float_as_int(fmaxf(rng, 0.f)));
            }
        }
        __syncthreads();

        // ---- the four decayed Gram blocks, one (row block, column block) tile pair per step
        for (int p = wave; p < NB * (NB + 1) / 2; p += 4) {
            int a = 0, rem = p;
            while (rem > a) { rem -= a + 1; ++a; }
            const int b = rem;  // b <= a
            const int r = 16 * a + lr, i = 16 * b + lr;
            f32x4 aqk = {0.f, 0.f, 0.f, 0.f}, aqa = aqk, bk = aqk, ba = aqk;
            for (int s = 0; s < DK / 4; ++s) {
                const int c = 4 * s + lk;
                const float gref = a ? sG[(16 * a - 1) * DKP + c] : 0.f;
                const float gprev = r ? sG[(r - 1) * DKP + c] : 0.f;
                const float xq = __expf(sG[r * DKP + c] - gref), xb = __expf(gprev - gref);
                const float cf = __expf(fminf(gref - sG[i * DKP + c], kMaxBlockDecay));
                const float qr = sQ[r * DKP + c] * xq, br = sB[r * DKP + c] * xb;
                const float kc = sK[i * DKP + c] * cf, ac = sA[i * DKP + c] * cf;
                aqk = mfma4(qr, kc, aqk);
                aqa = mfma4(qr, ac, aqa);
                bk = mfma4(br, kc, bk);
                ba = mfma4(br, ac, ba);
            }
            const bool exact = (a == b) && __int_as_float(sRange[a]) > kMaxBlockDecay;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 16 * a + 4 * lk + jj, ii = 16 * b + lr;
                float vqk = aqk[jj], vqa = aqa[jj], vbk = bk[jj], vba = ba[jj];
                if (exact) {  // pair-by-pair decay for a block that decays too fast
                    vqk = vqa = vbk = vba = 0.f;
                    for (int c = 0; c < DK; ++c) {
                        const float gp = rr ? sG[(rr - 1) * DKP + c] : 0.f;
                        const float dq = __expf(sG[rr * DKP + c] - sG[ii * DKP + c]);
                        const float db = __expf(fminf(gp - sG[ii * DKP + c], 0.f));
                        vqk += sQ[rr * DKP + c] * sK[ii * DKP + c] * dq;
                        vqa += sQ[rr * DKP + c] * sA[ii * DKP + c] * dq;
                        vbk += sB[rr * DKP + c] * sK[ii * DKP + c] * db;
                        vba += sB[rr * DKP + c] * sA[ii * DKP + c] * db;
                    }
                }
                sAq[rr * CP + ii] = ii <= rr ? vqk : 0.f;
                sAa[rr * CP + ii] = ii <= rr ? vqa : 0.f;
                sBk[rr * CP + ii] = ii < rr ? vbk : 0.f;
                sT[rr * CP + ii] = ii < rr ? vba : 0.f;
            }
        }
        for (int e = tid; e < C * C; e += 256) {  // upper tiles are zero
            const int r = e / C, i = e % C;
            if ((i >> 4) > (r >> 4)) {
                sAq[r * CP + i] = 0.f;
                sAa[r * CP + i] = 0.f;
                sBk[r * CP + i] = 0.f;
                sT[r * CP + i] = 0.f;
            }
        }
        __syncthreads();

        // ---- T = (I + B_a)^{-1} by forward substitution, in place, one column per lane of wave 0 (row r
        // reads B_a[r][i], i < r, and rows of T above it; entries above T's diagonal are 0)
        if (tid < C) {
            const int jcol = tid;
            for (int r = 0; r < C; ++r) {
                float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
                int i = 0;
                for (; i + 4 <= r; i += 4) {
                    a0 += sT[r * CP + i] * sT[i * CP + jcol];
                    a1 += sT[r * CP + i + 1] * sT[(i + 1) * CP + jcol];
                    a2 += sT[r * CP + i + 2] * sT[(i + 2) * CP + jcol];
                    a3 += sT[r * CP + i + 3] * sT[(i + 3) * CP + jcol];
                }
                for (; i < r; ++i) a0 += sT[r * CP + i] * sT[i * CP + jcol];
                sT[r * CP + jcol] = ((r == jcol) ? 1.f : 0.f) - ((a0 + a1) + (a2 + a3));
            }
        }
        // ---- R = (b e^{G_{r-1}}) S + B_k V and Y = (q e^G) S; wave = row block
        f32x4 accR[NCT], accY[NCT];
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            accR[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            accY[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const bool rowblk = wave < NB;
        if (rowblk) {
            const int r = 16 * wave + lr;
            for (int s = 0; s < DK / 4; ++s) {
                const int c = 4 * s + lk;
                const float gp = r ? sG[(r - 1) * DKP + c] : 0.f;
                const float ab = sB[r * DKP + c] * __expf(gp), aq = sQ[r * DKP + c] * __expf(sG[r * DKP + c]);
#pragma unroll
                for (int t = 0; t < NCT; ++t) {
                    const float bs = sS[c * BVP + 16 * t + lr];
                    accR[t] = mfma4(ab, bs, accR[t]);
                    accY[t] = mfma4(aq, bs, accY[t]);
                }
            }
            if (!pcols) {  // + B_k V (strictly lower: column blocks up to this row block)
                for (int s = 0; s < 4 * (wave + 1); ++s) {
                    const int i = 4 * s + lk;
                    const float bki = sBk[r * CP + i];
#pragma unroll
                    for (int t = 0; t < NCT; ++t) accR[t] = mfma4(bki, sV[i * BVP + 16 * t + lr], accR[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sX[(16 * wave + 4 * lk + jj) * BVP + 16 * t + lr] = accR[t][jj];
        }
        __syncthreads();

        // ---- X = T R (T unit lower triangular)
        f32x4 accX[NCT];
#pragma unroll
        for (int t = 0; t < NCT; ++t) accX[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (rowblk) {
            const int r = 16 * wave + lr;
            for (int s = 0; s < 4 * (wave + 1); ++s) {
                const int i = 4 * s + lk;
                const float at = sT[r * CP + i];
#pragma unroll
                for (int t = 0; t < NCT; ++t) accX[t] = mfma4(at, sX[i * BVP + 16 * t + lr], accX[t]);
            }
        }
        __syncthreads();
        if (rowblk) {
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sX[(16 * wave + 4 * lk + jj) * BVP + 16 * t + lr] = accX[t][jj];
        }
        __syncthreads();

        // ---- O = scale (Y + A_qk V - A_qa X)
        if (MODE == kOut && rowblk) {
            const int r = 16 * wave + lr;
            for (int s = 0; s < 4 * (wave + 1); ++s) {
                const int i = 4 * s + lk;
                const float aq = sAq[r * CP + i], aa = -sAa[r * CP + i];
#pragma unroll
                for (int t = 0; t < NCT; ++t) {
                    accY[t] = mfma4(aq, sV[i * BVP + 16 * t + lr], accY[t]);
                    accY[t] = mfma4(aa, sX[i * BVP + 16 * t + lr], accY[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rr = 16 * wave + 4 * lk + jj;
                    if (rr < L)
                        Out::store(o, ((c0 + rr) * H + h) * static_cast<int64_t>(DV) + j0 + 16 * t + lr,
                                   scale * accY[t][jj]);
                }
        }

        // ---- S <- e^{G_L} S + (e^{G_L - G} k)^T V - (e^{G_L - G} a)^T X ; 16-row dk tiles over waves
        for (int rt = wave; rt < DK / 16; rt += 4) {
            const int ic = 16 * rt + lr;  // dk index of this lane's A-operand row
            const float gl = sG[(C - 1) * DKP + ic];
            f32x4 acc[NCT];
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int ir = 16 * rt + 4 * lk + jj;
                    acc[t][jj] = __expf(sG[(C - 1) * DKP + ir]) * sS[ir * BVP + 16 * t + lr];
                }
            for (int s = 0; s < C / 4; ++s) {
                const int rr = 4 * s + lk;
                const float d = __expf(gl - sG[rr * DKP + ic]);
                const float kk = sK[rr * DKP + ic] * d, aa = -sA[rr * DKP + ic] * d;
#pragma unroll
                for (int t = 0; t < NCT; ++t) {
                    if (!pcols) acc[t] = mfma4(kk, sV[rr * BVP + 16 * t + lr], acc[t]);
                    acc[t] = mfma4(aa, sX[rr * BVP + 16 * t + lr], acc[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sS[(16 * rt + 4 * lk + jj) * BVP + 16 * t + lr] = acc[t][jj];
        }
        __syncthreads();
    }

    float *dst = nullptr;
    if (MODE == kOut) {
        if (last && Lp.hT) dst = Lp.hT + (static_cast<int64_t>(n) * H + h) * DK * DV;
    } else {
        dst = (pcols ? sv.P : sv.Hs) + (static_cast<int64_t>(seg) * H + h) * DK * ld;
    }
    if (dst) {
        for (int e = tid; e < DK * BV; e += 256) {
            const int i = e / BV, j = e % BV;
            dst[static_cast<int64_t>(i) * ld + j0 + j] = sS[i * BVP + j];
        }
    }
}

constexpr int kDplrChunk = 32;
constexpr int kDplrBV = 32;

template <int DK, int MODE>
void launch_pass(const DplrChunkLaunch &L, const SegmentView &sv, int max_segs) {
    const int slices = MODE == kOut ? L.dv / kDplrBV : (L.dv + DK) / kDplrBV;
    const dim3 grid(static_cast<unsigned>(slices * max_segs), L.H), block(256);
#define KDA_DPLR(IB, OB) \
    hipLaunchKernelGGL((dplr_chunk_kernel<DK, kDplrChunk, kDplrBV, IB, OB, MODE>), grid, block, 0, L.stream, L, sv)
    if (L.in_bf16 && L.out_bf16) KDA_DPLR(true, true);
    else if (L.in_bf16) KDA_DPLR(true, false);
    else if (L.out_bf16) KDA_DPLR(false, true);
    else KDA_DPLR(false, false);
#undef KDA_DPLR
}

// The ChunkLaunch the segment machinery takes: sizes, states and stream of the DPLR call.
ChunkLaunch segment_launch(const DplrChunkLaunch &L) {
    ChunkLaunch c{};
    c.h0 = L.h0;
    c.hT = L.hT;
    c.cu_seqlens = L.cu_seqlens;
    c.B = L.B; c.T = L.T; c.H = L.H; c.dk = L.dk; c.dv = L.dv; c.N = L.N;
    c.chunk = kDplrChunk;
    c.scale = L.scale;
    c.in_bf16 = L.in_bf16;
    c.workspace = L.workspace;
    c.stream = L.stream;
    return c;
}

}  // namespace

int dplr_chunk_size() { return kDplrChunk; }

size_t dplr_chunk_workspace_bytes(int B, int T, int H, int dk, int dv, int N, bool varlen) {
    return segment_states_bytes(B, T, H, dk, dv, N, varlen, kDplrChunk);
}

hipError_t launch_dplr_chunk(const DplrChunkLaunch &L) {
    const ChunkLaunch c = segment_launch(L);
    const SegmentStates ss = launch_segment_table(c);
    // fixed-length sequences no longer than a segment are one segment each: no local pass, no combine
    const bool chained = L.cu_seqlens != nullptr || L.T == 0 || L.T > ss.seg_len;
    if (chained) {
        if (L.dk == 128) launch_pass<128, kLocal>(L, ss.sv, ss.max_segs);
        else launch_pass<64, kLocal>(L, ss.sv, ss.max_segs);
        launch_segment_combine(c, ss);
    }
    if (L.dk == 128) launch_pass<128, kOut>(L, ss.sv, ss.max_segs);
    else launch_pass<64, kOut>(L, ss.sv, ss.max_segs);
    return hipGetLastError();
}

}  // namespace kda
