// kda_chunk.hip - chunkwise-parallel KDA prefill for gfx950, fp32 matrix cores.
//
// The sequence is cut into chunks of C tokens (Kimi Linear review notes,
// section "Chunkwise Algorithm", C = 64); only the fp32 state S crosses chunk
// boundaries.  Inside a chunk with rows r = 0..L-1 and entering state S
// (jxzklqfsx.com article, hardware-efficient chunkwise algorithm: WY
// representation, UT transform by row-wise forward substitution, inter-chunk
// recurrence with intra-chunk parallel output; the chunk equations below are
// derived from the recurrence and pinned against it by chunk-size invariance):
//
//   G_r      = g_0 + ... + g_r                  chunk-local log decay (a1);
//                                               gamma^{i->r} = exp(G_r - G_i)
//   A_kk[r,i]= beta_r sum_c k_r k_i exp(G_r-G_i), i <  r   (a2, decayed K K^T)
//   A_qk[r,i]= scale  sum_c q_r k_i exp(G_r-G_i), i <= r   (a2, decayed Q K^T)
//   T        = (I + A_kk)^{-1}                   UT transform (a3)
//   V_new    = T (beta * (V - (e^G * K) S))      = U - W S with the WY factors
//                                               U = T beta V, W = T beta e^G K (a4, a5)
//   O        = scale (e^G * Q) S + A_qk V_new    inter + intra output (a6)
//   S       <- e^{G_L} * S + (e^{G_L - G} * K)^T V_new       (a5)
//
// The two decayed Gram blocks are formed per 16-row block a with reference
// row ref = 16a - 1 (G_{-1} = 0): row factors exp(G_r - G_ref) <= 1 and
// column factors exp(G_ref - G_i), which are <= 1 left of the block and at
// most exp(range of 16 rows) inside it.  If some 16-row block decays by more
// than exp(-80) in a channel, its diagonal block is recomputed pair by pair
// (exp(G_r - G_i) directly), so no factor ever overflows fp32.
//
// Work split: one workgroup (4 waves) per (segment, head, 32-column slice),
// walking the segment's chunks in order.  All products run on
// v_mfma_f32_16x16x4f32 with fp32 operands staged in LDS.  This is the
// exact-fp32 path (fp32 inputs).  The same kernel serves the two parallel
// passes of the segmented prefill (see kda_segments.hip): kLocal computes a
// segment's local state H (zero start) and its transition P (identity start,
// v = 0); kOut replays the segment from its true entering state and writes o.
// The optional input transforms act as the chunk is loaded: the gate logit
// becomes the log-gate before the cumulative sum, and the k and q rows are
// L2-normalised in LDS before any product reads them.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr float kMaxBlockDecay = 80.0f;  // exp(80) is far below FLT_MAX

// Divide each of the C rows of k and q in LDS (row stride DKP) by its L2 norm
// over the DK channels (plus kL2Eps); 256 / C consecutive threads share a row.
template <int C, int DK, int DKP>
__device__ __forceinline__ void l2norm_rows(float *sK, float *sQ, int tid) {
    constexpr int TPR = 256 / C, CPT = DK / TPR;
    static_assert(kWave % TPR == 0 && DK % TPR == 0, "a row's threads sit in one wave");
    const int r = tid / TPR, part = tid % TPR;
    float kk = 0.f, qq = 0.f;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
        const float a = sK[r * DKP + part + TPR * m], b = sQ[r * DKP + part + TPR * m];
        kk += a * a;
        qq += b * b;
    }
#pragma unroll
    for (int msk = 1; msk < TPR; msk <<= 1) {
        kk += __shfl_xor(kk, msk, kWave);
        qq += __shfl_xor(qq, msk, kWave);
    }
    const float ik = rsqrtf(kk + kL2Eps), iq = rsqrtf(qq + kL2Eps);
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
        sK[r * DKP + part + TPR * m] *= ik;
        sQ[r * DKP + part + TPR * m] *= iq;
    }
}

template <int DK, int C, int BV, bool InBf16, bool OutBf16, int MODE>
__global__ void __launch_bounds__(256, 1)
chunk_fp32_kernel(const void *__restrict__ q_, const void *__restrict__ k_,
                  const void *__restrict__ v_, const float *__restrict__ g,
                  const void *__restrict__ beta_, float *hT, void *__restrict__ o_,
                  SegmentView sv, int H, int DV, float scale, InputXform ix) {
    using In = Elem<InBf16>;
    using Out = Elem<OutBf16>;
    const typename In::T *q = static_cast<const typename In::T *>(q_);
    const typename In::T *k = static_cast<const typename In::T *>(k_);
    const typename In::T *v = static_cast<const typename In::T *>(v_);
    const typename In::T *beta = static_cast<const typename In::T *>(beta_);
    typename Out::T *o = static_cast<typename Out::T *>(o_);

    constexpr int NB = C / 16;        // 16-row blocks per chunk
    constexpr int DKP = DK + 1;       // padded row strides (bank spread)
    constexpr int CP = C + 1;
    constexpr int BVP = BV + 1;
    constexpr int NCT = BV / 16;      // 16-column tiles in the slice
    static_assert(C % 16 == 0 && C <= 64 && BV % 16 == 0 && DK % 16 == 0, "tiling");

    __shared__ float sG[C * DKP];     // G (cumulative log decay)
    __shared__ float sK[C * DKP];     // k
    __shared__ float sQ[C * DKP];     // q
    __shared__ float sA[C * CP];      // beta-scaled A_kk (strictly lower), then T in place
    __shared__ float sAq[C * CP];     // scale-scaled A_qk (lower incl. diagonal)
    __shared__ float sS[DK * BVP];    // state slice, [dk][dv]
    __shared__ float sX[C * BVP];     // beta (V - e^G K S), then V_new
    __shared__ float sBeta[C];
    __shared__ int sRange[NB];        // float bits of each block's largest decay

    // grid.x = segment * slices + slice (a packed batch may hold more than grid.y's 65,535 segments),
    // grid.y = head
    const int slices = MODE == kOut ? DV / BV : (DV + DK) / BV;
    const int slice = static_cast<int>(blockIdx.x % slices), seg = static_cast<int>(blockIdx.x / slices);
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;   // MFMA row/col lane, k lane
    if (seg >= sv.count()) return;
    const int4 sd = sv.desc(seg);
    const int n = sd.x;
    const bool last = sd.w & kSegLast;
    if (MODE == kLocal && last) return;         // a last segment's P, H are never used
    const int64_t t0 = sd.y, t1 = sd.z;
    // kLocal: slices [0, DV/BV) are columns of H, the rest columns of P (dk x dk)
    const bool pcols = MODE == kLocal && slice >= DV / BV;
    const int j0 = (pcols ? slice - DV / BV : slice) * BV;
    const int ld = pcols ? DK : DV;             // row stride of the state being built

    // ---- entering state slice -> LDS
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
        // ---- a1: load the chunk, chunk-local cumulative log decay
        if (tid < NB) sRange[tid] = 0;
        for (int e = tid; e < C * DK; e += 256) {
            const int r = e / DK, c = e % DK;
            const int64_t gi = ((c0 + r) * H + h) * DK + c;
            const bool ok = r < L;
            sK[r * DKP + c] = ok ? In::load(k, gi) : 0.f;
            sQ[r * DKP + c] = ok ? In::load(q, gi) : 0.f;
        }
        if (tid < C) sBeta[tid] = tid < L ? In::load(beta, (c0 + tid) * H + h) : 0.f;
        {   // a1: per channel, 256/DK threads each scan C*DK/256 consecutive rows
            constexpr int PARTS = 256 / DK, RP = C / PARTS;
            const int c = tid % DK, part = tid / DK;
            float gv[RP];
#pragma unroll
            for (int m = 0; m < RP; ++m) {
                const int r = part * RP + m;
                const int64_t gi = ix.scalar_gate ? (c0 + r) * H + h : ((c0 + r) * H + h) * DK + c;
                gv[m] = r < L ? ix.log_gate(g[gi]) : 0.f;
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
        // k, q rows normalised; the barrier after the decay ranges orders this before the products
        if (ix.qk_l2norm) l2norm_rows<C, DK, DKP>(sK, sQ, tid);
        for (int c = tid; c < DK; c += 256) {
#pragma unroll
            for (int a = 0; a < NB; ++a) {
                const float gref = a ? sG[(16 * a - 1) * DKP + c] : 0.f;
                const float rng = gref - sG[(16 * a + 15) * DKP + c];
                atomicMax(&sRange[a], __float_as_int(fmaxf(rng, 0.f)));
            }
        }
        __syncthreads();

        // ---- a2: A_kk and A_qk, one (row block, column block) tile pair per step
        for (int p = wave; p < NB * (NB + 1) / 2; p += 4) {
            int a = 0, rem = p;
            while (rem > a) { rem -= a + 1; ++a; }
            const int b = rem;  // b <= a
            const int r = 16 * a + lr, i = 16 * b + lr;
            f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < DK / 4; ++s) {
                const int c = 4 * s + lk;
                const float gref = a ? sG[(16 * a - 1) * DKP + c] : 0.f;
                const float xf = __expf(sG[r * DKP + c] - gref);
                const float kc = sK[i * DKP + c] * __expf(fminf(gref - sG[i * DKP + c], kMaxBlockDecay));
                akk = mfma4(sK[r * DKP + c] * xf, kc, akk);
                aqk = mfma4(sQ[r * DKP + c] * xf, kc, aqk);
            }
            const bool exact = (a == b) && __int_as_float(sRange[a]) > kMaxBlockDecay;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 16 * a + 4 * lk + jj, ii = 16 * b + lr;
                float vk = akk[jj], vq = aqk[jj];
                if (exact) {  // pair-by-pair decay for a block that decays too fast
                    vk = 0.f;
                    vq = 0.f;
                    for (int c = 0; c < DK; ++c) {
                        const float d = __expf(sG[rr * DKP + c] - sG[ii * DKP + c]);
                        vk += sK[rr * DKP + c] * sK[ii * DKP + c] * d;
                        vq += sQ[rr * DKP + c] * sK[ii * DKP + c] * d;
                    }
                }
                sA[rr * CP + ii] = ii < rr ? sBeta[rr] * vk : 0.f;
                sAq[rr * CP + ii] = ii <= rr ? scale * vq : 0.f;
            }
        }
        // upper tiles are zero
        for (int e = tid; e < C * C; e += 256) {
            const int r = e / C, i = e % C;
            if ((i >> 4) > (r >> 4)) {
                sA[r * CP + i] = 0.f;
                sAq[r * CP + i] = 0.f;
            }
        }
        __syncthreads();

        // ---- a3: T = (I + A_kk)^{-1} by forward substitution, in place, one
        // column per lane of wave 0: row r reads A[r][i] (i < r) and rows of T
        // above it; the lanes reconverge before row r is overwritten, so every
        // read of row r sees A and every read of an earlier row sees T.
        // Entries above the diagonal of T are 0, so the sum may run over all
        // i < r; every lane then runs the same loop.
        if (tid < C) {
            const int jcol = tid;
            for (int r = 0; r < C; ++r) {
                float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
                int i = 0;
                for (; i + 4 <= r; i += 4) {
                    a0 += sA[r * CP + i] * sA[i * CP + jcol];
                    a1 += sA[r * CP + i + 1] * sA[(i + 1) * CP + jcol];
                    a2 += sA[r * CP + i + 2] * sA[(i + 2) * CP + jcol];
                    a3 += sA[r * CP + i + 3] * sA[(i + 3) * CP + jcol];
                }
                for (; i < r; ++i) a0 += sA[r * CP + i] * sA[i * CP + jcol];
                sA[r * CP + jcol] = ((r == jcol) ? 1.f : 0.f) - ((a0 + a1) + (a2 + a3));
            }
        }
        // ---- a5 (first half): X = beta (V - (e^G K) S), Y = (e^G Q) S; wave = row block
        f32x4 accX[NCT], accY[NCT];
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            accX[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            accY[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const bool rowblk = wave < NB;
        if (rowblk) {
            const int r = 16 * wave + lr;
            for (int s = 0; s < DK / 4; ++s) {
                const int c = 4 * s + lk;
                const float e = __expf(sG[r * DKP + c]);
                const float ak = sK[r * DKP + c] * e, aq = sQ[r * DKP + c] * e;
#pragma unroll
                for (int t = 0; t < NCT; ++t) {
                    const float bs = sS[c * BVP + 16 * t + lr];
                    accX[t] = mfma4(ak, bs, accX[t]);
                    accY[t] = mfma4(aq, bs, accY[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < NCT; ++t) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rr = 16 * wave + 4 * lk + jj, j = 16 * t + lr;
                    const float vv = (rr < L && !pcols)
                                         ? In::load(v, ((c0 + rr) * H + h) * static_cast<int64_t>(DV) + j0 + j)
                                         : 0.f;
                    sX[rr * BVP + j] = sBeta[rr] * (vv - accX[t][jj]);
                }
            }
        }
        __syncthreads();

        // ---- a4/a5: V_new = T X (T unit lower triangular)
        f32x4 accV[NCT];
#pragma unroll
        for (int t = 0; t < NCT; ++t) accV[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (rowblk) {
            const int r = 16 * wave + lr;
            for (int s = 0; s < 4 * (wave + 1); ++s) {
                const int i = 4 * s + lk;
                const float at = sA[r * CP + i];
#pragma unroll
                for (int t = 0; t < NCT; ++t) accV[t] = mfma4(at, sX[i * BVP + 16 * t + lr], accV[t]);
            }
        }
        __syncthreads();
        if (rowblk) {
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sX[(16 * wave + 4 * lk + jj) * BVP + 16 * t + lr] = accV[t][jj];
        }
        __syncthreads();

        // ---- a6: O = scale Y + A_qk V_new
        if (MODE == kOut && rowblk) {
            const int r = 16 * wave + lr;
#pragma unroll
            for (int t = 0; t < NCT; ++t) accY[t] *= scale;
            for (int s = 0; s < 4 * (wave + 1); ++s) {
                const int i = 4 * s + lk;
                const float aq = sAq[r * CP + i];
#pragma unroll
                for (int t = 0; t < NCT; ++t) accY[t] = mfma4(aq, sX[i * BVP + 16 * t + lr], accY[t]);
            }
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rr = 16 * wave + 4 * lk + jj;
                    if (rr < L) Out::store(o, ((c0 + rr) * H + h) * static_cast<int64_t>(DV) + j0 + 16 * t + lr, accY[t][jj]);
                }
        }

        // ---- a5: S <- e^{G_L} S + (e^{G_L - G} K)^T V_new ; 16-row dk tiles over waves
        for (int rt = wave; rt < DK / 16; rt += 4) {
            const int ic = 16 * rt + lr;  // dk index of this lane's A row
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
                const float ak = sK[rr * DKP + ic] * __expf(gl - sG[rr * DKP + ic]);
#pragma unroll
                for (int t = 0; t < NCT; ++t) acc[t] = mfma4(ak, sX[rr * BVP + 16 * t + lr], acc[t]);
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
        if (last && hT) dst = hT + (static_cast<int64_t>(n) * H + h) * DK * DV;
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

template <int DK, int C, int MODE>
static void launch_fp32_dk(const ChunkLaunch &L, const SegmentView &sv, int max_segs) {
    constexpr int BV = 32;
    const int slices = MODE == kOut ? L.dv / BV : (L.dv + DK) / BV;
    dim3 grid(static_cast<unsigned>(slices * max_segs), L.H), block(256);
#define KDA_CHUNK(IB, OB)                                                                               \
    hipLaunchKernelGGL((chunk_fp32_kernel<DK, C, BV, IB, OB, MODE>), grid, block, 0, L.stream, L.q, L.k, \
                       L.v, L.g, L.beta, L.hT, L.o, sv, L.H, L.dv, L.scale, L.xf)
    if (L.in_bf16 && L.out_bf16) KDA_CHUNK(true, true);
    else if (L.in_bf16) KDA_CHUNK(true, false);
    else if (L.out_bf16) KDA_CHUNK(false, true);
    else KDA_CHUNK(false, false);
#undef KDA_CHUNK
}

template <int MODE>
void launch_fp32_pass(const ChunkLaunch &L, const SegmentView &sv, int max_segs) {
    if (L.dk == 128) {
        if (L.chunk == 64) launch_fp32_dk<128, 64, MODE>(L, sv, max_segs);
        else if (L.chunk == 32) launch_fp32_dk<128, 32, MODE>(L, sv, max_segs);
        else launch_fp32_dk<128, 16, MODE>(L, sv, max_segs);
    } else {
        if (L.chunk == 64) launch_fp32_dk<64, 64, MODE>(L, sv, max_segs);
        else if (L.chunk == 32) launch_fp32_dk<64, 32, MODE>(L, sv, max_segs);
        else launch_fp32_dk<64, 16, MODE>(L, sv, max_segs);
    }
}

template void launch_fp32_pass<kLocal>(const ChunkLaunch &, const SegmentView &, int);
template void launch_fp32_pass<kOut>(const ChunkLaunch &, const SegmentView &, int);

}  // namespace kda
