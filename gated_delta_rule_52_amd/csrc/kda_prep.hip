// kda_prep.hip - per-chunk preparation of the chunkwise KDA prefill for bf16
// inputs on gfx950 matrix cores (dk = dv = 128, chunk 64).
//
// Everything in a chunk that does not depend on the state entering it is
// computed here, for all chunks of all sequences and heads at once (one
// workgroup per chunk and head, no ordering between them), and written as a
// compact fp16 operand pack (kda_mfma.h) that the serial scan kernels
// (kda_scan.hip) only stream (Kimi Linear review notes, section "Chunkwise
// Algorithm"; jxzklqfsx.com article, WY representation and UT transform):
//
//   a1  G = chunk-local cumulative log decay, gamma = exp(G_last);
//   a2  decayed Gram blocks A_kk (strictly lower, times beta) and A_qk
//       (lower, times the output scale) on bf16 MFMA;
//   a3  T = (I + A_kk)^{-1}: the four 16x16 diagonal blocks by forward
//       substitution, the rest implicitly by a blocked forward solve;
//   a4  the WY factors W = T beta (e^G k) and U = T beta v, so that a scan
//       step is V_new = U - W S, o = (scale e^G q) S + A_qk V_new,
//       S <- gamma S + (e^{G_last - G} k)^T V_new.
//
// Numerics:
// * Gram blocks: operands split into bf16 high and low parts, three products
//   (~16 significant bits, fp32 exponent range).  The decay is factored about
//   the per-channel midpoint m = G_last / 2: rows k_r exp(G_r - m),
//   q_r exp(G_r - m), columns k_i exp(m - G_i), each within exp(+-40).  A
//   chunk whose decay exceeds exp(-80) in some channel takes an exact
//   pair-by-pair fp32 path instead.
// * Everything stored is fp16 with a power-of-two scale per chunk and
//   matrix, chosen from the matrix's maximum, so fp16's range never binds.
//
// The optional input transforms (XF instantiation) act on the values as they
// arrive: the gate logit becomes the log-gate before the cumulative sum, and
// each row's 1/|k| and 1/|q| (reduced over the 16 lanes that hold the row)
// scale k and q before any product or maximum is formed.
//
// With one gate per token and head (SG instantiation, Gated DeltaNet's gate)
// the decay leaves the contraction: A_kk[r,i] = beta_r e^{G_r - G_i} (k_r.k_i)
// and A_qk[r,i] = scale e^{G_r - G_i} (q_r.k_i).  The Gram products then take
// the raw bf16 inputs as they arrive, one product each (bf16 x bf16 products
// are exact in the fp32 accumulator), the decay and the L2 norms scale the
// 64 x 64 results, and e^G, e^{G_L - G} are one exponential per row.  No
// chunk needs the exact path.
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace mc {
namespace {

constexpr int NW = 4, NT = NW * kWave;
constexpr int HC = DK / 2;  // channels per half of dk
// Gram operand tiles of one half of dk: [64 rows][64 channels] bf16, 128-byte
// rows whose 16-byte units are XOR-swizzled by (row / 2) mod 8: a 16-byte read
// of 16 consecutive rows (one MFMA operand) then touches every bank once
__device__ __forceinline__ int g_off(int r, int ch) {  // in halves
    return r * HC + ((((ch >> 3) ^ ((r >> 1) & 7)) << 3) | (ch & 7));
}
constexpr int KP = DK + 8;  // row stride (halves) of [row][dk] tiles
constexpr int GP = DK + 4;  // row stride (floats) of [row][dk] fp32 tiles
constexpr int BP = 16 + 8;  // row stride of 16x16 half blocks
// Blocks of A in "lane order": lane 16 g + n of a 16x16x16 product's A
// operand holds row n, columns 4 g .. 4 g + 3, as 4 consecutive halves at
// 8 lane.  The Gram products are formed transposed (column operand first),
// so that their accumulators hold exactly these values.
__device__ __forceinline__ int lane_pos(int row, int col) { return 4 * (row + 16 * (col >> 2)) + (col & 3); }
// fp32 diagonal blocks of A_kk: rows of 20 floats (16-byte aligned), blocks
// 324 floats apart (the four blocks a lane group reads fall on different banks)
constexpr int kAdRow = 20, kAdBlock = 16 * kAdRow + 4;
__device__ __forceinline__ int ad_off(int a, int r, int c) { return a * kAdBlock + r * kAdRow + c; }
constexpr float kMaxChunkDecay = 80.0f;
constexpr int NJOB = 20;    // Gram tile jobs: 10 A_kk block pairs, then 10 A_qk
constexpr int JPW = NJOB / NW;

struct alignas(16) PrepSmem {
    // The operand area comes first: every per-row access to it is one
    // per-thread base plus an immediate offset below 64 KiB.  The Gram
    // operands are dead once the Gram blocks are formed, and everything
    // after them lives in the same bytes.
    union alignas(16) {
        struct {  // Gram operands of one half of dk, bf16 high/low parts, [row][channel]
            uint16_t rkh[C * HC], rkl[C * HC];   // k_r e^{G_r - m}  (g_off layout)
            uint16_t rqh[C * HC], rql[C * HC];   // q_r e^{G_r - m}
            uint16_t ckh[C * HC], ckl[C * HC];   // k_i e^{m - G_i}
        } g;
        struct {
            _Float16 ek[C * KP];                   // k e^G 2^-ek; later W, swizzled [64][128]
            alignas(16) float ad[4 * kAdBlock];     // diagonal blocks of A_kk (fp32, true scale), ad_off
            alignas(16) _Float16 akk[6][64 * 4];    // off-diagonal blocks of A_kk, x 2^-2ek, in lane order
            alignas(16) _Float16 aqk[10][64 * 4];   // blocks of A_qk (incl. scale), x 2^-(eq+ek), in lane order
            alignas(16) _Float16 tinv[4][16 * BP];  // diagonal blocks of T, x 2^-et
            // v of the chunk (bf16), written after the Gram products: rows of 256 bytes whose 16-byte units
            // are XOR-swizzled by 2 ((row / 4) mod 4), so that the solve's reads in accumulator layout (four
            // rows four apart, 32 bytes of each) fall on distinct banks
            alignas(16) uint16_t v[C * DV];
        } s;
        float part[C / 4][DK];  // column sums of g per group of four rows (dead before the Gram operands)
    } op;
    float beta[C];
    float nrm[2 * C];                      // XF with the L2 norm: 1/|k_r|, then 1/|q_r|, per row
    alignas(16) float gam[DK];             // exp(G_last) per channel
    int imax[8];                           // |k|, |scale q|, |v|, -, |T|, exact flag, |W|, |U|
};
// three workgroups per compute unit (160 KiB of LDS), with room for coarse allocation granules
static_assert(3 * (sizeof(PrepSmem) + 2048) <= 160 * 1024, "three workgroups per compute unit");

// block-pair index p -> (a, b), b <= a, in the order (0,0),(1,0),(1,1),(2,0)...
__device__ __forceinline__ void pair_ab(int p, int &a, int &b) {
    a = 0;
    int rem = p;
    while (rem > a) { rem -= a + 1; ++a; }
    b = rem;
}
__device__ __forceinline__ int offdiag_index(int a, int b) {  // b < a
    return a * (a - 1) / 2 + b;
}

constexpr float kLog2e = 1.4426950408889634f;

// One chunk: chunk bx % per of segment bx / per, head h, into pack number
// bx * H + h.  RV (for the gradients) also writes the reverse pack's -Kd,
// -W^T and Q^T slots (kda_mfma.h) from the same fp16 values, into rpacks.  EXACT = false is the matrix-core path; a chunk whose decay
// exceeds exp(-kMaxChunkDecay) in some channel is not written there but
// flagged in its pack's header, and EXACT = true redoes it with the pair-by-pair
// Gram blocks.  Returns early (whole workgroup) for chunks past the segment end.
template <bool EXACT, bool XF, bool SG, bool RV>
__device__ __forceinline__ void prep_chunk(PrepSmem &sm, float *gx, float *nx, int bx, int h,
                                           const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                           const uint16_t *__restrict__ v, const float *__restrict__ g,
                                           const uint16_t *__restrict__ beta, const SegmentView &sv, int per,
                                           int H, float scale, char *packs, const InputXform ix, char *rpacks) {
    static_assert(!SG || (XF && !EXACT), "the scalar gate runs in the transform instantiation, fast path only");
    static_assert(!RV || (!XF && !SG), "the reverse pack serves the gradients, which take no input transform");
    const int seg = bx / per, jc = bx - seg * per;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    // key-side ownership: channels hh HC + 4 cq .. + 3 of both halves hh of dk, of rows 4 rq .. 4 rq + 3.
    // The 16 lanes of one DPP row hold a whole token row, and every load moves 8 bytes of a bf16 input or
    // 16 bytes of the gate.
    const int cq = tid & 15, rq = tid >> 4;
    // the fast path records in every slot's pack whether it leaves the chunk to the exact path (empty: no)
    char *pack = packs + (static_cast<int64_t>(bx) * H + h) * kPkBytes;
    int *xflag = reinterpret_cast<int *>(pack + kPkHdr + 4 * kHdrX);
    if (seg >= sv.count()) {
        if (!EXACT && tid == 0) *xflag = 0;
        return;
    }
    const int4 sd = sv.desc(seg);
    const int64_t c0 = sd.y + static_cast<int64_t>(C) * jc, t1 = sd.z;
    if (c0 >= t1) {
        if (!EXACT && tid == 0) *xflag = 0;
        return;
    }
    const int L = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);

    // the chunk's rows of head h; rows past L read as zero
    const uint32_t tok_stride = static_cast<uint32_t>(H) * DK;
    const int64_t base = (c0 * H + h) * DK;
    const uint32_t elems = static_cast<uint32_t>((L - 1) * tok_stride + DK);
    const rsrc_t rs_k = make_rsrc(k + base, 2 * elems);
    const rsrc_t rs_q = make_rsrc(q + base, 2 * elems);
    const rsrc_t rs_v = make_rsrc(v + base, 2 * elems);
    // the gate: [.., dk] per channel, or one value per row at stride H with a scalar gate (XF only);
    // the unused resource has size 0, so no load through it touches memory
    const bool sg = SG || (XF && ix.scalar_gate);
    const rsrc_t rs_g = make_rsrc(g + (sg ? 0 : base), sg ? 0 : 4 * elems);
    const rsrc_t rs_gs = make_rsrc(g + (sg ? c0 * H + h : 0), sg ? 4 * static_cast<uint32_t>((L - 1) * H + 1) : 0);
    const rsrc_t rs_p = make_rsrc(pack, kPkBytes);
    const rsrc_t rs_r = make_rsrc(RV ? rpacks + (static_cast<int64_t>(bx) * H + h) * kRvBytes : nullptr,
                                  RV ? kRvBytes : 0);
    const uint32_t key_lane = 4 * rq * tok_stride + 4 * cq;

    if (tid < 8) sm.imax[tid] = 0;
    // v in 16-byte units (unit tid + NT i: row / 16, 8 channels), consumed by the solve (a4) after a trip
    // through LDS.  Without the input transforms the loads are issued first, so that they are long done
    // when the units are staged after the Gram products; the transforms' extra registers leave no room to
    // hold them that long, and there they are issued once the Gram operands are dead.
    u4 vraw[C * DV / 8 / NT];
    auto load_v = [&]() {
#pragma unroll
        for (int i = 0; i < C * DV / 8 / NT; ++i) {
            const int u = tid + NT * i;
            vraw[i] = __builtin_amdgcn_raw_buffer_load_b128(rs_v, 2 * ((u >> 4) * tok_stride + 8 * (u & 15)), 0, 0);
        }
    };
    if constexpr (!XF) load_v();
    __syncthreads();

    // ============ a1: raw inputs to registers, maxima, chunk-local cumulative decay ============
    float G[2][4][4];  // [half][row][channel]
    u2 rk[2][4], rqv[2][4];  // four bf16 channels of k and q per [half][row]
    float nk[4], nq[4];  // XF: 1/|k| and 1/|q| of each of this thread's rows (1 without the L2 norm)
    {
        uint32_t mk2 = 0u, mq2 = 0u;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t e = m * tok_stride + hh * HC + key_lane;
                float gv[4];
                if (sg) {
                    const float gs = __uint_as_float(ld32(rs_gs, 4 * (4 * rq + m) * static_cast<uint32_t>(H)));
#pragma unroll
                    for (int i = 0; i < 4; ++i) gv[i] = gs;
                } else {
                    const u4 gg = __builtin_amdgcn_raw_buffer_load_b128(rs_g, 4 * e, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) gv[i] = __uint_as_float(gg[i]);
                }
                rk[hh][m] = ld64(rs_k, 2 * e);
                rqv[hh][m] = ld64(rs_q, 2 * e);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (XF)  // rows past the chunk end stay 0: they must not decay G_last
                        gv[i] = 4 * rq + m < L ? ix.log_gate(gv[i]) : 0.f;
                    run[i] += gv[i];
                    G[hh][m][i] = run[i];
                }
                mk2 = absmax2(absmax2(mk2, rk[hh][m][0]), rk[hh][m][1]);
                mq2 = absmax2(absmax2(mq2, rqv[hh][m][0]), rqv[hh][m][1]);
            }
            *reinterpret_cast<f4 *>(&sm.op.part[rq][hh * HC + 4 * cq]) = f4{run[0], run[1], run[2], run[3]};
        }
        if (tid < C) sm.beta[tid] = tid < L ? bf16_to_f32(beta[(c0 + tid) * H + h]) : 0.f;
        float mk = wave_max(absmax2_value(mk2)), mq = wave_max(absmax2_value(mq2));
#pragma unroll
        for (int m = 0; m < 4; ++m) nk[m] = nq[m] = 1.f;
        if (XF && ix.qk_l2norm) {
            // a row's 128 channels sit in the 16 lanes of one DPP row, eight per lane
            float ak = 0.f, aq = 0.f;  // largest |k|/|k_row|, |q|/|q_row| of this thread
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                float sk2 = 0.f, sq2 = 0.f, xk = 0.f, xq = 0.f;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        const float k0 = lo_f(rk[hh][m][w]), k1 = hi_f(rk[hh][m][w]);
                        const float q0 = lo_f(rqv[hh][m][w]), q1 = hi_f(rqv[hh][m][w]);
                        sk2 += k0 * k0 + k1 * k1;
                        sq2 += q0 * q0 + q1 * q1;
                        xk = fmaxf(xk, fmaxf(fabsf(k0), fabsf(k1)));
                        xq = fmaxf(xq, fmaxf(fabsf(q0), fabsf(q1)));
                    }
                nk[m] = rsqrtf(row16_sum(sk2) + kL2Eps);
                nq[m] = rsqrtf(row16_sum(sq2) + kL2Eps);
                ak = fmaxf(ak, xk * nk[m]);
                aq = fmaxf(aq, xq * nq[m]);
            }
            mk = wave_max(ak);
            mq = wave_max(aq);
            if (!SG && cq == 0)  // the Gram operands read them back in a2 (registers stay free in between)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    sm.nrm[4 * rq + m] = nk[m];
                    sm.nrm[C + 4 * rq + m] = nq[m];
                }
        }
        if constexpr (EXACT && XF) {  // the rows' norms (1 without the L2 norm) for the pairwise entries
            if (cq == 0)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    nx[4 * rq + m] = nk[m];
                    nx[C + 4 * rq + m] = nq[m];
                }
        }
        if (lane == 0) {
            atomicMax(&sm.imax[0], __float_as_int(mk));
            atomicMax(&sm.imax[1], __float_as_int(mq * fabsf(scale)));
        }
    }
    __syncthreads();  // (1)
    if (tid < DK) {  // channel tid: exclusive prefix over the row groups; part[0] takes the total
        float run = 0.f;
#pragma unroll
        for (int p = 0; p < C / 4; ++p) {
            const float x = sm.op.part[p][tid];
            if (p > 0) sm.op.part[p][tid] = run;
            run += x;
        }
        sm.op.part[0][tid] = run;
        sm.gam[tid] = __expf(run);
        if (!SG && run < -kMaxChunkDecay) atomicOr(&sm.imax[5], 1);
    }
    const int ek = exp_of(__int_as_float(sm.imax[0]));
    const int eq = exp_of(__int_as_float(sm.imax[1]));
    const float sk = pow2(-ek), sq = pow2(-eq) * scale;
    __syncthreads();  // (2) prefixes and flag settled
    float GL[2][4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = hh * HC + 4 * cq + e;
            const float off = rq == 0 ? 0.f : sm.op.part[rq][c];
#pragma unroll
            for (int m = 0; m < 4; ++m) G[hh][m][e] += off;
            GL[hh][e] = sm.op.part[0][c];
        }
    __syncthreads();  // (2b) the sums are read before the operand area takes the Gram operands
    if constexpr (!EXACT) {
        const bool exact = sm.imax[5] != 0;  // beyond the factored form's range: exact kernel
        if (tid == 0) *xflag = exact;
        if (exact) return;
    }

    // ============ a2: Gram tiles, one half of dk at a time ============
    f4 tacc[JPW];
#pragma unroll
    for (int u = 0; u < JPW; ++u) tacc[u] = zero4();
    u2 ekp[2][4];  // four fp16 channels of e^G k per [half][row], kept for the W solve
    // SG: per-row e^G 2^-ek, e^G 2^-eq scale, e^{G_L - G} 2^-ek, with the rows' L2 norms; and the
    // rows' G, 1/|k| and 1/|q| in LDS for the Gram epilogue ([C] each), in the low-part area that SG
    // leaves unused and that the later operand structures never reach
    float sgE[4], sgQ[4], sgD[4];
    float *const sgG = reinterpret_cast<float *>(sm.op.g.ckl), *const sgN = sgG + C;
    static_assert(offsetof(decltype(sm.op.s), v) <= 5 * C * HC * sizeof(uint16_t),
                  "the structures written before the Gram epilogue ends stay clear of the low-part area of the "
                  "column operand");
    if constexpr (SG) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float e = __expf(G[0][m][0]), d = __expf(GL[0][0] - G[0][m][0]);
            sgE[m] = e * sk * nk[m];
            sgQ[m] = e * sq * nq[m];
            sgD[m] = d * sk * nk[m];
            if (cq == 0) {
                sgG[4 * rq + m] = G[0][m][0];
                sgN[4 * rq + m] = nk[m];
                sgN[C + 4 * rq + m] = nq[m];
            }
        }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        // per channel: m log2(e) with m = G_L / 2, and e^m times the fp16 scales
        float mlg[4], em_sk[4], em_sq[4];
#pragma unroll
        for (int e = 0; e < 4 && !SG; ++e) {
            mlg[e] = 0.5f * kLog2e * GL[hh][e];
            const float em = __builtin_amdgcn_exp2f(mlg[e]);
            em_sk[e] = em * sk;
            em_sq[e] = em * sq;
        }
        u2 kdp[4];  // per channel: e^{G_L - G} k of the four rows, fp16
        u2 qdp[4];  // RV: the same for the rows of Q
        auto put_half = [](u2 &w, int m, uint32_t hb) {
            w[m >> 1] = (m & 1) ? (w[m >> 1] | (hb << 16)) : hb;
        };
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 4 * rq + m;
            float kk[4] = {lo_f(rk[hh][m][0]), hi_f(rk[hh][m][0]), lo_f(rk[hh][m][1]), hi_f(rk[hh][m][1])};
            float qq[4] = {lo_f(rqv[hh][m][0]), hi_f(rqv[hh][m][0]), lo_f(rqv[hh][m][1]), hi_f(rqv[hh][m][1])};
            if constexpr (SG) {  // the Gram operands are the raw inputs
                *reinterpret_cast<u2 *>(&sm.op.g.rkh[g_off(r, 4 * cq)]) = rk[hh][m];
                *reinterpret_cast<u2 *>(&sm.op.g.rqh[g_off(r, 4 * cq)]) = rqv[hh][m];
                ekp[hh][m] = u2{pack_h2(kk[0] * sgE[m], kk[1] * sgE[m]), pack_h2(kk[2] * sgE[m], kk[3] * sgE[m])};
                st64(rs_p, u2{pack_h2(qq[0] * sgQ[m], qq[1] * sgQ[m]), pack_h2(qq[2] * sgQ[m], qq[3] * sgQ[m])},
                     kPkQ + w_col(r, hh * HC + 4 * cq));
#pragma unroll
                for (int e = 0; e < 4; ++e) put_half(kdp[e], m, hbits(static_cast<_Float16>(kk[e] * sgD[m])));
                continue;
            }
            if (XF && ix.qk_l2norm) {
                const float nkm = sm.nrm[r], nqm = sm.nrm[C + r];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kk[e] *= nkm;
                    qq[e] *= nqm;
                }
            }
            float ekv[4], qsv[4], kdv[4], ra[4], rb[4], rc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float Gm = G[hh][m][e];
                if constexpr (!EXACT) {
                    // row factor e^{G - m}, column factor e^{m - G}, both within e^{+-40}
                    const float t = fmaf(Gm, kLog2e, -mlg[e]);
                    const float rf = __builtin_amdgcn_exp2f(t), cf = __builtin_amdgcn_exp2f(-t);
                    ra[e] = kk[e] * rf;          // Gram row operand k e^{G - m} (unscaled)
                    rb[e] = qq[e] * rf;          // ... q e^{G - m}
                    rc[e] = kk[e] * cf;          // Gram column operand k e^{m - G}
                    ekv[e] = ra[e] * em_sk[e];   // k e^G 2^-ek
                    qsv[e] = rb[e] * em_sq[e];   // scale q e^G 2^-eq
                    kdv[e] = rc[e] * em_sk[e];   // k e^{G_L - G} 2^-ek, G_L = 2m
                } else {
                    const float E = __expf(Gm);
                    ekv[e] = kk[e] * E * sk;
                    qsv[e] = qq[e] * E * sq;
                    kdv[e] = kk[e] * __expf(GL[hh][e] - Gm) * sk;
                    ra[e] = rb[e] = rc[e] = 0.f;
                }
            }
            ekp[hh][m] = u2{pack_h2(ekv[0], ekv[1]), pack_h2(ekv[2], ekv[3])};
            // Q: the four channels hh HC + 4cq .. + 3 of row r are 8 contiguous bytes of a 16-byte unit (the
            // gradients' passes read only the reverse pack's Q^T, so their forward pack goes without)
            if constexpr (!RV)
                st64(rs_p, u2{pack_h2(qsv[0], qsv[1]), pack_h2(qsv[2], qsv[3])}, kPkQ + w_col(r, hh * HC + 4 * cq));
            u2 kdw = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t hb = hbits(static_cast<_Float16>(kdv[e]));
                put_half(kdp[e], m, hb);
                put_half(kdw, e, hb);
                if constexpr (RV) put_half(qdp[e], m, hbits(static_cast<_Float16>(qsv[e])));
            }
            if constexpr (RV)  // -Kd, row-major like W (the sign bits flipped)
                st64(rs_r, u2{kdw[0] ^ 0x80008000u, kdw[1] ^ 0x80008000u}, kPkW + w_col(r, hh * HC + 4 * cq));
            if constexpr (!EXACT) {
                // high and low bf16 parts of four channels, 8 bytes each
                auto put_split = [&](const float (&x)[4], uint16_t *dh, uint16_t *dl) {
                    uint32_t h0, l0, h1, l1;
                    split2(x[0], x[1], h0, l0);
                    split2(x[2], x[3], h1, l1);
                    *reinterpret_cast<u2 *>(&dh[g_off(r, 4 * cq)]) = u2{h0, h1};
                    *reinterpret_cast<u2 *>(&dl[g_off(r, 4 * cq)]) = u2{l0, l1};
                };
                put_split(ra, sm.op.g.rkh, sm.op.g.rkl);
                put_split(rc, sm.op.g.ckh, sm.op.g.ckl);
                put_split(rb, sm.op.g.rqh, sm.op.g.rql);
            }
        }
        // KT: the four rows 4rq .. 4rq + 3 of one channel are 8 contiguous bytes
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            st64(rs_p, kdp[e], kPkKT + kt_col(hh * HC + 4 * cq + e, 4 * rq));
            if constexpr (RV)  // Q^T, laid out like KT
                st64(rs_r, qdp[e], kPkQ + kt_col(hh * HC + 4 * cq + e, 4 * rq));
        }
        if constexpr (!EXACT) {
            __syncthreads();  // (3a) this half's operands in LDS
#pragma unroll
            for (int u = 0; u < JPW; ++u) {
                const int j = wave + NW * u;
                const bool isq = j >= 10;
                int a, b;
                pair_ab(isq ? j - 10 : j, a, b);
                const uint16_t *rh = isq ? sm.op.g.rqh : sm.op.g.rkh;
                const uint16_t *rl = isq ? sm.op.g.rql : sm.op.g.rkl;
#pragma unroll
                for (int s = 0; s < HC / 32; ++s) {
                    const int ra = g_off(16 * a + n16, 32 * s + 8 * g4);
                    const int cb = g_off(16 * b + n16, 32 * s + 8 * g4);
                    if constexpr (SG) {  // raw k (columns) against raw k or q (rows): one exact product
                        const b8 xr = *reinterpret_cast<const b8 *>(rh + ra);
                        const b8 yc = *reinterpret_cast<const b8 *>(sm.op.g.rkh + cb);
                        tacc[u] = mmab(yc, xr, tacc[u]);
                        continue;
                    }
                    const b8 xh = *reinterpret_cast<const b8 *>(rh + ra);
                    const b8 xl = *reinterpret_cast<const b8 *>(rl + ra);
                    const b8 yh = *reinterpret_cast<const b8 *>(sm.op.g.ckh + cb);
                    const b8 yl = *reinterpret_cast<const b8 *>(sm.op.g.ckl + cb);
                    // transposed: accumulator (4 g4 + jj, n16) = entry (16 a + n16, 16 b + 4 g4 + jj)
                    tacc[u] = mmab(yh, xh, tacc[u]);
                    tacc[u] = mmab(yl, xh, tacc[u]);
                    tacc[u] = mmab(yh, xl, tacc[u]);
                }
            }
            __syncthreads();  // (3b) this half's operands consumed
        }
    }
    if constexpr (XF) load_v();
    if constexpr (!EXACT) {
        const float skk = sk * sk, sqk = sq * sk;  // stored A_kk x 2^-2ek, A_qk x 2^-(eq + ek)
#pragma unroll
        for (int u = 0; u < JPW; ++u) {
            const int j = wave + NW * u;
            const bool isq = j >= 10;
            const int p = isq ? j - 10 : j;
            int a, b;
            pair_ab(p, a, b);
            // this lane's entries: row 16 a + n16, columns 16 b + 4 g4 + jj
            f4 v = tacc[u];
            if constexpr (SG) {  // the decay e^{G_r - G_i} and the rows' L2 norms
                const int r = 16 * a + n16;
                const float Gr = sgG[r], nr = isq ? sgN[C + r] : sgN[r];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int i = 16 * b + 4 * g4 + jj;
                    v[jj] *= __expf(fminf(Gr - sgG[i], 0.f)) * nr * sgN[i];
                }
            }
            if (!isq) {  // A_kk = beta k k^T (decayed), strictly lower
                const float br = sm.beta[16 * a + n16];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) v[jj] = (a > b || 4 * g4 + jj < n16) ? br * v[jj] : 0.f;
                if (a == b) *reinterpret_cast<f4 *>(&sm.op.s.ad[ad_off(a, n16, 4 * g4)]) = v;
                else *reinterpret_cast<h4 *>(&sm.op.s.akk[offdiag_index(a, b)][4 * lane]) = to_h4(v, skk);
            } else {     // A_qk = scale q k^T (decayed), lower
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) v[jj] = (a > b || 4 * g4 + jj <= n16) ? v[jj] : 0.f;
                *reinterpret_cast<h4 *>(&sm.op.s.aqk[p][4 * lane]) = to_h4(v, sqk);
            }
        }
    } else {
        // exact path: A entries pair by pair from exp(G_r - G_i), fp32 (compiled for EXACT only)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int e = 0; e < 4; ++e) gx[(4 * rq + m) * GP + hh * HC + 4 * cq + e] = G[hh][m][e];
            }
        __syncthreads();
        for (int pr = tid; pr < C * C; pr += NT) {
            const int rr = pr / C, ii = pr % C;
            if (ii > rr) continue;
            float vk = 0.f, vq = 0.f;
            if (rr < L) {
                const int64_t br = ((c0 + rr) * H + h) * DK, bi = ((c0 + ii) * H + h) * DK;
                for (int c = 0; c < DK; ++c) {
                    const float d = __expf(gx[rr * GP + c] - gx[ii * GP + c]);
                    const float kk = bf16_to_f32(k[bi + c]) * d;
                    vk += bf16_to_f32(k[br + c]) * kk;
                    vq += bf16_to_f32(q[br + c]) * kk;
                }
            }
            if constexpr (XF) {  // the rows' L2 norms (1 without the transform)
                vk *= nx[rr] * nx[ii];
                vq *= nx[C + rr] * nx[ii];
            }
            const int a = rr >> 4, b = ii >> 4, rl4 = rr & 15, cl = ii & 15;
            const float ak = ii < rr ? sm.beta[rr] * vk : 0.f;
            if (a == b) sm.op.s.ad[ad_off(a, rl4, cl)] = ak;
            else sm.op.s.akk[offdiag_index(a, b)][lane_pos(rl4, cl)] = static_cast<_Float16>(ak * sk * sk);
            sm.op.s.aqk[a * (a + 1) / 2 + b][lane_pos(rl4, cl)] = static_cast<_Float16>(vq * sk * sq);
        }
        for (int pr = tid; pr < 4 * 256; pr += NT) {  // upper halves of the diagonal blocks
            const int a = pr >> 8, rl4 = (pr >> 4) & 15, cl = pr & 15;
            if (cl > rl4) {
                sm.op.s.ad[ad_off(a, rl4, cl)] = 0.f;
                sm.op.s.aqk[a * (a + 1) / 2 + a][lane_pos(rl4, cl)] = static_cast<_Float16>(0.f);
            }
        }
    }
    __syncthreads();  // (4) Gram results in LDS; operand area free

    // ============ a3: diagonal blocks of T; e^G k to LDS, Q and KT to the pack ============
    // v staged in LDS (swizzled units, see PrepSmem)
    auto v_at = [](int r, int c) { return r * DV + ((((c >> 3) ^ (2 * ((r >> 2) & 3)))) << 3) + (c & 7); };
#pragma unroll
    for (int i = 0; i < C * DV / 8 / NT; ++i) {
        const int u = tid + NT * i;
        *reinterpret_cast<u4 *>(&sm.op.s.v[v_at(u >> 4, 8 * (u & 15))]) = vraw[i];
    }
    float tcol[16];
    if (wave == 0) {  // lane 16a + j owns column j of T_aa = (I + A_aa)^{-1}
        const int a = g4, j = n16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i + 1 < r; i += 2) {
                s0 -= sm.op.s.ad[ad_off(a, r, i)] * tcol[i];
                s1 -= sm.op.s.ad[ad_off(a, r, i + 1)] * tcol[i + 1];
            }
            if (r & 1) s0 -= sm.op.s.ad[ad_off(a, r, r - 1)] * tcol[r - 1];
            tcol[r] = s0 + s1;
        }
        float tm = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) tm = fmaxf(tm, fabsf(tcol[r]));
        tm = wave_max(tm);
        if (lane == 0) sm.imax[4] = __float_as_int(tm);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            *reinterpret_cast<u2 *>(&sm.op.s.ek[(4 * rq + m) * KP + hh * HC + 4 * cq]) = ekp[hh][m];
    {   // |v| maximum, from the raw units (bf16 magnitudes order as integers)
        uint32_t mv = 0u;
#pragma unroll
        for (int i = 0; i < C * DV / 8 / NT; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) mv = absmax2(mv, vraw[i][w]);
        const float mvf = wave_max(absmax2_value(mv));
        if (lane == 0) atomicMax(&sm.imax[2], __float_as_int(mvf));
    }
    __syncthreads();  // (5)
    // the solve's v values in accumulator layout: rows 16 a + 4 g4 + jj of column 16 (2 wave + t) + n16
    uint32_t vpre[2][4][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                vpre[t][a][jj] = sm.op.s.v[v_at(16 * a + 4 * g4 + jj, 16 * (2 * wave + t) + n16)];
    const int et = exp_of(__int_as_float(sm.imax[4]));
    const int ev = exp_of(__int_as_float(sm.imax[2])) - 5;  // U's solve runs below 2^5
    const float svs = pow2(-ev);
    if (wave == 0) {
        const float st = pow2(-et);
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.op.s.tinv[g4][r * BP + n16] = static_cast<_Float16>(tcol[r] * st);
    }
    __syncthreads();  // (6)

    // ============ a4: W = T beta (e^G k) and U = T beta v by the blocked forward solve ============
    // wave w: column tiles 2w, 2w + 1 of both.  W is formed in the 2^-ek
    // frame of the stored e^G k, U in the 2^-ev frame.  Per row block a:
    //   Y_a = X_a - sum_{b<a} A_ab V_b,  V_a = T_aa Y_a.
    // V_a below is T_aa Y_a without T's 2^et: the products with it take the
    // factor in uns, the stored W and U and their maxima in their scales
    const float unt = pow2(et), uns = pow2(2 * ek) * unt;
    f4 Wr[2][4], Ur[2][4];
    float mw = 0.f, mu = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int col = 16 * (2 * wave + t) + n16;
#pragma unroll
        for (int kind = 0; kind < 2; ++kind) {
            h4 Vh[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f4 xp;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rr = 16 * a + 4 * g4 + jj;
                    const float x = kind == 0 ? static_cast<float>(sm.op.s.ek[rr * KP + col])
                                              : lo_f(vpre[t][a][jj]) * svs;
                    xp[jj] = sm.beta[rr] * x;
                }
                f4 accs = zero4();
#pragma unroll
                for (int b = 0; b < a; ++b) {
                    const h4 aab = *reinterpret_cast<const h4 *>(&sm.op.s.akk[offdiag_index(a, b)][4 * lane]);
                    accs = mma16(aab, Vh[b], accs);
                }
                f4 yv;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) yv[jj] = xp[jj] - accs[jj] * uns;
                const h4 ta = *reinterpret_cast<const h4 *>(&sm.op.s.tinv[a][n16 * BP + 4 * g4]);
                const f4 va = mma16(ta, to_h4(yv, 1.f), zero4());
                Vh[a] = to_h4(va, 1.f);
                if (kind == 0) {
                    Wr[t][a] = va;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) mw = fmaxf(mw, fabsf(va[jj]));
                } else {
                    Ur[t][a] = va;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) mu = fmaxf(mu, fabsf(va[jj]));
                }
            }
        }
    }
    mw = wave_max(mw) * unt;
    mu = wave_max(mu) * unt;
    if (lane == 0) {
        atomicMax(&sm.imax[6], __float_as_int(mw));
        atomicMax(&sm.imax[7], __float_as_int(mu));
    }
    __syncthreads();  // (7) all reads of e^G k done; its area takes W
    const int ew = exp_of(__int_as_float(sm.imax[6])), eu = exp_of(__int_as_float(sm.imax[7]));
    {
        const float swv = pow2(-ew) * unt, suv = pow2(-eu) * unt;
        char *wst = reinterpret_cast<char *>(sm.op.s.ek);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ct = 2 * wave + t, col = 16 * ct + n16;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rr = 16 * a + 4 * g4 + jj;
                    *reinterpret_cast<_Float16 *>(wst + w_col(rr, col)) =
                        static_cast<_Float16>(Wr[t][a][jj] * swv);
                }
                // U straight to the pack, in accumulator order: row blocks a - 1 and a are one 16-byte unit
                if (a & 1) {
                    const u2 ul = __builtin_bit_cast(u2, to_h4(Ur[t][a - 1], suv));
                    const u2 uh = __builtin_bit_cast(u2, to_h4(Ur[t][a], suv));
                    st128(rs_p, u4{ul[0], ul[1], uh[0], uh[1]}, kPkU + u_off(ct, a - 1, lane));
                }
                if constexpr (RV) {  // -W^T, laid out like KT: rows 16 a + 4 g4 .. + 3 of column col are 8 bytes
                    const u2 wh = __builtin_bit_cast(u2, to_h4(Wr[t][a], swv));
                    st64(rs_r, u2{wh[0] ^ 0x80008000u, wh[1] ^ 0x80008000u}, kPkKT + kt_col(col, 16 * a + 4 * g4));
                }
            }
        }
    }
    __syncthreads();  // (8) W staged
    // ---- the rest of the pack, 16-byte units, consecutive threads on consecutive units
    {
        const char *wst = reinterpret_cast<const char *>(sm.op.s.ek);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = tid + NT * i;  // 0 .. 1023
            st128(rs_p, *reinterpret_cast<const u4 *>(wst + 16 * u), kPkW + 16 * u);
        }
        for (int u = tid; u < 10 * 64 * 8 / 16; u += NT)  // A_qk blocks, already in lane order
            st128(rs_p, *reinterpret_cast<const u4 *>(reinterpret_cast<const char *>(sm.op.s.aqk) + 16 * u),
                  kPkA + 16 * u);
        if (tid < DK / 4)
            st128(rs_p, *reinterpret_cast<const u4 *>(&sm.gam[4 * tid]), kPkGamma + 16 * tid);
        if (tid == 0) {
            // true W = stored * 2^(ew + ek); U = stored * 2^(eu + ev); Q (scale
            // included) = stored * 2^eq; KT = stored * 2^ek; A_qk = stored * 2^(eq + ek)
            const u4 hd = {static_cast<unsigned>(ew + ek), static_cast<unsigned>(eq), static_cast<unsigned>(ek),
                           static_cast<unsigned>(eu + ev)};
            st128(rs_p, hd, kPkHdr);
            st32(rs_p, static_cast<unsigned>(eq + ek), kPkHdr + 16);
        }
    }
}

// fast path: one workgroup per chunk and head; grid.x = (segment * per + chunk) * H + head.
// XF: with the input transforms; SG: scalar gate (implies XF).
template <bool XF, bool SG, bool RV>
__global__ void __launch_bounds__(NT, 3)
chunk_prep_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const uint16_t *__restrict__ v, const float *__restrict__ g,
                  const uint16_t *__restrict__ beta, SegmentView sv, int per, int H, float scale,
                  char *__restrict__ packs, InputXform ix, char *__restrict__ rpacks) {
    __shared__ PrepSmem sm;
    // heads fastest: the workgroups in flight at once cover whole token rows ([T, H, d]: a chunk's H heads
    // read adjacent 256-byte pieces of the same rows) and write consecutive packs (measured at 64K x 16 heads:
    // 1.028 -> 0.984 ms per call against chunks fastest)
    const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(H));
    const int bx = static_cast<int>(blockIdx.x / static_cast<unsigned>(H));
    prep_chunk<false, XF, SG, RV>(sm, nullptr, nullptr, bx, h, q, k, v, g, beta, sv, per, H, scale, packs, ix, rpacks);
}

// exact path over the slots the fast path flagged (usually none): each workgroup takes NT consecutive slots
// at a time, gathers their flags by wave ballots, and runs the flagged ones
template <bool XF, bool RV>
__global__ void __launch_bounds__(NT, 1)
chunk_prep_exact_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                        const uint16_t *__restrict__ v, const float *__restrict__ g,
                        const uint16_t *__restrict__ beta, SegmentView sv, int per, int H, float scale,
                        char *__restrict__ packs, InputXform ix, char *__restrict__ rpacks, int nslots) {
    __shared__ PrepSmem sm;
    __shared__ float gx[C * GP];  // G of the chunk, for the pair-by-pair Gram entries
    __shared__ float nx[2 * C];   // XF: 1/|k| and 1/|q| of each row
    __shared__ unsigned long long s_mask[NT / 64];
    const int tid = threadIdx.x;
    for (int base = blockIdx.x * NT; base < nslots; base += gridDim.x * NT) {
        const bool f = base + tid < nslots &&
                       *reinterpret_cast<const int *>(packs + static_cast<int64_t>(base + tid) * kPkBytes + kPkHdr +
                                                      4 * kHdrX);
        const unsigned long long m = __ballot(f);
        if ((tid & 63) == 0) s_mask[tid >> 6] = m;
        __syncthreads();  // the masks are complete
        for (int w = 0; w < NT / 64; ++w) {
            for (unsigned long long mm = s_mask[w]; mm; mm &= mm - 1) {
                const int id = base + 64 * w + __builtin_ctzll(mm);
                __syncthreads();  // the previous chunk's last LDS reads are done
                prep_chunk<true, XF, false, RV>(sm, gx, nx, id / H, id % H, q, k, v, g, beta, sv, per, H, scale,
                                                packs, ix, rpacks);
            }
        }
        __syncthreads();  // every thread has read the masks
    }
}

}  // namespace
}  // namespace mc

bool f16_path_supported(bool in_bf16, int dk, int dv, int chunk) {
    return in_bf16 && dk == mc::DK && dv == mc::DV && chunk == mc::C;
}

size_t pack_bytes() { return mc::kPkBytes; }

void launch_prep(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, void *packs, void *rpacks) {
    const uint16_t *q = static_cast<const uint16_t *>(L.q), *k = static_cast<const uint16_t *>(L.k);
    const uint16_t *v = static_cast<const uint16_t *>(L.v), *b = static_cast<const uint16_t *>(L.beta);
    char *pk = static_cast<char *>(packs), *rp = static_cast<char *>(rpacks);
    const dim3 grid(static_cast<unsigned>(max_segs) * static_cast<unsigned>(per) * L.H), block(mc::NT);
    const int nslots = static_cast<int>(grid.x);
    if (rp) {  // the gradients: no input transform, and the reverse pack's slots besides
        hipLaunchKernelGGL((mc::chunk_prep_kernel<false, false, true>), grid, block, 0, L.stream, q, k, v, L.g, b, sv,
                           per, L.H, L.scale, pk, L.xf, rp);
        hipLaunchKernelGGL((mc::chunk_prep_exact_kernel<false, true>), dim3(256), block, 0, L.stream, q, k, v, L.g, b,
                           sv, per, L.H, L.scale, pk, L.xf, rp, nslots);
    } else if (L.xf.scalar_gate) {  // the scalar-gate Gram is exact at any decay: no exact pass
        hipLaunchKernelGGL((mc::chunk_prep_kernel<true, true, false>), grid, block, 0, L.stream, q, k, v, L.g, b, sv,
                           per, L.H, L.scale, pk, L.xf, rp);
    } else if (L.xf.any()) {
        hipLaunchKernelGGL((mc::chunk_prep_kernel<true, false, false>), grid, block, 0, L.stream, q, k, v, L.g, b, sv,
                           per, L.H, L.scale, pk, L.xf, rp);
        hipLaunchKernelGGL((mc::chunk_prep_exact_kernel<true, false>), dim3(256), block, 0, L.stream, q, k, v, L.g, b,
                           sv, per, L.H, L.scale, pk, L.xf, rp, nslots);
    } else {
        hipLaunchKernelGGL((mc::chunk_prep_kernel<false, false, false>), grid, block, 0, L.stream, q, k, v, L.g, b, sv,
                           per, L.H, L.scale, pk, L.xf, rp);
        hipLaunchKernelGGL((mc::chunk_prep_exact_kernel<false, false>), dim3(256), block, 0, L.stream, q, k, v, L.g, b,
                           sv, per, L.H, L.scale, pk, L.xf, rp, nslots);
    }
}

}  // namespace kda
