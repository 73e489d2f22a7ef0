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
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace mc {
namespace {

constexpr int NW = 4, NT = NW * kWave;
constexpr int HC = DK / 2;  // channels per half of dk
constexpr int HP = HC + 8;  // row stride (halves) of the half-dk Gram operand tiles
constexpr int KP = DK + 8;  // row stride (halves) of [row][dk] tiles
constexpr int GP = DK + 4;  // row stride (floats) of [row][dk] fp32 tiles
constexpr int BP = 16 + 8;  // row stride of 16x16 half blocks
constexpr float kMaxChunkDecay = 80.0f;
constexpr int NJOB = 20;    // Gram tile jobs: 10 A_kk block pairs, then 10 A_qk
constexpr int JPW = NJOB / NW;

struct alignas(16) PrepSmem {
    // The operand area comes first: every per-row access to it is one
    // per-thread base plus an immediate offset below 64 KiB.
    union alignas(16) {
        struct {  // Gram operands of one half of dk, bf16 high/low parts, [row][channel]
            uint16_t rkh[C * HP], rkl[C * HP];   // k_r e^{G_r - m} 2^-ek
            uint16_t rqh[C * HP], rql[C * HP];   // scale q_r e^{G_r - m} 2^-eq
            uint16_t ckh[C * HP], ckl[C * HP];   // k_i e^{m - G_i} 2^-ek
        } g;
        struct {  // fp16 operands
            _Float16 ek[C * KP];   // k e^G 2^-ek; later W, swizzled [64][128]
        } s;
        float gx[C * GP];          // G, for the exact path
    } op;
    float part[8][DK];                     // column sums of g per group of eight rows
    float beta[C];
    alignas(16) float gam[DK];             // exp(G_last) per channel
    int imax[8];                           // |k|, |scale q|, |v|, -, |T|, exact flag, |W|, |U|
    float ad[4][16][17];                   // diagonal blocks of A_kk (fp32, true scale)
    alignas(16) _Float16 akk[6][16 * BP];  // off-diagonal blocks of A_kk, x 2^-2ek
    alignas(16) _Float16 aqk[10][16 * BP]; // blocks of A_qk (incl. scale), x 2^-(eq+ek)
    alignas(16) _Float16 tinv[4][16 * BP]; // diagonal blocks of T, x 2^-et
};
static_assert(sizeof(PrepSmem) <= 80 * 1024, "two workgroups per compute unit");

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

// Grid: (segments x chunks per segment, heads).  Workgroup (seg * per + j, h)
// prepares chunk j of segment seg for head h into pack number
// (seg * per + j) * H + h.
__global__ void __launch_bounds__(NT, 2)
chunk_prep_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const uint16_t *__restrict__ v, const float *__restrict__ g,
                  const uint16_t *__restrict__ beta, SegmentView sv, int per, int H, float scale,
                  char *__restrict__ packs) {
    __shared__ PrepSmem sm;
    const int seg = blockIdx.x / per, jc = blockIdx.x - seg * per;
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    // key-side ownership: channels {2cq, 2cq + 1} and {HC + 2cq, HC + 2cq + 1}
    // of rows 8 rq8 .. 8 rq8 + 7
    const int cq = tid & 31, rq8 = tid >> 5;
    if (seg >= sv.count()) return;
    const int4 sd = sv.table[seg];
    const int64_t c0 = sd.y + static_cast<int64_t>(C) * jc, t1 = sd.z;
    if (c0 >= t1) return;
    const int L = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);

    // the chunk's rows of head h; rows past L read as zero
    const uint32_t tok_stride = static_cast<uint32_t>(H) * DK;
    const int64_t base = (c0 * H + h) * DK;
    const uint32_t elems = static_cast<uint32_t>((L - 1) * tok_stride + DK);
    const rsrc_t rs_k = make_rsrc(k + base, 2 * elems);
    const rsrc_t rs_q = make_rsrc(q + base, 2 * elems);
    const rsrc_t rs_v = make_rsrc(v + base, 2 * elems);
    const rsrc_t rs_g = make_rsrc(g + base, 4 * elems);
    char *pack = packs + (static_cast<int64_t>(blockIdx.x) * H + h) * kPkBytes;
    const rsrc_t rs_p = make_rsrc(pack, kPkBytes);
    const uint32_t key_lane = 8 * rq8 * tok_stride + 2 * cq;

    if (tid < 8) sm.imax[tid] = 0;
    __syncthreads();

    // ============ a1: raw inputs to registers, maxima, chunk-local cumulative decay ============
    float G[2][8][2];  // [half][row][channel]
    uint32_t rk[2][8], rq[2][8];
    {
        float mk = 0.f, mq = 0.f, mv = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint32_t e = m * tok_stride + hh * HC + key_lane;
                const u2 gg = ld64(rs_g, 4 * e);
                rk[hh][m] = ld32(rs_k, 2 * e);
                rq[hh][m] = ld32(rs_q, 2 * e);
                const uint32_t vv = ld32(rs_v, 2 * e);
                r0 += __uint_as_float(gg[0]);
                r1 += __uint_as_float(gg[1]);
                G[hh][m][0] = r0;
                G[hh][m][1] = r1;
                mk = fmaxf(mk, fmaxf(fabsf(lo_f(rk[hh][m])), fabsf(hi_f(rk[hh][m]))));
                mq = fmaxf(mq, fmaxf(fabsf(lo_f(rq[hh][m])), fabsf(hi_f(rq[hh][m]))));
                mv = fmaxf(mv, fmaxf(fabsf(lo_f(vv)), fabsf(hi_f(vv))));
            }
            sm.part[rq8][hh * HC + 2 * cq] = r0;
            sm.part[rq8][hh * HC + 2 * cq + 1] = r1;
        }
        if (tid < C) sm.beta[tid] = tid < L ? bf16_to_f32(beta[(c0 + tid) * H + h]) : 0.f;
        mk = wave_max(mk);
        mq = wave_max(mq);
        mv = wave_max(mv);
        if (lane == 0) {
            atomicMax(&sm.imax[0], __float_as_int(mk));
            atomicMax(&sm.imax[1], __float_as_int(mq * fabsf(scale)));
            atomicMax(&sm.imax[2], __float_as_int(mv));
        }
    }
    __syncthreads();  // (1)
    float GL[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = hh * HC + 2 * cq + e;
            float off = 0.f, tot = 0.f;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const float x = sm.part[p][c];
                off += p < rq8 ? x : 0.f;
                tot += x;
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) G[hh][m][e] += off;
            GL[hh][e] = tot;
            if (rq8 == 0) {
                sm.gam[c] = __expf(tot);
                if (tot < -kMaxChunkDecay) atomicOr(&sm.imax[5], 1);
            }
        }
    const int ek = exp_of(__int_as_float(sm.imax[0]));
    const int eq = exp_of(__int_as_float(sm.imax[1]));
    const int ev = exp_of(__int_as_float(sm.imax[2])) - 5;  // U's solve runs below 2^5
    const float sk = pow2(-ek), sq = pow2(-eq) * scale, svs = pow2(-ev);
    __syncthreads();  // (2) flag settled
    const bool exact_path = sm.imax[5] != 0;

    // ============ a2: Gram tiles, one half of dk at a time ============
    f4 tacc[JPW];
#pragma unroll
    for (int u = 0; u < JPW; ++u) tacc[u] = zero4();
    uint32_t ekp[2][8], qsp[2][8], kdp[2][2][4];  // fp16 operand pairs
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        float em[2], emi[2];  // e^{m}, e^{-m}, m = G_L / 2
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            em[e] = __expf(0.5f * GL[hh][e]);
            emi[e] = __expf(-0.5f * GL[hh][e]);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int r = 8 * rq8 + m;
            const float kk[2] = {lo_f(rk[hh][m]), hi_f(rk[hh][m])};
            const float qq[2] = {lo_f(rq[hh][m]), hi_f(rq[hh][m])};
            float ekv[2], qsv[2], kdv[2], rkv[2], rqv[2], ckv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float Gm = G[hh][m][e];
                const float E = __expf(Gm);
                ekv[e] = kk[e] * E * sk;
                qsv[e] = qq[e] * E * sq;
                if (!exact_path) {
                    const float Ec = __expf(-Gm) * em[e];  // e^{m - G}
                    rkv[e] = ekv[e] * emi[e];
                    rqv[e] = qsv[e] * emi[e];
                    ckv[e] = kk[e] * Ec * sk;
                    kdv[e] = ckv[e] * em[e];               // e^{G_L - G}, G_L = 2m
                } else {
                    rkv[e] = rqv[e] = ckv[e] = 0.f;
                    kdv[e] = kk[e] * __expf(GL[hh][e] - Gm) * sk;
                }
            }
            ekp[hh][m] = pack_h2(ekv[0], ekv[1]);
            qsp[hh][m] = pack_h2(qsv[0], qsv[1]);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t hb = hbits(static_cast<_Float16>(kdv[e]));
                kdp[hh][e][m >> 1] = (m & 1) ? (kdp[hh][e][m >> 1] | (hb << 16)) : hb;
            }
            if (!exact_path) {
                uint32_t hi, lo;
                split2(rkv[0], rkv[1], hi, lo);
                *reinterpret_cast<uint32_t *>(&sm.op.g.rkh[r * HP + 2 * cq]) = hi;
                *reinterpret_cast<uint32_t *>(&sm.op.g.rkl[r * HP + 2 * cq]) = lo;
                split2(ckv[0], ckv[1], hi, lo);
                *reinterpret_cast<uint32_t *>(&sm.op.g.ckh[r * HP + 2 * cq]) = hi;
                *reinterpret_cast<uint32_t *>(&sm.op.g.ckl[r * HP + 2 * cq]) = lo;
                split2(rqv[0], rqv[1], hi, lo);
                *reinterpret_cast<uint32_t *>(&sm.op.g.rqh[r * HP + 2 * cq]) = hi;
                *reinterpret_cast<uint32_t *>(&sm.op.g.rql[r * HP + 2 * cq]) = lo;
            }
        }
        if (!exact_path) {
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
                    const int ra = (16 * a + n16) * HP + 32 * s + 8 * g4;
                    const int cb = (16 * b + n16) * HP + 32 * s + 8 * g4;
                    const b8 xh = *reinterpret_cast<const b8 *>(rh + ra);
                    const b8 xl = *reinterpret_cast<const b8 *>(rl + ra);
                    const b8 yh = *reinterpret_cast<const b8 *>(sm.op.g.ckh + cb);
                    const b8 yl = *reinterpret_cast<const b8 *>(sm.op.g.ckl + cb);
                    tacc[u] = mmab(xh, yh, tacc[u]);
                    tacc[u] = mmab(xh, yl, tacc[u]);
                    tacc[u] = mmab(xl, yh, tacc[u]);
                }
            }
            __syncthreads();  // (3b) this half's operands consumed
        }
    }
    if (!exact_path) {
#pragma unroll
        for (int u = 0; u < JPW; ++u) {
            const int j = wave + NW * u;
            const bool isq = j >= 10;
            const int p = isq ? j - 10 : j;
            int a, b;
            pair_ab(p, a, b);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rl4 = 4 * g4 + jj, rr = 16 * a + rl4, ii = 16 * b + n16;
                if (!isq) {
                    const float vk = ii < rr ? sm.beta[rr] * tacc[u][jj] : 0.f;
                    if (a == b) sm.ad[a][rl4][n16] = vk * pow2(2 * ek);
                    else sm.akk[offdiag_index(a, b)][rl4 * BP + n16] = static_cast<_Float16>(vk);
                } else {
                    sm.aqk[p][rl4 * BP + n16] = static_cast<_Float16>(ii <= rr ? tacc[u][jj] : 0.f);
                }
            }
        }
    } else {
        // exact path: A entries pair by pair from exp(G_r - G_i), fp32
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                sm.op.gx[(8 * rq8 + m) * GP + hh * HC + 2 * cq] = G[hh][m][0];
                sm.op.gx[(8 * rq8 + m) * GP + hh * HC + 2 * cq + 1] = G[hh][m][1];
            }
        __syncthreads();
        for (int pr = tid; pr < C * C; pr += NT) {
            const int rr = pr / C, ii = pr % C;
            if (ii > rr) continue;
            float vk = 0.f, vq = 0.f;
            if (rr < L) {
                const int64_t br = ((c0 + rr) * H + h) * DK, bi = ((c0 + ii) * H + h) * DK;
                for (int c = 0; c < DK; ++c) {
                    const float d = __expf(sm.op.gx[rr * GP + c] - sm.op.gx[ii * GP + c]);
                    const float kk = bf16_to_f32(k[bi + c]) * d;
                    vk += bf16_to_f32(k[br + c]) * kk;
                    vq += bf16_to_f32(q[br + c]) * kk;
                }
            }
            const int a = rr >> 4, b = ii >> 4, rl4 = rr & 15, cl = ii & 15;
            const float ak = ii < rr ? sm.beta[rr] * vk : 0.f;
            if (a == b) sm.ad[a][rl4][cl] = ak;
            else sm.akk[offdiag_index(a, b)][rl4 * BP + cl] = static_cast<_Float16>(ak * sk * sk);
            sm.aqk[a * (a + 1) / 2 + b][rl4 * BP + cl] = static_cast<_Float16>(vq * sk * sq);
        }
        for (int pr = tid; pr < 4 * 256; pr += NT) {  // upper halves of the diagonal blocks
            const int a = pr >> 8, rl4 = (pr >> 4) & 15, cl = pr & 15;
            if (cl > rl4) {
                sm.ad[a][rl4][cl] = 0.f;
                sm.aqk[a * (a + 1) / 2 + a][rl4 * BP + cl] = static_cast<_Float16>(0.f);
            }
        }
    }
    __syncthreads();  // (4) Gram results in LDS; operand area free

    // ============ a3: diagonal blocks of T; e^G k to LDS, Q and KT to the pack ============
    // the solve's v values, in accumulator layout, fetched ahead
    uint32_t vpre[2][4][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                vpre[t][a][jj] = ld16(rs_v, 2 * ((16 * a + 4 * g4 + jj) * tok_stride + 16 * (2 * wave + t) + n16));
    float tcol[16];
    if (wave == 0) {  // lane 16a + j owns column j of T_aa = (I + A_aa)^{-1}
        const int a = g4, j = n16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i + 1 < r; i += 2) {
                s0 -= sm.ad[a][r][i] * tcol[i];
                s1 -= sm.ad[a][r][i + 1] * tcol[i + 1];
            }
            if (r & 1) s0 -= sm.ad[a][r][r - 1] * tcol[r - 1];
            tcol[r] = s0 + s1;
        }
        float tm = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) tm = fmaxf(tm, fabsf(tcol[r]));
        tm = wave_max(tm);
        if (lane == 0) sm.imax[4] = __float_as_int(tm);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        // Q: the channel pair (hh HC + 2cq, +1) of row r is 4 bytes of 16-byte unit hh*8 + cq/4
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int r = 8 * rq8 + m;
            *reinterpret_cast<uint32_t *>(&sm.op.s.ek[r * KP + hh * HC + 2 * cq]) = ekp[hh][m];
            st32(rs_p, qsp[hh][m], kPkQ + swz_w(r, hh * 8 + (cq >> 2)) + 4 * (cq & 3));
        }
        // KT: eight consecutive rows of one channel are one 16-byte unit
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const u4 w = {kdp[hh][e][0], kdp[hh][e][1], kdp[hh][e][2], kdp[hh][e][3]};
            st128(rs_p, w, kPkKT + swz_kt(hh * HC + 2 * cq + e, rq8));
        }
    }
    __syncthreads();  // (5)
    const int et = exp_of(__int_as_float(sm.imax[4]));
    if (wave == 0) {
        const float st = pow2(-et);
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.tinv[g4][r * BP + n16] = static_cast<_Float16>(tcol[r] * st);
    }
    __syncthreads();  // (6)

    // ============ a4: W = T beta (e^G k) and U = T beta v by the blocked forward solve ============
    // wave w: column tiles 2w, 2w + 1 of both.  W is formed in the 2^-ek
    // frame of the stored e^G k, U in the 2^-ev frame.  Per row block a:
    //   Y_a = X_a - sum_{b<a} A_ab V_b,  V_a = T_aa Y_a.
    const float uns = pow2(2 * ek), unt = pow2(et);
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
                    const h4 aab = *reinterpret_cast<const h4 *>(&sm.akk[offdiag_index(a, b)][n16 * BP + 4 * g4]);
                    accs = mma16(aab, Vh[b], accs);
                }
                f4 yv;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) yv[jj] = xp[jj] - accs[jj] * uns;
                const h4 ta = *reinterpret_cast<const h4 *>(&sm.tinv[a][n16 * BP + 4 * g4]);
                f4 va = mma16(ta, to_h4(yv, 1.f), zero4());
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) va[jj] *= unt;
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
    mw = wave_max(mw);
    mu = wave_max(mu);
    if (lane == 0) {
        atomicMax(&sm.imax[6], __float_as_int(mw));
        atomicMax(&sm.imax[7], __float_as_int(mu));
    }
    __syncthreads();  // (7) all reads of e^G k done; its area takes W
    const int ew = exp_of(__int_as_float(sm.imax[6])), eu = exp_of(__int_as_float(sm.imax[7]));
    {
        const float swv = pow2(-ew), suv = pow2(-eu);
        char *wst = reinterpret_cast<char *>(sm.op.s.ek);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ct = 2 * wave + t, col = 16 * ct + n16;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rr = 16 * a + 4 * g4 + jj;
                    *reinterpret_cast<_Float16 *>(wst + swz_w(rr, col >> 3) + 2 * (col & 7)) =
                        static_cast<_Float16>(Wr[t][a][jj] * swv);
                }
                // U straight to the pack, in accumulator order
                const h4 uh = to_h4(Ur[t][a], suv);
                st64(rs_p, __builtin_bit_cast(u2, uh), kPkU + u_off(ct, a, lane));
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
        for (int u = tid; u < 10 * 16 * 2; u += NT) {  // A_qk blocks, rows of 32 bytes
            // 16-byte half `half` of a stored row holds the row's logical half
            // half ^ (row >= 8) (the 8-byte units of a_off, pairwise)
            const int p = u >> 5, row = (u >> 1) & 15, half = u & 1, lh = half ^ (row >> 3);
            st128(rs_p, *reinterpret_cast<const u4 *>(&sm.aqk[p][row * BP + 8 * lh]), kPkA + 16 * u);
        }
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

}  // namespace
}  // namespace mc

bool f16_path_supported(bool in_bf16, int dk, int dv, int chunk) {
    return in_bf16 && dk == mc::DK && dv == mc::DV && chunk == mc::C;
}

size_t pack_bytes() { return mc::kPkBytes; }

void launch_prep(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, void *packs) {
    dim3 grid(max_segs * per, L.H), block(mc::NT);
    hipLaunchKernelGGL(mc::chunk_prep_kernel, grid, block, 0, L.stream, static_cast<const uint16_t *>(L.q),
                       static_cast<const uint16_t *>(L.k), static_cast<const uint16_t *>(L.v), L.g,
                       static_cast<const uint16_t *>(L.beta), sv, per, L.H, L.scale, static_cast<char *>(packs));
}

}  // namespace kda
