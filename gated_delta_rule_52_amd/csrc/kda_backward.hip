// kda_backward.hip - gradients of the KDA recurrence for gfx950, token by token.
//
// Reverse-mode differentiation of the recurrence of the Kimi Linear review
// notes (section "Method", the KDA recurrence in read-then-write form):
// S~ = Diag(alpha) S_{t-1}, u = v - S~^T k, S_t = S~ + beta k u^T,
// o_t = scale S_t^T q.  Walking the tokens backwards with dS, the gradient of
// the state that leaves token t (the final-state gradient before the last
// token):
//
//     dS += scale q do^T              dq = scale S_t do = scale (S~ do + beta k (u . do))
//     w   = dS^T k,  du = beta w      dv = du,  dbeta = w . u
//     dk  = beta dS u - S~ du
//     dS~ = dS - k du^T               dg = rowsum(S~ .* dS~)   (alpha = exp(g))
//     dS  = Diag(alpha) dS~           the gradient entering token t
//
// and the initial-state gradient is the dS left after the first token.
//
// Each step needs S_{t-1}.  The forward states are not kept: a forward sweep
// stores every kBlock-th state in the workspace, and the backward sweep
// rebuilds the states of each block of kBlock tokens from its stored state,
// kSub at a time held in registers (the later sub-block first).
//
// One workgroup per (sequence, head), one wave per 16-column slice of dv.
// The columns of S, and of dS, evolve independently, so each wave runs both
// sweeps on its slice alone and only meets the others at block boundaries.
// dq, dk, dg and dbeta are sums over all dv columns: each wave folds its 16
// columns with cross-lane swaps, and the workgroup adds the slices through LDS
// in a fixed order, so results are deterministic.
//
// Lane (c = lane / 4, rg = lane % 4) of a wave holds column c of its slice,
// rows rg R .. rg R + R - 1 (R = dk / 4) of the state and of its gradient.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kBlock = 8;  // tokens per stored state
constexpr int kSub = 3;    // states held in registers at once

// Pair sums over lanes (l, l ^ 32) for two values at once: one lane of each
// pair receives lo + lo', the other hi + hi'.  Which one gets which follows
// the swap instruction and is read at run time (fold32(0, 1) > 1 in the lanes
// left holding hi).
__device__ __forceinline__ float fold32(float lo, float hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same over lanes (l, l ^ 16).
__device__ __forceinline__ float fold16(float lo, float hi) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Over lanes (l, l ^ 8): lanes with bit 3 clear keep lo.
__device__ __forceinline__ float fold8(float lo, float hi, bool b3) {
    const float send = b3 ? lo : hi, keep = b3 ? hi : lo;
    return keep + dpp_mov<0x128>(send);  // row_ror:8, i.e. lane ^ 8 within a row of 16
}
// Over lanes (l, l ^ 4): lanes with bit 2 clear keep lo.
__device__ __forceinline__ float fold4(float lo, float hi, bool b2) {
    const float send = b2 ? lo : hi, keep = b2 ? hi : lo;
    // swizzle bitmask mode: and 0x1f, or 0, xor 4
    return keep + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(send), 0x101F));
}
// Sum over the 16 columns of a slice (lane bits 2..5), left in every lane.
__device__ __forceinline__ float column_total(float x) {
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
    x += dpp_mov<0x128>(x);
    x = fold16(x, x);
    return fold32(x, x);
}

__device__ __forceinline__ float4 lds4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// One forward step of this lane's R rows of one state column, X -> X~ + b k (v - X~^T k), X~ = Diag(alpha) X,
// with kx, ax the lane's rows of k and alpha in LDS.  The LDS reads are software-pipelined by hand: each
// group of four rows issues the next group's reads before its own arithmetic, and a scheduling fence
// keeps the compiler from hoisting every read to the top (which would cost 2 R registers).
template <int R>
__device__ __forceinline__ void advance_rows(float (&s)[R], const float *kx, const float *ax, float v, float b) {
    float p0 = 0.f, p1 = 0.f;
    float4 kc = lds4(kx), ac = lds4(ax);
#pragma unroll
    for (int i = 0; i < R; i += 4) {
        __builtin_amdgcn_sched_barrier(0);
        float4 kn = kc, an = ac;
        if (i + 4 < R) {
            kn = lds4(kx + i + 4);
            an = lds4(ax + i + 4);
        }
        s[i] *= ac.x; s[i + 1] *= ac.y; s[i + 2] *= ac.z; s[i + 3] *= ac.w;
        p0 += s[i] * kc.x;
        p1 += s[i + 1] * kc.y;
        p0 += s[i + 2] * kc.z;
        p1 += s[i + 3] * kc.w;
        kc = kn;
        ac = an;
    }
    kc = lds4(kx);  // k is read again rather than held: registers are scarce
    const float bd = b * (v - quad_sum(p0 + p1));
#pragma unroll
    for (int i = 0; i < R; i += 4) {
        __builtin_amdgcn_sched_barrier(0);
        float4 kn = kc;
        if (i + 4 < R) kn = lds4(kx + i + 4);
        s[i] += bd * kc.x; s[i + 1] += bd * kc.y; s[i + 2] += bd * kc.z; s[i + 3] += bd * kc.w;
        kc = kn;
    }
}

}  // namespace

// Token-by-token gradients of one segment per workgroup (a sequence, or a piece of one): the forward
// state entering the segment comes from the segmented forward (or is the initial state), the gradient
// of the state leaving it from the reverse combine (or is the final-state gradient).
template <int DK, int DV, bool InBf16>
__global__ void __launch_bounds__(DV / 16 * kWave)
recurrent_bwd_kernel(BackwardLaunch L, SegmentView sv, const float *dleave) {
    using In = Elem<InBf16>;
    using IT = typename In::T;
    constexpr int NS = DV / 16;   // waves, one per 16-column slice
    constexpr int NT = NS * kWave;
    constexpr int R = DK / 4;     // state rows per lane
    constexpr int KEEP = R / 16;  // rows of each row sum a lane holds after folding its slice
    constexpr int RP = R + 4;     // LDS stride of a row group: the four groups a quad reads fall in distinct banks
    static_assert(R % 16 == 0, "dk must be a multiple of 64");
    const IT *q = static_cast<const IT *>(L.q), *k = static_cast<const IT *>(L.k);
    const IT *v = static_cast<const IT *>(L.v), *beta = static_cast<const IT *>(L.beta);
    const IT *d_o = static_cast<const IT *>(L.d_o);
    const float *g = L.g;
    // grid.x = segment * H + head: a packed batch may hold more than grid.y's 65,535 segments
    const int H = L.H, h = static_cast<int>(blockIdx.x % H), seg = static_cast<int>(blockIdx.x / H);
    if (seg >= sv.count()) return;
    const int4 sd = sv.desc(seg);
    const int n = sd.x;
    const int64_t t0 = sd.y, t1 = sd.z;
    const int tid = threadIdx.x, lane = tid % kWave, slice = tid / kWave;
    const int c = lane >> 2, rg = lane & 3, col = 16 * slice + c;
    const int nb = static_cast<int>((t1 - t0 + kBlock - 1) / kBlock);
    // stored states: segment seg's block b sits in slot t0 / kBlock + seg + b (slots of different
    // segments never meet); inside a slot, each wave's slice is lane-contiguous
    const int64_t slot0 = t0 / kBlock + seg;
    const int64_t nbase = (static_cast<int64_t>(n) * H + h) * DK * DV;
    const bool one = (sd.w & (kSegFirst | kSegLast)) == (kSegFirst | kSegLast);
    // A sequence of one segment reads the final-state gradient in place (this workgroup then writes the
    // initial-state gradient, which may alias it); longer ones read the reverse combine's copy.
    const float *dS_end = one ? (L.dhT ? L.dhT + nbase : nullptr)
                              : dleave + (static_cast<int64_t>(seg) * H + h) * DK * DV;
    float *dS_begin = (sd.w & kSegFirst) && L.dh0 ? L.dh0 + nbase : nullptr;
    auto stored = [&](int b) { return L.ckpt + (((slot0 + b) * H + h) * NS + slice) * (R * kWave) + lane; };

    // which half each lane keeps in the first two folds, and the first row of its folded sums
    const bool hi32 = fold32(0.f, 1.f) > 1.f, hi16 = fold16(0.f, 1.f) > 1.f;
    const bool b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1;
    const int row_kept = rg * R + (hi32 ? R / 2 : 0) + (hi16 ? R / 4 : 0) + (b3 ? R / 8 : 0) + (b2 ? R / 16 : 0);

    // k, q, alpha of the staged tokens; channel rg R + r at rg RP + r
    __shared__ __attribute__((aligned(16))) float s_k[kBlock][4 * RP];
    __shared__ __attribute__((aligned(16))) float s_q[kBlock][4 * RP];
    __shared__ __attribute__((aligned(16))) float s_a[kBlock][4 * RP];
    __shared__ float s_v[kBlock][DV], s_do[kBlock][DV], s_b[kBlock];
    __shared__ __attribute__((aligned(16))) float s_part[kBlock][NS][3][DK];  // row sums per slice
    __shared__ float s_ps[kBlock][NS][2];  // per slice: sum_c u_c w_c (dbeta) and sum_c u_c scale do_c

    // this lane's part of a [dk, dv] state; null reads as zero
    auto load_slice = [&](float (&s)[R], const float *src) {
        if (src) {
            const float *p = src + static_cast<int64_t>(rg * R) * DV + col;
#pragma unroll
            for (int i = 0; i < R; ++i) s[i] = p[i * DV];
        } else {
#pragma unroll
            for (int i = 0; i < R; ++i) s[i] = 0.f;
        }
    };

    // tokens [tb, tb + m) of the sequence into LDS, all threads
    auto stage = [&](int64_t tb, int m, bool backward) {
        for (int e = tid; e < m * DK; e += NT) {
            const int x = e / DK, i = e % DK, li = (i / R) * RP + i % R;
            const int64_t idx = ((tb + x) * H + h) * DK + i;
            s_k[x][li] = In::load(k, idx);
            s_a[x][li] = __expf(g[L.scalar_gate ? (tb + x) * H + h : idx]);
            if (backward) s_q[x][li] = In::load(q, idx);
        }
        for (int e = tid; e < m * DV; e += NT) {
            const int x = e / DV, j = e % DV;
            const int64_t idx = ((tb + x) * H + h) * static_cast<int64_t>(DV) + j;
            s_v[x][j] = In::load(v, idx);
            if (backward) s_do[x][j] = In::load(d_o, idx);
        }
        if (tid < m) s_b[tid] = In::load(beta, (tb + tid) * H + h);
    };

    // s = S_{t-1} -> S_t for staged token x
    auto advance = [&](float (&s)[R], int x) {
        advance_rows<R>(s, &s_k[x][rg * RP], &s_a[x][rg * RP], s_v[x][col], s_b[x]);
    };

    float ds[R];  // gradient of the state leaving the token being processed

    // one backward step for staged token x (sequence position t), sp = S_{t-1} (overwritten)
    auto back = [&](float (&sp)[R], int x, int64_t t) {
        const float dos = L.scale * s_do[x][col], bt = s_b[x];
        float p0 = 0.f, p1 = 0.f, w0 = 0.f, w1 = 0.f;
        const float *kx = &s_k[x][rg * RP], *qx = &s_q[x][rg * RP], *ax = &s_a[x][rg * RP];
        float4 kc = lds4(kx), qc = lds4(qx), ac = lds4(ax);
#pragma unroll
        for (int i = 0; i < R; i += 4) {
            __builtin_amdgcn_sched_barrier(0);
            float4 kn = kc, qn = qc, an = ac;
            if (i + 4 < R) {
                kn = lds4(kx + i + 4);
                qn = lds4(qx + i + 4);
                an = lds4(ax + i + 4);
            }
            const float kk[4] = {kc.x, kc.y, kc.z, kc.w}, qq[4] = {qc.x, qc.y, qc.z, qc.w};
            const float aa[4] = {ac.x, ac.y, ac.z, ac.w};
            kc = kn;
            qc = qn;
            ac = an;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sp[i + e] *= aa[e];  // S~
                ds[i + e] += qq[e] * dos;  // dS of S_t, with the output's term
                if (e & 1) {
                    p1 += sp[i + e] * kk[e];
                    w1 += ds[i + e] * kk[e];
                } else {
                    p0 += sp[i + e] * kk[e];
                    w0 += ds[i + e] * kk[e];
                }
            }
        }
        const float u = s_v[x][col] - quad_sum(p0 + p1);
        const float wc = quad_sum(w0 + w1);
        const float du = bt * wc, bu = bt * u;
        // The per-row terms of dq, dk and dg, summed over the slice's 16 columns by a tree of folds.
        // The lane's i-th output (i < KEEP) collects rows i + KEEP (m0 + 2 m1) + (R/4) m2 and the same
        // rows + R/2: fold32 joins the +R/2 pairs, fold16 the m2 pairs, fold8 m1, fold4 m0.  Rows are
        // visited so that every fold runs as soon as both of its inputs exist.
        auto row_terms = [&](int r, float kr, float ar, float (&o)[3]) {
            o[0] = sp[r] * dos;                 // S~ do (beta k (u . do) is added over all slices)
            o[1] = bu * ds[r] - du * sp[r];     // beta dS u - S~ du
            const float dst = ds[r] - kr * du;  // dS~
            o[2] = sp[r] * dst;                 // S~ .* dS~
            ds[r] = ar * dst;
        };
        auto ld_keep = [&](const float *p, float (&o)[KEEP]) {  // KEEP consecutive rows
            if constexpr (KEEP == 2) {
                const float2 w = *reinterpret_cast<const float2 *>(p);
                o[0] = w.x;
                o[1] = w.y;
            } else {
#pragma unroll
                for (int i = 0; i < KEEP; ++i) o[i] = p[i];
            }
        };
        float e[2][2][3][KEEP];  // [m0][m1][quantity][i]
        float hf[2][3][KEEP];    // [m0][quantity][i]
        // k and alpha of one quarter of the rows: [m2][low, high half][i]
        auto ld_quarter = [&](int mp, float (&kq)[2][2][KEEP], float (&aq)[2][2][KEEP]) {
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int r = KEEP * mp + m2 * (R / 4) + hh * (R / 2);
                    ld_keep(kx + r, kq[m2][hh]);
                    ld_keep(ax + r, aq[m2][hh]);
                }
        };
        float kq[2][2][KEEP], aq[2][2][KEEP];
        ld_quarter(0, kq, aq);
#pragma unroll
        for (int oi = 0; oi < 4; ++oi) {
            __builtin_amdgcn_sched_barrier(0);
            const int mp = (oi >> 1) | ((oi & 1) << 1);  // m0 + 2 m1 in the order 0, 2, 1, 3
            const int m0 = mp & 1, m1 = mp >> 1;
            float kqc[2][2][KEEP], aqc[2][2][KEEP];
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int i = 0; i < KEEP; ++i) {
                        kqc[m2][hh][i] = kq[m2][hh][i];
                        aqc[m2][hh][i] = aq[m2][hh][i];
                    }
            if (oi < 3) ld_quarter(((oi + 1) >> 1) | (((oi + 1) & 1) << 1), kq, aq);
            float f[2][3][KEEP];
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                const int r = KEEP * mp + m2 * (R / 4);
                const float (&kl)[KEEP] = kqc[m2][0], (&al)[KEEP] = aqc[m2][0];
                const float (&kh)[KEEP] = kqc[m2][1], (&ah)[KEEP] = aqc[m2][1];
#pragma unroll
                for (int i = 0; i < KEEP; ++i) {
                    float lo[3], hi[3];
                    row_terms(r + i, kl[i], al[i], lo);
                    row_terms(r + i + R / 2, kh[i], ah[i], hi);
#pragma unroll
                    for (int qn = 0; qn < 3; ++qn) f[m2][qn][i] = fold32(lo[qn], hi[qn]);
                }
            }
#pragma unroll
            for (int qn = 0; qn < 3; ++qn)
#pragma unroll
                for (int i = 0; i < KEEP; ++i) e[m0][m1][qn][i] = fold16(f[0][qn][i], f[1][qn][i]);
            if (m1 == 1) {
#pragma unroll
                for (int qn = 0; qn < 3; ++qn)
#pragma unroll
                    for (int i = 0; i < KEEP; ++i) hf[m0][qn][i] = fold8(e[m0][0][qn][i], e[m0][1][qn][i], b3);
            }
        }
#pragma unroll
        for (int qn = 0; qn < 3; ++qn)
#pragma unroll
            for (int i = 0; i < KEEP; ++i) s_part[x][slice][qn][row_kept + i] = fold4(hf[0][qn][i], hf[1][qn][i], b2);
        if (rg == 0) L.dv[(t * H + h) * static_cast<int64_t>(DV) + col] = du;
        const float db = column_total(u * wc), ud = column_total(u * dos);
        if (lane == 0) {
            s_ps[x][slice][0] = db;
            s_ps[x][slice][1] = ud;
        }
    };

    // the slices' partial sums of staged tokens [0, m) -> dq, dk, dg, dbeta
    auto reduce = [&](int64_t tb, int m) {
        constexpr int V4 = DK / 4;
        for (int e = tid; e < m * 3 * V4; e += NT) {
            const int x = e / (3 * V4), r = e % (3 * V4), qty = r / V4, i = (r % V4) * 4;
            float4 acc = lds4(&s_part[x][0][qty][i]);
#pragma unroll
            for (int sl = 1; sl < NS; ++sl) {
                const float4 p = lds4(&s_part[x][sl][qty][i]);
                acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
            }
            if (qty == 0) {  // dq = scale (S~ do + beta k (u . do))
                float ud = 0.f;
#pragma unroll
                for (int sl = 0; sl < NS; ++sl) ud += s_ps[x][sl][1];
                const float4 k4 = lds4(&s_k[x][(i / R) * RP + i % R]);
                const float bud = s_b[x] * ud;
                acc.x += bud * k4.x; acc.y += bud * k4.y; acc.z += bud * k4.z; acc.w += bud * k4.w;
            }
            if (qty == 2 && L.scalar_gate) {  // kept for the sum over rows below (this thread's own slot)
                *reinterpret_cast<float4 *>(&s_part[x][0][2][i]) = acc;
                continue;
            }
            float *dst = qty == 0 ? L.dq : (qty == 1 ? L.dk : L.dg);
            *reinterpret_cast<float4 *>(dst + ((tb + x) * H + h) * DK + i) = acc;
        }
        if (tid < m) {
            float acc = 0.f;
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) acc += s_ps[tid][sl][0];
            L.dbeta[(tb + tid) * H + h] = acc;
        }
        if (L.scalar_gate) {  // one gate per token and head: its gradient is the sum over the dk rows
            __syncthreads();
            if (tid < m) {
                float acc = 0.f;
                for (int i = 0; i < DK; ++i) acc += s_part[tid][0][2][i];
                L.dg[(tb + tid) * H + h] = acc;
            }
        }
    };

    // forward sweep: the state entering every block.  Only whole blocks are swept (the last block, the
    // only one that may be short, is not), and the next block's inputs are fetched into registers while
    // the current one runs.
    constexpr int KPT = kBlock * DK / NT, VPT = kBlock * DV / NT;  // elements per thread and block
    static_assert(KPT * NT == kBlock * DK && VPT * NT == kBlock * DV, "staging split");
    struct Ahead {
        float k[KPT], g[KPT], v[VPT], b;
    } ahead;
    auto fetch_block = [&](int64_t tb) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int e = tid + j * NT;
            const int64_t idx = ((tb + e / DK) * H + h) * DK + e % DK;
            ahead.k[j] = In::load(k, idx);
            ahead.g[j] = g[L.scalar_gate ? (tb + e / DK) * H + h : idx];
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int e = tid + j * NT;
            ahead.v[j] = In::load(v, ((tb + e / DV) * H + h) * static_cast<int64_t>(DV) + e % DV);
        }
        if (tid < kBlock) ahead.b = In::load(beta, (tb + tid) * H + h);
    };
    auto put_block = [&]() {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int e = tid + j * NT, i = e % DK;
            s_k[e / DK][(i / R) * RP + i % R] = ahead.k[j];
            s_a[e / DK][(i / R) * RP + i % R] = __expf(ahead.g[j]);
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int e = tid + j * NT;
            s_v[e / DV][e % DV] = ahead.v[j];
        }
        if (tid < kBlock) s_b[tid] = ahead.b;
    };
    float st[kSub][R];
    load_slice(st[0], sv.entering(seg, sd, h, H, DK, DV));
    if (nb > 1) fetch_block(t0);
    for (int b = 0; b < nb; ++b) {
        float *cp = stored(b);
#pragma unroll
        for (int i = 0; i < R; ++i) cp[i * kWave] = st[0][i];
        if (b == nb - 1) break;
        __syncthreads();  // the previous block's tokens have been read
        put_block();
        if (b + 2 < nb) fetch_block(t0 + static_cast<int64_t>(b + 1) * kBlock);
        __syncthreads();
        for (int x = 0; x < kBlock; ++x) advance(st[0], x);
    }

    // backward sweep
    load_slice(ds, dS_end);
    for (int b = nb - 1; b >= 0; --b) {
        const int64_t tb = t0 + static_cast<int64_t>(b) * kBlock;
        const int m = static_cast<int>(t1 - tb < kBlock ? t1 - tb : kBlock);
        __syncthreads();  // the previous block's tokens and partial sums have been read
        stage(tb, m, true);
        __syncthreads();
        const float *cp = stored(b);
        for (int sub = (m - 1) / kSub; sub >= 0; --sub) {
            const int xb = sub * kSub, ms = m - xb < kSub ? m - xb : kSub;
#pragma unroll
            for (int i = 0; i < R; ++i) st[0][i] = cp[i * kWave];
            for (int x = 0; x < xb; ++x) advance(st[0], x);
            // st[j] = the state entering token xb + j
#pragma unroll
            for (int j = 1; j < kSub; ++j) {
                if (j < ms) {
#pragma unroll
                    for (int i = 0; i < R; ++i) st[j][i] = st[j - 1][i];
                    advance(st[j], xb + j - 1);
                }
            }
#pragma unroll
            for (int j = kSub - 1; j >= 0; --j)
                if (j < ms) back(st[j], xb + j, tb + xb + j);
        }
        __syncthreads();
        reduce(tb, m);
    }
    if (dS_begin) {
        float *p = dS_begin + static_cast<int64_t>(rg * R) * DV + col;
#pragma unroll
        for (int i = 0; i < R; ++i) p[i * DV] = ds[i];
    }
}

// The segmented forward's local pass, token by token in fp32, for every segment of a sequence of several:
// H from a zero state with the segment's tokens, and the columns of the transition P (dk x dk) from the
// identity with v = 0, both by one forward step per token.  One wave per 16 columns of [H | P].
template <int DK, int DV, bool InBf16, int NT>
__device__ __forceinline__ void segment_local_body(const BackwardLaunch &L, const SegmentView &sv) {
    using In = Elem<InBf16>;
    using IT = typename In::T;
    constexpr int R = DK / 4, RP = R + 4;
    static_assert(NT == (DV + DK) / 16 * kWave, "one wave per 16 columns of [H | P]");
    const IT *k = static_cast<const IT *>(L.k), *v = static_cast<const IT *>(L.v);
    const IT *beta = static_cast<const IT *>(L.beta);
    // grid.x = segment * H + head: a packed batch may hold more than grid.y's 65,535 segments
    const int H = L.H, h = static_cast<int>(blockIdx.x % H), seg = static_cast<int>(blockIdx.x / H);
    if (seg >= sv.count()) return;
    const int4 sd = sv.desc(seg);
    if ((sd.w & (kSegFirst | kSegLast)) == (kSegFirst | kSegLast)) return;  // one segment: nothing to chain
    const int64_t t0 = sd.y, t1 = sd.z;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int rg = lane & 3;
    const bool pcol = wave >= DV / 16;
    const int col = (pcol ? wave - DV / 16 : wave) * 16 + (lane >> 2);  // column of P, or of H
    __shared__ __attribute__((aligned(16))) float s_k[kBlock][4 * RP];
    __shared__ __attribute__((aligned(16))) float s_a[kBlock][4 * RP];
    __shared__ float s_v[kBlock][DV], s_b[kBlock];
    float s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = pcol && rg * R + i == col ? 1.f : 0.f;
    const int nb = static_cast<int>((t1 - t0 + kBlock - 1) / kBlock);
    for (int b = 0; b < nb; ++b) {
        const int64_t tb = t0 + static_cast<int64_t>(b) * kBlock;
        const int m = static_cast<int>(t1 - tb < kBlock ? t1 - tb : kBlock);
        __syncthreads();
        for (int e = tid; e < m * DK; e += NT) {
            const int x = e / DK, i = e % DK, li = (i / R) * RP + i % R;
            const int64_t idx = ((tb + x) * H + h) * DK + i;
            s_k[x][li] = In::load(k, idx);
            s_a[x][li] = __expf(L.g[L.scalar_gate ? (tb + x) * H + h : idx]);
        }
        for (int e = tid; e < m * DV; e += NT) {
            const int x = e / DV, j = e % DV;
            s_v[x][j] = In::load(v, ((tb + x) * H + h) * static_cast<int64_t>(DV) + j);
        }
        if (tid < m) s_b[tid] = In::load(beta, (tb + tid) * H + h);
        __syncthreads();
        for (int x = 0; x < m; ++x)
            advance_rows<R>(s, &s_k[x][rg * RP], &s_a[x][rg * RP], pcol ? 0.f : s_v[x][col], s_b[x]);
    }
    float *dst = pcol ? sv.P + (static_cast<int64_t>(seg) * H + h) * DK * DK + static_cast<int64_t>(rg * R) * DK + col
                      : sv.Hs + (static_cast<int64_t>(seg) * H + h) * DK * DV + static_cast<int64_t>(rg * R) * DV + col;
    const int ld = pcol ? DK : DV;
#pragma unroll
    for (int i = 0; i < R; ++i) dst[i * ld] = s[i];
}

// The gradient of the state entering a segment, from a zero gradient at its end (the part of dS that
// the segment's own output gradients contribute): walking its tokens backwards,
//     dS += scale q do^T;   dS <- Diag(alpha) (I - beta k k^T) dS,
// which needs no forward state.  Segments that are not the first of their sequence only.  The first
// dv / 16 waves of the NT threads each carry 16 columns; all NT threads stage the tokens.
template <int DK, int DV, bool InBf16, int NT>
__device__ __forceinline__ void reverse_local_body(const BackwardLaunch &L, const SegmentView &sv, float *hb) {
    using In = Elem<InBf16>;
    using IT = typename In::T;
    constexpr int NS = DV / 16, R = DK / 4, RP = R + 4;
    static_assert(NT >= NS * kWave, "a wave per 16 columns of dv");
    const IT *q = static_cast<const IT *>(L.q), *k = static_cast<const IT *>(L.k);
    const IT *beta = static_cast<const IT *>(L.beta), *d_o = static_cast<const IT *>(L.d_o);
    // grid.x = segment * H + head: a packed batch may hold more than grid.y's 65,535 segments
    const int H = L.H, h = static_cast<int>(blockIdx.x % H), seg = static_cast<int>(blockIdx.x / H);
    if (seg >= sv.count()) return;
    const int4 sd = sv.desc(seg);
    if (sd.w & kSegFirst) return;
    const int64_t t0 = sd.y, t1 = sd.z;
    const int tid = threadIdx.x, lane = tid % kWave, slice = tid / kWave;
    const int rg = lane & 3, col = 16 * slice + (lane >> 2);
    __shared__ __attribute__((aligned(16))) float s_k[kBlock][4 * RP];
    __shared__ __attribute__((aligned(16))) float s_q[kBlock][4 * RP];
    __shared__ __attribute__((aligned(16))) float s_a[kBlock][4 * RP];
    __shared__ float s_do[kBlock][DV], s_b[kBlock];
    float ds[R];
#pragma unroll
    for (int i = 0; i < R; ++i) ds[i] = 0.f;
    const int nb = static_cast<int>((t1 - t0 + kBlock - 1) / kBlock);
    for (int b = nb - 1; b >= 0; --b) {
        const int64_t tb = t0 + static_cast<int64_t>(b) * kBlock;
        const int m = static_cast<int>(t1 - tb < kBlock ? t1 - tb : kBlock);
        __syncthreads();
        for (int e = tid; e < m * DK; e += NT) {
            const int x = e / DK, i = e % DK, li = (i / R) * RP + i % R;
            const int64_t idx = ((tb + x) * H + h) * DK + i;
            s_k[x][li] = In::load(k, idx);
            s_q[x][li] = In::load(q, idx);
            s_a[x][li] = __expf(L.g[L.scalar_gate ? (tb + x) * H + h : idx]);
        }
        for (int e = tid; e < m * DV; e += NT) {
            const int x = e / DV, j = e % DV;
            s_do[x][j] = In::load(d_o, ((tb + x) * H + h) * static_cast<int64_t>(DV) + j);
        }
        if (tid < m) s_b[tid] = In::load(beta, (tb + tid) * H + h);
        __syncthreads();
        if (slice >= NS) continue;  // staging only
        for (int x = m - 1; x >= 0; --x) {
            const float *kx = &s_k[x][rg * RP], *qx = &s_q[x][rg * RP], *ax = &s_a[x][rg * RP];
            const float dos = L.scale * s_do[x][col];
            float w0 = 0.f, w1 = 0.f;
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const float4 k4 = lds4(kx + i), q4 = lds4(qx + i);
                ds[i] += q4.x * dos; ds[i + 1] += q4.y * dos; ds[i + 2] += q4.z * dos; ds[i + 3] += q4.w * dos;
                w0 += ds[i] * k4.x;
                w1 += ds[i + 1] * k4.y;
                w0 += ds[i + 2] * k4.z;
                w1 += ds[i + 3] * k4.w;
            }
            const float bw = s_b[x] * quad_sum(w0 + w1);
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const float4 k4 = lds4(kx + i), a4 = lds4(ax + i);
                ds[i] = a4.x * (ds[i] - k4.x * bw);
                ds[i + 1] = a4.y * (ds[i + 1] - k4.y * bw);
                ds[i + 2] = a4.z * (ds[i + 2] - k4.z * bw);
                ds[i + 3] = a4.w * (ds[i + 3] - k4.w * bw);
            }
        }
    }
    if (slice >= NS) return;
    float *dst = hb + (static_cast<int64_t>(seg) * H + h) * DK * DV + static_cast<int64_t>(rg * R) * DV + col;
#pragma unroll
    for (int i = 0; i < R; ++i) dst[i * DV] = ds[i];
}

// Both local passes in one launch (blockIdx.z: 0 the forward one, 1 the reverse one): the reverse
// workgroups fill the CUs the forward ones leave and the tail of one pass overlaps the other.  At
// dk = dv = 128 a workgroup holds a CU alone (111 VGPRs for 16 waves); capping the registers so that two
// fit spills, and is slower.
template <int DK, int DV, bool InBf16>
__global__ void __launch_bounds__((DV + DK) / 16 * kWave)
local_passes_kernel(BackwardLaunch L, SegmentView sv, float *hb) {
    constexpr int NT = (DV + DK) / 16 * kWave;
    if (blockIdx.z == 0) segment_local_body<DK, DV, InBf16, NT>(L, sv);
    else reverse_local_body<DK, DV, InBf16, NT>(L, sv, hb);
}

// Reverse combine: per (sequence, head, 16-column slice of dv), from the final-state gradient, walk the
// segments backwards storing the gradient of each segment's leaving state and carrying
//     dS_enter(s) = P_s^T dS_leave(s) + Hb_s,      dS_leave(s - 1) = dS_enter(s)
// (P_s the segment's forward transition, Hb_s from the reverse local pass).  Sequences of one segment
// are left to the token kernel; an empty one gets its initial-state gradient here (the final-state
// gradient itself).  fp32 FMA, P_s staged in LDS.
template <int DK>
__global__ void __launch_bounds__(256)
reverse_combine_kernel(SegmentView sv, const float *hb, const float *dhT, float *dleave, float *dh0, int H, int DV) {
    constexpr int BV = 16, DKP = DK + 1, RG = 256 / BV, ROWS = DK / RG, PV4 = DK * DK / 4 / 256;
    __shared__ float sP[DK * DKP];
    __shared__ float sS[DK * BV];
    int slice, h, n;
    slice_head_seq(slice, h, n);
    const int tid = threadIdx.x, j = tid % BV, ig = tid / BV, j0 = slice * BV;
    const int first = sv.first_seg(n), end = sv.first_seg(n + 1);
    if (end - first == 1) return;
    const int64_t nbase = (static_cast<int64_t>(n) * H + h) * DK * DV;
    float x[ROWS];
#pragma unroll
    for (int u = 0; u < ROWS; ++u)
        x[u] = dhT ? dhT[nbase + static_cast<int64_t>(ig + RG * u) * DV + j0 + j] : 0.f;
    if (first >= end) {
        if (dh0)
#pragma unroll
            for (int u = 0; u < ROWS; ++u) dh0[nbase + static_cast<int64_t>(ig + RG * u) * DV + j0 + j] = x[u];
        return;
    }
    for (int seg = end - 1;; --seg) {
        float *dl = dleave + (static_cast<int64_t>(seg) * H + h) * DK * DV;
#pragma unroll
        for (int u = 0; u < ROWS; ++u) dl[static_cast<int64_t>(ig + RG * u) * DV + j0 + j] = x[u];
        if (seg == first) break;
        __syncthreads();  // the previous product has finished with sP and sS
        const float4 *src = reinterpret_cast<const float4 *>(sv.P + (static_cast<int64_t>(seg) * H + h) * DK * DK);
#pragma unroll
        for (int mm = 0; mm < PV4; ++mm) {
            const float4 pv = src[tid + 256 * mm];
            const int e = 4 * (tid + 256 * mm), r = e / DK, cc = e % DK;
            sP[r * DKP + cc] = pv.x;
            sP[r * DKP + cc + 1] = pv.y;
            sP[r * DKP + cc + 2] = pv.z;
            sP[r * DKP + cc + 3] = pv.w;
        }
#pragma unroll
        for (int u = 0; u < ROWS; ++u) sS[(ig + RG * u) * BV + j] = x[u];
        __syncthreads();
        const float *hs = hb + (static_cast<int64_t>(seg) * H + h) * DK * DV;
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int i = ig + RG * u;
            float a0 = 0.f, a1 = 0.f;
            for (int m = 0; m < DK; m += 2) {  // (P^T x)[i] = sum_m P[m][i] x[m]
                a0 += sP[m * DKP + i] * sS[m * BV + j];
                a1 += sP[(m + 1) * DKP + i] * sS[(m + 1) * BV + j];
            }
            x[u] = (a0 + a1) + hs[static_cast<int64_t>(i) * DV + j0 + j];
        }
    }
}

// With the input transforms the gradients run on transformed copies of the inputs: a prepare pass writes,
// per (token, head), the L2-normalised q and k and their inverse norms, the log-gates, and fp32 copies of v,
// beta and grad_o; the passes above then run unchanged in fp32; a finish pass carries dq, dk and dg back to
// the raw inputs by the chain rule (dx = (dx^ - x^ (x^ . dx^)) / r for q and k, dz = dloggate * (-s sigmoid(z))
// for the gate logits z), in place.
struct XformBufs {
    float *q, *k, *g, *v, *b, *d, *iq, *ik;
};

// one wave per (token, head) u = t H + h, four per workgroup
template <int DK, int DV, bool InBf16>
__global__ void __launch_bounds__(256)
bwd_prepare_kernel(BackwardLaunch L, XformBufs X, int64_t units) {
    using In = Elem<InBf16>;
    using IT = typename In::T;
    constexpr int CPL = DK / kWave;
    const int64_t u = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
    if (u >= units) return;
    const int lane = threadIdx.x % kWave;
    const IT *q = static_cast<const IT *>(L.q), *k = static_cast<const IT *>(L.k);
    float qv[CPL], kv[CPL], qq = 0.f, kk = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        const int64_t i = u * DK + lane * CPL + e;
        qv[e] = In::load(q, i);
        kv[e] = In::load(k, i);
        qq += qv[e] * qv[e];
        kk += kv[e] * kv[e];
    }
    float iq = 1.f, ik = 1.f;
    if (L.xf.qk_l2norm) {  // the forward kernels' normalisation: x rsqrt(sum x^2 + eps)
        iq = rsqrtf(wave_sum(qq) + kL2Eps);
        ik = rsqrtf(wave_sum(kk) + kL2Eps);
    }
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        const int64_t i = u * DK + lane * CPL + e;
        X.q[i] = qv[e] * iq;
        X.k[i] = kv[e] * ik;
        if (!L.scalar_gate) X.g[i] = L.xf.log_gate(L.g[i]);
    }
    if (lane == 0) {
        X.iq[u] = iq;
        X.ik[u] = ik;
        if (L.scalar_gate) X.g[u] = L.xf.log_gate(L.g[u]);
        X.b[u] = In::load(static_cast<const IT *>(L.beta), u);
    }
    for (int j = lane; j < DV; j += kWave) {
        X.v[u * DV + j] = In::load(static_cast<const IT *>(L.v), u * DV + j);
        X.d[u * DV + j] = In::load(static_cast<const IT *>(L.d_o), u * DV + j);
    }
}

template <int DK>
__global__ void __launch_bounds__(256)
bwd_finish_kernel(BackwardLaunch L, XformBufs X, int64_t units) {
    constexpr int CPL = DK / kWave;
    const int64_t u = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
    if (u >= units) return;
    const int lane = threadIdx.x % kWave;
    if (L.xf.qk_l2norm) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {  // dq, then dk
            float *dx = w == 0 ? L.dq : L.dk;
            const float *xh = w == 0 ? X.q : X.k;
            const float ir = w == 0 ? X.iq[u] : X.ik[u];
            float d[CPL], xv[CPL], p = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const int64_t i = u * DK + lane * CPL + e;
                d[e] = dx[i];
                xv[e] = xh[i];
                p += d[e] * xv[e];
            }
            p = wave_sum(p);
#pragma unroll
            for (int e = 0; e < CPL; ++e) dx[u * DK + lane * CPL + e] = (d[e] - xv[e] * p) * ir;
        }
    }
    if (L.xf.gate_softplus) {  // d/dz of -s softplus(z) = -s sigmoid(z)
        const float s = L.xf.gate_scale;
        if (L.scalar_gate) {
            if (lane == 0) L.dg[u] *= -s / (1.f + __expf(-L.g[u]));
        } else {
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const int64_t i = u * DK + lane * CPL + e;
                L.dg[i] *= -s / (1.f + __expf(-L.g[i]));
            }
        }
    }
}

namespace {

// workspace: [segment table, P, H, entering states] [dS_leave per segment] [Hb per segment] [stored states]
// [with input transforms: q^, k^, log-gates, v, beta, grad_o in fp32, inverse norms];
// (the reverse local pass writes Hb beside the forward's H: the two local passes run in one launch)
struct BwdPlan {
    size_t off_dl, off_hb, off_ckpt, off_x, bytes;
    int max_segs;
};

BwdPlan bwd_plan(int B, int T, int H, int dk, int dv, int N, bool varlen, bool transforms, bool scalar_gate) {
    BwdPlan p{};
    auto a256 = [](size_t x) { return (x + 255) & ~size_t{255}; };
    const size_t seg_bytes = segment_states_bytes(B, T, H, dk, dv, N, varlen, 64);
    // the same bound on segments as the segmented forward's plan: at most one more than tokens / 64 per
    // sequence, and at least one
    const int64_t tokens = varlen ? T : static_cast<int64_t>(B) * T;
    const size_t state = static_cast<size_t>(H) * dk * dv * sizeof(float);
    const size_t max_segs = static_cast<size_t>(tokens / 64 + N + 1);
    p.off_dl = a256(seg_bytes);
    p.off_hb = a256(p.off_dl + max_segs * state);
    p.off_ckpt = a256(p.off_hb + max_segs * state);
    p.off_x = a256(p.off_ckpt + static_cast<size_t>(tokens / kBlock + max_segs) * state);
    const size_t th = static_cast<size_t>(tokens) * H;
    p.bytes = p.off_x + (transforms ? th * (2 * dk + (scalar_gate ? 1 : dk) + 2 * dv + 3) * sizeof(float) : 0);
    return p;
}

XformBufs xform_bufs(char *base, size_t th, int dk, int dv, bool scalar_gate) {
    XformBufs X;
    float *f = reinterpret_cast<float *>(base);
    X.q = f; f += th * dk;
    X.k = f; f += th * dk;
    X.g = f; f += th * (scalar_gate ? 1 : dk);
    X.v = f; f += th * dv;
    X.d = f; f += th * dv;
    X.b = f; f += th;
    X.iq = f; f += th;
    X.ik = f;
    return X;
}

}  // namespace

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int N, bool varlen, bool transforms,
                                bool scalar_gate) {
    return bwd_plan(B, T, H, dk, dv, N, varlen, transforms, scalar_gate).bytes;
}

template <int DK, int DV>
static hipError_t launch_bwd(const BackwardLaunch &Lin) {
    const bool varlen = Lin.cu_seqlens != nullptr;
    const bool transforms = Lin.xf.qk_l2norm || Lin.xf.gate_softplus;
    const BwdPlan p = bwd_plan(Lin.B, Lin.T, Lin.H, DK, DV, Lin.N, varlen, transforms, Lin.scalar_gate);
    char *ws = static_cast<char *>(Lin.workspace);
    const int64_t units = (varlen ? static_cast<int64_t>(Lin.T) : static_cast<int64_t>(Lin.B) * Lin.T) * Lin.H;
    BackwardLaunch L = Lin;
    XformBufs X{};
    if (transforms) {  // run the passes on transformed fp32 copies
        X = xform_bufs(ws + p.off_x, static_cast<size_t>(units), DK, DV, Lin.scalar_gate);
        if (units > 0) {
            const dim3 grid(static_cast<unsigned>((units + 3) / 4));
            if (Lin.in_bf16)
                hipLaunchKernelGGL((bwd_prepare_kernel<DK, DV, true>), grid, dim3(256), 0, Lin.stream, Lin, X, units);
            else
                hipLaunchKernelGGL((bwd_prepare_kernel<DK, DV, false>), grid, dim3(256), 0, Lin.stream, Lin, X, units);
        }
        L.q = X.q; L.k = X.k; L.g = X.g; L.v = X.v; L.beta = X.b; L.d_o = X.d;
        L.in_bf16 = false;
        L.xf = InputXform{};
    }
    ChunkLaunch c{};
    c.q = L.q; c.k = L.k; c.v = L.v; c.g = L.g; c.beta = L.beta;
    c.h0 = L.h0; c.hT = nullptr; c.o = nullptr;
    c.cu_seqlens = L.cu_seqlens;
    c.B = L.B; c.T = L.T; c.H = L.H; c.dk = DK; c.dv = DV; c.N = L.N;
    c.chunk = 64; c.scale = L.scale;
    c.in_bf16 = L.in_bf16; c.out_bf16 = false;
    c.xf = InputXform{};
    c.workspace = ws;
    c.workspace_bytes = p.off_dl;
    c.stream = L.stream;
    const SegmentStates ss = launch_segment_table(c);
    float *dleave = reinterpret_cast<float *>(ws + p.off_dl);
    BackwardLaunch b = L;
    b.ckpt = reinterpret_cast<float *>(ws + p.off_ckpt);
    float *hb = reinterpret_cast<float *>(ws + p.off_hb);
    const unsigned seg_heads = static_cast<unsigned>(L.H) * static_cast<unsigned>(ss.max_segs);
    const dim3 grid(seg_heads), block(DV / 16 * kWave);
    const dim3 grid_local(seg_heads, 1, 2), block_local((DV + DK) / 16 * kWave);
    if (L.in_bf16)
        hipLaunchKernelGGL((local_passes_kernel<DK, DV, true>), grid_local, block_local, 0, L.stream, b, ss.sv, hb);
    else
        hipLaunchKernelGGL((local_passes_kernel<DK, DV, false>), grid_local, block_local, 0, L.stream, b, ss.sv, hb);
    launch_segment_combine(c, ss);
    hipLaunchKernelGGL((reverse_combine_kernel<DK>), dim3(DV / 16, L.H, L.N), dim3(256), 0, L.stream, ss.sv,
                       static_cast<const float *>(hb), L.dhT, dleave, L.dh0, L.H, DV);
    if (L.in_bf16)
        hipLaunchKernelGGL((recurrent_bwd_kernel<DK, DV, true>), grid, block, 0, L.stream, b, ss.sv,
                           static_cast<const float *>(dleave));
    else
        hipLaunchKernelGGL((recurrent_bwd_kernel<DK, DV, false>), grid, block, 0, L.stream, b, ss.sv,
                           static_cast<const float *>(dleave));
    if (transforms && units > 0)
        hipLaunchKernelGGL((bwd_finish_kernel<DK>), dim3(static_cast<unsigned>((units + 3) / 4)), dim3(256), 0,
                           Lin.stream, Lin, X, units);
    return hipGetLastError();
}

hipError_t launch_backward(const BackwardLaunch &L) {
    if (L.dk_dim == 128) return L.dv_dim == 128 ? launch_bwd<128, 128>(L) : launch_bwd<128, 64>(L);
    return L.dv_dim == 128 ? launch_bwd<64, 128>(L) : launch_bwd<64, 64>(L);
}

}  // namespace kda
