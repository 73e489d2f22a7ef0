// kda_recurrent.hip - token-by-token KDA kernels for gfx950.
//
// Serve the single-token decode step (Kimi Linear review notes, section
// "Training and Inference": one step, or a segment of at most 64 tokens, goes
// to the fused recurrent kernel) and, looping over tokens, short prefill
// segments.  recurrent_kernel takes one token: per (sequence, head, dv slice)
// one workgroup holds its slice of the fp32 state S in registers;
// recurrent_seq_kernel loops over a sequence's tokens.  For every token,
//
//     S~ = Diag(exp(g)) S                     decay first (section "Method":
//     p  = S~^T k,  r = S~^T q                 KDA recurrence, read-then-write
//     S  = S~ + beta k (v - p)^T               form)
//     o  = scale (r + beta (k.q) (v - p))      = scale S^T q after the write
//
// so the state is read from HBM once and written once per call, whatever the
// number of tokens.  With the optional input transforms the gate is formed
// from its logit as each token is staged, and the L2 norms of q and k are
// reduced beside k.q and folded into p, r, k.q and the write (all linear in
// k or q), so the normalised vectors are never stored.
// The state is dk x dv, row-major with dv contiguous:
// thread (rg, cg) owns columns [4cg, 4cg+4) of rows rg, rg+RG, ..., so one
// wave's float4 loads cover whole 512-byte rows (fully coalesced).  The state
// is loaded and stored with the non-temporal hint: it streams through once
// each way, and a serving cache's states (every layer's) are far larger than
// the 256 MiB Infinity Cache (measured at 256 x 16 heads between two state
// buffers: 105 -> 94 us per step).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int BV, bool InBf16, bool OutBf16>
__global__ void __launch_bounds__(256)
recurrent_kernel(const void *__restrict__ q_, const void *__restrict__ k_,
                 const void *__restrict__ v_, const float *__restrict__ g,
                 const void *__restrict__ beta_, const float *h0, float *hT,
                 void *__restrict__ o_, int H, int DV, float scale, InputXform xf) {
    using In = Elem<InBf16>;
    using Out = Elem<OutBf16>;
    const typename In::T *q = static_cast<const typename In::T *>(q_);
    const typename In::T *k = static_cast<const typename In::T *>(k_);
    const typename In::T *v = static_cast<const typename In::T *>(v_);
    const typename In::T *beta = static_cast<const typename In::T *>(beta_);
    typename Out::T *o = static_cast<typename Out::T *>(o_);

    constexpr int NT = 256;
    constexpr int CG = BV / 4;         // column groups of 4 in the slice
    constexpr int RG = NT / CG;        // row groups
    constexpr int ROWS = DK / RG;      // rows held per thread
    constexpr int NWAVE = NT / kWave;
    static_assert(ROWS >= 1 && DK % RG == 0 && DK <= NT, "bad tiling");

    const int slice = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int cg = tid % CG, rg = tid / CG;
    const int col = slice * BV + cg * 4;
    const int64_t nh = static_cast<int64_t>(n) * H + h;
    const int64_t tk = nh * DK, tv = nh * DV;

    __shared__ float s_kqa[3][DK];          // k, q, alpha of the token
    __shared__ float s_red[NWAVE][2][BV];   // per-wave partial S~^T k, S~^T q

    // the token's inputs first, so that they arrive while the state streams in behind them
    float kx = 0.f, qx = 0.f, ax = 0.f;
    if (tid < DK) {
        kx = In::load(k, tk + tid);
        qx = In::load(q, tk + tid);
        ax = g[xf.scalar_gate ? nh : tk + tid];
    }
    const float bt = In::load(beta, nh);
    const float4 vv = In::load4(v, tv + col);

    // state slice -> registers
    const int64_t sbase = nh * DK * DV;
    float4 s[ROWS];
    if (h0) {
#pragma unroll
        for (int m = 0; m < ROWS; ++m) s[m] = load_stream(h0 + sbase + static_cast<int64_t>(rg + m * RG) * DV + col);
    } else {
#pragma unroll
        for (int m = 0; m < ROWS; ++m) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < DK) {
        s_kqa[0][tid] = kx;
        s_kqa[1][tid] = qx;
        s_kqa[2][tid] = __expf(xf.log_gate(ax));
    }
    __syncthreads();

    float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        const int i = rg + m * RG;
        const float a = s_kqa[2][i], ki = s_kqa[0][i], qi = s_kqa[1][i];
        s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
        p[0] += s[m].x * ki; p[1] += s[m].y * ki; p[2] += s[m].z * ki; p[3] += s[m].w * ki;
        r[0] += s[m].x * qi; r[1] += s[m].y * qi; r[2] += s[m].z * qi; r[3] += s[m].w * qi;
    }
    // reduce over the row groups held by this wave
#pragma unroll
    for (int msk = CG; msk < kWave; msk <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            p[c] += __shfl_xor(p[c], msk, kWave);
            r[c] += __shfl_xor(r[c], msk, kWave);
        }
    }
    if (lane < CG) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s_red[wave][0][cg * 4 + c] = p[c];
            s_red[wave][1][cg * 4 + c] = r[c];
        }
    }
    // k . q (and |k|^2, |q|^2 when normalising), reduced inside every wave (no extra barrier)
    float kq = 0.f, ik = 1.f, iq = 1.f;
    if (xf.qk_l2norm) {
        float kk = 0.f, qq = 0.f;
        for (int i = lane; i < DK; i += kWave) {
            const float a = s_kqa[0][i], c = s_kqa[1][i];
            kq += a * c;
            kk += a * a;
            qq += c * c;
        }
        ik = rsqrtf(wave_sum(kk) + kL2Eps);
        iq = rsqrtf(wave_sum(qq) + kL2Eps);
        kq = wave_sum(kq) * ik * iq;
    } else {
        for (int i = lane; i < DK; i += kWave) kq += s_kqa[0][i] * s_kqa[1][i];
        kq = wave_sum(kq);
    }
    __syncthreads();

#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float ps = 0.f, rs = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
            ps += s_red[w][0][cg * 4 + c];
            rs += s_red[w][1][cg * 4 + c];
        }
        p[c] = ps * ik;  // S~^T k with k normalised
        r[c] = rs * iq;
    }
    const float btk = bt * ik;  // the write's beta k, normalised
    const float d0 = vv.x - p[0], d1 = vv.y - p[1], d2 = vv.z - p[2], d3 = vv.w - p[3];
    if (rg == 0) {
        const float bkq = bt * kq;
        Out::store4(o, tv + col,
                    make_float4(scale * (r[0] + bkq * d0), scale * (r[1] + bkq * d1),
                                scale * (r[2] + bkq * d2), scale * (r[3] + bkq * d3)));
    }
    if (!hT) return;  // kda_recurrent_fwd may skip the final state
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        const int i = rg + m * RG;
        const float bk = btk * s_kqa[0][i];
        s[m].x += bk * d0; s[m].y += bk * d1; s[m].z += bk * d2; s[m].w += bk * d3;
        store_stream(hT + sbase + static_cast<int64_t>(i) * DV + col, s[m]);
    }
}

// Multi-token form: one wave per (sequence, head, 16-column slice of dv), no
// barriers.  Lane (c = lane / 4, rg = lane % 4) holds column c of the slice
// for rows rg R .. rg R + R - 1 (R = DK / 4) of the fp32 state.  Per token:
// * the token's k, q and alpha (and the L2 norms) are formed once, two
//   channels per lane, and handed to the lanes that need them through the
//   wave's own LDS (a wave's LDS accesses are ordered, so no barrier);
// * per token two passes over the lane's rows: the decay with S~^T k, then
//   the write with S_t^T q; each R-term partial sum is reduced over the four
//   lanes of a quad by two DPP moves;
// * the inputs of the next four tokens are in flight while one is processed.
template <int DK, bool InBf16, bool OutBf16>
__global__ void __launch_bounds__(64)
recurrent_seq_kernel(const void *__restrict__ q_, const void *__restrict__ k_, const void *__restrict__ v_,
                     const float *__restrict__ g, const void *__restrict__ beta_, const float *h0, float *hT,
                     void *__restrict__ o_, const int32_t *__restrict__ cu_seqlens, int T, int H, int DV,
                     float scale, InputXform xf) {
    using In = Elem<InBf16>;
    using Out = Elem<OutBf16>;
    const typename In::T *q = static_cast<const typename In::T *>(q_);
    const typename In::T *k = static_cast<const typename In::T *>(k_);
    const typename In::T *v = static_cast<const typename In::T *>(v_);
    const typename In::T *beta = static_cast<const typename In::T *>(beta_);
    typename Out::T *o = static_cast<typename Out::T *>(o_);
    constexpr int R = DK / 4;         // rows per lane
    constexpr int RP = R + 4;         // padded LDS stride of a row group: a quad's four groups in distinct banks
    constexpr int CPL = DK / kWave;   // channels each lane loads per token
    static_assert(R % 4 == 0 && CPL >= 1, "tiling");
    __shared__ __attribute__((aligned(16))) float s_in[2][3][4 * RP];  // [buffer][k, q, alpha][row]

    int slice, h, n;
    slice_head_seq(slice, h, n);
    const int lane = threadIdx.x, c = lane >> 2, rg = lane & 3;
    const int col = 16 * slice + c;
    int64_t t0, t1;
    if (cu_seqlens) {
        t0 = cu_seqlens[n];
        t1 = cu_seqlens[n + 1];
        if (t1 < t0) t1 = t0;
    } else {
        t0 = static_cast<int64_t>(n) * T;
        t1 = t0 + T;
    }
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;
    float s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = h0 ? h0[sbase + static_cast<int64_t>(rg * R + i) * DV + col] : 0.f;

    // A token's inputs, fetched four tokens ahead into a ring of registers
    // (a token's arithmetic is far shorter than a global load's latency).
    struct Tok {
        float k[CPL], q[CPL], g[CPL], v, b;
    };
    auto fetch = [&](int64_t t, Tok &f) {
        t = t < t1 ? t : t1 - 1;  // past the end: repeat the last token (never used)
        const int64_t tk = (t * H + h) * DK;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int ch = lane * CPL + e;
            f.k[e] = In::load(k, tk + ch);
            f.q[e] = In::load(q, tk + ch);
            f.g[e] = g[xf.scalar_gate ? t * H + h : tk + ch];
        }
        f.v = In::load(v, (t * H + h) * static_cast<int64_t>(DV) + col);
        f.b = In::load(beta, t * H + h);
    };
    auto process = [&](int64_t t, const Tok &f) {
        // the token's k, q, alpha through LDS, and its norms
        float ik = 1.f, iq = 1.f;
        if (xf.qk_l2norm) {
            float kk = 0.f, qq = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                kk += f.k[e] * f.k[e];
                qq += f.q[e] * f.q[e];
            }
            ik = rsqrtf(wave_sum(kk) + kL2Eps);
            iq = rsqrtf(wave_sum(qq) + kL2Eps);
        }
        const int b = static_cast<int>(t - t0) & 1;  // alternate buffers: no write lands on a row still being read
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int ch = lane * CPL + e, li = (ch / R) * RP + ch % R;
            s_in[b][0][li] = f.k[e];
            s_in[b][1][li] = f.q[e];
            s_in[b][2][li] = __expf(xf.log_gate(f.g[e]));
        }
        // two passes over the rows: decay and S~^T k, then the write and the read S_t^T q
        const float *kx = &s_in[b][0][rg * RP], *qx = &s_in[b][1][rg * RP], *ax = &s_in[b][2][rg * RP];
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int i = 0; i < R; i += 4) {
            const float4 k4 = *reinterpret_cast<const float4 *>(kx + i);
            const float4 a4 = *reinterpret_cast<const float4 *>(ax + i);
            s[i] *= a4.x; s[i + 1] *= a4.y; s[i + 2] *= a4.z; s[i + 3] *= a4.w;
            p0 += s[i] * k4.x;
            p1 += s[i + 1] * k4.y;
            p0 += s[i + 2] * k4.z;
            p1 += s[i + 3] * k4.w;
        }
        const float p = quad_sum(p0 + p1) * ik;  // S~^T k, k normalised
        const float bkd = f.b * ik * (f.v - p);  // the write's beta k (v - p), k normalised
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int i = 0; i < R; i += 4) {
            const float4 k4 = *reinterpret_cast<const float4 *>(kx + i);
            const float4 q4 = *reinterpret_cast<const float4 *>(qx + i);
            s[i] += bkd * k4.x; s[i + 1] += bkd * k4.y; s[i + 2] += bkd * k4.z; s[i + 3] += bkd * k4.w;
            r0 += s[i] * q4.x;
            r1 += s[i + 1] * q4.y;
            r0 += s[i + 2] * q4.z;
            r1 += s[i + 3] * q4.w;
        }
        const float r = quad_sum(r0 + r1) * iq;  // S_t^T q, q normalised
        if (rg == 0) Out::store(o, (t * H + h) * static_cast<int64_t>(DV) + col, scale * r);
    };

    if (t0 < t1) {
        Tok f0, f1, f2, f3;
        fetch(t0, f0);
        fetch(t0 + 1, f1);
        fetch(t0 + 2, f2);
        fetch(t0 + 3, f3);
        for (int64_t t = t0; t < t1; t += 4) {
            process(t, f0);
            fetch(t + 4, f0);
            if (t + 1 < t1) process(t + 1, f1);
            fetch(t + 5, f1);
            if (t + 2 < t1) process(t + 2, f2);
            fetch(t + 6, f2);
            if (t + 3 < t1) process(t + 3, f3);
            fetch(t + 7, f3);
        }
    }
    if (hT) {
#pragma unroll
        for (int i = 0; i < R; ++i) hT[sbase + static_cast<int64_t>(rg * R + i) * DV + col] = s[i];
    }
}

template <int DK, int BV>
static hipError_t launch_rec_dk(const RecurrentLaunch &L) {
    dim3 grid(L.dv / BV, L.H, L.N), block(256);
#define KDA_REC(IB, OB)                                                                       \
    hipLaunchKernelGGL((recurrent_kernel<DK, BV, IB, OB>), grid, block, 0, L.stream, L.q, L.k, \
                       L.v, L.g, L.beta, L.h0, L.hT, L.o, L.H, L.dv, L.scale, L.xf)
    if (L.in_bf16 && L.out_bf16) KDA_REC(true, true);
    else if (L.in_bf16) KDA_REC(true, false);
    else if (L.out_bf16) KDA_REC(false, true);
    else KDA_REC(false, false);
#undef KDA_REC
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_rec_seq(const RecurrentLaunch &L) {
    dim3 grid(L.dv / 16, L.H, L.N), block(64);
#define KDA_REC(IB, OB)                                                                                  \
    hipLaunchKernelGGL((recurrent_seq_kernel<DK, IB, OB>), grid, block, 0, L.stream, L.q, L.k, L.v, L.g, \
                       L.beta, L.h0, L.hT, L.o, L.cu_seqlens, L.T, L.H, L.dv, L.scale, L.xf)
    if (L.in_bf16 && L.out_bf16) KDA_REC(true, true);
    else if (L.in_bf16) KDA_REC(true, false);
    else if (L.out_bf16) KDA_REC(false, true);
    else KDA_REC(false, false);
#undef KDA_REC
    return hipGetLastError();
}

hipError_t launch_recurrent(const RecurrentLaunch &L) {
    // A decode step: one workgroup per head's whole state (or half), whose
    // wide row loads stream the state at the copy rate.  Several tokens: one
    // wave per 16-column slice, which runs the serial token loop without
    // barriers.
    if (L.multi_token) return L.dk == 128 ? launch_rec_seq<128>(L) : launch_rec_seq<64>(L);
    if (L.dk == 128) return L.dv == 128 ? launch_rec_dk<128, 128>(L) : launch_rec_dk<128, 64>(L);
    return L.dv == 128 ? launch_rec_dk<64, 128>(L) : launch_rec_dk<64, 64>(L);
}

}  // namespace kda
