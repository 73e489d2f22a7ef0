// kda_recurrent.hip - token-by-token KDA kernel for gfx950.
//
// Serves the single-token decode step (Kimi Linear review notes, section
// "Training and Inference": one step, or a segment of at most 64 tokens, goes
// to the fused recurrent kernel) and, looping over tokens, short prefill
// segments.  Per (sequence, head, dv slice) one workgroup keeps its slice of
// the fp32 state S in registers and, for every token,
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
// wave's float4 loads cover whole 512-byte rows (fully coalesced).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int BV, bool InBf16, bool OutBf16>
__global__ void __launch_bounds__(256)
recurrent_kernel(const void *__restrict__ q_, const void *__restrict__ k_,
                 const void *__restrict__ v_, const float *__restrict__ g,
                 const void *__restrict__ beta_, const float *h0, float *hT,
                 void *__restrict__ o_, const int32_t *__restrict__ cu_seqlens,
                 int T, int H, int DV, float scale, InputXform xf) {
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
    constexpr int RG_PER_WAVE = kWave / CG;
    constexpr int NWAVE = NT / kWave;
    static_assert(ROWS >= 1 && DK % RG == 0, "bad tiling");

    const int slice = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int cg = tid % CG, rg = tid / CG;
    const int col = slice * BV + cg * 4;

    int64_t t0, t1;
    if (cu_seqlens) {
        t0 = cu_seqlens[n];
        t1 = cu_seqlens[n + 1];
        if (t1 < t0) t1 = t0;
    } else {
        t0 = static_cast<int64_t>(n) * T;
        t1 = t0 + T;
    }

    __shared__ float s_kqa[2][3][DK];          // k, q, alpha of the current token
    __shared__ float s_beta[2];
    __shared__ float s_red[2][NWAVE][2][BV];   // per-wave partial S~^T k, S~^T q

    // state slice -> registers
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;
    float4 s[ROWS];
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        const int i = rg + m * RG;
        s[m] = h0 ? *reinterpret_cast<const float4 *>(h0 + sbase + static_cast<int64_t>(i) * DV + col)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int64_t t = t0; t < t1; ++t) {
        const int b = static_cast<int>(t - t0) & 1;
        const int64_t tk = (t * H + h) * DK, tv = (t * H + h) * static_cast<int64_t>(DV);
        for (int i = tid; i < DK; i += NT) {
            s_kqa[b][0][i] = In::load(k, tk + i);
            s_kqa[b][1][i] = In::load(q, tk + i);
            s_kqa[b][2][i] = __expf(xf.log_gate(g[xf.scalar_gate ? t * H + h : tk + i]));
        }
        if (tid == 0) s_beta[b] = In::load(beta, t * H + h);
        const float4 vv = In::load4(v, tv + col);
        __syncthreads();

        float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < ROWS; ++m) {
            const int i = rg + m * RG;
            const float a = s_kqa[b][2][i], ki = s_kqa[b][0][i], qi = s_kqa[b][1][i];
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
                s_red[b][wave][0][cg * 4 + c] = p[c];
                s_red[b][wave][1][cg * 4 + c] = r[c];
            }
        }
        // k . q (and |k|^2, |q|^2 when normalising), reduced inside every wave (no extra barrier)
        float kq = 0.f, ik = 1.f, iq = 1.f;
        if (xf.qk_l2norm) {
            float kk = 0.f, qq = 0.f;
            for (int i = lane; i < DK; i += kWave) {
                const float a = s_kqa[b][0][i], c = s_kqa[b][1][i];
                kq += a * c;
                kk += a * a;
                qq += c * c;
            }
            ik = rsqrtf(wave_sum(kk) + kL2Eps);
            iq = rsqrtf(wave_sum(qq) + kL2Eps);
            kq = wave_sum(kq) * ik * iq;
        } else {
            for (int i = lane; i < DK; i += kWave) kq += s_kqa[b][0][i] * s_kqa[b][1][i];
            kq = wave_sum(kq);
        }
        __syncthreads();

#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float ps = 0.f, rs = 0.f;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) {
                ps += s_red[b][w][0][cg * 4 + c];
                rs += s_red[b][w][1][cg * 4 + c];
            }
            p[c] = ps * ik;  // S~^T k with k normalised
            r[c] = rs * iq;
        }
        (void)RG_PER_WAVE;
        const float bt = s_beta[b];
        const float btk = bt * ik;  // the write's beta k, normalised
        const float d0 = vv.x - p[0], d1 = vv.y - p[1], d2 = vv.z - p[2], d3 = vv.w - p[3];
        if (rg == 0) {
            const float bkq = bt * kq;
            Out::store4(o, tv + col,
                        make_float4(scale * (r[0] + bkq * d0), scale * (r[1] + bkq * d1),
                                    scale * (r[2] + bkq * d2), scale * (r[3] + bkq * d3)));
        }
#pragma unroll
        for (int m = 0; m < ROWS; ++m) {
            const float bk = btk * s_kqa[b][0][rg + m * RG];
            s[m].x += bk * d0; s[m].y += bk * d1; s[m].z += bk * d2; s[m].w += bk * d3;
        }
    }

    if (hT) {
#pragma unroll
        for (int m = 0; m < ROWS; ++m) {
            const int i = rg + m * RG;
            *reinterpret_cast<float4 *>(hT + sbase + static_cast<int64_t>(i) * DV + col) = s[m];
        }
    }
}

template <int DK, int BV>
static hipError_t launch_rec_dk(const RecurrentLaunch &L) {
    dim3 grid(L.dv / BV, L.H, L.N), block(256);
#define KDA_REC(IB, OB)                                                                       \
    hipLaunchKernelGGL((recurrent_kernel<DK, BV, IB, OB>), grid, block, 0, L.stream, L.q, L.k, \
                       L.v, L.g, L.beta, L.h0, L.hT, L.o, L.cu_seqlens, L.T, L.H, L.dv, L.scale, L.xf)
    if (L.in_bf16 && L.out_bf16) KDA_REC(true, true);
    else if (L.in_bf16) KDA_REC(true, false);
    else if (L.out_bf16) KDA_REC(false, true);
    else KDA_REC(false, false);
#undef KDA_REC
    return hipGetLastError();
}

hipError_t launch_recurrent(const RecurrentLaunch &L) {
    // One slice per head for a single token (enough workgroups already);
    // 32-column slices when tokens are looped, to spread the serial work.
    const bool narrow = L.multi_token;
    if (L.dk == 128) return narrow ? launch_rec_dk<128, 32>(L) : (L.dv == 128 ? launch_rec_dk<128, 128>(L) : launch_rec_dk<128, 64>(L));
    return narrow ? launch_rec_dk<64, 32>(L) : (L.dv == 128 ? launch_rec_dk<64, 128>(L) : launch_rec_dk<64, 64>(L));
}

}  // namespace kda
