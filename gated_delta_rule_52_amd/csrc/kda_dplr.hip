// kda_dplr.hip - the general diagonal-plus-low-rank (DPLR) recurrence, token by token, for gfx950.
//
// KDA's transition is a DPLR matrix with D = Diag(alpha_t), a_t = beta_t k_t and b_t = alpha_t .* k_t
// (Kimi Linear review notes, section "Chunkwise Algorithm").  This kernel runs the general member of the
// family, with a_t and b_t free:
//
//     x   = b_t^T S_{t-1}                          (dv: the low-rank read, before the decay)
//     S_t = Diag(alpha_t) S_{t-1} - a_t x + k_t v_t^T,     alpha_t = exp(g_t)
//     o_t = scale * S_t^T q_t
//
// Work split as in the multi-token KDA kernel: one wave per (sequence, head, 16-column slice of dv), no
// barriers.  Lane (c = lane / 4, rg = lane % 4) holds column c of the slice for rows rg R .. rg R + R - 1
// (R = dk / 4) of the fp32 state.  A token's k, q, a, b and alpha are formed two channels per lane and
// handed to the lanes that need them through the wave's own LDS (row groups padded so that the four row
// groups a quad reads sit in distinct banks); sums over rows are quad sums.  Inputs are fetched four
// tokens ahead.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, bool InBf16, bool OutBf16>
__global__ void __launch_bounds__(64)
dplr_seq_kernel(DplrLaunch L) {
    using In = Elem<InBf16>;
    using Out = Elem<OutBf16>;
    using IT = typename In::T;
    const IT *q = static_cast<const IT *>(L.q), *k = static_cast<const IT *>(L.k);
    const IT *v = static_cast<const IT *>(L.v), *a = static_cast<const IT *>(L.a);
    const IT *bv = static_cast<const IT *>(L.b);
    const float *g = L.g;
    typename Out::T *o = static_cast<typename Out::T *>(L.o);
    constexpr int R = DK / 4, RP = R + 4;  // rows per lane; padded LDS stride of a row group
    constexpr int CPL = DK / kWave;        // channels each lane loads per token
    static_assert(R % 4 == 0 && CPL >= 1, "tiling");
    __shared__ __attribute__((aligned(16))) float s_in[2][5][4 * RP];  // [buffer][k, q, a, b, alpha][row]

    const int H = L.H, DV = L.dv;
    int slice, h, n;
    slice_head_seq(slice, h, n);
    const int lane = threadIdx.x, c = lane >> 2, rg = lane & 3;
    const int col = 16 * slice + c;
    int64_t t0, t1;
    if (L.cu_seqlens) {
        t0 = L.cu_seqlens[n];
        t1 = L.cu_seqlens[n + 1];
        if (t1 < t0) t1 = t0;
    } else {
        t0 = static_cast<int64_t>(n) * L.T;
        t1 = t0 + L.T;
    }
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;
    float s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = L.h0 ? L.h0[sbase + static_cast<int64_t>(rg * R + i) * DV + col] : 0.f;

    struct Tok {
        float k[CPL], q[CPL], a[CPL], b[CPL], g[CPL], v;
    };
    auto fetch = [&](int64_t t, Tok &f) {
        t = t < t1 ? t : t1 - 1;  // past the end: repeat the last token (never used)
        const int64_t tk = (t * H + h) * DK;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int ch = lane * CPL + e;
            f.k[e] = In::load(k, tk + ch);
            f.q[e] = In::load(q, tk + ch);
            f.a[e] = In::load(a, tk + ch);
            f.b[e] = In::load(bv, tk + ch);
            f.g[e] = g[tk + ch];
        }
        f.v = In::load(v, (t * H + h) * static_cast<int64_t>(DV) + col);
    };
    auto process = [&](int64_t t, const Tok &f) {
        const int buf = static_cast<int>(t - t0) & 1;  // alternate buffers: no write lands on a row still being read
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int ch = lane * CPL + e, li = (ch / R) * RP + ch % R;
            s_in[buf][0][li] = f.k[e];
            s_in[buf][1][li] = f.q[e];
            s_in[buf][2][li] = f.a[e];
            s_in[buf][3][li] = f.b[e];
            s_in[buf][4][li] = __expf(f.g[e]);
        }
        const float *row = &s_in[buf][0][rg * RP];
        float x0 = 0.f, x1 = 0.f;
#pragma unroll
        for (int i = 0; i < R; i += 4) {
            const float4 b4 = *reinterpret_cast<const float4 *>(row + 3 * 4 * RP + i);
            x0 += b4.x * s[i];
            x1 += b4.y * s[i + 1];
            x0 += b4.z * s[i + 2];
            x1 += b4.w * s[i + 3];
        }
        const float x = quad_sum(x0 + x1), vv = f.v;
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int i = 0; i < R; i += 4) {
            const float4 k4 = *reinterpret_cast<const float4 *>(row + i);
            const float4 q4 = *reinterpret_cast<const float4 *>(row + 4 * RP + i);
            const float4 a4 = *reinterpret_cast<const float4 *>(row + 2 * 4 * RP + i);
            const float4 al = *reinterpret_cast<const float4 *>(row + 4 * 4 * RP + i);
            s[i] = al.x * s[i] - a4.x * x + k4.x * vv;
            s[i + 1] = al.y * s[i + 1] - a4.y * x + k4.y * vv;
            s[i + 2] = al.z * s[i + 2] - a4.z * x + k4.z * vv;
            s[i + 3] = al.w * s[i + 3] - a4.w * x + k4.w * vv;
            o0 += q4.x * s[i];
            o1 += q4.y * s[i + 1];
            o0 += q4.z * s[i + 2];
            o1 += q4.w * s[i + 3];
        }
        const float ot = quad_sum(o0 + o1);
        if (rg == 0) Out::store(o, (t * H + h) * static_cast<int64_t>(DV) + col, L.scale * ot);
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
    if (L.hT) {
#pragma unroll
        for (int i = 0; i < R; ++i) L.hT[sbase + static_cast<int64_t>(rg * R + i) * DV + col] = s[i];
    }
}

template <int DK>
static hipError_t launch_dplr_dk(const DplrLaunch &L) {
    dim3 grid(L.dv / 16, L.H, L.N), block(64);
#define KDA_DPLR(IB, OB) hipLaunchKernelGGL((dplr_seq_kernel<DK, IB, OB>), grid, block, 0, L.stream, L)
    if (L.in_bf16 && L.out_bf16) KDA_DPLR(true, true);
    else if (L.in_bf16) KDA_DPLR(true, false);
    else if (L.out_bf16) KDA_DPLR(false, true);
    else KDA_DPLR(false, false);
#undef KDA_DPLR
    return hipGetLastError();
}

hipError_t launch_dplr(const DplrLaunch &L) {
    return L.dk == 128 ? launch_dplr_dk<128>(L) : launch_dplr_dk<64>(L);
}

}  // namespace kda
