// kda_chunk_bwd.hip - gradients of the chunkwise KDA prefill on gfx950 (bf16
// inputs, dk = dv = 128, chunks of 64), recomputing the forward chunk by chunk
// (Kimi Linear review notes, section "Training and Inference": training runs
// the chunk path; the gradients are those of the recurrence of section
// "Method").
//
// Per chunk with entering state S, leaving-state gradient dS' and output
// gradient dO, the chunk form of the forward (kda_prep.hip) differentiates to
//
//   dV_new = A_qk^T dO + Kd dS'          dS = gamma * dS' + Q^T dO - W^T dV_new
//   dQ     = dO S^T      dA_qk = dO V_new^T (lower)      dKd = V_new dS'^T
//   dW     = -dV_new S^T                 dgamma_c = sum_j S[c, j] dS'[c, j]
//   dY     = T^T [dW | dV_new]           (Y = beta [E | V], [W | U] = T Y)
//   dA_kk  = -(dY Y^T) T^T  (strictly lower)
//
// with Q = scale e^G q, E = e^G k, Kd = e^{G_last - G} k, T = (I + A_kk)^{-1},
// and then the decayed Gram products A_kk = beta (k k^T decayed), A_qk carry
// their gradients to q, k and the cumulative log decay G, which a reverse
// cumulative sum inside the chunk turns into dg.  (These equations are derived
// from the chunk form and were checked against the token recurrence's
// gradients in fp64.)
//
// Passes: the forward segmented prefill's prep, local pass and combine, then
//   kStates    replays each segment and keeps every chunk's S and V_new;
//   rev_pack   completes each reverse pack (kda_mfma.h; the prep wrote its
//              transposed slots) with A_qk^T dO on fp16 matrix cores;
//   kRevLocal, the reverse combine (bf16 matrix cores over P^T planes the local
//              pass writes), kRevOut walk the chunks last to first with
//              dS in the accumulators and keep every chunk's dS' and dV_new;
//   grad       one workgroup per chunk and head: everything above that is
//              local to the chunk, on fp32 matrix cores (16x16x4).
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace mc {
namespace {

// ---------------------------------------------------------------- reverse pack
constexpr int kRpThreads = 256;
constexpr int kDOP = DV + 8;  // row stride (halves) of the staged dO

// The reverse pack's -Kd, -W^T and Q^T slots come from the prep (its RV instantiation, from the same fp16
// values as the forward pack); this kernel adds A_qk^T dO (with its remainder plane), dO, gamma and the header.
__global__ void __launch_bounds__(kRpThreads)
rev_pack_kernel(const char *__restrict__ packs, char *__restrict__ rpacks, const uint16_t *__restrict__ d_o,
                SegmentView sv, int per, int H) {
    constexpr int kA = kPkU - kPkA;  // the A_qk blocks of the forward pack
    __shared__ __attribute__((aligned(16))) char sF[kA];
    __shared__ __attribute__((aligned(16))) uint16_t sDO[C * kDOP];
    __shared__ int sMax[2];
    const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(H));  // heads fastest
    const int slot = static_cast<int>(blockIdx.x / static_cast<unsigned>(H));
    const int seg = slot / per, jc = slot - seg * per;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, g4 = lane >> 4;
    if (seg >= sv.count()) return;
    const int4 sd = sv.desc(seg);
    const int64_t c0 = sd.y + static_cast<int64_t>(C) * jc, t1 = sd.z;
    if (c0 >= t1) return;
    const int L = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);
    const char *fp = packs + (static_cast<int64_t>(slot) * H + h) * kPkBytes;
    char *rp = rpacks + (static_cast<int64_t>(slot) * H + h) * kRvBytes;
    if (tid < 2) sMax[tid] = 0;
    for (int u = tid; u < kA / 16; u += kRpThreads)
        *reinterpret_cast<u4 *>(sF + 16 * u) = *reinterpret_cast<const u4 *>(fp + kPkA + 16 * u);
    uint32_t mx = 0u;
    for (int u = tid; u < C * (DV / 8); u += kRpThreads) {  // dO rows, 16 bytes at a time; rows past L are 0
        const int r = u / (DV / 8), cu = u % (DV / 8);
        u4 w = {0u, 0u, 0u, 0u};
        if (r < L) w = *reinterpret_cast<const u4 *>(d_o + ((c0 + r) * H + h) * DV + 8 * cu);
        *reinterpret_cast<u4 *>(sDO + r * kDOP + 8 * cu) = w;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = absmax2(mx, w[e]);
    }
    __syncthreads();  // sMax zeroed before any atomic below
    const float mxf = wave_max(absmax2_value(mx));
    if (lane == 0) atomicMax(&sMax[0], __float_as_int(mxf));
    __syncthreads();
    const int edo = exp_of(__int_as_float(sMax[0]));  // |dO| 2^-edo < 1
    const float sdo = pow2(-edo);
    const int *fh = reinterpret_cast<const int *>(fp + kPkHdr);

    // dO in accumulator order (as U), x 2^-edo
    for (int idx = tid; idx < 8 * 2 * 64; idx += kRpThreads) {
        const int ct = idx >> 7, pr = (idx >> 6) & 1, ln = idx & 63;
        const int n = ln & 15, g = ln >> 4;
        _Float16 e[8];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * (2 * pr + half) + 4 * g + jj;
                e[4 * half + jj] = static_cast<_Float16>(bf16_to_f32(sDO[r * kDOP + 16 * ct + n]) * sdo);
            }
        *reinterpret_cast<h8 *>(rp + kRvDO + ((ct * 2 + pr) * 64 + ln) * 16) = h8{e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]};
    }
    // A_qk^T dO: output block row a (16 rows), column tile ct: sum over b >= a of (A_ba)^T dO_b.  The A
    // operand (A_ba)^T [n16][4 g4 + i] = A_ba[4 g4 + i][n16] comes from the lane-order block (lane
    // 16 (y / 4) + x holds row x, columns 4 (y / 4) .. +3).
    f4 d0[2][4];
    float dmax = 0.f;
    const float unA = pow2(fh[kHdrA] + edo);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ct = 2 * wave + t;
        h4 bo[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bo[b][i] = static_cast<_Float16>(bf16_to_f32(sDO[(16 * b + 4 * g4 + i) * kDOP + 16 * ct + n16]) * sdo);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f4 acc = zero4();
#pragma unroll
            for (int b = a; b < 4; ++b) {
                const int p = b * (b + 1) / 2 + a;
                const _Float16 *blk = reinterpret_cast<const _Float16 *>(sF + 512 * p);
                h4 av;
#pragma unroll
                for (int i = 0; i < 4; ++i) av[i] = blk[4 * (16 * (n16 >> 2) + 4 * g4 + i) + (n16 & 3)];
                acc = mma16(av, bo[b], acc);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                acc[jj] *= unA;
                dmax = fmaxf(dmax, fabsf(acc[jj]));
            }
            d0[t][a] = acc;
        }
    }
    dmax = wave_max(dmax);
    if (lane == 0) atomicMax(&sMax[1], __float_as_int(dmax));
    __syncthreads();
    const int ed0 = exp_of(__int_as_float(sMax[1]));
    const float sd0 = pow2(-ed0);
    // U = fp16(A_qk^T dO 2^-ed0), and the remainder 2^11 times larger in the UL slot
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const h4 hi = to_h4(d0[t][a], sd0);
            f4 rest;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) rest[jj] = (d0[t][a][jj] * sd0 - static_cast<float>(hi[jj])) * 2048.f;
            *reinterpret_cast<h4 *>(rp + kPkU + u_off(2 * wave + t, a, lane)) = hi;
            *reinterpret_cast<h4 *>(rp + kRvUL + u_off(2 * wave + t, a, lane)) = to_h4(rest, 1.f);
        }
    if (tid < 32)  // gamma passes through
        *reinterpret_cast<u4 *>(rp + kPkGamma + 16 * tid) = *reinterpret_cast<const u4 *>(fp + kPkGamma + 16 * tid);
    if (tid == 32) {
        int hd[8] = {};
        hd[kHdrW] = fh[kHdrK];  // -Kd carries the forward KT's exponent
        hd[kHdrQ] = fh[kHdrQ];
        hd[kHdrK] = fh[kHdrW];  // -W^T carries W's
        hd[kHdrU] = ed0;
        hd[kHdrDO] = edo;
        hd[kHdrUL] = ed0 - 11;
        *reinterpret_cast<u4 *>(rp + kPkHdr) = u4{uint32_t(hd[0]), uint32_t(hd[1]), uint32_t(hd[2]), uint32_t(hd[3])};
        *reinterpret_cast<u4 *>(rp + kPkHdr + 16) = u4{uint32_t(hd[4]), uint32_t(hd[5]), uint32_t(hd[6]), uint32_t(hd[7])};
    }
}

// ---------------------------------------------------------------- chunk gradients
constexpr int kGT = 512;  // 8 waves: wave w owns column tile w (16 columns) of every [64 x 128] result
constexpr int LF = DK + 4;  // fp32 row stride of [rows][128] tiles (operand reads of 16 rows x 4 hit distinct banks)
constexpr int LH = DK + 8;  // bf16 row stride
constexpr int LA = C + 4;   // fp32 row stride of [64][64]
constexpr int LT = 20;      // fp32 row stride of 16 x 16 tiles
constexpr float kMaxChunkDecayG = 80.0f;
// LDS: phases 1-2 (state products) and phase 3 (chunk-local work) share the bytes.  The state products
// run on bf16 matrix cores from bf16 high and low planes (x = hi + lo to about 16 bits; dO is bf16 already):
// hi*hi + hi*lo + lo*hi per product
constexpr int kSSh = 0;                          // S, then dS': high plane [128][LH] bf16
constexpr int kSSl = kSSh + DK * LH * 2;         // low plane
constexpr int kSO = kSSl + DK * LH * 2;          // dO [64][LH] bf16
constexpr int kSXh = kSO + C * LH * 2;           // dV_new, then V_new: high plane [64][LH]
constexpr int kSXl = kSXh + C * LH * 2;          // low plane
constexpr int kP12 = kSXl + C * LH * 2;
constexpr int kK = 0;                            // k             [64][LH] bf16
constexpr int kQ = kK + C * LH * 2;              // q
constexpr int kRf = kQ + C * LH * 2;             // e^{G - m}, or G itself in an exact chunk   [64][LF]
constexpr int kAt = kRf + C * LF * 4;            // At = decayed k k^T, strictly lower   [64][LA]
constexpr int kDq = kAt + C * LA * 4;            // dA_qk, lower   [64][LA]
constexpr int kTd = kDq + C * LA * 4;            // diagonal blocks of T   [4][16][LT]
constexpr int kR = kTd + 4 * 16 * LT * 4;        // scratch
constexpr int kRBytes = C * LF * 4 + C * LA * 4;  // dY half + M; also the solves' tiles, then dA_kk
constexpr int kSm = kR + kRBytes;                // small vectors
constexpr int kSmBeta = kSm, kSmEm = kSmBeta + 256, kSmDgam = kSmEm + 512, kSmDb = kSmDgam + 512,
              kSmFlag = kSmDb + 8 * 64 * 4;
constexpr int kLds = kSmFlag + 16;
static_assert(kP12 <= kSm, "the state products stay clear of the small vectors");
static_assert(8 * 4 * 16 * LT * 4 <= kRBytes, "the dY solve tiles fit the scratch");
static_assert(kLds <= 160 * 1024, "one workgroup per compute unit");

__device__ __forceinline__ f4 mf(float a, float b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }

// x -> bf16 high part (round to nearest even) and low part (the rest, rounded)
__device__ __forceinline__ void split_hl(float x, uint16_t &hi, uint16_t &lo) {
    const __bf16 h = static_cast<__bf16>(x);
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x - static_cast<float>(h)));
}
// 8 consecutive bf16 of row `row` from column k0 of a [rows][LH] plane
__device__ __forceinline__ b8 rd8(const uint16_t *plane, int row, int k0) {
    return *reinterpret_cast<const b8 *>(plane + row * LH + k0);
}

// pair index t -> block (a, b), b <= a, in the order (0,0),(1,0),(1,1),(2,0)...
__device__ __forceinline__ void tri_ab(int t, int &a, int &b) {
    a = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
    b = t - a * (a + 1) / 2;
}

struct GradArgs {
    const uint16_t *q, *k, *v, *beta, *d_o;
    const float *g;
    const float *st, *vn, *dst, *dvn;  // per chunk: S, V_new, dS', dV_new (accumulator order; S and dS' as fp16)
    const int *stf, *dstf;             // per chunk and 16-column tile: the exponents of S's and dS''s fp16 frames
    float *dq, *dk, *dv, *dg, *dbeta;
    int per, H;
    float scale;
};

__global__ void __launch_bounds__(kGT, 1)
chunk_grad_kernel(GradArgs A, SegmentView sv) {
    __shared__ __attribute__((aligned(16))) char smem[kLds];
    const int H = A.H;
    const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(H));  // heads fastest
    const int slot = static_cast<int>(blockIdx.x / static_cast<unsigned>(H));
    const int seg = slot / A.per, jc = slot - seg * A.per;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    if (seg >= sv.count()) return;
    const int4 sd = sv.desc(seg);
    const int64_t c0 = sd.y + static_cast<int64_t>(C) * jc, t1 = sd.z;
    if (c0 >= t1) return;
    const int L = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);
    const int64_t sh = static_cast<int64_t>(slot) * H + h;
    // S and dS' arrive as fp16 in power-of-two frames, one per 16-column tile (unit u = tid + kGT i: tile i)
    const h4 *St = reinterpret_cast<const h4 *>(A.st + sh * (DK * DV)), *dSt = reinterpret_cast<const h4 *>(A.dst + sh * (DK * DV));
    const int *Sf = A.stf + sh * 8, *dSf = A.dstf + sh * 8;
    auto wide = [](h4 x, float s) { return f4{static_cast<float>(x[0]) * s, static_cast<float>(x[1]) * s,
                                             static_cast<float>(x[2]) * s, static_cast<float>(x[3]) * s}; };
    const float *Vt = A.vn + sh * (C * DV), *dVt = A.dvn + sh * (C * DV);
    const int64_t rowb = c0 * H + h;  // token row c0 + r of head h is (rowb + r H) * 128
    auto trow = [&](int r) { return (rowb + static_cast<int64_t>(r) * H) * DK; };
    float *sBeta = reinterpret_cast<float *>(smem + kSmBeta), *sEm = reinterpret_cast<float *>(smem + kSmEm);
    float *sDgam = reinterpret_cast<float *>(smem + kSmDgam), *sDb = reinterpret_cast<float *>(smem + kSmDb);
    int *sFlag = reinterpret_cast<int *>(smem + kSmFlag);
    const int cw = 16 * wave + n16;  // this lane's output column

    // accumulator-order [R x 16 column tiles] unit u -> (row, col) of its first element
    auto unit_rc = [](int u, int R, int &row, int &col) {
        const int ln = u & 63, t = u >> 6;
        row = 16 * (t % R) + 4 * (ln >> 4);
        col = 16 * (t / R) + (ln & 15);
    };

    // ================= phase 1: dQ = dO S^T, dWn = dV_new S^T =================
    uint16_t *sSh = reinterpret_cast<uint16_t *>(smem + kSSh), *sSl = reinterpret_cast<uint16_t *>(smem + kSSl);
    uint16_t *sO = reinterpret_cast<uint16_t *>(smem + kSO);
    uint16_t *sXh = reinterpret_cast<uint16_t *>(smem + kSXh), *sXl = reinterpret_cast<uint16_t *>(smem + kSXl);
    // an accumulator-order unit of R row tiles into the planes
    auto put_unit = [&](uint16_t *ph, uint16_t *pl, int u, int R, const f4 &x) {
        int row, col;
        unit_rc(u, R, row, col);
#pragma unroll
        for (int e = 0; e < 4; ++e) split_hl(x[e], ph[(row + e) * LH + col], pl[(row + e) * LH + col]);
    };
    if (tid == 0) *sFlag = 0;
    f4 pS[8];  // this thread's S units, kept for dgamma in phase 2
    // the kept states and V_new are read once, with the non-temporal hint
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int u = tid + kGT * i;
        pS[i] = wide(__builtin_nontemporal_load(St + u), pow2(Sf[i]));
        put_unit(sSh, sSl, u, 8, pS[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int u = tid + kGT * i;
        put_unit(sXh, sXl, u, 4, __builtin_nontemporal_load(reinterpret_cast<const f4 *>(dVt + 4 * u)));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + kGT * i, r = u >> 4, cu = u & 15;
        u4 w = {0u, 0u, 0u, 0u};
        if (r < L) w = *reinterpret_cast<const u4 *>(A.d_o + trow(r) + 8 * cu);
        *reinterpret_cast<u4 *>(sO + r * LH + 8 * cu) = w;
    }
    __syncthreads();
    // phase 2's inputs, fetched while phase 1 computes (dS' units match the S units above)
    f4 pdS[8], pVn[4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        pdS[i] = wide(__builtin_nontemporal_load(dSt + tid + kGT * i), pow2(dSf[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        pVn[i] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(Vt + 4 * (tid + kGT * i)));
    __builtin_amdgcn_sched_barrier(0);
    f4 dQh[4], dWn[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) dQh[a] = dWn[a] = zero4();
#pragma unroll
    for (int s = 0; s < DV / 32; ++s) {
        const int k0 = 32 * s + 8 * g4;
        const b8 bh = rd8(sSh, cw, k0), bl = rd8(sSl, cw, k0);  // B[j][c] = S[c][j]
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const b8 ao = rd8(sO, 16 * a + n16, k0);
            dQh[a] = mmab(ao, bh, dQh[a]);
            dQh[a] = mmab(ao, bl, dQh[a]);
            const b8 xh = rd8(sXh, 16 * a + n16, k0), xl = rd8(sXl, 16 * a + n16, k0);
            dWn[a] = mmab(xh, bh, dWn[a]);
            dWn[a] = mmab(xh, bl, dWn[a]);
            dWn[a] = mmab(xl, bh, dWn[a]);
        }
    }
    __syncthreads();

    // ================= phase 2: dKd = V_new dS'^T, dA_qk = dO V_new^T, dgamma =================
    {
        float dgp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // units (column tile i, row tile `wave`, lane): rows 16 wave + 4 g4 + e
            put_unit(sSh, sSl, tid + kGT * i, 8, pdS[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) dgp[e] += pdS[i][e] * pS[i][e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) dgp[e] += __shfl_xor(dgp[e], m, 16);
            if (n16 == 0) sDgam[16 * wave + 4 * g4 + e] = dgp[e];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) put_unit(sXh, sXl, tid + kGT * i, 4, pVn[i]);
    __syncthreads();
    // phase 3's inputs (k, q, v rows, the gate column pieces, beta), fetched while phase 2 computes
    const int gc = tid & (DK - 1), qq = tid >> 7;
    u4 pk[2], pq[2], pv[2];
    float pg[16], pbeta = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + kGT * i, r = u >> 4, cu = u & 15;
        pk[i] = pq[i] = pv[i] = u4{0u, 0u, 0u, 0u};
        if (r < L) {
            pk[i] = *reinterpret_cast<const u4 *>(A.k + trow(r) + 8 * cu);
            pq[i] = *reinterpret_cast<const u4 *>(A.q + trow(r) + 8 * cu);
            pv[i] = *reinterpret_cast<const u4 *>(A.v + trow(r) + 8 * cu);
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 16 * qq + i;
        pg[i] = r < L ? A.g[trow(r) + gc] : 0.f;
    }
    if (tid < L) pbeta = bf16_to_f32(A.beta[rowb + static_cast<int64_t>(tid) * H]);
    __builtin_amdgcn_sched_barrier(0);
    f4 dKd[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) dKd[a] = zero4();
#pragma unroll
    for (int s = 0; s < DV / 32; ++s) {
        const int k0 = 32 * s + 8 * g4;
        const b8 bh = rd8(sSh, cw, k0), bl = rd8(sSl, cw, k0);  // B[j][c] = dS'[c][j]
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const b8 xh = rd8(sXh, 16 * a + n16, k0), xl = rd8(sXl, 16 * a + n16, k0);
            dKd[a] = mmab(xh, bh, dKd[a]);
            dKd[a] = mmab(xh, bl, dKd[a]);
            dKd[a] = mmab(xl, bh, dKd[a]);
        }
    }
    // dA_qk blocks (a, b), b <= a: wave w takes block w, waves 0 and 1 also blocks 8 and 9
    f4 dAq[2] = {zero4(), zero4()};
    const int nq = wave < 2 ? 2 : 1;
    for (int t = 0; t < nq; ++t) {
        int a, b;
        tri_ab(wave + 8 * t, a, b);
        f4 acc = zero4();
#pragma unroll
        for (int s = 0; s < DV / 32; ++s) {
            const int k0 = 32 * s + 8 * g4;
            const b8 ao = rd8(sO, 16 * a + n16, k0);
            acc = mmab(ao, rd8(sXh, 16 * b + n16, k0), acc);
            acc = mmab(ao, rd8(sXl, 16 * b + n16, k0), acc);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)  // entry (16 a + 4 g4 + jj, 16 b + n16): lower incl. the diagonal
            if (!(a > b || n16 <= 4 * g4 + jj)) acc[jj] = 0.f;
        dAq[t] = acc;
    }
    __syncthreads();  // phase 1-2 buffers free

    // ================= phase 3: the chunk-local part =================
    uint16_t *sK = reinterpret_cast<uint16_t *>(smem + kK), *sQ = reinterpret_cast<uint16_t *>(smem + kQ);
    float *sRf = reinterpret_cast<float *>(smem + kRf), *sAt = reinterpret_cast<float *>(smem + kAt);
    float *sDq = reinterpret_cast<float *>(smem + kDq), *sTd = reinterpret_cast<float *>(smem + kTd);
    char *R = smem + kR;
    for (int u = tid; u < (kTd - kAt) / 16; u += kGT) *reinterpret_cast<u4 *>(smem + kAt + 16 * u) = u4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + kGT * i, r = u >> 4, cu = u & 15;
        *reinterpret_cast<u4 *>(sK + r * LH + 8 * cu) = pk[i];
        *reinterpret_cast<u4 *>(sQ + r * LH + 8 * cu) = pq[i];
    }
    if (tid < C) sBeta[tid] = pbeta;
    // G: channel c = tid % 128, rows 16 qq .. 16 qq + 15 (rows past L add nothing)
    float gv[16];
    {
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            run += pg[i];
            gv[i] = run;
        }
        reinterpret_cast<float *>(R)[qq * DK + gc] = run;
    }
    __syncthreads();
    float GL = 0.f, off = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float x = reinterpret_cast<const float *>(R)[p * DK + gc];
        if (p < qq) off += x;
        GL += x;
    }
    if (GL < -kMaxChunkDecayG) atomicOr(sFlag, 1);
    __syncthreads();
    const bool exact = *sFlag != 0;  // beyond the factored form's range: pair by pair
    const float mh = 0.5f * GL;
#pragma unroll
    for (int i = 0; i < 16; ++i) sRf[(16 * qq + i) * LF + gc] = exact ? gv[i] + off : __expf(gv[i] + off - mh);
    if (qq == 0) sEm[gc] = exact ? GL : __expf(mh);  // e^m (an exact chunk keeps G_last here)
    for (int t = 0; t < nq; ++t) {
        int a, b;
        tri_ab(wave + 8 * t, a, b);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sDq[(16 * a + 4 * g4 + jj) * LA + 16 * b + n16] = dAq[t][jj];
    }
    __syncthreads();
    auto kv = [&](int r, int c) { return bf16_to_f32(sK[r * LH + c]); };
    auto qv = [&](int r, int c) { return bf16_to_f32(sQ[r * LH + c]); };
    // e^G and e^{G_last - G} at (r, c)
    auto eG = [&](int r, int c) { return exact ? __expf(sRf[r * LF + c]) : sRf[r * LF + c] * sEm[c]; };
    auto eD = [&](int r, int c) {
        return exact ? __expf(sEm[c] - sRf[r * LF + c]) : sEm[c] * __builtin_amdgcn_rcpf(sRf[r * LF + c]);
    };

    // ---- At = decayed k k^T, strictly lower
    if (!exact) {
        for (int t = 0; t < nq; ++t) {
            int a, b;
            tri_ab(wave + 8 * t, a, b);
            f4 acc = zero4();
            for (int s = 0; s < DK / 4; ++s) {
                const int kk = 4 * s + g4, ra = 16 * a + n16, rb = 16 * b + n16;
                const float x = kv(ra, kk) * sRf[ra * LF + kk];
                const float y = kv(rb, kk) * __builtin_amdgcn_rcpf(sRf[rb * LF + kk]);
                acc = mf(x, y, acc);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                sAt[(16 * a + 4 * g4 + jj) * LA + 16 * b + n16] = (a > b || n16 < 4 * g4 + jj) ? acc[jj] : 0.f;
        }
    } else {
        for (int e = tid; e < C * C; e += kGT) {
            const int r = e / C, i = e % C;
            if (i >= r || r >= L) continue;
            float s0 = 0.f;
            for (int c = 0; c < DK; ++c) s0 += kv(r, c) * kv(i, c) * __expf(sRf[r * LF + c] - sRf[i * LF + c]);
            sAt[r * LA + i] = s0;
        }
    }
    __syncthreads();
    // ---- diagonal blocks of T = (I + beta At)^{-1}: lane 16 a + j owns column j of T_aa
    if (wave == 0) {
        const int a = g4, j = n16;
        float tc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s0 = r == j ? 1.f : 0.f;
            const float br = sBeta[16 * a + r];
#pragma unroll
            for (int i = 0; i < r; ++i) s0 -= br * sAt[(16 * a + r) * LA + 16 * a + i] * tc[i];
            tc[r] = s0;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sTd[(16 * a + r) * LT + j] = tc[r];
    }
    __syncthreads();

    // ---- dY = T^T dX, dX = [-dWn | dV_new], by blocks from the last: Y_a = dX_a - sum_{b > a} A_ba^T dY_b,
    // dY_a = T_aa^T Y_a; each wave its own column tile of each half, tiles staged in its own LDS area
    float *sc = reinterpret_cast<float *>(R) + wave * (4 * 16 * LT);
    auto solve_t = [&](const f4 (&x)[4], f4 (&y)[4]) {
#pragma unroll
        for (int a = 3; a >= 0; --a) {
            f4 acc = zero4();
#pragma unroll
            for (int b = a + 1; b < 4; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int kk = 4 * s + g4;
                    const float av = sBeta[16 * b + kk] * sAt[(16 * b + kk) * LA + 16 * a + n16];
                    acc = mf(av, sc[(16 * b + kk) * LT + n16], acc);
                }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sc[(16 * a + 4 * g4 + jj) * LT + n16] = x[a][jj] - acc[jj];
            __builtin_amdgcn_wave_barrier();
            f4 d = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int kk = 4 * s + g4;
                d = mf(sTd[(16 * a + kk) * LT + n16], sc[(16 * a + kk) * LT + n16], d);
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sc[(16 * a + 4 * g4 + jj) * LT + n16] = d[jj];
            __builtin_amdgcn_wave_barrier();
            y[a] = d;
        }
    };
    f4 dYE[4], dYV[4];
    {
        f4 x[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) x[a] = -dWn[a];
        solve_t(x, dYE);
#pragma unroll
        for (int a = 0; a < 4; ++a) x[a] = *reinterpret_cast<const f4 *>(dVt + 4 * ((wave * 4 + a) * 64 + lane));
        solve_t(x, dYV);
    }
    __syncthreads();  // solve tiles free

    // ---- M = dY Y^T, Y = beta [E | V].  dA_kk = -(M T^T) is needed strictly below the diagonal only, which
    // reads M[r][l] for l < r alone (T^T is upper triangular): the lower blocks of M, from dY staged in LDS
    // half by half (the E columns, then the V columns), with v in the bytes M takes afterwards
    float *sY = reinterpret_cast<float *>(R), *sM = reinterpret_cast<float *>(R + C * LF * 4);
    uint16_t *sV = reinterpret_cast<uint16_t *>(sM);  // v [64][LH] bf16 until M is written
    static_assert(C * LH * 2 <= C * LA * 4, "v fits where M goes");
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + kGT * i, r = u >> 4, cu = u & 15;
        *reinterpret_cast<u4 *>(sV + r * LH + 8 * cu) = pv[i];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sY[(16 * a + 4 * g4 + jj) * LF + cw] = dYE[a][jj];
    __syncthreads();
    // dv = beta dY_V; dbeta's Y terms (row partials over this lane's column, then over the 16 columns)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * a + 4 * g4 + jj;
            if (r < L) A.dv[trow(r) + cw] = sBeta[r] * dYV[a][jj];
            float pb = dYE[a][jj] * kv(r, cw) * eG(r, cw) + dYV[a][jj] * bf16_to_f32(sV[r * LH + cw]);
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) pb += __shfl_xor(pb, m, 16);
            if (n16 == 0) sDb[wave * C + r] = pb;
        }
    f4 mt[2] = {zero4(), zero4()};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (half == 1) {
            __syncthreads();  // the E half read
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sY[(16 * a + 4 * g4 + jj) * LF + cw] = dYV[a][jj];
            __syncthreads();
        }
        for (int t = 0; t < nq; ++t) {  // blocks (a, b), b <= a, as for At
            int a, b;
            tri_ab(wave + 8 * t, a, b);
            f4 acc = mt[t];
            for (int s = 0; s < DK / 4; ++s) {
                const int kk = 4 * s + g4, ri = 16 * b + n16;
                const float y = half == 0 ? kv(ri, kk) * eG(ri, kk) : bf16_to_f32(sV[ri * LH + kk]);
                acc = mf(sY[(16 * a + n16) * LF + kk], y, acc);
            }
            mt[t] = acc;
        }
    }
    __syncthreads();  // M's operands read; its bytes are free
    for (int t = 0; t < nq; ++t) {
        int a, b;
        tri_ab(wave + 8 * t, a, b);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sM[(16 * a + 4 * g4 + jj) * LA + 16 * b + n16] = mt[t][jj] * sBeta[16 * b + n16];
    }
    __syncthreads();
    // ---- Z^T = T M^T by blocks from the first (waves 0-3, one column tile each); dA_kk = -Z (strictly lower)
    // (rows a > ct of the solve give Z above the diagonal, which is not needed, and are skipped; M's upper
    // blocks are never read)
    f4 zt[4] = {zero4(), zero4(), zero4(), zero4()};
    if (wave < 4) {
        const int ct = wave;
        float *zc = reinterpret_cast<float *>(R) + wave * (4 * 16 * LT);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            if (a > ct) break;
            f4 acc = zero4();
#pragma unroll
            for (int b = 0; b < a; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int kk = 4 * s + g4;
                    const float av = sBeta[16 * a + n16] * sAt[(16 * a + n16) * LA + 16 * b + kk];
                    acc = mf(av, zc[(16 * b + kk) * LT + n16], acc);
                }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                zc[(16 * a + 4 * g4 + jj) * LT + n16] = sM[(16 * ct + n16) * LA + 16 * a + 4 * g4 + jj] - acc[jj];
            __builtin_amdgcn_wave_barrier();
            f4 d = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int kk = 4 * s + g4;
                d = mf(sTd[(16 * a + n16) * LT + kk], zc[(16 * a + kk) * LT + n16], d);
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) zc[(16 * a + 4 * g4 + jj) * LT + n16] = d[jj];
            __builtin_amdgcn_wave_barrier();
            zt[a] = d;
        }
    }
    __syncthreads();  // M and the Z tiles consumed
    float *sDa = reinterpret_cast<float *>(R + 4 * (4 * 16 * LT) * 4);  // dA_kk [64][LA], after the Z tiles
    if (wave < 4) {
        const int ct = wave;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * a + 4 * g4 + jj, r = 16 * ct + n16;  // Z^T[i][r] = Z[r][i]
                sDa[r * LA + i] = i < r ? -zt[a][jj] : 0.f;
            }
    }
    __syncthreads();
    // dbeta: the Y terms of every wave plus sum_i dA_kk[r][i] At[r][i]
    {
        const int r = tid >> 3, part = tid & 7;
        float s0 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s0 += sDa[r * LA + 8 * part + i] * sAt[r * LA + 8 * part + i];
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) s0 += __shfl_xor(s0, m, 8);
        if (part == 0 && r < L) {
            float tot = s0;
#pragma unroll
            for (int w = 0; w < 8; ++w) tot += sDb[w * C + r];
            A.dbeta[rowb + static_cast<int64_t>(r) * H] = tot;
        }
    }

    // ---- the Gram products' gradients into this lane's column: (rows 16 a + 4 g4 + jj, column cw)
    //   dKr = sum_i dAt[r][i] Kc[i]   dKc = sum_r dAt[r][i] Kr[r]   (dAt = beta_r dA_kk, strictly lower)
    //   dQr = sum_i dAqk[r][i] Kc[i]  dKq = sum_r dAqk[r][i] Qr[r]  (lower incl. the diagonal)
    // with Kr = k e^{G - m}, Kc = k e^{m - G}, Qr = q e^{G - m}; the row factors follow below
    f4 gKr[4], gKc[4], gQr[4], gKq[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) gKr[a] = gKc[a] = gQr[a] = gKq[a] = zero4();
    if (!exact) {
        for (int s = 0; s < C / 4; ++s) {
            const int kk = 4 * s + g4;  // the contracted row (i for dKr, dQr; r for dKc, dKq)
            const float kc = kv(kk, cw) * __builtin_amdgcn_rcpf(sRf[kk * LF + cw]);
            const float kr = kv(kk, cw) * sRf[kk * LF + cw];
            const float qr = qv(kk, cw) * sRf[kk * LF + cw];
            const int sb = s >> 2;  // block of the contracted row
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int ro = 16 * a + n16;  // output row of the A operand
                if (sb <= a) {  // i <= r
                    gKr[a] = mf(sBeta[ro] * sDa[ro * LA + kk], kc, gKr[a]);
                    gQr[a] = mf(sDq[ro * LA + kk], kc, gQr[a]);
                }
                if (sb >= a) {  // r >= i
                    gKc[a] = mf(sBeta[kk] * sDa[kk * LA + ro], kr, gKc[a]);
                    gKq[a] = mf(sDq[kk * LA + ro], qr, gKq[a]);
                }
            }
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * a + 4 * g4 + jj;
                const float rf = sRf[r * LF + cw], cf = __builtin_amdgcn_rcpf(rf);
                gKr[a][jj] *= rf;
                gKc[a][jj] *= cf;
                gQr[a][jj] *= A.scale * rf;
                gKq[a][jj] *= A.scale * cf;
            }
    } else {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * a + 4 * g4 + jj;
                const float Gr = sRf[r * LF + cw];
                float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
                for (int i = 0; i < C; ++i) {
                    const float Gi = sRf[i * LF + cw];
                    if (i < r) {  // r is the later row
                        const float d = __expf(Gr - Gi);
                        s0 += sBeta[r] * sDa[r * LA + i] * kv(i, cw) * d;
                    }
                    if (i <= r) s1 += sDq[r * LA + i] * kv(i, cw) * __expf(Gr - Gi);
                    if (i > r) s2 += sBeta[i] * sDa[i * LA + r] * kv(i, cw) * __expf(Gi - Gr);  // i is the later row
                    if (i >= r) s3 += sDq[i * LA + r] * qv(i, cw) * __expf(Gi - Gr);
                }
                gKr[a][jj] = s0;
                gQr[a][jj] = A.scale * s1;
                gKc[a][jj] = s2;
                gKq[a][jj] = A.scale * s3;
            }
    }

    // ---- elementwise: dq, dk, dG; then dG_last's terms and the reverse cumulative sum into dg
    const float gam = exact ? __expf(sEm[cw]) : sEm[cw] * sEm[cw];
    float dG[4][4], cs = 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * a + 4 * g4 + jj;
            const float k_ = kv(r, cw), q_ = qv(r, cw), e = eG(r, cw), dd = eD(r, cw);
            const float E = k_ * e, Kd = k_ * dd, Qh = A.scale * q_ * e;
            const float dE = sBeta[r] * dYE[a][jj];
            const float dq = gQr[a][jj] + A.scale * e * dQh[a][jj];
            const float dk = gKr[a][jj] + gKc[a][jj] + gKq[a][jj] + e * dE + dd * dKd[a][jj];
            dG[a][jj] = k_ * gKr[a][jj] - k_ * gKc[a][jj] + q_ * gQr[a][jj] - k_ * gKq[a][jj] + dQh[a][jj] * Qh +
                        dE * E - dKd[a][jj] * Kd;
            cs += dKd[a][jj] * Kd;
            if (r < L) {
                A.dq[trow(r) + cw] = dq;
                A.dk[trow(r) + cw] = dk;
            }
        }
    // sum over the column's 64 rows (lane groups g4 hold rows 4 g4 .. of each block)
    cs += __shfl_xor(cs, 16, 64);
    cs += __shfl_xor(cs, 32, 64);
    {
        const int rl = L - 1, al = rl >> 4, gl = (rl >> 2) & 3, jl = rl & 3;
        const float add = cs + sDgam[cw] * gam;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                if (a == al && jj == jl && g4 == gl) dG[a][jj] += add;
    }
    // reverse cumulative sum over rows r = 16 a + 4 g4 + jj
    float bs[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) bs[a] = dG[a][0] + dG[a][1] + dG[a][2] + dG[a][3];
    float after[4], btot[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        float x1 = __shfl(bs[a], n16 + 16, 64), x2 = __shfl(bs[a], n16 + 32, 64), x3 = __shfl(bs[a], n16 + 48, 64);
        const float x0 = __shfl(bs[a], n16, 64);
        btot[a] = x0 + x1 + x2 + x3;
        after[a] = (g4 < 1 ? x1 : 0.f) + (g4 < 2 ? x2 : 0.f) + (g4 < 3 ? x3 : 0.f);
    }
    float later = 0.f;
#pragma unroll
    for (int a = 3; a >= 0; --a) {
        float in = 0.f;
#pragma unroll
        for (int jj = 3; jj >= 0; --jj) {
            in += dG[a][jj];
            const int r = 16 * a + 4 * g4 + jj;
            if (r < L) A.dg[trow(r) + cw] = in + after[a] + later;
        }
        later += btot[a];
    }
}

}  // namespace
}  // namespace mc

// ---------------------------------------------------------------- host
namespace {

struct BwdChunkPlan {
    ChunkGradLayout fwd;
    size_t off_rp, off_st, off_vn, off_dst, off_dvn, off_hb, off_dl, off_pt, off_pzh, off_stf, off_dstf, bytes;
};

BwdChunkPlan bwd_chunk_plan(int B, int T, int H, int N, bool varlen) {
    BwdChunkPlan p{};
    p.fwd = chunk_grad_layout(B, T, H, N, varlen);
    auto a256 = [](size_t x) { return (x + 255) & ~size_t{255}; };
    const size_t sh = static_cast<size_t>(p.fwd.max_segs) * p.fwd.per * H;  // chunk slots x heads
    const size_t seg_state = static_cast<size_t>(p.fwd.max_segs) * H * mc::DK * mc::DV * sizeof(float);
    size_t o = a256(p.fwd.bytes);
    p.off_rp = o;  o = a256(o + sh * mc::kRvBytes);
    p.off_st = o;  o = a256(o + sh * mc::DK * mc::DV * sizeof(float));
    p.off_vn = o;  o = a256(o + sh * mc::C * mc::DV * sizeof(float));
    p.off_dst = o; o = a256(o + sh * mc::DK * mc::DV * sizeof(float));
    p.off_dvn = o; o = a256(o + sh * mc::C * mc::DV * sizeof(float));
    p.off_hb = o;  o = a256(o + seg_state);
    p.off_dl = o;  o = a256(o + seg_state);
    p.off_pt = o;  o = a256(o + seg_state);  // P^T planes: the same bytes as a fp32 state
    p.off_pzh = o; o = a256(o + static_cast<size_t>(p.fwd.max_segs) * H * 8);
    p.off_stf = o; o = a256(o + sh * 8 * sizeof(int));
    p.off_dstf = o; o = a256(o + sh * 8 * sizeof(int));
    p.bytes = o;
    return p;
}

}  // namespace

bool chunk_bwd_supported(bool in_bf16, int dk, int dv) { return in_bf16 && dk == 128 && dv == 128; }

size_t chunk_bwd_workspace_bytes(int B, int T, int H, int N, bool varlen) {
    return bwd_chunk_plan(B, T, H, N, varlen).bytes;
}

bool chunk_bwd_grids_fit(int B, int T, int H, int N, bool varlen) {
    const BwdChunkPlan p = bwd_chunk_plan(B, T, H, N, varlen);
    const uint64_t blocks = static_cast<uint64_t>(p.fwd.max_segs) * p.fwd.per * H;
    return blocks * mc::kGT < (uint64_t{1} << 32) && p.fwd.packs;
}

hipError_t launch_chunk_bwd(const BackwardLaunch &L) {
    const bool varlen = L.cu_seqlens != nullptr;
    const BwdChunkPlan p = bwd_chunk_plan(L.B, L.T, L.H, L.N, varlen);
    char *ws = static_cast<char *>(L.workspace);
    ChunkLaunch c{};
    c.q = L.q; c.k = L.k; c.v = L.v; c.g = L.g; c.beta = L.beta;
    c.h0 = L.h0; c.hT = nullptr; c.o = nullptr;
    c.cu_seqlens = L.cu_seqlens;
    c.B = L.B; c.T = L.T; c.H = L.H; c.dk = mc::DK; c.dv = mc::DV; c.N = L.N;
    c.chunk = mc::C; c.scale = L.scale;
    c.in_bf16 = true; c.out_bf16 = false;
    c.xf = InputXform{};
    c.workspace = ws;
    c.workspace_bytes = p.fwd.bytes;
    c.stream = L.stream;
    ScanGrad gf{};
    gf.st = reinterpret_cast<float *>(ws + p.off_st);
    gf.vn = reinterpret_cast<float *>(ws + p.off_vn);
    gf.stf = reinterpret_cast<int *>(ws + p.off_stf);
    gf.keep_last = true;
    gf.pt = ws + p.off_pt;
    gf.pzh = reinterpret_cast<uint8_t *>(ws + p.off_pzh);
    bool chained = false;
    void *packs = nullptr;
    char *rp = ws + p.off_rp;
    const SegmentView sv = launch_chunk_grad_forward(c, gf, rp, &chained, &packs);
    const int per = p.fwd.per, max_segs = p.fwd.max_segs;
    const unsigned blocks = static_cast<unsigned>(max_segs) * static_cast<unsigned>(per) * L.H;
    hipLaunchKernelGGL(mc::rev_pack_kernel, dim3(blocks), dim3(mc::kRpThreads), 0, L.stream,
                       static_cast<const char *>(packs), rp, static_cast<const uint16_t *>(L.d_o), sv, per, L.H);
    ScanGrad gr{};
    gr.vn = reinterpret_cast<float *>(ws + p.off_dvn);
    gr.dst = reinterpret_cast<float *>(ws + p.off_dst);
    gr.dstf = reinterpret_cast<int *>(ws + p.off_dstf);
    gr.dleave = reinterpret_cast<const float *>(ws + p.off_dl);
    gr.dhT = L.dhT;
    gr.dh0 = L.dh0;
    gr.hb = reinterpret_cast<float *>(ws + p.off_hb);
    gr.pzh = gf.pzh;
    if (chained) {
        launch_scan_grad<kRevLocal>(c, sv, max_segs, per, rp, gr);
        launch_reverse_combine_bf16(sv, gf.pt, gr.hb, L.dhT, reinterpret_cast<float *>(ws + p.off_dl), L.dh0, L.H,
                                    L.N, L.stream);
    }
    launch_scan_grad<kRevOut>(c, sv, max_segs, per, rp, gr);
    mc::GradArgs A{};
    A.q = static_cast<const uint16_t *>(L.q); A.k = static_cast<const uint16_t *>(L.k);
    A.v = static_cast<const uint16_t *>(L.v); A.beta = static_cast<const uint16_t *>(L.beta);
    A.d_o = static_cast<const uint16_t *>(L.d_o); A.g = L.g;
    A.st = gf.st; A.vn = gf.vn; A.dst = gr.dst; A.dvn = gr.vn;
    A.stf = gf.stf; A.dstf = gr.dstf;
    A.dq = L.dq; A.dk = L.dk; A.dv = L.dv; A.dg = L.dg; A.dbeta = L.dbeta;
    A.per = per; A.H = L.H; A.scale = L.scale;
    hipLaunchKernelGGL(mc::chunk_grad_kernel, dim3(blocks), dim3(mc::kGT), 0, L.stream, A, sv);
    return hipGetLastError();
}

}  // namespace kda
