// kda_chunk_f16.hip - chunkwise KDA prefill for bf16 inputs on fp16/bf16
// matrix cores (gfx950), dk = dv = 128, chunk 64.
//
// Same chunk equations as the exact-fp32 kernel (kda_chunk.hip); what differs
// is how they are mapped onto the CDNA4 compute unit:
//
// * One workgroup owns one (segment, head) and every state column, so the
//   chunk's key-side work (decay, Gram blocks, UT inverse) is done once.
//   Each wave owns a 32-column slice of the fp32 state, kept in MFMA
//   accumulators for the whole segment; waves share only the chunk's
//   key-side operands, read-only from LDS.
// * Decayed Gram blocks (a2) A_kk, A_qk: 16x16 tiles on bf16 MFMA with every
//   operand split into a bf16 high and low part (three products), so they
//   carry ~16 significant bits and bf16's exponent range.  Per 16-row block
//   a the factors are exp(G_r - G_ref) (<= 1, rows) and exp(G_ref - G_i)
//   (columns), G_ref the row before the block, formed as products of
//   exp(G) and exp(-G).  A chunk whose decay exceeds exp(-80) in some
//   channel takes an exact pair-by-pair path instead.
// * UT transform (a3/a4): only the four 16x16 diagonal blocks of
//   T = (I + A_kk)^{-1} are inverted (forward substitution, one column per
//   lane); V_new = T X' is then a blocked forward solve
//       Y_a = X'_a - sum_{b<a} A_ab V_b ,   V_a = T_aa Y_a ,
//   on 16x16x16 MFMAs, whose accumulator layout is exactly their B-operand
//   layout, so V_new never leaves registers.
// * State products (X = e^G K S, O_inter = e^G Q S, S update) on
//   16x16x32 fp16 MFMAs with fp32 accumulation.  fp16 operands carry 11
//   significant bits; their range is kept by per-chunk power-of-two scales:
//   one for k, one for scale*q, and one for the "value space" (S, V, X',
//   V_new), chosen from max|S| and max|V| with 2^11 headroom.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace f16core {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int DK = 128, DV = 128, C = 64;
constexpr int KP = DK + 8;        // half-precision row stride of [row][dk] tiles
constexpr int EP = DK + 4;        // fp32 row stride of [row][dk] tiles
constexpr int RP = C + 8;         // half-precision row stride of [dk][row] tiles
constexpr int BP = 16 + 8;        // row stride of 16x16 half blocks
constexpr float kMaxChunkDecay = 80.0f;

__device__ __forceinline__ f4 mma32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma16(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mmab(b8 a, b8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// 2^e as a float (|e| < 127)
__device__ __forceinline__ float pow2(int e) { return __int_as_float((e + 127) << 23); }

// Exponent e with m * 2^-e in [0.5, 1) for m > 0 (0 for m == 0 or denormal m).
__device__ __forceinline__ int exp_of(float m) {
    const int b = (__float_as_int(m) >> 23) & 0xff;
    return b == 0 ? 0 : b - 126;
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    const _Float16 x = static_cast<_Float16>(a), y = static_cast<_Float16>(b);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, y)) << 16);
}
__device__ __forceinline__ h4 to_h4(f4 v, float s) {
    return h4{static_cast<_Float16>(v[0] * s), static_cast<_Float16>(v[1] * s),
              static_cast<_Float16>(v[2] * s), static_cast<_Float16>(v[3] * s)};
}

__device__ __forceinline__ int bperm(int src_lane, uint32_t v) {
    return __builtin_amdgcn_ds_bpermute(src_lane << 2, static_cast<int>(v));
}

// Two vertically stacked 16x16 accumulator tiles (rows 0-15 in f0, 16-31 in
// f1; lane = 16*g + n holds rows 4g..4g+3 of column n) -> the B operand of a
// 16x16x32 product (lane = 16*g + n holds rows 8g..8g+7 of column n), scaled
// by s and rounded to fp16.  Pure cross-lane movement, no LDS storage.
__device__ __forceinline__ h8 acc_to_b32(f4 f0, f4 f1, float s, int lane) {
    const int g = lane >> 4, n = lane & 15;
    const uint32_t p0a = pack_h2(f0[0] * s, f0[1] * s), p0b = pack_h2(f0[2] * s, f0[3] * s);
    const uint32_t p1a = pack_h2(f1[0] * s, f1[1] * s), p1b = pack_h2(f1[2] * s, f1[3] * s);
    const int s0 = ((g & 1) << 5) | n, s1 = s0 + 16;
    const bool hi = g >= 2;
    // every lane takes part in every permute (a permute reading an inactive
    // lane returns garbage), then each lane keeps the tile it needs
    const int a0 = bperm(s0, p0a), a1 = bperm(s0, p1a);
    const int b0 = bperm(s0, p0b), b1 = bperm(s0, p1b);
    const int c0 = bperm(s1, p0a), c1 = bperm(s1, p1a);
    const int e0 = bperm(s1, p0b), e1 = bperm(s1, p1b);
    const int d0 = hi ? a1 : a0, d1 = hi ? b1 : b0, d2 = hi ? c1 : c0, d3 = hi ? e1 : e0;
    typedef int i4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(h8, (i4{d0, d1, d2, d3}));
}

// bf16 high/low split of 8 fp32 values
__device__ __forceinline__ void split_b8(const float *x, b8 &hi, b8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(x[e]);
        hi[e] = h;
        lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
    }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
    return x;
}

struct alignas(16) Smem {
    // R1: G -> exp(G) (fp32), later EK16 | Qs16 (half)
    union alignas(16) {
        float e[C * EP];
        struct {
            _Float16 ek[C * KP];
            _Float16 qs[C * KP];
        } h;
    } r1;
    // R2: exp(-G) (fp32), later KdT16 (half, [dk][row])
    union alignas(16) {
        float einv[C * EP];
        _Float16 kdt[DK * RP];
    } r2;
    alignas(16) uint16_t k[C * KP];       // k (bf16 bits), [row][dk]
    alignas(16) uint16_t q[C * KP];       // q (bf16 bits)
    alignas(16) uint16_t vt[DV * RP];     // v transposed (bf16 bits), [dv][row]
    float ad[4][16][17];      // diagonal blocks of A_kk (fp32, true scale)
    alignas(16) _Float16 akk[6][16 * BP]; // off-diagonal blocks of A_kk, scaled by 2^-2ek
    alignas(16) _Float16 aqk[10][16 * BP];// blocks of A_qk (incl. scale), scaled by 2^-(eq+ek)
    alignas(16) _Float16 tinv[4][16 * BP];// diagonal blocks of T, scaled by 2^-et
    float beta[C];
    float gam[DK];            // exp(G_last) per channel
    int imax[8];              // 0: |k|, 1: |scale q|, 2: |v|, 3: |S|, 4: |T|, 5: decay ok flag
};

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

template <int MODE, bool OutBf16>
__global__ void __launch_bounds__(MODE == kOut ? 256 : 512, 1)
chunk_f16_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                 const uint16_t *__restrict__ v, const float *__restrict__ g,
                 const uint16_t *__restrict__ beta, float *hT, void *__restrict__ o_,
                 SegmentView sv, int H, float scale) {
    constexpr int NW = MODE == kOut ? 4 : 8;
    constexpr int NT = NW * kWave;
    __shared__ Smem sm;

    const int seg = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, g4 = lane >> 4;
    if (seg >= sv.count()) return;
    const int4 sd = sv.table[seg];
    const int nseq = sd.x;
    const bool last = sd.w & kSegLast;
    if (MODE == kLocal && last) return;
    const int64_t t0 = sd.y, t1 = sd.z;
    // this wave's 32 state columns; in the local pass waves >= 4 build P
    const bool pcols = MODE == kLocal && wave >= 4;
    const int col0 = 32 * (wave & 3);

    // ---- state accumulators: S[16*rt + 4*g4 + jj][col0 + 16*ct + n16] = acc[rt][ct][jj]
    f4 acc[8][2];
    if (MODE == kOut) {
        const float *src = sv.sin + (static_cast<int64_t>(seg) * H + h) * DK * DV;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    acc[rt][ct][jj] = src[(16 * rt + 4 * g4 + jj) * DV + col0 + 16 * ct + n16];
    } else {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    acc[rt][ct][jj] = (pcols && 16 * rt + 4 * g4 + jj == col0 + 16 * ct + n16) ? 1.f : 0.f;
    }
    float smax = 0.f;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) smax = fmaxf(smax, fabsf(acc[rt][ct][jj]));

    typename Elem<OutBf16>::T *o = static_cast<typename Elem<OutBf16>::T *>(o_);

    for (int64_t c0 = t0; c0 < t1; c0 += C) {
        const int L = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);
        // ================= load (a1 input) =================
        if (tid < 8) sm.imax[tid] = 0;
        __syncthreads();
        {
            smax = wave_max(smax);
            if (lane == 0) atomicMax(&sm.imax[3], __float_as_int(smax));
        }
        float mk = 0.f, mq = 0.f, mv = 0.f;
        // g: 64 x 128 fp32 as float4
        for (int e = tid; e < C * DK / 4; e += NT) {
            const int r = e / (DK / 4), c4 = (e % (DK / 4)) * 4;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < L) x = *reinterpret_cast<const float4 *>(g + ((c0 + r) * H + h) * DK + c4);
            *reinterpret_cast<float4 *>(&sm.r1.e[r * EP + c4]) = x;
        }
        // k, q, v: 64 x 128 bf16 as 8-element vectors
        for (int e = tid; e < C * DK / 8; e += NT) {
            const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            uint4 xk = make_uint4(0, 0, 0, 0), xq = xk, xv = xk;
            if (r < L) {
                const int64_t base = ((c0 + r) * H + h) * DK + c8;
                xk = *reinterpret_cast<const uint4 *>(k + base);
                if (MODE == kOut) xq = *reinterpret_cast<const uint4 *>(q + base);
                xv = *reinterpret_cast<const uint4 *>(v + base);
            }
            *reinterpret_cast<uint4 *>(&sm.k[r * KP + c8]) = xk;
            *reinterpret_cast<uint4 *>(&sm.q[r * KP + c8]) = xq;
            const uint32_t wv[4] = {xv.x, xv.y, xv.z, xv.w};
            const uint32_t wk[4] = {xk.x, xk.y, xk.z, xk.w};
            const uint32_t wq[4] = {xq.x, xq.y, xq.z, xq.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float v0 = bf16_to_f32(wv[u] & 0xffff), v1 = bf16_to_f32(wv[u] >> 16);
                sm.vt[(c8 + 2 * u) * RP + r] = static_cast<uint16_t>(wv[u] & 0xffff);
                sm.vt[(c8 + 2 * u + 1) * RP + r] = static_cast<uint16_t>(wv[u] >> 16);
                mv = fmaxf(mv, fmaxf(fabsf(v0), fabsf(v1)));
                mk = fmaxf(mk, fmaxf(fabsf(bf16_to_f32(wk[u] & 0xffff)), fabsf(bf16_to_f32(wk[u] >> 16))));
                mq = fmaxf(mq, fmaxf(fabsf(bf16_to_f32(wq[u] & 0xffff)), fabsf(bf16_to_f32(wq[u] >> 16))));
            }
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
        __syncthreads();
        // ================= a1: chunk-local cumulative decay =================
        {
            constexpr int PARTS = NT / DK, RPP = C / PARTS;
            const int c = tid % DK, part = tid / DK;
            float run = 0.f;
#pragma unroll 4
            for (int m = 0; m < RPP; ++m) {
                float &x = sm.r1.e[(part * RPP + m) * EP + c];
                run += x;
                x = run;
            }
            __syncthreads();
            float off = 0.f;
            for (int pp = 0; pp < part; ++pp) off += sm.r1.e[((pp + 1) * RPP - 1) * EP + c];
            __syncthreads();
            if (part > 0) {
                for (int m = 0; m < RPP; ++m) sm.r1.e[(part * RPP + m) * EP + c] += off;
            }
            __syncthreads();
            // decay range check (the last row holds the most negative G), then
            // exp(G) in place and exp(-G)
            if (part == 0 && sm.r1.e[(C - 1) * EP + c] < -kMaxChunkDecay) atomicOr(&sm.imax[5], 1);
            if (part == 0) sm.gam[c] = __expf(sm.r1.e[(C - 1) * EP + c]);
        }
        __syncthreads();
        const bool exact_path = sm.imax[5] != 0;
        const int ek = exp_of(__int_as_float(sm.imax[0]));
        const int eq = exp_of(__int_as_float(sm.imax[1]));
        const float vmax = fmaxf(__int_as_float(sm.imax[2]), __int_as_float(sm.imax[3]));
        const int ev = exp_of(vmax) - 5;  // value-space operands below 2^5
        const float sk = pow2(-ek), sq = pow2(-eq) * scale, sv_ = pow2(-ev);
        if (!exact_path) {
            for (int e = tid; e < C * DK; e += NT) {
                const int r = e / DK, c = e % DK;
                const float G = sm.r1.e[r * EP + c];
                sm.r2.einv[r * EP + c] = __expf(-G);
                sm.r1.e[r * EP + c] = __expf(G);
            }
        }
        __syncthreads();

        // ================= a2: A_kk, A_qk tiles =================
        {
            constexpr int NPAIR = 10;
            for (int p = wave; p < NPAIR; p += NW) {
                int a, b;
                pair_ab(p, a, b);
                const int r = 16 * a + n16, i = 16 * b + n16;
                const int ref = 16 * a - 1;
                f4 akk = zero4(), aqk = zero4();
                if (!exact_path) {
#pragma unroll
                    for (int s = 0; s < DK / 32; ++s) {
                        const int cb = 32 * s + 8 * g4;
                        float xr[8], xq[8], xc[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int c = cb + e;
                            const float einv_ref = ref >= 0 ? sm.r2.einv[ref * EP + c] : 1.f;
                            const float e_ref = ref >= 0 ? sm.r1.e[ref * EP + c] : 1.f;
                            const float rf = sm.r1.e[r * EP + c] * einv_ref;       // exp(G_r - G_ref) <= 1
                            const float cf = e_ref * sm.r2.einv[i * EP + c];       // exp(G_ref - G_i)
                            xr[e] = bf16_to_f32(sm.k[r * KP + c]) * rf * sk;
                            xq[e] = bf16_to_f32(sm.q[r * KP + c]) * rf * sq;
                            xc[e] = bf16_to_f32(sm.k[i * KP + c]) * cf * sk;
                        }
                        b8 rh, rl, qh, ql, ch, cl;
                        split_b8(xr, rh, rl);
                        split_b8(xc, ch, cl);
                        akk = mmab(rh, ch, akk);
                        akk = mmab(rh, cl, akk);
                        akk = mmab(rl, ch, akk);
                        if (MODE == kOut) {
                            split_b8(xq, qh, ql);
                            aqk = mmab(qh, ch, aqk);
                            aqk = mmab(qh, cl, aqk);
                            aqk = mmab(ql, ch, aqk);
                        }
                    }
                } else {
                    // exact path: exp(G_r - G_i) pair by pair, fp32
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int rr = 16 * a + 4 * g4 + jj, ii = 16 * b + n16;
                        float vk = 0.f, vq = 0.f;
                        if (ii <= rr) {
                            for (int c = 0; c < DK; ++c) {
                                const float d = __expf(sm.r1.e[rr * EP + c] - sm.r1.e[ii * EP + c]);
                                const float kk = bf16_to_f32(sm.k[ii * KP + c]) * d;
                                vk += bf16_to_f32(sm.k[rr * KP + c]) * kk;
                                vq += bf16_to_f32(sm.q[rr * KP + c]) * kk;
                            }
                        }
                        akk[jj] = vk * sk * sk;
                        aqk[jj] = vq * sk * sq;
                    }
                }
                const float unk = pow2(2 * ek);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rl = 4 * g4 + jj, rr = 16 * a + rl, ii = 16 * b + n16;
                    const float vk = ii < rr ? sm.beta[rr] * akk[jj] : 0.f;
                    const float vq = ii <= rr ? aqk[jj] : 0.f;
                    if (a == b) sm.ad[a][rl][n16] = vk * unk;
                    else sm.akk[offdiag_index(a, b)][rl * BP + n16] = static_cast<_Float16>(vk);
                    if (MODE == kOut) sm.aqk[p][rl * BP + n16] = static_cast<_Float16>(vq);
                }
            }
        }
        __syncthreads();

        // ================= a3: diagonal blocks of T; key-side operands =================
        // wave 0: T_aa = (I + A_aa)^{-1}, lane 16a + j owns column j of block a
        float tcol[16];
        if (wave == 0) {
            const int a = g4, j = n16;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) s -= sm.ad[a][r][i] * tcol[i];
                tcol[r] = s;
            }
            float tm = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) tm = fmaxf(tm, fabsf(tcol[r]));
            tm = wave_max(tm);
            if (lane == 0) sm.imax[4] = __float_as_int(tm);
        }
        // every thread: its share of e^G K, scale e^G Q, (e^{G_L - G} K)^T
        constexpr int PER = C * DK / NT;
        _Float16 hk[PER], hq[PER], hd[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + NT * u, r = e / DK, c = e % DK;
            const float kk = bf16_to_f32(sm.k[r * KP + c]);
            float E, Ed;
            if (!exact_path) {
                E = sm.r1.e[r * EP + c];
                Ed = sm.gam[c] * sm.r2.einv[r * EP + c];
            } else {
                E = __expf(sm.r1.e[r * EP + c]);
                Ed = __expf(sm.r1.e[(C - 1) * EP + c] - sm.r1.e[r * EP + c]);
            }
            hk[u] = static_cast<_Float16>(kk * E * sk);
            hq[u] = static_cast<_Float16>(bf16_to_f32(sm.q[r * KP + c]) * E * sq);
            hd[u] = static_cast<_Float16>(kk * Ed * sk);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + NT * u, r = e / DK, c = e % DK;
            sm.r1.h.ek[r * KP + c] = hk[u];
            if (MODE == kOut) sm.r1.h.qs[r * KP + c] = hq[u];
            sm.r2.kdt[c * RP + r] = hd[u];
        }
        const int et = exp_of(__int_as_float(sm.imax[4]));
        if (wave == 0) {
            const float st = pow2(-et);
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.tinv[g4][r * BP + n16] = static_cast<_Float16>(tcol[r] * st);
        }
        __syncthreads();

        // ================= scan: this wave's 32 columns =================
        // B operands of S for the dk contraction (4 steps of 32 rows, 2 column tiles)
        h8 sb[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) sb[s][ct] = acc_to_b32(acc[2 * s][ct], acc[2 * s + 1][ct], sv_, lane);
        // X = (e^G K) S  and  Y = (scale e^G Q) S
        f4 X[4][2], Y[4][2];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                X[a][ct] = zero4();
                Y[a][ct] = zero4();
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const h8 ak = *reinterpret_cast<const h8 *>(&sm.r1.h.ek[(16 * a + n16) * KP + 32 * s + 8 * g4]);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) X[a][ct] = mma32(ak, sb[s][ct], X[a][ct]);
                if (MODE == kOut) {
                    const h8 aq = *reinterpret_cast<const h8 *>(&sm.r1.h.qs[(16 * a + n16) * KP + 32 * s + 8 * g4]);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) Y[a][ct] = mma32(aq, sb[s][ct], Y[a][ct]);
                }
            }
        }
        // X' = beta (V - X), then the blocked forward solve V_new = T X'
        const float unx = pow2(ek + ev);
        const float uns = pow2(2 * ek + ev);
        const float unt = pow2(et + ev);
        f4 Vn[4][2];
        h4 Vh[4][2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int col = col0 + 16 * ct + n16;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f4 xp;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rr = 16 * a + 4 * g4 + jj;
                    const float vv = pcols ? 0.f : bf16_to_f32(sm.vt[col * RP + rr]);
                    xp[jj] = sm.beta[rr] * (vv - X[a][ct][jj] * unx);
                }
                f4 accs = zero4();
#pragma unroll
                for (int b = 0; b < a; ++b) {
                    const h4 aab = *reinterpret_cast<const h4 *>(&sm.akk[offdiag_index(a, b)][n16 * BP + 4 * g4]);
                    accs = mma16(aab, Vh[b][ct], accs);
                }
                f4 yv;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) yv[jj] = xp[jj] - accs[jj] * uns;
                const h4 ta = *reinterpret_cast<const h4 *>(&sm.tinv[a][n16 * BP + 4 * g4]);
                f4 va = mma16(ta, to_h4(yv, sv_), zero4());
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) va[jj] *= unt;
                Vn[a][ct] = va;
                Vh[a][ct] = to_h4(va, sv_);
            }
        }
        // ================= a6: O = scale e^G Q S + A_qk V_new =================
        if (MODE == kOut) {
            const float unq = pow2(eq + ev), unqk = pow2(eq + ek + ev);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int col = col0 + 16 * ct + n16;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f4 oi = zero4();
#pragma unroll
                    for (int b = 0; b <= a; ++b) {
                        const int p = a * (a + 1) / 2 + b;
                        const h4 aq = *reinterpret_cast<const h4 *>(&sm.aqk[p][n16 * BP + 4 * g4]);
                        oi = mma16(aq, Vh[b][ct], oi);
                    }
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int rr = 16 * a + 4 * g4 + jj;
                        if (rr < L)
                            Elem<OutBf16>::store(o, ((c0 + rr) * H + h) * static_cast<int64_t>(DV) + col,
                                                 Y[a][ct][jj] * unq + oi[jj] * unqk);
                    }
                }
            }
        }
        // ================= a5: S <- e^{G_L} S + (e^{G_L - G} K)^T V_new =================
        {
            h8 vb[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) vb[s][ct] = acc_to_b32(Vn[2 * s][ct], Vn[2 * s + 1][ct], sv_, lane);
            const float down = pow2(-(ek + ev)), up = pow2(ek + ev);
            smax = 0.f;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                float gr[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) gr[jj] = sm.gam[16 * rt + 4 * g4 + jj] * down;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[rt][ct][jj] *= gr[jj];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const h8 ad = *reinterpret_cast<const h8 *>(&sm.r2.kdt[(16 * rt + n16) * RP + 32 * s + 8 * g4]);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mma32(ad, vb[s][ct], acc[rt][ct]);
                }
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        acc[rt][ct][jj] *= up;
                        smax = fmaxf(smax, fabsf(acc[rt][ct][jj]));
                    }
            }
        }
        __syncthreads();  // LDS of this chunk is reused by the next
    }

    // ---- leaving state
    float *dst = nullptr;
    int ld = DV;
    if (MODE == kOut) {
        if (last && hT) dst = hT + (static_cast<int64_t>(nseq) * H + h) * DK * DV;
    } else {
        dst = (pcols ? sv.P : sv.Hs) + (static_cast<int64_t>(seg) * H + h) * DK * (pcols ? DK : DV);
        ld = pcols ? DK : DV;
    }
    if (dst) {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    dst[static_cast<int64_t>(16 * rt + 4 * g4 + jj) * ld + col0 + 16 * ct + n16] = acc[rt][ct][jj];
    }
}

}  // namespace f16core

bool f16_pass_supported(const ChunkLaunch &L) {
    return L.in_bf16 && L.dk == 128 && L.dv == 128 && L.chunk == 64;
}

template <int MODE>
void launch_f16_pass(const ChunkLaunch &L, const SegmentView &sv, int max_segs) {
    dim3 grid(max_segs, L.H), block(MODE == kOut ? 256 : 512);
    const uint16_t *q = static_cast<const uint16_t *>(L.q), *k = static_cast<const uint16_t *>(L.k);
    const uint16_t *v = static_cast<const uint16_t *>(L.v), *b = static_cast<const uint16_t *>(L.beta);
    if (L.out_bf16)
        hipLaunchKernelGGL((f16core::chunk_f16_kernel<MODE, true>), grid, block, 0, L.stream, q, k, v, L.g, b,
                           L.hT, L.o, sv, L.H, L.scale);
    else
        hipLaunchKernelGGL((f16core::chunk_f16_kernel<MODE, false>), grid, block, 0, L.stream, q, k, v, L.g, b,
                           L.hT, L.o, sv, L.H, L.scale);
}

template void launch_f16_pass<kLocal>(const ChunkLaunch &, const SegmentView &, int);
template void launch_f16_pass<kOut>(const ChunkLaunch &, const SegmentView &, int);

}  // namespace kda
