// kda_scan.hip - the serial part of the chunkwise KDA prefill on gfx950
// matrix cores: walking a segment's chunks in order with the fp32 state in
// MFMA accumulators (Kimi Linear review notes, section "Chunkwise Algorithm":
// only the state crosses chunk boundaries).
//
// Per chunk, from the operand pack the prep kernel wrote (kda_mfma.h):
//   X     = W S                         (a5, W = T beta e^G k)
//   V_new = U - X                       (U = T beta v)
//   o     = (scale e^G q) S + A_qk V_new                     (a6, output pass)
//   S    <- gamma * S + (e^{G_last - G} k)^T V_new           (a5)
// The pack is copied HBM -> LDS by global_load_lds (no registers), U goes
// straight to registers in accumulator order.  Each wave owns 32 state
// columns; its state and V_new are rounded to fp16 for the products with a
// power-of-two scale of its own (from the wave's maxima), so the waves never
// exchange anything but the pack in LDS.
//
// Modes: kLocal (grid 2 x segments: an H workgroup, zero start, and a P
// workgroup, identity start with v = 0, so that leaving = P entering + H)
// and kOut (replay from the entering state, write o and the final state).
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace mc {
namespace {

constexpr int NW = 4, NT = NW * kWave;
constexpr int NCT = 2;  // 16-column state tiles per wave

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

template <int MODE, bool OutBf16>
__global__ void __launch_bounds__(NT, 2)
chunk_scan_kernel(const char *__restrict__ packs, int per, float *hT, void *__restrict__ o_, SegmentView sv,
                  int H) {
    constexpr bool kOutPass = MODE == kOut;
    constexpr int kBytes = kOutPass ? kPkOut : kPkLocal;
    __shared__ __attribute__((aligned(16))) char lds[kBytes];

    const int seg = kOutPass ? blockIdx.x : (blockIdx.x >> 1);
    const bool pcols = !kOutPass && (blockIdx.x & 1);
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    if (seg >= sv.count()) return;
    const int4 sd = sv.table[seg];
    const int nseq = sd.x;
    const bool last = sd.w & kSegLast;
    if (!kOutPass && last) return;
    const int64_t t0 = sd.y, t1 = sd.z;
    const int nch = static_cast<int>((t1 - t0 + C - 1) / C);
    const int col0 = 32 * wave;  // this wave's state columns

    // a state tile element (16 rt + 4 g4 + jj, col0 + 16 ct + n16) of a
    // row-major 128 x 128 fp32 matrix: one per-lane byte offset plus a constant
    const uint32_t st_lane = 4 * (4 * g4 * 128 + col0 + n16);
    auto st_off = [](int rt, int ct, int jj) { return 4 * ((16 * rt + jj) * 128 + 16 * ct); };
    f4 acc[8][NCT];
    if (kOutPass) {
        const rsrc_t rs = make_rsrc(sv.sin + (static_cast<int64_t>(seg) * H + h) * DK * DV, 4 * DK * DV);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    acc[rt][ct][jj] = __uint_as_float(ld32(rs, st_lane, st_off(rt, ct, jj)));
    } else {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    acc[rt][ct][jj] = (pcols && 16 * rt + 4 * g4 + jj == col0 + 16 * ct + n16) ? 1.f : 0.f;
    }
    float smax = 0.f;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) smax = fmaxf(smax, fabsf(acc[rt][ct][jj]));
    smax = wave_max(smax);

    // o of the segment's tokens: element (t, c) at (t - t0) H DV + c from the
    // segment base; rows past the segment end are dropped
    const uint32_t tok_stride = static_cast<uint32_t>(H) * DV;
    const int64_t seg_base = (t0 * H + h) * DV;
    const uint32_t seg_elems = static_cast<uint32_t>((t1 - t0 - 1) * tok_stride + DV);
    constexpr int ob = OutBf16 ? 2 : 4;
    const rsrc_t rs_o = make_rsrc(static_cast<char *>(o_) + seg_base * ob, kOutPass ? ob * seg_elems : 0);

    for (int j = 0; j < nch; ++j) {
        const char *pack = packs + (static_cast<int64_t>(seg * per + j) * H + h) * kPkBytes;
        // pack -> LDS, 1 KiB per wave instruction
        for (int u = wave; u < kBytes / 1024; u += NW)
            __builtin_amdgcn_global_load_lds((gptr_t)(pack + 1024 * u + 16 * lane), (lptr_t)(lds + 1024 * u), 16, 0, 0);
        // U, accumulator order, for this wave's two column tiles
        u2 ur[NCT][4] = {};
        if (!pcols) {
            const rsrc_t rs_p = make_rsrc(pack, kPkBytes);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    ur[ct][a] = ld64(rs_p, kPkU + 8 * lane, (((2 * wave + ct) * 4 + a) * kWave) * 8);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // (1) pack in LDS

        const int *hdr = reinterpret_cast<const int *>(lds + kPkHdr);
        const int ew = hdr[kHdrW], ek = hdr[kHdrK];
        const float *gam = reinterpret_cast<const float *>(lds + kPkGamma);
        const int es = exp_of(smax);  // this wave's state, stored below 1
        const float ss = pow2(-es), unx = pow2(ew + es);
        float smax_new = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int col = col0 + 16 * ct + n16;
            h8 sb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) sb[s] = acc_to_b32(acc[2 * s][ct], acc[2 * s + 1][ct], ss, lane);
            // X = W S, Y = Q S
            f4 X[4], Y[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                X[a] = zero4();
                Y[a] = zero4();
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const h8 wa = *reinterpret_cast<const h8 *>(lds + kPkW + swz(16 * a + n16, 4 * s + g4, 2 * DK));
                    X[a] = mma32(wa, sb[s], X[a]);
                    if (kOutPass) {
                        const h8 qa = *reinterpret_cast<const h8 *>(lds + kPkQ + swz(16 * a + n16, 4 * s + g4, 2 * DK));
                        Y[a] = mma32(qa, sb[s], Y[a]);
                    }
                }
            }
            // V_new = U - X (fp32), then its own fp16 scale
            f4 Vn[4];
            float mv = 0.f;
            {
                const float unu = pcols ? 0.f : pow2(hdr[kHdrU]);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const h4 uh = __builtin_bit_cast(h4, ur[ct][a]);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float uval = pcols ? 0.f : static_cast<float>(uh[jj]) * unu;
                        Vn[a][jj] = uval - X[a][jj] * unx;
                        mv = fmaxf(mv, fabsf(Vn[a][jj]));
                    }
                }
            }
            const int evn = exp_of(wave_max(mv));
            const float svn = pow2(-evn);
            // a6: o = Q S + A_qk V_new
            if (kOutPass) {
                const float unq = pow2(hdr[kHdrQ] + es), una = pow2(hdr[kHdrA] + evn);
                h4 Vh[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) Vh[a] = to_h4(Vn[a], svn);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f4 oi = zero4();
#pragma unroll
                    for (int b = 0; b <= a; ++b) {
                        const h4 aq = *reinterpret_cast<const h4 *>(lds + kPkA + (a * (a + 1) / 2 + b) * 512 +
                                                                    n16 * 32 + g4 * 8);
                        oi = mma16(aq, Vh[b], oi);
                    }
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int rr = 16 * a + 4 * g4 + jj;
                        const float val = Y[a][jj] * unq + oi[jj] * una;
                        const uint32_t e = (static_cast<uint32_t>(C * j + rr)) * tok_stride + col;
                        if constexpr (OutBf16)
                            __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(f32_to_bf16(val)), rs_o,
                                                                  static_cast<int>(2 * e), 0, 0);
                        else
                            st32(rs_o, __float_as_uint(val), 4 * e);
                    }
                }
            }
            // a5: S <- gamma S + KT V_new
            const h8 vb0 = acc_to_b32(Vn[0], Vn[1], svn, lane), vb1 = acc_to_b32(Vn[2], Vn[3], svn, lane);
            const float down = pow2(-(ek + evn)), up = pow2(ek + evn);
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const f4 gm = *reinterpret_cast<const f4 *>(gam + 16 * rt + 4 * g4);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[rt][ct][jj] *= gm[jj] * down;
                const h8 k0 = *reinterpret_cast<const h8 *>(lds + kPkKT + swz(16 * rt + n16, g4, 2 * C));
                const h8 k1 = *reinterpret_cast<const h8 *>(lds + kPkKT + swz(16 * rt + n16, 4 + g4, 2 * C));
                acc[rt][ct] = mma32(k0, vb0, acc[rt][ct]);
                acc[rt][ct] = mma32(k1, vb1, acc[rt][ct]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    acc[rt][ct][jj] *= up;
                    smax_new = fmaxf(smax_new, fabsf(acc[rt][ct][jj]));
                }
            }
        }
        smax = wave_max(smax_new);
        __syncthreads();  // (2) LDS is refilled by the next chunk
    }

    // ---- leaving state (DK = DV: H and P are both 128 x 128)
    float *dst = nullptr;
    if (kOutPass) {
        if (last && hT) dst = hT + (static_cast<int64_t>(nseq) * H + h) * DK * DV;
    } else {
        dst = (pcols ? sv.P : sv.Hs) + (static_cast<int64_t>(seg) * H + h) * DK * DV;
    }
    if (dst) {
        const rsrc_t rs = make_rsrc(dst, 4 * DK * DV);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    st32(rs, __float_as_uint(acc[rt][ct][jj]), st_lane, st_off(rt, ct, jj));
    }
}

}  // namespace
}  // namespace mc

template <int MODE>
void launch_scan(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, const void *packs) {
    dim3 grid(MODE == kOut ? max_segs : 2 * max_segs, L.H), block(mc::NT);
    const char *pk = static_cast<const char *>(packs);
    if (L.out_bf16)
        hipLaunchKernelGGL((mc::chunk_scan_kernel<MODE, true>), grid, block, 0, L.stream, pk, per, L.hT, L.o, sv, L.H);
    else
        hipLaunchKernelGGL((mc::chunk_scan_kernel<MODE, false>), grid, block, 0, L.stream, pk, per, L.hT, L.o, sv, L.H);
}

template void launch_scan<kLocal>(const ChunkLaunch &, const SegmentView &, int, int, const void *);
template void launch_scan<kOut>(const ChunkLaunch &, const SegmentView &, int, int, const void *);

}  // namespace kda
