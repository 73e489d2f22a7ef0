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
//
// Streaming: the pack is copied HBM -> LDS by global_load_lds (no
// registers) into one of two buffers while the other one is in use, so the
// copy of chunk j + 1 overlaps the products of chunk j and a chunk costs one
// barrier; U goes straight to registers in accumulator order, also one chunk
// ahead.  Each wave owns one 16-column tile of the state.  The state and
// V_new feed the 16x16x32 products straight from the accumulator layout
// (permuted contraction index, see w_col).  They are
// rounded to fp16 with power-of-two scales of the wave's own (from its
// maxima), so waves share nothing but the pack.  o is staged in LDS per wave
// and written with 16-byte stores.
//
// Modes: kLocal, 16 waves: waves 0-7 build H (the dv columns, zero start)
// and waves 8-15 build P (the dk x dk transition: identity start, v = 0), so
// that leaving = P entering + H; kOut, 8 waves: replay from the entering
// state, write o and, for a sequence's last segment, the final state.
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace mc {
namespace {

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

template <int MODE>
struct ScanCfg {
    static constexpr int NCT = 1;                    // 16-column state tiles per wave
    static constexpr int NWH = 8 / NCT;              // waves per 128 columns
    static constexpr int NW = MODE == kOut ? NWH : 2 * NWH;
    static constexpr int NT = NW * kWave;
    static constexpr int kBytes = MODE == kOut ? kPkOut : kPkLocal;  // pack bytes staged in LDS
};

template <int MODE, bool OutBf16>
__global__ void __launch_bounds__(ScanCfg<MODE>::NT, 1)
chunk_scan_kernel(const char *__restrict__ packs, int per, float *hT, void *__restrict__ o_, SegmentView sv,
                  int H) {
    constexpr bool kOutPass = MODE == kOut;
    constexpr int NW = ScanCfg<MODE>::NW, NWH = ScanCfg<MODE>::NWH, NCT = ScanCfg<MODE>::NCT;
    constexpr int kBytes = ScanCfg<MODE>::kBytes;
    // two pack buffers as separate objects, so that the compiler can tell a
    // copy into one from reads of the other and does not wait for the copy
    __shared__ __attribute__((aligned(16))) char lds0[kBytes];
    __shared__ __attribute__((aligned(16))) char lds1[kBytes];
    // o of a chunk, per wave: 64 rows x its columns, rows padded by 16 bytes
    // (the four row groups of an accumulator tile land on different banks)
    constexpr int kStageRow = 16 * NCT * (OutBf16 ? 2 : 4) + 16;
    __shared__ __attribute__((aligned(16))) char ostage[kOutPass ? NW : 1][kOutPass ? 64 * kStageRow : 16];

    const int seg = blockIdx.x, h = blockIdx.y;
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
    const bool pcols = !kOutPass && wave >= NWH;  // this wave builds P
    const int ctile0 = NCT * (wave % NWH);         // this wave's first 16-column tile
    const int col0 = 16 * ctile0;

    // a state tile element (16 rt + 4 g4 + jj, col0 + 16 ct + n16) of a
    // row-major 128 x 128 fp32 matrix: one per-lane byte offset plus a constant
    const uint32_t st_lane = 4 * (4 * g4 * 128 + col0 + n16);
    auto st_off = [](int rt, int ct, int jj) { return 4 * ((16 * rt + jj) * 128 + 16 * ct); };
    f4 acc[8][NCT];
    if (kOutPass) {
        // a zero-sized resource reads zeros: the zero initial state
        const float *src = sv.entering(seg, sd, h, H, DK, DV);
        const rsrc_t rs = make_rsrc(src, src ? 4 * DK * DV : 0);
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
    // acc[.][ct] holds the state times 2^-fr[ct], a power-of-two frame of the
    // wave's own, kept so that |acc| stays below 96: the state then feeds the
    // fp16 products as is.  smax[ct] = max |acc|.
    int fr[NCT];
    float smax[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        float m = 0.f;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) m = fmaxf(m, fabsf(acc[rt][ct][jj]));
        m = wave_max(m);
        fr[ct] = m > 0.f ? exp_of(m) : 0;  // entering state below 1 in its frame
        const float s = pow2(-fr[ct]);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[rt][ct][jj] *= s;
        smax[ct] = m * s;
    }

    // o of the segment's tokens: element (t, c) at (t - t0) H DV + c from the
    // segment base; rows past the segment end are dropped
    const uint32_t tok_stride = static_cast<uint32_t>(H) * DV;
    const int64_t seg_base = (t0 * H + h) * DV;
    const uint32_t seg_elems = static_cast<uint32_t>((t1 - t0 - 1) * tok_stride + DV);
    constexpr int ob = OutBf16 ? 2 : 4;
    const rsrc_t rs_o = make_rsrc(static_cast<char *>(o_) + seg_base * ob, kOutPass ? ob * seg_elems : 0);

    // chunk j's pack -> dst and its U -> registers
    auto fetch = [&](int j, char *dst, u4 (&ur)[NCT][2]) {
        const char *pack = packs + (static_cast<int64_t>(seg * per + j) * H + h) * kPkBytes;
        for (int u = wave; u < kBytes / 1024; u += NW)
            __builtin_amdgcn_global_load_lds((gptr_t)(pack + 1024 * u + 16 * lane), (lptr_t)(dst + 1024 * u), 16, 0, 0);
        if (!pcols) {
            const rsrc_t rs_p = make_rsrc(pack, kPkBytes);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr)
                    ur[ct][pr] = __builtin_amdgcn_raw_buffer_load_b128(rs_p, kPkU + 16 * lane,
                                                                       u_off(ctile0 + ct, 2 * pr, 0), 0);
        }
    };
    u4 urA[NCT][2] = {}, urB[NCT][2] = {};  // U of the chunk in use / of the next one (zero for P)
    fetch(0, lds0, urA);

    // one chunk: its pack is in L, the next one's goes to Lnext
    auto step = [&](int j, const char *L, char *Lnext, const u4 (&ur_cur)[NCT][2], u4 (&ur_nxt)[NCT][2]) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // chunk j in L; every wave is done with chunk j - 1
        if (j + 1 < nch) fetch(j + 1, Lnext, ur_nxt);

        const int *hdr = reinterpret_cast<const int *>(L + kPkHdr);
        const int ew = hdr[kHdrW], ek = hdr[kHdrK];
        const float *gam = reinterpret_cast<const float *>(L + kPkGamma);
        // The accumulator layout of two 16-row state tiles is the B operand
        // layout of a 16x16x32 product with a permuted contraction index (see
        // w_col), and |acc| < 96: the state feeds products as is, in fp16.
        h8 sb[NCT][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const h4 lo = to_h4(acc[2 * p][ct], 1.f), hi = to_h4(acc[2 * p + 1][ct], 1.f);
                sb[ct][p] = h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        // X = W S, Y = Q S
        f4 X[NCT][4], Y[NCT][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                X[ct][a] = zero4();
                Y[ct][a] = zero4();
            }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const h8 wa = *reinterpret_cast<const h8 *>(L + kPkW + w_unit(16 * a + n16, p, g4));
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) X[ct][a] = mma32(wa, sb[ct][p], X[ct][a]);
                if (kOutPass) {
                    const h8 qa = *reinterpret_cast<const h8 *>(L + kPkQ + w_unit(16 * a + n16, p, g4));
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) Y[ct][a] = mma32(qa, sb[ct][p], Y[ct][a]);
                }
            }
        }
        // V_new = U - X (fp32; U = 0 for P), then the frame of the new state:
        // kept when the update fits it (V_new 2^(ek - fr) within [2^-11, 1])
        // and the state sits in [2^-6, 32], otherwise moved to the larger of
        // the update's and the state's scales.  Then |KT_h V_h| <= 64 and
        // |acc| stays below 96.
        f4 Vn[NCT][4];
        h4 Vh[NCT][4];
        int frn[NCT];
        {
            const float unu = pow2(hdr[kHdrU]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float unx = pow2(ew + fr[ct]);
                float mv = 0.f;
                if (pcols) {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            Vn[ct][a][jj] = X[ct][a][jj] * -unx;
                            mv = fmaxf(mv, fabsf(Vn[ct][a][jj]));
                        }
                } else {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const u4 w = ur_cur[ct][a >> 1];
                        const h4 uh = __builtin_bit_cast(h4, (a & 1) ? u2{w[2], w[3]} : u2{w[0], w[1]});
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            Vn[ct][a][jj] = static_cast<float>(uh[jj]) * unu - X[ct][a][jj] * unx;
                            mv = fmaxf(mv, fabsf(Vn[ct][a][jj]));
                        }
                    }
                }
                const int eu = ek + exp_of(wave_max(mv));  // |V_new| 2^ek < 2^eu
                const float sm = smax[ct];
                const bool keep = eu <= fr[ct] && fr[ct] <= eu + 10 && sm <= 32.f && sm >= 0.015625f;
                frn[ct] = keep ? fr[ct] : max(eu, sm > 0.f ? fr[ct] + exp_of(sm) : eu);
                const float svn = pow2(ek - frn[ct]);  // V_h = V_new 2^(ek - frn)
#pragma unroll
                for (int a = 0; a < 4; ++a) Vh[ct][a] = to_h4(Vn[ct][a], svn);
            }
        }
        // a6: o = Q S + A_qk V_new, staged per wave in LDS, then 16-byte stores
        if (kOutPass) {
            char *st = ostage[wave];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float unq = pow2(hdr[kHdrQ] + fr[ct]), una = pow2(hdr[kHdrA] + frn[ct] - ek);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f4 oi = zero4();
#pragma unroll
                    for (int b = 0; b <= a; ++b) {
                        const h4 aq = *reinterpret_cast<const h4 *>(L + kPkA + 512 * (a * (a + 1) / 2 + b) + 8 * lane);
                        oi = mma16(aq, Vh[ct][b], oi);
                    }
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int rr = 16 * a + 4 * g4 + jj, cc = 16 * ct + n16;
                        const float val = Y[ct][a][jj] * unq + oi[jj] * una;
                        if constexpr (OutBf16)
                            *reinterpret_cast<__bf16 *>(st + rr * kStageRow + 2 * cc) = static_cast<__bf16>(val);
                        else
                            *reinterpret_cast<float *>(st + rr * kStageRow + 4 * cc) = val;
                    }
                }
            }
            // 64 rows x this wave's columns: 16-byte units, rows past the
            // segment end dropped by the buffer range
            constexpr int kUnitsPerRow = 16 * NCT * ob / 16;
#pragma unroll
            for (int k = 0; k < 64 * kUnitsPerRow / kWave; ++k) {
                const int i = lane + kWave * k, rr = i / kUnitsPerRow, un = i % kUnitsPerRow;
                const u4 w = *reinterpret_cast<const u4 *>(st + rr * kStageRow + 16 * un);
                st128(rs_o, w, ob * ((static_cast<uint32_t>(C * j + rr)) * tok_stride + col0) + 16 * un);
            }
        }
        // a5: S <- gamma S + KT V_new in the frame frn, where the product
        // KT_h V_h = KT V_new 2^-frn needs no scaling
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if (frn[ct] == fr[ct]) {
#pragma unroll
                for (int rt = 0; rt < 8; ++rt) {
                    const f4 gm = *reinterpret_cast<const f4 *>(gam + 16 * rt + 4 * g4);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[rt][ct][jj] *= gm[jj];
                }
            } else {
                const float gsc = pow2(fr[ct] - frn[ct]);
#pragma unroll
                for (int rt = 0; rt < 8; ++rt) {
                    const f4 gm = *reinterpret_cast<const f4 *>(gam + 16 * rt + 4 * g4);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[rt][ct][jj] *= gm[jj] * gsc;
                }
                fr[ct] = frn[ct];
            }
        }
        float mx[NCT] = {};
        h8 vb[NCT][2];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const h4 lo = Vh[ct][2 * p], hi = Vh[ct][2 * p + 1];
                vb[ct][p] = h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const h8 kt = *reinterpret_cast<const h8 *>(L + kPkKT + kt_unit(16 * rt + n16, p, g4));
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = mma32(kt, vb[ct][p], acc[rt][ct]);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) mx[ct] = fmaxf(mx[ct], fabsf(acc[rt][ct][jj]));
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) smax[ct] = wave_max(mx[ct]);
    };
    for (int j = 0; j < nch; j += 2) {
        step(j, lds0, lds1, urA, urB);
        if (j + 1 < nch) step(j + 1, lds1, lds0, urB, urA);
    }

    // ---- leaving state (DK = DV: H and P are both 128 x 128)
    float *dst = nullptr;
    if (kOutPass) {
        if (last && hT) dst = hT + (static_cast<int64_t>(nseq) * H + h) * DK * DV;
    } else {
        dst = (pcols ? sv.P : sv.Hs) + (static_cast<int64_t>(seg) * H + h) * DK * DV;
    }
    if (dst && pcols) {
        // P as bf16 high and low planes (P = hi + lo to about 16 bits), the operands of the combine's
        // bf16 products: element (r, c) at 2 (128 r + c) bytes, the low plane 32 KiB further
        const rsrc_t rs = make_rsrc(dst, 4 * DK * DK);
        constexpr uint32_t kLoPlane = 2 * DK * DK;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; jj += 2) {
                    uint32_t hi, lo;
                    split2(acc[rt][ct][jj] * pow2(fr[ct]), acc[rt][ct][jj + 1] * pow2(fr[ct]), hi, lo);
                    const uint32_t o0 = (st_lane + st_off(rt, ct, jj)) / 2, o1 = (st_lane + st_off(rt, ct, jj + 1)) / 2;
                    st16(rs, hi, o0);
                    st16(rs, hi >> 16, o1);
                    st16(rs, lo, kLoPlane + o0);
                    st16(rs, lo >> 16, kLoPlane + o1);
                }
    } else if (dst) {
        const rsrc_t rs = make_rsrc(dst, 4 * DK * DV);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    st32(rs, __float_as_uint(acc[rt][ct][jj] * pow2(fr[ct])), st_lane, st_off(rt, ct, jj));
    }
}

}  // namespace
}  // namespace mc

template <int MODE>
void launch_scan(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, const void *packs) {
    dim3 grid(max_segs, L.H), block(mc::ScanCfg<MODE>::NT);
    const char *pk = static_cast<const char *>(packs);
    if (L.out_bf16)
        hipLaunchKernelGGL((mc::chunk_scan_kernel<MODE, true>), grid, block, 0, L.stream, pk, per, L.hT, L.o, sv, L.H);
    else
        hipLaunchKernelGGL((mc::chunk_scan_kernel<MODE, false>), grid, block, 0, L.stream, pk, per, L.hT, L.o, sv, L.H);
}

template void launch_scan<kLocal>(const ChunkLaunch &, const SegmentView &, int, int, const void *);
template void launch_scan<kOut>(const ChunkLaunch &, const SegmentView &, int, int, const void *);

}  // namespace kda
