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
// maxima), so waves share nothing but the pack.  A bf16 o is staged in LDS
// for the whole workgroup and stored one chunk later, after the next
// barrier, as whole 256-byte rows with the non-temporal hint (each wave
// holds only 32 bytes of a row, and partial-line writes from several waves
// cost HBM time); an fp32 o is staged per wave and stored at once.
//
// Modes: kLocal, 16 waves: waves 0-7 build H (the dv columns, zero start)
// and waves 8-15 build P (the dk x dk transition: identity start, v = 0), so
// that leaving = P entering + H; kOut, 8 waves: replay from the entering
// state, write o and, for a sequence's last segment, the final state.
//
// The gradients use three more (8 waves each).  kStates replays like kOut but
// keeps every chunk's entering state and V_new instead of writing o.  The
// reverse modes walk a segment's chunks last to first over the reverse pack
// (kda_mfma.h) with the state gradient dS in the accumulators: the step is
// the forward one with U <- A_qk^T dO, W <- -Kd, KT <- -W^T and one more
// product Q^T dO in the update.  kRevLocal starts from zero at the segment end
// and leaves Hb (dS_enter = P^T dS_leave + Hb); kRevOut starts from the
// segment's true leaving gradient, keeps each chunk's dS and dV_new, and
// writes the initial-state gradient at a sequence's first segment.
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace mc {
namespace {

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

// chunks at a segment's end the local pass walks first (the rest only if their transition is not zero)
constexpr int kTail = 4;

template <int MODE>
struct ScanCfg {
    static constexpr bool kRev = MODE == kRevLocal || MODE == kRevOut;
    static constexpr int NCT = 1;                    // 16-column state tiles per wave
    static constexpr int NWH = 8 / NCT;              // waves per 128 columns
    static constexpr int NW = MODE == kLocal ? 2 * NWH : NWH;
    static constexpr int NT = NW * kWave;
    // pack bytes staged in LDS, and the stride of the packs
    static constexpr int kBytes = MODE == kOut ? kPkOut : (kRev ? kRvStage : kPkLocal);
    static constexpr int kStride = kRev ? kRvBytes : kPkBytes;
};

template <int MODE, bool OutBf16>
__global__ void __launch_bounds__(ScanCfg<MODE>::NT, 1)
chunk_scan_kernel(const char *__restrict__ packs, int per, float *hT, void *__restrict__ o_, SegmentView sv,
                  int H, ScanGrad gr, int redo) {
    constexpr bool kOutPass = MODE == kOut;
    constexpr bool kRev = ScanCfg<MODE>::kRev;
    constexpr bool kReplay = MODE == kOut || MODE == kStates || MODE == kRevOut;  // from a true boundary state
    constexpr bool kKeep = MODE == kStates || MODE == kRevOut;                     // per-chunk states kept
    constexpr int NW = ScanCfg<MODE>::NW, NWH = ScanCfg<MODE>::NWH, NCT = ScanCfg<MODE>::NCT;
    constexpr int kBytes = ScanCfg<MODE>::kBytes, kStride = ScanCfg<MODE>::kStride;
    // two pack buffers as separate objects, so that the compiler can tell a
    // copy into one from reads of the other and does not wait for the copy
    __shared__ __attribute__((aligned(16))) char lds0[kBytes];
    __shared__ __attribute__((aligned(16))) char lds1[kBytes];
    // o of a chunk, per wave: 64 rows x its columns, rows padded by 16 bytes
    // (the four row groups of an accumulator tile land on different banks)
    constexpr bool kRowsOut = kOutPass && OutBf16;  // bf16 o: whole-workgroup rows, two chunks in turn
    constexpr int kStageRow = 16 * NCT * (OutBf16 ? 2 : 4) + 16;
    constexpr int kRowBytes = 2 * DV + 16;
    __shared__ __attribute__((aligned(16))) char ostage[kOutPass && !kRowsOut ? NW : 1]
                                                       [kOutPass && !kRowsOut ? 64 * kStageRow : 16];
    __shared__ __attribute__((aligned(16))) char orows[kRowsOut ? 2 : 1][kRowsOut ? 64 * kRowBytes : 16];

    const int seg = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    if (seg >= sv.count()) return;
    const int4 sd = sv.desc(seg);
    const int nseq = sd.x;
    const bool last = sd.w & kSegLast, first = sd.w & kSegFirst;
    // a last segment's P and H serve only the reverse combine; a one-segment sequence needs neither
    if (MODE == kLocal && last && (first || !gr.keep_last)) return;
    if (MODE == kRevLocal && first) return;  // Hb of a first segment is never used
    const int64_t t0 = sd.y, t1 = sd.z;
    const int nch = static_cast<int>((t1 - t0 + C - 1) / C);
    // The local pass first walks only a segment's last kTail chunks (redo = 0).  If the transition over them,
    // P_tail, is exactly zero (it underflows fp32: strong gates forget within a few chunks), then the segment's
    // P = P_tail P_head is zero as well, and H = P_tail H_head + H_tail is H_tail, the state those chunks reach
    // from zero: the earlier chunks' part lies below fp32's range, just as a zero P drops the entering state in
    // the combine.  The flags in sv.pz record whether P_tail is zero; a second launch (redo = 1) walks the
    // whole of every segment whose tail transition is not.
    __shared__ int s_live;  // kLocal: some P tile of the tail walk is not zero
    if (MODE == kLocal && tid == 0) s_live = 0;
    // The gradients' reverse local pass walks a segment last to first from zero at its end.  Where the forward
    // transition over the segment's first kTail chunks is exactly zero, the chunks after them reach the segment's
    // start only through that transition's transpose, so the walk takes those first chunks alone.  The forward
    // local pass finds that transition in a second grid layer (blockIdx.z = 1, P waves only, flags in gr.pzh).
    const bool head = MODE == kLocal && blockIdx.z == 1;
    int i0 = 0, iend = nch;  // the walked steps
    if constexpr (MODE == kLocal) {
        if (head) {
            if (nch <= kTail || !gr.pzh) return;
            iend = kTail;
        } else {
            const bool tail = nch > kTail && sv.pz;
            if (redo && (!tail || *reinterpret_cast<const uint64_t *>(sv.pz + (static_cast<int64_t>(seg) * H + h) * 8) ==
                                      0x0101010101010101ull))
                return;
            if (!redo && tail) i0 = nch - kTail;
        }
    }
    if constexpr (MODE == kRevLocal) {
        if (gr.pzh && nch > kTail &&
            *reinterpret_cast<const uint64_t *>(gr.pzh + (static_cast<int64_t>(seg) * H + h) * 8) == 0x0101010101010101ull)
            i0 = nch - kTail;
    }
    const bool pcols = MODE == kLocal && wave >= NWH;  // this wave builds P
    const int ctile0 = NCT * (wave % NWH);         // this wave's first 16-column tile
    const int col0 = 16 * ctile0;

    // a state tile element (16 rt + 4 g4 + jj, col0 + 16 ct + n16) of a
    // row-major 128 x 128 fp32 matrix: one per-lane byte offset plus a constant
    const uint32_t st_lane = 4 * (4 * g4 * 128 + col0 + n16);
    auto st_off = [](int rt, int ct, int jj) { return 4 * ((16 * rt + jj) * 128 + 16 * ct); };
    f4 acc[8][NCT];
    if (kReplay) {
        // a zero-sized resource reads zeros: the zero initial state (or final-state gradient)
        const float *src;
        if constexpr (MODE == kRevOut) {
            // the gradient leaving a segment whose successor's P is exactly zero is that successor's Hb (the
            // reverse combine leaves it unwritten when a sequence has no nonzero P)
            if (first && last) src = gr.dhT ? gr.dhT + (static_cast<int64_t>(nseq) * H + h) * DK * DV : nullptr;
            else if (!last && sv.pz_all(seg + 1, h, H)) src = gr.hb + (static_cast<int64_t>(seg + 1) * H + h) * DK * DV;
            else src = gr.dleave + (static_cast<int64_t>(seg) * H + h) * DK * DV;
        } else {
            src = sv.entering(seg, sd, h, H, DK, DV);
        }
        const rsrc_t rs = make_rsrc(src, src ? 4 * DK * DV : 0);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    acc[rt][ct][jj] = __uint_as_float(ld32(rs, st_lane, st_off(rt, ct, jj)));
    } else {  // H from zero, P from the identity
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

    // chunk j's pack -> dst and its U (and, reversed, dO) -> registers
    auto fetch = [&](int j, char *dst, u4 (&ur)[NCT][2], u4 (&dr)[NCT][2], u4 (&ul)[NCT][2]) {
        const char *pack = packs + (static_cast<int64_t>(seg * per + j) * H + h) * kStride;
        for (int u = wave; u < kBytes / 1024; u += NW)
            __builtin_amdgcn_global_load_lds((gptr_t)(pack + 1024 * u + 16 * lane), (lptr_t)(dst + 1024 * u), 16, 0, 0);
        if (!pcols) {
            const rsrc_t rs_p = make_rsrc(pack, kStride);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    ur[ct][pr] = __builtin_amdgcn_raw_buffer_load_b128(rs_p, kPkU + 16 * lane,
                                                                       u_off(ctile0 + ct, 2 * pr, 0), 0);
                    if (kRev) {
                        dr[ct][pr] = __builtin_amdgcn_raw_buffer_load_b128(rs_p, kRvDO + 16 * lane,
                                                                           u_off(ctile0 + ct, 2 * pr, 0), 0);
                        ul[ct][pr] = __builtin_amdgcn_raw_buffer_load_b128(rs_p, kRvUL + 16 * lane,
                                                                           u_off(ctile0 + ct, 2 * pr, 0), 0);
                    }
                }
        }
    };
    // the i-th chunk walked: first to last, or last to first in the reverse modes
    auto chunk_of = [&](int i) { return kRev ? nch - 1 - i : i; };
    // bf16 o of chunk j from orows[j & 1]: 16 lanes per 256-byte row
    auto store_rows = [&](int j) {
        const char *src = orows[j & 1];
#pragma unroll
        for (int k = 0; k < 64 * 16 / ScanCfg<MODE>::NT; ++k) {
            const int u = tid + ScanCfg<MODE>::NT * k, rr = u >> 4, cu = u & 15;
            const u4 w = *reinterpret_cast<const u4 *>(src + rr * kRowBytes + 16 * cu);
            st128_nt(rs_o, w, 2 * (static_cast<uint32_t>(C * j + rr) * tok_stride) + 16 * cu);
        }
    };
    // U (and dO) of the chunk in use / of the next one (zero for P)
    u4 urA[NCT][2] = {}, urB[NCT][2] = {}, drA[NCT][2] = {}, drB[NCT][2] = {}, ulA[NCT][2] = {}, ulB[NCT][2] = {};

    // one chunk: its pack is in L, the next one's goes to Lnext
    auto step = [&](int i, const char *L, char *Lnext, const u4 (&ur_cur)[NCT][2], u4 (&ur_nxt)[NCT][2],
                    const u4 (&dr_cur)[NCT][2], u4 (&dr_nxt)[NCT][2], const u4 (&ul_cur)[NCT][2],
                    u4 (&ul_nxt)[NCT][2]) {
        const int j = chunk_of(i);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // chunk j in L; every wave is done with the previous chunk
        if (i + 1 < iend) fetch(chunk_of(i + 1), Lnext, ur_nxt, dr_nxt, ul_nxt);
        if constexpr (kRowsOut)  // every wave's part of the previous chunk's o is in orows now
            if (i > 0) store_rows(j - 1);
        // A P tile that has decayed to exactly zero stays zero (gamma 0 + KT (0 - W 0) = 0), so its wave only
        // takes its share of the copies from here on.  Under strong gates P underflows within a few chunks.
        if constexpr (MODE == kLocal)
            if (pcols ? smax[0] == 0.f : head) return;  // the head layer builds P only

        const int *hdr = reinterpret_cast<const int *>(L + kPkHdr);
        const int ew = hdr[kHdrW], ek = hdr[kHdrK];
        const float *gam = reinterpret_cast<const float *>(L + kPkGamma);
        const int64_t slot = (static_cast<int64_t>(seg) * per + j) * H + h;
        if constexpr (kKeep) {
            // the state entering chunk j (forward) or the gradient of the one leaving it, as the fp16 operand the
            // walk itself multiplies with (|acc| < 96 in the wave's frame) and the frame's exponent per tile
            h4 *sd_ = reinterpret_cast<h4 *>((MODE == kStates ? gr.st : gr.dst) + slot * (DK * DV));
            int *sf = (MODE == kStates ? gr.stf : gr.dstf) + slot * 8;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                if (lane == 0) sf[ctile0 + ct] = fr[ct];
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)  // whole 512-byte pieces, read once much later: non-temporal
                    __builtin_nontemporal_store(to_h4(acc[rt][ct], 1.f), sd_ + ((ctile0 + ct) * 8 + rt) * 64 + lane);
            }
        }
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
                    const float unl = kRev ? pow2(hdr[kHdrUL]) : 0.f;
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const u4 w = ur_cur[ct][a >> 1];
                        const h4 uh = __builtin_bit_cast(h4, (a & 1) ? u2{w[2], w[3]} : u2{w[0], w[1]});
                        const u4 wl = ul_cur[ct][a >> 1];
                        const h4 ulh = __builtin_bit_cast(h4, (a & 1) ? u2{wl[2], wl[3]} : u2{wl[0], wl[1]});
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            float u = static_cast<float>(uh[jj]) * unu;
                            if (kRev) u += static_cast<float>(ulh[jj]) * unl;  // A_qk^T dO to about 22 bits
                            Vn[ct][a][jj] = u - X[ct][a][jj] * unx;
                            mv = fmaxf(mv, fabsf(Vn[ct][a][jj]));
                        }
                    }
                }
                int eu = ek + exp_of(wave_max(mv));  // |V_new| 2^ek < 2^eu
                // reversed: the frame also holds Q^T dO (Q^T stored < 1, dO < 2^(e_dO + e_q) in the frame's units)
                if (kRev) eu = max(eu, hdr[kHdrQ] + hdr[kHdrDO]);
                const float sm = smax[ct];
                const bool keep = eu <= fr[ct] && fr[ct] <= eu + 10 && sm <= 32.f && sm >= 0.015625f;
                frn[ct] = keep ? fr[ct] : max(eu, sm > 0.f ? fr[ct] + exp_of(sm) : eu);
                const float svn = pow2(ek - frn[ct]);  // V_h = V_new 2^(ek - frn)
#pragma unroll
                for (int a = 0; a < 4; ++a) Vh[ct][a] = to_h4(Vn[ct][a], svn);
                if constexpr (kKeep) {  // V_new (forward) or dV_new (reversed), true scale
                    float *vd = gr.vn + slot * (C * DV);
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        f4 *dst4 = reinterpret_cast<f4 *>(vd + 4 * (((ctile0 + ct) * 4 + a) * 64 + lane));
                        __builtin_nontemporal_store(Vn[ct][a], dst4);
                    }
                }
            }
        }
        // reversed: dO in the new frame, dO 2^(e_q - frn), as the B operand of the extra product
        h8 db[NCT][2];
        if constexpr (kRev) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float sdo = pow2(hdr[kHdrDO] + hdr[kHdrQ] - frn[ct]);
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const h8 d = __builtin_bit_cast(h8, dr_cur[ct][pr]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) db[ct][pr][e] = static_cast<_Float16>(static_cast<float>(d[e]) * sdo);
                }
            }
        }
        // a6: o = Q S + A_qk V_new, staged in LDS, then 16-byte stores
        if (kOutPass) {
            char *st = kRowsOut ? orows[j & 1] : ostage[wave];
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
                        if constexpr (kRowsOut)
                            *reinterpret_cast<__bf16 *>(st + rr * kRowBytes + 2 * (col0 + cc)) =
                                static_cast<__bf16>(val);
                        else if constexpr (OutBf16)
                            *reinterpret_cast<__bf16 *>(st + rr * kStageRow + 2 * cc) = static_cast<__bf16>(val);
                        else
                            *reinterpret_cast<float *>(st + rr * kStageRow + 4 * cc) = val;
                    }
                }
            }
            if constexpr (!kRowsOut) {
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
                if constexpr (kRev) {
                    const h8 qt = *reinterpret_cast<const h8 *>(L + kPkQ + kt_unit(16 * rt + n16, p, g4));
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = mma32(qt, db[ct][p], acc[rt][ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) mx[ct] = fmaxf(mx[ct], fabsf(acc[rt][ct][jj]));
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) smax[ct] = wave_max(mx[ct]);
    };
    fetch(chunk_of(i0), lds0, urA, drA, ulA);
    for (int i = i0; i < iend; i += 2) {
        step(i, lds0, lds1, urA, urB, drA, drB, ulA, ulB);
        if (i + 1 < iend) step(i + 1, lds1, lds0, urB, urA, drB, drA, ulB, ulA);
    }
    if (head) {  // the head layer leaves its flags only
        if (pcols && lane == 0) gr.pzh[(static_cast<int64_t>(seg) * H + h) * 8 + (wave - NWH)] = smax[0] == 0.f;
        return;
    }
    if constexpr (kRowsOut) {
        if (nch > 0) {
            __syncthreads();  // the last chunk's o is staged by every wave
            store_rows(nch - 1);
        }
    }

    if constexpr (MODE == kLocal) {
        // a tail walk whose P is not zero stores nothing but its flags: the second launch writes H and P
        if (i0 > 0) {
            if (pcols && lane == 0 && smax[0] != 0.f) atomicOr(&s_live, 1);
            __syncthreads();  // s_live complete
            if (s_live) {
                if (pcols && lane == 0) sv.pz[(static_cast<int64_t>(seg) * H + h) * 8 + (wave - NWH)] = smax[0] == 0.f;
                return;
            }
        }
    }

    // ---- leaving state (DK = DV: H and P are both 128 x 128), or the gradient at the segment start
    float *dst = nullptr;
    if (kOutPass) {
        if (last && hT) {
            // the final state through the free pack buffers (rows 0-63 in one, 64-127 in the other, 528-byte
            // rows) and out as whole 512-byte rows with the non-temporal hint: a wave holds 16 columns only
            constexpr int kSR = DV + 4;
            static_assert(64 * kSR * 4 <= kBytes, "half the state fits one pack buffer");
            __syncthreads();  // every wave is done with the pack buffers
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        float *half = reinterpret_cast<float *>(rt < 4 ? lds0 : lds1);
                        half[((16 * rt + 4 * g4 + jj) & 63) * kSR + col0 + 16 * ct + n16] =
                            acc[rt][ct][jj] * pow2(fr[ct]);
                    }
            __syncthreads();
            const rsrc_t rs = make_rsrc(hT + (static_cast<int64_t>(nseq) * H + h) * DK * DV, 4 * DK * DV);
#pragma unroll
            for (int i = 0; i < DK * DV / 4 / ScanCfg<MODE>::NT; ++i) {
                const int u = tid + ScanCfg<MODE>::NT * i, r = u >> 5, cu = u & 31;
                const float *half = reinterpret_cast<const float *>(r < 64 ? lds0 : lds1);
                st128_nt(rs, *reinterpret_cast<const u4 *>(half + (r & 63) * kSR + 4 * cu), 4 * (r * DV + 4 * cu));
            }
        }
    } else if (MODE == kLocal) {
        dst = (pcols ? sv.P : sv.Hs) + (static_cast<int64_t>(seg) * H + h) * DK * DV;
    } else if (MODE == kRevLocal) {
        dst = gr.hb + (static_cast<int64_t>(seg) * H + h) * DK * DV;
    } else if (MODE == kRevOut) {
        if (first && gr.dh0) dst = gr.dh0 + (static_cast<int64_t>(nseq) * H + h) * DK * DV;
    }
    // the combines read P from an empty buffer range (zeros, no memory traffic) where every tile is zero
    if (MODE == kLocal && pcols && sv.pz && lane == 0)
        sv.pz[(static_cast<int64_t>(seg) * H + h) * 8 + (wave - NWH)] = smax[0] == 0.f;
    if (MODE == kLocal && pcols && gr.pt) {
        // P^T planes for the gradients' reverse combine: element (c, r) of P^T at 2 (128 c + r) bytes, so the
        // four rows 16 rt + 4 g4 .. + 3 of this lane's column are 8 contiguous bytes of each plane
        char *ptd = gr.pt + (static_cast<int64_t>(seg) * H + h) * DK * DK * 4;
        const rsrc_t rs = make_rsrc(ptd, 4 * DK * DK);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                uint32_t hi0, lo0, hi1, lo1;
                const float sc = pow2(fr[ct]);
                split2(acc[rt][ct][0] * sc, acc[rt][ct][1] * sc, hi0, lo0);
                split2(acc[rt][ct][2] * sc, acc[rt][ct][3] * sc, hi1, lo1);
                const uint32_t off = 2 * ((col0 + 16 * ct + n16) * DK + 16 * rt + 4 * g4);
                st64(rs, u2{hi0, hi1}, off);
                st64(rs, u2{lo0, lo1}, 2 * DK * DK + off);
            }
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
void launch_scan_grad(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, const void *packs,
                      const ScanGrad &gr) {
    // the forward local pass of the gradients also finds the transitions over the segments' first chunks
    dim3 grid(max_segs, L.H, MODE == kLocal && gr.pzh ? 2 : 1), block(mc::ScanCfg<MODE>::NT);
    const char *pk = static_cast<const char *>(packs);
    if (MODE == kOut && L.out_bf16)
        hipLaunchKernelGGL((mc::chunk_scan_kernel<MODE, true>), grid, block, 0, L.stream, pk, per, L.hT, L.o, sv, L.H,
                           gr, 0);
    else
        hipLaunchKernelGGL((mc::chunk_scan_kernel<MODE, false>), grid, block, 0, L.stream, pk, per, L.hT, L.o, sv,
                           L.H, gr, 0);
    // the local pass walked only the segments' tails: whole walks of those whose tail transition is not zero
    if (MODE == kLocal && per > mc::kTail && sv.pz)
        hipLaunchKernelGGL((mc::chunk_scan_kernel<MODE, false>), dim3(max_segs, L.H), block, 0, L.stream, pk, per,
                           L.hT, L.o, sv, L.H, gr, 1);
}

template <int MODE>
void launch_scan(const ChunkLaunch &L, const SegmentView &sv, int max_segs, int per, const void *packs) {
    launch_scan_grad<MODE>(L, sv, max_segs, per, packs, ScanGrad{});
}

template void launch_scan<kLocal>(const ChunkLaunch &, const SegmentView &, int, int, const void *);
template void launch_scan<kOut>(const ChunkLaunch &, const SegmentView &, int, int, const void *);
template void launch_scan_grad<kLocal>(const ChunkLaunch &, const SegmentView &, int, int, const void *,
                                       const ScanGrad &);
template void launch_scan_grad<kStates>(const ChunkLaunch &, const SegmentView &, int, int, const void *,
                                        const ScanGrad &);
template void launch_scan_grad<kRevLocal>(const ChunkLaunch &, const SegmentView &, int, int, const void *,
                                          const ScanGrad &);
template void launch_scan_grad<kRevOut>(const ChunkLaunch &, const SegmentView &, int, int, const void *,
                                        const ScanGrad &);

}  // namespace kda
