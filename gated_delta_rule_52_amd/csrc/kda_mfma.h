// kda_mfma.h - helpers shared by the fp16/bf16 matrix-core prefill kernels
// (kda_prep.hip, kda_scan.hip) for gfx950: MFMA wrappers, power-of-two
// scaling, packed conversions, cross-lane moves, buffer-resource accesses and
// the layout of the per-chunk operand pack that the two kernels exchange.
#pragma once

#include "kda_device.h"

namespace kda {
namespace mc {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));
typedef int i2 __attribute__((ext_vector_type(2)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

constexpr int DK = 128, DV = 128, C = 64;

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

// 2^e as a float, saturating: 0 below the normal range (a true underflow of
// the scaled quantity), 2^127 above it
__device__ __forceinline__ float pow2(int e) {
    return e < -126 ? 0.f : __int_as_float((min(e, 127) + 127) << 23);
}

// Exponent e with m * 2^-e in [0.5, 1) for m > 0 (0 for m == 0 or denormal m).
__device__ __forceinline__ int exp_of(float m) {
    const int b = (__float_as_int(m) >> 23) & 0xff;
    return b == 0 ? 0 : b - 126;
}

__device__ __forceinline__ uint32_t hbits(_Float16 x) { return __builtin_bit_cast(uint16_t, x); }
__device__ __forceinline__ uint32_t bbits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }
typedef float fl2 __attribute__((ext_vector_type(2)));
typedef _Float16 hf2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
// two floats -> packed fp16 pair (round to nearest even), one instruction
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((fl2{a, b}), hf2));
}
__device__ __forceinline__ h4 to_h4(f4 v, float s) {
    const hf2 lo = __builtin_convertvector((fl2{v[0] * s, v[1] * s}), hf2);
    const hf2 hi = __builtin_convertvector((fl2{v[2] * s, v[3] * s}), hf2);
    return h4{lo[0], lo[1], hi[0], hi[1]};
}
// bf16 high and low parts of two values, each pair packed in one word
// (hi = round(x), lo = round(x - hi): ~16 significant bits together)
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((fl2{a, b}), bf2));
    const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((fl2{a - ha, b - hb}), bf2));
}
// running maximum of |x| over packed bf16 pairs, as 16-bit integers (the
// order of non-negative floats is the order of their bit patterns)
__device__ __forceinline__ uint32_t absmax2(uint32_t acc, uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, acc),
                                                                  __builtin_bit_cast(us2, w & 0x7fff7fffu)));
}
// the larger of the two halves of absmax2's result, as a float
__device__ __forceinline__ float absmax2_value(uint32_t acc) {
    const uint32_t m = (acc & 0xffffu) > (acc >> 16) ? (acc & 0xffffu) : (acc >> 16);
    return __uint_as_float(m << 16);
}
// the two bf16 values packed in a word, widened
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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
    return __builtin_bit_cast(h8, (i4{d0, d1, d2, d3}));
}

// Maximum over the wave of non-negative values, returned wave-uniform, by
// DPP moves on the VALU (no trip through the LDS pipe): shifts within each
// row of 16 lanes leave the row maximum in its lane 15, two row broadcasts
// carry it into lane 63.  Lanes a move reads from outside its row range
// contribute 0, which never raises a maximum of non-negative values.
template <int Ctrl>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_move<0x111>(x));  // row_shr:1
    x = fmaxf(x, dpp_move<0x112>(x));  // row_shr:2
    x = fmaxf(x, dpp_move<0x114>(x));  // row_shr:4
    x = fmaxf(x, dpp_move<0x118>(x));  // row_shr:8
    x = fmaxf(x, dpp_move<0x142>(x));  // row_bcast:15
    x = fmaxf(x, dpp_move<0x143>(x));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
// Sum over each half-wave (lanes 0-31 and 32-63 separately), the result in
// every lane: butterflies over lane bits 0-3 as DPP moves (quad permutes
// [1,0,3,2] and [2,3,0,1]; half-row and row mirrors, which pair the two
// quads of an 8-lane group and the two 8-lane groups of a row once every lane
// of each holds its group's sum), then bit 4 by a swizzle (xor mask 16 in the
// 32-lane bit mode).
__device__ __forceinline__ float half_wave_sum(float x) {
    x += dpp_move<0xB1>(x);
    x += dpp_move<0x4E>(x);
    x += dpp_move<0x141>(x);
    x += dpp_move<0x140>(x);
    return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// Sum over each row of 16 lanes, the result in every lane of the row: the
// first four butterflies of half_wave_sum.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_move<0xB1>(x);
    x += dpp_move<0x4E>(x);
    x += dpp_move<0x141>(x);
    return x + dpp_move<0x140>(x);
}

// Buffer resource over [base, base + bytes): raw buffer accesses at or past
// the end read as zero and their stores are dropped.  Offsets are 32-bit
// bytes from a wave-uniform base, so ragged tails need no masking and no
// per-lane 64-bit address has to live across a loop.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off, int soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), soff, 0);
}
__device__ __forceinline__ uint32_t ld16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, 0);
}
__device__ __forceinline__ u2 ld64(rsrc_t r, uint32_t off, int soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), soff, 0);
}
__device__ __forceinline__ void st16(rsrc_t r, uint32_t v, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v), r, static_cast<int>(off), 0, 0);
}
__device__ __forceinline__ void st32(rsrc_t r, uint32_t v, uint32_t off, int soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, static_cast<int>(off), soff, 0);
}
__device__ __forceinline__ void st64(rsrc_t r, u2 v, uint32_t off, int soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(off), soff, 0);
}
__device__ __forceinline__ void st128(rsrc_t r, u4 v, uint32_t off, int soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), soff, 0);
}
// the same with the non-temporal hint (cache policy bit 1, "nt" on gfx950), for output that is written
// once in whole 128-byte lines and not read back soon; partial lines written this way cost far more
__device__ __forceinline__ void st128_nt(rsrc_t r, u4 v, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, 2);
}

// ---- per-chunk operand pack (one per chunk and head, written by the prep
// kernel, streamed by the scan kernels).  Every fp16 matrix carries a
// power-of-two scale: stored = true value * 2^-e.  The pack is copied into
// LDS as a straight line; the 16-byte units of W, KT and Q are XOR-swizzled
// by row so that the scan's operand reads hit distinct banks, and the A
// blocks are stored in the order their 8-byte operand reads go.
//
//   [0, 512)        gamma: exp(G_last) per channel, fp32
//   [512, 1024)     header: int exponents e_w, e_q, e_k, e_u, e_a
//   W   [64][128]   T beta (e^G k)            A operand of W S       (w_col)
//   KT  [128][64]   (e^{G_last - G} k)^T      A operand of the update (kt_col)
//   Q   [64][128]   scale e^G q               A operand of Q S       (w_col)
//   A   [10][64][4]  blocks (a, b), b <= a, of the decayed scale q k^T, each in
//                   lane order: lane 16 g + n holds row n, columns 4g .. 4g + 3
//   U   T beta v in accumulator order: [16-column tile][row-block pair]
//                   [lane][row block a, a + 1][row within lane]
constexpr int kPkGamma = 0;
constexpr int kPkHdr = 512;
constexpr int kPkW = 1024;
constexpr int kPkKT = kPkW + C * DK * 2;
constexpr int kPkQ = kPkKT + DK * C * 2;
constexpr int kPkA = kPkQ + C * DK * 2;
constexpr int kPkU = kPkA + 10 * 16 * 16 * 2;
constexpr int kPkBytes = kPkU + C * DV * 2;
constexpr int kPkLocal = kPkQ;   // bytes the local pass copies to LDS
constexpr int kPkOut = kPkU;     // bytes the output pass copies to LDS
static_assert(kPkLocal % 1024 == 0 && kPkOut % 1024 == 0, "whole 1 KiB wave copies");
enum { kHdrW = 0, kHdrQ = 1, kHdrK = 2, kHdrU = 3, kHdrA = 4, kHdrDO = 5, kHdrUL = 6 };
// header word 7 of a forward pack: 1 when the fast prep left the chunk to its exact path, written for every
// slot (an empty slot's pack holds only this word); each pack's own line, so no two workgroups share it
constexpr int kHdrX = 7;

// ---- reverse pack (gradients), one per chunk and head, same slots: the walk
// over the chunks in reverse order carries dS (the gradient of the state a
// chunk leaves) as the forward walk carries S, since
//     dV_new = A_qk^T dO + Kd dS,   dS_enter = gamma * dS + Q^T dO - W^T dV_new
// (Kd = e^{G_last - G} k).  With U <- A_qk^T dO, W <- -Kd, KT <- -W^T it is the
// forward step plus one more product Q^T dO:
//   W   slot  -Kd          [64][128]  w_col,  exponent hdr[kHdrW]
//   KT  slot  -W^T         [128][64]  kt_col, exponent hdr[kHdrK]
//   Q   slot  Q^T          [128][64]  kt_col, exponent hdr[kHdrQ]  (Q = scale e^G q)
//   U   slot  A_qk^T dO    accumulator order, exponent hdr[kHdrU]
//   DO        dO           accumulator order (as U), exponent hdr[kHdrDO]
//   UL        the rest of A_qk^T dO after U's fp16 rounding, accumulator
//             order, exponent hdr[kHdrUL] (U + UL to about 22 bits)
//   gamma as in the forward pack; the A slot is unused.
constexpr int kRvDO = kPkBytes;
constexpr int kRvUL = kRvDO + C * DV * 2;
constexpr int kRvBytes = kRvUL + C * DV * 2;
constexpr int kRvStage = kPkA;  // bytes the reverse passes copy to LDS (gamma, header, W, KT, Q)
static_assert(kRvStage % 1024 == 0, "whole 1 KiB wave copies");

// W, Q ([64][128] fp16) and KT ([128][64] fp16) are read as A operands of
// 16x16x32 products whose contraction index is permuted: in step p, lane
// (g, n) supplies rows 16 (2p) + 4g .. +3 and 16 (2p + 1) + 4g .. +3 of the B
// matrix (exactly what its accumulators hold, so B needs no cross-lane
// movement), and the A operand the matching columns.  The pack therefore
// stores, in 16-byte unit 4p + g of a row, the columns 32p + 4g .. +3 and
// 32p + 16 + 4g .. +3 (one b128 read per lane and step).  Units are
// XOR-swizzled by row so that the 16 rows a read touches hit distinct banks.
// byte offset of column c of row r
__device__ __forceinline__ int w_col(int r, int c) {   // W, Q: 16 units a row
    const int u = 4 * (c >> 5) + ((c >> 2) & 3);
    return r * 256 + ((u ^ (r & 15)) << 4) + (((c >> 4) & 1) << 3) + ((c & 3) << 1);
}
__device__ __forceinline__ int kt_col(int r, int c) {  // KT: 8 units a row, rows 2i, 2i+1 128 bytes apart
    const int u = 4 * (c >> 5) + ((c >> 2) & 3);
    return r * 128 + ((u ^ ((r >> 1) & 7)) << 4) + (((c >> 4) & 1) << 3) + ((c & 3) << 1);
}
// byte offset of the 16-byte A operand unit (step p, lane group g) of row r
__device__ __forceinline__ int w_unit(int r, int p, int g) { return r * 256 + (((4 * p + g) ^ (r & 15)) << 4); }
__device__ __forceinline__ int kt_unit(int r, int p, int g) { return r * 128 + (((4 * p + g) ^ ((r >> 1) & 7)) << 4); }
// byte offset of the 8 bytes of U (tile ct, row block a) that lane `lane` holds
__device__ __forceinline__ int u_off(int ct, int a, int lane) {
    return ((ct * 2 + (a >> 1)) * 64 + lane) * 16 + (a & 1) * 8;
}

}  // namespace mc
}  // namespace kda
