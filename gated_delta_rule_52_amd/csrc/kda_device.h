// kda_device.h - device helpers shared by the KDA kernels (gfx950 / CDNA4).
//
// bf16 <-> fp32 conversion (bf16 is the upper half of an IEEE binary32, so
// widening is a shift and narrowing rounds to nearest, ties to even), typed
// loads for the two input dtypes, and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even narrowing; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Element loads/stores for a tensor whose dtype is a template parameter:
// IsBf16 == true means uint16_t storage holding bf16, false means float.
template <bool IsBf16>
struct Elem;

template <>
struct Elem<true> {
    using T = uint16_t;
    __device__ __forceinline__ static float load(const T *p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void store(T *p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
    // four consecutive elements (8-byte aligned)
    __device__ __forceinline__ static float4 load4(const T *p, int64_t i) {
        const uint2 w = *reinterpret_cast<const uint2 *>(p + i);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    }
    __device__ __forceinline__ static void store4(T *p, int64_t i, float4 x) {
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16(x.z)) | (static_cast<uint32_t>(f32_to_bf16(x.w)) << 16);
        *reinterpret_cast<uint2 *>(p + i) = w;
    }
};

template <>
struct Elem<false> {
    using T = float;
    __device__ __forceinline__ static float load(const T *p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(T *p, int64_t i, float x) { p[i] = x; }
    __device__ __forceinline__ static float4 load4(const T *p, int64_t i) {
        return *reinterpret_cast<const float4 *>(p + i);
    }
    __device__ __forceinline__ static void store4(T *p, int64_t i, float4 x) {
        *reinterpret_cast<float4 *>(p + i) = x;
    }
};

// A DPP move inside each row of 16 lanes (bound_ctrl: lanes without a
// source read 0; every control used here has one for every lane).
template <int Ctrl>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xf, 0xf, true));
}
// Sum over the four lanes of each quad, left in all four.
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp_mov<0xB1>(x);  // quad permute [1, 0, 3, 2]
    return x + dpp_mov<0x4E>(x);  // quad permute [2, 3, 0, 1]
}

// The (slice, head, sequence) a workgroup of a grid (slices, H, N) works on.  Workgroups go round-robin
// over the GPU's 8 XCDs, each with its own L2, in order of their linear index.  The slices of one
// (sequence, head) read the same token inputs and share the cache lines of every state row, so their
// indexes are made congruent mod 8: they run on one XCD and its L2 fetches each line once.  When N H is
// not a multiple of 8 the slices stay consecutive.
__device__ __forceinline__ void slice_head_seq(int &slice, int &h, int &n) {
    const int64_t nsl = gridDim.x, groups = static_cast<int64_t>(gridDim.y) * gridDim.z;
    const int64_t id = blockIdx.x + nsl * (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z);
    int64_t gi;
    if (groups % 8 == 0) {
        const int64_t kq = id >> 3;
        gi = (id & 7) + 8 * (kq / nsl);
        slice = static_cast<int>(kq % nsl);
    } else {
        gi = id / nsl;
        slice = static_cast<int>(id % nsl);
    }
    h = static_cast<int>(gi % gridDim.y);
    n = static_cast<int>(gi / gridDim.y);
}

// Non-temporal 16-byte load and store, for data a kernel streams exactly once
// each way (a decode step's state): the hint keeps it from displacing lines
// that are reused, such as the token inputs every workgroup of a head reads.
typedef float nt_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float *p) {
    const nt_f4 x = __builtin_nontemporal_load(reinterpret_cast<const nt_f4 *>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_stream(float *p, float4 v) {
    __builtin_nontemporal_store(nt_f4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_f4 *>(p));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

}  // namespace kda
