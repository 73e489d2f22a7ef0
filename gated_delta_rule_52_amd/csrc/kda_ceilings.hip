// kda_ceilings.hip - measured ceilings for the roofline figures: a streaming
// copy kernel (the HBM bandwidth a plain read-once/write-once kernel reaches)
// and a bf16 matrix-core loop (the MFMA rate a kernel with no memory traffic
// reaches).  Built into its own library (libkda_ceilings.so), not part of
// the operator's C ABI; only the benchmark loads it.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kPerThread = 4;  // 16-byte units per thread: 64 bytes

// Each thread copies four 16-byte units, kThreads * 16 bytes apart, so every
// load and store instruction of a wave covers 1 KiB of consecutive bytes.
template <bool NonTemporal>
__global__ void __launch_bounds__(kThreads) copy_kernel(const f4 *__restrict__ src, f4 *__restrict__ dst, size_t n16) {
    const size_t base = static_cast<size_t>(blockIdx.x) * kThreads * kPerThread + threadIdx.x;
    f4 r[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const size_t j = base + static_cast<size_t>(i) * kThreads;
        if (j < n16) r[i] = NonTemporal ? __builtin_nontemporal_load(src + j) : src[j];
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const size_t j = base + static_cast<size_t>(i) * kThreads;
        if (j < n16) {
            if (NonTemporal) __builtin_nontemporal_store(r[i], dst + j);
            else dst[j] = r[i];
        }
    }
}

// Eight independent 16x16x32 bf16 products per iteration and wave, each
// accumulating into its own registers; operands come from the lane index so
// that nothing folds.  Every lane writes its sum so the products stay live.
__global__ void __launch_bounds__(kThreads) mfma_kernel(float *out, int iters) {
    const int lane = threadIdx.x & 63;
    b8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[0][i] = static_cast<__bf16>(static_cast<float>((lane + i) & 7) * 0.125f);
        b[0][i] = static_cast<__bf16>(static_cast<float>((lane * 3 + i) & 7) * 0.0625f);
        a[1][i] = static_cast<__bf16>(static_cast<float>((lane + 2 * i) & 7) * 0.25f);
        b[1][i] = static_cast<__bf16>(static_cast<float>((lane * 5 + i) & 7) * 0.03125f);
    }
    // distinct starting values, so that no two chains compute the same thing
    f4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f4{static_cast<float>(j), 0.f, 0.f, static_cast<float>(lane)};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j & 1], b[(j >> 1) & 1], acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16) from src to dst on `stream`; 0 on success.
int kda_ceiling_copy(const void *src, void *dst, size_t bytes, int non_temporal, void *stream) {
    if (bytes % 16) return 1;
    const size_t n16 = bytes / 16;
    const size_t per_block = static_cast<size_t>(kThreads) * kPerThread;
    const dim3 grid(static_cast<unsigned>((n16 + per_block - 1) / per_block));
    if (non_temporal)
        hipLaunchKernelGGL(copy_kernel<true>, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                           static_cast<const f4 *>(src), static_cast<f4 *>(dst), n16);
    else
        hipLaunchKernelGGL(copy_kernel<false>, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                           static_cast<const f4 *>(src), static_cast<f4 *>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// `blocks` workgroups of 4 waves, each wave issuing iters * 8 MFMA
// 16x16x32 bf16 (16,384 flops each); `out` holds blocks * 256 floats.
int kda_ceiling_mfma(float *out, int blocks, int iters, void *stream) {
    if (blocks <= 0 || iters <= 0) return 1;
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Flops of one kda_ceiling_mfma launch.
double kda_ceiling_mfma_flops(int blocks, int iters) {
    return static_cast<double>(blocks) * 4.0 * iters * 8.0 * 16.0 * 16.0 * 32.0 * 2.0;
}

}  // extern "C"
