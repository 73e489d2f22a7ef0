// kda_internal.h - launch descriptors shared by the host entry points
// (kda_api.cpp) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Token-by-token kernel: decode step (T = 1, N = number of sequences) or a
// loop over the tokens of each sequence.
struct RecurrentLaunch {
    const void *q, *k, *v;
    const float *g;
    const void *beta;
    const float *h0;
    float *hT;
    void *o;
    const int32_t *cu_seqlens;  // device, or nullptr: N sequences of T tokens
    int N, T, H, dk, dv;
    float scale;
    bool in_bf16, out_bf16;
    bool multi_token;           // split dv into narrow slices for long loops
    hipStream_t stream;
};

hipError_t launch_recurrent(const RecurrentLaunch &L);

// Chunkwise prefill.
struct ChunkLaunch {
    const void *q, *k, *v;
    const float *g;
    const void *beta;
    const float *h0;
    float *hT;
    void *o;
    const int32_t *cu_seqlens;  // device, or nullptr
    int B, T, H, dk, dv, N;
    int chunk;
    float scale;
    bool in_bf16, out_bf16;
    void *workspace;
    size_t workspace_bytes;
    hipStream_t stream;
};

size_t chunk_workspace_bytes(int B, int T, int H, int dk, int dv, int N, int chunk, bool varlen);
hipError_t launch_chunk(const ChunkLaunch &L);

}  // namespace kda
