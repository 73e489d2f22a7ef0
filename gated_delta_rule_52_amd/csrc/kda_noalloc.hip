// kda_noalloc.hip - kda_chunk_fwd_noalloc: the chunkwise prefill for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Instead of a caller workspace, the
// prefill's scratch (segment table, segment transitions and states, operand
// packs) lives in one file-scope device array of fixed size.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  That address is looked up once per device
// (hipGetSymbolAddress, with the device current) and cached; host code never
// uses the array's name as an address.  Every call on a GPU shares that GPU's
// array, so calls that overlap in time on one GPU (different streams, or
// different host threads) race; the prefill needs no part of its scratch to
// start at zero, so nothing is cleared between calls.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>

#include "kda_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t{64} << 20;  // KDA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == KDA_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // the array's device address on each device, once looked up

kda_status fail(kda_status s, const char *text) {
    kda::set_last_error(text);
    return s;
}

// The array's address on the current device, looked up on the first call there.
kda_status scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        char buf[256];
        std::snprintf(buf, sizeof buf, "kda_chunk_fwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
        return fail(KDA_ERR_HIP, buf);
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_fwd_noalloc: device index >= 64");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char buf[256];
            std::snprintf(buf, sizeof buf, "kda_chunk_fwd_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                          hipGetErrorString(e));
            return fail(KDA_ERR_HIP, buf);
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KDA_OK;
}

}  // namespace

extern "C" size_t kda_chunk_fwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

extern "C" kda_status kda_chunk_fwd_noalloc(const kda_chunk_fwd_args *user) {
    if (!user) return fail(KDA_ERR_NULL_POINTER, "args is NULL");
    if (user->struct_size != sizeof(kda_chunk_fwd_args)) {
        char buf[128];
        std::snprintf(buf, sizeof buf, "struct_size %u (expected %zu)", user->struct_size, sizeof(kda_chunk_fwd_args));
        return fail(KDA_ERR_BAD_STRUCT, buf);
    }
    kda_chunk_fwd_args a;
    std::memcpy(&a, user, sizeof a);
    a.workspace = nullptr;
    a.workspace_bytes = 0;
    const size_t need = kda_chunk_fwd_workspace_bytes(&a);
    // invalid arguments: kda_chunk_fwd reports which one, before any launch
    if (need == static_cast<size_t>(-1)) return kda_chunk_fwd(&a);
    if (need > kScratchBytes) {
        char buf[256];
        std::snprintf(buf, sizeof buf,
                      "kda_chunk_fwd_noalloc: this problem needs %zu bytes of scratch; the built-in scratch holds %zu "
                      "(use kda_chunk_fwd with a workspace)",
                      need, kScratchBytes);
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, buf);
    }
    if (need > 0) {
        void *p = nullptr;
        const kda_status st = scratch_on_current_device(&p);
        if (st != KDA_OK) return st;
        a.workspace = p;
        a.workspace_bytes = kScratchBytes;
    }
    return kda_chunk_fwd(&a);
}
