// kda_api.cpp - host entry points of the C ABI declared in include/kda.h.
//
// Every argument is validated here, before anything is enqueued, so that a
// bad call returns a status code and launches nothing.  The kernels never
// allocate; the caller's stream carries all work.
#include "kda.h"

#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdio>
#include <cstring>
#include <string>

#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
kda_status fail(kda_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool valid_dtype(kda_dtype d) { return d == KDA_DTYPE_BF16 || d == KDA_DTYPE_FP32; }
size_t dsize(kda_dtype d) { return d == KDA_DTYPE_BF16 ? 2 : 4; }
bool valid_dim(int32_t d) { return d == 64 || d == 128; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void *p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

kda_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return KDA_OK;
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Copies the caller's struct into `out`: the struct of this ABI version, or
// that of version 1, which ends before `flags` (then no input transform).
// Checks the size and the transform fields.
template <class Args>
kda_status read_args(const Args *a, Args &out) {
    if (!a) return fail(KDA_ERR_NULL_POINTER, "args is NULL");
    const size_t v1 = offsetof(Args, flags);
    if (a->struct_size != sizeof(Args) && a->struct_size != v1)
        return fail(KDA_ERR_BAD_STRUCT, "struct_size %u (expected %zu, or %zu for ABI version 1)", a->struct_size,
                    sizeof(Args), v1);
    std::memset(&out, 0, sizeof out);
    std::memcpy(&out, a, a->struct_size);
    if (a->struct_size == v1) {
        out.flags = 0;
        out.gate_scale = 1.f;
    }
    if (out.flags & ~(KDA_FLAG_QK_L2NORM | KDA_FLAG_GATE_SOFTPLUS | KDA_FLAG_SCALAR_GATE))
        return fail(KDA_ERR_UNSUPPORTED, "unknown flags 0x%x", out.flags);
    if ((out.flags & KDA_FLAG_GATE_SOFTPLUS) && !(std::isfinite(out.gate_scale) && out.gate_scale >= 0.f))
        return fail(KDA_ERR_BAD_SHAPE, "gate_scale must be finite and >= 0");
    return KDA_OK;
}

template <class Args>
kda::InputXform xform_of(const Args *a) {
    kda::InputXform x{};
    x.qk_l2norm = (a->flags & KDA_FLAG_QK_L2NORM) != 0;
    x.gate_softplus = (a->flags & KDA_FLAG_GATE_SOFTPLUS) != 0;
    x.gate_scale = a->gate_scale;
    x.scalar_gate = (a->flags & KDA_FLAG_SCALAR_GATE) != 0;
    return x;
}

// fp32 gate values per token and head: dk, or 1 with a scalar gate
template <class Args>
size_t gate_width(const Args *a) {
    return (a->flags & KDA_FLAG_SCALAR_GATE) ? 1 : static_cast<size_t>(a->dk);
}

// Checks shared by kda_chunk_fwd and kda_chunk_fwd_workspace_bytes (on a struct read by read_args).
kda_status check_chunk_sizes(const kda_chunk_fwd_args *a) {
    if (a->B < 0 || a->T < 0 || a->H <= 0 || a->num_seqs < 0)
        return fail(KDA_ERR_BAD_SHAPE, "B=%d T=%d H=%d num_seqs=%d", a->B, a->T, a->H, a->num_seqs);
    if (!valid_dim(a->dk) || !valid_dim(a->dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d dv=%d (supported: 64, 128)", a->dk, a->dv);
    if (!valid_dtype(a->in_dtype) || !valid_dtype(a->out_dtype))
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype=%d out_dtype=%d", a->in_dtype, a->out_dtype);
    if (a->chunk_size != 64 && a->chunk_size != 32 && a->chunk_size != 16)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size=%d (supported: 16, 32, 64)", a->chunk_size);
    if (!std::isfinite(a->scale)) return fail(KDA_ERR_BAD_SHAPE, "scale is not finite");
    if (a->cu_seqlens) {
        if (a->B != 1) return fail(KDA_ERR_BAD_SHAPE, "packed variable-length input needs B == 1 (B=%d)", a->B);
    } else if (a->num_seqs != a->B) {
        return fail(KDA_ERR_BAD_SHAPE, "num_seqs=%d must equal B=%d without cu_seqlens", a->num_seqs, a->B);
    }
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    if (tokens > INT32_MAX)  // the segment table holds 32-bit token offsets
        return fail(KDA_ERR_BAD_SHAPE, "B*T=%lld tokens (at most %d)", static_cast<long long>(tokens), INT32_MAX);
    if (tokens * a->H * (a->dk > a->dv ? a->dk : a->dv) > (int64_t{1} << 40))
        return fail(KDA_ERR_BAD_SHAPE, "problem too large");
    return KDA_OK;
}

// Checks of the prefill-style arguments that kda_chunk_fwd and
// kda_recurrent_fwd share: pointers, output aliasing, sizes.
kda_status check_prefill_buffers(const kda_chunk_fwd_args *a) {
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    const int N = a->num_seqs;
    if (tokens > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o))
        return fail(KDA_ERR_NULL_POINTER, "q, k, v, g, beta and o are required");
    const size_t th = static_cast<size_t>(tokens) * a->H;
    const size_t in_sz = dsize(a->in_dtype);
    const Range ro = range_of(a->o, th * a->dv * dsize(a->out_dtype));
    const Range ins[] = {range_of(a->q, th * a->dk * in_sz), range_of(a->k, th * a->dk * in_sz),
                         range_of(a->v, th * a->dv * in_sz), range_of(a->g, th * gate_width(a) * 4),
                         range_of(a->beta, th * in_sz)};
    const size_t sbytes = static_cast<size_t>(N) * a->H * a->dk * a->dv * 4;
    const Range rh0 = range_of(a->initial_state, a->initial_state ? sbytes : 0);
    const Range rcu = range_of(a->cu_seqlens, a->cu_seqlens ? (static_cast<size_t>(N) + 1) * 4 : 0);
    for (const Range &r : ins)
        if (overlap(ro, r)) return fail(KDA_ERR_ALIAS, "o overlaps an input");
    // o is written while other workgroups still read the initial state and the sequence offsets
    if (overlap(ro, rh0)) return fail(KDA_ERR_ALIAS, "o overlaps initial_state");
    if (overlap(ro, rcu)) return fail(KDA_ERR_ALIAS, "o overlaps cu_seqlens");
    if (a->final_state) {
        const Range rf = range_of(a->final_state, sbytes);
        for (const Range &r : ins)
            if (overlap(rf, r)) return fail(KDA_ERR_ALIAS, "final_state overlaps an input");
        if (overlap(rf, ro)) return fail(KDA_ERR_ALIAS, "final_state overlaps o");
        if (overlap(rf, rcu)) return fail(KDA_ERR_ALIAS, "final_state overlaps cu_seqlens");
        if (a->initial_state && a->initial_state != a->final_state && overlap(rf, rh0))
            return fail(KDA_ERR_ALIAS, "final_state partially overlaps initial_state");
    }
    if (N > 65535 || a->H > 65535) return fail(KDA_ERR_UNSUPPORTED, "N=%d H=%d (at most 65535 each)", N, a->H);
    return KDA_OK;
}

// Size checks of kda_recurrent_bwd, shared with its workspace query.
kda_status check_bwd_sizes(const kda_recurrent_bwd_args *a) {
    if (a->B < 0 || a->T < 0 || a->H <= 0 || a->num_seqs < 0)
        return fail(KDA_ERR_BAD_SHAPE, "B=%d T=%d H=%d num_seqs=%d", a->B, a->T, a->H, a->num_seqs);
    if (!valid_dim(a->dk) || !valid_dim(a->dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d dv=%d (supported: 64, 128)", a->dk, a->dv);
    if (!valid_dtype(a->in_dtype)) return fail(KDA_ERR_UNSUPPORTED, "in_dtype=%d", a->in_dtype);
    if (!std::isfinite(a->scale)) return fail(KDA_ERR_BAD_SHAPE, "scale is not finite");
    if (a->cu_seqlens ? a->B != 1 : a->num_seqs != a->B)
        return fail(KDA_ERR_BAD_SHAPE, "num_seqs=%d with B=%d (%s)", a->num_seqs, a->B,
                    a->cu_seqlens ? "packed input needs B = 1" : "num_seqs must equal B");
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    if (tokens > INT32_MAX)
        return fail(KDA_ERR_BAD_SHAPE, "B*T=%lld tokens (at most %d)", static_cast<long long>(tokens), INT32_MAX);
    if (tokens * a->H * (a->dk > a->dv ? a->dk : a->dv) > (int64_t{1} << 40))
        return fail(KDA_ERR_BAD_SHAPE, "problem too large");
    if (a->num_seqs > 65535 || a->H > 65535)
        return fail(KDA_ERR_UNSUPPORTED, "N=%d H=%d (at most 65535 each)", a->num_seqs, a->H);
    return KDA_OK;
}

kda_status read_bwd_args(const kda_recurrent_bwd_args *a, kda_recurrent_bwd_args &out) {
    if (!a) return fail(KDA_ERR_NULL_POINTER, "args is NULL");
    if (a->struct_size != sizeof(kda_recurrent_bwd_args))
        return fail(KDA_ERR_BAD_STRUCT, "struct_size %u (expected %zu)", a->struct_size,
                    sizeof(kda_recurrent_bwd_args));
    out = *a;
    if (out.flags & ~(KDA_FLAG_QK_L2NORM | KDA_FLAG_GATE_SOFTPLUS | KDA_FLAG_SCALAR_GATE))
        return fail(KDA_ERR_UNSUPPORTED, "unknown flags 0x%x", out.flags);
    if ((out.flags & KDA_FLAG_GATE_SOFTPLUS) && !(std::isfinite(out.gate_scale) && out.gate_scale >= 0.f))
        return fail(KDA_ERR_BAD_SHAPE, "gate_scale must be finite and >= 0");
    return check_bwd_sizes(&out);
}

// Buffer checks of the gradient entry points (null pointers, workspace size, overlaps); tokens > 0 or a
// requested initial-state gradient.
kda_status check_bwd_buffers(const kda_recurrent_bwd_args *a, size_t need) {
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    const int N = a->num_seqs;
    if (tokens > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->grad_o || !a->grad_q || !a->grad_k ||
                       !a->grad_v || !a->grad_g || !a->grad_beta))
        return fail(KDA_ERR_NULL_POINTER, "q, k, v, g, beta, grad_o and every token gradient are required");
    const size_t th = static_cast<size_t>(tokens) * a->H, in_sz = dsize(a->in_dtype);
    const size_t gw = (a->flags & KDA_FLAG_SCALAR_GATE) ? 1 : static_cast<size_t>(a->dk);
    const size_t sbytes = static_cast<size_t>(N) * a->H * a->dk * a->dv * 4;
    if (a->workspace_bytes < need || (need > 0 && !a->workspace))
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", a->workspace_bytes, need);
    const Range ins[] = {range_of(a->q, th * a->dk * in_sz), range_of(a->k, th * a->dk * in_sz),
                         range_of(a->v, th * a->dv * in_sz), range_of(a->g, th * gw * 4),
                         range_of(a->beta, th * in_sz), range_of(a->grad_o, th * a->dv * in_sz),
                         range_of(a->cu_seqlens, a->cu_seqlens ? (static_cast<size_t>(N) + 1) * 4 : 0)};
    const Range outs[] = {range_of(a->grad_q, th * a->dk * 4), range_of(a->grad_k, th * a->dk * 4),
                          range_of(a->grad_v, th * a->dv * 4), range_of(a->grad_g, th * gw * 4),
                          range_of(a->grad_beta, th * 4), range_of(a->workspace, need)};
    const Range rh0 = range_of(a->initial_state, a->initial_state ? sbytes : 0);
    const Range rdhT = range_of(a->grad_final_state, a->grad_final_state ? sbytes : 0);
    const size_t n_outs = sizeof outs / sizeof outs[0];
    for (size_t i = 0; i < n_outs; ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r)) return fail(KDA_ERR_ALIAS, "a gradient or the workspace overlaps an input");
        if (overlap(outs[i], rh0) || overlap(outs[i], rdhT))
            return fail(KDA_ERR_ALIAS, "a gradient or the workspace overlaps a state input");
        for (size_t j = i + 1; j < n_outs; ++j)
            if (overlap(outs[i], outs[j])) return fail(KDA_ERR_ALIAS, "two gradients (or the workspace) overlap");
    }
    if (a->grad_initial_state) {
        const Range rd = range_of(a->grad_initial_state, sbytes);
        for (const Range &r : ins)
            if (overlap(rd, r)) return fail(KDA_ERR_ALIAS, "grad_initial_state overlaps an input");
        for (const Range &r : outs)
            if (overlap(rd, r)) return fail(KDA_ERR_ALIAS, "grad_initial_state overlaps another gradient");
        if (a->grad_initial_state != a->initial_state && overlap(rd, rh0))
            return fail(KDA_ERR_ALIAS, "grad_initial_state partially overlaps initial_state");
        if (a->grad_initial_state != a->grad_final_state && overlap(rd, rdhT))
            return fail(KDA_ERR_ALIAS, "grad_initial_state partially overlaps grad_final_state");
    }
    return KDA_OK;
}

}  // namespace

void kda::set_last_error(const char *text) { g_last_error = text; }

extern "C" {

const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL_POINTER: return "null pointer";
        case KDA_ERR_BAD_SHAPE: return "bad shape";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case KDA_ERR_BAD_STRUCT: return "argument struct size mismatch";
        case KDA_ERR_HIP: return "HIP error";
        case KDA_ERR_ALIAS: return "output overlaps an input";
    }
    return "unknown status";
}

const char *kda_last_error(void) { return g_last_error.c_str(); }

const char *kda_last_hip_error(void) { return g_last_error.c_str(); }

int kda_abi_version(void) { return KDA_ABI_VERSION; }

int kda_version(void) { return KDA_ABI_VERSION; }

size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_fwd_args *user) {
    kda_chunk_fwd_args args;
    if (read_args(user, args) != KDA_OK || check_chunk_sizes(&args) != KDA_OK) return static_cast<size_t>(-1);
    const kda_chunk_fwd_args *a = &args;
    return kda::chunk_workspace_bytes(a->B, a->T, a->H, a->dk, a->dv, a->num_seqs, a->chunk_size,
                                      a->cu_seqlens != nullptr, a->in_dtype == KDA_DTYPE_BF16);
}

kda_status kda_chunk_fwd(const kda_chunk_fwd_args *user) {
    g_last_error.clear();
    kda_chunk_fwd_args args;
    kda_status st = read_args(user, args);
    if (st != KDA_OK) return st;
    const kda_chunk_fwd_args *a = &args;
    st = check_chunk_sizes(a);
    if (st != KDA_OK) return st;
    st = check_prefill_buffers(a);
    if (st != KDA_OK) return st;
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    const int N = a->num_seqs;
    if (N == 0 || (tokens == 0 && !a->final_state)) return KDA_OK;
    // the workspace must not overlap any input or output
    const size_t th = static_cast<size_t>(tokens) * a->H;
    const size_t in_sz = dsize(a->in_dtype);
    const Range ro = range_of(a->o, th * a->dv * dsize(a->out_dtype));
    const Range ins[] = {range_of(a->q, th * a->dk * in_sz), range_of(a->k, th * a->dk * in_sz),
                         range_of(a->v, th * a->dv * in_sz), range_of(a->g, th * gate_width(a) * 4),
                         range_of(a->beta, th * in_sz)};
    const size_t sbytes = static_cast<size_t>(N) * a->H * a->dk * a->dv * 4;
    const size_t need = kda::chunk_workspace_bytes(a->B, a->T, a->H, a->dk, a->dv, N, a->chunk_size,
                                                   a->cu_seqlens != nullptr, a->in_dtype == KDA_DTYPE_BF16);
    if (a->workspace_bytes < need || (need > 0 && !a->workspace))
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", a->workspace_bytes, need);
    if (!kda::chunk_grids_fit(a->B, a->T, a->H, a->dk, a->dv, N, a->chunk_size, a->cu_seqlens != nullptr,
                              a->in_dtype == KDA_DTYPE_BF16))
        return fail(KDA_ERR_UNSUPPORTED, "problem too large for one launch (more than 2^32 threads in a grid)");
    if (a->workspace) {
        const Range rw = range_of(a->workspace, need);
        for (const Range &r : ins)
            if (overlap(rw, r)) return fail(KDA_ERR_ALIAS, "workspace overlaps an input");
        if (overlap(rw, ro)) return fail(KDA_ERR_ALIAS, "workspace overlaps o");
        if (a->final_state && overlap(rw, range_of(a->final_state, sbytes)))
            return fail(KDA_ERR_ALIAS, "workspace overlaps final_state");
        if (a->initial_state && overlap(rw, range_of(a->initial_state, sbytes)))
            return fail(KDA_ERR_ALIAS, "workspace overlaps initial_state");
        if (a->cu_seqlens && overlap(rw, range_of(a->cu_seqlens, (static_cast<size_t>(N) + 1) * 4)))
            return fail(KDA_ERR_ALIAS, "workspace overlaps cu_seqlens");
    }

    kda::ChunkLaunch L{};
    L.q = a->q; L.k = a->k; L.v = a->v; L.g = a->g; L.beta = a->beta;
    L.h0 = a->initial_state; L.hT = a->final_state; L.o = a->o;
    L.cu_seqlens = a->cu_seqlens;
    L.B = a->B; L.T = a->T; L.H = a->H; L.dk = a->dk; L.dv = a->dv; L.N = N;
    L.chunk = a->chunk_size; L.scale = a->scale;
    L.in_bf16 = a->in_dtype == KDA_DTYPE_BF16;
    L.out_bf16 = a->out_dtype == KDA_DTYPE_BF16;
    L.xf = xform_of(a);
    L.workspace = a->workspace; L.workspace_bytes = a->workspace_bytes;
    L.stream = static_cast<hipStream_t>(a->stream);
    return hip_status(kda::launch_chunk(L), "kda_chunk_fwd launch");
}

kda_status kda_recurrent_fwd(const kda_chunk_fwd_args *user) {
    g_last_error.clear();
    kda_chunk_fwd_args args;
    kda_status st = read_args(user, args);
    if (st != KDA_OK) return st;
    const kda_chunk_fwd_args *a = &args;
    if (a->B < 0 || a->T < 0 || a->H <= 0 || a->num_seqs < 0)
        return fail(KDA_ERR_BAD_SHAPE, "B=%d T=%d H=%d num_seqs=%d", a->B, a->T, a->H, a->num_seqs);
    if (!valid_dim(a->dk) || !valid_dim(a->dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d dv=%d (supported: 64, 128)", a->dk, a->dv);
    if (!valid_dtype(a->in_dtype) || !valid_dtype(a->out_dtype))
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype=%d out_dtype=%d", a->in_dtype, a->out_dtype);
    if (!std::isfinite(a->scale)) return fail(KDA_ERR_BAD_SHAPE, "scale is not finite");
    if (a->cu_seqlens ? a->B != 1 : a->num_seqs != a->B)
        return fail(KDA_ERR_BAD_SHAPE, "num_seqs=%d with B=%d (%s)", a->num_seqs, a->B,
                    a->cu_seqlens ? "packed input needs B = 1" : "num_seqs must equal B");
    st = check_prefill_buffers(a);
    if (st != KDA_OK) return st;
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    if (a->num_seqs == 0 || (tokens == 0 && !a->final_state)) return KDA_OK;
    // Appends of more than kRouteTokens tokens per sequence (on average) run faster chunkwise (measured on
    // MI355X, 16 heads, d = 128: the token kernel wins up to about 16 new tokens per sequence, the chunk path
    // from 64 on).  With a caller workspace big enough for kda_chunk_fwd (chunk 64) such a call goes there;
    // without one it stays token by token, so no workspace is ever required.
    constexpr int64_t kRouteTokens = 16;
    if (a->workspace && tokens > kRouteTokens * a->num_seqs) {
        kda_chunk_fwd_args c = *a;
        c.chunk_size = 64;
        const size_t need = kda_chunk_fwd_workspace_bytes(&c);
        if (need != static_cast<size_t>(-1) && a->workspace_bytes >= need) return kda_chunk_fwd(&c);
    }

    kda::RecurrentLaunch L{};
    L.q = a->q; L.k = a->k; L.v = a->v; L.g = a->g; L.beta = a->beta;
    L.h0 = a->initial_state; L.hT = a->final_state; L.o = a->o;
    L.cu_seqlens = a->cu_seqlens;
    L.N = a->num_seqs; L.T = a->T; L.H = a->H; L.dk = a->dk; L.dv = a->dv; L.scale = a->scale;
    L.in_bf16 = a->in_dtype == KDA_DTYPE_BF16;
    L.out_bf16 = a->out_dtype == KDA_DTYPE_BF16;
    // one token per sequence is a decode step: the decode kernel's wide rows stream the state at the copy
    // rate, where the multi-token kernel's 16-column slices reach about half of it
    L.multi_token = a->cu_seqlens != nullptr || a->T != 1;
    L.xf = xform_of(a);
    L.stream = static_cast<hipStream_t>(a->stream);
    return hip_status(kda::launch_recurrent(L), "kda_recurrent_fwd launch");
}

kda_status kda_recurrent_step(const kda_recurrent_step_args *user) {
    g_last_error.clear();
    kda_recurrent_step_args args;
    const kda_status st = read_args(user, args);
    if (st != KDA_OK) return st;
    const kda_recurrent_step_args *a = &args;
    if (a->N < 0 || a->H <= 0) return fail(KDA_ERR_BAD_SHAPE, "N=%d H=%d", a->N, a->H);
    if (!valid_dim(a->dk) || !valid_dim(a->dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d dv=%d (supported: 64, 128)", a->dk, a->dv);
    if (!valid_dtype(a->in_dtype) || !valid_dtype(a->out_dtype))
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype=%d out_dtype=%d", a->in_dtype, a->out_dtype);
    if (!std::isfinite(a->scale)) return fail(KDA_ERR_BAD_SHAPE, "scale is not finite");
    if (a->N == 0) return KDA_OK;
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o || !a->final_state)
        return fail(KDA_ERR_NULL_POINTER, "q, k, v, g, beta, o and final_state are required");
    const size_t nh = static_cast<size_t>(a->N) * a->H, in_sz = dsize(a->in_dtype);
    const size_t sbytes = nh * a->dk * a->dv * 4;
    const Range ro = range_of(a->o, nh * a->dv * dsize(a->out_dtype));
    const Range rf = range_of(a->final_state, sbytes);
    const Range ins[] = {range_of(a->q, nh * a->dk * in_sz), range_of(a->k, nh * a->dk * in_sz),
                         range_of(a->v, nh * a->dv * in_sz), range_of(a->g, nh * gate_width(a) * 4),
                         range_of(a->beta, nh * in_sz)};
    for (const Range &r : ins)
        if (overlap(ro, r) || overlap(rf, r)) return fail(KDA_ERR_ALIAS, "an output overlaps an input");
    if (overlap(ro, rf)) return fail(KDA_ERR_ALIAS, "o overlaps final_state");
    if (a->initial_state && overlap(ro, range_of(a->initial_state, sbytes)))
        return fail(KDA_ERR_ALIAS, "o overlaps initial_state");
    if (a->initial_state && a->initial_state != a->final_state &&
        overlap(rf, range_of(a->initial_state, sbytes)))
        return fail(KDA_ERR_ALIAS, "final_state partially overlaps initial_state");

    kda::RecurrentLaunch L{};
    L.q = a->q; L.k = a->k; L.v = a->v; L.g = a->g; L.beta = a->beta;
    L.h0 = a->initial_state; L.hT = a->final_state; L.o = a->o;
    L.cu_seqlens = nullptr;
    L.N = a->N; L.T = 1; L.H = a->H; L.dk = a->dk; L.dv = a->dv; L.scale = a->scale;
    L.in_bf16 = a->in_dtype == KDA_DTYPE_BF16;
    L.out_bf16 = a->out_dtype == KDA_DTYPE_BF16;
    L.multi_token = false;
    L.xf = xform_of(a);
    L.stream = static_cast<hipStream_t>(a->stream);
    return hip_status(kda::launch_recurrent(L), "kda_recurrent_step launch");
}

size_t kda_recurrent_bwd_workspace_bytes(const kda_recurrent_bwd_args *user) {
    kda_recurrent_bwd_args a;
    if (read_bwd_args(user, a) != KDA_OK) return static_cast<size_t>(-1);
    return kda::backward_workspace_bytes(a.B, a.T, a.H, a.dk, a.dv, a.num_seqs, a.cu_seqlens != nullptr,
                                         (a.flags & (KDA_FLAG_QK_L2NORM | KDA_FLAG_GATE_SOFTPLUS)) != 0,
                                         (a.flags & KDA_FLAG_SCALAR_GATE) != 0);
}

kda_status kda_recurrent_bwd(const kda_recurrent_bwd_args *user) {
    g_last_error.clear();
    kda_recurrent_bwd_args args;
    const kda_status st = read_bwd_args(user, args);
    if (st != KDA_OK) return st;
    const kda_recurrent_bwd_args *a = &args;
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    const int N = a->num_seqs;
    if (N == 0 || (tokens == 0 && !a->grad_initial_state)) return KDA_OK;
    const size_t need = kda::backward_workspace_bytes(a->B, a->T, a->H, a->dk, a->dv, N, a->cu_seqlens != nullptr,
                                                      (a->flags & (KDA_FLAG_QK_L2NORM | KDA_FLAG_GATE_SOFTPLUS)) != 0,
                                                      (a->flags & KDA_FLAG_SCALAR_GATE) != 0);
    const kda_status sb = check_bwd_buffers(a, need);
    if (sb != KDA_OK) return sb;

    kda::BackwardLaunch L{};
    L.q = a->q; L.k = a->k; L.v = a->v; L.g = a->g; L.beta = a->beta; L.d_o = a->grad_o;
    L.h0 = a->initial_state; L.dhT = a->grad_final_state;
    L.dq = a->grad_q; L.dk = a->grad_k; L.dv = a->grad_v; L.dg = a->grad_g; L.dbeta = a->grad_beta;
    L.dh0 = a->grad_initial_state;
    L.cu_seqlens = a->cu_seqlens;
    L.B = a->B; L.N = N; L.T = a->T; L.H = a->H; L.dk_dim = a->dk; L.dv_dim = a->dv;
    L.scale = a->scale;
    L.in_bf16 = a->in_dtype == KDA_DTYPE_BF16;
    L.scalar_gate = (a->flags & KDA_FLAG_SCALAR_GATE) != 0;
    L.xf = xform_of(a);
    L.workspace = a->workspace;
    L.stream = static_cast<hipStream_t>(a->stream);
    return hip_status(kda::launch_backward(L), "kda_recurrent_bwd launch");
}

size_t kda_chunk_bwd_workspace_bytes(const kda_recurrent_bwd_args *user) {
    kda_recurrent_bwd_args a;
    if (read_bwd_args(user, a) != KDA_OK || a.flags != 0 ||
        !kda::chunk_bwd_supported(a.in_dtype == KDA_DTYPE_BF16, a.dk, a.dv))
        return static_cast<size_t>(-1);
    return kda::chunk_bwd_workspace_bytes(a.B, a.T, a.H, a.num_seqs, a.cu_seqlens != nullptr);
}

kda_status kda_chunk_bwd(const kda_recurrent_bwd_args *user) {
    g_last_error.clear();
    kda_recurrent_bwd_args args;
    const kda_status st = read_bwd_args(user, args);
    if (st != KDA_OK) return st;
    const kda_recurrent_bwd_args *a = &args;
    if (a->flags != 0)
        return fail(KDA_ERR_UNSUPPORTED, "flags 0x%x: the chunkwise gradients take no input transforms "
                    "(kda_recurrent_bwd does)", a->flags);
    if (!kda::chunk_bwd_supported(a->in_dtype == KDA_DTYPE_BF16, a->dk, a->dv))
        return fail(KDA_ERR_UNSUPPORTED, "the chunkwise gradients need bf16 inputs and dk = dv = 128 "
                    "(kda_recurrent_bwd takes the rest)");
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    const int N = a->num_seqs;
    if (N == 0 || (tokens == 0 && !a->grad_initial_state)) return KDA_OK;
    const bool varlen = a->cu_seqlens != nullptr;
    const size_t need = kda::chunk_bwd_workspace_bytes(a->B, a->T, a->H, N, varlen);
    const kda_status sb = check_bwd_buffers(a, need);
    if (sb != KDA_OK) return sb;
    if (!kda::chunk_bwd_grids_fit(a->B, a->T, a->H, N, varlen))
        return fail(KDA_ERR_UNSUPPORTED, "problem too large for one launch of the chunkwise gradients");

    kda::BackwardLaunch L{};
    L.q = a->q; L.k = a->k; L.v = a->v; L.g = a->g; L.beta = a->beta; L.d_o = a->grad_o;
    L.h0 = a->initial_state; L.dhT = a->grad_final_state;
    L.dq = a->grad_q; L.dk = a->grad_k; L.dv = a->grad_v; L.dg = a->grad_g; L.dbeta = a->grad_beta;
    L.dh0 = a->grad_initial_state;
    L.cu_seqlens = a->cu_seqlens;
    L.B = a->B; L.N = N; L.T = a->T; L.H = a->H; L.dk_dim = a->dk; L.dv_dim = a->dv;
    L.scale = a->scale;
    L.in_bf16 = true;
    L.workspace = a->workspace;
    L.stream = static_cast<hipStream_t>(a->stream);
    return hip_status(kda::launch_chunk_bwd(L), "kda_chunk_bwd launch");
}

}  // extern "C"

namespace {

// Checks shared by the token-level and chunkwise DPLR entry points (same field names).
template <class A>
kda_status check_dplr(const A *a, bool *nothing_to_do) {
    *nothing_to_do = false;
    if (a->B < 0 || a->T < 0 || a->H <= 0 || a->num_seqs < 0)
        return fail(KDA_ERR_BAD_SHAPE, "B=%d T=%d H=%d num_seqs=%d", a->B, a->T, a->H, a->num_seqs);
    if (!valid_dim(a->dk) || !valid_dim(a->dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d dv=%d (supported: 64, 128)", a->dk, a->dv);
    if (!valid_dtype(a->in_dtype) || !valid_dtype(a->out_dtype))
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype=%d out_dtype=%d", a->in_dtype, a->out_dtype);
    if (!std::isfinite(a->scale)) return fail(KDA_ERR_BAD_SHAPE, "scale is not finite");
    if (a->cu_seqlens ? a->B != 1 : a->num_seqs != a->B)
        return fail(KDA_ERR_BAD_SHAPE, "num_seqs=%d with B=%d (%s)", a->num_seqs, a->B,
                    a->cu_seqlens ? "packed input needs B = 1" : "num_seqs must equal B");
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    if (tokens > INT32_MAX)
        return fail(KDA_ERR_BAD_SHAPE, "B*T=%lld tokens (at most %d)", static_cast<long long>(tokens), INT32_MAX);
    if (tokens * a->H * (a->dk > a->dv ? a->dk : a->dv) > (int64_t{1} << 40))
        return fail(KDA_ERR_BAD_SHAPE, "problem too large");
    const int N = a->num_seqs;
    if (N > 65535 || a->H > 65535) return fail(KDA_ERR_UNSUPPORTED, "N=%d H=%d (at most 65535 each)", N, a->H);
    if (N == 0 || (tokens == 0 && !a->final_state)) {
        *nothing_to_do = true;
        return KDA_OK;
    }
    if (tokens > 0 && (!a->q || !a->k || !a->v || !a->g || !a->a || !a->b || !a->o))
        return fail(KDA_ERR_NULL_POINTER, "q, k, v, g, a, b and o are required");
    const size_t th = static_cast<size_t>(tokens) * a->H, in_sz = dsize(a->in_dtype);
    const size_t sbytes = static_cast<size_t>(N) * a->H * a->dk * a->dv * 4;
    const Range ro = range_of(a->o, th * a->dv * dsize(a->out_dtype));
    const Range ins[] = {range_of(a->q, th * a->dk * in_sz), range_of(a->k, th * a->dk * in_sz),
                         range_of(a->v, th * a->dv * in_sz), range_of(a->g, th * a->dk * 4),
                         range_of(a->a, th * a->dk * in_sz), range_of(a->b, th * a->dk * in_sz)};
    const Range rh0 = range_of(a->initial_state, a->initial_state ? sbytes : 0);
    const Range rcu = range_of(a->cu_seqlens, a->cu_seqlens ? (static_cast<size_t>(N) + 1) * 4 : 0);
    for (const Range &r : ins)
        if (overlap(ro, r)) return fail(KDA_ERR_ALIAS, "o overlaps an input");
    if (overlap(ro, rh0)) return fail(KDA_ERR_ALIAS, "o overlaps initial_state");
    if (overlap(ro, rcu)) return fail(KDA_ERR_ALIAS, "o overlaps cu_seqlens");
    if (a->final_state) {
        const Range rf = range_of(a->final_state, sbytes);
        for (const Range &r : ins)
            if (overlap(rf, r)) return fail(KDA_ERR_ALIAS, "final_state overlaps an input");
        if (overlap(rf, ro)) return fail(KDA_ERR_ALIAS, "final_state overlaps o");
        if (overlap(rf, rcu)) return fail(KDA_ERR_ALIAS, "final_state overlaps cu_seqlens");
        if (a->initial_state && a->initial_state != a->final_state && overlap(rf, rh0))
            return fail(KDA_ERR_ALIAS, "final_state partially overlaps initial_state");
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_dplr_recurrent_fwd(const kda_dplr_args *user) {
    g_last_error.clear();
    if (!user) return fail(KDA_ERR_NULL_POINTER, "args is NULL");
    if (user->struct_size != sizeof(kda_dplr_args))
        return fail(KDA_ERR_BAD_STRUCT, "struct_size %u (expected %zu)", user->struct_size, sizeof(kda_dplr_args));
    const kda_dplr_args *a = user;
    bool none = false;
    const kda_status st = check_dplr(a, &none);
    if (st != KDA_OK || none) return st;
    kda::DplrLaunch L{};
    L.q = a->q; L.k = a->k; L.v = a->v; L.a = a->a; L.b = a->b; L.g = a->g;
    L.h0 = a->initial_state; L.hT = a->final_state; L.o = a->o;
    L.cu_seqlens = a->cu_seqlens;
    L.N = a->num_seqs; L.T = a->T; L.H = a->H; L.dk = a->dk; L.dv = a->dv; L.scale = a->scale;
    L.in_bf16 = a->in_dtype == KDA_DTYPE_BF16;
    L.out_bf16 = a->out_dtype == KDA_DTYPE_BF16;
    L.stream = static_cast<hipStream_t>(a->stream);
    return hip_status(kda::launch_dplr(L), "kda_dplr_recurrent_fwd launch");
}

size_t kda_dplr_chunk_fwd_workspace_bytes(const kda_dplr_chunk_args *a) {
    if (!a || a->struct_size != sizeof(kda_dplr_chunk_args)) return static_cast<size_t>(-1);
    if (a->B < 0 || a->T < 0 || a->H <= 0 || a->num_seqs < 0 || !valid_dim(a->dk) || !valid_dim(a->dv))
        return static_cast<size_t>(-1);
    if (a->cu_seqlens ? a->B != 1 : a->num_seqs != a->B) return static_cast<size_t>(-1);
    return kda::dplr_chunk_workspace_bytes(a->B, a->T, a->H, a->dk, a->dv, a->num_seqs, a->cu_seqlens != nullptr);
}

kda_status kda_dplr_chunk_fwd(const kda_dplr_chunk_args *user) {
    g_last_error.clear();
    if (!user) return fail(KDA_ERR_NULL_POINTER, "args is NULL");
    if (user->struct_size != sizeof(kda_dplr_chunk_args))
        return fail(KDA_ERR_BAD_STRUCT, "struct_size %u (expected %zu)", user->struct_size,
                    sizeof(kda_dplr_chunk_args));
    const kda_dplr_chunk_args *a = user;
    bool none = false;
    kda_status st = check_dplr(a, &none);
    if (st != KDA_OK || none) return st;
    const int N = a->num_seqs;
    const size_t need = kda::dplr_chunk_workspace_bytes(a->B, a->T, a->H, a->dk, a->dv, N, a->cu_seqlens != nullptr);
    if (a->workspace_bytes < need || (need > 0 && !a->workspace))
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", a->workspace_bytes, need);
    {   // the workspace must not overlap any input or output
        const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
        const size_t th = static_cast<size_t>(tokens) * a->H, in_sz = dsize(a->in_dtype);
        const size_t sbytes = static_cast<size_t>(N) * a->H * a->dk * a->dv * 4;
        const Range rw = range_of(a->workspace, need);
        const Range others[] = {range_of(a->q, th * a->dk * in_sz), range_of(a->k, th * a->dk * in_sz),
                                range_of(a->v, th * a->dv * in_sz), range_of(a->g, th * a->dk * 4),
                                range_of(a->a, th * a->dk * in_sz), range_of(a->b, th * a->dk * in_sz),
                                range_of(a->o, th * a->dv * dsize(a->out_dtype)),
                                range_of(a->initial_state, a->initial_state ? sbytes : 0),
                                range_of(a->final_state, a->final_state ? sbytes : 0),
                                range_of(a->cu_seqlens, a->cu_seqlens ? (static_cast<size_t>(N) + 1) * 4 : 0)};
        for (const Range &r : others)
            if (overlap(rw, r)) return fail(KDA_ERR_ALIAS, "workspace overlaps an input or output");
    }
    kda::DplrChunkLaunch L{};
    L.q = a->q; L.k = a->k; L.v = a->v; L.a = a->a; L.b = a->b; L.g = a->g;
    L.h0 = a->initial_state; L.hT = a->final_state; L.o = a->o;
    L.cu_seqlens = a->cu_seqlens;
    L.B = a->B; L.T = a->T; L.H = a->H; L.dk = a->dk; L.dv = a->dv; L.N = N; L.scale = a->scale;
    L.in_bf16 = a->in_dtype == KDA_DTYPE_BF16;
    L.out_bf16 = a->out_dtype == KDA_DTYPE_BF16;
    L.workspace = a->workspace;
    L.stream = static_cast<hipStream_t>(a->stream);
    return hip_status(kda::launch_dplr_chunk(L), "kda_dplr_chunk_fwd launch");
}

}  // extern "C"
