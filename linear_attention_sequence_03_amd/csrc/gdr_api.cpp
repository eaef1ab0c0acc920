// gdr_api.cpp -- the C ABI declared in include/gdr.h: argument checking on the
// host (nothing is launched unless every check passes), then dispatch to the
// kernel launchers.
#include "gdr.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "gdr_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

gdr_status fail(gdr_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};

Range rng(const char* name, const void* p, int64_t elems, size_t esize) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + (uintptr_t)elems * esize : lo};
}

bool overlap(const Range& a, const Range& b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a*b*... without int64 overflow; returns -1 on overflow.
int64_t mul(std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x != 0 && r > INT64_MAX / x) return -1;
        r *= x;
    }
    return r;
}

constexpr unsigned kPrologueAll = GDR_PROLOGUE_L2NORM_QK | GDR_PROLOGUE_BETA_SIGMOID |
                                   GDR_PROLOGUE_DECAY_SOFTPLUS;

gdr_status check_common(int64_t B, int64_t H, int64_t dk, int64_t dv, gdr_dtype io, gdr_gate gate) {
    if (B < 1 || H < 1 || dk < 1 || dv < 1)
        return fail(GDR_ERR_INVALID_ARG, "sizes must be positive (B=%lld H=%lld dk=%lld dv=%lld)",
                    (long long)B, (long long)H, (long long)dk, (long long)dv);
    if (io != GDR_F32 && io != GDR_BF16) return fail(GDR_ERR_INVALID_ARG, "bad io dtype %d", (int)io);
    if (gate != GDR_GATE_SCALAR && gate != GDR_GATE_CHANNEL)
        return fail(GDR_ERR_INVALID_ARG, "bad gate kind %d", (int)gate);
    if (dk != dv || (dk != 64 && dk != 128))
        return fail(GDR_ERR_UNSUPPORTED, "unsupported head dims dk=%lld dv=%lld (need dk=dv in {64,128})",
                    (long long)dk, (long long)dv);
    return GDR_OK;
}

gdr_status check_ptrs(const Range* rs, int n, int first_output) {
    for (int i = 0; i < n; ++i)
        if (rs[i].lo && !aligned16(reinterpret_cast<const void*>(rs[i].lo)))
            return fail(GDR_ERR_INVALID_ARG, "%s is not 16-byte aligned", rs[i].name);
    // every output against every other buffer
    for (int i = first_output; i < n; ++i)
        for (int j = 0; j < n; ++j)
            if (i != j && overlap(rs[i], rs[j]))
                return fail(GDR_ERR_INVALID_ARG, "%s overlaps %s", rs[i].name, rs[j].name);
    return GDR_OK;
}

}  // namespace

extern "C" {

const char* gdr_status_string(gdr_status s) {
    switch (s) {
        case GDR_OK: return "GDR_OK";
        case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
        case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
        case GDR_ERR_HIP: return "GDR_ERR_HIP";
    }
    return "GDR_UNKNOWN_STATUS";
}

const char* gdr_last_error(void) { return g_last_error; }

gdr_status gdr_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                        int64_t chunk, gdr_dtype io, gdr_gate gate, size_t* bytes) {
    g_last_error[0] = 0;
    if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    gdr_status s = check_common(B, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    if (T < 0) return fail(GDR_ERR_INVALID_ARG, "T must be >= 0 (T=%lld)", (long long)T);
    if (chunk < 1) return fail(GDR_ERR_INVALID_ARG, "chunk must be positive");
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(GDR_ERR_UNSUPPORTED, "unsupported chunk %lld (need 16, 32 or 64)", (long long)chunk);
    const int64_t units = mul({B, H, (T + chunk - 1) / chunk});
    if (units < 0 || units > INT32_MAX)
        return fail(GDR_ERR_UNSUPPORTED, "B*H*ceil(T/chunk) too large");
    *bytes = gdr::chunk_workspace_bytes(B, T, H, dk, chunk, io == GDR_BF16, gate == GDR_GATE_CHANNEL);
    return GDR_OK;
}

gdr_status gdr_chunk_fwd_prologue_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk,
                                                 int64_t dv, int64_t chunk, gdr_dtype io,
                                                 gdr_gate gate, unsigned flags, size_t* bytes) {
    gdr_status s = gdr_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate, bytes);
    if (s != GDR_OK) return s;
    if (flags & ~kPrologueAll) {
        *bytes = 0;
        return fail(GDR_ERR_INVALID_ARG, "unknown prologue flags 0x%x", flags);
    }
    if (mul({B, T, H, dk, 4}) < 0) {
        *bytes = 0;
        return fail(GDR_ERR_UNSUPPORTED, "tensor sizes overflow");
    }
    *bytes = gdr::chunk_prologue_workspace_bytes(B, T, H, dk, chunk, io == GDR_BF16,
                                                 gate == GDR_GATE_CHANNEL, flags);
    return GDR_OK;
}

}  // extern "C"

namespace {

gdr_status chunk_fwd_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                                 const float* beta, const float* S0, void* o, float* S_T, int64_t B,
                                 int64_t T, int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                                 gdr_dtype io, gdr_gate gate, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, unsigned prologue, bool noalloc = false) {
    size_t need = 0;
    gdr_status s = gdr_chunk_fwd_prologue_workspace_size(B, T, H, dk, dv, chunk, io, gate, prologue, &need);
    if (s != GDR_OK) return s;
    const int64_t ntok = mul({B, T, H});
    if (ntok < 0 || mul({ntok, dk}) < 0 || mul({B, H, dv, dk}) < 0)
        return fail(GDR_ERR_UNSUPPORTED, "tensor sizes overflow");
    if (mul({B, H, dv / 16}) > INT32_MAX) return fail(GDR_ERR_UNSUPPORTED, "B*H too large");
    // The kernels address one chunk's rows with 32-bit byte offsets from the
    // chunk's first row (row stride at most H*d*4 bytes: fp32 rows, or the
    // per-channel decay).
    if (mul({chunk, H, dk > dv ? dk : dv, 4}) > INT32_MAX)
        return fail(GDR_ERR_UNSUPPORTED, "H too large (chunk*H*d*4 bytes must stay below 2^31)");
    if (T > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, log_alpha, beta and o must be non-NULL");
    if (noalloc) {
        if (need > GDR_NOALLOC_SCRATCH_BYTES)
            return fail(GDR_ERR_UNSUPPORTED,
                        "this call needs %zu bytes of workspace, above the %zu-byte fixed scratch",
                        need, (size_t)GDR_NOALLOC_SCRATCH_BYTES);
    } else {
        if (need > 0 && !workspace) return fail(GDR_ERR_INVALID_ARG, "workspace is NULL");
        if (workspace_bytes < need)
            return fail(GDR_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes,
                        need);
    }
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const int64_t la_elems = gate == GDR_GATE_CHANNEL ? ntok * dk : ntok;
    const Range rs[] = {
        rng("q", q, ntok * dk, es),          rng("k", k, ntok * dk, es),
        rng("v", v, ntok * dv, es),          rng("log_alpha", log_alpha, la_elems, 4),
        rng("beta", beta, ntok, 4),          rng("S0", S0, B * H * dv * dk, 4),
        rng("o", o, ntok * dv, es),          rng("S_T", S_T, B * H * dv * dk, 4),
        rng("workspace", workspace, (int64_t)need, 1),
    };
    s = check_ptrs(rs, 9, 6);
    if (s != GDR_OK) return s;
    if (noalloc && need > 0) {
        // the fixed scratch stands in for the workspace; every byte of it the
        // state pass reads is written by this call's preparation kernel first
        const hipError_t e = gdr::noalloc_scratch(stream, &workspace);
        if (e != hipSuccess)
            return fail(GDR_ERR_HIP, "no device scratch on this stream's device: %s", hipGetErrorString(e));
    }
    gdr::ChunkArgs a{q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk,
                     io == GDR_BF16, gate == GDR_GATE_CHANNEL, workspace, stream, prologue};
    const hipError_t err = gdr::chunk_fwd_launch(a);
    if (err == hipErrorNotSupported)
        return fail(GDR_ERR_UNSUPPORTED, "this gate/dtype combination is not available");
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* S0, void* o, float* S_T, int64_t B,
                         int64_t T, int64_t H, int64_t dk, int64_t dv, int64_t chunk, gdr_dtype io,
                         gdr_gate gate, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk, io, gate,
                          workspace, workspace_bytes, stream, 0);
}

gdr_status gdr_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                 const float* beta, const float* S0, void* o, float* S_T, int64_t B,
                                 int64_t T, int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                                 gdr_dtype io, gdr_gate gate, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk, io, gate,
                          nullptr, 0, stream, 0, true);
}

gdr_status gdr_chunk_fwd_prologue(const void* q, const void* k, const void* v,
                                  const float* log_alpha, const float* beta, const float* S0,
                                  void* o, float* S_T, int64_t B, int64_t T, int64_t H, int64_t dk,
                                  int64_t dv, int64_t chunk, gdr_dtype io, gdr_gate gate,
                                  void* workspace, size_t workspace_bytes, unsigned flags,
                                  hipStream_t stream) {
    g_last_error[0] = 0;
    if (flags & ~kPrologueAll) return fail(GDR_ERR_INVALID_ARG, "unknown prologue flags 0x%x", flags);
    return chunk_fwd_impl(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk, io, gate,
                          workspace, workspace_bytes, stream, flags);
}

gdr_status gdr_decode_step_prologue(const void* q, const void* k, const void* v,
                                    const float* log_alpha, const float* beta, const float* S_in,
                                    float* S_out, void* o, int64_t B, int64_t H, int64_t dk, int64_t dv,
                                    gdr_dtype io, gdr_gate gate, unsigned flags, hipStream_t stream);

gdr_status gdr_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* S_in, float* S_out, void* o, int64_t B,
                           int64_t H, int64_t dk, int64_t dv, gdr_dtype io, gdr_gate gate,
                           hipStream_t stream) {
    return gdr_decode_step_prologue(q, k, v, log_alpha, beta, S_in, S_out, o, B, H, dk, dv, io, gate,
                                    0, stream);
}

gdr_status gdr_decode_step_prologue(const void* q, const void* k, const void* v,
                                    const float* log_alpha, const float* beta, const float* S_in,
                                    float* S_out, void* o, int64_t B, int64_t H, int64_t dk, int64_t dv,
                                    gdr_dtype io, gdr_gate gate, unsigned flags, hipStream_t stream) {
    g_last_error[0] = 0;
    gdr_status s = check_common(B, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    const int64_t nst = mul({B, H, dv, dk});
    if (nst < 0 || mul({B, H, dv}) > ((int64_t)INT32_MAX) * 4)
        return fail(GDR_ERR_UNSUPPORTED, "state too large");
    if (!q || !k || !v || !log_alpha || !beta || !S_in || !S_out || !o)
        return fail(GDR_ERR_INVALID_ARG, "all pointers must be non-NULL");
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const int64_t bh = B * H;
    const Range in_state = rng("S_in", S_in, nst, 4);
    const Range out_state = rng("S_out", S_out, nst, 4);
    if (S_in != S_out && overlap(in_state, out_state))
        return fail(GDR_ERR_INVALID_ARG, "S_out partially overlaps S_in");
    const Range rs[] = {
        rng("q", q, bh * dk, es), rng("k", k, bh * dk, es), rng("v", v, bh * dv, es),
        rng("log_alpha", log_alpha, gate == GDR_GATE_CHANNEL ? bh * dk : bh, 4),
        rng("beta", beta, bh, 4),
        S_in == S_out ? Range{"S_in", 0, 0} : in_state,
        out_state, rng("o", o, bh * dv, es),
    };
    if (!aligned16(S_in)) return fail(GDR_ERR_INVALID_ARG, "S_in is not 16-byte aligned");
    s = check_ptrs(rs, 8, 6);
    if (s != GDR_OK) return s;
    if (flags & ~kPrologueAll) return fail(GDR_ERR_INVALID_ARG, "unknown prologue flags 0x%x", flags);
    gdr::DecodeArgs a{q, k, v, log_alpha, beta, S_in, S_out, o, B, H, dk, dv,
                      io == GDR_BF16, gate == GDR_GATE_CHANNEL, stream, nullptr, nullptr, flags};
    const hipError_t err = gdr::decode_step_launch(a);
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

gdr_status gdr_decode_multi(const void* q, const void* k, const void* v, const float* log_alpha,
                            const float* beta, const float* S_in, float* S_out,
                            const int32_t* accepted, void* o, int64_t B, int64_t Td, int64_t H,
                            int64_t dk, int64_t dv, gdr_dtype io, gdr_gate gate, hipStream_t stream) {
    g_last_error[0] = 0;
    gdr_status s = check_common(B, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    if (Td < 1 || Td > 64)
        return fail(GDR_ERR_UNSUPPORTED, "Td must be in [1, 64] (Td=%lld); use gdr_chunk_fwd for longer runs",
                    (long long)Td);
    const int64_t nst = mul({B, H, dv, dk});
    if (nst < 0 || mul({B, H, dv}) > ((int64_t)INT32_MAX) * 4 || mul({B, Td, H, dk}) < 0)
        return fail(GDR_ERR_UNSUPPORTED, "tensors too large");
    if (!q || !k || !v || !log_alpha || !beta || !S_in)
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, log_alpha, beta and S_in must be non-NULL");
    if (!S_out && !o) return GDR_OK;   // nothing requested
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const int64_t ntok = B * Td * H;
    const Range in_state = rng("S_in", S_in, nst, 4);
    const Range out_state = rng("S_out", S_out, nst, 4);
    if (S_out && S_in != S_out && overlap(in_state, out_state))
        return fail(GDR_ERR_INVALID_ARG, "S_out partially overlaps S_in");
    const Range acc = rng("accepted", accepted, B, 4);
    if (accepted && (reinterpret_cast<uintptr_t>(accepted) & 3u))
        return fail(GDR_ERR_INVALID_ARG, "accepted is not 4-byte aligned");
    const Range rs[] = {
        rng("q", q, ntok * dk, es), rng("k", k, ntok * dk, es), rng("v", v, ntok * dv, es),
        rng("log_alpha", log_alpha, gate == GDR_GATE_CHANNEL ? ntok * dk : ntok, 4),
        rng("beta", beta, ntok, 4),
        S_in == S_out ? Range{"S_in", 0, 0} : in_state,
        out_state, rng("o", o, ntok * dv, es),
    };
    if (!aligned16(S_in)) return fail(GDR_ERR_INVALID_ARG, "S_in is not 16-byte aligned");
    s = check_ptrs(rs, 8, 6);
    if (s != GDR_OK) return s;
    for (int i = 6; i < 8; ++i)
        if (overlap(rs[i], acc)) return fail(GDR_ERR_INVALID_ARG, "%s overlaps accepted", rs[i].name);
    gdr::DecodeMultiArgs a{q, k, v, log_alpha, beta, S_in, S_out, accepted, o, B, Td, H, dk, dv,
                           io == GDR_BF16, gate == GDR_GATE_CHANNEL, stream};
    const hipError_t err = gdr::decode_multi_launch(a);
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

namespace {

gdr_status tree_common(int64_t B, int64_t Td, int64_t H, int64_t dk, int64_t dv, gdr_dtype io, gdr_gate gate) {
    gdr_status s = check_common(B, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    if (Td < 1 || Td > 64)
        return fail(GDR_ERR_UNSUPPORTED, "Td must be in [1, 64] (Td=%lld)", (long long)Td);
    if (mul({B, H, dv, dk}) < 0 || mul({B, Td, H, dk > dv ? dk : dv}) < 0 || mul({B, H, dv / 64}) > INT32_MAX)
        return fail(GDR_ERR_UNSUPPORTED, "tensors too large");
    return GDR_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

gdr_status gdr_decode_tree(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* S_in, const int32_t* parent, void* o, float* D,
                           int64_t B, int64_t Td, int64_t H, int64_t dk, int64_t dv, gdr_dtype io,
                           gdr_gate gate, hipStream_t stream) {
    g_last_error[0] = 0;
    gdr_status s = tree_common(B, Td, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    if (!q || !k || !v || !log_alpha || !beta || !S_in || !parent)
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, log_alpha, beta, S_in and parent must be non-NULL");
    if (!aligned4(parent)) return fail(GDR_ERR_INVALID_ARG, "parent is not 4-byte aligned");
    if (!o && !D) return GDR_OK;   // nothing requested
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const int64_t ntok = B * Td * H;
    const Range par = rng("parent", parent, B * Td, 4);
    const Range rs[] = {
        rng("q", q, ntok * dk, es), rng("k", k, ntok * dk, es), rng("v", v, ntok * dv, es),
        rng("log_alpha", log_alpha, gate == GDR_GATE_CHANNEL ? ntok * dk : ntok, 4),
        rng("beta", beta, ntok, 4), rng("S_in", S_in, B * H * dv * dk, 4),
        rng("o", o, ntok * dv, es), rng("D", D, ntok * dv, 4),
    };
    s = check_ptrs(rs, 8, 6);
    if (s != GDR_OK) return s;
    for (int i = 6; i < 8; ++i)
        if (overlap(rs[i], par)) return fail(GDR_ERR_INVALID_ARG, "%s overlaps parent", rs[i].name);
    gdr::TreeArgs a{q, k, v, log_alpha, beta, S_in, parent, o, D, nullptr, nullptr, B, Td, H, dk, dv,
                    io == GDR_BF16, gate == GDR_GATE_CHANNEL, stream};
    const hipError_t err = gdr::decode_tree_launch(a);
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

gdr_status gdr_decode_tree_commit(const void* k, const float* log_alpha, const int32_t* parent,
                                  const float* D, const int32_t* accepted, const float* S_in, float* S_out,
                                  int64_t B, int64_t Td, int64_t H, int64_t dk, int64_t dv, gdr_dtype io,
                                  gdr_gate gate, hipStream_t stream) {
    g_last_error[0] = 0;
    gdr_status s = tree_common(B, Td, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    if (!k || !log_alpha || !parent || !D || !accepted || !S_in || !S_out)
        return fail(GDR_ERR_INVALID_ARG, "k, log_alpha, parent, D, accepted, S_in and S_out must be non-NULL");
    if (!aligned4(parent) || !aligned4(accepted))
        return fail(GDR_ERR_INVALID_ARG, "parent and accepted must be 4-byte aligned");
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const int64_t ntok = B * Td * H, nst = B * H * dv * dk;
    const Range in_state = rng("S_in", S_in, nst, 4), out_state = rng("S_out", S_out, nst, 4);
    if (S_in != S_out && overlap(in_state, out_state))
        return fail(GDR_ERR_INVALID_ARG, "S_out partially overlaps S_in");
    const Range rs[] = {
        rng("k", k, ntok * dk, es), rng("log_alpha", log_alpha, gate == GDR_GATE_CHANNEL ? ntok * dk : ntok, 4),
        rng("D", D, ntok * dv, 4), S_in == S_out ? Range{"S_in", 0, 0} : in_state, out_state,
    };
    s = check_ptrs(rs, 5, 4);
    if (s != GDR_OK) return s;
    const Range small[] = {rng("parent", parent, B * Td, 4), rng("accepted", accepted, B, 4)};
    for (const Range& r : small)
        if (overlap(out_state, r)) return fail(GDR_ERR_INVALID_ARG, "S_out overlaps %s", r.name);
    if (!aligned16(S_in)) return fail(GDR_ERR_INVALID_ARG, "S_in is not 16-byte aligned");
    gdr::TreeArgs a{nullptr, k, nullptr, log_alpha, nullptr, S_in, parent, nullptr, const_cast<float*>(D),
                    accepted, S_out, B, Td, H, dk, dv, io == GDR_BF16, gate == GDR_GATE_CHANNEL, stream};
    const hipError_t err = gdr::decode_tree_commit_launch(a);
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

gdr_status gdr_gdn2_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* erase, const float* write, const float* S0, void* o, float* S_T,
                        int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, gdr_dtype io,
                        gdr_gate gate, hipStream_t stream) {
    g_last_error[0] = 0;
    gdr_status s = check_common(B, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    if (T < 0) return fail(GDR_ERR_INVALID_ARG, "T must be >= 0 (T=%lld)", (long long)T);
    const int64_t ntok = mul({B, T, H});
    if (ntok < 0 || mul({ntok, dk}) < 0 || mul({B, H, dv, dk}) < 0 || mul({B, H, dv / 16}) > INT32_MAX)
        return fail(GDR_ERR_UNSUPPORTED, "tensor sizes overflow");
    if (T > 0 && (!q || !k || !v || !log_alpha || !erase || !write || !o))
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, log_alpha, erase, write and o must be non-NULL");
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const Range rs[] = {
        rng("q", q, ntok * dk, es),          rng("k", k, ntok * dk, es),
        rng("v", v, ntok * dv, es),
        rng("log_alpha", log_alpha, gate == GDR_GATE_CHANNEL ? ntok * dk : ntok, 4),
        rng("erase", erase, ntok * dk, 4),   rng("write", write, ntok * dv, 4),
        rng("S0", S0, B * H * dv * dk, 4),   rng("o", o, ntok * dv, es),
        rng("S_T", S_T, B * H * dv * dk, 4),
    };
    s = check_ptrs(rs, 9, 7);
    if (s != GDR_OK) return s;
    if (T == 0) {   // no tokens: S_T = S0 (zeros when S0 is NULL), same as gdr_chunk_fwd
        if (!S_T) return GDR_OK;
        gdr::ChunkArgs c{q, k, v, log_alpha, nullptr, S0, o, S_T, B, 0, H, dk, dv, 64,
                         io == GDR_BF16, gate == GDR_GATE_CHANNEL, nullptr, stream};
        const hipError_t err = gdr::chunk_fwd_launch(c);
        if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
        return GDR_OK;
    }
    gdr::Gdn2Args a{q, k, v, log_alpha, erase, write, S0, o, S_T, B, T, H, dk, dv,
                    io == GDR_BF16, gate == GDR_GATE_CHANNEL, stream};
    const hipError_t err = gdr::gdn2_fwd_launch(a);
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

gdr_status gdr_gdn2_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk,
                                             int64_t dv, int64_t chunk, gdr_dtype io, gdr_gate gate,
                                             size_t* bytes) {
    g_last_error[0] = 0;
    if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    gdr_status s = check_common(B, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    if (T < 0) return fail(GDR_ERR_INVALID_ARG, "T must be >= 0 (T=%lld)", (long long)T);
    if (chunk < 1) return fail(GDR_ERR_INVALID_ARG, "chunk must be positive");
    if (!gdr::gdn2_chunk_supported(dk, dv, chunk, io == GDR_BF16))
        return fail(GDR_ERR_UNSUPPORTED,
                    "the chunkwise form takes bf16 io and chunk 64 (chunk=%lld); gdr_gdn2_fwd takes the rest",
                    (long long)chunk);
    const int64_t units = mul({B, H, (T + chunk - 1) / chunk});
    if (units < 0 || units > INT32_MAX) return fail(GDR_ERR_UNSUPPORTED, "B*H*ceil(T/chunk) too large");
    *bytes = gdr::gdn2_chunk_workspace_bytes(B, T, H, dk);
    return GDR_OK;
}

gdr_status gdr_gdn2_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* erase, const float* write, const float* S0, void* o,
                              float* S_T, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              int64_t chunk, gdr_dtype io, gdr_gate gate, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    size_t need = 0;
    gdr_status s = gdr_gdn2_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate, &need);
    if (s != GDR_OK) return s;
    const int64_t ntok = mul({B, T, H});
    if (ntok < 0 || mul({ntok, dk}) < 0 || mul({B, H, dv, dk}) < 0 || mul({B, H, dv / 16}) > INT32_MAX)
        return fail(GDR_ERR_UNSUPPORTED, "tensor sizes overflow");
    if (mul({H, dv, 4, 64}) > INT32_MAX) return fail(GDR_ERR_UNSUPPORTED, "H too large");
    if (T > 0 && (!q || !k || !v || !log_alpha || !erase || !write || !o))
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, log_alpha, erase, write and o must be non-NULL");
    if (need > 0 && !workspace) return fail(GDR_ERR_INVALID_ARG, "workspace is NULL");
    if (workspace_bytes < need)
        return fail(GDR_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, need);
    const int64_t la_elems = gate == GDR_GATE_CHANNEL ? ntok * dk : ntok;
    const Range rs[] = {
        rng("q", q, ntok * dk, 2),           rng("k", k, ntok * dk, 2),
        rng("v", v, ntok * dv, 2),           rng("log_alpha", log_alpha, la_elems, 4),
        rng("erase", erase, ntok * dk, 4),   rng("write", write, ntok * dv, 4),
        rng("S0", S0, B * H * dv * dk, 4),   rng("o", o, ntok * dv, 2),
        rng("S_T", S_T, B * H * dv * dk, 4), rng("workspace", workspace, (int64_t)need, 1),
    };
    s = check_ptrs(rs, 10, 7);
    if (s != GDR_OK) return s;
    if (T == 0) {   // no tokens: S_T = S0 (zeros when S0 is NULL)
        if (!S_T) return GDR_OK;
        gdr::ChunkArgs c{q, k, v, log_alpha, nullptr, S0, o, S_T, B, 0, H, dk, dv, 64,
                         true, gate == GDR_GATE_CHANNEL, nullptr, stream};
        const hipError_t err = gdr::chunk_fwd_launch(c);
        if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
        return GDR_OK;
    }
    gdr::Gdn2Args a{q, k, v, log_alpha, erase, write, S0, o, S_T, B, T, H, dk, dv,
                    true, gate == GDR_GATE_CHANNEL, stream};
    const hipError_t err = gdr::gdn2_chunk_fwd_launch(a, workspace);
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

gdr_status gdr_fg2_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t dk,
                                            int64_t dv, int64_t chunk, gdr_dtype io, gdr_gate gate,
                                            size_t* bytes) {
    gdr_status s = gdr_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate, bytes);
    if (s != GDR_OK) return s;
    const int64_t groups = mul({B, T, H, (dk + dv) / 8});   // one prologue thread each
    if (groups < 0 || groups > (int64_t)UINT32_MAX - 256)
        return fail(GDR_ERR_UNSUPPORTED, "B*T*H too large for the rate prologue");
    *bytes = gdr::fg2_workspace_bytes(B, T, H, dk, dv, chunk, io == GDR_BF16, gate == GDR_GATE_CHANNEL);
    return GDR_OK;
}

gdr_status gdr_fg2_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta_k, const float* beta_v, const float* S0, void* o,
                             float* S_T, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             int64_t chunk, gdr_dtype io, gdr_gate gate, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    size_t need = 0;
    gdr_status s = gdr_fg2_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate, &need);
    if (s != GDR_OK) return s;
    const int64_t ntok = mul({B, T, H});
    if (ntok < 0 || mul({ntok, dk}) < 0 || mul({B, H, dv, dk}) < 0)
        return fail(GDR_ERR_UNSUPPORTED, "tensor sizes overflow");
    if (mul({B, H, dv / 16}) > INT32_MAX) return fail(GDR_ERR_UNSUPPORTED, "B*H too large");
    // The kernels address one chunk's rows with 32-bit byte offsets from the
    // chunk's first row (row stride at most H*d*4 bytes: fp32 rows, or the
    // per-channel decay).
    if (mul({chunk, H, dk > dv ? dk : dv, 4}) > INT32_MAX)
        return fail(GDR_ERR_UNSUPPORTED, "H too large (chunk*H*d*4 bytes must stay below 2^31)");
    if (T > 0 && (!q || !k || !v || !log_alpha || !beta_k || !o))
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, log_alpha, beta_k and o must be non-NULL");
    if (need > 0 && !workspace) return fail(GDR_ERR_INVALID_ARG, "workspace is NULL");
    if (workspace_bytes < need)
        return fail(GDR_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, need);
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const int64_t la_elems = gate == GDR_GATE_CHANNEL ? ntok * dk : ntok;
    const Range rs[] = {
        rng("q", q, ntok * dk, es),          rng("k", k, ntok * dk, es),
        rng("v", v, ntok * dv, es),          rng("log_alpha", log_alpha, la_elems, 4),
        rng("beta_k", beta_k, ntok * dk, 4), rng("beta_v", beta_v, ntok * dv, 4),
        rng("S0", S0, B * H * dv * dk, 4),   rng("o", o, ntok * dv, es),
        rng("S_T", S_T, B * H * dv * dk, 4), rng("workspace", workspace, (int64_t)need, 1),
    };
    s = check_ptrs(rs, 10, 7);
    if (s != GDR_OK) return s;
    gdr::ChunkArgs a{q, k, v, log_alpha, nullptr, S0, o, S_T, B, T, H, dk, dv, chunk,
                     io == GDR_BF16, gate == GDR_GATE_CHANNEL, workspace, stream};
    const hipError_t err = gdr::fg2_chunk_fwd_launch(a, beta_k, beta_v);
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

gdr_status gdr_fg2_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                               const float* beta_k, const float* beta_v, const float* S_in,
                               float* S_out, void* o, int64_t B, int64_t H, int64_t dk, int64_t dv,
                               gdr_dtype io, gdr_gate gate, hipStream_t stream) {
    g_last_error[0] = 0;
    gdr_status s = check_common(B, H, dk, dv, io, gate);
    if (s != GDR_OK) return s;
    const int64_t nst = mul({B, H, dv, dk});
    if (nst < 0 || mul({B, H, dv}) > ((int64_t)INT32_MAX) * 4)
        return fail(GDR_ERR_UNSUPPORTED, "state too large");
    if (!q || !k || !v || !log_alpha || !beta_k || !S_in || !S_out || !o)
        return fail(GDR_ERR_INVALID_ARG, "all pointers except beta_v must be non-NULL");
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const int64_t bh = B * H;
    const Range in_state = rng("S_in", S_in, nst, 4);
    const Range out_state = rng("S_out", S_out, nst, 4);
    if (S_in != S_out && overlap(in_state, out_state))
        return fail(GDR_ERR_INVALID_ARG, "S_out partially overlaps S_in");
    const Range rs[] = {
        rng("q", q, bh * dk, es), rng("k", k, bh * dk, es), rng("v", v, bh * dv, es),
        rng("log_alpha", log_alpha, gate == GDR_GATE_CHANNEL ? bh * dk : bh, 4),
        rng("beta_k", beta_k, bh * dk, 4), rng("beta_v", beta_v, bh * dv, 4),
        S_in == S_out ? Range{"S_in", 0, 0} : in_state,
        out_state, rng("o", o, bh * dv, es),
    };
    if (!aligned16(S_in)) return fail(GDR_ERR_INVALID_ARG, "S_in is not 16-byte aligned");
    s = check_ptrs(rs, 9, 7);
    if (s != GDR_OK) return s;
    gdr::DecodeArgs a{q, k, v, log_alpha, nullptr, S_in, S_out, o, B, H, dk, dv,
                      io == GDR_BF16, gate == GDR_GATE_CHANNEL, stream, beta_k, beta_v};
    const hipError_t err = gdr::decode_step_launch(a);
    if (err != hipSuccess) return fail(GDR_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

}  // extern "C"
