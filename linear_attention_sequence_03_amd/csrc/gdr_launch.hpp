// gdr_launch.hpp -- internal interface between the C ABI (argument checking)
// and the kernel launchers.  Arguments reaching these functions are validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

struct DecodeArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *S_in;
    float* S_out;
    void* o;
    int64_t B, H, dk, dv;
    bool bf16, channel;
    hipStream_t stream;
    // Channel-wise write rates (beta unused then): beta_k [B,H,dk], beta_v
    // [B,H,dv] or NULL for beta_k.  NULL beta_k selects the scalar rate.
    const float *beta_k = nullptr, *beta_v = nullptr;
    unsigned prologue = 0;   // gate prologue flags (scalar-rate step only)
};

// Several tokens per sequence in one pass over the state (draft verification
// and accepted-prefix commit).
struct DecodeMultiArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *S_in;
    float* S_out;               // NULL: no state written
    const int32_t* accepted;    // [B] or NULL (= Td)
    void* o;                    // NULL: no outputs written
    int64_t B, Td, H, dk, dv;
    bool bf16, channel;
    hipStream_t stream;
};

// Gate prologue flags (in-kernel L2 normalisation of q and k, beta and the
// log decay from their logits).
constexpr unsigned kPrologueL2NormQK = 1u, kPrologueBetaSigmoid = 2u, kPrologueDecaySoftplus = 4u;
constexpr unsigned kPrologueGates = kPrologueBetaSigmoid | kPrologueDecaySoftplus;

struct ChunkArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *S0;
    void* o;
    float* S_T;
    int64_t B, T, H, dk, dv, chunk;
    bool bf16, channel;
    void* ws;
    hipStream_t stream;
    unsigned prologue = 0;   // kPrologue* flags (fused into the loads, or a staging pass first)
};

hipError_t decode_step_launch(const DecodeArgs& a);
hipError_t decode_multi_launch(const DecodeMultiArgs& a);

// Draft trees (verify every node; rebuild the accepted node's state).
struct TreeArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *S_in;
    const int32_t* parent;      // [B, Td]
    void* o;                    // verify: outputs, or NULL
    float* D;                   // verify: written values (out); commit: in
    const int32_t* accepted;    // commit: [B]
    float* S_out;               // commit
    int64_t B, Td, H, dk, dv;
    bool bf16, channel;
    hipStream_t stream;
};
hipError_t decode_tree_launch(const TreeArgs& a);
hipError_t decode_tree_commit_launch(const TreeArgs& a);
size_t tree_verify_lds_bytes(int64_t Td, int64_t dk);

// Workspace bytes of one (b, h, chunk) block and of the whole call.
size_t chunk_block_bytes(int64_t dk, int64_t chunk, bool bf16, bool channel);
size_t chunk_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t chunk,
                             bool bf16, bool channel);
hipError_t chunk_fwd_launch(const ChunkArgs& a);
// Device address of the fixed scratch array (GDR_NOALLOC_SCRATCH_BYTES) on the
// device of `stream`; looked up on the first call per device, then cached.
hipError_t noalloc_scratch(hipStream_t stream, void** out);
// Which chunk calls fuse the gate prologue into their loads; the others run
// it as a separate pass into the workspace, which grows by
// prologue_stage_bytes then.
bool prologue_fused(int64_t chunk, bool bf16, bool channel);
size_t prologue_stage_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, bool bf16, bool channel,
                            unsigned flags);
size_t chunk_prologue_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t chunk,
                                      bool bf16, bool channel, unsigned flags);

// Single-kernel path (bf16, scalar gate, 64-token chunks): needs no workspace.
bool fused_chunk_supported(int64_t dk, int64_t chunk, bool bf16, bool channel);
hipError_t fused_chunk_launch(const ChunkArgs& a);

// Channel-wise write rates: a prologue scales k and v into the workspace, then
// the chunk path above runs with unit rate.
size_t fg2_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                           bool bf16, bool channel);
hipError_t fg2_chunk_fwd_launch(const ChunkArgs& a, const float* beta_k, const float* beta_v);

// Decoupled erase / write gates (token-sequential scan).
struct Gdn2Args {
    const void *q, *k, *v;
    const float *log_alpha, *erase, *write, *S0;
    void* o;
    float* S_T;
    int64_t B, T, H, dk, dv;
    bool bf16, channel;
    hipStream_t stream;
};
hipError_t gdn2_fwd_launch(const Gdn2Args& a);

// Chunkwise form of the same recurrence (bf16 io, 64-token chunks, dk = dv in
// {64, 128}): a per-chunk preparation into the workspace, then the sequential
// pass.  T > 0.
bool gdn2_chunk_supported(int64_t dk, int64_t dv, int64_t chunk, bool bf16);
size_t gdn2_chunk_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk);
hipError_t gdn2_chunk_fwd_launch(const Gdn2Args& a, void* ws);

}  // namespace gdr
