/*
 * gdr.h -- C ABI of the gated delta rule forward pass on MI355X (gfx950).
 *
 * The operation (per batch b and head h, tokens t = 0..T-1):
 *
 *   S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   o_t = S_t q_t                                   (read-out after the update)
 *
 * S is d_v x d_k (row = value channel, column = key channel), alpha_t =
 * exp(log_alpha_t) is one scalar per (t,h) for Gated DeltaNet or one value per
 * key channel for Kimi Delta Attention (KDA).  Sources on the pages:
 *  - "FG2-GDN" page, section 1: Gated DeltaNet's scalar decay alpha_t in (0,1),
 *    KDA's channel-wise decay Diag(alpha_t), scalar writing rate beta_t;
 *  - same page, section 3.6 (Chunkwise Parallel Training): the chunkwise WY /
 *    UT-transform algorithm that gdr_chunk_fwd implements (triangular solve for
 *    the UT factor, inter-chunk state propagation, intra-chunk causal product);
 *  - same page, section 5 ("Linear Attention as Recurrent Memory"): the state
 *    update / read-out family (the page's S is the transpose of the S here);
 *  - same page, "Limitations / Inference Challenges": a fixed-size d_k x d_v
 *    state per head that decoding carries and serving may roll back, which is
 *    why gdr_decode_step may write its new state out of place.
 *
 * Conventions shared by every call
 *  - All pointers are device pointers owned by the caller; the library never
 *    allocates, frees or retains them.  Work is enqueued asynchronously on
 *    `stream` (0 = the null stream); buffers must stay valid until it is done.
 *  - All tensors are dense, row-major and contiguous, with 16-byte aligned base
 *    addresses.
 *  - q, k, v and o are fp32 (GDR_F32) or bf16 (GDR_BF16, raw 16-bit words);
 *    log_alpha, beta and every state are always fp32.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error nothing is launched and the call returns a non-zero status.  Input
 *    values are not inspected: NaN and Inf propagate.
 *  - Supported shapes: d_k = d_v in {64, 128}; chunk in {16, 32, 64};
 *    B >= 1, H >= 1, T >= 0 (T = 0 copies S0 to S_T).
 *  - The functions keep no state between calls and are reentrant
 *    (gdr_chunk_fwd_noalloc aside: it shares one scratch array per GPU).
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_OK = 0,
    GDR_ERR_INVALID_ARG = 1, /* null / misaligned / overlapping pointer, bad size or enum */
    GDR_ERR_UNSUPPORTED = 2, /* valid request outside the supported shapes      */
    GDR_ERR_HIP = 3          /* the HIP runtime reported an error at launch     */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;               /* q, k, v, o */
typedef enum { GDR_GATE_SCALAR = 0, GDR_GATE_CHANNEL = 1 } gdr_gate; /* GDN / KDA  */

/*
 * Bytes of device workspace gdr_chunk_fwd needs for these sizes (written to
 * *bytes).  The workspace holds the per-chunk WY factors (UT factor T, the
 * masked intra-chunk product, decay-scaled keys and queries for the channel
 * gate); it is produced and consumed inside one gdr_chunk_fwd call.
 * Returns GDR_OK, or an error status for unsupported / invalid sizes.
 */
gdr_status gdr_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H,
                                        int64_t dk, int64_t dv, int64_t chunk,
                                        gdr_dtype io, gdr_gate gate, size_t *bytes);

/*
 * Whole-sequence (prefill) forward pass, chunkwise-parallel WY form
 * ("FG2-GDN" page, section 3.6).
 *
 *   q, k       [B, T, H, dk]   io dtype
 *   v          [B, T, H, dv]   io dtype
 *   log_alpha  [B, T, H]       fp32, natural log of the decay (GDR_GATE_SCALAR)
 *              [B, T, H, dk]   fp32, per key channel            (GDR_GATE_CHANNEL)
 *   beta       [B, T, H]       fp32 writing rate
 *   S0         [B, H, dv, dk]  fp32 initial state, or NULL for zeros
 *   o          [B, T, H, dv]   io dtype, written (must not overlap any input)
 *   S_T        [B, H, dv, dk]  fp32 final state, written; or NULL to skip
 *   chunk      chunk length C; changes speed only, never the result beyond
 *              rounding
 *   workspace  device buffer of at least gdr_chunk_fwd_workspace_size() bytes
 *              (NULL allowed when that size is 0); its contents on entry are
 *              ignored and on return are unspecified; concurrent calls need
 *              separate workspaces.
 * The final chunk may be partial; tokens beyond T are never read or written.
 *
 * Precision.  fp32 io computes in fp32 throughout (fp32 matrix-core products
 * and an fp32 triangular solve).  bf16 io multiplies bf16 operands on the
 * matrix cores with fp32 accumulation and keeps the state in fp32; its
 * triangular solve (bf16, scalar gate, chunk 64) runs partly in fp16, which
 * assumes |beta_r k_r.k_i| <= 1 within a chunk, i.e. keys of norm at most 1 and
 * beta in [0, 1] as the pages' models feed them (L2-normalised keys, sigmoid
 * rates).  Keys of larger norm belong on fp32 io.  Chunks whose keys nearly
 * repeat or cancel (an off-diagonal |beta_r k_r.k_i decay| above 1/2) apply the
 * UT factor as a bf16 hi/lo pair automatically.
 */
gdr_status gdr_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *beta, const float *S0,
                         void *o, float *S_T,
                         int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                         int64_t chunk, gdr_dtype io, gdr_gate gate,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gdr_chunk_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * arguments are gdr_chunk_fwd's without the workspace; the caller still owns
 * every input and output.  In place of the workspace the call uses a fixed
 * device array of GDR_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on, from the first call there until the process ends (its device
 * address is looked up on that first call, which therefore should not be made
 * inside a graph capture).  The call itself allocates and frees nothing.
 *  - A request whose gdr_chunk_fwd_workspace_size exceeds
 *    GDR_NOALLOC_SCRATCH_BYTES returns GDR_ERR_UNSUPPORTED before any launch.
 *    Calls that need no workspace (bf16, scalar gate, chunk 64) take any size.
 *  - Every call on one GPU shares that GPU's array: calls that overlap in time
 *    on one GPU (different streams, or different threads with no ordering)
 *    race and give undefined results.  Calls ordered on one stream are safe;
 *    each call writes every scratch byte it reads before reading it, so nothing
 *    carries over from the previous call.
 *  - Errors as in gdr_chunk_fwd, plus GDR_ERR_HIP if the array's address on
 *    the stream's device cannot be obtained.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

gdr_status gdr_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                 const float *log_alpha, const float *beta, const float *S0,
                                 void *o, float *S_T,
                                 int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                 int64_t chunk, gdr_dtype io, gdr_gate gate, hipStream_t stream);

/*
 * One recurrent decode step (one token per sequence), reading the fixed-size
 * state and writing the next one ("FG2-GDN" page, section 5 and "Limitations /
 * Inference Challenges").
 *
 *   q, k       [B, H, dk]       io dtype
 *   v          [B, H, dv]       io dtype
 *   log_alpha  [B, H] or [B, H, dk]  fp32 (scalar / channel gate)
 *   beta       [B, H]           fp32
 *   S_in       [B, H, dv, dk]   fp32 state before the token
 *   S_out      [B, H, dv, dk]   fp32 state after the token; may equal S_in
 *                               (in place) but must not partially overlap it
 *   o          [B, H, dv]       io dtype, written
 */
gdr_status gdr_decode_step(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const float *S_in, float *S_out, void *o,
                           int64_t B, int64_t H, int64_t dk, int64_t dv,
                           gdr_dtype io, gdr_gate gate, hipStream_t stream);

/*
 * The gate prologue, applied to raw projections inside the library ("FG2-GDN"
 * page, section 3.5: queries and keys are L2-normalised, the write rate is the
 * sigmoid of its projection, and the decay comes from KDA's gated-decay
 * transform of channel-wise projections).  `flags` is a bitwise OR of:
 *   GDR_PROLOGUE_L2NORM_QK       q and k are normalised per token and head,
 *                                x / sqrt(sum x^2 + 1e-6)
 *   GDR_PROLOGUE_BETA_SIGMOID    beta holds logits; the call uses 1 / (1 + e^-beta)
 *   GDR_PROLOGUE_DECAY_SOFTPLUS  log_alpha holds decay logits x (per token and
 *                                head, or per key channel); the call uses
 *                                log alpha = -softplus(x) = -ln(1 + e^x), i.e.
 *                                alpha = 1 / (1 + e^x) in (0, 1).  The page does
 *                                not print the transform; the NVFP4 abstract on
 *                                the "Daily Papers" DeltaNet search page (its
 *                                finding ii) names softplus / exponential
 *                                parameterisations of the decay gate, and this is
 *                                the plainest map of that kind into (0, 1).
 * Arguments are otherwise those of gdr_chunk_fwd / gdr_decode_step, with q, k,
 * beta and log_alpha holding the raw values the flags name.  The bf16 prefill
 * calls with chunk 64 and the scalar gate, and every bf16 call with the channel
 * gate, fold the maps into their own loads.  The other prefill calls (fp32 io;
 * bf16 with the scalar gate at chunks 16 and 32) first run an elementwise pass
 * that writes the mapped q, k (io dtype), beta and log alpha into the workspace,
 * whose size for any flags comes from gdr_chunk_fwd_prologue_workspace_size.
 * The decode step maps inside its kernel for every dtype and gate.  flags = 0
 * is exactly gdr_chunk_fwd / gdr_decode_step; unknown bits return
 * GDR_ERR_INVALID_ARG.
 */
enum { GDR_PROLOGUE_L2NORM_QK = 1, GDR_PROLOGUE_BETA_SIGMOID = 2, GDR_PROLOGUE_DECAY_SOFTPLUS = 4 };

gdr_status gdr_chunk_fwd_prologue_workspace_size(int64_t B, int64_t T, int64_t H,
                                                 int64_t dk, int64_t dv, int64_t chunk,
                                                 gdr_dtype io, gdr_gate gate, unsigned flags,
                                                 size_t *bytes);

gdr_status gdr_chunk_fwd_prologue(const void *q, const void *k, const void *v,
                                  const float *log_alpha, const float *beta, const float *S0,
                                  void *o, float *S_T,
                                  int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                  int64_t chunk, gdr_dtype io, gdr_gate gate,
                                  void *workspace, size_t workspace_bytes, unsigned flags,
                                  hipStream_t stream);

gdr_status gdr_decode_step_prologue(const void *q, const void *k, const void *v,
                                    const float *log_alpha, const float *beta,
                                    const float *S_in, float *S_out, void *o,
                                    int64_t B, int64_t H, int64_t dk, int64_t dv,
                                    gdr_dtype io, gdr_gate gate, unsigned flags,
                                    hipStream_t stream);

/*
 * Several tokens per sequence in one pass over the state: verifying a run of
 * draft tokens in speculative decoding, then keeping the state of the accepted
 * prefix (the pages name both the per-token rollback of the recurrent state
 * and its fixed d_k x d_v size as the serving problem: "FG2-GDN" page,
 * "Limitations / Inference Challenges").  Tokens t = 0..Td-1 of each sequence
 * are applied to S_in in order, exactly as Td calls of gdr_decode_step would:
 *
 *   q, k       [B, Td, H, dk]   io dtype
 *   v          [B, Td, H, dv]   io dtype
 *   log_alpha  [B, Td, H] or [B, Td, H, dk]   fp32 (scalar / channel gate)
 *   beta       [B, Td, H]       fp32
 *   S_in       [B, H, dv, dk]   fp32 state before the first token; only read
 *                               (unless S_out == S_in)
 *   S_out      [B, H, dv, dk]   fp32, receives the state after the first n_b
 *                               tokens of sequence b; may equal S_in (in place),
 *                               must not partially overlap it; NULL writes no
 *                               state (a read-only verification pass)
 *   accepted   [B] int32 device array of n_b, each clamped to [0, Td]; NULL
 *              means n_b = Td for every sequence.  4-byte aligned.
 *   o          [B, Td, H, dv]   io dtype, o_t for every token; NULL skips them
 * 1 <= Td <= 64 (longer runs belong to gdr_chunk_fwd).  The state is read once
 * and written at most once, so the call costs about one decode step of HBM
 * traffic whatever Td is.  A typical round: gdr_decode_multi(S_in, S_out=NULL,
 * o) to score the drafts, then gdr_decode_multi(S_in, S_out, accepted, o=NULL)
 * to commit the accepted prefix.
 */
gdr_status gdr_decode_multi(const void *q, const void *k, const void *v,
                            const float *log_alpha, const float *beta,
                            const float *S_in, float *S_out, const int32_t *accepted, void *o,
                            int64_t B, int64_t Td, int64_t H, int64_t dk, int64_t dv,
                            gdr_dtype io, gdr_gate gate, hipStream_t stream);

/*
 * Draft trees: verify every node of a tree of draft tokens in one pass over the
 * committed state, then rebuild the state of the accepted node (the TreeWY
 * note on the mindpattern "Gated DeltaNet-2" page: one tree-structured WY
 * transform yields every node's output, and the accepted state is rebuilt on
 * commit from a small matrix of pseudo-values, with no per-node state
 * snapshots).  Node i of sequence b follows parent[b][i]: an earlier node, or
 * -1 for a child of the committed state.  Its state is the delta rule applied
 * along its root path, one token per node, and o_i = S_i q_i; a chain of
 * parents i - 1 is exactly gdr_decode_multi.
 *
 * gdr_decode_tree:
 *   q, k       [B, Td, H, dk]   io dtype, one token per node
 *   v          [B, Td, H, dv]   io dtype
 *   log_alpha  [B, Td, H] or [B, Td, H, dk]   fp32 (scalar / channel gate)
 *   beta       [B, Td, H]       fp32
 *   S_in       [B, H, dv, dk]   fp32 committed state, only read
 *   parent     [B, Td]          int32 device array, 4-byte aligned; an entry
 *                               that is neither -1 nor an earlier node is read
 *                               as -1 (values are not otherwise inspected)
 *   o          [B, Td, H, dv]   io dtype, every node's output; or NULL
 *   D          [B, Td, H, dv]   fp32, every node's written value
 *                               u_i = beta_i (v_i - S_parent Diag(alpha_i) k_i),
 *                               the pseudo-values the commit needs; or NULL
 * gdr_decode_tree_commit: S_out = the state after node accepted[b] (an int32
 * device array [B], 4-byte aligned; -1 or any value outside [0, Td) keeps
 * S_in), from S_in, the keys, decays and parents of the accepted node's path
 * and D from gdr_decode_tree.  S_out may equal S_in (in place) but must not
 * partially overlap it.
 * 1 <= Td <= 64.  The verify pass reads the state once and costs about one
 * decode step of HBM traffic plus O(Td^2 d) work per (b, h); the commit reads
 * and writes the state once.  Errors as in gdr_decode_multi.
 */
gdr_status gdr_decode_tree(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta, const float *S_in,
                           const int32_t *parent, void *o, float *D,
                           int64_t B, int64_t Td, int64_t H, int64_t dk, int64_t dv,
                           gdr_dtype io, gdr_gate gate, hipStream_t stream);

gdr_status gdr_decode_tree_commit(const void *k, const float *log_alpha, const int32_t *parent,
                                  const float *D, const int32_t *accepted,
                                  const float *S_in, float *S_out,
                                  int64_t B, int64_t Td, int64_t H, int64_t dk, int64_t dv,
                                  gdr_dtype io, gdr_gate gate, hipStream_t stream);

/*
 * Channel-wise write rates: FG2-GDN and FG2-GDN+ ("FG2-GDN" page, sections 3.2,
 * 3.4-3.6).  The scalar beta_t becomes a vector beta^k_t in R^{d_k} that enters
 * through the scaled key k~ = sqrt(beta^k) * k (elementwise); the value is
 * scaled the same way, v~ = sqrt(beta^v) * v, with beta^v = beta^k for FG2-GDN
 * and a separate d_v-vector for FG2-GDN+.  The update is the tied delta rule
 * with unit rate on the scaled vectors,
 *
 *   S_t = S_{t-1} Diag(alpha_t) (I - k~_t k~_t^T) + v~_t k~_t^T,   o_t = S_t q_t,
 *
 * which is KDA (Gated DeltaNet with a scalar decay) when every channel has the
 * same rate.  The page prints neither equation; this is the reading that keeps
 * its stated properties (tied diagonal-plus-rank-1 transition, elementwise
 * square roots and scalings, the chunkwise algorithm unchanged).
 *
 *   beta_k     [B, T, H, dk]   fp32 key-side rates     ([B, H, dk] for decode)
 *   beta_v     [B, T, H, dv]   fp32 value-side rates, or NULL for beta_k
 *                              ([B, H, dv] for decode)
 * Everything else is as in gdr_chunk_fwd / gdr_decode_step (log_alpha may be
 * scalar or channel-wise, selected by `gate`).  The prefill workspace also
 * holds the scaled k and v of the whole call, so it is larger than
 * gdr_chunk_fwd's; its size comes from gdr_fg2_chunk_fwd_workspace_size.
 */
gdr_status gdr_fg2_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H,
                                            int64_t dk, int64_t dv, int64_t chunk,
                                            gdr_dtype io, gdr_gate gate, size_t *bytes);

gdr_status gdr_fg2_chunk_fwd(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta_k, const float *beta_v,
                             const float *S0, void *o, float *S_T,
                             int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             int64_t chunk, gdr_dtype io, gdr_gate gate,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

gdr_status gdr_fg2_decode_step(const void *q, const void *k, const void *v,
                               const float *log_alpha, const float *beta_k, const float *beta_v,
                               const float *S_in, float *S_out, void *o,
                               int64_t B, int64_t H, int64_t dk, int64_t dv,
                               gdr_dtype io, gdr_gate gate, hipStream_t stream);

/*
 * Decoupled erase and write gates: Gated DeltaNet-2 ("Daily Papers" pages, the
 * Gated DeltaNet-2 abstract and citation notes).  A channel-wise erase gate
 * b_t in R^{d_k} (key side) and a channel-wise write gate w_t in R^{d_v} (value
 * side) replace the tied scalar beta_t:
 *
 *   S_t = S_{t-1} Diag(alpha_t) (I - k_t (b_t * k_t)^T) + (w_t * v_t) k_t^T,
 *   o_t = S_t q_t
 *
 * (read the decayed memory at k, erase the read along b*k, write w*v along k).
 * The pages give no equation; this reading keeps what they state, including
 * KDA / Gated DeltaNet when b_t and w_t collapse to the same scalar.
 *
 *   erase      [B, T, H, dk]   fp32 b_t
 *   write      [B, T, H, dv]   fp32 w_t
 * The other arguments are as in gdr_chunk_fwd (no chunk, no workspace).  This
 * implementation is a token-sequential scan with the state in registers (one
 * pass over the state; time linear in T per sequence).
 */
gdr_status gdr_gdn2_fwd(const void *q, const void *k, const void *v,
                        const float *log_alpha, const float *erase, const float *write,
                        const float *S0, void *o, float *S_T,
                        int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                        gdr_dtype io, gdr_gate gate, hipStream_t stream);

/*
 * The same recurrence in chunkwise form (the organisation of the "FG2-GDN"
 * page, section 3.6, carried over to the decoupled gates): per chunk of 64
 * tokens, the reads of the chunk come from a unit-lower triangular solve
 * against the erase directions, and everything that involves neither the
 * state nor v is folded into per-chunk operands that a sequential pass over
 * the chunks then applies on the matrix cores.  The result is the token
 * recurrence above, reorganised with no approximation.
 *
 * Arguments as in gdr_gdn2_fwd, plus chunk and a caller-owned device
 * workspace of gdr_gdn2_chunk_fwd_workspace_size bytes (72.5 KiB per
 * 64-token chunk and head at dk = 128; no contents kept between calls).
 * Supported: io = GDR_BF16, chunk = 64, dk = dv in {64, 128}; anything else
 * returns GDR_ERR_UNSUPPORTED (gdr_gdn2_fwd takes those).  The preparation
 * works in fp16 on matrix-core products whose entries stay small for keys of
 * unit norm and gates in [0, 1]; keys of much larger norm should use
 * gdr_gdn2_fwd.  Errors as in gdr_chunk_fwd.
 */
gdr_status gdr_gdn2_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H,
                                             int64_t dk, int64_t dv, int64_t chunk,
                                             gdr_dtype io, gdr_gate gate, size_t *bytes);

gdr_status gdr_gdn2_chunk_fwd(const void *q, const void *k, const void *v,
                              const float *log_alpha, const float *erase, const float *write,
                              const float *S0, void *o, float *S_T,
                              int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              int64_t chunk, gdr_dtype io, gdr_gate gate,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char *gdr_status_string(gdr_status s);

/* Details of the last error reported on the calling thread ("" if none). */
const char *gdr_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GDR_H */
