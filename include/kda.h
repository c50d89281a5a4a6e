/* kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention operator.
 *
 * The operator is the channel-gated delta rule of "Understanding Kimi Delta
 * Attention" (section "The KDA Recurrence: Scalar Gate vs Channel-wise
 * Gate") and "kimi delta attn from first principles" (sections "KDA" and
 * "three gates"): for every chain (one sequence, one head) a state S of
 * d_k x d_v fp32 values, rows indexed by key channels, evolves per token as
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * i.e. decay each row by its own gate, take the delta-rule error against the
 * decayed state, write rank 1, and read the updated state with the query.
 * g is the log forget gate (alpha = exp(g), expected <= 0); beta is the
 * update gate; q and k are used exactly as given (the layer normalises them
 * upstream); `scale` multiplies the read-out (typically 1/sqrt(d_k)).
 *
 * Two modes, as on the first page ("Two execution modes"): chunked prefill
 * over whole sequences (kda_chunk_fwd) and a single-token step that updates
 * the state in place (kda_decode_step).  The caller chooses the mode.
 *
 * Conventions for every entry point:
 *  - every tensor pointer is a device pointer owned by the caller, except
 *    arguments whose name ends in _host; nothing is retained after return;
 *  - tensors are dense, row-major, in the shapes given below (innermost last);
 *  - all work is enqueued on `stream` (a hipStream_t; NULL is the default
 *    stream) and is asynchronous; outputs are valid after the stream is
 *    synchronised;
 *  - arguments are validated on the host before anything is enqueued; on an
 *    error a status is returned, nothing is launched and no output is
 *    written.  Device-side faults surface at the caller's next sync, as
 *    usual in HIP.  Non-finite inputs propagate; they are not checked;
 *  - supported head sizes: d_k, d_v in {16, 32, 64, 128}; q/k/v in fp32 or
 *    bf16; g, beta, states in fp32; o in fp32 or bf16;
 *  - pointers to fp32/bf16 tensors must be 16-byte aligned; beta and
 *    cu_seqlens 4-byte aligned;
 *  - the library allocates no device memory; scratch comes from the
 *    caller's workspace.
 *  - No C++ exception crosses this interface.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,       /* a size is negative or inconsistent */
    KDA_ERR_DTYPE = 3,       /* unknown dtype code */
    KDA_ERR_UNSUPPORTED = 4, /* valid but not supported (head size, variant) */
    KDA_ERR_SEQLENS = 5,     /* cu_seqlens_host not 0 = c0 <= c1 <= ... <= cN = T */
    KDA_ERR_ALIAS = 6,       /* an output overlaps an input or another output */
    KDA_ERR_ALIGN = 7,       /* a pointer is not aligned as required */
    KDA_ERR_WORKSPACE = 8,   /* workspace NULL or smaller than required */
    KDA_ERR_HIP = 9          /* a HIP launch or copy failed */
} kda_status;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Prefill implementations.  AUTO picks the fastest one that supports the
 * arguments; the others exist to compare paths against each other.
 *  RECURRENT  token-sequential fused recurrent kernel, any supported shape;
 *  CHUNK      chunkwise kernel on fp16 MFMA, 32-token chunks, one workgroup
 *             of 12 waves per (sequence, head): 8 waves prepare the next
 *             chunk's gate-side operands while 4 run the state pass (bf16
 *             inputs, d_k = d_v = 128);
 *  CHUNK_SCAN CHUNK on segments of long sequences: each segment's affine
 *             state map is computed in parallel, composed by a scan, and the
 *             segments then run in parallel from their initial states (same
 *             inputs as CHUNK).  AUTO takes it when the longest sequence
 *             would otherwise dominate the run time.
 *  CHUNK64    chunkwise kernel on 64-token chunks (four 16-token
 *             sub-blocks), 8 waves per (sequence, head) doing the gate-side
 *             and then the state work of each chunk; same inputs as CHUNK.
 *             Never chosen by AUTO.
 *  CHUNK8     chunkwise kernel in fp32 arithmetic throughout (fp32 MFMA,
 *             8-token sub-chunks), workgroups of state, gate and solve waves
 *             pipelined over sub-chunks, one or more per (sequence, head)
 *             by state columns; any supported head size, fp32 or bf16
 *             inputs, results within fp32 rounding of the token-by-token
 *             recurrence.  AUTO takes it for the arguments CHUNK does not
 *             support (fp32 inputs, d_k or d_v other than 128). */
typedef enum kda_variant {
    KDA_VARIANT_AUTO = 0,
    KDA_VARIANT_RECURRENT = 1,
    KDA_VARIANT_CHUNK = 2,
    KDA_VARIANT_CHUNK_SCAN = 3,
    KDA_VARIANT_CHUNK64 = 4,
    KDA_VARIANT_CHUNK8 = 5
} kda_variant;

/* ABI version (KDA_ABI_VERSION of the built library). */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* kda_status_str(kda_status status);

/* Bytes of device workspace kda_chunk_fwd needs for these sizes, sequence
 * lengths and variant (0 is a valid answer).  N is the number of sequences
 * (B, or the length of cu_seqlens minus one); cu_seqlens_host is the host
 * copy of cu_seqlens or NULL, exactly as later passed to kda_chunk_fwd.
 * RECURRENT needs none; every chunked variant (AUTO included, for any
 * dtype and head size) needs at least a list of one small item per
 * sequence, CHUNK_SCAN also room for the segment maps.  Returns 0 for
 * arguments kda_chunk_fwd would reject. */
size_t kda_chunk_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                    int32_t N, const int32_t* cu_seqlens_host, kda_dtype in_dtype,
                                    kda_variant variant);

/* Chunked prefill over N independent sequences ("Understanding Kimi Delta
 * Attention", section "The Chunkwise DPLR Algorithm": chunks of the
 * sequence, results equal to the sequential recurrence).
 *
 *  q, k        [B, T, H, d_k]  in_dtype
 *  v           [B, T, H, d_v]  in_dtype
 *  g           [B, T, H, d_k]  fp32, log forget gate
 *  beta        [B, T, H]       fp32, update gate
 *  scale       read-out scale
 *  initial_state [N, H, d_k, d_v] fp32, or NULL for zero states
 *  cu_seqlens  [N+1] int32 device, or NULL: then N must equal B and row b of
 *              the batch is sequence b.  With cu_seqlens B must be 1 and
 *              sequence n is tokens cu[n] .. cu[n+1]-1 of the packed axis.
 *  cu_seqlens_host  host copy of cu_seqlens (required with it; validated:
 *              cu[0] = 0, non-decreasing, cu[N] = T).  Empty sequences are
 *              allowed (their final state is the initial state).
 *  o           [B, T, H, d_v] out_dtype (written for every token)
 *  final_state [N, H, d_k, d_v] fp32, or NULL to skip; may be the same
 *              pointer as initial_state (in-place update); no other overlap
 *              between outputs and inputs is allowed.
 *  workspace   device scratch of at least kda_chunk_fwd_workspace_size()
 *              bytes (may be NULL when that is 0), 256-byte aligned; its
 *              contents on entry do not matter and are overwritten.
 * Every variant accepts any g <= 0 with |g| < 1e38, down to full
 * forgetting.  The chunked variants may treat a log-gate below -100 as -100
 * (alpha = e^-100, about 4e-44, is zero next to any fp32 state value); for
 * alpha = 0 pass a large negative value rather than -inf.  g > 0 (a gate
 * above one) is accepted without a range guarantee.
 * T = 0 or N = 0 is a successful no-op. */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, const float* initial_state,
                         const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                         int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t N,
                         kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* final_state,
                         void* workspace, size_t workspace_bytes, kda_variant variant,
                         void* stream);

/* kda_chunk_fwd whose output is the layer's gated, normalised read-out
 * ("kimi delta attn from first principles", section "three gates": RMSNorm
 * is applied to o_t = S_t^T q_t, then multiplied elementwise by the output
 * gate): for every token and head, with o the read-out of kda_chunk_fwd,
 *
 *     o <- out_gate * norm_weight * o / sqrt(mean_j(o_j^2) + norm_eps)
 *
 * the mean over the d_v channels of that token and head.
 *  out_gate    [B, T, H, d_v] in_dtype, the gate values as they multiply (the
 *              caller applies the gate's activation); an input.
 *  norm_weight [d_v] fp32, shared by all heads; an input.
 *  norm_eps    >= 0 and finite (else KDA_ERR_SHAPE).
 * The 12-wave chunk kernel (CHUNK, CHUNK_SCAN) applies this in its o store;
 * RECURRENT, CHUNK64 and CHUNK8 write o and then rewrite it in place.  The
 * workspace is that of kda_chunk_fwd_workspace_size(); every other argument
 * and error behaviour is that of kda_chunk_fwd. */
kda_status kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* g,
                               const float* beta, float scale, const float* initial_state,
                               const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                               int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                               int32_t N, kda_dtype in_dtype, kda_dtype out_dtype,
                               const void* out_gate, const float* norm_weight, float norm_eps,
                               void* o, float* final_state, void* workspace,
                               size_t workspace_bytes, kda_variant variant, void* stream);

/* The gate inputs of kda_chunk_fwd from their projections ("kimi delta attn
 * from first principles", section "three gates": the forget gate alpha comes
 * from a low-rank projection -- down to rank r, then up to the key channels
 * -- and the update gate beta is the sigmoid of its projection):
 *
 *     g[m, h, c] = -softplus(sum_j z[m, j] w_up[h d_k + c, j] + b_up[h d_k + c])
 *     beta[m, h] = 1 / (1 + exp(-u[m, h]))
 *
 * so that alpha = exp(g) lies in (0, 1).  The pages give the projection's
 * structure but not the activation that makes it a log-decay; -softplus is
 * this library's choice (documented as such).  m runs over the M tokens of
 * the batch (B T, or the packed tokens).
 *  z       [M, r] bf16, the down-projected activations (r in {32, 64, 128, 256})
 *  w_up    [H d_k, r] bf16 (a linear layer's weight: one row per output
 *          channel, d_k = 128)
 *  b_up    [H d_k] fp32 or NULL (no bias); 16-byte aligned
 *  u       [M, H] fp32, the beta projection
 *  g       [M, H, d_k] fp32, written (the layout kda_chunk_fwd reads)
 *  beta    [M, H] fp32, written
 * Only in_dtype = KDA_BF16 with d_k = 128 is supported (else
 * KDA_ERR_UNSUPPORTED); H above 65535 returns KDA_ERR_SHAPE.  g and beta
 * must not overlap the inputs or each other.  M = 0 or H = 0 is a
 * successful no-op. */
kda_status kda_fused_gate(const void* z, const void* w_up, const float* b_up, const float* u,
                          int32_t M, int32_t r, int32_t H, int32_t d_k, kda_dtype in_dtype,
                          float* g, float* beta, void* stream);

/* Largest workspace kda_chunk_fwd_noalloc can provide (32 MiB per GPU). */
#define KDA_CHUNK_FWD_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)

/* kda_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * It takes no workspace: the workspace is a device array of
 * KDA_CHUNK_FWD_NOALLOC_MAX_WORKSPACE bytes built into the library, one per
 * GPU, held until the process ends.  The call itself allocates nothing.
 * Every argument, output and error behaviour is that of kda_chunk_fwd, plus:
 *  - if the workspace kda_chunk_fwd_workspace_size() gives for these
 *    arguments exceeds the maximum, AUTO falls back to KDA_VARIANT_CHUNK
 *    (one work item per sequence) when that fits; otherwise the call returns
 *    KDA_ERR_WORKSPACE and launches nothing;
 *  - all calls on one GPU share its array (its contents on entry do not
 *    matter): calls that overlap on one GPU, from two streams or two host
 *    threads, race and must be serialised by the caller;
 *  - the first call on a device resolves that device's array address
 *    (hipGetSymbolAddress) with the current device; the stream must belong
 *    to the current device. */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, float scale, const float* initial_state,
                                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                 int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                 int32_t N, kda_dtype in_dtype, kda_dtype out_dtype, void* o,
                                 float* final_state, kda_variant variant, void* stream);

/* Bytes of device workspace kda_chunk_fwd_snapshots needs (the same
 * arguments as kda_chunk_fwd_workspace_size plus the snapshot interval);
 * 0 for arguments it would reject. */
size_t kda_chunk_fwd_snapshots_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k,
                                              int32_t d_v, int32_t N,
                                              const int32_t* cu_seqlens_host, kda_dtype in_dtype,
                                              kda_variant variant, int32_t snap_interval);

/* kda_chunk_fwd that also writes the state of every sequence after each
 * `snap_interval` tokens: states kept at prefix boundaries so that a later
 * request sharing the prefix can resume from them (the concept page "Kimi
 * Delta Attention (KDA)", section "KV Caching Challenges & vLLM
 * Contribution": a KDA-aware prefix cache keeps the recurrent state at
 * prefix boundaries rather than keys and values).  Resuming is a call with
 * the snapshot as initial_state on the remaining tokens.
 *
 *  snap_interval  tokens between snapshots, a positive multiple of 64 (other
 *              values: KDA_ERR_SHAPE if <= 0, else KDA_ERR_UNSUPPORTED).
 *  snapshots   [total, H, d_k, d_v] fp32, where sequence n of length L_n
 *              contributes floor(L_n / snap_interval) snapshots, stored in
 *              sequence order and, within a sequence, in position order:
 *              snapshot j of sequence n is row sum_{m<n} floor(L_m /
 *              snap_interval) + j and holds the state after tokens
 *              0 .. (j + 1) snap_interval - 1 of that sequence.  May be NULL
 *              when total is 0; must not overlap any other argument.
 *  workspace   at least kda_chunk_fwd_snapshots_workspace_size() bytes.
 * Every other argument, the outputs o and final_state, and all error
 * behaviour are those of kda_chunk_fwd. */
kda_status kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, float scale, const float* initial_state,
                                   const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                   int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                   int32_t N, kda_dtype in_dtype, kda_dtype out_dtype, void* o,
                                   float* final_state, int32_t snap_interval, float* snapshots,
                                   void* workspace, size_t workspace_bytes, kda_variant variant,
                                   void* stream);

/* One token for each of N independent sequences, state updated in place
 * ("Understanding Kimi Delta Attention", section "Two execution modes":
 * the fused recurrent step with constant memory; the recurrence of section
 * "The KDA Recurrence").
 *
 *  q, k        [N, H, d_k]  in_dtype
 *  v           [N, H, d_v]  in_dtype
 *  g           [N, H, d_k]  fp32
 *  beta        [N, H]       fp32
 *  scale       read-out scale (the same convention as kda_chunk_fwd)
 *  state       [N, H, d_k, d_v] fp32, read and overwritten with S_t
 *  o           [N, H, d_v] out_dtype; must not overlap any input or state.
 * N = 0 is a successful no-op. */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float scale, float* state, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, kda_dtype in_dtype, kda_dtype out_dtype,
                           void* o, void* stream);

/* Longest run kda_fused_recurrent_fwd accepts. */
#define KDA_FUSED_RECURRENT_MAX_T 64

/* T consecutive tokens for each of N independent sequences, state updated in
 * place: the fused recurrent mode of "Understanding Kimi Delta Attention"
 * (section "Two execution modes": token by token with the state resident)
 * over a short run, as when a draft of several tokens is verified or a short
 * prompt is appended to a cached state.  The result equals T calls of
 * kda_decode_step, one per token in order, but the state is read and
 * written once for the whole run.
 *
 *  q, k        [N, T, H, d_k]  in_dtype
 *  v           [N, T, H, d_v]  in_dtype
 *  g           [N, T, H, d_k]  fp32, log forget gate
 *  beta        [N, T, H]       fp32
 *  scale       read-out scale
 *  state       [N, H, d_k, d_v] fp32, read and overwritten with the state
 *              after token T-1
 *  o           [N, T, H, d_v]  out_dtype, written for every token; must not
 *              overlap any input or the state.
 * 0 <= T <= KDA_FUSED_RECURRENT_MAX_T (longer runs return
 * KDA_ERR_UNSUPPORTED: kda_chunk_fwd is the path for them).  N = 0, H = 0 or
 * T = 0 is a successful no-op.  Arithmetic is fp32 throughout: with
 * d_k = d_v = 128 the run is taken 8 tokens at a time in the chunk form of
 * the same section on fp32 matrix cores, otherwise token by token, and the
 * results agree with kda_decode_step to fp32 rounding.  Speed: the state is
 * read and written once, but every 8 tokens cost a pass of fp32 products over
 * it, so for bf16 inputs with d_k = d_v = 128 and runs of about 24 tokens or
 * more, kda_chunk_fwd (B = N, no cu_seqlens, initial_state = final_state =
 * the state) is faster, within the bf16 tolerance rather than fp32 agreement
 * with kda_decode_step. */
kda_status kda_fused_recurrent_fwd(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, float scale, float* state, int32_t N,
                                   int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                   kda_dtype in_dtype, kda_dtype out_dtype, void* o,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
