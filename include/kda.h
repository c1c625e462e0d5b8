/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) KDA token mixer.
 *
 * KDA (Kimi Delta Attention) keeps, per batch row b and head h, a fixed-size
 * memory S (d_k x d_v, fp32, row = key channel).  Token t updates and reads it:
 *
 *   lambda = max(log_alpha_t, log_alpha_min)            per key channel
 *   S     <- diag(exp(lambda)) S                        channel-wise retention
 *   kh, qh = k_t / |k_t|, q_t / |q_t|                   (|x| floored at 1e-6)
 *   u      = beta_t (v_t - S^T kh);   S <- S + kh u^T   delta-rule corrective write
 *   out_t  = (S^T qh) * sigmoid(g_t)                    full-rank output gate
 *
 * Sources: zuoshipin.com/article/18261 §二 (channel-wise forget gate, delta-
 * rule corrective write, full-rank output gate, per-step retention lower
 * bound that keeps the parallel form inside bf16 range); devpress.csdn.net K3
 * article §二 (predict from memory, take the error, write the correction).
 * The pages print no formula; the exact step order above is the plainest
 * reading of their words.
 *
 * Conventions for every call:
 *  - Array pointers are DEVICE pointers, C-contiguous and 16-byte aligned;
 *    beta only needs 4-byte alignment (so one decode step's slice of a
 *    step-major [T, N, H] array can be passed as is).  Token arrays are
 *    token-major [B, T, H, d]; states are [B, H, d_k, d_v] fp32.  A
 *    segmented sequence [B, n*Ts, H, d] is the same memory as
 *    [B*n, Ts, H, d], so segments are simply extra batch rows.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous on it; buffers must stay alive until the work completes.
 *  - The caller owns all memory, including the workspace.  Nothing on the
 *    path allocates, and apart from kda_prefill_noalloc's fixed scratch area
 *    the library keeps no mutable global state, so calls are reentrant and
 *    may run concurrently on different streams.
 *  - A call puts nothing on its streams but kernel launches (and, for
 *    kda_prefill_pipelined, event records and waits): no memset, copy,
 *    allocation or synchronisation, so it can be captured into a HIP graph
 *    and replayed.  kda_prefill_noalloc looks up its scratch address on its
 *    first call on a device; make that first call outside a capture.
 *  - All checks are synchronous and happen before any launch.  Invalid
 *    arguments return an error and launch nothing.  A failed launch returns
 *    KDA_ERR_HIP.  No data-dependent checks are made.  A NaN log_alpha entry
 *    acts as the floor (the maximum with log_alpha_min returns the floor);
 *    NaN/Inf in every other input propagate.
 *  - Preconditions that are documented but not checked: log_alpha <= 0 and
 *    beta in [0, 1] (then every per-token map is a contraction).
 *  - Supported shapes: d_k == d_v in {64, 128}; chunk == 64; any seqlen >= 0
 *    (a partial last chunk is padded with identity tokens inside the kernels).
 *  - log_alpha_min must lie in [-80/chunk, 0): the floor keeps the decay
 *    folded into one chunk's operands, exp(chunk * |log_alpha_min|), inside
 *    fp32/bf16 range.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad size, out-of-range floor */
    KDA_ERR_UNSUPPORTED = 2,        /* shape or dtype the library does not implement */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERR_HIP = 4,                /* a HIP runtime call or kernel launch failed */
    /* not codes: they give the type the whole int32 range, so any int a
     * caller passes is a value of it (kda_status_string then reports it unknown) */
    KDA_STATUS_RANGE_MIN_ = -2147483647 - 1,
    KDA_STATUS_RANGE_MAX_ = 2147483647
} kda_status;

typedef enum {
    KDA_F32 = 0,                    /* q, k, v, g, out are float32 */
    KDA_BF16 = 1,                   /* q, k, v, g, out are bfloat16 */
    /* not dtypes: the whole int32 range, so any other value is an invalid argument */
    KDA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    KDA_DTYPE_RANGE_MAX_ = 2147483647
} kda_dtype;

typedef struct {
    int64_t batch;          /* B (rows; for segments: B * n_seg)                 */
    int64_t seqlen;         /* T (for segments: the segment length), >= 0        */
    int32_t heads;          /* H                                                 */
    int32_t dk, dv;         /* head dims; d_k == d_v in {64, 128}                */
    int32_t chunk;          /* chunk length C; 64                                */
    kda_dtype io_dtype;     /* dtype of q, k, v, g and out                       */
    float log_alpha_min;    /* per-step retention floor, in log space            */
} kda_problem;

/* Bytes of "update cards" kda_chunk_prepare writes for problem p: one card per
 * (batch row, head, chunk).  Returns 0 if p is invalid or unsupported. */
size_t kda_workspace_size(const kda_problem* p);

/* Stage 1 of the chunk method: prepare every chunk's update card in parallel
 * [zuoshipin.com/article/18261 §四, FlashKDA paragraph: the forget gate,
 * query/key normalisation, decay and the intra-chunk correction matrix are
 * prepared per chunk ahead of the ordered stage].
 *   q, k: [B,T,H,dk] io_dtype;  v: [B,T,H,dv] io_dtype
 *   log_alpha: [B,T,H,dk] fp32 (the floor is applied here);  beta: [B,T,H] fp32
 *   workspace: >= kda_workspace_size(p) bytes, written entirely. */
kda_status kda_chunk_prepare(const kda_problem* p, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2: the ordered state hand-off and the gated read-out (same passage:
 * only the hand-off and the output read-out stay sequential).
 *   workspace: the cards of kda_chunk_prepare for the same p
 *   g: [B,T,H,dv] io_dtype;  out: [B,T,H,dv] io_dtype
 *   state_in: [B,H,dk,dv] fp32, or NULL for an empty memory
 *   state_out: [B,H,dk,dv] fp32, or NULL; may equal state_in (in-place resume,
 *   the KDA state checkpoint of devpress.csdn.net K3 article §十四). */
kda_status kda_chunk_scan(const kda_problem* p, const void* workspace, size_t workspace_bytes,
                          const void* g, const float* state_in, void* out, float* state_out,
                          void* stream);

/* kda_chunk_scan that also emits state checkpoints for a prefix cache: the
 * KDA state is saved at reusable boundaries so a later request that shares
 * the prefix resumes from it [devpress.csdn.net K3 article §十四: KDA state
 * checkpoints kept alongside the paged cache].  With NC = ceil(seqlen/64)
 * chunks and J = ceil(NC / every):
 *   checkpoints: [B, H, J + 1, dk, dv] fp32; entry j (j < J) is the state
 *   after the first 64*every*j tokens (entry 0 = state_in, or 0), entry J the
 *   final state.  every in [1, INT32_MAX]; a value above NC acts as NC
 *   (J = 1).  Other arguments as for kda_chunk_scan. */
kda_status kda_chunk_scan_checkpoints(const kda_problem* p, const void* workspace, size_t workspace_bytes,
                                      const void* g, const float* state_in, void* out, float* state_out,
                                      int32_t every, float* checkpoints, void* stream);

/* Per-segment summary of the context-parallel scheme [zuoshipin.com/article/
 * 18261 §三, "KDA 上下文并行" paragraph: each segment reports how it changes an
 * existing memory and what it builds from an empty one].  For every
 * (batch row, head) of p, with the cards of kda_chunk_prepare:
 *   transition: [B,H,dk,dk] fp32 -- A with S_end = A S_start + zero_state
 *   zero_state: [B,H,dk,dv] fp32 -- the state built from S_start = 0 */
kda_status kda_segment_summarize(const kda_problem* p, const void* workspace, size_t workspace_bytes,
                                 float* transition, float* zero_state, void* stream);

/* In-order prefix merge of segment summaries (same paragraph): for each (b, h)
 *   S(0) = state_init (or 0 if NULL);  seg_state_in[n] = S(n);
 *   S(n+1) = transition[n] S(n) + zero_state[n];  state_final = S(n_seg).
 *   transition: [B,n_seg,H,dk,dk]; zero_state, seg_state_in: [B,n_seg,H,dk,dv];
 *   state_init, state_final: [B,H,dk,dv] (state_final may be NULL).  fp32. */
kda_status kda_segment_combine(int64_t B, int32_t n_seg, int32_t H, int32_t dk, int32_t dv,
                               const float* transition, const float* zero_state,
                               const float* state_init, float* seg_state_in, float* state_final,
                               void* stream);

/* One decode step for N independent sequences: the fixed-size memory is
 * updated in place instead of growing a per-token cache [devpress.csdn.net K3
 * article §十六: KDA keeps a recursive state, not per-token K/V; §十四: state
 * checkpoints].
 *   q, k: [N,H,dk]; v, g, out: [N,H,dv] io_dtype;  log_alpha: [N,H,dk] fp32;
 *   beta: [N,H] fp32;  state: [N,H,dk,dv] fp32, read and written in place. */
kda_status kda_decode_step(int64_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype io_dtype,
                           float log_alpha_min, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const void* g,
                           float* state, void* out, void* stream);

/* Packed variable-length batches: n_seq sequences of different lengths packed
 * back to back along the token axis of one row, as serving batches requests
 * that each carry their own fixed-size state [devpress.csdn.net K3 article
 * §十六: per-request recursive state instead of a growing cache].  The problem
 * p has batch == 1 and seqlen == the packed token count; sequence s is tokens
 * [cu_seqlens[s], cu_seqlens[s+1]) (cu_seqlens: device int32 [n_seq+1],
 * non-decreasing, from 0 to seqlen; values outside [0, seqlen] are clamped,
 * and offsets that go back make later sequences lose chunks once the chunk
 * count reaches what the workspace holds, so no offset array makes an access
 * leave the arrays or the workspace).  Chunks never straddle two sequences,
 * and every sequence's tail is padded inside the kernels.
 *
 * Workspace bytes: chunk offsets, a sequence index per chunk and at most
 * ceil(seqlen/C) + n_seq chunks' cards per head.  Returns 0 if p is invalid or unsupported (batch != 1), or
 * if n_seq is 0. */
size_t kda_varlen_workspace_size(const kda_problem* p, int64_t n_seq);

/* kda_chunk_prepare for a packed batch (same arrays, [1, seqlen, H, d]). */
kda_status kda_varlen_prepare(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens,
                              const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, void* workspace, size_t workspace_bytes, void* stream);

/* kda_chunk_scan for a packed batch, with the workspace kda_varlen_prepare
 * filled for the same p, n_seq and cu_seqlens (the chunk offsets it wrote are
 * read back, clamped to the workspace and to each sequence's length: another
 * workspace or other offsets give wrong values, never an access outside the
 * arrays or the workspace).  g, out: [1, seqlen, H, dv];
 * state_in, state_out: [n_seq, H, dk, dv] fp32 or NULL (state_out may equal
 * state_in); an empty sequence passes its state_in through. */
kda_status kda_varlen_scan(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens,
                           const void* workspace, size_t workspace_bytes, const void* g,
                           const float* state_in, void* out, float* state_out, void* stream);

/* Bytes of scratch kda_backward needs for problem p: per (b, h), the update
 * card and the reverse-pass card of every chunk, the forward output, the
 * state entering every chunk plus the final state, and the state gradient
 * leaving every chunk (fp32 states), each region rounded up to 256 bytes.
 * Returns 0 if p is invalid or unsupported, or if p has no tokens. */
size_t kda_backward_workspace_size(const kda_problem* p);

/* Gradients for training [zuoshipin.com/article/18261 §四: the fused kernels
 * serve training throughput as well as inference; the recurrence is the one
 * at the top of this file, zuoshipin §二].  With
 *   L = <d_out, out> + <d_state, S_T>,
 * out and S_T being what kda_chunk_prepare + kda_chunk_scan compute from the
 * same inputs, writes dL/dq, dL/dk, dL/dv, dL/dlog_alpha, dL/dbeta, dL/dg and
 * dL/dstate_in.  Where log_alpha <= log_alpha_min the floor binds and
 * dlog_alpha is 0; where |k_t| or |q_t| is below 1e-6 the normaliser is the
 * constant 1e-6.
 *   q, k, v, log_alpha, beta, g, state_in: as for prefill (state_in may be NULL)
 *   d_out: [B,T,H,dv] io_dtype, or NULL (zero);  d_state: [B,H,dk,dv] fp32, or NULL
 *   dq, dk: [B,T,H,dk], dv, dg: [B,T,H,dv] io_dtype;  dlog_alpha: [B,T,H,dk] fp32;
 *   dbeta: [B,T,H] fp32 (4-byte alignment suffices);  d_state_in: [B,H,dk,dv] fp32,
 *   or NULL.  Every output is overwritten, not accumulated.
 *   workspace: >= kda_backward_workspace_size(p) bytes (contents on entry unused). */
kda_status kda_backward(const kda_problem* p, const void* q, const void* k, const void* v,
                        const float* log_alpha, const float* beta, const void* g, const float* state_in,
                        const void* d_out, const float* d_state, void* dq, void* dk, void* dv,
                        float* dlog_alpha, float* dbeta, void* dg, float* d_state_in,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Prefill for training: the output and final state of kda_chunk_prepare +
 * kda_chunk_scan, computed so that the update cards and the state entering
 * every chunk stay in a kda_backward workspace for kda_backward_after_prefill
 * [zuoshipin.com/article/18261 §四: the kernels serve training throughput;
 * the forward's hand-off states are what the backward consumes].
 *   q, k, v, log_alpha, beta, g, state_in, out, state_out: as for
 *   kda_chunk_prepare and kda_chunk_scan (state_out may equal state_in).
 *   workspace: >= kda_backward_workspace_size(p) bytes, caller-owned; it then
 *   holds the forward pass of these inputs until it is reused. */
kda_status kda_prefill_for_backward(const kda_problem* p, const void* q, const void* k, const void* v,
                                    const float* log_alpha, const float* beta, const void* g,
                                    const float* state_in, void* out, float* state_out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* kda_backward without its forward pass: the same gradients, read from the
 * workspace that kda_prefill_for_backward filled for the same problem and the
 * same q, k, v, log_alpha, beta, g and state_in, with `out` the output it
 * wrote (unchanged since).  Other arguments as for kda_backward (there is no
 * state_in: the workspace holds the state entering every chunk).  Inputs that
 * differ from that prefill's give gradients of the wrong point; this is not
 * checked.  The workspace keeps the forward pass, so a second call with other
 * d_out / d_state is valid too. */
kda_status kda_backward_after_prefill(const kda_problem* p, const void* q, const void* k, const void* v,
                                      const float* log_alpha, const float* beta, const void* g, const void* out,
                                      const void* d_out, const float* d_state, void* dq, void* dk, void* dv,
                                      float* dlog_alpha, float* dbeta, void* dg, float* d_state_in,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch kda_varlen_backward needs for a packed batch of n_seq
 * sequences over p->seqlen tokens (p->batch must be 1): the chunk offsets
 * and chunk -> sequence map, then the regions of kda_backward's workspace
 * sized for the most chunks n_seq sequences can have, ceil(seqlen / 64) +
 * n_seq per head.  Returns 0 if p is invalid or unsupported, or if there are
 * no sequences or no tokens. */
size_t kda_varlen_backward_workspace_size(const kda_problem* p, int64_t n_seq);

/* Gradients of a packed variable-length batch for training [zuoshipin.com/
 * article/18261 §四: the kernels serve training throughput; devpress.csdn.net
 * K3 article §十六: each sequence keeps its own state]: kda_backward for every
 * sequence of kda_varlen_prepare + kda_varlen_scan at once, all sequences'
 * chunks in one launch per kernel.  The gradients equal kda_backward's on each
 * sequence alone, bit for bit.
 *   cu_seqlens: as for kda_varlen_prepare (same validity rules; a sequence
 *   whose range is empty passes its state gradient through; token rows that
 *   no sequence covers, possible only with offsets outside the rules, are
 *   not written).
 *   q, k, v, log_alpha, beta, g, d_out and the token gradients dq, dk, dv,
 *   dlog_alpha, dbeta, dg: the packed [1, T, H, d] arrays, as for kda_backward.
 *   state_in, d_state, d_state_in: [n_seq, H, dk, dv] fp32, or NULL.
 *   workspace: >= kda_varlen_backward_workspace_size(p, n_seq) bytes. */
kda_status kda_varlen_backward(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens, const void* q,
                               const void* k, const void* v, const float* log_alpha, const float* beta,
                               const void* g, const float* state_in, const void* d_out, const float* d_state,
                               void* dq, void* dk, void* dv, float* dlog_alpha, float* dbeta, void* dg,
                               float* d_state_in, void* workspace, size_t workspace_bytes, void* stream);

/* The split training pair for a packed batch [the same passages]: a
 * kda_varlen_prepare + kda_varlen_scan whose cards and chunk states stay in a
 * kda_varlen_backward workspace, then the backward without its own forward
 * pass.  Arguments as for kda_varlen_backward, plus out and state_out as for
 * kda_varlen_scan; kda_varlen_backward_after_prefill takes the same problem,
 * cu_seqlens, inputs and workspace, and `out` as the first call left it, and
 * gives kda_varlen_backward's gradients bit for bit (inputs that differ from
 * the first call's give gradients of the wrong point; this is not checked).
 * The second call reads back the chunk offsets the first one wrote into the
 * workspace, clamped to the workspace and to each sequence's length: a
 * workspace that call did not fill, or other cu_seqlens, give wrong values
 * but no access outside the arrays or the workspace. */
kda_status kda_varlen_prefill_for_backward(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens,
                                           const void* q, const void* k, const void* v, const float* log_alpha,
                                           const float* beta, const void* g, const float* state_in, void* out,
                                           float* state_out, void* workspace, size_t workspace_bytes,
                                           void* stream);
kda_status kda_varlen_backward_after_prefill(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens,
                                             const void* q, const void* k, const void* v, const float* log_alpha,
                                             const float* beta, const void* g, const void* out, const void* d_out,
                                             const float* d_state, void* dq, void* dk, void* dv, float* dlog_alpha,
                                             float* dbeta, void* dg, float* d_state_in, void* workspace,
                                             size_t workspace_bytes, void* stream);

/* Workspace bytes of kda_prefill_pipelined with ranges of range_chunks
 * chunks: the carried state (B*H*dk*dv fp32), then the update cards of one
 * range for every (row, head), twice when the sequence spans more than one
 * range, each part rounded up to 256 bytes.  Returns 0 if p is invalid or
 * unsupported or range_chunks < 1. */
size_t kda_pipelined_workspace_size(const kda_problem* p, int32_t range_chunks);

/* Chunked prefill with the two stages overlapped [lotamate.com Kimi K3
 * training analysis, §四 基础设施: FlashKDA overlaps the intra-chunk work with
 * the state passed from chunk to chunk].  The sequence is cut into ranges of
 * range_chunks whole chunks (the last may be shorter); the cards of range
 * i + 1 are prepared on aux_stream into one of two buffers while the scan of
 * range i runs on `stream` from the other, carrying the state from range to
 * range, so the cards in use stay a bounded size.  Results are identical to
 * kda_chunk_prepare + kda_chunk_scan on the same inputs.
 *   q, k, v, log_alpha, beta, g, out, state_in, state_out: as for
 *   kda_chunk_prepare and kda_chunk_scan (state_out may equal state_in).
 *   range_chunks: >= 1 chunks per range.
 *   workspace: >= kda_pipelined_workspace_size(p, range_chunks) bytes,
 *   caller-owned; contents on entry unused.
 *   stream, aux_stream: hipStream_t; aux_stream may equal stream (then the
 *   ranges run one after the other).  aux_stream first waits for the work
 *   already on `stream`, and `stream` waits for everything this call put on
 *   aux_stream before any later work on `stream`, so the caller orders
 *   against `stream` alone.  The call creates and releases its own HIP events.
 * Errors as for the other calls; KDA_ERR_HIP also when an event cannot be
 * created or recorded. */
kda_status kda_prefill_pipelined(const kda_problem* p, const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* beta, const void* g,
                                 const float* state_in, void* out, float* state_out, int32_t range_chunks,
                                 void* workspace, size_t workspace_bytes, void* stream, void* aux_stream);

/* Bytes of the fixed device scratch area of kda_prefill_noalloc (per GPU). */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Chunked prefill (kda_chunk_prepare + kda_chunk_scan) that allocates
 * nothing and takes no workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The update cards go to a fixed scratch area of
 * KDA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  Tokens are processed in ranges of whole chunks
 * whose cards for all (row, head) fit that area; between ranges the state
 * travels in state_out, or, when state_out is NULL, at the front of the area.
 * Results are the same as kda_chunk_prepare + kda_chunk_scan on the same
 * inputs.
 *   q, k, v, log_alpha, beta, g, out, state_in, state_out: as for
 *   kda_chunk_prepare and kda_chunk_scan (state_out may equal state_in).
 * Returns KDA_ERR_WORKSPACE_TOO_SMALL, launching nothing, when the cards of
 * one chunk for every (row, head) (B*H cards of 74,240 bytes at bf16 d=128)
 * do not fit the area beside the carried state.  Every call on a GPU uses
 * that GPU's one area, which keeps the last call's contents: calls that
 * overlap on one GPU (other streams, other threads) race, so serialise them. */
kda_status kda_prefill_noalloc(const kda_problem* p, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const void* g,
                               const float* state_in, void* out, float* state_out, void* stream);

/* Static text for a status code. */
const char* kda_status_string(kda_status s);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
