/*
 * kda.h -- C ABI of libkda.so: Kimi Delta Attention (KDA) on AMD Instinct
 * MI355X (gfx950).
 *
 * KDA is linear attention with one fixed-size state per (sequence, head): a
 * dk x dv fp32 matrix S whose rows are key channels.  Each token forgets old
 * content per key channel and writes new content by a delta rule:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T (scale * q_t)
 *
 * Sources (page title, section):
 *  - neurohive.io Kimi K3 review, "Sequence length: hybrid KDA and Gated MLA
 *    attention": delta rule (forget + write), retention factor per channel, log
 *    decay bounded below at -5, every tile on dense matrix multiplies.
 *  - best.xiaohu.ai "Kimi K3 tech report", "Sequence length: replacing most
 *    attention layers with fixed-size memory": state size independent of context
 *    length; older context decays gradually across channels.
 *  - neurohive.io review, "Training and inference infrastructure", and
 *    best.xiaohu.ai, "Infrastructure efficiency": one fixed-size state per
 *    request, restored from snapshots for prefix caching (state in -> state out).
 * The pages give the rule in words; the equation above is its plainest reading
 * (decay first, then the delta correction on the decayed state; the output reads
 * the state after the token's own write).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, contiguous and
 *    row-major.
 *  - Workspaces.  Prefill on bf16 input at d = 128 with 256 or more (sequence, head)
 *    streams runs fused and needs none.  Fixed-length bf16 prefill at d = 128 with 4
 *    to 32 streams and long sequences cuts each sequence into R segments and needs
 *    3R - 2 fp32 [dk, dv] states per stream.  Every other prefill, the backward and the
 *    transition need one per call, sized by the matching *_workspace_size function
 *    (pure host arithmetic).  The *_ws entry points and kda_prefill run on a
 *    workspace the caller owns (256-byte aligned, contents irrelevant, garbage on
 *    exit; calls that may overlap need distinct ones) and allocate nothing.  The
 *    entry points without a workspace argument are a convenience layer over them:
 *    they take a block the library keeps per device.  A call takes a free block at
 *    least as large as it needs, its stream first waiting for the event recorded
 *    when the block was last released, or allocates one (hipMallocFromPoolAsync on
 *    `stream` from a pool the library creates per device); at the end it records
 *    that event on `stream` and keeps the block while the device's free blocks total
 *    at most 4 GiB, returning the largest to the pool beyond that (hipFreeAsync,
 *    which on ROCm 7 blocks the host until the stream has drained).  Blocks too
 *    small for a request are returned the same way when a larger one is allocated.
 *    An allocation failure returns KDA_ERR_HIP.  Decode and kda_state_compose
 *    allocate nothing.
 *  - Alignment (KDA_ERR_ALIGN otherwise): prefill v and out 16 bytes, q, k, g and
 *    the states 4 bytes, beta its element size; decode state 16 bytes, every
 *    other pointer its element size.
 *  - Layouts: q, k, g  [tokens, H, dk];  v, out [tokens, H, dv];  beta [tokens, H];
 *    states [seqs, H, dk, dv] fp32 (row i = key channel i).
 *  - `dtype` (KDA_BF16 or KDA_F32) is the element type of q, k, v, g, beta and
 *    out.  States are always fp32.  Arithmetic is fp32 with bf16 matrix-core
 *    operands for KDA_BF16 and fp32 matrix-core operands for KDA_F32.
 *  - q and k are used as given (the library does not normalise them) and no
 *    output gate or norm is applied.
 *  - Value preconditions, not checked: -5 <= g <= 0, 0 <= beta <= 1, all finite,
 *    |k| <= 1.  Outside them the result is unspecified (never a memory fault).
 *  - Work is enqueued on `stream` and returns immediately; execution errors
 *    surface at the caller's next synchronisation.  No entry point keeps state
 *    between calls other than the kept workspace blocks above (event-ordered, so
 *    calls never share a live workspace); calls on different streams may overlap
 *    when their buffers do not.
 *  - Return value: KDA_OK, or a negative KDA_ERR_* code.  Argument codes
 *    (everything but KDA_ERR_HIP) are returned before anything is enqueued.
 *    A call clears any error an earlier HIP call left pending on the calling
 *    thread, then launches its kernels one after another, checking each launch,
 *    and stops at the first that fails: KDA_ERR_HIP means some of its kernels may
 *    already be enqueued, and its outputs are unspecified.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

enum kda_dtype { KDA_BF16 = 0, KDA_F32 = 1 };

enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  KDA_ERR_SHAPE = -2,       /* a size is <= 0, or too large for 32-bit grids */
  KDA_ERR_HEAD_DIM = -3,    /* dk or dv not in {64, 128}, dk != dv, or the
                               fp32 prologue / snapshot prefill at dk = 128 */
  KDA_ERR_DTYPE = -4,       /* dtype is not KDA_BF16 or KDA_F32              */
  KDA_ERR_ALIGN = -5,       /* a pointer is not aligned as required          */
  KDA_ERR_HIP = -6,         /* the HIP runtime reported a launch error       */
  KDA_ERR_NO_DEVICE = -7,   /* the current device is not gfx950              */
  KDA_ERR_WORKSPACE = -8    /* workspace NULL, misaligned or too small       */
};

/* ABI version of the loaded library (KDA_ABI_VERSION). */
int kda_abi_version(void);

/* Static, human-readable text for a kda_status value. */
const char* kda_status_string(int status);

/*
 * Chunked prefill over B sequences of T tokens each (chunk = 64 tokens).
 *
 *  q, k, g        [B, T, H, dk]  (dtype)
 *  v              [B, T, H, dv]  (dtype)
 *  beta           [B, T, H]      (dtype)
 *  initial_state  [B, H, dk, dv] fp32, or NULL for a zero state
 *  out            [B, T, H, dv]  (dtype), written for every token
 *  final_state    [B, H, dk, dv] fp32, or NULL to skip; may equal
 *                 initial_state (updated in place)
 *  scale          multiplies q (typically 1/sqrt(dk))
 * dk == dv, both 64 or 128.  Produces the same result as running the recurrence
 * token by token, up to floating-point rounding.  KDA_F32 at d = 128 runs on fp32
 * chunk operands (the backward's) in windows of up to 16 chunks, one fp32 state per
 * (sequence, head) carried between windows; its gate-prologue and snapshot forms
 * are not provided (KDA_ERR_HEAD_DIM).
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* initial_state, void* out,
                  float* final_state, int B, int T, int H, int dk, int dv,
                  float scale, int dtype, hipStream_t stream);

/*
 * Names of the kernels a prefill call with these sizes launches, for reports and
 * profiling (N sequences; fixed length: T tokens each; varlen != 0: packed, total_T
 * tokens).  Static, thread-local text, valid until the calling thread calls this
 * again; "" when the sizes or dtype are not accepted.  Pure host logic.
 */
const char* kda_chunk_fwd_schedule(int N, int T, int total_T, int H, int dk, int dv,
                                   int dtype, int varlen);

/*
 * Bytes of workspace kda_chunk_fwd_ws needs for these sizes (the same schedule
 * kda_chunk_fwd runs), or 0 when the sizes or dtype are not accepted by
 * kda_chunk_fwd.  Pure host arithmetic: no device call.
 */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype);

/*
 * kda_chunk_fwd on a workspace the caller owns, so the call allocates and frees
 * nothing and returns as soon as its kernels are enqueued.
 *  workspace        device memory of at least kda_chunk_fwd_workspace_size(B, T,
 *                   H, dk, dv, dtype) bytes, 256-byte aligned; its contents on
 *                   entry do not matter and are garbage on exit.  Calls that may
 *                   overlap (other streams) need distinct workspaces.
 *  workspace_bytes  its size; NULL, misaligned or too small -> KDA_ERR_WORKSPACE.
 * Every other argument, and every result, is exactly as for kda_chunk_fwd.
 */
int kda_chunk_fwd_ws(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* initial_state, void* out,
                     float* final_state, int B, int T, int H, int dk, int dv, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Every prefill variant on a caller workspace, in one descriptor: fixed length or
 * packed, plain or with the gate prologue, with or without snapshots.  The fields
 * mean exactly what the arguments of the named entry points mean:
 *  q, k, v, g, beta, initial_state, out, final_state  as for kda_chunk_fwd (raw
 *                     activations for q, k, g, beta when `prologue` is nonzero,
 *                     see kda_chunk_fwd_prologue);
 *  cu_seqlens         NULL: N sequences of T tokens each (fixed length); else the
 *                     packed offsets of kda_chunk_fwd_varlen, with total_T tokens;
 *  N                  number of sequences (B for fixed length);
 *  snapshots, snapshot_tokens  NULL and 0 for none; else as for
 *                     kda_chunk_fwd_snapshots / kda_chunk_fwd_varlen_snapshots.
 * kda_prefill_workspace_size writes the bytes of workspace the call needs (0 when
 * it needs none) after the same argument checks kda_prefill makes, and returns
 * their code; it makes no device call.  kda_prefill runs the call on `workspace`
 * (NULL allowed when 0 bytes are needed; else 256-byte aligned and at least that
 * large, or KDA_ERR_WORKSPACE) and allocates nothing.  Results equal those of the
 * matching named entry point bit for bit.
 */
typedef struct kda_prefill_desc {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* initial_state;
  void* out;
  float* final_state;
  const int32_t* cu_seqlens;
  int N;
  int T;
  int total_T;
  int H;
  int dk;
  int dv;
  float scale;
  int dtype;
  int prologue;
  float* snapshots;
  int snapshot_tokens;
} kda_prefill_desc;

int kda_prefill_workspace_size(const kda_prefill_desc* desc, size_t* bytes);
int kda_prefill(const kda_prefill_desc* desc, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * kda_chunk_fwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): same arguments and results
 * within the bf16 / fp32 tolerances of the other entry points, and it calls no
 * hipMalloc, hipFree or allocating routine.  Its scratch is a fixed 64 MiB device
 * array inside the library, one per GPU, held until the process ends; the fused
 * schedule needs none, a schedule whose workspace fits it runs as kda_chunk_fwd
 * would, the others run in windows of chunks short enough for it (down to one
 * chunk per window).  Sizes for which even one-chunk windows do not
 * fit (the carried fp32 states plus two windows' chunk operands exceed 64 MiB, e.g.
 * fp32 at d = 64 with 400 heads) return KDA_ERR_WORKSPACE before anything is
 * enqueued.  Every call on a GPU uses that GPU's one array and nothing in it needs
 * clearing between calls; calls that overlap on one GPU (other streams, other
 * threads) race on it and must be serialised by the caller.
 */
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* initial_state, void* out,
                          float* final_state, int B, int T, int H, int dk, int dv, float scale,
                          int dtype, hipStream_t stream);

/*
 * kda_chunk_fwd with the gate and normalisation prologue fused into the kernels'
 * loads, so the activations that produce q, k, g and beta are not written out
 * and read back.  The pages bound the log of the per-channel retention factor
 * below at -5 (neurohive.io Kimi K3 review, "Sequence length: hybrid KDA and
 * Gated MLA attention") but give no gate formula; the plainest reading, used
 * here, is
 *     q = q_raw / sqrt(|q_raw|^2 + 1e-6),   k = k_raw / sqrt(|k_raw|^2 + 1e-6)
 *                                           (per token and head, over dk)
 *     g = max(-5, -softplus(g_raw)) = max(-5, -log(1 + exp(g_raw)))   (per channel)
 *     beta = sigmoid(beta_raw) = 1 / (1 + exp(-beta_raw))
 * followed by exactly the computation of kda_chunk_fwd.  Normalised q and k are
 * rounded to the input precision before use (as if they had been stored in it);
 * g and beta are used in fp32.  Arguments, layouts and codes are those of
 * kda_chunk_fwd, with the raw tensors in place of q, k, g and beta.
 */
int kda_chunk_fwd_prologue(const void* q_raw, const void* k_raw, const void* v,
                           const void* g_raw, const void* beta_raw, const float* initial_state,
                           void* out, float* final_state, int B, int T, int H, int dk, int dv,
                           float scale, int dtype, hipStream_t stream);

/*
 * kda_chunk_fwd that also keeps the state at regular token boundaries, for
 * prefix caching: one fixed-size state per request is restored from the nearest
 * snapshot instead of re-running the prefix (neurohive.io Kimi K3 review,
 * "Training and inference infrastructure"; best.xiaohu.ai "Kimi K3 tech
 * report", "Infrastructure efficiency": state checkpoints at sparse boundaries).
 *
 *  snapshots        [B, H, ceil(T / snapshot_tokens), dk, dv] fp32, required.
 *                   Snapshot i is the state after min((i + 1) * snapshot_tokens,
 *                   T) tokens, i.e. exactly the final state of a run over that
 *                   prefix; the last one equals final_state.
 *  snapshot_tokens  > 0 and a multiple of 64 (chunk-aligned), else KDA_ERR_SHAPE.
 * Every other argument, and the values of out and final_state, are exactly as
 * for kda_chunk_fwd.
 */
int kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, void* out,
                            float* final_state, float* snapshots, int snapshot_tokens,
                            int B, int T, int H, int dk, int dv, float scale, int dtype,
                            hipStream_t stream);

/*
 * Chunked prefill over N packed sequences of different lengths.
 *
 *  cu_seqlens     int32 DEVICE array of N+1 non-decreasing token offsets,
 *                 cu_seqlens[0] == 0, cu_seqlens[N] == total_T.  A sequence of
 *                 length 0 gets out untouched and final_state = initial_state.
 *  q, k, g        [total_T, H, dk]; v, out [total_T, H, dv]; beta [total_T, H]
 *  initial_state  [N, H, dk, dv] fp32 or NULL;  final_state [N, H, dk, dv] or NULL
 * Chunks restart at every sequence start and no state crosses a sequence
 * boundary.  Sequences are scheduled longest first when N <= 256.  The offsets
 * are read on the device only; inconsistent offsets are clamped to [0, total_T].
 * Head sizes as for kda_chunk_fwd.
 */
int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, void* out,
                         float* final_state, const int32_t* cu_seqlens, int N,
                         int total_T, int H, int dk, int dv, float scale, int dtype,
                         hipStream_t stream);

/*
 * Workspace bytes kda_chunk_fwd_varlen_ws needs (0: none, the fused schedule, or
 * sizes not accepted -- kda_prefill_workspace_size tells the two apart).  The
 * packed schedules that take one need a 64-token slot per chunk per head for
 * ceil(total_T / 64) + N chunks (66,048 bytes each for bf16 at d = 128), so it is
 * bounded by the packed tokens, never by the longest sequence alone.
 */
size_t kda_chunk_fwd_varlen_workspace_size(int N, int total_T, int H, int dk, int dv,
                                           int dtype);

/*
 * kda_chunk_fwd_varlen on a caller workspace (see the conventions above): same
 * arguments, same results, allocates nothing.
 */
int kda_chunk_fwd_varlen_ws(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, void* out,
                            float* final_state, const int32_t* cu_seqlens, int N, int total_T,
                            int H, int dk, int dv, float scale, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd_varlen on raw activations, with the gate and normalisation
 * prologue of kda_chunk_fwd_prologue (same formulas, same rounding) fused into the
 * loads.  Arguments, layouts and codes are those of kda_chunk_fwd_varlen, with the
 * raw tensors in place of q, k, g and beta.
 */
int kda_chunk_fwd_varlen_prologue(const void* q_raw, const void* k_raw, const void* v,
                                  const void* g_raw, const void* beta_raw,
                                  const float* initial_state, void* out, float* final_state,
                                  const int32_t* cu_seqlens, int N, int total_T, int H, int dk,
                                  int dv, float scale, int dtype, hipStream_t stream);

/*
 * kda_chunk_fwd_varlen that also keeps each sequence's state every
 * snapshot_tokens tokens, for prefix caching of a packed batch (the sources of
 * kda_chunk_fwd_snapshots).
 *  snapshots        fp32, required: [S_total, H, dk, dv] with
 *                   S_total = sum over sequences n of ceil(L_n / snapshot_tokens),
 *                   L_n = cu_seqlens[n+1] - cu_seqlens[n].  Sequence n owns rows
 *                   off_n .. off_n + ceil(L_n / snapshot_tokens) - 1, where off_n is
 *                   the same sum over the sequences before n; row off_n + i holds,
 *                   for every head, the state after min((i + 1) * snapshot_tokens,
 *                   L_n) tokens of sequence n (the last one equals its final state).
 *                   An empty sequence has no row.  The caller sizes the buffer from
 *                   its own copy of the lengths.
 *  snapshot_tokens  > 0 and a multiple of 64, else KDA_ERR_SHAPE.
 * Every other argument, and the values of out and final_state, are exactly as for
 * kda_chunk_fwd_varlen.
 */
int kda_chunk_fwd_varlen_snapshots(const void* q, const void* k, const void* v, const void* g,
                                   const void* beta, const float* initial_state, void* out,
                                   float* final_state, float* snapshots, int snapshot_tokens,
                                   const int32_t* cu_seqlens, int N, int total_T, int H, int dk,
                                   int dv, float scale, int dtype, hipStream_t stream);

/*
 * Backward pass of kda_chunk_fwd (fixed length): the gradients of
 *     L = sum over tokens of <grad_out, out> + <grad_final_state, final_state>
 * with respect to q, k, v, g, beta and initial_state.  The pages train KDA at up
 * to 1M tokens of context (best.xiaohu.ai "Kimi K3 tech report", context
 * curriculum) but print no backward; the gradients are the plain derivatives of
 * the recurrence above.
 *
 *  q, k, v, g, beta, initial_state, B, T, H, dk, dv, scale, dtype: the forward
 *                      call's arguments (initial_state NULL = zero).
 *  grad_out            [B, T, H, dv] (dtype), required.
 *  grad_final_state    [B, H, dk, dv] fp32 or NULL (zero).
 *  grad_q, grad_k, grad_g [B, T, H, dk]; grad_v [B, T, H, dv]; grad_beta [B, T, H]
 *                      (dtype), required, fully overwritten.
 *  grad_initial_state  [B, H, dk, dv] fp32 or NULL (not computed).
 * dk == dv in {64, 128} for both dtypes.  q, k, v, g and grad_out are read up to
 * 16 bytes at a time and must be 16-byte aligned; every other pointer needs only
 * its element alignment (else KDA_ERR_ALIGN).  The forward is recomputed inside
 * the call (nothing is kept from kda_chunk_fwd).  fp32 inputs: fp32 throughout
 * (fp32 matrix cores).  bf16 inputs: every product over 32 or more terms takes
 * bf16 operands rounded from fp32 values, with fp32 accumulation, and the
 * per-chunk states, state gradients, Delta and dU are kept as bf16; the inverse,
 * the 16-term sub-tile products and the decayed products stay fp32.  The call's
 * one-pass workspace (kda_chunk_bwd_workspace_size) takes, per 64-token chunk per
 * head, 418,304 bytes for bf16 and 410,112 for fp32 at d = 128 (246,016 and 213,248
 * at d = 64), so T = 65,536 with 32 heads would need about 14 GB: this call takes at
 * most 2 GiB and runs in windows of chunks beyond that (see
 * kda_chunk_bwd_window_workspace_size).
 * Outputs must not alias inputs.
 */
int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  const float* initial_state, const void* grad_out,
                  const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v,
                  void* grad_g, void* grad_beta, float* grad_initial_state, int B, int T, int H,
                  int dk, int dv, float scale, int dtype, hipStream_t stream);

/* Workspace bytes of kda_chunk_bwd for these sizes (0: sizes not accepted). */
size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype);

/*
 * Workspace bytes of kda_chunk_bwd run in windows of window_chunks 64-token chunks
 * (0: no windows, the same as kda_chunk_bwd_workspace_size; 0 returned for sizes not
 * accepted or a negative window).  In windows the call keeps one window's chunk items
 * plus one [B, H, dk, dv] fp32 state per window and two state-gradient buffers, so the
 * workspace no longer grows by a chunk's items per 64 tokens (training at long
 * contexts, best.xiaohu.ai "Kimi K3 tech report", context-curriculum section); the
 * cost is a second pass over each window's operands and forward scan.
 */
size_t kda_chunk_bwd_window_workspace_size(int B, int T, int H, int dk, int dv, int dtype,
                                           int window_chunks);

/*
 * kda_chunk_bwd on a caller workspace (256-byte aligned): same arguments and results,
 * allocates nothing.  With at least kda_chunk_bwd_workspace_size bytes the call runs
 * in one pass; with less it runs in the largest windows whose
 * kda_chunk_bwd_window_workspace_size fits (results equal to the one-pass call's,
 * bit for bit); below the one-chunk-window size it returns KDA_ERR_WORKSPACE.  The
 * self-allocating kda_chunk_bwd (and kda_chunk_bwd_varlen) take at most 2 GiB and
 * run in windows beyond that.
 */
int kda_chunk_bwd_ws(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     const float* initial_state, const void* grad_out,
                     const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v,
                     void* grad_g, void* grad_beta, float* grad_initial_state, int B, int T,
                     int H, int dk, int dv, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_bwd for packed variable-length input (the layout of
 * kda_chunk_fwd_varlen): the gradients of
 *     L = sum over tokens of <grad_out, out> + <grad_final_state, final_state>
 * for kda_chunk_fwd_varlen's inputs.
 *  q, k, g, grad_q, grad_k, grad_g [total_T, H, dk];  v, grad_out, grad_v
 *  [total_T, H, dv];  beta, grad_beta [total_T, H]  (dtype);
 *  initial_state, grad_final_state, grad_initial_state  [N, H, dk, dv] fp32 or NULL;
 *  cu_seqlens       int32 [N + 1] on the device, as for kda_chunk_fwd_varlen.
 * Chunks start at each sequence's first token; no state crosses a sequence
 * boundary.  Tokens outside every sequence get no gradient written.  Precision,
 * alignment, head sizes and codes are those of kda_chunk_bwd; the workspace
 * takes the same bytes per chunk per head for ceil(total_T / 64) + N chunks.
 */
int kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, const void* grad_out,
                         const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v,
                         void* grad_g, void* grad_beta, float* grad_initial_state,
                         const int32_t* cu_seqlens, int N, int total_T, int H, int dk, int dv,
                         float scale, int dtype, hipStream_t stream);

/* Workspace bytes of kda_chunk_bwd_varlen for these sizes (0: sizes not accepted). */
size_t kda_chunk_bwd_varlen_workspace_size(int N, int total_T, int H, int dk, int dv, int dtype);

/* kda_chunk_bwd_window_workspace_size for kda_chunk_bwd_varlen (windows count chunks
 * from each sequence's start; ceil(total_T / 64) bounds every sequence's chunks). */
size_t kda_chunk_bwd_varlen_window_workspace_size(int N, int total_T, int H, int dk, int dv,
                                                  int dtype, int window_chunks);

/* kda_chunk_bwd_varlen on a caller workspace, as kda_chunk_bwd_ws is to kda_chunk_bwd
 * (windows as there). */
int kda_chunk_bwd_varlen_ws(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, const void* grad_out,
                            const float* grad_final_state, void* grad_q, void* grad_k,
                            void* grad_v, void* grad_g, void* grad_beta,
                            float* grad_initial_state, const int32_t* cu_seqlens, int N,
                            int total_T, int H, int dk, int dv, float scale, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Context parallelism for one long sequence split into R segments (design for
 * several GPUs, one segment per GPU; every step also runs on one GPU).  A
 * segment maps its entry state affinely to its exit state,
 *     S_exit = P S_entry + R_part,
 * where R_part is the final state of kda_chunk_fwd over the segment with no
 * initial state and P is the segment's transition.  The pages keep one
 * fixed-size state per request that a prefix cache can restore (neurohive.io
 * Kimi K3 review, "Training and inference infrastructure"); they describe no
 * context-parallel scheme, so this is a plain reading of the chunked form.  The
 * steps: every segment computes R_part (kda_chunk_fwd) and P
 * (kda_chunk_transition); the (P, R_part) of all segments are gathered;
 * kda_state_compose gives every entry state; every segment reruns kda_chunk_fwd
 * from its entry state for its outputs.
 *
 * kda_chunk_transition: P for each of B independent segments.
 *  k, g, beta      as for kda_chunk_fwd ([B, T, H, .], dtype), except that k and
 *                  g are read four elements at a time and must be 16-byte
 *                  aligned (else KDA_ERR_ALIGN).  The transition depends on
 *                  neither q nor v: q is not read and may be NULL (if given, it
 *                  must be 16-byte aligned); v is not an argument.
 *  transition      [B, H, dk, dk] fp32, required: the exit state of the segment
 *                  run with v = 0 from the identity, i.e. the product of its
 *                  per-token maps (I - beta_t k_t k_t^T) Diag(exp g_t), latest
 *                  token leftmost.
 * dk == dv in {64, 128} for both dtypes.  fp32 inputs are computed on fp32
 * operands; bf16 inputs on bf16 matrix-core operands with fp32 accumulation and
 * an fp32 state, the precision of the bf16 prefill.  Its workspace
 * (kda_chunk_transition_workspace_size) takes, per 64-token chunk per head,
 * 213,504 bytes for fp32 and 320,000 for bf16 at d = 128 (147,712 and 213,248 at
 * d = 64); none for bf16 at d = 128 with B H >= 256, which runs on the fused
 * prefill kernel (one workgroup per (segment, head)).
 */
int kda_chunk_transition(const void* q, const void* k, const void* g, const void* beta,
                         float* transition, int B, int T, int H, int dk, int dv, int dtype,
                         hipStream_t stream);

/* Workspace bytes of kda_chunk_transition for these sizes (0: sizes not accepted). */
size_t kda_chunk_transition_workspace_size(int B, int T, int H, int dk, int dv, int dtype);

/* kda_chunk_transition on a caller workspace: same arguments and results, allocates nothing. */
int kda_chunk_transition_ws(const void* q, const void* k, const void* g, const void* beta,
                            float* transition, int B, int T, int H, int dk, int dv, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_state_compose: the sequential composition over R segments,
 *     entry_states[0] = initial_state (NULL = zero),
 *     entry_states[r + 1] = transitions[r] entry_states[r] + partial_states[r],
 * so entry_states[r] is the state entering segment r and entry_states[R] the
 * state after the last one.
 *  transitions     [R, B, H, dk, dk] fp32;  partial_states [R, B, H, dk, dv] fp32;
 *  initial_state   [B, H, dk, dv] fp32 or NULL;  entry_states [R + 1, B, H, dk, dv].
 * All fp32, 16-byte aligned; entry_states must not alias the inputs.  dk == dv in
 * {64, 128}.  Allocates nothing.
 */
int kda_state_compose(const float* transitions, const float* partial_states,
                      const float* initial_state, float* entry_states, int R, int B, int H,
                      int dk, int dv, hipStream_t stream);

/*
 * One decode token for B sequences, updating `state` in place.
 *
 *  q, k, g  [B, H, dk] (dtype);  v, out [B, H, dv] (dtype);  beta [B, H] (dtype)
 *  state    [B, H, dk, dv] fp32, read and overwritten with the new state
 * Same result as kda_chunk_fwd with T = 1 and final_state == initial_state.
 */
int kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, float* state, void* out, int B, int H, int dk,
                    int dv, float scale, int dtype, hipStream_t stream);

/*
 * kda_decode_step on raw activations, with the gate and normalisation prologue of
 * kda_chunk_fwd_prologue (same formulas: q and k divided by sqrt(|x|^2 + 1e-6)
 * over dk and rounded to the input precision, g = max(-5, -softplus(g_raw)),
 * beta = sigmoid(beta_raw)) applied inside the step.  Arguments, layouts and codes
 * are those of kda_decode_step, with the raw tensors in place of q, k, g and beta.
 * Same result as kda_chunk_fwd_prologue with T = 1 and final_state == initial_state.
 */
int kda_decode_step_prologue(const void* q_raw, const void* k_raw, const void* v,
                             const void* g_raw, const void* beta_raw, float* state, void* out,
                             int B, int H, int dk, int dv, float scale, int dtype,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
