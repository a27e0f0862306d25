// Internal launcher interface between the C ABI shim and the HIP kernels.
// Arguments arrive here already validated by kda_api.cpp.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
  const void *q, *k, *v, *g, *beta;
  float* state;
  void* out;
  int B, H, d;
  float scale;
  bool dtype_f32;
  hipStream_t stream;
  bool prologue = false;       // q, k, g, beta raw: normalise / gate in the kernel
};

struct PrefillArgs {
  const void *q, *k, *v, *g, *beta;
  const float* initial_state;  // may be null
  void* out;
  float* final_state;          // may be null; may alias initial_state
  const int32_t* cu_seqlens;   // device offsets (varlen) or null (fixed length)
  int N;                       // sequences
  int T;                       // tokens per sequence (fixed length)
  int total_T;                 // tokens in the packed buffers
  int H, d;
  float scale;
  bool dtype_f32;
  hipStream_t stream;
  float* snapshots = nullptr;  // [N, H, nsnap, d, d] (fixed length), [sum_n nsnap_n, H, d, d]
                               // (varlen), or null
  int snap_chunks = 0;         // snapshot every snap_chunks chunks (and at the end)
  int nsnap = 0;
  bool prologue = false;       // q, k, g, beta raw: normalise / gate in the kernel
  void* workspace = nullptr;   // caller's workspace (null: the call allocates its own)
  size_t workspace_bytes = 0;
  int window_chunks = 0;       // > 0: fixed length runs in windows of this many chunks
};

struct BackwardArgs {
  const void *q, *k, *v, *g, *beta;
  const float* initial_state;   // may be null (zero)
  const void* d_out;            // cotangent of out, same layout and dtype as v
  const float* d_final_state;   // may be null (zero)
  void *dq, *dk, *dv, *dg, *dbeta;
  float* d_initial_state;       // may be null (not written)
  int B, T, H, d;
  float scale;
  bool dtype_f32;
  hipStream_t stream;
  const int32_t* cu_seqlens = nullptr;   // packed sequences: B offsets + 1 (device); T unused
  int total_T = 0;                       // tokens in the packed buffers
  void* workspace = nullptr;             // caller's workspace (null: the call takes a block)
  size_t workspace_bytes = 0;
  int window_chunks = 0;                 // > 0: run in windows of this many chunks
};

struct TransitionArgs {
  const void *q, *k, *g, *beta;
  float* transition;            // [B, H, d, d]
  int B, T, H, d;
  bool dtype_f32;
  hipStream_t stream;
  void* workspace = nullptr;    // caller's workspace (null: the call takes a block)
  size_t workspace_bytes = 0;
};

struct ComposeArgs {
  const float* transitions;     // [R, B, H, d, d]
  const float* partial_states;  // [R, B, H, d, d]
  const float* initial_state;   // [B, H, d, d] or null (zero)
  float* entry_states;          // [R + 1, B, H, d, d]
  int R, B, H, d;
  hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_transition(const TransitionArgs& a);
hipError_t launch_compose(const ComposeArgs& a);
hipError_t launch_backward(const BackwardArgs& a);
// Workspace bytes launch_backward / launch_transition need for these arguments.
size_t backward_workspace_bytes(const BackwardArgs& a);
// fp32 prefill at d = 128 (kda_prefill_fp32.hip): chunk operands of kda_chunk_ops.h
// and a scan that writes the outputs, in windows of chunks.
bool exact_prefill_path(const PrefillArgs& a);
size_t exact_prefill_workspace_bytes(const PrefillArgs& a);
int exact_prefill_fit_window(const PrefillArgs& a, size_t bytes);
const char* exact_prefill_schedule(const PrefillArgs& a);
hipError_t launch_exact_prefill(const PrefillArgs& a);
// Largest window (chunks) whose backward workspace fits in `bytes`: 0 when the whole
// call fits, -1 when not even one-chunk windows do.
int backward_fit_window(const BackwardArgs& a, size_t bytes);
size_t transition_workspace_bytes(const TransitionArgs& a);

hipError_t launch_prefill(const PrefillArgs& a);
// Fused prefill (one workgroup per (sequence, head), no workspace): bf16, d = 128,
// without the prologue or snapshots.
bool fused_prefill_supported(const PrefillArgs& a);
hipError_t launch_fused_prefill(const PrefillArgs& a);
// The same kernel over R segments of every fixed-length sequence (R >= 2): exit
// states and transitions of the first R - 1 segments, their composition into entry
// states, then every segment's output; fused_segmented_bytes of workspace.
size_t fused_segmented_bytes(const PrefillArgs& a, int R);
hipError_t launch_fused_segmented(const PrefillArgs& a, int R);
// Transitions with the fused kernel (bf16, d = 128, 256 or more (segment, head)
// streams; no workspace).
bool fused_transition_supported(const TransitionArgs& a);
hipError_t launch_fused_transition(const TransitionArgs& a);
// Kernels launch_prefill runs for these arguments (static text, for reports).
const char* prefill_schedule(const PrefillArgs& a);
// Workspace bytes launch_prefill needs for these arguments (0 if unsupported).
size_t prefill_workspace_bytes(const PrefillArgs& a);
// Longest window (in chunks) whose workspace fits in max_bytes, for fixed-length
// input off the fused schedule; 0 when not even one-chunk windows fit.
int prefill_fit_window(const PrefillArgs& a, size_t max_bytes);

// The file-scope scratch array of the allocation-free prefill (kda_noalloc.hip): its
// size, and its address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** p);

// Workspace blocks the library keeps for the calls that take no workspace (see
// kda_api.cpp): ws_alloc takes a block of at least `bytes` for work enqueued on
// `stream`, ws_free gives it back once that work has been enqueued.
hipError_t ws_alloc(void** p, size_t bytes, hipStream_t stream);
hipError_t ws_free(void* p, hipStream_t stream);

// The caller's workspace when there is one (too small: invalid value), else a block
// from ws_alloc; ws_release gives back what ws_acquire took.
inline hipError_t ws_acquire(void* caller, size_t caller_bytes, size_t need, hipStream_t stream,
                             char** p) {
  if (need == 0) {
    *p = nullptr;
    return hipSuccess;
  }
  if (caller != nullptr) {
    if (caller_bytes < need) return hipErrorInvalidValue;
    *p = static_cast<char*>(caller);
    return hipSuccess;
  }
  return ws_alloc(reinterpret_cast<void**>(p), need, stream);
}
inline hipError_t ws_release(void* caller, char* p, hipStream_t stream) {
  return caller != nullptr || p == nullptr ? hipSuccess : ws_free(p, stream);
}

// Launch a kernel unless an earlier step of the call failed, and record the launch's
// own error: a call stops at its first failed launch.
#define KDA_TRY_LAUNCH(err, ...)          \
  do {                                    \
    if ((err) == hipSuccess) {            \
      hipLaunchKernelGGL(__VA_ARGS__);    \
      (err) = hipGetLastError();          \
    }                                     \
  } while (0)

}  // namespace kda
