// C ABI of libkda.so: argument checks, then one kernel launch on the caller's
// stream.  The contract of every entry point is documented in include/kda.h.

#include "kda.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <initializer_list>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "kda_launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, -1 = another architecture.
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_NO_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KDA_ERR_HIP;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? KDA_OK : KDA_ERR_NO_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_common(int dk, int dv, int H, int dtype) {
  if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_DTYPE;
  if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_HEAD_DIM;
  if (H <= 0) return KDA_ERR_SHAPE;
  return KDA_OK;
}

struct PtrReq {
  const void* p;
  uintptr_t align;
  bool required;
};

int check_ptrs(std::initializer_list<PtrReq> ptrs) {
  for (const PtrReq& r : ptrs) {
    if (r.p == nullptr) {
      if (r.required) return KDA_ERR_NULL;
      continue;
    }
    if (!aligned(r.p, r.align)) return KDA_ERR_ALIGN;
  }
  return KDA_OK;
}

// Prefill pointer rules: q, k, g are read two elements at a time (4 bytes),
// beta one element at a time, v and out 16 bytes at a time, states as fp32.
int check_prefill_ptrs(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const void* s0, const void* out, const void* sT,
                       int dtype) {
  const uintptr_t elt = dtype == KDA_F32 ? 4 : 2;
  return check_ptrs({{q, 4, true}, {k, 4, true}, {g, 4, true}, {beta, elt, true},
                     {v, 16, true}, {out, 16, true}, {s0, 4, false}, {sT, 4, false}});
}

// One workspace pool per device, created on first use and kept for the process.
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxDevices];

hipError_t device_pool(hipMemPool_t* out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (g_pool[dev] == nullptr) {
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    err = hipMemPoolCreate(&pool, &props);
    if (err != hipSuccess) return err;
    uint64_t keep = UINT64_MAX;
    err = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (err != hipSuccess) {
      hipMemPoolDestroy(pool);
      return err;
    }
    g_pool[dev] = pool;
  }
  *out = g_pool[dev];
  return hipSuccess;
}

// Workspace blocks kept for reuse.  A call takes a free block of its device that
// is large enough, after making its stream wait for the event recorded when the
// block was last released (on whatever stream that was), or else allocates a new
// block from the pool; releasing records that event and keeps the block.  No call
// therefore frees memory (hipFreeAsync blocks the host on ROCm 7 until the stream
// has drained), except free blocks too small for a request, which are returned to
// the pool when a larger one is allocated.  Blocks live until the process ends.
struct WsBlock {
  void* p;
  size_t bytes;
  int dev;
  bool busy;
  bool used;          // `done` has been recorded
  hipEvent_t done;
  hipStream_t last;   // stream of the last release
};
std::mutex g_ws_mu;
std::vector<WsBlock> g_ws;

}  // namespace

namespace kda {

hipError_t ws_alloc(void** p, size_t bytes, hipStream_t stream) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  hipMemPool_t pool = nullptr;
  err = device_pool(&pool);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int best = -1;
  for (int i = 0; i < static_cast<int>(g_ws.size()); ++i) {
    const WsBlock& b = g_ws[i];
    if (b.busy || b.dev != dev || b.bytes < bytes) continue;
    // prefer the block last used on this stream, then the smallest
    if (best < 0 || (b.last == stream && g_ws[best].last != stream) ||
        ((b.last == stream) == (g_ws[best].last == stream) && b.bytes < g_ws[best].bytes))
      best = i;
  }
  if (best >= 0) {
    WsBlock& b = g_ws[best];
    if (b.used && (err = hipStreamWaitEvent(stream, b.done, 0)) != hipSuccess) return err;
    b.busy = true;
    *p = b.p;
    return hipSuccess;
  }
  // free blocks of this device are all too small: give them back, then allocate
  for (int i = static_cast<int>(g_ws.size()) - 1; i >= 0; --i) {
    WsBlock& b = g_ws[i];
    if (b.busy || b.dev != dev) continue;
    if (b.used && (err = hipStreamWaitEvent(stream, b.done, 0)) != hipSuccess) return err;
    if ((err = hipFreeAsync(b.p, stream)) != hipSuccess) return err;
    hipEventDestroy(b.done);
    g_ws.erase(g_ws.begin() + i);
  }
  WsBlock nb{nullptr, bytes, dev, true, false, nullptr, stream};
  if ((err = hipEventCreateWithFlags(&nb.done, hipEventDisableTiming)) != hipSuccess) return err;
  if ((err = hipMallocFromPoolAsync(&nb.p, bytes, pool, stream)) != hipSuccess) {
    hipEventDestroy(nb.done);
    return err;
  }
  g_ws.push_back(nb);
  *p = nb.p;
  return hipSuccess;
}

hipError_t ws_free(void* p, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  for (WsBlock& b : g_ws) {
    if (b.p != p || !b.busy) continue;
    const hipError_t err = hipEventRecord(b.done, stream);
    if (err != hipSuccess) return err;   // the block stays taken: never reused unordered
    b.busy = false;
    b.used = true;
    b.last = stream;
    return hipSuccess;
  }
  return hipErrorInvalidValue;
}

}  // namespace kda

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is non-positive or too large";
    case KDA_ERR_HEAD_DIM: return "dk and dv must be equal and 64 or 128 (64 for fp32 prefill)";
    case KDA_ERR_DTYPE: return "dtype must be KDA_BF16 or KDA_F32";
    case KDA_ERR_ALIGN: return "a pointer is not aligned as required";
    case KDA_ERR_HIP: return "the HIP runtime reported an error";
    case KDA_ERR_NO_DEVICE: return "the current device is not gfx950";
    case KDA_ERR_WORKSPACE: return "the workspace is NULL, not 256-byte aligned or too small";
    default: return "unknown status";
  }
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* initial_state, void* out,
                  float* final_state, int B, int T, int H, int dk, int dv, float scale,
                  int dtype, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype == KDA_F32 && dk != 64) return KDA_ERR_HEAD_DIM;
  if (B <= 0 || T <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > (1 << 24)) return KDA_ERR_SHAPE;
  rc = check_prefill_ptrs(q, k, v, g, beta, initial_state, out, final_state, dtype);
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a{q, k, v, g, beta, initial_state, out, final_state, nullptr,
                     B, T, B * T, H, dk, scale, dtype == KDA_F32, stream};
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype) {
  if (check_common(dk, dv, H, dtype) != KDA_OK) return 0;
  if (dtype == KDA_F32 && dk != 64) return 0;
  if (B <= 0 || T <= 0) return 0;
  if (static_cast<int64_t>(B) * T > INT32_MAX / 2) return 0;
  if (static_cast<int64_t>(B) * H > (1 << 24)) return 0;
  kda::PrefillArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     B, T, B * T, H, dk, 1.f, dtype == KDA_F32, nullptr};
  return kda::prefill_workspace_bytes(a);
}

const char* kda_chunk_fwd_schedule(int N, int T, int total_T, int H, int dk, int dv, int dtype,
                                   int varlen) {
  if (check_common(dk, dv, H, dtype) != KDA_OK || N <= 0) return "";
  if (varlen ? total_T <= 0 : T <= 0) return "";
  kda::PrefillArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     varlen ? reinterpret_cast<const int32_t*>(uintptr_t{16}) : nullptr,
                     N, varlen ? 0 : T, varlen ? total_T : N * T, H, dk, 1.f, dtype == KDA_F32,
                     nullptr};
  return kda::prefill_schedule(a);
}

int kda_chunk_fwd_ws(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* initial_state, void* out,
                     float* final_state, int B, int T, int H, int dk, int dv, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype == KDA_F32 && dk != 64) return KDA_ERR_HEAD_DIM;
  if (B <= 0 || T <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > (1 << 24)) return KDA_ERR_SHAPE;
  rc = check_prefill_ptrs(q, k, v, g, beta, initial_state, out, final_state, dtype);
  if (rc != KDA_OK) return rc;
  if (workspace == nullptr || !aligned(workspace, 256) ||
      workspace_bytes < kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype))
    return KDA_ERR_WORKSPACE;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a{q, k, v, g, beta, initial_state, out, final_state, nullptr,
                     B, T, B * T, H, dk, scale, dtype == KDA_F32, stream};
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd_prologue(const void* q_raw, const void* k_raw, const void* v,
                           const void* g_raw, const void* beta_raw, const float* initial_state,
                           void* out, float* final_state, int B, int T, int H, int dk, int dv,
                           float scale, int dtype, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype == KDA_F32 && dk != 64) return KDA_ERR_HEAD_DIM;
  if (B <= 0 || T <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > (1 << 24)) return KDA_ERR_SHAPE;
  rc = check_prefill_ptrs(q_raw, k_raw, v, g_raw, beta_raw, initial_state, out, final_state, dtype);
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a{q_raw, k_raw, v, g_raw, beta_raw, initial_state, out, final_state, nullptr,
                     B, T, B * T, H, dk, scale, dtype == KDA_F32, stream};
  a.prologue = true;
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, void* out,
                            float* final_state, float* snapshots, int snapshot_tokens, int B,
                            int T, int H, int dk, int dv, float scale, int dtype,
                            hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype == KDA_F32 && dk != 64) return KDA_ERR_HEAD_DIM;
  if (B <= 0 || T <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > (1 << 24)) return KDA_ERR_SHAPE;
  if (snapshot_tokens <= 0 || snapshot_tokens % 64 != 0) return KDA_ERR_SHAPE;
  if (snapshots == nullptr) return KDA_ERR_NULL;
  rc = check_prefill_ptrs(q, k, v, g, beta, initial_state, out, final_state, dtype);
  if (rc == KDA_OK && !aligned(snapshots, 4)) rc = KDA_ERR_ALIGN;
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a{q, k, v, g, beta, initial_state, out, final_state, nullptr,
                     B, T, B * T, H, dk, scale, dtype == KDA_F32, stream};
  a.snapshots = snapshots;
  a.snap_chunks = snapshot_tokens / 64;
  a.nsnap = (T + snapshot_tokens - 1) / snapshot_tokens;
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, void* out,
                         float* final_state, const int32_t* cu_seqlens, int N,
                         int total_T, int H, int dk, int dv, float scale, int dtype,
                         hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype == KDA_F32 && dk != 64) return KDA_ERR_HEAD_DIM;
  if (N <= 0 || total_T <= 0 || total_T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(N) * H > (1 << 24)) return KDA_ERR_SHAPE;
  if (cu_seqlens == nullptr) return KDA_ERR_NULL;
  rc = check_prefill_ptrs(q, k, v, g, beta, initial_state, out, final_state, dtype);
  if (rc == KDA_OK && !aligned(cu_seqlens, 4)) rc = KDA_ERR_ALIGN;
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a{q, k, v, g, beta, initial_state, out, final_state, cu_seqlens,
                     N, 0, total_T, H, dk, scale, dtype == KDA_F32, stream};
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd_varlen_prologue(const void* q_raw, const void* k_raw, const void* v,
                                  const void* g_raw, const void* beta_raw,
                                  const float* initial_state, void* out, float* final_state,
                                  const int32_t* cu_seqlens, int N, int total_T, int H, int dk,
                                  int dv, float scale, int dtype, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype == KDA_F32 && dk != 64) return KDA_ERR_HEAD_DIM;
  if (N <= 0 || total_T <= 0 || total_T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(N) * H > (1 << 24)) return KDA_ERR_SHAPE;
  if (cu_seqlens == nullptr) return KDA_ERR_NULL;
  rc = check_prefill_ptrs(q_raw, k_raw, v, g_raw, beta_raw, initial_state, out, final_state, dtype);
  if (rc == KDA_OK && !aligned(cu_seqlens, 4)) rc = KDA_ERR_ALIGN;
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a{q_raw, k_raw, v, g_raw, beta_raw, initial_state, out, final_state, cu_seqlens,
                     N, 0, total_T, H, dk, scale, dtype == KDA_F32, stream};
  a.prologue = true;
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd_varlen_snapshots(const void* q, const void* k, const void* v, const void* g,
                                   const void* beta, const float* initial_state, void* out,
                                   float* final_state, float* snapshots, int snapshot_tokens,
                                   const int32_t* cu_seqlens, int N, int total_T, int H, int dk,
                                   int dv, float scale, int dtype, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype == KDA_F32 && dk != 64) return KDA_ERR_HEAD_DIM;
  if (N <= 0 || total_T <= 0 || total_T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(N) * H > (1 << 24)) return KDA_ERR_SHAPE;
  if (snapshot_tokens <= 0 || snapshot_tokens % 64 != 0) return KDA_ERR_SHAPE;
  if (cu_seqlens == nullptr || snapshots == nullptr) return KDA_ERR_NULL;
  rc = check_prefill_ptrs(q, k, v, g, beta, initial_state, out, final_state, dtype);
  if (rc == KDA_OK && (!aligned(cu_seqlens, 4) || !aligned(snapshots, 4))) rc = KDA_ERR_ALIGN;
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a{q, k, v, g, beta, initial_state, out, final_state, cu_seqlens,
                     N, 0, total_T, H, dk, scale, dtype == KDA_F32, stream};
  a.snapshots = snapshots;
  a.snap_chunks = snapshot_tokens / 64;
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  const float* initial_state, const void* grad_out,
                  const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v,
                  void* grad_g, void* grad_beta, float* grad_initial_state, int B, int T, int H,
                  int dk, int dv, float scale, int dtype, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (B <= 0 || T <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > (1 << 24)) return KDA_ERR_SHAPE;
  const uintptr_t elt = dtype == KDA_F32 ? 4 : 2;
  rc = check_ptrs({{q, 16, true}, {k, 16, true}, {v, 16, true}, {g, 16, true},
                   {beta, elt, true}, {grad_out, 16, true}, {grad_q, elt, true},
                   {grad_k, elt, true}, {grad_v, elt, true}, {grad_g, elt, true},
                   {grad_beta, elt, true}, {initial_state, 4, false},
                   {grad_final_state, 4, false}, {grad_initial_state, 4, false}});
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::BackwardArgs a{q, k, v, g, beta, initial_state, grad_out, grad_final_state,
                      grad_q, grad_k, grad_v, grad_g, grad_beta, grad_initial_state,
                      B, T, H, dk, scale, dtype == KDA_F32, stream};
  return kda::launch_backward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, const void* grad_out,
                         const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v,
                         void* grad_g, void* grad_beta, float* grad_initial_state,
                         const int32_t* cu_seqlens, int N, int total_T, int H, int dk, int dv,
                         float scale, int dtype, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (N <= 0 || total_T <= 0 || total_T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(N) * H > (1 << 24)) return KDA_ERR_SHAPE;
  if ((static_cast<int64_t>(total_T) / 64 + N + 1) * H > INT32_MAX) return KDA_ERR_SHAPE;
  if (cu_seqlens == nullptr) return KDA_ERR_NULL;
  const uintptr_t elt = dtype == KDA_F32 ? 4 : 2;
  rc = check_ptrs({{q, 16, true}, {k, 16, true}, {v, 16, true}, {g, 16, true},
                   {beta, elt, true}, {grad_out, 16, true}, {grad_q, elt, true},
                   {grad_k, elt, true}, {grad_v, elt, true}, {grad_g, elt, true},
                   {grad_beta, elt, true}, {initial_state, 4, false},
                   {grad_final_state, 4, false}, {grad_initial_state, 4, false},
                   {cu_seqlens, 4, true}});
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::BackwardArgs a{q, k, v, g, beta, initial_state, grad_out, grad_final_state,
                      grad_q, grad_k, grad_v, grad_g, grad_beta, grad_initial_state,
                      N, 0, H, dk, scale, dtype == KDA_F32, stream};
  a.cu_seqlens = cu_seqlens;
  a.total_T = total_T;
  return kda::launch_backward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_transition(const void* q, const void* k, const void* g, const void* beta,
                         float* transition, int B, int T, int H, int dk, int dv, int dtype,
                         hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (B <= 0 || T <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * T > INT32_MAX / 2) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > (1 << 24)) return KDA_ERR_SHAPE;
  const uintptr_t elt = dtype == KDA_F32 ? 4 : 2;
  rc = check_ptrs({{q, 16, false}, {k, 16, true}, {g, 16, true}, {beta, elt, true},
                   {transition, 4, true}});
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::TransitionArgs a{q, k, g, beta, transition, B, T, H, dk, dtype == KDA_F32, stream};
  return kda::launch_transition(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_state_compose(const float* transitions, const float* partial_states,
                      const float* initial_state, float* entry_states, int R, int B, int H,
                      int dk, int dv, hipStream_t stream) {
  int rc = check_common(dk, dv, H, KDA_F32);
  if (rc != KDA_OK) return rc;
  if (R <= 0 || B <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > (1 << 24)) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(R + 1) * B * H * dk * dv > (int64_t{1} << 40)) return KDA_ERR_SHAPE;
  rc = check_ptrs({{transitions, 16, true}, {partial_states, 16, true},
                   {initial_state, 16, false}, {entry_states, 16, true}});
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::ComposeArgs a{transitions, partial_states, initial_state, entry_states, R, B, H, dk, stream};
  return kda::launch_compose(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, float* state, void* out, int B, int H, int dk, int dv,
                    float scale, int dtype, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (B <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > INT32_MAX / 2) return KDA_ERR_SHAPE;
  const uintptr_t elt = dtype == KDA_F32 ? 4 : 2;
  rc = check_ptrs({{q, elt, true}, {k, elt, true}, {v, elt, true}, {g, elt, true},
                   {beta, elt, true}, {state, 16, true}, {out, elt, true}});
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::DecodeArgs a{q, k, v, g, beta, state, out, B, H, dk, scale, dtype == KDA_F32, stream};
  return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step_prologue(const void* q_raw, const void* k_raw, const void* v,
                             const void* g_raw, const void* beta_raw, float* state, void* out,
                             int B, int H, int dk, int dv, float scale, int dtype,
                             hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (B <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H > INT32_MAX / 2) return KDA_ERR_SHAPE;
  const uintptr_t elt = dtype == KDA_F32 ? 4 : 2;
  rc = check_ptrs({{q_raw, elt, true}, {k_raw, elt, true}, {v, elt, true}, {g_raw, elt, true},
                   {beta_raw, elt, true}, {state, 16, true}, {out, elt, true}});
  if (rc != KDA_OK) return rc;
  rc = check_device();
  if (rc != KDA_OK) return rc;
  kda::DecodeArgs a{q_raw, k_raw, v, g_raw, beta_raw, state, out, B, H, dk, scale,
                    dtype == KDA_F32, stream};
  a.prologue = true;
  return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
