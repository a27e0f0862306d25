// C ABI of libkda.so: argument checks, then the kernel launches on the caller's
// stream.  The contract of every entry point is documented in include/kda.h.

#include "kda.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "kda_launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, -1 = another architecture.
std::atomic<int> g_arch_ok[kMaxDevices];

// The current device is gfx950.  Runs right before a call's first launch; it also
// clears an error an earlier HIP call left pending on this thread, so that a launch
// check reports this call's own launches only.
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
  if (state != 1) return KDA_ERR_NO_DEVICE;
  (void)hipGetLastError();
  return KDA_OK;
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

// Sizes of a fixed-length (B sequences of T tokens) or packed (N sequences, total_T
// tokens) call.
int check_sizes(bool packed, int N, int T, int total_T, int H) {
  if (N <= 0) return KDA_ERR_SHAPE;
  if (static_cast<int64_t>(N) * H > (1 << 24)) return KDA_ERR_SHAPE;
  if (packed) {
    if (total_T <= 0 || total_T > INT32_MAX / 2) return KDA_ERR_SHAPE;
    if ((static_cast<int64_t>(total_T) / 64 + N + 1) * H > INT32_MAX) return KDA_ERR_SHAPE;
  } else {
    if (T <= 0 || static_cast<int64_t>(N) * T > INT32_MAX / 2) return KDA_ERR_SHAPE;
    if (static_cast<int64_t>(N) * ((T + 63) / 64) * H > INT32_MAX) return KDA_ERR_SHAPE;
  }
  return KDA_OK;
}

// Everything a prefill call is checked for, except the workspace and the device.
int check_prefill(const kda_prefill_desc& d) {
  int rc = check_common(d.dk, d.dv, d.H, d.dtype);
  if (rc != KDA_OK) return rc;
  // fp32 at d = 128 has the plain forms only (no gate prologue, no snapshots)
  if (d.dtype == KDA_F32 && d.dk != 64 && (d.prologue != 0 || d.snapshots != nullptr ||
                                           d.snapshot_tokens != 0))
    return KDA_ERR_HEAD_DIM;
  const bool packed = d.cu_seqlens != nullptr;
  rc = check_sizes(packed, d.N, d.T, d.total_T, d.H);
  if (rc != KDA_OK) return rc;
  if (d.snapshots != nullptr || d.snapshot_tokens != 0) {
    if (d.snapshot_tokens <= 0 || d.snapshot_tokens % 64 != 0) return KDA_ERR_SHAPE;
    if (d.snapshots == nullptr) return KDA_ERR_NULL;
  }
  // q, k, g are read two elements at a time (4 bytes), beta one element at a time,
  // v and out 16 bytes at a time, states and snapshots as fp32
  const uintptr_t elt = d.dtype == KDA_F32 ? 4 : 2;
  return check_ptrs({{d.q, 4, true}, {d.k, 4, true}, {d.g, 4, true}, {d.beta, elt, true},
                     {d.v, 16, true}, {d.out, 16, true}, {d.initial_state, 4, false},
                     {d.final_state, 4, false}, {d.snapshots, 4, false},
                     {d.cu_seqlens, 4, false}});
}

kda::PrefillArgs prefill_args(const kda_prefill_desc& d, hipStream_t stream) {
  const bool packed = d.cu_seqlens != nullptr;
  kda::PrefillArgs a{d.q, d.k, d.v, d.g, d.beta, d.initial_state, d.out, d.final_state,
                     d.cu_seqlens, d.N, packed ? 0 : d.T, packed ? d.total_T : d.N * d.T, d.H,
                     d.dk, d.scale, d.dtype == KDA_F32, stream};
  a.prologue = d.prologue != 0;
  if (d.snapshots != nullptr) {
    a.snapshots = d.snapshots;
    a.snap_chunks = d.snapshot_tokens / 64;
    a.nsnap = packed ? 0 : (d.T + d.snapshot_tokens - 1) / d.snapshot_tokens;
  }
  return a;
}

// A checked prefill: with `caller_ws` the call runs on the caller's workspace (which
// must be large enough) and allocates nothing; without, it takes a kept block.
int run_prefill(const kda_prefill_desc& d, bool caller_ws, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  int rc = check_prefill(d);
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a = prefill_args(d, stream);
  if (caller_ws && kda::exact_prefill_path(a)) {
    // fp32 at d = 128 runs in windows of chunks: the largest that fit the workspace
    if (workspace == nullptr || !aligned(workspace, 256)) return KDA_ERR_WORKSPACE;
    const int cw = kda::prefill_fit_window(a, workspace_bytes);
    if (cw <= 0) return KDA_ERR_WORKSPACE;
    a.window_chunks = cw;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
  } else if (caller_ws) {
    const size_t need = kda::prefill_workspace_bytes(a);
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need))
      return KDA_ERR_WORKSPACE;
    if (need > 0) {
      a.workspace = workspace;
      a.workspace_bytes = workspace_bytes;
    }
  }
  rc = check_device();
  if (rc != KDA_OK) return rc;
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_prefill_desc fixed_desc(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* s0, void* out, float* sT, int B,
                            int T, int H, int dk, int dv, float scale, int dtype) {
  kda_prefill_desc d;
  std::memset(&d, 0, sizeof d);
  d.q = q; d.k = k; d.v = v; d.g = g; d.beta = beta;
  d.initial_state = s0; d.out = out; d.final_state = sT;
  d.N = B; d.T = T; d.H = H; d.dk = dk; d.dv = dv; d.scale = scale; d.dtype = dtype;
  return d;
}

kda_prefill_desc packed_desc(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, const float* s0, void* out, float* sT,
                             const int32_t* cu, int N, int total_T, int H, int dk, int dv,
                             float scale, int dtype) {
  kda_prefill_desc d = fixed_desc(q, k, v, g, beta, s0, out, sT, N, 0, H, dk, dv, scale, dtype);
  d.cu_seqlens = cu;
  d.total_T = total_T;
  return d;
}

// The code a packed call without offsets returns: size and head errors first, as a
// call with offsets would report them, else KDA_ERR_NULL.
int packed_without_offsets(int N, int total_T, int H, int dk, int dv, int dtype) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc == KDA_OK) rc = check_sizes(true, N, 0, total_T, H);
  return rc != KDA_OK ? rc : KDA_ERR_NULL;
}

// Snapshot tokens out of range: the checks that come before, else KDA_ERR_SHAPE.
int bad_snapshot_tokens(const kda_prefill_desc& d) {
  int rc = check_common(d.dk, d.dv, d.H, d.dtype);
  if (rc == KDA_OK && d.dtype == KDA_F32 && d.dk != 64) rc = KDA_ERR_HEAD_DIM;
  if (rc == KDA_OK) rc = check_sizes(d.cu_seqlens != nullptr, d.N, d.T, d.total_T, d.H);
  return rc != KDA_OK ? rc : KDA_ERR_SHAPE;
}

// ---------------------------------------------------------------- kept workspace blocks

// One memory pool per device, created on first use and kept for the process.
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
      (void)hipMemPoolDestroy(pool);
      return err;
    }
    g_pool[dev] = pool;
  }
  *out = g_pool[dev];
  return hipSuccess;
}

// Workspace blocks for the entry points that take no workspace.  A call takes a free
// block of its device that is large enough, after making its stream wait for the
// event recorded when the block was last released (on whatever stream that was), or
// else allocates a new block from the device's pool; releasing records that event
// and keeps the block.  Free blocks of a device are kept while they total at most
// kKeepBytes; beyond that the largest free blocks are returned to the pool
// (hipFreeAsync, ordered after their last use).  Blocks too small for a request are
// returned the same way when a larger one is allocated.
constexpr size_t kKeepBytes = size_t{4} << 30;

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

// Return free block i to the pool on `stream`, after its last use.  Caller holds g_ws_mu.
hipError_t drop_block(int i, hipStream_t stream) {
  WsBlock& b = g_ws[i];
  hipError_t err = hipSuccess;
  if (b.used) err = hipStreamWaitEvent(stream, b.done, 0);
  if (err == hipSuccess) err = hipFreeAsync(b.p, stream);
  (void)hipEventDestroy(b.done);
  g_ws.erase(g_ws.begin() + i);
  return err;
}

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
    if (g_ws[i].busy || g_ws[i].dev != dev) continue;
    if ((err = drop_block(i, stream)) != hipSuccess) return err;
  }
  WsBlock nb{nullptr, bytes, dev, true, false, nullptr, stream};
  if ((err = hipEventCreateWithFlags(&nb.done, hipEventDisableTiming)) != hipSuccess) return err;
  if ((err = hipMallocFromPoolAsync(&nb.p, bytes, pool, stream)) != hipSuccess) {
    (void)hipEventDestroy(nb.done);
    return err;
  }
  g_ws.push_back(nb);
  *p = nb.p;
  return hipSuccess;
}

hipError_t ws_free(void* p, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  for (int i = 0; i < static_cast<int>(g_ws.size()); ++i) {
    WsBlock& b = g_ws[i];
    if (b.p != p || !b.busy) continue;
    const hipError_t err = hipEventRecord(b.done, stream);
    if (err != hipSuccess) {
      // the block's last use cannot be ordered by its event: return it to the pool
      // on the stream instead, after the work enqueued there
      (void)hipFreeAsync(b.p, stream);
      (void)hipEventDestroy(b.done);
      g_ws.erase(g_ws.begin() + i);
      return err;
    }
    b.busy = false;
    b.used = true;
    b.last = stream;
    const int dev = b.dev;
    // keep at most kKeepBytes of free blocks on this device: give back the largest
    for (;;) {
      size_t kept = 0;
      int largest = -1;
      for (int j = 0; j < static_cast<int>(g_ws.size()); ++j) {
        if (g_ws[j].busy || g_ws[j].dev != dev) continue;
        kept += g_ws[j].bytes;
        if (largest < 0 || g_ws[j].bytes > g_ws[largest].bytes) largest = j;
      }
      if (kept <= kKeepBytes || largest < 0) break;
      const hipError_t derr = drop_block(largest, stream);
      if (derr != hipSuccess) return derr;
    }
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
    case KDA_ERR_HEAD_DIM:
      return "dk and dv must be equal and 64 or 128 (64 for the fp32 prologue and snapshot forms)";
    case KDA_ERR_DTYPE: return "dtype must be KDA_BF16 or KDA_F32";
    case KDA_ERR_ALIGN: return "a pointer is not aligned as required";
    case KDA_ERR_HIP: return "the HIP runtime reported an error";
    case KDA_ERR_NO_DEVICE: return "the current device is not gfx950";
    case KDA_ERR_WORKSPACE: return "the workspace is NULL, not 256-byte aligned or too small";
    default: return "unknown status";
  }
}

// ---------------------------------------------------------------- prefill

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

int kda_prefill_workspace_size(const kda_prefill_desc* desc, size_t* bytes) {
  if (desc == nullptr || bytes == nullptr) return KDA_ERR_NULL;
  const int rc = check_prefill(*desc);
  if (rc != KDA_OK) return rc;
  *bytes = kda::prefill_workspace_bytes(prefill_args(*desc, nullptr));
  return KDA_OK;
}

int kda_prefill(const kda_prefill_desc* desc, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  if (desc == nullptr) return KDA_ERR_NULL;
  return run_prefill(*desc, true, workspace, workspace_bytes, stream);
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* initial_state, void* out,
                  float* final_state, int B, int T, int H, int dk, int dv, float scale,
                  int dtype, hipStream_t stream) {
  return run_prefill(fixed_desc(q, k, v, g, beta, initial_state, out, final_state, B, T, H, dk,
                                dv, scale, dtype),
                     false, nullptr, 0, stream);
}

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype) {
  // sizes only: stand-in pointers satisfy the pointer checks and are never used
  const void* p = reinterpret_cast<const void*>(uintptr_t{256});
  kda_prefill_desc d = fixed_desc(p, p, p, p, p, nullptr, const_cast<void*>(p), nullptr, B, T,
                                  H, dk, dv, 1.f, dtype);
  size_t bytes = 0;
  return kda_prefill_workspace_size(&d, &bytes) == KDA_OK ? bytes : 0;
}

int kda_chunk_fwd_ws(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* initial_state, void* out,
                     float* final_state, int B, int T, int H, int dk, int dv, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_prefill(fixed_desc(q, k, v, g, beta, initial_state, out, final_state, B, T, H, dk,
                                dv, scale, dtype),
                     true, workspace, workspace_bytes, stream);
}

int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* initial_state, void* out,
                          float* final_state, int B, int T, int H, int dk, int dv, float scale,
                          int dtype, hipStream_t stream) {
  const kda_prefill_desc d = fixed_desc(q, k, v, g, beta, initial_state, out, final_state, B, T,
                                        H, dk, dv, scale, dtype);
  int rc = check_prefill(d);
  if (rc != KDA_OK) return rc;
  kda::PrefillArgs a = prefill_args(d, stream);
  if (kda::prefill_workspace_bytes(a) > kda::noalloc_scratch_bytes()) {
    // windows short enough for the scratch array; none fit: refused before any device call
    const int cg = kda::prefill_fit_window(a, kda::noalloc_scratch_bytes());
    if (cg <= 0) return KDA_ERR_WORKSPACE;
    a.window_chunks = cg;
  }
  rc = check_device();
  if (rc != KDA_OK) return rc;
  if (kda::prefill_workspace_bytes(a) > 0) {
    void* ptr = nullptr;
    if (kda::noalloc_scratch(&ptr) != hipSuccess) return KDA_ERR_HIP;
    a.workspace = ptr;
    a.workspace_bytes = kda::noalloc_scratch_bytes();
  }
  return kda::launch_prefill(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd_prologue(const void* q_raw, const void* k_raw, const void* v,
                           const void* g_raw, const void* beta_raw, const float* initial_state,
                           void* out, float* final_state, int B, int T, int H, int dk, int dv,
                           float scale, int dtype, hipStream_t stream) {
  kda_prefill_desc d = fixed_desc(q_raw, k_raw, v, g_raw, beta_raw, initial_state, out,
                                  final_state, B, T, H, dk, dv, scale, dtype);
  d.prologue = 1;
  return run_prefill(d, false, nullptr, 0, stream);
}

int kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, void* out,
                            float* final_state, float* snapshots, int snapshot_tokens, int B,
                            int T, int H, int dk, int dv, float scale, int dtype,
                            hipStream_t stream) {
  kda_prefill_desc d = fixed_desc(q, k, v, g, beta, initial_state, out, final_state, B, T, H,
                                  dk, dv, scale, dtype);
  if (snapshot_tokens <= 0 || snapshot_tokens % 64 != 0) return bad_snapshot_tokens(d);
  d.snapshots = snapshots;
  d.snapshot_tokens = snapshot_tokens;
  return run_prefill(d, false, nullptr, 0, stream);
}

int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, void* out,
                         float* final_state, const int32_t* cu_seqlens, int N,
                         int total_T, int H, int dk, int dv, float scale, int dtype,
                         hipStream_t stream) {
  kda_prefill_desc d = packed_desc(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens,
                                   N, total_T, H, dk, dv, scale, dtype);
  if (cu_seqlens == nullptr) return packed_without_offsets(N, total_T, H, dk, dv, dtype);
  return run_prefill(d, false, nullptr, 0, stream);
}

size_t kda_chunk_fwd_varlen_workspace_size(int N, int total_T, int H, int dk, int dv, int dtype) {
  const void* p = reinterpret_cast<const void*>(uintptr_t{256});
  kda_prefill_desc d = packed_desc(p, p, p, p, p, nullptr, const_cast<void*>(p), nullptr,
                                   static_cast<const int32_t*>(p), N, total_T, H, dk, dv, 1.f, dtype);
  size_t bytes = 0;
  return kda_prefill_workspace_size(&d, &bytes) == KDA_OK ? bytes : 0;
}

int kda_chunk_fwd_varlen_ws(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, void* out,
                            float* final_state, const int32_t* cu_seqlens, int N, int total_T,
                            int H, int dk, int dv, float scale, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  kda_prefill_desc d = packed_desc(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens,
                                   N, total_T, H, dk, dv, scale, dtype);
  if (cu_seqlens == nullptr) return packed_without_offsets(N, total_T, H, dk, dv, dtype);
  return run_prefill(d, true, workspace, workspace_bytes, stream);
}

int kda_chunk_fwd_varlen_prologue(const void* q_raw, const void* k_raw, const void* v,
                                  const void* g_raw, const void* beta_raw,
                                  const float* initial_state, void* out, float* final_state,
                                  const int32_t* cu_seqlens, int N, int total_T, int H, int dk,
                                  int dv, float scale, int dtype, hipStream_t stream) {
  kda_prefill_desc d = packed_desc(q_raw, k_raw, v, g_raw, beta_raw, initial_state, out,
                                   final_state, cu_seqlens, N, total_T, H, dk, dv, scale, dtype);
  if (cu_seqlens == nullptr) return packed_without_offsets(N, total_T, H, dk, dv, dtype);
  d.prologue = 1;
  return run_prefill(d, false, nullptr, 0, stream);
}

int kda_chunk_fwd_varlen_snapshots(const void* q, const void* k, const void* v, const void* g,
                                   const void* beta, const float* initial_state, void* out,
                                   float* final_state, float* snapshots, int snapshot_tokens,
                                   const int32_t* cu_seqlens, int N, int total_T, int H, int dk,
                                   int dv, float scale, int dtype, hipStream_t stream) {
  kda_prefill_desc d = packed_desc(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens,
                                   N, total_T, H, dk, dv, scale, dtype);
  if (snapshot_tokens <= 0 || snapshot_tokens % 64 != 0) return bad_snapshot_tokens(d);
  if (cu_seqlens == nullptr) return packed_without_offsets(N, total_T, H, dk, dv, dtype);
  d.snapshots = snapshots;
  d.snapshot_tokens = snapshot_tokens;
  return run_prefill(d, false, nullptr, 0, stream);
}

// ---------------------------------------------------------------- backward

namespace {

int check_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                   const float* s0, const void* dout, const float* dsT, void* dq, void* dk_,
                   void* dv_, void* dg, void* dbeta, float* ds0, const int32_t* cu, bool packed,
                   int N, int T, int total_T, int H, int dk, int dv, int dtype) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  if (packed && cu == nullptr) return KDA_ERR_NULL;
  rc = check_sizes(packed, N, T, total_T, H);
  if (rc != KDA_OK) return rc;
  const uintptr_t elt = dtype == KDA_F32 ? 4 : 2;
  return check_ptrs({{q, 16, true}, {k, 16, true}, {v, 16, true}, {g, 16, true},
                     {beta, elt, true}, {dout, 16, true}, {dq, elt, true}, {dk_, elt, true},
                     {dv_, elt, true}, {dg, elt, true}, {dbeta, elt, true}, {s0, 4, false},
                     {dsT, 4, false}, {ds0, 4, false}, {cu, 4, false}});
}

// A self-allocating backward takes at most this much workspace; beyond it the call runs
// in windows of chunks (see kda_chunk_bwd).
constexpr size_t kBackwardSelfBytes = size_t{2} << 30;

int run_backward(kda::BackwardArgs a, bool caller_ws, void* workspace, size_t workspace_bytes) {
  if (caller_ws) {
    if (workspace == nullptr || !aligned(workspace, 256)) return KDA_ERR_WORKSPACE;
    const int cw = kda::backward_fit_window(a, workspace_bytes);
    if (cw < 0) return KDA_ERR_WORKSPACE;
    a.window_chunks = cw;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
  } else {
    const int cw = kda::backward_fit_window(a, kBackwardSelfBytes);
    a.window_chunks = cw < 0 ? 1 : cw;
  }
  const int rc = check_device();
  if (rc != KDA_OK) return rc;
  return kda::launch_backward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

int kda_chunk_bwd_ws(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     const float* initial_state, const void* grad_out,
                     const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v,
                     void* grad_g, void* grad_beta, float* grad_initial_state, int B, int T,
                     int H, int dk, int dv, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  const int rc = check_backward(q, k, v, g, beta, initial_state, grad_out, grad_final_state,
                                grad_q, grad_k, grad_v, grad_g, grad_beta, grad_initial_state,
                                nullptr, false, B, T, 0, H, dk, dv, dtype);
  if (rc != KDA_OK) return rc;
  kda::BackwardArgs a{q, k, v, g, beta, initial_state, grad_out, grad_final_state,
                      grad_q, grad_k, grad_v, grad_g, grad_beta, grad_initial_state,
                      B, T, H, dk, scale, dtype == KDA_F32, stream};
  return run_backward(a, workspace != nullptr || workspace_bytes != 0, workspace, workspace_bytes);
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  const float* initial_state, const void* grad_out,
                  const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v,
                  void* grad_g, void* grad_beta, float* grad_initial_state, int B, int T, int H,
                  int dk, int dv, float scale, int dtype, hipStream_t stream) {
  return kda_chunk_bwd_ws(q, k, v, g, beta, initial_state, grad_out, grad_final_state, grad_q,
                          grad_k, grad_v, grad_g, grad_beta, grad_initial_state, B, T, H, dk, dv,
                          scale, dtype, nullptr, 0, stream);
}

size_t kda_chunk_bwd_window_workspace_size(int B, int T, int H, int dk, int dv, int dtype,
                                           int window_chunks) {
  if (check_common(dk, dv, H, dtype) != KDA_OK || check_sizes(false, B, T, 0, H) != KDA_OK ||
      window_chunks < 0)
    return 0;
  kda::BackwardArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      B, T, H, dk, 1.f, dtype == KDA_F32, nullptr};
  a.window_chunks = window_chunks;
  return kda::backward_workspace_bytes(a);
}

size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype) {
  return kda_chunk_bwd_window_workspace_size(B, T, H, dk, dv, dtype, 0);
}

int kda_chunk_bwd_varlen_ws(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* initial_state, const void* grad_out,
                            const float* grad_final_state, void* grad_q, void* grad_k,
                            void* grad_v, void* grad_g, void* grad_beta,
                            float* grad_initial_state, const int32_t* cu_seqlens, int N,
                            int total_T, int H, int dk, int dv, float scale, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int rc = check_backward(q, k, v, g, beta, initial_state, grad_out, grad_final_state,
                                grad_q, grad_k, grad_v, grad_g, grad_beta, grad_initial_state,
                                cu_seqlens, true, N, 0, total_T, H, dk, dv, dtype);
  if (rc != KDA_OK) return rc;
  kda::BackwardArgs a{q, k, v, g, beta, initial_state, grad_out, grad_final_state,
                      grad_q, grad_k, grad_v, grad_g, grad_beta, grad_initial_state,
                      N, 0, H, dk, scale, dtype == KDA_F32, stream};
  a.cu_seqlens = cu_seqlens;
  a.total_T = total_T;
  return run_backward(a, workspace != nullptr || workspace_bytes != 0, workspace, workspace_bytes);
}

int kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, const void* grad_out,
                         const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v,
                         void* grad_g, void* grad_beta, float* grad_initial_state,
                         const int32_t* cu_seqlens, int N, int total_T, int H, int dk, int dv,
                         float scale, int dtype, hipStream_t stream) {
  return kda_chunk_bwd_varlen_ws(q, k, v, g, beta, initial_state, grad_out, grad_final_state,
                                 grad_q, grad_k, grad_v, grad_g, grad_beta, grad_initial_state,
                                 cu_seqlens, N, total_T, H, dk, dv, scale, dtype, nullptr, 0,
                                 stream);
}

size_t kda_chunk_bwd_varlen_window_workspace_size(int N, int total_T, int H, int dk, int dv,
                                                  int dtype, int window_chunks) {
  if (check_common(dk, dv, H, dtype) != KDA_OK || check_sizes(true, N, 0, total_T, H) != KDA_OK ||
      window_chunks < 0)
    return 0;
  kda::BackwardArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      N, 0, H, dk, 1.f, dtype == KDA_F32, nullptr};
  a.cu_seqlens = reinterpret_cast<const int32_t*>(uintptr_t{256});
  a.total_T = total_T;
  a.window_chunks = window_chunks;
  return kda::backward_workspace_bytes(a);
}

size_t kda_chunk_bwd_varlen_workspace_size(int N, int total_T, int H, int dk, int dv, int dtype) {
  return kda_chunk_bwd_varlen_window_workspace_size(N, total_T, H, dk, dv, dtype, 0);
}

// ---------------------------------------------------------------- context parallelism

int kda_chunk_transition_ws(const void* q, const void* k, const void* g, const void* beta,
                            float* transition, int B, int T, int H, int dk, int dv, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_common(dk, dv, H, dtype);
  if (rc != KDA_OK) return rc;
  rc = check_sizes(false, B, T, 0, H);
  if (rc != KDA_OK) return rc;
  const uintptr_t elt = dtype == KDA_F32 ? 4 : 2;
  rc = check_ptrs({{q, 16, false}, {k, 16, true}, {g, 16, true}, {beta, elt, true},
                   {transition, 4, true}});
  if (rc != KDA_OK) return rc;
  kda::TransitionArgs a{q, k, g, beta, transition, B, T, H, dk, dtype == KDA_F32, stream};
  if (workspace != nullptr || workspace_bytes != 0) {
    if (workspace == nullptr || !aligned(workspace, 256) ||
        workspace_bytes < kda::transition_workspace_bytes(a))
      return KDA_ERR_WORKSPACE;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
  }
  rc = check_device();
  if (rc != KDA_OK) return rc;
  return kda::launch_transition(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_transition(const void* q, const void* k, const void* g, const void* beta,
                         float* transition, int B, int T, int H, int dk, int dv, int dtype,
                         hipStream_t stream) {
  return kda_chunk_transition_ws(q, k, g, beta, transition, B, T, H, dk, dv, dtype, nullptr, 0,
                                 stream);
}

size_t kda_chunk_transition_workspace_size(int B, int T, int H, int dk, int dv, int dtype) {
  if (check_common(dk, dv, H, dtype) != KDA_OK || check_sizes(false, B, T, 0, H) != KDA_OK) return 0;
  kda::TransitionArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, B, T, H, dk,
                        dtype == KDA_F32, nullptr};
  return kda::transition_workspace_bytes(a);
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

// ---------------------------------------------------------------- decode

namespace {

int run_decode(const void* q, const void* k, const void* v, const void* g, const void* beta,
               float* state, void* out, int B, int H, int dk, int dv, float scale, int dtype,
               bool prologue, hipStream_t stream) {
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
  a.prologue = prologue;
  return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

int kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, float* state, void* out, int B, int H, int dk, int dv,
                    float scale, int dtype, hipStream_t stream) {
  return run_decode(q, k, v, g, beta, state, out, B, H, dk, dv, scale, dtype, false, stream);
}

int kda_decode_step_prologue(const void* q_raw, const void* k_raw, const void* v,
                             const void* g_raw, const void* beta_raw, float* state, void* out,
                             int B, int H, int dk, int dv, float scale, int dtype,
                             hipStream_t stream) {
  return run_decode(q_raw, k_raw, v, g_raw, beta_raw, state, out, B, H, dk, dv, scale, dtype, true,
                    stream);
}

}  // extern "C"
