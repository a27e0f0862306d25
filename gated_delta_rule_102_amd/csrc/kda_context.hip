// Context-parallel building blocks for one long sequence split into segments.
//
// A segment of KDA (any run of tokens) maps its entry state to its exit state
// affinely: S_exit = P S_entry + R, where R is the exit state from a zero entry
// (an ordinary prefill with no initial state) and P, the segment's transition,
// is the exit state obtained with v = 0 from the identity.  Chunk by chunk (the
// operands of kda_chunk_ops.h) P is the product of the chunk maps
// Diag(Lam) - Kt^T W, since with V = 0 a chunk sends S to Lam S - Kt^T W S.
// Segments are then joined by the sequential composition
//     S_entry(0) = S_0,   S_entry(r + 1) = P_r S_entry(r) + R_r,
// after which every segment reruns its prefill from its own entry state.  The
// pages give KDA's state as one fixed-size matrix per request that a prefix
// cache can restore (neurohive.io Kimi K3 review, "Training and inference
// infrastructure"), which is what makes a segment's effect a fixed-size affine
// map; they describe no context-parallel scheme, so this is a plain reading of
// the chunked form.
//
//   transition_scan_kernel: per (sequence, head, 32 columns of P) the scan
//       S <- Lam S - Kt^T (W S) from the identity's columns, fp32 throughout
//       (fp32 inputs).
//   transition_scan_bf16_kernel: the same scan for bf16 inputs with bf16
//       matrix-core operands (W and Kt^T as the chunk operands' bf16 copies, the
//       state and W S as bf16 transposes) and the fp32 state in registers, the
//       precision of the bf16 prefill.
//   compose_kernel: per (sequence, head, 32 value columns) the composition over
//       the segments, S <- P_r S + R_r, writing every entry state and the exit
//       state of the last segment.

#include "kda_chunk_ops.h"
#include "kda_launch.h"

namespace kda {

namespace {

template <int D>
__global__ __launch_bounds__(256) void transition_scan_kernel(const float* __restrict__ ws,
                                                              float* __restrict__ trans,
                                                              int nc, int BH) {
  using L = BwdLayout<D>;
  constexpr int LD = L::LD;
  constexpr int NTW = D / 32;   // state tiles per wave: (D/16) x 2 tiles over 4 waves
  __shared__ __attribute__((aligned(16))) float sm[2 * CR * LD + CR * LV + D * LV + D];
  float* Ws = sm;
  float* KTs = Ws + CR * LD;
  float* Dls = KTs + CR * LD;
  float* Ss = Dls + CR * LV;
  float* Lm = Ss + D * LV;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int l16 = lane16(), g4 = lane_g4();
  constexpr int NSL = D / SL;
  int bh, c0;
  if (!scan_block<NSL>(BH, bh, c0)) return;

  f32x4_t S[NTW];
#pragma unroll
  for (int x = 0; x < NTW; ++x) {   // columns c0 .. c0 + 31 of the identity
    const int j = wave * NTW + x, rt = j >> 1, ct = j & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) S[x][i] = (16 * rt + 4 * g4 + i == c0 + 16 * ct + l16) ? 1.f : 0.f;
  }
  for (int c = 0; c < nc; ++c) {
    const float* w = ws + (static_cast<int64_t>(bh) * nc + c) * L::WS;
    {
      GTile<256, CR, D> t_w, t_kt;
      t_w.load(w + L::W, D);
      t_kt.load(w + L::KT, D);
      float lm = w[L::LAM + (tid & (D - 1))];
      t_w.pin_all();
      t_kt.pin_all();
      pin(lm);
      t_w.store(Ws, LD);
      t_kt.store(KTs, LD);
      if (tid < D) Lm[tid] = lm;
    }
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
      const int j = wave * NTW + x, rt = j >> 1, ct = j & 1;
      put(Ss + 16 * rt * LV + 16 * ct, LV, S[x]);
    }
    __syncthreads();
#pragma unroll
    for (int y = 0; y < 2; ++y) {   // W S: 4 x 2 tiles (Delta = -W S)
      const int j = wave * 2 + y, rt = j >> 1, ct = j & 1;
      const f32x4_t d = mm<false, false>(zero4(), Ws + 16 * rt * LD, LD, Ss + 16 * ct, LV, D);
      put(Dls + 16 * rt * LV + 16 * ct, LV, d);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NTW; ++x) {   // S = Lam S - Kt^T (W S)
      const int j = wave * NTW + x, rt = j >> 1, ct = j & 1;
      const f32x4_t kd = mm<true, false>(zero4(), KTs + 16 * rt, LD, Dls + 16 * ct, LV, CR);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[x][i] = Lm[16 * rt + 4 * g4 + i] * S[x][i] - kd[i];
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < NTW; ++x) {
    const int j = wave * NTW + x, rt = j >> 1, ct = j & 1;
    put(trans + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D, S[x]);
  }
}

template <int D>
__global__ __launch_bounds__(kScanThreads) void transition_scan_bf16_kernel(
    const float* __restrict__ ws, const __bf16* __restrict__ wsb, float* __restrict__ trans,
    int nc, int BH) {
  using L = BwdLayout<D>;
  using ST = ScanTiles<D>;
  constexpr int LB = D + 8, L64 = CR + 8;
  __shared__ __attribute__((aligned(16))) __bf16 sb[CR * LB + D * L64 + SL * LB + SL * L64];
  __shared__ float Lm[D];
  __bf16* Ws = sb;                  // W      [t][i]
  __bf16* KTT = Ws + CR * LB;       // Kt^T   [i][t]
  __bf16* STr = KTT + D * L64;      // S^T    [j][i]
  __bf16* UT = STr + SL * LB;       // (W S)^T [j][t]
  const int tid = threadIdx.x, wave = tid >> 6;
  const int l16 = lane16(), g4 = lane_g4();
  constexpr int NSL = D / SL;
  int bh, c0;
  if (!scan_block<NSL>(BH, bh, c0)) return;

  f32x4_t S[ST::NTW];
#pragma unroll
  for (int x = 0; x < ST::NTW; ++x) {   // columns c0 .. c0 + 31 of the identity
    const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) S[x][i] = (16 * rt + 4 * g4 + i == c0 + 16 * ct + l16) ? 1.f : 0.f;
  }
  BTile<kScanThreads, CR, D> t_w;
  BTile<kScanThreads, D, CR> t_ktt;
  float lm;
  auto issue = [&](int c) {
    const int64_t item = static_cast<int64_t>(bh) * nc + c;
    const __bf16* wb = wsb + item * L::WSB;
    t_w.load(wb + L::BW);
    t_ktt.load(wb + L::BKTT);
    lm = ws[item * L::WS + L::LAM + (tid & (D - 1))];
  };
  issue(0);
  for (int c = 0; c < nc; ++c) {
    t_w.pin_all();
    t_ktt.pin_all();
    pin(lm);
    t_w.store(Ws, LB);
    t_ktt.store(KTT, L64);
    if (tid < D) Lm[tid] = lm;
    issue(min(c + 1, nc - 1));   // unconditional: the last step reloads its own chunk
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put_t_bf16(STr + 16 * ct * LB + 16 * rt, LB, S[x]);
    }
    __syncthreads();
    {   // W S: 4 x 2 tiles, one per wavefront
      const int rt = wave >> 1, ct = wave & 1;
      const f32x4_t u = mmb<D>(zero4(), Ws + 16 * rt * LB, LB, STr + 16 * ct * LB, LB);
      put_t_bf16(UT + 16 * ct * L64 + 16 * rt, L64, u);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {   // S = Lam S - Kt^T (W S)
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      const f32x4_t kd = mmb<CR>(zero4(), KTT + 16 * rt * L64, L64, UT + 16 * ct * L64, L64);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[x][i] = Lm[16 * rt + 4 * g4 + i] * S[x][i] - kd[i];
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < ST::NTW; ++x) {
    const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
    put(trans + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D, S[x]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void compose_kernel(const float* __restrict__ trans,
                                                      const float* __restrict__ part,
                                                      const float* __restrict__ s0,
                                                      float* __restrict__ entry, int R,
                                                      int BH) {
  constexpr int LD = D + 4;
  constexpr int NTW = D / 32;
  __shared__ __attribute__((aligned(16))) float sm[D * LD + D * LV];
  float* Ps = sm;
  float* Ss = Ps + D * LD;
  const int tid = threadIdx.x, wave = tid >> 6;
  constexpr int NSL = D / SL;
  int bh, c0;
  if (!scan_block<NSL>(BH, bh, c0)) return;
  const int64_t DD = static_cast<int64_t>(D) * D;
  const int64_t off = static_cast<int64_t>(bh) * DD + c0;

  f32x4_t S[NTW];
#pragma unroll
  for (int x = 0; x < NTW; ++x) {
    const int j = wave * NTW + x, rt = j >> 1, ct = j & 1;
    S[x] = s0 ? get(s0 + off + 16 * rt * D + 16 * ct, D) : zero4();
    put(entry + off + 16 * rt * D + 16 * ct, D, S[x]);
  }
  for (int r = 0; r < R; ++r) {
    const int64_t seg = static_cast<int64_t>(r) * BH * DD;
    {
      GTile<256, D, D> t_p;
      t_p.load(trans + seg + static_cast<int64_t>(bh) * DD, D);
      t_p.pin_all();
      t_p.store(Ps, LD);
    }
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
      const int j = wave * NTW + x, rt = j >> 1, ct = j & 1;
      put(Ss + 16 * rt * LV + 16 * ct, LV, S[x]);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NTW; ++x) {   // S = P_r S + R_r
      const int j = wave * NTW + x, rt = j >> 1, ct = j & 1;
      f32x4_t acc = get(part + seg + off + 16 * rt * D + 16 * ct, D);
      S[x] = mm<false, false>(acc, Ps + 16 * rt * LD, LD, Ss + 16 * ct, LV, D);
      put(entry + seg + BH * DD + off + 16 * rt * D + 16 * ct, D, S[x]);
    }
    __syncthreads();
  }
}

// Floats of workspace per 64-token chunk per head of a transition call.
template <int D, typename TIn>
constexpr int64_t transition_floats_per_item() {
  using L = BwdLayout<D>;
  return L::WS + (IsBf16<TIn>::value ? L::WSB / 2 : 0);
}

template <int D, typename TIn>
hipError_t launch_transition_t(const TransitionArgs& a) {
  using L = BwdLayout<D>;
  const int nc = (a.T + CR - 1) / CR;
  const int64_t items = static_cast<int64_t>(a.B) * a.H * nc;
  constexpr bool BF = IsBf16<TIn>::value;
  char* raw = nullptr;
  hipError_t err = ws_acquire(a.workspace, a.workspace_bytes,
                              items * transition_floats_per_item<D, TIn>() * sizeof(float), a.stream, &raw);
  if (err != hipSuccess) return err;
  float* ws = reinterpret_cast<float*>(raw);
  __bf16* wsb = BF ? reinterpret_cast<__bf16*>(ws + items * L::WS) : nullptr;
  const int BH = a.B * a.H;
  if constexpr (BF) {   // bf16 operands, the prefill's precision
    KDA_TRY_LAUNCH(err, (chunk_ops_kernel<D, TIn, false, false>), dim3(items), dim3(kOpsThreads), 0,
                   a.stream, static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                   static_cast<const TIn*>(a.g), static_cast<const TIn*>(a.beta), ws, wsb,
                   SeqMap{nullptr, a.B, a.T, a.B * a.T, a.H, nc}, 1.0f);
    KDA_TRY_LAUNCH(err, (transition_scan_bf16_kernel<D>), dim3(scan_grid(BH, D / SL)),
                   dim3(kScanThreads), 0, a.stream, ws, wsb, a.transition, nc, BH);
  } else {
    KDA_TRY_LAUNCH(err, (chunk_ops_kernel<D, TIn, true, false>), dim3(items), dim3(kOpsThreads), 0,
                   a.stream, static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                   static_cast<const TIn*>(a.g), static_cast<const TIn*>(a.beta), ws, nullptr,
                   SeqMap{nullptr, a.B, a.T, a.B * a.T, a.H, nc}, 1.0f);
    KDA_TRY_LAUNCH(err, (transition_scan_kernel<D>), dim3(scan_grid(BH, D / SL)), dim3(256), 0,
                   a.stream, ws, a.transition, nc, BH);
  }
  const hipError_t ferr = ws_release(a.workspace, raw, a.stream);
  return err != hipSuccess ? err : ferr;
}

}  // namespace

size_t transition_workspace_bytes(const TransitionArgs& a) {
  if (fused_transition_supported(a)) return 0;
  const int64_t items = static_cast<int64_t>(a.B) * a.H * ((a.T + CR - 1) / CR);
  int64_t per = 0;
  if (a.d == 128) per = a.dtype_f32 ? transition_floats_per_item<128, float>() : transition_floats_per_item<128, bf16_t>();
  else per = a.dtype_f32 ? transition_floats_per_item<64, float>() : transition_floats_per_item<64, bf16_t>();
  return static_cast<size_t>(items * per) * sizeof(float);
}

hipError_t launch_transition(const TransitionArgs& a) {
  if (fused_transition_supported(a)) return launch_fused_transition(a);
  if (a.d == 128) {
    return a.dtype_f32 ? launch_transition_t<128, float>(a) : launch_transition_t<128, bf16_t>(a);
  }
  return a.dtype_f32 ? launch_transition_t<64, float>(a) : launch_transition_t<64, bf16_t>(a);
}

hipError_t launch_compose(const ComposeArgs& a) {
  const int BH = a.B * a.H;
  if (a.d == 128) {
    hipLaunchKernelGGL((compose_kernel<128>), dim3(scan_grid(BH, 128 / SL)), dim3(256), 0, a.stream,
                       a.transitions, a.partial_states, a.initial_state, a.entry_states, a.R, BH);
  } else {
    hipLaunchKernelGGL((compose_kernel<64>), dim3(scan_grid(BH, 64 / SL)), dim3(256), 0, a.stream,
                       a.transitions, a.partial_states, a.initial_state, a.entry_states, a.R, BH);
  }
  return hipGetLastError();
}

}  // namespace kda
