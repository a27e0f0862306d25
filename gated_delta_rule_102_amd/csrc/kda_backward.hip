// Backward pass of chunked KDA on gfx950: gradients of
//     L = sum_t <dO_t, o_t> + <dS_T, S_T>
// with respect to q, k, v, g, beta and the initial state, for fixed-length
// sequences.  The pages train KDA at up to 1M tokens of context (best.xiaohu.ai
// "Kimi K3 tech report", context-curriculum section) but print no backward; the
// gradients are the plain derivatives of the forward rule (neurohive.io Kimi K3
// review, section "Sequence length: hybrid KDA and Gated MLA attention").
//
// With each chunk written as the affine map of kda_chunk_ops.h
//     Delta = Tb V - W S,   O = Q' S + P V,   S_next = Lam S + Kt^T Delta,
// the backward runs in four launches:
//   chunk_ops    per chunk: Tb, Ti, A', M', P, W, Q', Kt, G, Lam (fp32 workspace);
//   bwd_fwd_scan per (sequence, head, 32 value columns): S at every chunk start
//                and Delta, walking the chunks forwards;
//   bwd_scan     the same grid walking backwards from dS_T:
//                dU = Kt dS, dV = P^T dO + Tb^T dU, dS <- Lam dS + Q'^T dO - W^T dU;
//   bwd_grad_chunk per chunk, three stages in one workgroup: the operand
//                gradients, contractions over the value columns (dQ' = dO S^T,
//                dW = -dU S^T, dKt = Delta dS^T, dLam = rowsum(S * dS),
//                dP = dO V^T, dTb = dU V^T); the 64 x 64 algebra through P, Q', W,
//                Tb and the inverse (dP_tot, dKg, dTb_tot, dM', dA', dbeta); the
//                decayed products of dA' and dM' with k and q, and the chain to
//                dq, dk and dg (a reverse running sum).  The operand gradients
//                never leave the workgroup.
// Products run on the matrix cores from LDS: fp32 16x16x4 for fp32 inputs; for
// bf16 inputs the scans, the operand gradients and the 64 x 64 algebra use bf16
// operands (16x16x32) with fp32 accumulation, and the decayed products stay fp32.

#include <type_traits>

#include "kda_chunk_ops.h"
#include "kda_launch.h"

namespace kda {

namespace {

// One element through a buffer range (stores past the range are dropped).
__device__ __forceinline__ void store_elem(bf16_t x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(x.bits, r, off, 0, 0);
}
__device__ __forceinline__ void store_elem(float x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), r, off, 0, 0);
}

// ---------------------------------------------------------------- scans
// Each scan step loads the next chunk's operands before it issues its own global
// stores. The step's memory operations form one fixed sequence without branches:
// the next-chunk load is unconditional (the last step reloads its own chunk), and
// rows past a chunk's end fall outside a store's buffer range instead of being
// skipped by a branch.

template <int D, typename TIn>
__global__ __launch_bounds__(kScanThreads) void bwd_fwd_scan_kernel(const TIn* __restrict__ v,
                                                           const float* __restrict__ s0,
                                                           const float* __restrict__ ws,
                                                           float* __restrict__ st,
                                                           float* __restrict__ dl, SeqMap m,
                                                           int BH, float* __restrict__ s_end) {
  constexpr bool BF = IsBf16<TIn>::value;   // bf16 matrix-core operands for bf16 inputs
  using L = BwdLayout<D>;
  using ST = ScanTiles<D>;
  constexpr int LD = L::LD;
  __shared__ __attribute__((aligned(16))) float sm[CR * LS + 2 * CR * LD + 2 * CR * LV + D * LV + D];
  float* TBs = sm;
  float* Ws = TBs + CR * LS;
  float* KTs = Ws + CR * LD;
  float* Vs = KTs + CR * LD;
  float* Dls = Vs + CR * LV;
  float* Ss = Dls + CR * LV;
  float* Lm = Ss + D * LV;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int l16 = lane16(), g4 = lane_g4();
  constexpr int NSL = D / SL;
  int bh, c0;
  if (!scan_block<NSL>(BH, bh, c0)) return;
  const int H = m.H, h = bh % m.H;
  const StreamPos sp = stream_pos(m, bh);

  f32x4_t S[ST::NTW];
#pragma unroll
  for (int x = 0; x < ST::NTW; ++x) {
    const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
    S[x] = s0 ? get(s0 + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D) : zero4();
  }
  // the next chunk's operands are loaded into registers while this chunk computes
  GTile<kScanThreads, CR, CR> t_tb;
  GTile<kScanThreads, CR, D> t_w, t_kt;
  ITile<kScanThreads, SL, TIn> t_v;
  float lm;
  auto issue = [&](int c) {
    const float* w = ws + (sp.item0 + c * sp.istride) * L::WS;
    const int64_t row0 = (static_cast<int64_t>(sp.tok0) + static_cast<int64_t>(c) * CR) * H + h;
    t_tb.load(w + L::TB, CR);
    t_w.load(w + L::W, D);
    t_kt.load(w + L::KT, D);
    t_v.load(v + row0 * D + c0, static_cast<int64_t>(H) * D, min(CR, sp.len - c * CR));
    lm = w[L::LAM + (tid & (D - 1))];
  };
  if (sp.nch > 0) issue(0);
  for (int c = 0; c < sp.nch; ++c) {
    const int64_t item = sp.item0 + c * sp.istride;
    {
      t_tb.pin_all();
      t_w.pin_all();
      t_kt.pin_all();
      t_v.pin_all();
      pin(lm);
      t_tb.store(TBs, LS);
      t_w.store(Ws, LD);
      t_kt.store(KTs, LD);
      t_v.store(Vs, LV);
      if (tid < D) Lm[tid] = lm;
    }
    // the next chunk's loads go out before this step's stores: loads and stores
    // retire in order, so the next wait for those loads does not wait for the stores
    issue(min(c + 1, sp.nch - 1));   // unconditional: the last step reloads its own chunk
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(Ss + 16 * rt * LV + 16 * ct, LV, S[x]);
      put(st + item * D * D + 16 * rt * D + c0 + 16 * ct, D, S[x]);
    }
    __syncthreads();
    {   // Delta = Tb V - W S: 4 x 2 tiles
      const int j = wave, rt = j >> 1, ct = j & 1;
      const f32x4_t tv = mmx<BF, false, false>(zero4(), TBs + 16 * rt * LS, LS, Vs + 16 * ct, LV, CR);
      const f32x4_t wsv = mmx<BF, false, false>(zero4(), Ws + 16 * rt * LD, LD, Ss + 16 * ct, LV, D);
      f32x4_t d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = tv[i] - wsv[i];
      put(Dls + 16 * rt * LV + 16 * ct, LV, d);
      put(dl + item * CR * D + 16 * rt * D + c0 + 16 * ct, D, d);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {   // S = Lam S + Kt^T Delta
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      f32x4_t acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Lm[16 * rt + 4 * g4 + i] * S[x][i];
      S[x] = mmx<BF, true, false>(acc, KTs + 16 * rt, LD, Dls + 16 * ct, LV, CR);
    }
    __syncthreads();
  }
  if (s_end) {   // the state after the last chunk (a window's end, for the next window)
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(s_end + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D, S[x]);
    }
  }
  (void)l16;
}

template <int D, typename TIn>
__global__ __launch_bounds__(kScanThreads) void bwd_scan_kernel(const TIn* __restrict__ dout,
                                                       const float* __restrict__ dsT,
                                                       const float* __restrict__ ws,
                                                       float* __restrict__ dst,
                                                       float* __restrict__ du,
                                                       TIn* __restrict__ dv,
                                                       float* __restrict__ ds0, SeqMap m,
                                                       int BH) {
  // fp32 operands throughout: the bf16 form needs more registers than the two
  // wavefronts per SIMD leave, and spills cost more than it saves
  using L = BwdLayout<D>;
  using ST = ScanTiles<D>;
  constexpr int LD = L::LD;
  __shared__ __attribute__((aligned(16))) float sm[2 * CR * LD + 2 * CR * LS + 2 * CR * LV + D * LV + D];
  float* KQs = sm;                 // Kt, then Q'
  float* Ws = KQs + CR * LD;
  float* Ps = Ws + CR * LD;
  float* TBs = Ps + CR * LS;
  float* dOs = TBs + CR * LS;
  float* dUs = dOs + CR * LV;
  float* dSs = dUs + CR * LV;
  float* Lm = dSs + D * LV;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int l16 = lane16(), g4 = lane_g4();
  constexpr int NSL = D / SL;
  int bh, c0;
  if (!scan_block<NSL>(BH, bh, c0)) return;
  const int H = m.H, h = bh % m.H;
  const StreamPos sp = stream_pos(m, bh);
  const int64_t rs = static_cast<int64_t>(H) * D;

  f32x4_t dS[ST::NTW];
#pragma unroll
  for (int x = 0; x < ST::NTW; ++x) {
    const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
    dS[x] = dsT ? get(dsT + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D) : zero4();
  }
  // the previous chunk's operands are loaded into registers while this chunk computes
  GTile<kScanThreads, CR, D> t_kt, t_w;
  GTile<kScanThreads, CR, CR> t_p, t_tb;
  ITile<kScanThreads, SL, TIn> t_do;
  float lm;
  auto issue = [&](int c) {
    const float* w = ws + (sp.item0 + c * sp.istride) * L::WS;
    const int64_t row0 = (static_cast<int64_t>(sp.tok0) + static_cast<int64_t>(c) * CR) * H + h;
    t_kt.load(w + L::KT, D);
    t_w.load(w + L::W, D);
    t_p.load(w + L::PP, CR);
    t_tb.load(w + L::TB, CR);
    t_do.load(dout + row0 * D + c0, rs, min(CR, sp.len - c * CR));
    lm = w[L::LAM + (tid & (D - 1))];
  };
  if (sp.nch > 0) issue(sp.nch - 1);
  for (int c = sp.nch - 1; c >= 0; --c) {
    const int64_t item = sp.item0 + c * sp.istride;
    const int nrow = min(CR, sp.len - c * CR);
    const int64_t row0 = (static_cast<int64_t>(sp.tok0) + static_cast<int64_t>(c) * CR) * H + h;
    {
      t_kt.pin_all();
      t_w.pin_all();
      t_p.pin_all();
      t_tb.pin_all();
      t_do.pin_all();
      pin(lm);
      t_kt.store(KQs, LD);
      t_w.store(Ws, LD);
      t_p.store(Ps, LS);
      t_tb.store(TBs, LS);
      t_do.store(dOs, LV);
      if (tid < D) Lm[tid] = lm;
    }
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(dSs + 16 * rt * LV + 16 * ct, LV, dS[x]);
    }
    __syncthreads();
    f32x4_t u;
    {   // dU = Kt dS
      const int j = wave, rt = j >> 1, ct = j & 1;
      u = mm<false, false>(zero4(), KQs + 16 * rt * LD, LD, dSs + 16 * ct, LV, D);
      put(dUs + 16 * rt * LV + 16 * ct, LV, u);
    }
    __syncthreads();
    {   // Q' replaces Kt (no longer needed); its loads and the previous chunk's go
        // out before this step's global stores, so no wait holds for those stores
      GTile<kScanThreads, CR, D> t_qp;
      t_qp.load(ws + item * L::WS + L::QP, D);
      issue(c > 0 ? c - 1 : 0);   // unconditional: the last step reloads its own chunk
      t_qp.pin_all();
      t_qp.store(KQs, LD);
    }
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(dst + item * D * D + 16 * rt * D + c0 + 16 * ct, D, dS[x]);
    }
    {
      const int j = wave, rt = j >> 1, ct = j & 1;
      put(du + item * CR * D + 16 * rt * D + c0 + 16 * ct, D, u);
    }
    {   // dV = P^T dO + Tb^T dU
      const int j = wave, rt = j >> 1, ct = j & 1;
      f32x4_t acc = mm<true, false>(zero4(), Ps + 16 * rt, LS, dOs + 16 * ct, LV, CR);
      acc = mm<true, false>(acc, TBs + 16 * rt, LS, dUs + 16 * ct, LV, CR);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rt + 4 * g4 + i;
        if (t < nrow) dv[(row0 + static_cast<int64_t>(t) * H) * D + c0 + 16 * ct + l16] = Elem<TIn>::from(acc[i]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {   // dS = Lam dS + Q'^T dO - W^T dU
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      f32x4_t acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Lm[16 * rt + 4 * g4 + i] * dS[x][i];
      acc = mm<true, false>(acc, KQs + 16 * rt, LD, dOs + 16 * ct, LV, CR);
      const f32x4_t wu = mm<true, false>(zero4(), Ws + 16 * rt, LD, dUs + 16 * ct, LV, CR);
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[x][i] = acc[i] - wu[i];
    }
    __syncthreads();
  }
  if (ds0) {
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(ds0 + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D, dS[x]);
    }
  }
}

// ---------------------------------------------------------------- scans, bf16 operands
//
// For bf16 inputs both scans keep every matrix-core operand in LDS as bf16, laid
// out so that each is k-contiguous: a lane reads one 16-byte run per operand per
// 16x16x32 product.  The chunk operands come from the bf16 copies chunk_ops
// writes in exactly those layouts (Tb, W, Kt^T for the forward scan; Kt, W^T,
// Q'^T, P^T, Tb^T for the reverse one) and are staged by plain 16-byte copies;
// only V and dO are transposed while staged, and the fp32 state and the
// per-step products (Delta, dU) go to LDS as bf16 transposes.  The per-chunk
// states and state gradients and Delta, dU are stored as bf16 for the operand
// gradient kernel, which rounds them to bf16 for its products in any case.

// a 64 x COLS input tile (bf16) to LDS transposed ([c][r])
template <int NT, int COLS>
__device__ __forceinline__ void stage_bf16_t(const ITile<NT, COLS, bf16_t>& t, __bf16* dst, int ld) {
  using I = ITile<NT, COLS, bf16_t>;
#pragma unroll
  for (int j = 0; j < I::PER; ++j) {
    const int e = static_cast<int>(threadIdx.x) + j * NT;
    const int rr = e / COLS, c = e - rr * COLS;
    dst[c * ld + rr] = static_cast<__bf16>(t.val(j));
  }
}
template <int D>
__global__ __launch_bounds__(kScanThreads) void bwd_fwd_scan_bf16_kernel(
    const bf16_t* __restrict__ v, const float* __restrict__ s0, const float* __restrict__ ws,
    const __bf16* __restrict__ wsb, __bf16* __restrict__ st, __bf16* __restrict__ dl, SeqMap m,
    int BH, float* __restrict__ s_end) {
  using L = BwdLayout<D>;
  using ST = ScanTiles<D>;
  constexpr int LB = D + 8, L64 = CR + 8;   // bf16 leading dimensions (16-byte rows)
  __shared__ __attribute__((aligned(16))) __bf16 sb[CR * L64 + CR * LB + D * L64 + SL * L64 + SL * LB + SL * L64];
  __shared__ float Lm[D];
  __bf16* TBs = sb;                 // Tb      [t][s]
  __bf16* Ws = TBs + CR * L64;      // W       [t][i]
  __bf16* KTT = Ws + CR * LB;       // Kt^T    [i][s]
  __bf16* VT = KTT + D * L64;       // V^T     [j][s]
  __bf16* STr = VT + SL * L64;      // S^T     [j][i]
  __bf16* DT = STr + SL * LB;       // Delta^T [j][s]
  const int tid = threadIdx.x, wave = tid >> 6;
  const int g4 = lane_g4();
  constexpr int NSL = D / SL;
  int bh, c0;
  if (!scan_block<NSL>(BH, bh, c0)) return;
  const int H = m.H, h = bh % m.H;
  const StreamPos sp = stream_pos(m, bh);

  f32x4_t S[ST::NTW];
#pragma unroll
  for (int x = 0; x < ST::NTW; ++x) {
    const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
    S[x] = s0 ? get(s0 + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D) : zero4();
  }
  BTile<kScanThreads, CR, CR> t_tb;
  BTile<kScanThreads, CR, D> t_w;
  BTile<kScanThreads, D, CR> t_ktt;
  ITile<kScanThreads, SL, bf16_t> t_v;
  float lm;
  auto issue = [&](int c) {
    const int64_t item = sp.item0 + c * sp.istride;
    const __bf16* wb = wsb + item * L::WSB;
    const int64_t row0 = (static_cast<int64_t>(sp.tok0) + static_cast<int64_t>(c) * CR) * H + h;
    t_tb.load(wb + L::BTB);
    t_w.load(wb + L::BW);
    t_ktt.load(wb + L::BKTT);
    t_v.load(v + row0 * D + c0, static_cast<int64_t>(H) * D, min(CR, sp.len - c * CR));
    lm = ws[item * L::WS + L::LAM + (tid & (D - 1))];
  };
  if (sp.nch > 0) issue(0);
  for (int c = 0; c < sp.nch; ++c) {
    const int64_t item = sp.item0 + c * sp.istride;
    t_tb.pin_all();
    t_w.pin_all();
    t_ktt.pin_all();
    t_v.pin_all();
    pin(lm);
    t_tb.store(TBs, L64);
    t_w.store(Ws, LB);
    t_ktt.store(KTT, L64);
    stage_bf16_t(t_v, VT, L64);
    if (tid < D) Lm[tid] = lm;
    // the next chunk's loads go out before this step's global stores
    issue(min(c + 1, sp.nch - 1));   // unconditional: the last step reloads its own chunk
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put_t_bf16(STr + 16 * ct * LB + 16 * rt, LB, S[x]);
      put_bf16(st + item * D * D + 16 * rt * D + c0 + 16 * ct, D, S[x]);
    }
    __syncthreads();
    {   // Delta = Tb V - W S: 4 x 2 tiles, one per wavefront
      const int rt = wave >> 1, ct = wave & 1;
      const f32x4_t tv = mmb<CR>(zero4(), TBs + 16 * rt * L64, L64, VT + 16 * ct * L64, L64);
      const f32x4_t wsv = mmb<D>(zero4(), Ws + 16 * rt * LB, LB, STr + 16 * ct * LB, LB);
      f32x4_t d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = tv[i] - wsv[i];
      put_t_bf16(DT + 16 * ct * L64 + 16 * rt, L64, d);
      put_bf16(dl + item * CR * D + 16 * rt * D + c0 + 16 * ct, D, d);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {   // S = Lam S + Kt^T Delta
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      f32x4_t acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Lm[16 * rt + 4 * g4 + i] * S[x][i];
      S[x] = mmb<CR>(acc, KTT + 16 * rt * L64, L64, DT + 16 * ct * L64, L64);
    }
    __syncthreads();
  }
  if (s_end) {   // the state after the last chunk (a window's end, for the next window)
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(s_end + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D, S[x]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kScanThreads) void bwd_scan_bf16_kernel(
    const bf16_t* __restrict__ dout, const float* __restrict__ dsT, const float* __restrict__ ws,
    const __bf16* __restrict__ wsb, __bf16* __restrict__ dst, __bf16* __restrict__ du,
    bf16_t* __restrict__ dv, float* __restrict__ ds0, SeqMap m, int BH) {
  using L = BwdLayout<D>;
  using ST = ScanTiles<D>;
  constexpr int LB = D + 8, L64 = CR + 8;
  __shared__ __attribute__((aligned(16))) __bf16 sb[CR * LB + SL * LB + 2 * CR * L64 + 2 * SL * L64 + 2 * D * L64];
  __shared__ float Lm[D];
  __bf16* KTs = sb;                 // Kt    [t][i]
  __bf16* dST = KTs + CR * LB;      // dS^T  [j][i]
  __bf16* PT = dST + SL * LB;       // P^T   [t'][t]
  __bf16* TBT = PT + CR * L64;      // Tb^T  [t'][t]
  __bf16* dOT = TBT + CR * L64;     // dO^T  [j][t]
  __bf16* dUT = dOT + SL * L64;     // dU^T  [j][t]
  __bf16* QPT = dUT + SL * L64;     // Q'^T  [i][t]
  __bf16* WT = QPT + D * L64;       // W^T   [i][t]
  const int tid = threadIdx.x, wave = tid >> 6;
  const int l16 = lane16(), g4 = lane_g4();
  constexpr int NSL = D / SL;
  int bh, c0;
  if (!scan_block<NSL>(BH, bh, c0)) return;
  const int H = m.H, h = bh % m.H;
  const StreamPos sp = stream_pos(m, bh);
  const int64_t rs = static_cast<int64_t>(H) * D;

  f32x4_t dS[ST::NTW];
#pragma unroll
  for (int x = 0; x < ST::NTW; ++x) {
    const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
    dS[x] = dsT ? get(dsT + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D) : zero4();
  }
  BTile<kScanThreads, CR, D> t_kt;
  BTile<kScanThreads, D, CR> t_wt, t_qpt;
  BTile<kScanThreads, CR, CR> t_pt, t_tbt;
  ITile<kScanThreads, SL, bf16_t> t_do;
  float lm;
  auto issue = [&](int c) {
    const int64_t item = sp.item0 + c * sp.istride;
    const __bf16* wb = wsb + item * L::WSB;
    const int64_t row0 = (static_cast<int64_t>(sp.tok0) + static_cast<int64_t>(c) * CR) * H + h;
    t_kt.load(wb + L::BKT);
    t_wt.load(wb + L::BWT);
    t_qpt.load(wb + L::BQPT);
    t_pt.load(wb + L::BPT);
    t_tbt.load(wb + L::BTBT);
    t_do.load(dout + row0 * D + c0, rs, min(CR, sp.len - c * CR));
    lm = ws[item * L::WS + L::LAM + (tid & (D - 1))];
  };
  if (sp.nch > 0) issue(sp.nch - 1);
  for (int c = sp.nch - 1; c >= 0; --c) {
    const int64_t item = sp.item0 + c * sp.istride;
    const int nrow = min(CR, sp.len - c * CR);
    const int64_t row0 = (static_cast<int64_t>(sp.tok0) + static_cast<int64_t>(c) * CR) * H + h;
    t_kt.pin_all();
    t_wt.pin_all();
    t_qpt.pin_all();
    t_pt.pin_all();
    t_tbt.pin_all();
    t_do.pin_all();
    pin(lm);
    t_kt.store(KTs, LB);
    t_wt.store(WT, L64);
    t_qpt.store(QPT, L64);
    t_pt.store(PT, L64);
    t_tbt.store(TBT, L64);
    stage_bf16_t(t_do, dOT, L64);
    if (tid < D) Lm[tid] = lm;
    // the previous chunk's loads go out before this step's global stores
    issue(c > 0 ? c - 1 : 0);   // unconditional: the last step reloads its own chunk
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put_t_bf16(dST + 16 * ct * LB + 16 * rt, LB, dS[x]);
      put_bf16(dst + item * D * D + 16 * rt * D + c0 + 16 * ct, D, dS[x]);
    }
    __syncthreads();
    {   // dU = Kt dS: one tile per wavefront
      const int rt = wave >> 1, ct = wave & 1;
      const f32x4_t u = mmb<D>(zero4(), KTs + 16 * rt * LB, LB, dST + 16 * ct * LB, LB);
      put_t_bf16(dUT + 16 * ct * L64 + 16 * rt, L64, u);
      put_bf16(du + item * CR * D + 16 * rt * D + c0 + 16 * ct, D, u);
    }
    __syncthreads();
    {   // dV = P^T dO + Tb^T dU; rows past the chunk's end fall outside the store
        // range (no branch, so the stores per step are a fixed count)
      const int rt = wave >> 1, ct = wave & 1;
      f32x4_t acc = mmb<CR>(zero4(), PT + 16 * rt * L64, L64, dOT + 16 * ct * L64, L64);
      acc = mmb<CR>(acc, TBT + 16 * rt * L64, L64, dUT + 16 * ct * L64, L64);
      const uint32_t rsb = static_cast<uint32_t>(H) * D * 2;   // token row stride (bytes)
      const auto rdv = make_rsrc(dv + row0 * D, (nrow - 1) * rsb + D * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rt + 4 * g4 + i;
        __builtin_amdgcn_raw_buffer_store_b16(Elem<bf16_t>::from(acc[i]).bits, rdv,
                                              t * rsb + (c0 + 16 * ct + l16) * 2, 0, 0);
      }
    }
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {   // dS = Lam dS + Q'^T dO - W^T dU
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      f32x4_t acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Lm[16 * rt + 4 * g4 + i] * dS[x][i];
      acc = mmb<CR>(acc, QPT + 16 * rt * L64, L64, dOT + 16 * ct * L64, L64);
      const f32x4_t wu = mmb<CR>(zero4(), WT + 16 * rt * L64, L64, dUT + 16 * ct * L64, L64);
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[x][i] = acc[i] - wu[i];
    }
    __syncthreads();
  }
  if (ds0) {
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(ds0 + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D, dS[x]);
    }
  }
}

// ---------------------------------------------------------------- operand gradients

// Tiles of the operand gradients: 16 x 16 tiles j = wave + 8x, x < NTW, of [dQ', -dW,
// dKt] (64 x D each, NBIG tiles each) and then [dP, dTb] (64 x 64, 16 tiles each).
// Wave w's tiles x = XP, XP + 1 are tiles w and w + 8 of dP; x = XP + 2, XP + 3 the
// same tiles of dTb.  The first NBIG / 8 tiles (dQ') and the tiles from 2 NBIG / 8
// (dKt) sit where the decayed-product stage wants them: tile j covers rows
// 16 (j / CT) .., columns 16 (j % CT) ...
template <int D>
struct DvTiles {
  static constexpr int CT = D / 16, NBIG = 4 * CT, NTOT = 3 * NBIG + 32, NTW = NTOT / 8;
  static constexpr int XP = 3 * NBIG / 8;
  static_assert(NTOT % 8 == 0 && (3 * NBIG) % 8 == 0, "tile split");
};

// fp32 per-chunk states: the contractions over the value columns, in 32-column
// slices staged through LDS (2 D + 4 * 64 rows of LV floats); dlam (threads < D) =
// rowsum(S * dS_next).  Ends with a barrier: LDS is free afterwards.
template <int D, typename TIn>
__device__ __forceinline__ void dv_accumulate(float* sm, const TIn* v, const TIn* dout, const float* st,
                                              const float* dst, const float* dl, const float* du,
                                              int64_t item, const ChunkPos& p, int64_t rs,
                                              f32x4_t (&acc)[DvTiles<D>::NTW], float& dlam) {
  constexpr bool BF = IsBf16<TIn>::value;   // bf16 matrix-core operands for bf16 inputs
  using DT = DvTiles<D>;
  constexpr int CT = DT::CT, NBIG = DT::NBIG, NTW = DT::NTW;
  float* Ss = sm;
  float* dSs = Ss + D * LV;
  float* dOs = dSs + D * LV;
  float* dUs = dOs + CR * LV;
  float* Dls = dUs + CR * LV;
  float* Vs = Dls + CR * LV;
  const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
  for (int x = 0; x < NTW; ++x) acc[x] = zero4();
  dlam = 0.f;
  for (int c0 = 0; c0 < D; c0 += SL) {
    {
      GTile<512, D, SL> t_s, t_ds;
      GTile<512, CR, SL> t_dl, t_du;
      ITile<512, SL, TIn> t_do, t_v;
      t_s.load(st + item * D * D + c0, D);
      t_ds.load(dst + item * D * D + c0, D);
      t_dl.load(dl + item * CR * D + c0, D);
      t_du.load(du + item * CR * D + c0, D);
      t_do.load(dout + p.row0 * D + c0, rs, p.nrow);
      t_v.load(v + p.row0 * D + c0, rs, p.nrow);
      t_s.pin_all();
      t_ds.pin_all();
      t_dl.pin_all();
      t_du.pin_all();
      t_do.pin_all();
      t_v.pin_all();
      t_s.store(Ss, LV);
      t_ds.store(dSs, LV);
      t_dl.store(Dls, LV);
      t_du.store(dUs, LV);
      t_do.store(dOs, LV);
      t_v.store(Vs, LV);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
      const int j = wave + 8 * x;
      if (j < 3 * NBIG) {   // dQ' = dO S^T, -dW = dU S^T, dKt = Delta dS^T
        const int m = j / NBIG, r = j - m * NBIG, rt = r / CT, ct = r - rt * CT;
        const float* A = (m == 0 ? dOs : m == 1 ? dUs : Dls) + 16 * rt * LV;
        const float* Bm = (m == 2 ? dSs : Ss) + 16 * ct * LV;
        acc[x] = mmx<BF, false, true>(acc[x], A, LV, Bm, LV, SL);
      } else {              // dP = dO V^T, dTb = dU V^T
        const int j2 = j - 3 * NBIG, m = j2 >> 4, rt = (j2 & 15) >> 2, ct = j2 & 3;
        acc[x] = mmx<BF, false, true>(acc[x], (m == 0 ? dOs : dUs) + 16 * rt * LV, LV,
                                 Vs + 16 * ct * LV, LV, SL);
      }
    }
    if (tid < D) {
#pragma unroll 8
      for (int jj = 0; jj < SL; ++jj) dlam += Ss[tid * LV + jj] * dSs[tid * LV + jj];
    }
    __syncthreads();
  }
}

// bf16 inputs: the same contractions from bf16 per-chunk states (S, dS_next),
// Delta, dU and the bf16 inputs, every product in natural row-major layouts
// (A(r, k) row-major, B(k, c) = X[c][k] with X row-major) on bf16 matrix cores.
template <int NT, int ROWS, int COLS>
struct BTileS {   // ROWS x COLS bf16 slice of a matrix with row stride gld
  static constexpr int C8 = COLS / 8, N = ROWS * C8, PER = (N + NT - 1) / NT;
  bf16x8_t r[PER];
  int nrow_;   // rows >= nrow_ are stored as zero (masked at the store, not the load)
  static __device__ __forceinline__ bool live(int e) { return N % NT == 0 || e < N; }
  __device__ __forceinline__ void load(const __bf16* src, int64_t gld) {
    nrow_ = ROWS;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT, rr = e / C8, c = (e - rr * C8) * 8;
      if (live(e)) r[j] = *reinterpret_cast<const bf16x8_t*>(src + rr * gld + c);
    }
  }
  // 64 input rows (row stride gld), rows >= nrow as zero (clamped loads)
  __device__ __forceinline__ void load_rows(const bf16_t* src, int64_t gld, int nrow) {
    nrow_ = nrow;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT, rr = e / C8, c = (e - rr * C8) * 8;
      if (live(e))
        r[j] = *reinterpret_cast<const bf16x8_t*>(src + static_cast<int64_t>(min(rr, nrow - 1)) * gld + c);
    }
  }
  __device__ __forceinline__ void pin_all() {
#pragma unroll
    for (int j = 0; j < PER; ++j) pin(r[j]);
  }
  __device__ __forceinline__ void store(__bf16* dst, int ld) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT, rr = e / C8, c = (e - rr * C8) * 8;
      if (live(e)) *reinterpret_cast<bf16x8_t*>(dst + rr * ld + c) = rr < nrow_ ? r[j] : bf16x8_t{};
    }
  }
};

constexpr int LVB = SL + 8;   // bf16 leading dimension of the 32-column slices

template <int D>
__device__ __forceinline__ void dv_accumulate_bf16(__bf16* sm, const bf16_t* v, const bf16_t* dout,
                                                   const __bf16* st, const __bf16* dst,
                                                   const __bf16* dl, const __bf16* du, int64_t item,
                                                   const ChunkPos& p, int64_t rs,
                                                   f32x4_t (&acc)[DvTiles<D>::NTW], float& dlam) {
  using DT = DvTiles<D>;
  constexpr int CT = DT::CT, NBIG = DT::NBIG, NTW = DT::NTW;
  __bf16* Ss = sm;
  __bf16* dSs = Ss + D * LVB;
  __bf16* dOs = dSs + D * LVB;
  __bf16* dUs = dOs + CR * LVB;
  __bf16* Dls = dUs + CR * LVB;
  __bf16* Vs = Dls + CR * LVB;
  const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
  for (int x = 0; x < NTW; ++x) acc[x] = zero4();
  dlam = 0.f;
  // the next slice's loads are issued before this slice's products (the last slice
  // reloads itself, so no load sits behind a branch)
  BTileS<512, D, SL> t_s, t_ds;
  BTileS<512, CR, SL> t_dl, t_du, t_do, t_v;
  auto load = [&](int c0) {
    t_s.load(st + item * D * D + c0, D);
    t_ds.load(dst + item * D * D + c0, D);
    t_dl.load(dl + item * CR * D + c0, D);
    t_du.load(du + item * CR * D + c0, D);
    t_do.load_rows(dout + p.row0 * D + c0, rs, p.nrow);
    t_v.load_rows(v + p.row0 * D + c0, rs, p.nrow);
  };
  load(0);
  for (int c0 = 0; c0 < D; c0 += SL) {
    t_s.pin_all();
    t_ds.pin_all();
    t_dl.pin_all();
    t_du.pin_all();
    t_do.pin_all();
    t_v.pin_all();
    t_s.store(Ss, LVB);
    t_ds.store(dSs, LVB);
    t_dl.store(Dls, LVB);
    t_du.store(dUs, LVB);
    t_do.store(dOs, LVB);
    t_v.store(Vs, LVB);
    load(min(c0 + SL, D - SL));
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
      const int j = wave + 8 * x;
      if (j < 3 * NBIG) {   // dQ' = dO S^T, -dW = dU S^T, dKt = Delta dS^T
        const int m = j / NBIG, r = j - m * NBIG, rt = r / CT, ct = r - rt * CT;
        const __bf16* A = (m == 0 ? dOs : m == 1 ? dUs : Dls) + 16 * rt * LVB;
        const __bf16* Bm = (m == 2 ? dSs : Ss) + 16 * ct * LVB;
        acc[x] = mmb<SL>(acc[x], A, LVB, Bm, LVB);
      } else {              // dP = dO V^T, dTb = dU V^T
        const int j2 = j - 3 * NBIG, m = j2 >> 4, rt = (j2 & 15) >> 2, ct = j2 & 3;
        acc[x] = mmb<SL>(acc[x], (m == 0 ? dOs : dUs) + 16 * rt * LVB, LVB, Vs + 16 * ct * LVB, LVB);
      }
    }
    if (tid < D) {
#pragma unroll 8
      for (int jj = 0; jj < SL; ++jj)
        dlam += static_cast<float>(Ss[tid * LVB + jj]) * static_cast<float>(dSs[tid * LVB + jj]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- 64 x 64 algebra

constexpr int kNnThreads = 512;   // 8 wavefronts: two per SIMD

template <int D>
struct NnLds {
  static constexpr int LD = D + 4;
  static constexpr int A = 3 * CR * LD + CR * LS, B = 5 * CR * LS;
  static constexpr int FRONT = A > B ? A : B;      // phase A: Kg, dQ', dW, P; phase B: 5 matrices
  static constexpr int TOTAL = FRONT + CR * LS + CR;
};

// LDS of bwd_grad_chunk: the operand-gradient slices first, then the algebra
// (NnLds), then the decayed products: k colf, k rowf, q rowf in the first
// 3 * 64 * LD floats, dA' and dM' (written by the algebra's last phases, where
// nothing live sits then: dM' over Tb, dA' over P, or past the algebra's region),
// then G at the sub-tile ends and the pair factors.
template <int D>
struct ChunkLds {
  using NL = NnLds<D>;
  static constexpr int KQ = 3 * CR * (D + 4);
  static constexpr bool DA_IN_FRONT = KQ >= 4 * CR * LS && KQ + CR * LS <= NL::FRONT;
  static constexpr int DAS = DA_IN_FRONT ? KQ : NL::TOTAL;
  static constexpr int DMS = NL::FRONT;
  static constexpr int RF = NL::TOTAL > DAS + CR * LS ? NL::TOTAL : DAS + CR * LS;
  static constexpr int TOTAL = RF + 10 * D;
  static_assert(KQ <= DMS && KQ <= DAS, "decay operands below dA', dM'");
  static_assert(TOTAL >= (2 * D + 4 * CR) * LV, "operand-gradient slices fit");
  static_assert(TOTAL * 4 <= 160 * 1024, "LDS budget");
};

// Element type of the per-chunk states, Delta and dU the scans store.
template <typename TIn>
using StateElem = typename std::conditional<IsBf16<TIn>::value, __bf16, float>::type;

// One workgroup per (chunk, head): the operand gradients (contractions over the
// value columns), the 64 x 64 algebra and the decayed products, in one pass, so no
// operand gradient leaves the workgroup: dQ', dKt and dKg stay in registers in the
// accumulator tiles the last stage needs, dA' and dM' in LDS.  The algebra's inputs
// are loaded at the top in two register sets: X (G, P, Tb, k), written to LDS
// right after the contractions, and Y (M', Ti, A', beta), used by the later phases;
// vector-memory counters retire in order, so the first use of Y waits only for Y,
// and both groups' latency hides behind the contractions.
template <int D, typename TIn>
__global__ __launch_bounds__(kNnThreads) void bwd_grad_chunk_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ beta,
    const TIn* __restrict__ v, const TIn* __restrict__ dout, const StateElem<TIn>* __restrict__ st,
    const StateElem<TIn>* __restrict__ dst, const StateElem<TIn>* __restrict__ dl,
    const StateElem<TIn>* __restrict__ du, const float* __restrict__ ws, TIn* __restrict__ dq,
    TIn* __restrict__ dk, TIn* __restrict__ dg, TIn* __restrict__ dbeta, SeqMap m,
    float scale) {
  constexpr bool BF = IsBf16<TIn>::value;   // bf16 matrix-core operands for bf16 inputs
  using L = BwdLayout<D>;
  using NL = NnLds<D>;
  using CL = ChunkLds<D>;
  using DT = DvTiles<D>;
  constexpr int LD = L::LD;
  __shared__ __attribute__((aligned(16))) float sm[CL::TOTAL];
  // phase A
  float* Kg = sm;
  float* dQ = Kg + CR * LD;
  float* dW = dQ + CR * LD;
  float* Ps = dW + CR * LD;
  float* TBs = sm + NL::FRONT;   // kept through phase B
  float* BT = TBs + CR * LS;
  // phase B
  float* B0 = sm;                // dP_tot, then X = dTi Ti^T
  float* B1 = B0 + CR * LS;      // M', then dA
  float* B2 = B1 + CR * LS;      // Ti
  float* B3 = B2 + CR * LS;      // dTb_tot, then A'
  float* B4 = B3 + CR * LS;      // dTi
  // decayed products
  float* Ki = sm;                // k e^{R - G}  (column side)
  float* Ko = Ki + CR * LD;      // k e^{G - R}  (row side), later dG
  float* Qo = Ko + CR * LD;      // q e^{G - R}  (row side), later dKt Kt
  float* dAs = sm + CL::DAS;     // dA', written by the algebra
  float* dMs = sm + CL::DMS;     // dM', written by the algebra
  float* Rf = sm + CL::RF;       // [4][D] G at each sub-tile's last row
  float* FP = Rf + 4 * D;        // [6][D] e^{R_I - R_J}
  const int tid = threadIdx.x, wave = tid >> 6;
  const int l16 = lane16(), g4 = lane_g4();
  const int H = m.H;
  const int64_t rs = static_cast<int64_t>(H) * D;
  constexpr int CT = D / 16;
  const int64_t item = blockIdx.x;
  const ChunkPos p = chunk_pos(blockIdx.x, m);
  if (!p.valid) return;            // unused item of packed sequences
  const float* w = ws + item * L::WS;

  GTile<kNnThreads, CR, D> t_g;
  GTile<kNnThreads, CR, CR> t_p, t_tb, t_m, t_ti, t_ap;
  ITile4<kNnThreads, D, TIn> t_k;
  t_g.load(w + L::G, D);
  t_p.load(w + L::PP, CR);
  t_tb.load(w + L::TB, CR);
  t_k.load(k + p.row0 * D, rs, p.nrow);
  t_m.load(w + L::MP, CR);
  t_ti.load(w + L::TI, CR);
  t_ap.load(w + L::AP, CR);
  const float bt0 = to_f32(beta[p.row0 + static_cast<int64_t>(min(tid & (CR - 1), p.nrow - 1)) * H]);

  f32x4_t acc[DT::NTW];
  float dlam;
  if constexpr (BF)
    dv_accumulate_bf16<D>(reinterpret_cast<__bf16*>(sm), v, dout, st, dst, dl, du, item, p, rs, acc, dlam);
  else
    dv_accumulate<D, TIn>(sm, v, dout, st, dst, dl, du, item, p, rs, acc, dlam);

  // bf16 inputs: the operands of the next products go to LDS once as bf16 (rounded
  // as the products would round them), each in the orientations its products read
  // with 16-byte runs of k: dQ' and -dW by rows and by columns, Kg by rows, P^T and
  // Tb^T; the products are then the bf16 ones bit for bit
  constexpr int LDB = D + 8, LT = CR + 8;
  __bf16* smb = reinterpret_cast<__bf16*>(sm);
  __bf16* KgB = smb;                          // [64][LDB] Kg
  __bf16* dQB = KgB + CR * LDB;               // [64][LDB] dQ'
  __bf16* dWB = dQB + CR * LDB;               // [64][LDB] -dW
  __bf16* dQT = dWB + CR * LDB;               // [D][LT]  dQ'^T
  __bf16* dWT = dQT + D * LT;                 // [D][LT]  -dW^T
  __bf16* PT = dWT + D * LT;                  // [64][LT] P^T
  __bf16* TBT = PT + CR * LT;                 // [64][LT] Tb^T
  static_assert(3 * CR * LDB + 2 * D * LT + 2 * CR * LT <= 2 * NL::FRONT, "bf16 operands fit");

  // dQ' and dW to LDS; dQ' and dKt also stay in registers for the decayed products
#pragma unroll
  for (int x = 0; x < 2 * DT::NBIG / 8; ++x) {
    const int j = wave + 8 * x;
    const int m = j / DT::NBIG, r = j - m * DT::NBIG, rt = r / CT, ct = r - rt * CT;
    f32x4_t vv = acc[x];
    if (m != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = -vv[i];
    }
    if constexpr (BF) {
      __bf16* rows = (m == 0 ? dQB : dWB) + 16 * rt * LDB + 16 * ct;
      __bf16* cols = (m == 0 ? dQT : dWT) + 16 * ct * LT + 16 * rt;
#pragma unroll
      for (int i = 0; i < 4; ++i) rows[(4 * g4 + i) * LDB + l16] = static_cast<__bf16>(vv[i]);
      *reinterpret_cast<bf16x4_t*>(cols + l16 * LT + 4 * g4) =
          bf16x4_t{static_cast<__bf16>(vv[0]), static_cast<__bf16>(vv[1]),
                   static_cast<__bf16>(vv[2]), static_cast<__bf16>(vv[3])};
    } else {
      put((m == 0 ? dQ : dW) + 16 * rt * LD + 16 * ct, LD, vv);
    }
  }

  {
    t_g.pin_all();
    t_p.pin_all();
    t_tb.pin_all();
    t_k.pin_all();
    // Kg = k e^G (same element order in both tiles)
#pragma unroll
    for (int j = 0; j < t_g.PER; ++j) {
      const f32x4_t kv = t_k.get(j, p.nrow);
#pragma unroll
      for (int i = 0; i < 4; ++i) t_g.r[j][i] = kv[i] * fexp(t_g.r[j][i]);
    }
    if constexpr (BF) {
#pragma unroll
      for (int j = 0; j < t_g.PER; ++j) {   // element order of GTile<512, 64, D>
        const int e = tid + j * kNnThreads, rr = e / (D / 4), c = (e - rr * (D / 4)) * 4;
        *reinterpret_cast<bf16x4_t*>(KgB + rr * LDB + c) =
            bf16x4_t{static_cast<__bf16>(t_g.r[j][0]), static_cast<__bf16>(t_g.r[j][1]),
                     static_cast<__bf16>(t_g.r[j][2]), static_cast<__bf16>(t_g.r[j][3])};
      }
#pragma unroll
      for (int j = 0; j < t_p.PER; ++j) {   // element order of GTile<512, 64, 64>
        const int e = tid + j * kNnThreads, rr = e / (CR / 4), c = (e - rr * (CR / 4)) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          PT[(c + i) * LT + rr] = static_cast<__bf16>(t_p.r[j][i]);
          TBT[(c + i) * LT + rr] = static_cast<__bf16>(t_tb.r[j][i]);
        }
      }
    } else {
      t_g.store(Kg, LD);
      t_p.store(Ps, LS);
    }
    t_tb.store(TBs, LS);
    __syncthreads();

    // dP_tot = dP - dQ' Kg^T and dTb_part = dTb + dW Kg^T (tiles wave + 8x)
    f32x4_t dPt[2], dTt[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = wave + 8 * x, rt = j >> 2, ct = j & 3;
      f32x4_t qk, wk;
      if constexpr (BF) {
        qk = mmb<D>(zero4(), dQB + 16 * rt * LDB, LDB, KgB + 16 * ct * LDB, LDB);
        wk = mmb<D>(zero4(), dWB + 16 * rt * LDB, LDB, KgB + 16 * ct * LDB, LDB);
      } else {
        qk = mmx<BF, false, true>(zero4(), dQ + 16 * rt * LD, LD, Kg + 16 * ct * LD, LD, D);
        wk = mmx<BF, false, true>(zero4(), dW + 16 * rt * LD, LD, Kg + 16 * ct * LD, LD, D);
      }
      dPt[x] = acc[DT::XP + x];
      dTt[x] = acc[DT::XP + 2 + x];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dPt[x][i] -= qk[i];
        dTt[x][i] += wk[i];
      }
    }
    // dKg = -P^T dQ' + Tb^T dW, kept in registers for the decayed-product stage
    f32x4_t dkg[DT::NBIG / 8];
#pragma unroll
    for (int x = 0; x < DT::NBIG / 8; ++x) {
      const int j = wave + 8 * x, rt = j / CT, ct = j - rt * CT;
      f32x4_t pq;
      if constexpr (BF) {
        pq = mmb<CR>(zero4(), PT + 16 * rt * LT, LT, dQT + 16 * ct * LT, LT);
        dkg[x] = mmb<CR>(zero4(), TBT + 16 * rt * LT, LT, dWT + 16 * ct * LT, LT);
      } else {
        pq = mmx<BF, true, false>(zero4(), Ps + 16 * rt, LS, dQ + 16 * ct, LD, CR);
        dkg[x] = mmx<BF, true, false>(zero4(), TBs + 16 * rt, LS, dW + 16 * ct, LD, CR);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) dkg[x][i] -= pq[i];
    }
    __syncthreads();

#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = wave + 8 * x, rt = j >> 2, ct = j & 3;
      put(B0 + 16 * rt * LS + 16 * ct, LS, dPt[x]);
    }
    t_m.store(B1, LS);
    t_ti.store(B2, LS);
    if (tid < CR) BT[tid] = tid < p.nrow ? bt0 : 0.f;
    __syncthreads();
    // dTb_tot = dTb_part + scale M'^T dP_tot;  dM' = scale (dP_tot Tb^T) on s <= t
    f32x4_t dmv[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = wave + 8 * x, rt = j >> 2, ct = j & 3;
      const f32x4_t mp = mmx<BF, true, false>(zero4(), B1 + 16 * rt, LS, B0 + 16 * ct, LS, CR);
      dmv[x] = mmx<BF, false, true>(zero4(), B0 + 16 * rt * LS, LS, TBs + 16 * ct * LS, LS, CR);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rt + 4 * g4 + i, s = 16 * ct + l16;
        dTt[x][i] += scale * mp[i];
        dmv[x][i] = s <= t ? scale * dmv[x][i] : 0.f;
      }
      put(B3 + 16 * rt * LS + 16 * ct, LS, dTt[x]);
      f32x4_t dti = dTt[x];
      const float bc = BT[16 * ct + l16];
#pragma unroll
      for (int i = 0; i < 4; ++i) dti[i] *= bc;
      put(B4 + 16 * rt * LS + 16 * ct, LS, dti);
    }
    __syncthreads();
    // dbeta_s (through Tb = Ti Diag(beta)) = sum_t Ti[t,s] dTb_tot[t,s]
    float db = 0.f;
    if (tid < CR) {
      for (int t = 0; t < CR; ++t) db += B2[t * LS + tid] * B3[t * LS + tid];
    }
    f32x4_t X[2];   // X = dTi Ti^T
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = wave + 8 * x, rt = j >> 2, ct = j & 3;
      X[x] = mmx<BF, false, true>(zero4(), B4 + 16 * rt * LS, LS, B2 + 16 * ct * LS, LS, CR);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = wave + 8 * x, rt = j >> 2, ct = j & 3;
      put(B0 + 16 * rt * LS + 16 * ct, LS, X[x]);
      put(dMs + 16 * rt * LS + 16 * ct, LS, dmv[x]);   // Tb is no longer read
    }
    t_ap.store(B3, LS);
    // the decayed products' G, k and q, in flight while the algebra finishes
    const TIn* qc = q + p.row0 * D;
    const TIn* kc = k + p.row0 * D;
    GTile<kNnThreads, CR, D> t_gg;
    ITile4<kNnThreads, D, TIn> t_kk, t_qq;
    t_gg.load(w + L::G, D);
    t_kk.load(kc, rs, p.nrow);
    t_qq.load(qc, rs, p.nrow);
    __syncthreads();
    // dA = -Ti^T X on s < t;  dA' = Diag(beta) dA
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = wave + 8 * x, rt = j >> 2, ct = j & 3;
      f32x4_t da = mmx<BF, true, false>(zero4(), B2 + 16 * rt, LS, B0 + 16 * ct, LS, CR);
      f32x4_t dap;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rt + 4 * g4 + i, s = 16 * ct + l16;
        da[i] = s < t ? -da[i] : 0.f;
        dap[i] = BT[t] * da[i];
      }
      put(B1 + 16 * rt * LS + 16 * ct, LS, da);
      put(dAs + 16 * rt * LS + 16 * ct, LS, dap);
    }
    __syncthreads();
    if (tid < p.nrow) {   // dbeta_t (through A = Diag(beta) A') += sum_s dA[t,s] A'[t,s]
      for (int s = 0; s < CR; ++s) db += B1[tid * LS + s] * B3[tid * LS + s];
      dbeta[p.row0 + static_cast<int64_t>(tid) * H] = Elem<TIn>::from(db);
    }
    __syncthreads();

    // ---- decayed products of dA' and dM' with k and q, then dq, dk and dg.  Every
    // product here stays on fp32 operands, also for bf16 inputs: dG combines the
    // row-side and column-side products with opposite signs (X_A - Z_A - Z_M), and
    // with bf16 operands that cancellation took dg past its tolerance.
    if (tid < D) {
#pragma unroll
      for (int I = 0; I < 4; ++I) Rf[I * D + tid] = w[L::G + (16 * I + 15) * D + tid];
      for (int I = 1; I < 4; ++I)
        for (int J = 0; J < I; ++J)
          FP[pair_index(I, J) * D + tid] = fexp(Rf[I * D + tid] - Rf[J * D + tid]);
    }
    {
      t_gg.pin_all();
      t_kk.pin_all();
      t_qq.pin_all();
      __syncthreads();   // Rf
      // k colf, k rowf, q rowf (same element order in the three tiles)
#pragma unroll
      for (int j = 0; j < t_gg.PER; ++j) {
        const int e = tid + j * kNnThreads, t = e / (D / 4), i0 = (e - t * (D / 4)) * 4;
        const f32x4_t kv = t_kk.get(j, p.nrow), qv = t_qq.get(j, p.nrow);
        f32x4_t ki, ko, qo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float G = t_gg.r[j][i], RI = Rf[(t >> 4) * D + i0 + i];
          const float rowf = fexp(G - RI), colf = fexp(RI - G);
          ki[i] = kv[i] * colf;
          ko[i] = kv[i] * rowf;
          qo[i] = qv[i] * rowf;
        }
        *reinterpret_cast<f32x4_t*>(Ki + t * LD + i0) = ki;
        *reinterpret_cast<f32x4_t*>(Ko + t * LD + i0) = ko;
        *reinterpret_cast<f32x4_t*>(Qo + t * LD + i0) = qo;
      }
    }
    __syncthreads();

    // Output tile (R, cc) of the 64 x D results (the tiles of dQ', dKt, dKg above);
    // X-side sums run over column sub-tiles J <= R, Z-side sums over row sub-tiles I >= R.
    constexpr int NTD = DT::NBIG / 8;
    f32x4_t xa[NTD], xm[NTD], za[NTD], zm[NTD];
#pragma unroll
    for (int x = 0; x < NTD; ++x) {
      const int j = wave + 8 * x, R = j / CT, cc = j - R * CT;
      xa[x] = xm[x] = za[x] = zm[x] = zero4();
      for (int J = 0; J <= R; ++J) {
        const float* kb = Ki + 16 * J * LD + 16 * cc;
        const f32x4_t ta = mm<false, false>(zero4(), dAs + 16 * R * LS + 16 * J, LS, kb, LD, 16);
        const f32x4_t tm = mm<false, false>(zero4(), dMs + 16 * R * LS + 16 * J, LS, kb, LD, 16);
        const float f = J < R ? FP[pair_index(R, J) * D + 16 * cc + l16] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xa[x][i] += f * ta[i];
          xm[x][i] += f * tm[i];
        }
      }
      for (int I = R; I < 4; ++I) {
        const f32x4_t ta = mm<true, false>(zero4(), dAs + 16 * I * LS + 16 * R, LS,
                                           Ko + 16 * I * LD + 16 * cc, LD, 16);
        const f32x4_t tm = mm<true, false>(zero4(), dMs + 16 * I * LS + 16 * R, LS,
                                           Qo + 16 * I * LD + 16 * cc, LD, 16);
        const float f = I > R ? FP[pair_index(I, R) * D + 16 * cc + l16] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          za[x][i] += f * ta[i];
          zm[x][i] += f * tm[i];
        }
      }
    }
    __syncthreads();
    // the element inputs of two tiles are loaded first (rows clamped into the chunk,
    // all loads in flight together), then those elements are formed and stored
    constexpr int XG = 2;
    const uint32_t rsb = static_cast<uint32_t>(H) * D * static_cast<uint32_t>(sizeof(TIn));
    const uint32_t range = (p.nrow - 1) * rsb + D * static_cast<uint32_t>(sizeof(TIn));
    const auto rdq = make_rsrc(dq + p.row0 * D, range);
    const auto rdk = make_rsrc(dk + p.row0 * D, range);
#pragma unroll
    for (int x0 = 0; x0 < NTD; x0 += XG) {
      float eG[XG][4], eq[XG][4], ek[XG][4];
#pragma unroll
      for (int xx = 0; xx < XG; ++xx) {
        const int j = wave + 8 * (x0 + xx), R = j / CT, cc = j - R * CT;
        const int col = 16 * cc + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * R + 4 * g4 + i;
          const int tc = min(t, p.nrow - 1);
          eG[xx][i] = w[L::G + t * D + col];
          eq[xx][i] = to_f32(qc[tc * rs + col]);
          ek[xx][i] = to_f32(kc[tc * rs + col]);
        }
      }
#pragma unroll
      for (int xx = 0; xx < XG; ++xx) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pin(eG[xx][i]);
          pin(eq[xx][i]);
          pin(ek[xx][i]);
        }
      }
#pragma unroll
      for (int xx = 0; xx < XG; ++xx) {
        const int x = x0 + xx, j = wave + 8 * x, R = j / CT, cc = j - R * CT;
        const int col = 16 * cc + l16;
        const float RI = Rf[R * D + col], Gl = Rf[3 * D + col];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * R + 4 * g4 + i;
          const float G = eG[xx][i];
          const float rowf = fexp(G - RI), colf = fexp(RI - G), eg = fexp(G), et = fexp(Gl - G);
          const float XA = rowf * xa[x][i], XM = rowf * xm[x][i];
          const float ZA = colf * za[x][i], ZM = colf * zm[x][i];
          const bool ok = t < p.nrow;
          const float kv = ok ? ek[xx][i] : 0.f, qv = ok ? eq[xx][i] : 0.f;
          const float dKg = dkg[x][i], dKt = acc[2 * NTD + x][i];
          const float dqv = scale * acc[x][i] * eg + XM;
          const float kg = dKg * eg, kt = dKt * et;
          const float dkv = kg + kt + XA + ZA + ZM;
          Ko[t * LD + col] = qv * dqv + kv * (kg + XA - kt - ZA - ZM);
          Qo[t * LD + col] = kv * kt;
          // rows past the chunk's end fall outside the store ranges (no branch)
          const uint32_t off = t * rsb + col * static_cast<uint32_t>(sizeof(TIn));
          store_elem(Elem<TIn>::from(dqv), rdq, off);
          store_elem(Elem<TIn>::from(dkv), rdk, off);
        }
      }
    }
    __syncthreads();
    // dg = reverse running sum of dG plus the last row's terms (dlam Lambda and the
    // sum of the Qo column), in 512 / D row segments per column: segment sums to LDS
    // (over k colf, dead since the pair products), then each thread runs its own rows
    // from the sums of the segments below it.
    {
      constexpr int NSEG = kNnThreads / D, SR = CR / NSEG;
      static_assert(NSEG * D == kNnThreads && NSEG * SR == CR, "dg segments");
      const int c = tid % D, sg = tid / D, t0 = SR * sg;
      float* segq = Ki;                 // [NSEG][D] column sums of Qo per segment
      float* segk = Ki + NSEG * D;      // [NSEG][D] column sums of Ko per segment
      float* base = Ki + 2 * NSEG * D;  // [D] dlam Lambda (dlam lives in threads < D)
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int t = 0; t < SR; ++t) {
        sq += Qo[(t0 + t) * LD + c];
        sk += Ko[(t0 + t) * LD + c];
      }
      segq[sg * D + c] = sq;
      segk[sg * D + c] = sk;
      if (tid < D) base[tid] = dlam * w[L::LAM + tid];
      __syncthreads();
      const auto rdg = make_rsrc(dg + p.row0 * D, range);   // rows past the end: dropped
      float run = base[c];
#pragma unroll
      for (int u = 0; u < NSEG; ++u) run += segq[u * D + c] + (u > sg ? segk[u * D + c] : 0.f);
#pragma unroll
      for (int t = SR - 1; t >= 0; --t) {
        run += Ko[(t0 + t) * LD + c];
        store_elem(Elem<TIn>::from(run), rdg, (t0 + t) * rsb + c * static_cast<uint32_t>(sizeof(TIn)));
      }
    }
  }
}

// Chunk items of a backward call: fixed length, every chunk of every stream; packed,
// the slot numbering of the forward (some items unused).
inline int64_t backward_items(const BackwardArgs& a) {
  const int nc = a.cu_seqlens == nullptr ? (a.T + CR - 1) / CR : 0;
  return a.cu_seqlens == nullptr ? static_cast<int64_t>(a.B) * a.H * nc
                                 : (static_cast<int64_t>(a.total_T + CR - 1) / CR + a.B) * a.H;
}

// Most chunks any sequence of the call can have (for packed input the lengths are on
// the device: ceil(total_T / 64) bounds them).
inline int backward_chunks_max(const BackwardArgs& a) {
  return a.cu_seqlens == nullptr ? (a.T + CR - 1) / CR : (a.total_T + CR - 1) / CR;
}

// Floats of workspace per chunk item: the fp32 operands, then the states, state
// gradients, Delta and dU (fp32, or bf16 for bf16 inputs: half the floats), then for
// bf16 inputs the bf16 scan operands.
template <int D, typename TIn>
constexpr int64_t backward_floats_per_item() {
  using L = BwdLayout<D>;
  constexpr bool BF = IsBf16<TIn>::value;
  return L::WS + (BF ? 1 : 2) * (D * D + CR * D) + (BF ? L::WSB / 2 : 0);
}

// Workspace bytes with windows of cw chunks (cw = 0: every chunk at once).  A window
// holds its chunks' items, plus, over the call, the state at the start of every window
// but the first and two state-gradient buffers.
template <int D, typename TIn>
size_t backward_bytes_t(const BackwardArgs& a, int cw) {
  const int64_t items = cw == 0 ? backward_items(a) : static_cast<int64_t>(a.B) * a.H * cw;
  int64_t floats = items * backward_floats_per_item<D, TIn>();
  if (cw > 0) {
    const int64_t nwin = (backward_chunks_max(a) + cw - 1) / cw;
    floats += (nwin - 1 + 2) * a.B * a.H * D * D;
  }
  return static_cast<size_t>(floats) * sizeof(float);
}

size_t backward_bytes(const BackwardArgs& a, int cw) {
  if (a.d == 128) return a.dtype_f32 ? backward_bytes_t<128, float>(a, cw) : backward_bytes_t<128, bf16_t>(a, cw);
  return a.dtype_f32 ? backward_bytes_t<64, float>(a, cw) : backward_bytes_t<64, bf16_t>(a, cw);
}

// Windowed form of the backward (cw > 0 chunks per window, fewer than the longest
// sequence has): a first pass walks the windows forwards, each computing its chunks'
// operands and its forward scan from the state the previous window ended with, and
// keeps only that end state; the second pass walks the windows backwards, recomputing
// each window's operands and forward scan from its stored start state, then its
// reverse scan (from the state gradient the later window left) and its gradients.
// The result equals the one-pass backward's up to rounding; the workspace no longer
// grows with the sequence but by one state per window.
template <int D, typename TIn>
hipError_t launch_backward_t(const BackwardArgs& a) {
  using L = BwdLayout<D>;
  const int nc = a.cu_seqlens == nullptr ? (a.T + CR - 1) / CR : 0;
  const SeqMap sm{a.cu_seqlens, a.B, a.T, a.cu_seqlens == nullptr ? a.B * a.T : a.total_T, a.H, nc};
  const int nc_max = backward_chunks_max(a);
  const int cw = a.window_chunks > 0 && a.window_chunks < nc_max ? a.window_chunks : 0;
  const int nwin = cw == 0 ? 1 : (nc_max + cw - 1) / cw;
  const int64_t items = cw == 0 ? backward_items(a) : static_cast<int64_t>(a.B) * a.H * cw;
  constexpr bool BF = IsBf16<TIn>::value;
  const int64_t sdu = (BF ? 1 : 2) * (D * D + CR * D);
  char* raw = nullptr;
  hipError_t err = ws_acquire(a.workspace, a.workspace_bytes, backward_bytes_t<D, TIn>(a, cw),
                              a.stream, &raw);
  if (err != hipSuccess) return err;
  float* ws = reinterpret_cast<float*>(raw);
  float* sreg = ws + items * L::WS;   // S, dS, Delta, dU in the element type chosen above
  __bf16* wsb = BF ? reinterpret_cast<__bf16*>(sreg + items * sdu) : nullptr;
  float* st = sreg;
  float* dst = st + items * D * D;
  float* dl = dst + items * D * D;
  float* du = dl + items * CR * D;
  __bf16* sb = reinterpret_cast<__bf16*>(sreg);
  __bf16* stb = sb;
  __bf16* dstb = stb + items * D * D;
  __bf16* dlb = dstb + items * D * D;
  __bf16* dub = dlb + items * CR * D;
  const int BH = a.B * a.H;
  const int64_t state = static_cast<int64_t>(D) * D;
  float* ckpt = ws + items * backward_floats_per_item<D, TIn>();   // windows 1 .. nwin - 1
  float* pp = ckpt + static_cast<int64_t>(nwin - 1) * BH * state;  // two dS buffers
  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
  const TIn* v = static_cast<const TIn*>(a.v);
  const TIn* g = static_cast<const TIn*>(a.g);
  const TIn* beta = static_cast<const TIn*>(a.beta);
  const TIn* dout = static_cast<const TIn*>(a.d_out);
  const int scan_blocks = scan_grid(BH, D / SL);
  const unsigned grid = static_cast<unsigned>(items);
  // one window: operands and forward scan from s0 (end state to s_end if given); with
  // `grads`, then the reverse scan from dsT (state gradient at its start to ds0) and
  // the gradients
  auto window = [&](const SeqMap& m, const float* s0, float* s_end, bool grads, const float* dsT,
                    float* ds0) {
    KDA_TRY_LAUNCH(err, (chunk_ops_kernel<D, TIn, false, true>), dim3(grid), dim3(kOpsThreads), 0,
                   a.stream, q, k, g, beta, ws, wsb, m, a.scale);
    if constexpr (IsBf16<TIn>::value) {
      KDA_TRY_LAUNCH(err, (bwd_fwd_scan_bf16_kernel<D>), dim3(scan_blocks), dim3(kScanThreads), 0,
                     a.stream, v, s0, ws, wsb, stb, dlb, m, BH, s_end);
      if (!grads) return;
      KDA_TRY_LAUNCH(err, (bwd_scan_bf16_kernel<D>), dim3(scan_blocks), dim3(kScanThreads), 0,
                     a.stream, dout, dsT, ws, wsb, dstb, dub, static_cast<TIn*>(a.dv), ds0, m, BH);
      KDA_TRY_LAUNCH(err, (bwd_grad_chunk_kernel<D, TIn>), dim3(grid), dim3(kNnThreads), 0, a.stream,
                     q, k, beta, v, dout, stb, dstb, dlb, dub, ws, static_cast<TIn*>(a.dq),
                     static_cast<TIn*>(a.dk), static_cast<TIn*>(a.dg), static_cast<TIn*>(a.dbeta),
                     m, a.scale);
    } else {
      KDA_TRY_LAUNCH(err, (bwd_fwd_scan_kernel<D, TIn>), dim3(scan_blocks), dim3(kScanThreads), 0,
                     a.stream, v, s0, ws, st, dl, m, BH, s_end);
      if (!grads) return;
      KDA_TRY_LAUNCH(err, (bwd_scan_kernel<D, TIn>), dim3(scan_blocks), dim3(kScanThreads), 0,
                     a.stream, dout, dsT, ws, dst, du, static_cast<TIn*>(a.dv), ds0, m, BH);
      KDA_TRY_LAUNCH(err, (bwd_grad_chunk_kernel<D, TIn>), dim3(grid), dim3(kNnThreads), 0, a.stream,
                     q, k, beta, v, dout, st, dst, dl, du, ws, static_cast<TIn*>(a.dq),
                     static_cast<TIn*>(a.dk), static_cast<TIn*>(a.dg), static_cast<TIn*>(a.dbeta),
                     m, a.scale);
    }
  };
  if (cw == 0) {
    window(sm, a.initial_state, nullptr, true, a.d_final_state, a.d_initial_state);
  } else {
    auto wmap = [&](int w) {
      SeqMap m = sm;
      m.c_lo = w * cw;
      m.cw = cw;
      return m;
    };
    auto start = [&](int w) -> const float* { return w == 0 ? a.initial_state : ckpt + (w - 1) * BH * state; };
    for (int w = 0; w + 1 < nwin && err == hipSuccess; ++w)
      window(wmap(w), start(w), ckpt + static_cast<int64_t>(w) * BH * state, false, nullptr, nullptr);
    for (int w = nwin - 1; w >= 0 && err == hipSuccess; --w)
      window(wmap(w), start(w), nullptr, true,
             w == nwin - 1 ? a.d_final_state : pp + static_cast<int64_t>((w + 1) & 1) * BH * state,
             w == 0 ? a.d_initial_state : pp + static_cast<int64_t>(w & 1) * BH * state);
  }
  const hipError_t ferr = ws_release(a.workspace, raw, a.stream);
  return err != hipSuccess ? err : ferr;
}

}  // namespace

size_t backward_workspace_bytes(const BackwardArgs& a) {
  const int nc_max = backward_chunks_max(a);
  return backward_bytes(a, a.window_chunks > 0 && a.window_chunks < nc_max ? a.window_chunks : 0);
}

int backward_fit_window(const BackwardArgs& a, size_t bytes) {
  const int nc_max = backward_chunks_max(a);
  if (bytes >= backward_bytes(a, 0)) return 0;
  for (int cw = nc_max - 1; cw >= 1; --cw)
    if (backward_bytes(a, cw) <= bytes) return cw;
  return -1;
}

hipError_t launch_backward(const BackwardArgs& a) {
  if (a.d == 128) {
    return a.dtype_f32 ? launch_backward_t<128, float>(a) : launch_backward_t<128, bf16_t>(a);
  }
  return a.dtype_f32 ? launch_backward_t<64, float>(a) : launch_backward_t<64, bf16_t>(a);
}


}  // namespace kda
