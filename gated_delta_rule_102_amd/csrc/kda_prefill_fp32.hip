// fp32 prefill at dk = dv = 128.  The bf16 kernels' operand tiles do not fit this
// precision at this head size (the preparation's swizzled fp32 rows and its register
// layout assume at most 16 KB per 64-row tile), so fp32 inputs at d = 128 take the
// chunk operands of kda_chunk_ops.h -- the same per-chunk affine map the backward
// runs on (neurohive.io Kimi K3 review, section "Sequence length: hybrid KDA and
// Gated MLA attention")
//     Delta = Tb V - W S,   O = Q' S + P V,   S <- Diag(Lambda) S + Kt^T Delta,
// all on fp32 operands (16x16x4 matrix cores): chunk_ops_kernel forms Tb, W, Q', P,
// Kt, Lambda for a window of chunks, then exact_scan_kernel walks the window's chunks
// per (sequence, head, 32 value columns), writing the outputs and carrying the state
// to the next window through a [N, H, d, d] fp32 buffer.

#include "kda_chunk_ops.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kExactWindow = 16;   // chunks per window unless the caller's workspace asks fewer

// The forward scan of the backward (kda_backward.hip) with the chunk outputs added: per
// chunk, S to LDS, then Delta and O (one 16 x 16 tile of each per wavefront, Q' and P
// read from the workspace), then the state update.  s0 may alias s_end: each workgroup
// reads its own columns of s0 first and writes the same columns of s_end last.
template <int D>
__global__ __launch_bounds__(kScanThreads) void exact_scan_kernel(const float* __restrict__ v,
                                                                 const float* s0,
                                                                 const float* __restrict__ ws,
                                                                 float* __restrict__ out,
                                                                 float* s_end, SeqMap m, int BH) {
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
  GTile<kScanThreads, CR, CR> t_tb;
  GTile<kScanThreads, CR, D> t_w, t_kt;
  ITile<kScanThreads, SL, float> t_v;
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
    const float* w = ws + (sp.item0 + c * sp.istride) * L::WS;
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
    issue(min(c + 1, sp.nch - 1));   // unconditional: the last step reloads its own chunk
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(Ss + 16 * rt * LV + 16 * ct, LV, S[x]);
    }
    __syncthreads();
    {   // Delta = Tb V - W S and O = Q' S + P V: 4 x 2 tiles each, one of each per wavefront
      const int rt = wave >> 1, ct = wave & 1;
      const f32x4_t tv = mm<false, false>(zero4(), TBs + 16 * rt * LS, LS, Vs + 16 * ct, LV, CR);
      const f32x4_t wsv = mm<false, false>(zero4(), Ws + 16 * rt * LD, LD, Ss + 16 * ct, LV, D);
      f32x4_t d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = tv[i] - wsv[i];
      put(Dls + 16 * rt * LV + 16 * ct, LV, d);
      f32x4_t o = mm<false, false>(zero4(), w + L::QP + 16 * rt * D, D, Ss + 16 * ct, LV, D);
      o = mm<false, false>(o, w + L::PP + 16 * rt * CR, CR, Vs + 16 * ct, LV, CR);
      const int nrow = min(CR, sp.len - c * CR);
      const int64_t row0 = static_cast<int64_t>(sp.tok0) + static_cast<int64_t>(c) * CR;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rt + 4 * g4 + i;
        if (t < nrow) out[((row0 + t) * H + h) * D + c0 + 16 * ct + l16] = o[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {   // S = Lam S + Kt^T Delta
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      f32x4_t acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Lm[16 * rt + 4 * g4 + i] * S[x][i];
      S[x] = mm<true, false>(acc, KTs + 16 * rt, LD, Dls + 16 * ct, LV, CR);
    }
    __syncthreads();
  }
  if (s_end) {
#pragma unroll
    for (int x = 0; x < ST::NTW; ++x) {
      const int rt = ST::rt(wave, x), ct = ST::ct(wave, x);
      put(s_end + static_cast<int64_t>(bh) * D * D + 16 * rt * D + c0 + 16 * ct, D, S[x]);
    }
  }
  (void)l16;
}

int exact_chunks_max(const PrefillArgs& a) {
  return a.cu_seqlens == nullptr ? (a.T + CR - 1) / CR : (a.total_T + CR - 1) / CR;
}

int exact_window(const PrefillArgs& a) {
  const int nc = exact_chunks_max(a);
  const int cw = a.window_chunks > 0 ? a.window_chunks : kExactWindow;
  return cw < nc ? cw : (nc > 0 ? nc : 1);
}

size_t exact_bytes(const PrefillArgs& a, int cw) {
  using L = BwdLayout<128>;
  const int64_t bh = static_cast<int64_t>(a.N) * a.H;
  return static_cast<size_t>(bh * cw * L::WS + bh * 128 * 128) * sizeof(float);
}

}  // namespace

bool exact_prefill_path(const PrefillArgs& a) { return a.dtype_f32 && a.d == 128; }

size_t exact_prefill_workspace_bytes(const PrefillArgs& a) { return exact_bytes(a, exact_window(a)); }

int exact_prefill_fit_window(const PrefillArgs& a, size_t bytes) {
  for (int cw = exact_chunks_max(a); cw >= 1; --cw)
    if (exact_bytes(a, cw) <= bytes) return cw;
  return 0;
}

const char* exact_prefill_schedule(const PrefillArgs& a) {
  static thread_local char buf[160];
  const int cw = exact_window(a);
  std::snprintf(buf, sizeof buf,
                "chunk_ops_kernel<128,f32> + exact_scan_kernel<128> x %d windows of %d chunks",
                (exact_chunks_max(a) + cw - 1) / cw, cw);
  return buf;
}

hipError_t launch_exact_prefill(const PrefillArgs& a) {
  constexpr int D = 128;
  using L = BwdLayout<D>;
  const int nc_max = exact_chunks_max(a);
  if (nc_max == 0) return hipSuccess;
  const int cw = exact_window(a);
  const int nwin = (nc_max + cw - 1) / cw;
  const int BH = a.N * a.H;
  const int64_t items = static_cast<int64_t>(BH) * cw;
  char* raw = nullptr;
  hipError_t err = ws_acquire(a.workspace, a.workspace_bytes, exact_bytes(a, cw), a.stream, &raw);
  if (err != hipSuccess) return err;
  float* ws = reinterpret_cast<float*>(raw);
  float* carry = ws + items * L::WS;   // the state between windows
  const SeqMap sm{a.cu_seqlens, a.N, a.T, a.cu_seqlens == nullptr ? a.N * a.T : a.total_T, a.H,
                  a.cu_seqlens == nullptr ? (a.T + CR - 1) / CR : 0};
  const float* q = static_cast<const float*>(a.q);
  const float* k = static_cast<const float*>(a.k);
  const float* g = static_cast<const float*>(a.g);
  const float* beta = static_cast<const float*>(a.beta);
  for (int w = 0; w < nwin && err == hipSuccess; ++w) {
    SeqMap m = sm;
    m.c_lo = w * cw;
    m.cw = cw;
    KDA_TRY_LAUNCH(err, (chunk_ops_kernel<D, float, false, true>), dim3(static_cast<unsigned>(items)),
                   dim3(kOpsThreads), 0, a.stream, q, k, g, beta, ws, nullptr, m, a.scale);
    KDA_TRY_LAUNCH(err, (exact_scan_kernel<D>), dim3(scan_grid(BH, D / SL)), dim3(kScanThreads), 0,
                   a.stream, static_cast<const float*>(a.v), w == 0 ? a.initial_state : carry, ws,
                   static_cast<float*>(a.out), w == nwin - 1 ? a.final_state : carry, m, BH);
  }
  const hipError_t ferr = ws_release(a.workspace, raw, a.stream);
  return err != hipSuccess ? err : ferr;
}

}  // namespace kda
