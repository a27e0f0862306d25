// Per-chunk operands of chunked KDA in fp32, and the fp32 matrix-core helpers
// the backward pass and the context-parallel building blocks share.
//
// Per (sequence, head), every 64-token chunk is an affine map of the entering
// state S and the chunk's values V (neurohive.io Kimi K3 review, section
// "Sequence length: hybrid KDA and Gated MLA attention": a delta rule that
// forgets per key channel and writes per token), with operands that depend only
// on the chunk's q, k, g, beta (G = running sum of g inside the chunk):
//     A'[t,s] = sum_c k_tc k_sc e^{G_tc - G_sc} (s < t),  Ti = (I + Diag(beta) A')^-1
//     M'[t,s] = sum_c q_tc k_sc e^{G_tc - G_sc} (s <= t), Tb = Ti Diag(beta)
//     W = Tb (k e^G),  P = scale M' Tb,  Q' = scale q e^G - P (k e^G),
//     Kt = k e^{G_last - G},  Lam = e^{G_last}
//     Delta = Tb V - W S,   O = Q' S + P V,   S_next = Lam S + Kt^T Delta.
// chunk_ops_kernel writes these operands for every (chunk, head) to a workspace.
// Products run on the fp32 16x16x4 matrix cores from padded LDS tiles; decayed
// products use 16-row sub-tile references (G at each sub-tile's last row) so that
// every factor stays inside fp32's range when the log-decay is >= -5.
#pragma once

#include <type_traits>

#include "kda_device.h"

namespace kda {

namespace {

constexpr int CR = 64;    // rows per chunk
constexpr int SL = 32;    // value columns per scan workgroup / per contraction slice
constexpr int LS = 68;    // leading dimension of 64 x 64 LDS matrices
constexpr int LV = 36;    // leading dimension of 32-column LDS slices

template <int D>
struct BwdLayout {
  static constexpr int LD = D + 4;   // leading dimension of 64 x D LDS matrices
  // workspace per chunk, written by chunk_ops (floats, row-major; for bf16 inputs
  // W, QP and KT are written only as the bf16 copies below)
  static constexpr int TB = 0, TI = 4096, AP = 8192, MP = 12288, PP = 16384;
  static constexpr int W = 20480, QP = W + CR * D, KT = QP + CR * D, G = KT + CR * D;
  static constexpr int LAM = G + CR * D, WS = LAM + D;
  // bf16 copies of the scan operands per chunk, written by chunk_ops for bf16
  // inputs (bf16 elements), each in the layout a scan reads k-contiguously:
  // Tb, Tb^T, P^T, W, W^T, Kt, Kt^T, Q'^T
  static constexpr int BTB = 0, BTBT = 4096, BPT = 8192, BW = 12288, BWT = BW + CR * D;
  static constexpr int BKT = BWT + CR * D, BKTT = BKT + CR * D, BQPT = BKTT + CR * D;
  static constexpr int WSB = BQPT + CR * D;
};

__device__ __forceinline__ int lane16() { return threadIdx.x & 15; }
__device__ __forceinline__ int lane_g4() { return (threadIdx.x >> 4) & 3; }

// acc += op(A) op(B) for one 16 x 16 output tile; K is a multiple of 16.
//   op(A)(r, k) = TA ? a[k * lda + r] : a[r * lda + k]     (r < 16, k < K)
//   op(B)(k, c) = TB ? b[c * ldb + k] : b[k * ldb + c]     (c < 16)
// With KS, op(A)(r, k) is multiplied by ks[k].  At step j of each 16-wide block
// lane (g4, l16) feeds A(l16, k0 + 4 g4 + j) and B(k0 + 4 g4 + j, l16); the
// result is acc[i] = C(4 g4 + i, l16).
template <bool TA, bool TB, bool KS = false>
__device__ __forceinline__ f32x4_t mm(f32x4_t acc, const float* a, int lda, const float* b,
                                      int ldb, int K, const float* ks = nullptr) {
  const int l16 = lane16(), g4 = lane_g4();
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int kb = k0 + 4 * g4;
    float av[4], bv[4];
    if constexpr (TA) {
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = a[(kb + j) * lda + l16];
    } else {
      const float4 t = *reinterpret_cast<const float4*>(a + l16 * lda + kb);
      av[0] = t.x; av[1] = t.y; av[2] = t.z; av[3] = t.w;
    }
    if constexpr (TB) {
      const float4 t = *reinterpret_cast<const float4*>(b + l16 * ldb + kb);
      bv[0] = t.x; bv[1] = t.y; bv[2] = t.z; bv[3] = t.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = b[(kb + j) * ldb + l16];
    }
    if constexpr (KS) {
      const float4 s = *reinterpret_cast<const float4*>(ks + kb);
      av[0] *= s.x; av[1] *= s.y; av[2] *= s.z; av[3] *= s.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc, 0, 0, 0);
  }
  return acc;
}

// mm with bf16 operands when BF: the fp32 LDS operands are rounded to bf16 (round
// to nearest even) and fed to the 16x16x32 bf16 matrix cores with fp32
// accumulation, 8x the work per instruction of the fp32 16x16x4 form.  K is a
// multiple of 32; lane (g4, l16) feeds A(l16, k0 + 8 g4 + j) and
// B(k0 + 8 g4 + j, l16), j < 8, and the result layout is mm's.
template <bool BF, bool TA, bool TB, bool KS = false>
__device__ __forceinline__ f32x4_t mmx(f32x4_t acc, const float* a, int lda, const float* b,
                                       int ldb, int K, const float* ks = nullptr) {
  if constexpr (!BF) {
    return mm<TA, TB, KS>(acc, a, lda, b, ldb, K, ks);
  } else {
    const int l16 = lane16(), g4 = lane_g4();
    for (int k0 = 0; k0 < K; k0 += 32) {
      const int kb = k0 + 8 * g4;
      float av[8], bv[8];
      if constexpr (TA) {
#pragma unroll
        for (int j = 0; j < 8; ++j) av[j] = a[(kb + j) * lda + l16];
      } else {
        const float4 t0 = *reinterpret_cast<const float4*>(a + l16 * lda + kb);
        const float4 t1 = *reinterpret_cast<const float4*>(a + l16 * lda + kb + 4);
        av[0] = t0.x; av[1] = t0.y; av[2] = t0.z; av[3] = t0.w;
        av[4] = t1.x; av[5] = t1.y; av[6] = t1.z; av[7] = t1.w;
      }
      if constexpr (TB) {
        const float4 t0 = *reinterpret_cast<const float4*>(b + l16 * ldb + kb);
        const float4 t1 = *reinterpret_cast<const float4*>(b + l16 * ldb + kb + 4);
        bv[0] = t0.x; bv[1] = t0.y; bv[2] = t0.z; bv[3] = t0.w;
        bv[4] = t1.x; bv[5] = t1.y; bv[6] = t1.z; bv[7] = t1.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = b[(kb + j) * ldb + l16];
      }
      if constexpr (KS) {
        const float4 s0 = *reinterpret_cast<const float4*>(ks + kb);
        const float4 s1 = *reinterpret_cast<const float4*>(ks + kb + 4);
        av[0] *= s0.x; av[1] *= s0.y; av[2] *= s0.z; av[3] *= s0.w;
        av[4] *= s1.x; av[5] *= s1.y; av[6] *= s1.z; av[7] *= s1.w;
      }
      bf16x8_t A, B;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        A[j] = static_cast<__bf16>(av[j]);
        B[j] = static_cast<__bf16>(bv[j]);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
    }
    return acc;
  }
}

// e^x on the hardware base-2 exponential: the arguments here lie in [-461, 110]
// (log-decay >= -5 per token, 16-row sub-tile references), so x * log2(e) never
// overflows and the relative error stays within a few 1e-6; results below fp32's
// normal range may flush to zero, where every use of them is negligible.
__device__ __forceinline__ float fexp(float x) { return fast_exp2(x * kLog2e); }

template <typename TIn>
struct IsBf16 { static constexpr bool value = false; };
template <>
struct IsBf16<bf16_t> { static constexpr bool value = true; };

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// tile (accumulator layout) <-> memory at the tile's origin with leading dimension ld
__device__ __forceinline__ void put(float* dst, int ld, const f32x4_t& v) {
  const int l16 = lane16(), g4 = lane_g4();
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(4 * g4 + i) * ld + l16] = v[i];
}
__device__ __forceinline__ f32x4_t get(const float* src, int ld) {
  const int l16 = lane16(), g4 = lane_g4();
  f32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[(4 * g4 + i) * ld + l16];
  return v;
}

// Pins a loaded value: the empty asm consumes and redefines it, so the load
// that produced it is issued before this point and cannot be sunk next to its
// use.  Pinning a group of tile loads keeps all of them in flight together.
template <typename V>
__device__ __forceinline__ void pin(V& v) { asm volatile("" : "+v"(v)); }

// ROWS x COLS fp32 global -> LDS (COLS % 4 == 0, both sides 16-byte aligned).
// load() issues every global load of the tile before store() writes LDS, so a
// thread has all its loads in flight at once; several tiles can be loaded
// before any of them is stored.
template <int NT, int ROWS, int COLS>
struct GTile {
  static constexpr int C4 = COLS / 4, N = ROWS * C4, PER = (N + NT - 1) / NT;
  f32x4_t r[PER];
  __device__ __forceinline__ void load(const float* src, int64_t gld) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT;
      if (N % NT == 0 || e < N) {
        const int rr = e / C4, c = (e - rr * C4) * 4;
        r[j] = *reinterpret_cast<const f32x4_t*>(src + rr * gld + c);
      }
    }
  }
  __device__ __forceinline__ void pin_all() {
#pragma unroll
    for (int j = 0; j < PER; ++j) pin(r[j]);
  }
  __device__ __forceinline__ void store(float* dst, int lld) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT;
      if (N % NT == 0 || e < N) {
        const int rr = e / C4, c = (e - rr * C4) * 4;
        *reinterpret_cast<f32x4_t*>(dst + rr * lld + c) = r[j];
      }
    }
  }
};
template <int NT, int ROWS, int COLS>
__device__ __forceinline__ void l2g(float* dst, int64_t gld, const float* src, int lld) {
  constexpr int C4 = COLS / 4, N = ROWS * C4;
#pragma unroll
  for (int j = 0; j < (N + NT - 1) / NT; ++j) {
    const int e = static_cast<int>(threadIdx.x) + j * NT;
    if (N % NT == 0 || e < N) {
      const int r = e / C4, c = (e - r * C4) * 4;
      *reinterpret_cast<float4*>(dst + r * gld + c) = *reinterpret_cast<const float4*>(src + r * lld + c);
    }
  }
}
// 64 x COLS input rows (bf16 or fp32) -> fp32 in LDS; rows >= nrow read as zero.
// The row index is clamped so every load is unconditional (a load under a
// branch is waited for inside the branch, which serialises the loads).  The
// elements stay raw until they are read (val, store): converting or masking them
// right after the load would wait for the load there, and a prefetch issued a step
// ahead would then be waited for at once.
template <int NT, int COLS, typename TIn>
struct ITile {
  static constexpr int N = CR * COLS, PER = N / NT;
  static_assert(N % NT == 0, "tile split");
  static constexpr bool BF = IsBf16<TIn>::value;
  using Raw = typename std::conditional<BF, uint32_t, float>::type;   // bf16: the bits
  Raw r[PER];
  int nrow_;
  __device__ __forceinline__ void load(const TIn* src, int64_t row_stride, int nrow) {
    nrow_ = nrow;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT;
      const int rr = e / COLS, c = e - rr * COLS;
      const TIn x = src[min(rr, nrow - 1) * row_stride + c];
      if constexpr (BF) r[j] = x.bits;
      else r[j] = x;
    }
  }
  __device__ __forceinline__ void pin_all() {
#pragma unroll
    for (int j = 0; j < PER; ++j) pin(r[j]);
  }
  // element j as fp32 (zero for rows past nrow)
  __device__ __forceinline__ float val(int j) const {
    const int rr = (static_cast<int>(threadIdx.x) + j * NT) / COLS;
    float x;
    if constexpr (BF) x = __uint_as_float(r[j] << 16);
    else x = r[j];
    return rr < nrow_ ? x : 0.f;
  }
  __device__ __forceinline__ void store(float* dst, int lld) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT;
      const int rr = e / COLS, c = e - rr * COLS;
      dst[rr * lld + c] = val(j);
    }
  }
};

// 64 x COLS input rows (bf16 or fp32) held as raw words, 4 consecutive elements per
// thread in the GTile<NT, 64, COLS> element order; rows >= nrow read as zero.
template <int NT, int COLS, typename TIn>
struct ITile4 {
  static constexpr int C4 = COLS / 4, N = CR * C4, PER = N / NT;
  static_assert(N % NT == 0, "tile split");
  static constexpr bool BF = IsBf16<TIn>::value;
  using Raw = typename std::conditional<BF, i32x2_t, f32x4_t>::type;
  Raw r[PER];
  __device__ __forceinline__ void load(const TIn* src, int64_t row_stride, int nrow) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT;
      const int rr = e / C4, c = (e - rr * C4) * 4;
      r[j] = *reinterpret_cast<const Raw*>(src + min(rr, nrow - 1) * row_stride + c);
    }
  }
  __device__ __forceinline__ void pin_all() {
#pragma unroll
    for (int j = 0; j < PER; ++j) pin(r[j]);
  }
  __device__ __forceinline__ f32x4_t get(int j, int nrow) const {
    const int rr = (static_cast<int>(threadIdx.x) + j * NT) / C4;
    f32x4_t x;
    if constexpr (BF) {
      const uint32_t w0 = static_cast<uint32_t>(r[j][0]), w1 = static_cast<uint32_t>(r[j][1]);
      x = f32x4_t{bf16lo(w0), bf16hi(w0), bf16lo(w1), bf16hi(w1)};
    } else {
      x = r[j];
    }
    return rr < nrow ? x : zero4();
  }
};

// Block id -> (sequence-head bh, first column c0) for the column-sliced scans.
// The NSL slices of one sequence-head get block ids that are equal mod 8, so the
// round-robin dispatch over the eight XCDs puts them on one XCD, whose L2 then
// serves their shared per-chunk operands once.  Grids have scan_grid(BH, NSL)
// blocks; a block past the last sequence-head gets false and returns at once.
template <int NSL>
__device__ __forceinline__ bool scan_block(int BH, int& bh, int& c0) {
  const int w = static_cast<int>(blockIdx.x), local = w >> 3;
  bh = (local / NSL) * 8 + (w & 7);
  c0 = (local % NSL) * SL;
  return bh < BH;
}
inline int scan_grid(int BH, int nsl) { return (BH + 7) / 8 * 8 * nsl; }

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

// an accumulator tile (rows r0.., cols c0..) as bf16, transposed: dst points at
// element (c0, r0) of the transposed matrix (8 contiguous bytes per lane)
__device__ __forceinline__ void put_t_bf16(__bf16* dst, int ld, const f32x4_t& v) {
  const int l16 = lane16(), g4 = lane_g4();
  const bf16x4_t w = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]),
                      static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
  *reinterpret_cast<bf16x4_t*>(dst + l16 * ld + 4 * g4) = w;
}
// the same tile as bf16 in its own orientation; dst points at element (r0, c0)
__device__ __forceinline__ void put_bf16(__bf16* dst, int ld, const f32x4_t& v) {
  const int l16 = lane16(), g4 = lane_g4();
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(4 * g4 + i) * ld + l16] = static_cast<__bf16>(v[i]);
}

// ROWS x COLS bf16 (row stride COLS) global -> LDS (leading dimension ld), 16
// bytes per lane; load(), pin_all() and store() as for GTile
template <int NT, int ROWS, int COLS>
struct BTile {
  static constexpr int C8 = COLS / 8, N = ROWS * C8, PER = (N + NT - 1) / NT;
  bf16x8_t r[PER];
  __device__ __forceinline__ void load(const __bf16* src) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT;
      if (N % NT == 0 || e < N) {
        const int rr = e / C8, c = (e - rr * C8) * 8;
        r[j] = *reinterpret_cast<const bf16x8_t*>(src + rr * COLS + c);
      }
    }
  }
  __device__ __forceinline__ void pin_all() {
#pragma unroll
    for (int j = 0; j < PER; ++j) pin(r[j]);
  }
  __device__ __forceinline__ void store(__bf16* dst, int ld) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * NT;
      if (N % NT == 0 || e < N) {
        const int rr = e / C8, c = (e - rr * C8) * 8;
        *reinterpret_cast<bf16x8_t*>(dst + rr * ld + c) = r[j];
      }
    }
  }
};

// Scan workgroups have 8 wavefronts (two per SIMD, so one's LDS and memory waits
// overlap the other's matrix work).  State tiles of one workgroup: D x 32 columns
// = (D/16) x 2 tiles, D/64 per wavefront; the 64 x 32 per-chunk products are
// 4 x 2 tiles, one per wavefront.
constexpr int kScanThreads = 512;

template <int D>
struct ScanTiles {
  static constexpr int NTW = D / 64;
  static __device__ __forceinline__ int rt(int wave, int x) { return (wave * NTW + x) >> 1; }
  static __device__ __forceinline__ int ct(int wave, int x) { return (wave * NTW + x) & 1; }
};

// acc += A B, A(r, k) = a[r * lda + k], B(k, c) = b[c * ldb + k] (bf16 in LDS)
template <int K>
__device__ __forceinline__ f32x4_t mmb(f32x4_t acc, const __bf16* a, int lda, const __bf16* b,
                                       int ldb) {
  const int l16 = lane16(), g4 = lane_g4();
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const int kb = k0 + 8 * g4;
    const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(a + l16 * lda + kb);
    const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(b + l16 * ldb + kb);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
  }
  return acc;
}

// sub-tile pairs J < I of a 64-row chunk -> 0..5
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// The sequences of a call: N sequences of T tokens (cu == null; chunk c of stream
// (n, h) is item (n * H + h) * nc + c), or N packed sequences whose tokens are
// [cu[n], cu[n+1]) of total_T (clamped into [0, total_T]; chunk c of stream (n, h)
// is item (floor(cu[n] / 64) + n + c) * H + h, ranges that never overlap).
// A window (cw > 0) restricts every sequence to its chunks c_lo .. c_lo + cw - 1 and
// numbers the items window-locally: chunk c_lo + l of stream (n, h) is item
// (n * H + h) * cw + l for fixed length, (n * cw + l) * H + h for packed input.
struct SeqMap {
  const int32_t* cu;
  int N, T, total_T, H, nc;
  int c_lo = 0, cw = 0;
};

__device__ __forceinline__ void seq_span(const SeqMap& m, int n, int& tok0, int& len) {
  if (m.cu == nullptr) {
    tok0 = n * m.T;
    len = m.T;
  } else {
    const int x0 = min(max(m.cu[n], 0), m.total_T);
    const int x1 = min(max(m.cu[n + 1], x0), m.total_T);
    tok0 = x0;
    len = x1 - x0;
  }
}

// Stream bh = n * H + h: its tokens, chunk count, and the items of its chunks (in a
// window: the tokens of the window's chunks only).
struct StreamPos {
  int tok0, len, nch;
  int64_t item0, istride;   // item of chunk c: item0 + c * istride
};
__device__ __forceinline__ StreamPos stream_pos(const SeqMap& m, int bh) {
  StreamPos s;
  const int n = bh / m.H, h = bh - n * m.H;
  seq_span(m, n, s.tok0, s.len);
  if (m.cw > 0) {
    const int skip = min(s.len, m.c_lo * CR);
    s.tok0 += skip;
    s.len = min(s.len - skip, m.cw * CR);
    s.nch = (s.len + CR - 1) / CR;
    s.item0 = m.cu == nullptr ? static_cast<int64_t>(bh) * m.cw : static_cast<int64_t>(n) * m.cw * m.H + h;
    s.istride = m.cu == nullptr ? 1 : m.H;
    return s;
  }
  s.nch = (s.len + CR - 1) / CR;
  if (m.cu == nullptr) {
    s.item0 = static_cast<int64_t>(bh) * m.nc;
    s.istride = 1;
  } else {
    s.item0 = (static_cast<int64_t>(s.tok0 / CR) + n) * m.H + h;
    s.istride = m.H;
  }
  return s;
}

struct ChunkPos {
  int b, h, c, nrow;
  int64_t row0;   // (first token of the chunk) * H + h: token-row index of its row 0
  bool valid;     // false for the unused items of packed sequences
};
__device__ __forceinline__ ChunkPos chunk_pos(int item, const SeqMap& m) {
  ChunkPos p;
  const int H = m.H;
  if (m.cw > 0) {   // window: items are (stream, local chunk), the chunk may lie past the end
    int n, l;
    if (m.cu == nullptr) {
      l = item % m.cw;
      const int bh = item / m.cw;
      n = bh / H;
      p.h = bh - n * H;
    } else {
      const int slot = item / H;
      p.h = item - slot * H;
      n = slot / m.cw;
      l = slot - n * m.cw;
    }
    int t0, len;
    seq_span(m, n, t0, len);
    p.b = n;
    p.c = m.c_lo + l;
    p.valid = p.c * CR < len;
    p.nrow = p.valid ? min(CR, len - p.c * CR) : 0;
    p.row0 = (static_cast<int64_t>(t0) + static_cast<int64_t>(p.c) * CR) * H + p.h;
    return p;
  }
  if (m.cu == nullptr) {
    p.c = item % m.nc;
    const int bh = item / m.nc;
    p.b = bh / H;
    p.h = bh - p.b * H;
    p.nrow = min(CR, m.T - p.c * CR);
    p.row0 = (static_cast<int64_t>(p.b) * m.T + static_cast<int64_t>(p.c) * CR) * H + p.h;
    p.valid = true;
    return p;
  }
  const int slot = item / H;
  p.h = item - slot * H;
  int lo = 0, hi = m.N - 1;   // largest n whose first slot is at most `slot`
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    int t0, l;
    seq_span(m, mid, t0, l);
    if (t0 / CR + mid <= slot) lo = mid; else hi = mid - 1;
  }
  int t0, len;
  seq_span(m, lo, t0, len);
  p.b = lo;
  p.c = slot - (t0 / CR + lo);
  p.valid = p.c >= 0 && p.c * CR < len;
  p.nrow = p.valid ? min(CR, len - p.c * CR) : 0;
  p.row0 = (static_cast<int64_t>(t0) + static_cast<int64_t>(p.c) * CR) * H + p.h;
  return p;
}

// Threads of one chunk_ops workgroup: 8 wavefronts, two per SIMD, so that one
// wavefront's LDS and memory latency hides behind the other's work.
constexpr int kOpsThreads = 512;
constexpr int kOpsWaves = kOpsThreads / 64;

// ---------------------------------------------------------------- chunk operands

// EXACT keeps every product on fp32 operands; otherwise bf16 inputs use bf16
// matrix-core operands (fp32 accumulation) for the products over 32 or more terms.
// FULL writes every operand the backward reads; otherwise only what a chunk's
// transition Diag(Lam) - Kt^T W needs (W, Kt, Lam), skipping q, M', P, Q', G and
// the inverse's copies.
template <int D, typename TIn, bool EXACT, bool FULL>
__global__ __launch_bounds__(kOpsThreads) void chunk_ops_kernel(const TIn* __restrict__ q,
                                                       const TIn* __restrict__ k,
                                                       const TIn* __restrict__ g,
                                                       const TIn* __restrict__ beta,
                                                       float* __restrict__ ws,
                                                       __bf16* __restrict__ wsb, SeqMap sm_,
                                                       float scale) {
  constexpr bool BF = IsBf16<TIn>::value && !EXACT;
  using L = BwdLayout<D>;
  constexpr int LD = L::LD;
  __shared__ __attribute__((aligned(16))) float sm[3 * CR * LD + 3 * CR * LS + 6 * D + CR];
  float* R0 = sm;                 // G, then (phase 5 on) unused
  float* R1 = R0 + CR * LD;       // k rowf -> q rowf -> k e^G
  float* R2 = R1 + CR * LD;       // k colf -> inverse scratch -> scale q e^G
  float* S0 = R2 + CR * LD;       // A' -> P
  float* S1 = S0 + CR * LS;       // M'
  float* S2 = S1 + CR * LS;       // Ti
  float* FP = S2 + CR * LS;       // [6][D] pair factors e^{R_I - R_J}
  float* BT = FP + 6 * D;         // beta
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane16(), g4 = lane_g4();
  const ChunkPos p = chunk_pos(blockIdx.x, sm_);
  if (!p.valid) return;            // unused item of packed sequences
  const int H = sm_.H;
  const int64_t rs = static_cast<int64_t>(H) * D;
  const TIn* qc = q + p.row0 * D;
  const TIn* kc = k + p.row0 * D;
  const TIn* gc = g + p.row0 * D;
  float* w = ws + static_cast<int64_t>(blockIdx.x) * L::WS;
  __bf16* wb = BF ? wsb + static_cast<int64_t>(blockIdx.x) * L::WSB : nullptr;

  // g, k and q of the chunk, four consecutive channels per load, all in flight
  // together; k and q stay in registers for every stage below
  using IT = ITile4<kOpsThreads, D, TIn>;
  constexpr int C4 = D / 4;
  IT gt, kt, qt;
  gt.load(gc, rs, p.nrow);
  kt.load(kc, rs, p.nrow);
  if constexpr (FULL) qt.load(qc, rs, p.nrow);
  const float bt = to_f32(beta[p.row0 + static_cast<int64_t>(min(tid & (CR - 1), p.nrow - 1)) * H]);
  for (int e = tid; e < 3 * CR * LS; e += kOpsThreads) S0[e] = 0.f;
  gt.pin_all();
  kt.pin_all();
  if constexpr (FULL) qt.pin_all();
  if (tid < CR) BT[tid] = tid < p.nrow ? bt : 0.f;
#pragma unroll
  for (int j = 0; j < IT::PER; ++j) {
    const int e = tid + j * kOpsThreads, t = e / C4, i0 = (e - t * C4) * 4;
    *reinterpret_cast<f32x4_t*>(R0 + t * LD + i0) = gt.get(j, p.nrow);
  }
  __syncthreads();
  if (tid < D) {   // running sum of g down the chunk (padding rows hold 0)
    float acc = 0.f;
#pragma unroll 8
    for (int t = 0; t < CR; ++t) {
      acc += R0[t * LD + tid];
      R0[t * LD + tid] = acc;
    }
  }
  __syncthreads();

  if (tid < D) {
    for (int I = 1; I < 4; ++I)
      for (int J = 0; J < I; ++J)
        FP[pair_index(I, J) * D + tid] =
            fexp(R0[(16 * I + 15) * LD + tid] - R0[(16 * J + 15) * LD + tid]);
    w[L::LAM + tid] = fexp(R0[(CR - 1) * LD + tid]);
  }
  // k rowf into R1, k colf into R2; G and Kt to the workspace
#pragma unroll
  for (int j = 0; j < IT::PER; ++j) {
    const int e = tid + j * kOpsThreads, t = e / C4, i0 = (e - t * C4) * 4;
    const f32x4_t G = *reinterpret_cast<const f32x4_t*>(R0 + t * LD + i0);
    const f32x4_t RI = *reinterpret_cast<const f32x4_t*>(R0 + (t | 15) * LD + i0);
    const f32x4_t Gl = *reinterpret_cast<const f32x4_t*>(R0 + (CR - 1) * LD + i0);
    const f32x4_t kv = kt.get(j, p.nrow);
    f32x4_t r1, r2, ktv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r1[i] = kv[i] * fexp(G[i] - RI[i]);
      r2[i] = kv[i] * fexp(RI[i] - G[i]);
      ktv[i] = kv[i] * fexp(Gl[i] - G[i]);
    }
    *reinterpret_cast<f32x4_t*>(R1 + t * LD + i0) = r1;
    *reinterpret_cast<f32x4_t*>(R2 + t * LD + i0) = r2;
    if constexpr (FULL) *reinterpret_cast<f32x4_t*>(w + L::G + t * D + i0) = G;
    if constexpr (!BF) {   // bf16 inputs: only the bf16 copies are read
      *reinterpret_cast<f32x4_t*>(w + L::KT + t * D + i0) = ktv;
    } else if constexpr (FULL) {
      bf16x4_t kb;
#pragma unroll
      for (int i = 0; i < 4; ++i) kb[i] = static_cast<__bf16>(ktv[i]);
      *reinterpret_cast<bf16x4_t*>(wb + L::BKT + t * D + i0) = kb;
    }
  }
  __syncthreads();

  // A' and M' by sub-tile pairs (I, J), J <= I: 10 tiles each
  auto pair_gram = [&](float* dst, bool strict) {
    for (int pt = wave; pt < 10; pt += kOpsWaves) {
      int I = 0;
      while ((I + 1) * (I + 2) / 2 <= pt) ++I;
      const int J = pt - I * (I + 1) / 2;
      f32x4_t acc = zero4();
      if (I == J) {
        acc = mmx<BF, false, true>(acc, R1 + 16 * I * LD, LD, R2 + 16 * J * LD, LD, D);
      } else {
        acc = mmx<BF, false, true, true>(acc, R1 + 16 * I * LD, LD, R2 + 16 * J * LD, LD, D,
                                    FP + pair_index(I, J) * D);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * I + 4 * g4 + i, s = 16 * J + l16;
        dst[t * LS + s] = (strict ? s < t : s <= t) ? acc[i] : 0.f;
      }
    }
  };
  pair_gram(S0, true);
  __syncthreads();
  if constexpr (FULL) {
    // q rowf into R1
#pragma unroll
    for (int j = 0; j < IT::PER; ++j) {
      const int e = tid + j * kOpsThreads, t = e / C4, i0 = (e - t * C4) * 4;
      const f32x4_t G = *reinterpret_cast<const f32x4_t*>(R0 + t * LD + i0);
      const f32x4_t RI = *reinterpret_cast<const f32x4_t*>(R0 + (t | 15) * LD + i0);
      const f32x4_t qv = qt.get(j, p.nrow);
      f32x4_t r1;
#pragma unroll
      for (int i = 0; i < 4; ++i) r1[i] = qv[i] * fexp(G[i] - RI[i]);
      *reinterpret_cast<f32x4_t*>(R1 + t * LD + i0) = r1;
    }
    __syncthreads();
    pair_gram(S1, false);
    __syncthreads();
    l2g<kOpsThreads, CR, CR>(w + L::AP, CR, S0, LS);
    l2g<kOpsThreads, CR, CR>(w + L::MP, CR, S1, LS);
  }
  if constexpr (BF) {   // Kt in R1 (free until k e^G goes there), for its bf16 transpose
#pragma unroll
    for (int j = 0; j < IT::PER; ++j) {
      const int e = tid + j * kOpsThreads, t = e / C4, i0 = (e - t * C4) * 4;
      const f32x4_t G = *reinterpret_cast<const f32x4_t*>(R0 + t * LD + i0);
      const f32x4_t Gl = *reinterpret_cast<const f32x4_t*>(R0 + (CR - 1) * LD + i0);
      const f32x4_t kv = kt.get(j, p.nrow);
      f32x4_t r1;
#pragma unroll
      for (int i = 0; i < 4; ++i) r1[i] = kv[i] * fexp(Gl[i] - G[i]);
      *reinterpret_cast<f32x4_t*>(R1 + t * LD + i0) = r1;
    }
  }

  // Ti = (I + Diag(beta) A')^-1: diagonal 16 x 16 blocks by substitution (one
  // column per lane), then the blocks below them level by level:
  //   Ti_IJ = -Ti_II Diag(beta_I) sum_{J <= m < I} A'_Im Ti_mJ
  if (wave < 4 && lane < 16) {
    const int I = wave, j = lane;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float s = t == j ? 1.f : 0.f;
      const float bt = BT[16 * I + t];
#pragma unroll
      for (int u = 0; u < t; ++u) s -= bt * S0[(16 * I + t) * LS + 16 * I + u] * x[u];
      x[t] = s;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) S2[(16 * I + t) * LS + 16 * I + j] = x[t];
  }
  __syncthreads();
  float* xs = R2 + wave * 16 * 17;
  for (int I = 1; I < 4; ++I) {
    if (wave < I) {
      const int J = wave;
      f32x4_t y = mm<false, false>(zero4(), S0 + 16 * I * LS + 16 * J, LS,
                                   S2 + 16 * J * LS + 16 * J, LS, 16 * (I - J));
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] *= BT[16 * I + 4 * g4 + i];
      put(xs, 17, y);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const f32x4_t tt = mm<false, false>(zero4(), S2 + 16 * I * LS + 16 * I, LS, xs, 17, 16);
      put(S2 + 16 * I * LS + 16 * J, LS, -tt);
    }
    __syncthreads();
  }
  if constexpr (FULL) {
    for (int e = tid; e < CR * CR; e += kOpsThreads) {
      const int t = e / CR, s = e - t * CR;
      const float ti = S2[t * LS + s];
      w[L::TI + e] = ti;
      w[L::TB + e] = ti * BT[s];
      if constexpr (BF) wb[L::BTB + e] = static_cast<__bf16>(ti * BT[s]);
    }
  }
  if constexpr (BF) {   // Tb^T and Kt^T (consecutive threads take consecutive rows)
    if constexpr (FULL) {
      for (int e = tid; e < CR * CR; e += kOpsThreads) {
        const int s = e / CR, t = e - s * CR;
        wb[L::BTBT + e] = static_cast<__bf16>(S2[t * LS + s] * BT[s]);
      }
    }
    for (int e = tid; e < CR * D; e += kOpsThreads) {
      const int i = e / CR, t = e - i * CR;
      wb[L::BKTT + e] = static_cast<__bf16>(R1[t * LD + i]);
    }
    __syncthreads();   // R1 is rewritten next
  }
  // k e^G into R1, scale q e^G into R2
#pragma unroll
  for (int j = 0; j < IT::PER; ++j) {
    const int e = tid + j * kOpsThreads, t = e / C4, i0 = (e - t * C4) * 4;
    const f32x4_t G = *reinterpret_cast<const f32x4_t*>(R0 + t * LD + i0);
    const f32x4_t kv = kt.get(j, p.nrow);
    f32x4_t r1;
#pragma unroll
    for (int i = 0; i < 4; ++i) r1[i] = kv[i] * fexp(G[i]);
    *reinterpret_cast<f32x4_t*>(R1 + t * LD + i0) = r1;
    if constexpr (FULL) {
      const f32x4_t qv = qt.get(j, p.nrow);
      f32x4_t r2;
#pragma unroll
      for (int i = 0; i < 4; ++i) r2[i] = scale * qv[i] * fexp(G[i]);
      *reinterpret_cast<f32x4_t*>(R2 + t * LD + i0) = r2;
    }
  }
  __syncthreads();

  // P = scale M' Tb (into S0 and the workspace); W = Tb (k e^G)
  for (int j = wave; FULL && j < 16; j += kOpsWaves) {
    const int rt = j >> 2, ct = j & 3;
    f32x4_t acc = mmx<BF, false, false>(zero4(), S1 + 16 * rt * LS, LS, S2 + 16 * ct, LS, CR);
    const float f = scale * BT[16 * ct + l16];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= f;
    put(S0 + 16 * rt * LS + 16 * ct, LS, acc);
    put(w + L::PP + 16 * rt * CR + 16 * ct, CR, acc);
    if constexpr (BF) put_t_bf16(wb + L::BPT + 16 * ct * CR + 16 * rt, CR, acc);
  }
  constexpr int CT = D / 16;
  for (int j = wave; j < 4 * CT; j += kOpsWaves) {
    const int rt = j / CT, ct = j - rt * CT;
    const f32x4_t acc = mmx<BF, false, false, true>(zero4(), S2 + 16 * rt * LS, LS, R1 + 16 * ct, LD,
                                               CR, BT);
    if constexpr (!BF) put(w + L::W + 16 * rt * D + 16 * ct, D, acc);
    if constexpr (BF) {
      put_bf16(wb + L::BW + 16 * rt * D + 16 * ct, D, acc);
      if constexpr (FULL) put_t_bf16(wb + L::BWT + 16 * ct * CR + 16 * rt, CR, acc);
    }
  }
  if constexpr (!FULL) return;
  __syncthreads();
  // Q' = scale q e^G - P (k e^G)
  for (int j = wave; j < 4 * CT; j += kOpsWaves) {
    const int rt = j / CT, ct = j - rt * CT;
    const f32x4_t pk = mmx<BF, false, false>(zero4(), S0 + 16 * rt * LS, LS, R1 + 16 * ct, LD, CR);
    f32x4_t acc = get(R2 + 16 * rt * LD + 16 * ct, LD);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] -= pk[i];
    if constexpr (!BF) put(w + L::QP + 16 * rt * D + 16 * ct, D, acc);
    if constexpr (BF) put_t_bf16(wb + L::BQPT + 16 * ct * CR + 16 * rt, CR, acc);
  }
}

}  // namespace

}  // namespace kda
