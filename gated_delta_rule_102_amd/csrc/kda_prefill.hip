// Chunked KDA prefill on gfx950: a chunk-parallel preparation kernel and a
// serial state-scan kernel (chunk = 64 tokens, 16-row sub-tiles).
//
// The token rule (neurohive.io Kimi K3 review, section "Sequence length: hybrid
// KDA and Gated MLA attention": a delta rule that forgets and writes, with a
// per-key-channel retention factor whose log is bounded below at -5)
//     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
//     o_t = S_t^T (scale q_t)
// is applied 64 tokens at a time.  With G the cumulative log-decay inside a
// chunk (per token and key channel, zero before the chunk):
//     A[t,s] = beta_t sum_c k_tc k_sc e^{G_tc - G_sc}   (s < t)   decayed key Gram
//     M[t,s] =        sum_c q_tc k_sc e^{G_tc - G_sc}   (s <= t)  decayed query-key
//     Tb     = (I + A)^{-1} Diag(beta)                  (UT transform)
//     W      = Tb (K e^G),   P = scale M Tb,   Q' = scale (Q e^G) - P (K e^G)
//     Kt     = K e^{G_n - G}, Lambda = e^{G_n}
// all of which are independent of the state, and then, chunk after chunk,
//     Delta = Tb V - W S,   O = Q' S + P V,   S <- Diag(Lambda) S + Kt^T Delta.
// Unrolling the recurrence inside the chunk gives (I + A) Delta = Diag(beta)(V -
// (K e^G) S), so the result equals the token-by-token one up to rounding.
//
// Kernel 1 (chunk_prep_kernel, or chunk_prep8_kernel with 8 wavefronts per item
// for bf16 at d = 128) does all state-independent work, one workgroup per
// (chunk, head), fully parallel: the elementwise decay factors, A and M on
// v_mfma_f32_16x16x32_bf16, the fp32 inverse, and W, Q', P, Tb.  It writes them,
// in the layouts the matrix cores read, to a stream-ordered workspace.
// Kernel 2 (state_scan_kernel) walks the chunks of one (sequence, head) and one
// dv slice; the dv columns of S evolve independently, so slices never talk.  Per
// chunk it only runs the four state products, reading operand fragments straight
// from the workspace into registers.
//
// The -5 bound is what lets every tile be a plain bf16 matrix-core product: over
// a whole chunk e^{-G} reaches e^{320}, so A and M are built from 16-row sub-tiles
// referenced to the cumulative decay at the end of their own sub-tile -- row side
// e^{G_t - R_I} in [1, e^80], column side e^{R_I - G_s} <= 1, both in bf16 range.

#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC = 64;
constexpr int kThreads = 256;

// ---------------------------------------------------------------- helpers

// Byte offset of (row, byte) in an LDS tile whose rows are RB bytes long, with the
// 16-byte chunks of each row permuted by the row index (conflict-free column reads).
template <int RB>
__device__ __forceinline__ int swz(int row, int byte) {
  constexpr int NCH = RB / 16;
  static_assert(NCH == 4 || NCH == 8 || NCH == 16, "row length");
  return row * RB + ((((byte >> 4) ^ (row & (NCH - 1)))) << 4) + (byte & 15);
}

template <bool F32> struct Frag;
template <> struct Frag<false> { bf16x8_t v; };
template <> struct Frag<true> { float v[8]; };

template <bool F32>
__device__ __forceinline__ f32x4_t mma32(f32x4_t acc, const Frag<F32>& a, const Frag<F32>& b) {
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
    return acc;
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
  }
}

// 8 consecutive operand elements (16 bytes bf16, 32 bytes fp32) of a swizzled tile.
template <bool F32, int RB>
__device__ __forceinline__ Frag<F32> lds_frag(const char* base, int row, int byte) {
  Frag<F32> f;
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4*>(base + swz<RB>(row, byte));
    const float4 b = *reinterpret_cast<const float4*>(base + swz<RB>(row, byte + 16));
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  } else {
    f.v = *reinterpret_cast<const bf16x8_t*>(base + swz<RB>(row, byte));
  }
  return f;
}

// One fragment stored in fragment order at byte offset voff (lane's 16 bytes; the
// fp32 second half sits 1 KB further).
template <bool F32>
__device__ __forceinline__ Frag<F32> buf_frag2(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  Frag<F32> f;
  if constexpr (F32) {
    const i32x4_t a = buf_ld128(r, voff, 0);
    const i32x4_t b = buf_ld128(r, voff + 1024, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) { f.v[i] = __int_as_float(a[i]); f.v[4 + i] = __int_as_float(b[i]); }
  } else {
    f.v = __builtin_bit_cast(bf16x8_t, buf_ld128(r, voff, 0));
  }
  return f;
}

template <bool F32>
__device__ __forceinline__ Frag<F32> frag_from_f32(const float* x) {
  Frag<F32> f;
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = x[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = static_cast<__bf16>(x[i]);
  }
  return f;
}

template <bool F32>
__device__ __forceinline__ void frag_to_f32(const Frag<F32>& f, float* x) {
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = f.v[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(f.v[i]);
  }
}

// 4 consecutive values as operand elements: 8 bytes (bf16) or 16 bytes (fp32).
template <bool F32>
__device__ __forceinline__ void lds_put4(char* p, float a, float b, float c, float d) {
  if constexpr (F32) {
    *reinterpret_cast<float4*>(p) = float4{a, b, c, d};
  } else {
    *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
  }
}
template <bool F32>
__device__ __forceinline__ void buf_put4(__amdgpu_buffer_rsrc_t r, uint32_t voff, float a, float b,
                                         float c, float d) {
  if constexpr (F32) {
    buf_st128(i32x4_t{__float_as_int(a), __float_as_int(b), __float_as_int(c), __float_as_int(d)},
              r, voff, 0);
  } else {
    buf_st64(i32x2_t{static_cast<int>(pack_bf16x2(a, b)), static_cast<int>(pack_bf16x2(c, d))}, r,
             voff, 0);
  }
}

template <bool F32>
__device__ __forceinline__ float lds_get1(const char* p) {
  if constexpr (F32) return *reinterpret_cast<const float*>(p);
  else return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
}

template <bool F32>
__device__ __forceinline__ void lds_set1(char* p, float x) {
  if constexpr (F32) *reinterpret_cast<float*>(p) = x;
  else *reinterpret_cast<uint16_t*>(p) = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Sub-tile pairs (I, J), J <= I, in the order (0,0),(1,0),(1,1),(2,0),...,(3,3).
__device__ __forceinline__ void pair_of(int p, int& I, int& J) {
  I = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
  J = p - I * (I + 1) / 2;
}
// Off-diagonal pairs J < I -> 0..5.
__device__ __forceinline__ constexpr int offdiag_index(int I, int J) { return I * (I - 1) / 2 + J; }
// Strictly-upper sub-tile pairs (I, J), J > I, numbered 0..5.
__device__ __forceinline__ void upper_pair(int b, int& I, int& J) {
  I = b < 3 ? 0 : b < 5 ? 1 : 2;
  J = b < 3 ? b + 1 : b < 5 ? b - 1 : 3;
}

// ---------------------------------------------------------------- sequences

struct SeqArgs {
  const int32_t* cu;   // varlen offsets, or null
  int N, T, total_T, H;
};

__device__ __forceinline__ void seq_bounds(const SeqArgs& a, int n, int& tok0, int& len) {
  if (a.cu == nullptr) {
    tok0 = n * a.T;
    len = a.T;
  } else {
    const int x0 = min(max(a.cu[n], 0), a.total_T);
    const int x1 = min(max(a.cu[n + 1], x0), a.total_T);
    tok0 = x0;
    len = x1 - x0;
  }
}

// Workspace slots: sequence n owns [floor(tok0/64) + n, ... + ceil(len/64)); these
// ranges never overlap and all lie below ceil(total_T/64) + N.
__device__ __forceinline__ int slot_base(int tok0, int n) { return tok0 / kC + n; }

// Which (sequence, chunk) a workspace slot holds; false for unused slots.
__device__ __forceinline__ bool locate_slot(const SeqArgs& a, int slot, int& n, int& chunk,
                                            int& tok0, int& len) {
  int lo = 0, hi = a.N - 1;            // largest n with slot_base(n) <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    int t0, l;
    seq_bounds(a, mid, t0, l);
    if (slot_base(t0, mid) <= slot) lo = mid; else hi = mid - 1;
  }
  n = lo;
  seq_bounds(a, n, tok0, len);
  chunk = slot - slot_base(tok0, n);
  return chunk >= 0 && chunk * kC < len;
}

// ---------------------------------------------------------------- workspace slot

template <int D, bool F32>
struct Slot {
  static constexpr int E = F32 ? 4 : 2;
  static constexpr int W = 0;                          // [64][D]  W
  static constexpr int QP = W + kC * D * E;            // [64][D]  Q'
  static constexpr int KT = QP + kC * D * E;           // [D][64]  Kt^T
  static constexpr int TB = KT + D * kC * E;           // [64][64] Tb
  static constexpr int PP = TB + kC * kC * E;          // [64][64] P
  static constexpr int LAM = PP + kC * kC * E;         // [D] fp32 Lambda
  static constexpr int BYTES = (LAM + D * 4 + 255) / 256 * 256;
};

// Byte offset of element (row, k) of a workspace operand stored in fragment order:
// the operand is cut into 16-row x 32-k fragments (f = (row/16) * (K/32) + k/32), and
// each fragment is laid out exactly as a wavefront holds it for the matrix cores --
// lane (k%32)/8*16 + row%16 owns 8 consecutive k -- so one 16-byte load per lane
// reads a contiguous 1 KB (fp32: two such halves of 4 elements each).
template <int K, bool F32>
__device__ __forceinline__ uint32_t frag_off(int row, int k) {
  const int f = (row >> 4) * (K / 32) + (k >> 5);
  const int l = ((k & 31) >> 3) * 16 + (row & 15);
  const int e = k & 7;
  if constexpr (F32) return static_cast<uint32_t>(((f * 2 + (e >> 2)) * 64 + l) * 16 + (e & 3) * 4);
  else return static_cast<uint32_t>((f * 64 + l) * 16 + e * 2);
}

// ================================================================= kernel 1

template <int D, typename TIn>
struct PrepCfg {
  static constexpr bool F32 = std::is_same<TIn, float>::value;
  static constexpr int E = F32 ? 4 : 2;          // operand element bytes
  static constexpr int EI = sizeof(TIn);         // input element bytes
  static constexpr int CPL = D / 64;             // key channels per lane
  static constexpr int RBD = D * E;              // bytes per row of [64][D]
  static constexpr int RBC = kC * E;             // bytes per row of [D][64], [64][64]
  static constexpr int NKK = D / 32;
  // R1, phase 1: sub-tile referenced operands
  static constexpr int QS = 0, KS = QS + kC * RBD, KT = KS + kC * RBD, R1A = KT + kC * RBD;
  // R1, phase 2: chunk-referenced operands, P, and the 32x32 inverse intermediate
  static constexpr int QB = 0, KBT = QB + kC * RBD, PB = KBT + D * RBC, XS = PB + kC * RBC;
  static constexpr int XLD = 17;                 // fp32 row stride of the 16x16 X tiles
  static constexpr int R1B = XS + 4 * 16 * XLD * 4;
  static constexpr int RAW = 0;                  // q, k, g of the chunk as loaded
  static constexpr int R1R = 3 * kC * D * (F32 ? 4 : 2);
  static constexpr int R1AB = R1A > R1B ? R1A : R1B;
  static constexpr int R1 = ((R1AB > R1R ? R1AB : R1R) + 15) / 16 * 16;
  static constexpr int AT = R1;                  // [64][64] fp32: A, then T in place
  static constexpr int MB = AT + kC * kC * 4;    // [64][64] operand: M
  static constexpr int FIJ = MB + kC * RBC;      // [6][D] fp32 pair factors
  static constexpr int BTOT = FIJ + 6 * D * 4;   // [8][D] fp32 totals per wavefront's rows
  static constexpr int BETA = BTOT + 8 * D * 4;  // [64] fp32
  static constexpr int LDS = BETA + kC * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

struct PrepParams {
  const void *q, *k, *g, *beta;
  char* ws;
  SeqArgs sa;
  float scale;
  int items;       // work items of the launch
  int c_lo, cg;    // cg > 0: items cover chunks [c_lo, c_lo + cg) of every sequence
  int prologue;    // 1: q, k, g, beta are raw (see kda_chunk_fwd_prologue)
};

// Raw input words of one token row for the CPL channels a lane owns.
template <typename TIn, int CPL> struct RawRow;
template <> struct RawRow<bf16_t, 2> { using type = uint32_t; };
template <> struct RawRow<bf16_t, 1> { using type = uint16_t; };
template <> struct RawRow<float, 1> { using type = uint32_t; };

template <typename TIn, int CPL, int ROWS = 16>
struct RawChunk {
  using R = typename RawRow<TIn, CPL>::type;
  R g[ROWS], k[ROWS], q[ROWS];
  uint32_t beta;
};

// Everything that names one (chunk, head) work item.
struct PrepItem {
  bool valid;
  int slot, h, t0, nrow;
};

__device__ __forceinline__ PrepItem prep_item(const PrepParams& p, int item) {
  PrepItem it{false, 0, 0, 0, 0};
  if (item >= p.items) return it;
  it.slot = item / p.sa.H;
  it.h = item % p.sa.H;
  int n, chunk, tok0, len;
  if (!locate_slot(p.sa, it.slot, n, chunk, tok0, len)) return it;
  it.valid = true;
  it.t0 = tok0 + chunk * kC;
  it.nrow = min(kC, len - chunk * kC);
  return it;
}

// Group mode: item -> (sequence n, chunk c_lo + lc, head h), written to slot
// (n * cg + lc) * H + h of the launch's group workspace; chunks past the end of
// the sequence are no work.
__device__ __forceinline__ PrepItem prep_group_item(const PrepParams& p, int item, int& slot) {
  PrepItem it{false, 0, 0, 0, 0};
  const int H = p.sa.H;
  if (item >= p.items) return it;
  it.h = item % H;
  const int lc = (item / H) % p.cg, n = item / (H * p.cg);
  int tok0, len;
  seq_bounds(p.sa, n, tok0, len);
  const int c = p.c_lo + lc;
  if (c * kC >= len) return it;
  it.valid = true;
  it.t0 = tok0 + c * kC;
  it.nrow = min(kC, len - c * kC);
  slot = n * p.cg + lc;
  return it;
}

// All state-independent work of one (chunk, head) item, by one workgroup; the
// results go to the workspace slot at `slot_ptr`.
// NW = 4 or 8 wavefronts per item.  With 8 (d = 128, bf16 only) a wavefront owns
// half a 16-row sub-tile in the elementwise phases and one sub-tile pair or two
// diagonal ones in the decayed products, and the workgroups are small enough in
// registers for two of them (16 wavefronts) to share a CU.
template <int D, typename TIn, int NW = 4>
__device__ __forceinline__ void prep_body(const PrepParams& p, char* smem, const PrepItem& cur_it,
                                          char* slot_ptr) {
  using CF = PrepCfg<D, TIn>;
  using SL = Slot<D, CF::F32>;
  constexpr int RW = kC / NW;                    // token rows per wavefront
  using RC = RawChunk<TIn, CF::CPL, RW>;
  constexpr bool F32 = CF::F32;
  constexpr int CPL = CF::CPL;
  constexpr int E = CF::E;
  constexpr int EI = CF::EI;
  constexpr int NT = 64 * NW;                    // threads per item
  static_assert(NW == 4 || (NW == 8 && D == 128 && !F32), "wavefronts per item");

  // the wavefront index is uniform: keeping it scalar makes per-wavefront branches
  // and offsets scalar work
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int H = p.sa.H;
  const uint32_t rs_qk = static_cast<uint32_t>(H) * D * EI;    // token row stride (bytes)

  char* atc = smem + CF::AT;
  float* btot = reinterpret_cast<float*>(smem + CF::BTOT);
  float* betas = reinterpret_cast<float*>(smem + CF::BETA);
  float* fij = reinterpret_cast<float*>(smem + CF::FIJ);
  auto at_el = [&](int row, int col) -> float& {
    return *reinterpret_cast<float*>(atc + swz<256>(row, col * 4));
  };
  // elements col0 .. col0+3 of a row (col0 a multiple of 4: one 16-byte chunk)
  auto at_row4 = [&](int row, int col0) -> float4 {
    return *reinterpret_cast<const float4*>(atc + swz<256>(row, col0 * 4));
  };

  // the strictly-upper sub-tiles of A/T and of M are read as zeros; nothing else
  // writes them, so clearing them once serves every item of this workgroup
  for (int e = tid; e < 6 * 256; e += NT) {
    int I, J;
    upper_pair(e >> 8, I, J);
    const int row = 16 * I + ((e >> 4) & 15), col = 16 * J + (e & 15);
    at_el(row, col) = 0.f;
    lds_set1<F32>(smem + CF::MB + swz<CF::RBC>(row, col * E), 0.f);
  }

  // q, k, g of the chunk go straight from memory into region 1 (16 bytes per lane,
  // 1 KB contiguous per instruction); each lane then picks up its own channels.
  auto load_raw = [&](const PrepItem& it, RC& rc) {
    const int64_t base_qk = (static_cast<int64_t>(it.t0) * H + it.h) * D;
    const uint32_t bytes_qk = (it.nrow - 1) * rs_qk + D * EI;   // rows past the end read 0
    const __amdgpu_buffer_rsrc_t rsrc[3] = {
        make_rsrc(static_cast<const TIn*>(p.g) + base_qk, bytes_qk),
        make_rsrc(static_cast<const TIn*>(p.k) + base_qk, bytes_qk),
        make_rsrc(static_cast<const TIn*>(p.q) + base_qk, bytes_qk)};
    constexpr int RBI = D * EI;                 // bytes of one token row of one head
    constexpr int RPI = 1024 / RBI;             // rows per 1 KB instruction
    constexpr int LPR = RBI / 16;               // lanes per row
    const int uw = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int x = 0; x < 3; ++x) {
#pragma unroll
      for (int j = 0; j < RW / RPI; ++j) {
        const int row0 = RW * uw + j * RPI;
        const int row = row0 + lane / LPR;
        char* dst = smem + CF::RAW + x * kC * RBI + row0 * RBI;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc[x], (__attribute__((address_space(3))) void*)dst, 16,
            row * rs_qk + (lane % LPR) * 16, 0, 0, 0);
      }
    }
    if (tid < kC) {
      const auto rb = make_rsrc(static_cast<const TIn*>(p.beta) + static_cast<int64_t>(it.t0) * H + it.h,
                                (it.nrow - 1) * H * EI + EI);
      if constexpr (F32) rc.beta = buf_ld32(rb, tid * H * EI, 0);
      else rc.beta = static_cast<uint32_t>(buf_ld16(rb, tid * H * EI, 0)) << 16;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (p.prologue) {
      // unit L2 norm of q and k per (token, head): two threads per row sum squares
      // over half the channels, straight from the raw tiles (the FIJ region is
      // free until the decay phase); the first 256 threads
      float* nrm = reinterpret_cast<float*>(smem + CF::FIJ);   // [k, q][64]
      const int tq = tid & 255;
      const int x = 1 + (tq >> 7), row = (tq & 127) >> 1, half = tq & 1;
      const char* src = smem + CF::RAW + x * kC * RBI + row * RBI + half * (RBI / 2);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < RBI / 2; i += 16) {
        const i32x4_t w4 = *reinterpret_cast<const i32x4_t*>(src + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (F32) {
            const float f = __int_as_float(w4[j]);
            ss += f * f;
          } else {
            // the element goes through a scalar first: a bit cast applied directly
            // to a vector-element expression compiled to a read of element 0
            const int wj = w4[j];
            const bf16x2_t b2 = __builtin_bit_cast(bf16x2_t, wj);
            ss = __builtin_amdgcn_fdot2_f32_bf16(b2, b2, ss, false);
          }
        }
      }
      ss += __shfl_xor(ss, 1);
      if (half == 0 && tid < 256) nrm[(x - 1) * kC + row] = __builtin_amdgcn_rsqf(ss + kNormEps);
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int off = (RW * wave + r) * RBI + lane * CPL * EI;
      if constexpr (!F32 && CPL == 1) {
        rc.g[r] = *reinterpret_cast<const uint16_t*>(smem + CF::RAW + 0 * kC * RBI + off);
        rc.k[r] = *reinterpret_cast<const uint16_t*>(smem + CF::RAW + 1 * kC * RBI + off);
        rc.q[r] = *reinterpret_cast<const uint16_t*>(smem + CF::RAW + 2 * kC * RBI + off);
      } else {
        rc.g[r] = *reinterpret_cast<const uint32_t*>(smem + CF::RAW + 0 * kC * RBI + off);
        rc.k[r] = *reinterpret_cast<const uint32_t*>(smem + CF::RAW + 1 * kC * RBI + off);
        rc.q[r] = *reinterpret_cast<const uint32_t*>(smem + CF::RAW + 2 * kC * RBI + off);
      }
      if (p.prologue) {   // normalised q, k kept in the input precision
        const float* nrm = reinterpret_cast<const float*>(smem + CF::FIJ);
        const float fk = nrm[RW * wave + r], fq = nrm[kC + RW * wave + r];
        if constexpr (F32) {
          rc.k[r] = __float_as_uint(__uint_as_float(rc.k[r]) * fk);
          rc.q[r] = __float_as_uint(__uint_as_float(rc.q[r]) * fq);
        } else if constexpr (CPL == 1) {
          rc.k[r] = static_cast<uint16_t>(pack_bf16x2(__uint_as_float(uint32_t(rc.k[r]) << 16) * fk, 0.f));
          rc.q[r] = static_cast<uint16_t>(pack_bf16x2(__uint_as_float(uint32_t(rc.q[r]) << 16) * fq, 0.f));
        } else {
          rc.k[r] = pack_bf16x2(bf16lo(rc.k[r]) * fk, bf16hi(rc.k[r]) * fk);
          rc.q[r] = pack_bf16x2(bf16lo(rc.q[r]) * fq, bf16hi(rc.q[r]) * fq);
        }
      }
    }
  };

  RC cur;
  load_raw(cur_it, cur);
  {
    const auto rw = make_rsrc(slot_ptr, SL::BYTES);

    // ------------------------------------------------ phase E: decay factors
    // wavefront `wave` owns token rows RW*wave .. +RW-1; lane owns key channels
    // lane*CPL .. +CPL-1; the cumulative decay is a running product over the rows.
    // q and k stay in their packed input words (cur.q, cur.k) and are widened where
    // used, which keeps the live register set small across the matrix-core phases
    auto kval = [&](int r, int e) -> float {
      if constexpr (F32) return __uint_as_float(cur.k[r]);
      else if constexpr (CPL == 1) return __uint_as_float(uint32_t(cur.k[r]) << 16);
      else return e ? bf16hi(cur.k[r]) : bf16lo(cur.k[r]);
    };
    auto qval = [&](int r, int e) -> float {
      if constexpr (F32) return __uint_as_float(cur.q[r]);
      else if constexpr (CPL == 1) return __uint_as_float(uint32_t(cur.q[r]) << 16);
      else return e ? bf16hi(cur.q[r]) : bf16lo(cur.q[r]);
    };
    float rowf[RW][CPL], colf[RW][CPL];
    {
      float ed[RW][CPL];
#pragma unroll
      for (int r = 0; r < RW; ++r) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          float gv;
          if constexpr (F32) gv = __uint_as_float(cur.g[r]);
          else if constexpr (CPL == 1) gv = __uint_as_float(uint32_t(cur.g[r]) << 16);
          else gv = e ? bf16hi(cur.g[r]) : bf16lo(cur.g[r]);
          // prologue: g = max(-5, -softplus(x)), so e^g = max(e^-5, 1 / (1 + e^x));
          // rows past the sequence end keep retention 1, as g = 0 does without it
          ed[r][e] = !p.prologue ? fast_exp2(gv * kLog2e)
                     : RW * wave + r < cur_it.nrow
                         ? fmaxf(kMinRetention, __builtin_amdgcn_rcpf(1.f + fast_exp2(gv * kLog2e)))
                         : 1.f;
        }
      }
      if (tid < kC) {   // prologue: beta = sigmoid(x)
        const float bx = __uint_as_float(cur.beta);
        betas[tid] = !p.prologue ? bx
                     : tid < cur_it.nrow ? __builtin_amdgcn_rcpf(1.f + fast_exp2(-bx * kLog2e)) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        // products over this wavefront's rows, from their start (rowf) and to their
        // end (colf); for NW = 4 the rows are the sub-tile
        float run = 1.f;
#pragma unroll
        for (int r = 0; r < RW; ++r) { run *= ed[r][e]; rowf[r][e] = run; }
        btot[wave * D + lane * CPL + e] = run;
        float back = 1.f;
#pragma unroll
        for (int r = RW - 1; r >= 0; --r) { colf[r][e] = back; back *= ed[r][e]; }
      }
    }
    __syncthreads();

    // this wavefront's rows lie in sub-tile `sub` (R_{sub+1}: the cumulative decay at
    // its end); BPS wavefronts share a sub-tile
    constexpr int BPS = NW / 4;
    const int sub = wave / BPS;
    float eR1[CPL], fI3[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int c = lane * CPL + e;
      float bb[NW], b4[4];
#pragma unroll
      for (int m = 0; m < NW; ++m) bb[m] = btot[m * D + c];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        b4[I] = bb[I * BPS];
#pragma unroll
        for (int x = 1; x < BPS; ++x) b4[I] *= bb[I * BPS + x];   // e^{R_{I+1} - R_I}
      }
      float pre = 1.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) if (m <= sub) pre *= b4[m];
      eR1[e] = pre;                                    // e^{R_{sub+1}}
      // the sub-tile's rows before / after this wavefront's (none for NW = 4)
      float before = 1.f, after = 1.f;
#pragma unroll
      for (int m = 0; m < NW; ++m) {
        if (m / BPS == sub && m < wave) before *= bb[m];
        if (m / BPS == sub && m > wave) after *= bb[m];
      }
      const float inv_bt = __builtin_amdgcn_rcpf(b4[sub]) * before;   // b4 in [e^-80, 1]
      float acc = 1.f;
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        if (I > sub) {
          acc *= b4[I];
          if (wave % BPS == 0) fij[offdiag_index(I, sub) * D + c] = acc;   // e^{R_{I+1} - R_{sub+1}}
        }
      }
      fI3[e] = acc;                                    // e^{G_n - R_{sub+1}}
      if (wave == 0) {
        const float lam = b4[0] * b4[1] * b4[2] * b4[3];
        buf_st32(__float_as_uint(lam), rw, SL::LAM + c * 4, 0);
      }
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        rowf[r][e] *= inv_bt;   // now e^{G_t - R_{sub+1}} in [1, e^80]
        colf[r][e] *= after;    // now e^{R_{sub+1} - G_t}
      }
    }
    // row-side operands (referenced to the end of the own sub-tile) and the
    // column-side keys of the diagonal pairs
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int t = RW * wave + r;
      const int byte = lane * CPL * E;
      if constexpr (CPL == 2 && !F32) {
        const float k0 = kval(r, 0), k1 = kval(r, 1), q0 = qval(r, 0), q1 = qval(r, 1);
        *reinterpret_cast<uint32_t*>(smem + CF::QS + swz<CF::RBD>(t, byte)) =
            pack_bf16x2(q0 * rowf[r][0], q1 * rowf[r][1]);
        *reinterpret_cast<uint32_t*>(smem + CF::KS + swz<CF::RBD>(t, byte)) =
            pack_bf16x2(k0 * rowf[r][0], k1 * rowf[r][1]);
        *reinterpret_cast<uint32_t*>(smem + CF::KT + swz<CF::RBD>(t, byte)) =
            pack_bf16x2(k0 * colf[r][0], k1 * colf[r][1]);
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const int b = byte + e * E;
          lds_set1<F32>(smem + CF::QS + swz<CF::RBD>(t, b), qval(r, e) * rowf[r][e]);
          lds_set1<F32>(smem + CF::KS + swz<CF::RBD>(t, b), kval(r, e) * rowf[r][e]);
          lds_set1<F32>(smem + CF::KT + swz<CF::RBD>(t, b), kval(r, e) * colf[r][e]);
        }
      }
    }
    // Kt^T = (K e^{G_n - G})^T straight to the workspace: RW consecutive tokens per channel
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int c = lane * CPL + e;
      float x[RW];
#pragma unroll
      for (int r = 0; r < RW; ++r) x[r] = kval(r, e) * colf[r][e] * fI3[e];
#pragma unroll
      for (int q4 = 0; q4 < RW / 4; ++q4)
        buf_put4<F32>(rw, SL::KT + frag_off<kC, F32>(c, RW * wave + 4 * q4), x[4 * q4], x[4 * q4 + 1],
                      x[4 * q4 + 2], x[4 * q4 + 3]);
    }
    __syncthreads();

    // ------------------------------------------------ phase AM: A and M
    // computed transposed (rows s) so each lane stores 4 consecutive s of row t.
    // Off-diagonal pairs cost about twice a diagonal one (their column operand is
    // rescaled), so each wavefront takes two off-diagonal pairs or one off-diagonal
    // and two diagonal ones: pair numbers from pair_of, -1 = none.  With 8
    // wavefronts each takes one off-diagonal pair or two diagonal ones.
    constexpr int kPairs4[4][3] = {{1, 3, -1}, {4, 6, -1}, {7, 0, 2}, {8, 5, 9}};
    constexpr int kPairs8[8][3] = {{1, -1, -1}, {3, -1, -1}, {4, -1, -1}, {6, -1, -1},
                                   {7, -1, -1}, {8, -1, -1}, {0, 2, -1}, {5, 9, -1}};
#pragma unroll
    for (int pp = 0; pp < (NW == 4 ? 3 : 2); ++pp) {
      const int pr = NW == 4 ? kPairs4[wave][pp] : kPairs8[wave][pp];
      if (pr >= 0) {
        int I, J;
        pair_of(pr, I, J);
        f32x4_t aA = {0.f, 0.f, 0.f, 0.f}, aM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < CF::NKK; ++kk) {
          const int kb = (kk * 32 + g4 * 8) * E;
          Frag<F32> a = lds_frag<F32, CF::RBD>(smem + CF::KT, 16 * J + l16, kb);
          if (J < I) {   // carry column sub-tile J to row sub-tile I's reference
            const float* f = fij + offdiag_index(I, J) * D + kk * 32 + g4 * 8;
            float x[8];
            frag_to_f32<F32>(a, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= f[e];
            a = frag_from_f32<F32>(x);
          }
          const Frag<F32> bk = lds_frag<F32, CF::RBD>(smem + CF::KS, 16 * I + l16, kb);
          const Frag<F32> bq = lds_frag<F32, CF::RBD>(smem + CF::QS, 16 * I + l16, kb);
          aA = mma32<F32>(aA, a, bk);
          aM = mma32<F32>(aM, a, bq);
        }
        const int t = 16 * I + l16, s0 = 16 * J + 4 * g4;
        const float bt = betas[t];
        float av[4], mv[4];
        if (I == J) {   // diagonal sub-tile: A strictly lower, M lower
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            av[i] = (s0 + i < t) ? bt * aA[i] : 0.f;
            mv[i] = (s0 + i <= t) ? aM[i] : 0.f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            av[i] = bt * aA[i];
            mv[i] = aM[i];
          }
        }
        *reinterpret_cast<float4*>(atc + swz<256>(t, s0 * 4)) = float4{av[0], av[1], av[2], av[3]};
        lds_put4<F32>(smem + CF::MB + swz<CF::RBC>(t, s0 * E), mv[0], mv[1], mv[2], mv[3]);
      }
    }
    __syncthreads();

    // ------------------------------------------------ phase E2 + diagonal inverses
    // chunk-referenced Q e^G ([t][c]) and (K e^G)^T ([c][t]) into region 1
    {
      float kb[CPL][RW];
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int t = RW * wave + r;
        float qv[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const float ef = rowf[r][e] * eR1[e];          // e^{G_t}
          qv[e] = qval(r, e) * ef;
          kb[e][r] = kval(r, e) * ef;
        }
        if constexpr (CPL == 2 && !F32) {
          *reinterpret_cast<uint32_t*>(smem + CF::QB + swz<CF::RBD>(t, lane * 4)) = pack_bf16x2(qv[0], qv[1]);
        } else {
#pragma unroll
          for (int e = 0; e < CPL; ++e) lds_set1<F32>(smem + CF::QB + swz<CF::RBD>(t, (lane * CPL + e) * E), qv[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < CPL; ++e)
#pragma unroll
        for (int q4 = 0; q4 < RW / 4; ++q4)
          lds_put4<F32>(smem + CF::KBT + swz<CF::RBC>(lane * CPL + e, (RW * wave + 4 * q4) * E),
                        kb[e][4 * q4], kb[e][4 * q4 + 1], kb[e][4 * q4 + 2], kb[e][4 * q4 + 3]);
    }
    {   // T_ww = (I + A_ww)^{-1} = (I - A)(I + A^2)(I + A^4)(I + A^8): A_ww is strictly
        // lower, so A^16 = 0.  Six 16x16 products on fp32 matrix cores per wavefront.
        // A 16x16x4 product reads its A operand in row layout (lane: row l16, columns
        // 4*g4 .. +3) and its B operand in the accumulator layout (lane: rows 4*g4 ..
        // +3 of column l16), so a result feeds the next product's B side directly and
        // its A side after a transpose through this wavefront's 16x17 scratch.
        // Wavefronts 0-3 (one per diagonal block).
     if (NW == 4 || wave < 4) {
      const int base = 16 * wave;
      float* sc = reinterpret_cast<float*>(smem + CF::XS) + wave * 16 * CF::XLD;
      auto mm = [&](const float (&xr)[4], const float (&yc)[4]) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[st], yc[st], acc, 0, 0, 0);
        return acc;
      };
      auto to_row = [&](const f32x4_t& c, float (&r)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[(4 * g4 + i) * CF::XLD + l16] = c[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = sc[l16 * CF::XLD + 4 * g4 + i];
      };
      const float4 ar4 = at_row4(base + l16, base + 4 * g4);
      const float a_r[4] = {ar4.x, ar4.y, ar4.z, ar4.w};
      float a_c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a_c[i] = at_el(base + 4 * g4 + i, base + l16);
      const f32x4_t p1 = mm(a_r, a_c);                         // A^2
      const float p1_c[4] = {p1[0], p1[1], p1[2], p1[3]};
      float p1_r[4];
      to_row(p1, p1_r);
      const f32x4_t p2 = mm(p1_r, p1_c);                       // A^4
      const f32x4_t a3 = mm(a_r, p1_c);                        // A^3
      const float p2_c[4] = {p2[0], p2[1], p2[2], p2[3]};
      float p2_r[4];
      to_row(p2, p2_r);
      const f32x4_t p3 = mm(p2_r, p2_c);                       // A^8
      const float p3_c[4] = {p3[0], p3[1], p3[2], p3[3]};
      f32x4_t t1;                                              // I - A + A^2 - A^3
#pragma unroll
      for (int i = 0; i < 4; ++i) t1[i] = (4 * g4 + i == l16 ? 1.f : 0.f) - a_c[i] + p1[i] - a3[i];
      float t1_r[4];
      to_row(t1, t1_r);
      f32x4_t t2 = mm(t1_r, p2_c);                             // T1 (I + A^4)
#pragma unroll
      for (int i = 0; i < 4; ++i) t2[i] += t1[i];
      float t2_r[4];
      to_row(t2, t2_r);
      f32x4_t t3 = mm(t2_r, p3_c);                             // T2 (I + A^8)
#pragma unroll
      for (int i = 0; i < 4; ++i) at_el(base + 4 * g4 + i, base + l16) = t3[i] + t2[i];
     }
    }
    __syncthreads();

    // ------------------------------------------------ off-diagonal inverse blocks
    // I + A = [[L1, 0], [B, L2]] in 32x32 halves: the inverse is
    // [[L1^-1, 0], [-L2^-1 B L1^-1, L2^-1]], with L1^-1 and L2^-1 from their
    // diagonal 16x16 inverses (fp32 16x16x4 matrix-core products, in place of A)
    if (wave < 2) {   // T_10 = -T_11 A_10 T_00 and T_32 = -T_33 A_32 T_22
      const int I = wave ? 3 : 1, J = I - 1;
      f32x4_t y = {0.f, 0.f, 0.f, 0.f}, tt = y;
      const float4 aIJ = at_row4(16 * I + l16, 16 * J + 4 * g4);
      const float4 aII = at_row4(16 * I + l16, 16 * I + 4 * g4);
      const float aij[4] = {aIJ.x, aIJ.y, aIJ.z, aIJ.w}, aii[4] = {aII.x, aII.y, aII.z, aII.w};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(aij[st], at_el(16 * J + 4 * g4 + st, 16 * J + l16), y, 0, 0, 0);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        tt = __builtin_amdgcn_mfma_f32_16x16x4f32(aii[st], y[st], tt, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) at_el(16 * I + 4 * g4 + i, 16 * J + l16) = -tt[i];
    }
    __syncthreads();
    float* xs = reinterpret_cast<float*>(smem + CF::XS);
    const int bi = 2 + ((wave & 3) >> 1), bj = wave & 1;   // lower-left 16x16 block (waves 0-3)
    if (NW == 4 || wave < 4) {   // X_{bi,bj} = sum_{m=bj}^{1} A_{bi,m} T_{m,bj}
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m >= bj) {
          const float4 a4 = at_row4(16 * bi + l16, 16 * m + 4 * g4);
          const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int st = 0; st < 4; ++st)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], at_el(16 * m + 4 * g4 + st, 16 * bj + l16), acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[(wave * 16 + 4 * g4 + i) * CF::XLD + l16] = acc[i];
    }
    __syncthreads();
    if (NW == 4 || wave < 4) {   // T_{bi,bj} = -sum_{m=2}^{bi} T_{bi,m} X_{m,bj}
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 2; m < 4; ++m) {
        if (m <= bi) {
          const int xw = (m - 2) * 2 + bj;
          const float4 a4 = at_row4(16 * bi + l16, 16 * m + 4 * g4);
          const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int st = 0; st < 4; ++st)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], xs[(xw * 16 + 4 * g4 + st) * CF::XLD + l16],
                                                       acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) at_el(16 * bi + 4 * g4 + i, 16 * bj + l16) = -acc[i];
    }
    __syncthreads();
    // bf16 operands: Tb = T Diag(beta) row-major (TBR) and transposed (TBT), in place
    // of the fp32 T, so the later products read whole 16-byte fragments
    char* tbr = atc;
    char* tbt = atc + kC * CF::RBC;
    // each thread handles VPTH consecutive entries of one row
    constexpr int TPR = NT / kC, VPTH = kC / TPR;
    if constexpr (!F32) {
      const int t = tid / TPR, s0 = (tid % TPR) * VPTH;
      float x[VPTH];
#pragma unroll
      for (int q4 = 0; q4 < VPTH / 4; ++q4) {
        const float4 u = at_row4(t, s0 + 4 * q4);
        const float4 b = *reinterpret_cast<const float4*>(betas + s0 + 4 * q4);
        x[4 * q4] = u.x * b.x; x[4 * q4 + 1] = u.y * b.y; x[4 * q4 + 2] = u.z * b.z; x[4 * q4 + 3] = u.w * b.w;
      }
      __syncthreads();   // all of T is read before its space is reused
#pragma unroll
      for (int h8 = 0; h8 < VPTH / 8; ++h8) {
        const int o = 8 * h8;
        *reinterpret_cast<i32x4_t*>(tbr + swz<CF::RBC>(t, (s0 + o) * 2)) = i32x4_t{
            static_cast<int>(pack_bf16x2(x[o], x[o + 1])), static_cast<int>(pack_bf16x2(x[o + 2], x[o + 3])),
            static_cast<int>(pack_bf16x2(x[o + 4], x[o + 5])), static_cast<int>(pack_bf16x2(x[o + 6], x[o + 7]))};
      }
#pragma unroll
      for (int e = 0; e < VPTH; ++e) lds_set1<false>(tbt + swz<CF::RBC>(s0 + e, t * 2), x[e]);
      __syncthreads();
    }

    // ------------------------------------------------ P = scale M Tb, stored as P[t][t']
    // computed transposed: P^T[t'][t] = sum_s Tb[s][t'] M[t][s], nonzero for t' <= t
#pragma unroll
    for (int pp = 0; pp < (10 + NW - 1) / NW; ++pp) {
      const int pr = wave + NW * pp;
      if (pr < 10) {
        int C, R;
        pair_of(pr, C, R);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int sb = kk * 32 + g4 * 8;
          Frag<F32> a;
          if constexpr (F32) {
            const float bcol = betas[16 * R + l16];     // Tb[s][t'] = T[s][t'] beta_t'
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = at_el(sb + e, 16 * R + l16) * bcol;
            a = frag_from_f32<F32>(x);
          } else {
            a = lds_frag<F32, CF::RBC>(tbt, 16 * R + l16, sb * E);
          }
          const Frag<F32> bm = lds_frag<F32, CF::RBC>(smem + CF::MB, 16 * C + l16, sb * E);
          acc = mma32<F32>(acc, a, bm);
        }
        const int t = 16 * C + l16, tp = 16 * R + 4 * g4;
        lds_put4<F32>(smem + CF::PB + swz<CF::RBC>(t, tp * E), acc[0], acc[1], acc[2], acc[3]);
        buf_put4<F32>(rw, SL::PP + frag_off<kC, F32>(t, tp), p.scale * acc[0], p.scale * acc[1],
                      p.scale * acc[2], p.scale * acc[3]);
      }
    }
    for (int e = tid; e < 6 * 64; e += NT) {   // P[t][t'] = 0 for t' sub-tile > t sub-tile
      int C, R;
      upper_pair(e >> 6, C, R);
      const int t = 16 * C + ((e >> 2) & 15), tp = 16 * R + 4 * (e & 3);
      lds_put4<F32>(smem + CF::PB + swz<CF::RBC>(t, tp * E), 0.f, 0.f, 0.f, 0.f);
      buf_put4<F32>(rw, SL::PP + frag_off<kC, F32>(t, tp), 0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    // ------------------------------------------------ W and Q'
    // W^T = (K e^G)^T Tb^T and Q'^T = scale ((Q e^G)^T - (K e^G)^T P^T); lane holds
    // 4 consecutive channels of one token row -> 4-element stores of W[t][c], Q'[t][c]
    {
      constexpr int RPW = D / (16 * NW);  // 16-row channel tiles per wavefront
      f32x4_t aw[RPW][4], aq[RPW][4];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          aw[rr][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          aq[rr][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int t = 16 * ct + l16;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk == 1 && ct < 2) continue;     // Tb[t][s] = P[t][s] = 0 for s > t
          const int sb = kk * 32 + g4 * 8;
          Frag<F32> bw;
          if constexpr (F32) {
            float x[8];
            const float4 u0 = *reinterpret_cast<const float4*>(atc + swz<256>(t, sb * 4));
            const float4 u1 = *reinterpret_cast<const float4*>(atc + swz<256>(t, sb * 4 + 16));
            const float4 b0 = *reinterpret_cast<const float4*>(betas + sb);
            const float4 b1 = *reinterpret_cast<const float4*>(betas + sb + 4);
            x[0] = u0.x * b0.x; x[1] = u0.y * b0.y; x[2] = u0.z * b0.z; x[3] = u0.w * b0.w;
            x[4] = u1.x * b1.x; x[5] = u1.y * b1.y; x[6] = u1.z * b1.z; x[7] = u1.w * b1.w;
            bw = frag_from_f32<F32>(x);
          } else {
            bw = lds_frag<F32, CF::RBC>(tbr, t, sb * E);
          }
          const Frag<F32> bq = lds_frag<F32, CF::RBC>(smem + CF::PB, t, sb * E);
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) {
            const int c = 16 * (wave * RPW + rr) + l16;
            const Frag<F32> a = lds_frag<F32, CF::RBC>(smem + CF::KBT, c, sb * E);
            aw[rr][ct] = mma32<F32>(aw[rr][ct], a, bw);
            aq[rr][ct] = mma32<F32>(aq[rr][ct], a, bq);
          }
        }
      }
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const int c = 16 * (wave * RPW + rr) + 4 * g4;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int t = 16 * ct + l16;
          buf_put4<F32>(rw, SL::W + frag_off<D, F32>(t, c), aw[rr][ct][0], aw[rr][ct][1],
                        aw[rr][ct][2], aw[rr][ct][3]);
          float qb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) qb[i] = lds_get1<F32>(smem + CF::QB + swz<CF::RBD>(t, (c + i) * E));
          buf_put4<F32>(rw, SL::QP + frag_off<D, F32>(t, c), p.scale * (qb[0] - aq[rr][ct][0]),
                        p.scale * (qb[1] - aq[rr][ct][1]), p.scale * (qb[2] - aq[rr][ct][2]),
                        p.scale * (qb[3] - aq[rr][ct][3]));
        }
      }
    }
    // Tb = T Diag(beta) -> workspace, VPTH consecutive entries per thread
    if constexpr (!F32) {
      const int t = tid / TPR, s0 = (tid % TPR) * VPTH;
#pragma unroll
      for (int h8 = 0; h8 < VPTH / 8; ++h8) {
        const i32x4_t w = *reinterpret_cast<const i32x4_t*>(tbr + swz<CF::RBC>(t, (s0 + 8 * h8) * 2));
        buf_st64(i32x2_t{w[0], w[1]}, rw, SL::TB + frag_off<kC, F32>(t, s0 + 8 * h8), 0);
        buf_st64(i32x2_t{w[2], w[3]}, rw, SL::TB + frag_off<kC, F32>(t, s0 + 8 * h8 + 4), 0);
      }
    } else {
      const int t = tid >> 2, s0 = (tid & 3) * 16;
      float x[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 u = *reinterpret_cast<const float4*>(atc + swz<256>(t, (s0 + 4 * q4) * 4));
        const float4 b = *reinterpret_cast<const float4*>(betas + s0 + 4 * q4);
        x[4 * q4] = u.x * b.x; x[4 * q4 + 1] = u.y * b.y; x[4 * q4 + 2] = u.z * b.z; x[4 * q4 + 3] = u.w * b.w;
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        buf_put4<F32>(rw, SL::TB + frag_off<kC, F32>(t, s0 + 4 * q4), x[4 * q4], x[4 * q4 + 1],
                      x[4 * q4 + 2], x[4 * q4 + 3]);
    }
  }
}

// One workgroup per (workspace slot, head) item.
template <int D, typename TIn>
__global__ __launch_bounds__(kThreads, 2) void chunk_prep_kernel(PrepParams p) {
  __shared__ __attribute__((aligned(16))) char smem[PrepCfg<D, TIn>::LDS];
  const PrepItem it = prep_item(p, blockIdx.x);
  if (!it.valid) return;         // unused workspace slot
  prep_body<D, TIn>(p, smem, it,
                    p.ws + (static_cast<int64_t>(it.slot) * p.sa.H + it.h) *
                               Slot<D, std::is_same<TIn, float>::value>::BYTES);
}

// The same with 8 wavefronts per item (d = 128, bf16): two workgroups, 16
// wavefronts, share a CU.
__global__ __launch_bounds__(2 * kThreads, 2) void chunk_prep8_kernel(PrepParams p) {
  __shared__ __attribute__((aligned(16))) char smem[PrepCfg<128, bf16_t>::LDS];
  const PrepItem it = prep_item(p, blockIdx.x);
  if (!it.valid) return;         // unused workspace slot
  prep_body<128, bf16_t, 8>(p, smem, it,
                            p.ws + (static_cast<int64_t>(it.slot) * p.sa.H + it.h) *
                                       Slot<128, false>::BYTES);
}

// ================================================================= kernel 2

template <int D, int DVS, typename TIn>
struct ScanCfg {
  static constexpr bool F32 = std::is_same<TIn, float>::value;
  static constexpr int E = F32 ? 4 : 2;
  static constexpr int EI = sizeof(TIn);
  static constexpr int NJT = DVS / 16;
  static constexpr int NKK = D / 32;
  static constexpr int RT = D / 64;             // state row tiles per wavefront
  static constexpr int NSPLIT = D / DVS;
  static constexpr int RBD = D * E;             // SB rows [j][c]
  static constexpr int RBC = kC * E;            // VT, DT rows [j][t]
  static constexpr int RBO = DVS * E + 16;      // OST rows [t][j] (padded)
  static constexpr int SB = 0;
  static constexpr int VT = SB + DVS * RBD;
  static constexpr int DT = VT + DVS * RBC;
  static constexpr int OST = DT + DVS * RBC;
  static constexpr int OSTB = kC * RBO;         // one output stage; two alternate
  static constexpr int ORD = OST + 2 * OSTB;
  static constexpr int SNAP = ORD + 256 * 4;    // varlen: first snapshot row of the sequence
  static constexpr int LDS = SNAP + 16;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

struct ScanParams {
  const void* v;
  const float* s0;     // initial states (null: zero), read by the window holding chunk 0
  void* out;
  float* sT;           // final states (null: not written), written by the window holding
                       // a sequence's last chunk
  float* sbuf;         // states carried between windows
  const char* ws;
  SeqArgs sa;
  int c_lo, c_hi;      // chunk window [c_lo, c_hi) of every sequence
  int cg;              // > 0: group workspace, slot (n * cg + c - c_lo) * H + h;
                       // 0: slot (tok0 / 64 + n + c) * H + h
  float* snap;         // [N, H, nsnap, D, D]: state after every snap_chunks chunks and
  int snap_chunks;     // after the last chunk; null: none
  int nsnap;
};

// The chunks of one window of one (sequence, head, dv slice), in order, by one
// workgroup (`bid` numbers the scan workgroups of the launch from 0).  PACKED =
// false compiles out what only packed (varlen) input needs, for the windowed
// schedule, which runs fixed-length input only.
template <int D, int DVS, typename TIn, bool PACKED = true>
__device__ __forceinline__ void scan_body(const ScanParams& p, char* smem, const int bid) {
  using CF = ScanCfg<D, DVS, TIn>;
  using SL = Slot<D, CF::F32>;
  constexpr bool F32 = CF::F32;
  constexpr int E = CF::E, EI = CF::EI, NJT = CF::NJT, NKK = CF::NKK, RT = CF::RT;

  // the wavefront index is uniform: keeping it scalar makes per-wavefront branches
  // and offsets scalar work
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int H = p.sa.H, N = p.sa.N;

  // XCD-aware placement: the dv slices of one (sequence, head) land on one XCD
  const int xcd = bid & 7, r8 = bid >> 3;
  const int grp = (r8 / CF::NSPLIT) * 8 + xcd;
  const int split = r8 % CF::NSPLIT;
  if (grp >= N * H) return;
  const int rank = grp / H, h = grp % H;
  int n = rank;
  if (PACKED && p.sa.cu != nullptr && N <= 256) {   // longest sequence first
    int* ord = reinterpret_cast<int*>(smem + CF::ORD);
    int mylen = 0;
    if (tid < N) {
      int a, l;
      seq_bounds(p.sa, tid, a, l);
      mylen = l;
      ord[tid] = l;
    }
    __syncthreads();
    int rk = 0;
    if (tid < N)
      for (int m = 0; m < N; ++m) {
        const int lm = ord[m];
        rk += (lm > mylen) || (lm == mylen && m < tid);
      }
    __syncthreads();
    if (tid < N) ord[rk] = tid;
    __syncthreads();
    n = ord[rank];
    __syncthreads();
  }
  int tok0, len;
  seq_bounds(p.sa, n, tok0, len);
  const int nchunks = (len + kC - 1) / kC;
  const int c_begin = p.c_lo, c_end = min(p.c_hi, nchunks);
  if (c_begin >= c_end && c_begin > 0) return;   // the sequence ended in an earlier window
  const int sbase = p.cg > 0 ? n * p.cg - p.c_lo : slot_base(tok0, n);
  const int j0 = split * DVS;

  // Snapshot i of this (sequence, head): fixed length, [N, H, nsnap] order; varlen,
  // row off_n + i of [snapshots, H], where off_n counts the snapshots of the
  // sequences before n (ceil(chunks / snap_chunks) each).  Wavefront 0 sums off_n
  // over its lanes into LDS (ordered by the barrier after the state load), where
  // the snapshot stores read it, so no register holds it across the steps.
  if (PACKED && p.snap != nullptr && p.sa.cu != nullptr && wave == 0) {
    int part = 0;
    for (int m = lane; m < n; m += 64) {
      int t0m, lm;
      seq_bounds(p.sa, m, t0m, lm);
      part += ((lm + kC - 1) / kC + p.snap_chunks - 1) / p.snap_chunks;
    }
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) *reinterpret_cast<int*>(smem + CF::SNAP) = part;
  }
  auto snap_ptr = [&](int si) -> float* {
    if (!PACKED || p.sa.cu == nullptr)
      return p.snap + ((static_cast<int64_t>(n) * H + h) * p.nsnap + si) * D * D;
    const int off = *reinterpret_cast<const int*>(smem + CF::SNAP);
    return p.snap + (static_cast<int64_t>(off + si) * H + h) * D * D;
  };
  const float* s_in = c_begin == 0 ? p.s0 : p.sbuf;
  float* s_out = p.c_hi >= nchunks ? p.sT : p.sbuf;

  // state tiles (rt, jt): rows c = 16*rt + 4*g4 + i, columns j = 16*jt + l16
  f32x4_t S[RT][NJT];
  {
    const float* s0 = s_in ? s_in + (static_cast<int64_t>(n) * H + h) * D * D : nullptr;
#pragma unroll
    for (int ri = 0; ri < RT; ++ri)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const int rt = wave * RT + ri;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[ri][jt][i] = s0 ? s0[(16 * rt + 4 * g4 + i) * D + j0 + 16 * jt + l16] : 0.f;
        lds_put4<F32>(smem + CF::SB + swz<CF::RBD>(16 * jt + l16, (16 * rt + 4 * g4) * E),
                      S[ri][jt][0], S[ri][jt][1], S[ri][jt][2], S[ri][jt][3]);
      }
  }
  __syncthreads();

  const uint32_t rs_v = static_cast<uint32_t>(H) * D * EI;
  constexpr int VPR = DVS / 8;                      // 8-value pieces per V row
  constexpr int VPT = (kC * VPR + kThreads - 1) / kThreads;   // pieces per thread

  // Everything one chunk needs from memory, held in registers so the next chunk's
  // loads can be issued before the current chunk's products start.
  struct ChunkRegs {
    Frag<F32> fw[NKK], fq[NKK], ftb[2], fpp[2], fkt[RT][2];
    i32x4_t lam[RT];
    i32x4_t vv[VPT][F32 ? 2 : 1];
  };
  // Loads of one chunk come in three groups, issued at three points of the previous
  // step so that the memory pipeline streams while the wavefront computes instead of
  // stalling the wavefront at issue: V, Tb and P (first used at the top of the step),
  // W and Q' (first products), Kt and Lambda (state update).  Vector-memory counters
  // retire in order, so each use waits only for its own group.
  constexpr uint32_t FB = F32 ? 2048 : 1024;      // bytes per fragment (see frag_off)
  auto slot_rsrc = [&](int ci) {
    return make_rsrc(p.ws + (static_cast<int64_t>(sbase + ci) * H + h) * SL::BYTES, SL::BYTES);
  };
  auto load_group1 = [&](int ci, ChunkRegs& cr) {
    const int t0 = tok0 + ci * kC;
    const int nrow = min(kC, len - ci * kC);
    const auto rw = slot_rsrc(ci);
    const int64_t vbase = (static_cast<int64_t>(t0) * H + h) * D + j0;
    const auto rv = make_rsrc(static_cast<const TIn*>(p.v) + vbase, (nrow - 1) * rs_v + DVS * EI);
#pragma unroll
    for (int pi = 0; pi < VPT; ++pi) {
      // pieces beyond the tile (narrow slices) re-read the last row; they are not stored
      const int pc = min(tid + pi * kThreads, kC * VPR - 1);
      const int vrow = pc / VPR, vcol = (pc % VPR) * 8;   // rows past the end read zero
      // per-lane offsets go in the vector offset (a per-lane scalar offset would
      // serialise the instruction over the distinct values)
      const uint32_t vo = vrow * rs_v + vcol * EI;
      cr.vv[pi][0] = buf_ld128(rv, vo, 0);
      if constexpr (F32) cr.vv[pi][1] = buf_ld128(rv, vo + 16, 0);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t o = (wave * 2 + kk) * FB + lane * 16;
      cr.ftb[kk] = buf_frag2<F32>(rw, SL::TB + o);
      cr.fpp[kk] = buf_frag2<F32>(rw, SL::PP + o);
    }
  };
  auto load_group2 = [&](int ci, ChunkRegs& cr) {
    const auto rw = slot_rsrc(ci);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint32_t o = (wave * NKK + kk) * FB + lane * 16;
      cr.fw[kk] = buf_frag2<F32>(rw, SL::W + o);
      cr.fq[kk] = buf_frag2<F32>(rw, SL::QP + o);
    }
  };
  auto load_group3 = [&](int ci, ChunkRegs& cr) {
    const auto rw = slot_rsrc(ci);
#pragma unroll
    for (int ri = 0; ri < RT; ++ri)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        cr.fkt[ri][kk] = buf_frag2<F32>(rw, SL::KT + ((wave * RT + ri) * 2 + kk) * FB + lane * 16);
#pragma unroll
    for (int ri = 0; ri < RT; ++ri)
      cr.lam[ri] = buf_ld128(rw, SL::LAM + (16 * (wave * RT + ri) + 4 * g4) * 4, 0);
  };

  // Output of chunk cj, staged in LDS by its step, is written one step later, after
  // that step's loads have been waited for: stores share the loads' counter, so a
  // store issued just before a wait would make the wait cover its completion.
  auto store_out = [&](const int cj) {
    const int t0 = tok0 + cj * kC;
    const int nrow = min(kC, len - cj * kC);
    const int64_t vbase = (static_cast<int64_t>(t0) * H + h) * D + j0;
    const auto ro = make_rsrc(static_cast<TIn*>(p.out) + vbase, (nrow - 1) * rs_v + DVS * EI);
    const char* ost = smem + CF::OST + (cj & 1) * CF::OSTB;
    constexpr int PPR = DVS * E / 16;    // 16-byte pieces per output row
    for (int pc = tid; pc < kC * PPR; pc += kThreads) {
      const int t = pc / PPR, part = pc % PPR;
      const i32x4_t val = *reinterpret_cast<const i32x4_t*>(ost + t * CF::RBO + part * 16);
      // plain stores (a row's other column slices arrive from other workgroups, and
      // the cache joins the pieces into whole lines: with the non-temporal hint each
      // piece went to memory on its own, measured as extra write traffic); rows past
      // the sequence end are dropped by the range check
      buf_st128(val, ro, t * rs_v + part * 16, 0);
    }
  };

  // This workgroup's columns of the state, to a [D][D] fp32 matrix.
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int ri = 0; ri < RT; ++ri)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * (wave * RT + ri) + 4 * g4 + i) * D + j0 + 16 * jt + l16] = S[ri][jt][i];
  };

  // Two register sets alternate.  Step ci computes from `cur` while the loads of chunk cn (ci + 1, clamped so the
  // last step re-reads itself and no load sits behind a branch) fill `nxt`.
  auto process = [&](const int ci, const ChunkRegs& cur, const int cn, ChunkRegs& nxt) {
    load_group1(cn, nxt);
    __builtin_amdgcn_sched_barrier(0);
    // V slice, transposed to [j][t]
#pragma unroll
    for (int pi = 0; pi < VPT; ++pi) {
      const int pc = tid + pi * kThreads;
      if ((kC * VPR) % kThreads == 0 || pc < kC * VPR) {
        const int vrow = pc / VPR, vcol = (pc % VPR) * 8;
        if constexpr (F32) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<int*>(smem + CF::VT + swz<CF::RBC>(vcol + i, vrow * 4)) = cur.vv[pi][0][i];
            *reinterpret_cast<int*>(smem + CF::VT + swz<CF::RBC>(vcol + 4 + i, vrow * 4)) = cur.vv[pi][1][i];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint16_t*>(smem + CF::VT + swz<CF::RBC>(vcol + e, vrow * 2)) =
                static_cast<uint16_t>(static_cast<uint32_t>(cur.vv[pi][0][e >> 1]) >> (16 * (e & 1)));
        }
      }
    }
    if (ci > c_begin) store_out(ci - 1);
    __syncthreads();

    // U = Tb V and O_v = P V (state independent), W S and Q' S (state products).
    // All B fragments are read from LDS first so their latencies overlap.
    Frag<F32> bv[NJT][2], bs[NJT][NKK];
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        bv[jt][kk] = lds_frag<F32, CF::RBC>(smem + CF::VT, 16 * jt + l16, (kk * 32 + g4 * 8) * E);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        bs[jt][kk] = lds_frag<F32, CF::RBD>(smem + CF::SB, 16 * jt + l16, (kk * 32 + g4 * 8) * E);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_group2(cn, nxt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      f32x4_t u = {0.f, 0.f, 0.f, 0.f}, ov = u, ws = u, qs = u;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u = mma32<F32>(u, cur.ftb[kk], bv[jt][kk]);
        ov = mma32<F32>(ov, cur.fpp[kk], bv[jt][kk]);
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        ws = mma32<F32>(ws, cur.fw[kk], bs[jt][kk]);
        qs = mma32<F32>(qs, cur.fq[kk], bs[jt][kk]);
      }
      // Delta = U - W S -> [j][t];  O = Q' S + P V -> [t][j]
      const int j = 16 * jt + l16, t = 16 * wave + 4 * g4;
      lds_put4<F32>(smem + CF::DT + swz<CF::RBC>(j, t * E), u[0] - ws[0], u[1] - ws[1],
                    u[2] - ws[2], u[3] - ws[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lds_set1<F32>(smem + CF::OST + (ci & 1) * CF::OSTB + (t + i) * CF::RBO + j * E, qs[i] + ov[i]);
    }
    __syncthreads();

    // S <- Diag(Lambda) S + Kt^T Delta
    load_group3(cn, nxt);
    __builtin_amdgcn_sched_barrier(0);
    Frag<F32> bd[NJT][2];
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        bd[jt][kk] = lds_frag<F32, CF::RBC>(smem + CF::DT, 16 * jt + l16, (kk * 32 + g4 * 8) * E);
#pragma unroll
    for (int ri = 0; ri < RT; ++ri) {
      const int rt = wave * RT + ri;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        f32x4_t acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = S[ri][jt][i] * __int_as_float(cur.lam[ri][i]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) acc = mma32<F32>(acc, cur.fkt[ri][kk], bd[jt][kk]);
        S[ri][jt] = acc;
        lds_put4<F32>(smem + CF::SB + swz<CF::RBD>(16 * jt + l16, (16 * rt + 4 * g4) * E),
                      acc[0], acc[1], acc[2], acc[3]);
      }
    }
    if (p.snap != nullptr && (ci + 1 == nchunks || (ci + 1) % p.snap_chunks == 0)) {
      // state after chunk ci: a prefix-cache snapshot
      // the last snapshot is number ceil(nchunks / snap_chunks) - 1 (nsnap - 1 for
      // fixed length)
      const int si = ci + 1 != nchunks ? (ci + 1) / p.snap_chunks - 1
                     : !PACKED || p.sa.cu == nullptr ? p.nsnap - 1 : (nchunks - 1) / p.snap_chunks;
      store_state(snap_ptr(si));
    }
    __syncthreads();
  };

  ChunkRegs bufA, bufB;
  if (c_end > c_begin) {
    load_group1(c_begin, bufA);
    load_group2(c_begin, bufA);
    load_group3(c_begin, bufA);
  }
  for (int ci = c_begin; ci < c_end; ci += 2) {
    process(ci, bufA, min(ci + 1, c_end - 1), bufB);
    if (ci + 1 >= c_end) break;
    process(ci + 1, bufB, min(ci + 2, c_end - 1), bufA);
  }
  if (c_end > c_begin) store_out(c_end - 1);

  if (s_out) store_state(s_out + (static_cast<int64_t>(n) * H + h) * D * D);
}

template <int D, int DVS, typename TIn>
__global__ __launch_bounds__(kThreads, 1) void state_scan_kernel(ScanParams p) {
  __shared__ __attribute__((aligned(16))) char smem[ScanCfg<D, DVS, TIn>::LDS];
  scan_body<D, DVS, TIn>(p, smem, blockIdx.x);
}

// ================================================================= grouped launch
// Fixed-length prefill runs in windows of cg chunks.  Launch k carries the scan of
// window k-1 (workgroups 0 .. nscan-1) and the preparation of window k (the rest),
// whose workspaces alternate between two buffers.  The two roles are independent
// within a launch -- the scan reads what the previous launch prepared -- so the
// memory-bound scan and the arithmetic-bound preparation share the CUs, and the
// workspace a scan reads was written one launch earlier, small enough to still be
// in cache.
struct GroupParams {
  PrepParams pp;
  ScanParams sp;
  int nscan;
};

template <int D, int DVS, typename TIn>
struct GroupCfg {
  static constexpr int A = PrepCfg<D, TIn>::LDS, B = ScanCfg<D, DVS, TIn>::LDS;
  static constexpr int LDS = A > B ? A : B;
};

template <int D, int DVS, typename TIn>
__global__ __launch_bounds__(kThreads, 2) void prefill_group_kernel(GroupParams g) {
  __shared__ __attribute__((aligned(16))) char smem[GroupCfg<D, DVS, TIn>::LDS];
  const int bid = blockIdx.x;
  if (bid < g.nscan) {
    scan_body<D, DVS, TIn, false>(g.sp, smem, bid);
    return;
  }
  int slot = 0;
  const PrepItem it = prep_group_item(g.pp, bid - g.nscan, slot);
  if (!it.valid) return;
  prep_body<D, TIn>(g.pp, smem, it,
                    g.pp.ws + (static_cast<int64_t>(slot) * g.pp.sa.H + it.h) *
                                  Slot<D, std::is_same<TIn, float>::value>::BYTES);
}

// ---------------------------------------------------------------- launch

// Scan workgroups for N*H (sequence, head) streams cut into D/DVS slices, padded so
// that the slices of one stream share an XCD.
template <int D, int DVS>
int scan_grid(int streams) { return ((streams + 7) / 8) * 8 * (D / DVS); }

template <int D, int DVS, typename TIn>
hipError_t launch_scan(const PrefillArgs& a, const SeqArgs& sa, const char* ws) {
  const ScanParams sp{a.v, a.initial_state, a.out, a.final_state, nullptr, ws, sa, 0, 1 << 30, 0,
                      a.snapshots, std::max(a.snap_chunks, 1), a.nsnap};
  hipLaunchKernelGGL((state_scan_kernel<D, DVS, TIn>), dim3(scan_grid<D, DVS>(a.N * a.H)),
                     dim3(kThreads), 0, a.stream, sp);
  return hipGetLastError();
}

// Chunks per window of the grouped launch.
inline int group_chunks(int nchunks) {
  // at most 8 windows (each launch boundary drains the machine) and at least 16
  // chunks per window (the scan role needs enough steps to amortise its state
  // round trip through memory)
  const int cg = std::max(16, (nchunks + 7) / 8);
  return std::min(cg, nchunks);
}

// Workspace of a windowed call: two window buffers of slots (one if a single window
// covers the sequences) and, with more than one window, the states carried between
// windows.
template <int D, typename TIn>
size_t grouped_bytes(const PrefillArgs& a, int cg) {
  using SL = Slot<D, std::is_same<TIn, float>::value>;
  const int nchunks = (a.T + kC - 1) / kC;
  const int windows = (nchunks + cg - 1) / cg;
  const size_t wbytes = static_cast<size_t>(a.N) * cg * a.H * SL::BYTES;
  const size_t sbytes = windows > 1 ? static_cast<size_t>(a.N) * a.H * D * D * 4 : 0;
  return (windows > 1 ? 2 : 1) * wbytes + sbytes;
}

// Workspace of a two-kernel call: one slot for every chunk (see slot_base).
template <int D, typename TIn>
size_t all_chunks_bytes(const PrefillArgs& a) {
  using SL = Slot<D, std::is_same<TIn, float>::value>;
  const int64_t slots = (a.total_T + kC - 1) / kC + a.N;
  return static_cast<size_t>(slots) * a.H * SL::BYTES;
}

// The caller's workspace when it passed one (too small: invalid value), else a block
// from the library's kept blocks.
hipError_t ws_acquire(const PrefillArgs& a, size_t bytes, char** p) {
  return kda::ws_acquire(a.workspace, a.workspace_bytes, bytes, a.stream, p);
}

hipError_t ws_release(const PrefillArgs& a, char* p) {
  return kda::ws_release(a.workspace, p, a.stream);
}

template <int D, int DVS, typename TIn>
hipError_t launch_grouped(const PrefillArgs& a, int cg) {
  constexpr bool F32 = std::is_same<TIn, float>::value;
  using SL = Slot<D, F32>;
  const SeqArgs sa{a.cu_seqlens, a.N, a.T, a.total_T, a.H};
  const int nchunks = (a.T + kC - 1) / kC;
  const int windows = (nchunks + cg - 1) / cg;
  const size_t wbytes = static_cast<size_t>(a.N) * cg * a.H * SL::BYTES;
  const int nbuf = windows > 1 ? 2 : 1;
  char* ws = nullptr;
  hipError_t err = ws_acquire(a, grouped_bytes<D, TIn>(a, cg), &ws);
  if (err != hipSuccess) return err;
  float* sbuf = windows > 1 ? reinterpret_cast<float*>(ws + nbuf * wbytes) : nullptr;
  const int nscan = scan_grid<D, DVS>(a.N * a.H);
  const int items = a.N * cg * a.H;
  for (int k = 0; k <= windows && err == hipSuccess; ++k) {
    GroupParams gp{};
    gp.nscan = k >= 1 ? nscan : 0;
    gp.sp = ScanParams{a.v, a.initial_state, a.out, a.final_state, sbuf,
                       ws + ((k + 1) % nbuf) * wbytes, sa, (k - 1) * cg, k * cg, cg,
                       a.snapshots, std::max(a.snap_chunks, 1), a.nsnap};
    gp.pp = PrepParams{a.q, a.k, a.g, a.beta, ws + (k % nbuf) * wbytes, sa, a.scale,
                       k < windows ? items : 0, k * cg, cg, a.prologue ? 1 : 0};
    const int grid = gp.nscan + gp.pp.items;
    hipLaunchKernelGGL((prefill_group_kernel<D, DVS, TIn>), dim3(grid), dim3(kThreads), 0,
                       a.stream, gp);
    err = hipGetLastError();
  }
  const hipError_t ferr = ws_release(a, ws);
  return err != hipSuccess ? err : ferr;
}

// Streams from which the two-kernel schedule with 64-column scan slices is used:
// 2 workgroups per stream then still cover the 256 CUs, and every chunk's operands
// are read by 2 workgroups instead of 4 (a CU takes in operands at a fixed rate, so
// the scan's time follows the operand bytes each CU moves).
constexpr int kWideStreams = 128;

// Chunks per window of a fixed-length call; 0 selects the two-kernel schedule:
// always for varlen input and from kWideStreams streams on; for bf16 at d = 128
// also from 64 streams on when the sequences have at most 64 chunks, where the
// windowed schedule's first and last launches (preparation alone, scan alone) are
// a large share of the call and the 8-wavefront preparation is available instead.
inline int prefill_cg(const PrefillArgs& a) {
  if (a.cu_seqlens != nullptr) return 0;
  const int nchunks = (a.T + kC - 1) / kC;
  if (a.window_chunks > 0) return std::min(a.window_chunks, nchunks);
  const int cg = group_chunks(nchunks);
  const int streams = a.N * a.H;
  if (streams >= kWideStreams) return 0;
  if (!a.dtype_f32 && a.d == 128 && streams >= 64 && nchunks <= 64) return 0;
  return cg;
}

// Streams from which bf16 d = 128 prefill runs fused (fused_prefill_kernel): one
// workgroup per (sequence, head) keeps every CU busy and no chunk operand goes
// through memory.
constexpr int kFusedStreams = 256;

inline bool use_fused(const PrefillArgs& a) {
  return a.window_chunks == 0 && fused_prefill_supported(a) &&
         static_cast<int64_t>(a.N) * a.H >= kFusedStreams;
}

// Segments per sequence for fixed-length bf16 d = 128 prefill from 4 to 32 streams
// (0: not segmented): as many as keep every launch within one workgroup per CU (at
// most 32), each of at least 16 chunks.  The segmented schedule runs the fused
// kernel over about three times the chunks of one pass, spread over R times the
// workgroups: measured against the windowed schedule it wins from 8 segments of 16
// chunks on (1 x 65536 tokens x 32 heads: 1.91 against 2.12 ms; x 16 heads: 0.95
// against 1.72 ms) and loses with 4 or 5 segments or 8-chunk segments.
inline int fused_segments(const PrefillArgs& a) {
  if (a.window_chunks != 0 || a.cu_seqlens != nullptr || !fused_prefill_supported(a)) return 0;
  const int64_t streams = static_cast<int64_t>(a.N) * a.H;
  if (streams < 4 || streams > 32) return 0;
  const int R = static_cast<int>(std::min<int64_t>(32, kFusedStreams / streams));
  const int nchunks = (a.T + kC - 1) / kC;
  return nchunks >= 16 * R ? R : 0;
}

template <int D, typename TIn>
size_t workspace_bytes(const PrefillArgs& a) {
  if (use_fused(a)) return 0;
  if (const int R = fused_segments(a)) return fused_segmented_bytes(a, R);
  const int cg = prefill_cg(a);
  return cg > 0 ? grouped_bytes<D, TIn>(a, cg) : all_chunks_bytes<D, TIn>(a);
}

template <int D, typename TIn>
hipError_t launch_all(const PrefillArgs& a) {
  const int cg = prefill_cg(a);
  if (cg > 0) {   // fixed length: windows of cg chunks
    // slices of at most 32 columns keep the scan role within 256 registers, so a
    // scan and a preparation workgroup fit on one CU together; 16-column slices
    // only for fewer than 32 streams, where the scan's own latency dominates
    if (a.N * a.H < 32) return launch_grouped<D, 16, TIn>(a, cg);
    return launch_grouped<D, 32, TIn>(a, cg);
  }
  const SeqArgs sa{a.cu_seqlens, a.N, a.T, a.total_T, a.H};
  const int64_t slots = (a.total_T + kC - 1) / kC + a.N;
  char* ws = nullptr;
  hipError_t err = ws_acquire(a, all_chunks_bytes<D, TIn>(a), &ws);
  if (err != hipSuccess) return err;
  const int64_t items = slots * a.H;
  PrepParams pp{a.q, a.k, a.g, a.beta, ws, sa, a.scale, static_cast<int>(items), 0, 0,
                a.prologue ? 1 : 0};
  const unsigned prep_grid = static_cast<unsigned>(items);
  if (D == 128 && std::is_same<TIn, bf16_t>::value)
    hipLaunchKernelGGL(chunk_prep8_kernel, dim3(prep_grid), dim3(2 * kThreads), 0, a.stream, pp);
  else
    hipLaunchKernelGGL((chunk_prep_kernel<D, TIn>), dim3(prep_grid), dim3(kThreads), 0, a.stream, pp);
  err = hipGetLastError();
  if (err == hipSuccess) {
    // enough (sequence, head, dv slice) workgroups to cover the machine's 256 CUs;
    // 32-column slices from 64 streams on (within 256 registers; at 2048 packed
    // streams the scan took 11.7 ms against 16.5 ms with whole-state workgroups)
    const int streams = a.N * a.H;
    if (streams < 64) err = launch_scan<D, 16, TIn>(a, sa, ws);
    else if (streams < kWideStreams) err = launch_scan<D, 32, TIn>(a, sa, ws);
    else err = launch_scan<D, 64, TIn>(a, sa, ws);
  }
  const hipError_t ferr = ws_release(a, ws);
  return err != hipSuccess ? err : ferr;
}

}  // namespace

template <int D, typename TIn>
int fit_window(const PrefillArgs& a, size_t max_bytes) {
  for (int cg = group_chunks((a.T + kC - 1) / kC); cg >= 1; --cg)
    if (grouped_bytes<D, TIn>(a, cg) <= max_bytes) return cg;
  return 0;
}

int prefill_fit_window(const PrefillArgs& a, size_t max_bytes) {
  if (exact_prefill_path(a)) return exact_prefill_fit_window(a, max_bytes);
  if (a.cu_seqlens != nullptr || a.T <= 0) return 0;
  if (a.dtype_f32) return a.d == 64 ? fit_window<64, float>(a, max_bytes) : 0;
  if (a.d == 128) return fit_window<128, bf16_t>(a, max_bytes);
  return fit_window<64, bf16_t>(a, max_bytes);
}

size_t prefill_workspace_bytes(const PrefillArgs& a) {
  if (exact_prefill_path(a)) return exact_prefill_workspace_bytes(a);
  if (a.dtype_f32) return a.d == 64 ? workspace_bytes<64, float>(a) : 0;
  if (a.d == 128) return workspace_bytes<128, bf16_t>(a);
  return workspace_bytes<64, bf16_t>(a);
}

const char* prefill_schedule(const PrefillArgs& a) {
  if (use_fused(a)) return "fused_prefill_kernel (one workgroup per (sequence, head))";
  if (exact_prefill_path(a)) return exact_prefill_schedule(a);
  if (const int R = fused_segments(a)) {
    static thread_local char buf0[200];
    std::snprintf(buf0, sizeof buf0,
                  "fused_prefill_kernel x 3 + compose_kernel<128> (sequences in %d segments: "
                  "exit states and transitions of %d, composition, outputs of all)",
                  R, R - 1);
    return buf0;
  }
  const bool f32 = a.dtype_f32;
  const int D = a.d;
  const int cg = prefill_cg(a);
  if (cg > 0) {
    const int nchunks = (a.T + kC - 1) / kC;
    const int windows = (nchunks + cg - 1) / cg;
    const int dvs = a.N * a.H < 32 ? 16 : 32;
    static thread_local char buf[160];
    std::snprintf(buf, sizeof buf,
                  "prefill_group_kernel<%d,%d,%s> x %d launches (windows of %d chunks: "
                  "scan of window k-1 beside preparation of window k)",
                  D, dvs, f32 ? "f32" : "bf16", windows + 1, cg);
    return buf;
  }
  const int streams = a.N * a.H;
  const int dvs = streams < 64 ? 16 : streams < kWideStreams ? 32 : 64;
  static thread_local char buf2[160];
  std::snprintf(buf2, sizeof buf2, "%s + state_scan_kernel<%d,%d,%s>",
                (D == 128 && !f32) ? "chunk_prep8_kernel" : (D == 128 ? "chunk_prep_kernel<128,f32>"
                 : f32 ? "chunk_prep_kernel<64,f32>" : "chunk_prep_kernel<64,bf16>"),
                D, dvs, f32 ? "f32" : "bf16");
  return buf2;
}

hipError_t launch_prefill(const PrefillArgs& a) {
  if (a.dtype_f32) {
    if (a.d == 64) return launch_all<64, float>(a);
    return launch_exact_prefill(a);
  }
  if (a.d == 128) {
    if (use_fused(a)) return launch_fused_prefill(a);
    if (const int R = fused_segments(a)) return launch_fused_segmented(a, R);
    return launch_all<128, bf16_t>(a);
  }
  return launch_all<64, bf16_t>(a);
}

}  // namespace kda
