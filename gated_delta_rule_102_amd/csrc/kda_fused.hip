// Fused chunked KDA prefill on gfx950: one workgroup per (sequence, head) walks the
// sequence's 64-token chunks, computes each chunk's operands in LDS and applies
// them to the state held in registers.  Nothing leaves the CU but q, k, v, g, beta
// (read once), the output (written once) and the states.
//
// The token rule (neurohive.io Kimi K3 review, section "Sequence length: hybrid KDA
// and Gated MLA attention": a delta rule that forgets per key channel and writes,
// the log of the retention factor bounded below at -5)
//     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
//     o_t = S_t^T (scale q_t)
// is applied a chunk at a time.  With L the cumulative log-decay inside the chunk
// (per token and key channel, zero before the chunk) and Ln its value at the end:
//     A[t,s] = beta_t sum_c k_tc k_sc e^{L_tc - L_sc}     (s < t)
//     M[t,s] = scale sum_c q_tc k_sc e^{L_tc - L_sc}      (s <= t)
//     Tb = (I + A)^{-1} Diag(beta)
//     Kb = K e^L,  Qb = scale Q e^L,  Kt = K e^{Ln - L},  Lambda = e^{Ln}
// and, from the state S at the chunk start,
//     X = V - Kb S,   Delta = Tb X,   O = Qb S + M Delta,
//     S <- Diag(Lambda) S + Kt^T Delta.
// Unrolling the token rule inside the chunk gives (I + A) Delta = Diag(beta)(V - Kb S),
// so this equals the token-by-token result up to rounding.
//
// The -5 bound is what lets every tile be a plain bf16 matrix-core product.  Over a
// whole chunk e^{-L} reaches e^{320}, so A and M are built from 16-row sub-tiles I
// referenced to the cumulative decay R_I at the end of the sub-tile: the row side
// carries e^{L_t - R_I} in [1, e^80], the column side e^{R_I - L_s} <= 1, both within
// bf16 range.  Off-diagonal pairs (I > J): for J = 0 the decay from the chunk start is
// itself in range (L >= -80 over 16 tokens), so the pairs (I, 0), the diagonal (0, 0)
// included, take Kb and Qb (the state step's operands) as row sides and K e^{-L} as
// the column side; pairs (3, J) take Kt = K e^{Ln - L} = K e^{R_3 - L} as their column
// side; pair (2, 1) scales sub-tile 1's column side by e^{R_2 - R_1} <= 1.
//
// Two roles share the workgroup's 8 wavefronts, one of each on every SIMD (wavefront
// w runs on SIMD w % 4), so that one role's vector-ALU work and the other's
// matrix-core work issue side by side:
//  - Operand wavefronts 0-3 build the operands of chunk c.  Wavefront I owns the
//    chunk's rows 16 I .. +15 (sub-tile I) and all 128 key channels; lane (r, g)
//    holds row r and, in each 32-channel block b, channels 32 b + 8 g .. +7 -- one
//    operand fragment of v_mfma_f32_16x16x32_bf16, loaded with one 16-byte load.
//  - State wavefronts 4-7 apply chunk c - 1 to the state.  Wavefront 4 + j owns value
//    columns 32 j .. +31 of S for all 128 key channels, as two 16-column halves of 8
//    accumulator tiles.  Accumulator row r holds key channel
//        sigma(r) = 32 b + 8 g + 4 h + i   for r = 32 b + 16 h + 4 g + i,
//    so that an accumulator tile pair (2 b, 2 b + 1) read as one operand fragment
//    holds channels 32 b + 8 g .. +7 in order: the state feeds the products with the
//    key-side operands with one conversion to bf16 and no transpose.  Products that
//    contract over the chunk's tokens take Delta and Kt^T with the tokens of a
//    32-token block in the order 4 g + i, 16 + 4 g + i on both sides.
// Every iteration has three barrier windows; iteration c runs
//   A: operand: E2, the decayed operands of chunk c (Kb, Qb, Kt^T to LDS; the row and
//      column sides of the sub-tile products kept in registers);
//      state: chunk c - 1's output and state step (O = Qb S + M Delta, Delta by block
//      forward substitution, S <- Lambda S + Kt^T Delta);
//   B: operand: the decayed sub-tile products (A, M) of chunk c, then the cumulative
//      log-decay of chunk c + 1;  state: X = Diag(beta)(V - Kb S) of chunk c;
//   C: per-channel decay factors of chunk c + 1, all 512 threads.
// The state role starts the diagonal inverses (I + A_II)^{-1} of chunk c, one per
// wavefront, inside window B, each as soon as its block is written (an LDS flag).
// Operands read by the state role one iteration after they were written (Qb, Kt^T,
// Lambda, beta) alternate between two LDS copies by chunk parity; the rest are
// written and read in windows that a barrier separates.

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kD = 128;      // dk = dv
constexpr int kCh = 64;      // chunk
constexpr int kThreadsF = 512;

// LDS regions (bytes).  Fragment-ordered operands are [tile][block][lane][bytes].
namespace fl {
constexpr int KBN = 0;                      // -Kb       [4 t-tiles][4 c-blocks] x 16 B
constexpr int QB = KBN + 16384;             // Qb        [2 parities][4 t-tiles][4 c-blocks] x 16 B
constexpr int KTT = QB + 2 * 16384;         // Kt^T      [2 parities][8 state tiles][2 s-blocks] x 16 B
constexpr int MF = KTT + 2 * 16384;         // M         [4 t-tiles][2 s-blocks] x 16 B
constexpr int AOF = MF + 8192;              // -A_IJ, J < I: [6][64 lanes] x 8 B (16x16x16 A)
constexpr int TDF = AOF + 6 * 512;          // T_II:        [4][64 lanes] x 8 B
constexpr int AII = TDF + 4 * 512;          // beta-scaled A_II^T, accumulator layout [4][64] x 16 B
constexpr int LAM = AII + 4 * 1024;         // Lambda, state row order [2 parities][128] fp32
constexpr int BETA = LAM + 2 * 512;         // [2 parities][64] fp32
constexpr int CS = BETA + 512;              // off-diagonal column sides [4][4 c-blocks][64][16]:
                                            //   0: K e^{-L} of sub-tile 0 (pairs (I, 0)),
                                            //   1: pair (2, 1), 2: pair (3, 1), 3: pair (3, 2)
constexpr int TOT = CS + 4 * 4096;          // sub-tile decay totals [4][128] fp32
constexpr int TOTL = TOT + 4 * 128 * 4;     // the same times log2 e
constexpr int FAC = TOTL + 4 * 128 * 4;     // per (sub-tile, channel) factors [4][3][128]
constexpr int F21 = FAC + 4 * 3 * 128 * 4;  // e^{R_2 - R_1} [128]
constexpr int AIIF = F21 + 128 * 4;         // per sub-tile: 1 + the last chunk whose A_II is in AII [4] int
constexpr int BYTES = AIIF + 16;
constexpr int ORD = CS;                     // sequence order (packed input) [<= 256], start only
static_assert(BYTES <= 160 * 1024, "LDS budget");
}  // namespace fl

struct FusedParams {
  const bf16_t *q, *k, *v, *g, *beta;
  const float* s0;        // [N, H, D, D] or null (zero)
  bf16_t* out;
  float* sT;              // [N, H, D, D] or null
  const int32_t* cu;      // packed sequence offsets [N + 1], or null (fixed length T)
  int N, T, total_T, H;
  float scale;
  // Segmented fixed-length input (segR > 0): sequence n is cut into segR segments of
  // whole chunks, segment r covering chunks floor(r nc / segR) .. floor((r + 1) nc /
  // segR) - 1; the launch covers segments 0 .. segs - 1 of every sequence, workgroup
  // ((n segs + r) H + h).  States are indexed r N + n; with sT_last only the last
  // segment writes its final state, at index n.  s0_eye: the initial state is the
  // identity.  v_on = 0: v reads as zero (with the identity, the run gives the
  // segment's transition); out_on = 0: nothing is written to out.
  int segR = 0, segs = 0;
  int s0_eye = 0, sT_last = 0;
  int v_on = 1, out_on = 1;
};

// The kD x kD identity, the initial state from which a segment's run gives its
// transition.
struct EyeMatrix {
  float v[kD * kD];
  constexpr EyeMatrix() : v() {
    for (int i = 0; i < kD; ++i) v[i * (kD + 1)] = 1.f;
  }
};
__device__ EyeMatrix kEye{};   // global (not constant) memory: the initial state loads stay global loads

// Chunk that starts segment r of a sequence of nc chunks cut into R segments.
__device__ __forceinline__ int seg_chunk(const int r, const int nc, const int R) {
  return static_cast<int>((static_cast<int64_t>(r) * nc) / R);
}

__device__ __forceinline__ void fused_seq(const FusedParams& p, int n, int& tok0, int& len) {
  if (p.segR > 0) {   // n is (sequence, segment) here: n = s segs + r
    const int sq = n / p.segs, r = n % p.segs;
    const int nc = (p.T + kCh - 1) / kCh;
    const int c0 = seg_chunk(r, nc, p.segR), c1 = seg_chunk(r + 1, nc, p.segR);
    tok0 = sq * p.T + c0 * kCh;
    len = min(c1 * kCh, p.T) - c0 * kCh;
  } else if (p.cu == nullptr) {
    tok0 = n * p.T;
    len = p.T;
  } else {
    const int x0 = min(max(p.cu[n], 0), p.total_T);
    const int x1 = min(max(p.cu[n + 1], x0), p.total_T);
    tok0 = x0;
    len = x1 - x0;
  }
}

// Key channel held by state accumulator row r (see the layout notes above).
__device__ __forceinline__ constexpr int sigma(int r) {
  return 32 * (r >> 5) + 8 * ((r >> 2) & 3) + 4 * ((r >> 4) & 1) + (r & 3);
}

// Byte offset of fragment (tile, blk) of an operand with NB blocks per tile, for `lane`.
__device__ __forceinline__ int frag_at(int tile, int blk, int nb, int lane) {
  return ((tile * nb + blk) * 64 + lane) * 16;
}

// Workgroup barrier ordering LDS only: this wavefront's LDS operations complete, then
// s_barrier.  (__syncthreads() also waits for every global load in flight, the next
// chunk's prefetch included.)  The two roles run separate loops that pass the same
// number of these barriers.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8_t to_frag(const float (&x)[8]) {
  bf16x8_t f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = static_cast<__bf16>(x[e]);
  return f;
}

// Accumulator tiles (2 b, 2 b + 1) as one 32-deep operand fragment.
__device__ __forceinline__ bf16x8_t acc_frag(const f32x4_t& lo, const f32x4_t& hi) {
  bf16x8_t f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = static_cast<__bf16>(lo[i]);
    f[4 + i] = static_cast<__bf16>(hi[i]);
  }
  return f;
}

typedef __attribute__((ext_vector_type(4))) short bf16x4_t;   // 16x16x16 operand

// One accumulator tile as a 16-deep operand fragment.
__device__ __forceinline__ bf16x4_t acc_frag4(const f32x4_t& a) {
  return __builtin_bit_cast(bf16x4_t, uint2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])});
}

__device__ __forceinline__ bf16x8_t lds_frag(const char* smem, int off) {
  return *reinterpret_cast<const bf16x8_t*>(smem + off);
}
__device__ __forceinline__ bf16x4_t lds_frag4(const char* smem, int off) {
  return *reinterpret_cast<const bf16x4_t*>(smem + off);
}

__device__ __forceinline__ f32x4_t mma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma16(const bf16x4_t& a, const bf16x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Two 16-deep operands side by side as one 32-deep operand: lane (l16, g) carries
// x's elements 4 g .. +3 then y's.  With both sides of a 16x16x32 product built this
// way the contraction runs over x's 16 and y's 16 terms, so
//     mma(cat(a1, a2), cat(b1, b2), c) = a1 b1 + a2 b2 + c,
// one instruction where two 16x16x16 products take twice as long (on gfx950 a
// 16x16x16 bf16 product occupies the matrix core as long as a 16x16x32 one).
__device__ __forceinline__ bf16x8_t cat(const bf16x4_t& x, const bf16x4_t& y) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Compile-time sub-tile index for the per-sub-tile variants.
template <int N>
struct Ic {
  static constexpr int value = N;
};

// Off-diagonal sub-tile pairs J < I -> 0..5.
__device__ __forceinline__ constexpr int off_id(int I, int J) { return I * (I - 1) / 2 + J; }

// Key-side inputs of one chunk for one operand wavefront as loaded (32 channels of
// one row per lane, four 16-byte fragments each): g and beta, loaded an iteration
// before the decay scan that reads them, and q, k, loaded an iteration before the
// operand phase that reads them.
struct DecayIn {
  i32x4_t g[4];
  uint32_t beta;
};
struct KeyIn {
  i32x4_t q[4], k[4];
};

// Per-channel factors of chunk c for sub-tile m and channel ch (one item; the 512
// items are spread over all threads of the workgroup).
__device__ __forceinline__ void factor_item(const FusedParams& p, char* smem, const int c, const int m,
                                            const int ch) {
  const float* tot = reinterpret_cast<const float*>(smem + fl::TOT);
  float R[4];
  R[0] = tot[ch];
#pragma unroll
  for (int x = 1; x < 4; ++x) R[x] = R[x - 1] + tot[x * kD + ch];
  float* fac = reinterpret_cast<float*>(smem + fl::FAC);
  if (m == 0) {   // sub-tile 0 is referenced to the chunk start: only e^{Ln}
    const float eln = fast_exp2(R[3] * kLog2e);
    fac[2 * kD + ch] = eln;
    // Lambda in state row order: row r holds channel sigma(r)
    const int r = 32 * (ch >> 5) + 16 * ((ch >> 2) & 1) + 4 * ((ch >> 3) & 3) + (ch & 3);
    reinterpret_cast<float*>(smem + fl::LAM)[(c & 1) * kD + r] = eln;
  } else {
    // e^{R_m} as e^{tot_m} e^{R_{m-1}}: each factor alone is in range
    const float em = fast_exp2(tot[m * kD + ch] * kLog2e) * fast_exp2(R[m - 1] * kLog2e);
    fac[(m * 3 + 0) * kD + ch] = -em;                                 // -e^{R_m}
    fac[(m * 3 + 1) * kD + ch] = p.scale * em;                        // scale e^{R_m}
    fac[(m * 3 + 2) * kD + ch] = fast_exp2((R[3] - R[m]) * kLog2e);   // e^{Ln - R_m}
    if (m == 1) reinterpret_cast<float*>(smem + fl::F21)[ch] = fast_exp2((R[2] - R[1]) * kLog2e);
  }
}

// LDS flag handoff inside a barrier window: the writer's LDS stores complete, then it
// publishes `value`; the reader polls until the flag reaches it.  The poll is bounded
// (about 2^20 polls) so that a wavefront always leaves it; the writer never waits on
// the reader, so the flag is set within the window.
__device__ __forceinline__ void flag_set(char* smem, const int off, const int value) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(reinterpret_cast<int*>(smem + off), value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void flag_wait(char* smem, const int off, const int value) {
  for (int n = 0; n < (1 << 20); ++n) {
    const int v = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(reinterpret_cast<int*>(smem + off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (v >= value) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ operand role
// Wavefront I (0..3) of the workgroup, sub-tile I of every chunk.
// OUT = false: the run's output is not wanted (a segment's exit state or transition,
// launched with out_on = 0), so the operand role computes nothing that only the output
// needs: no q loads, Qb or q row sides, no M products.  The state role is the same in
// both forms; without these operands its output products read whatever LDS holds and
// their stores are dropped.
template <bool OUT>
__device__ __forceinline__ void operand_role(const FusedParams& p, char* smem, const int I,
                                             const int h, const int tok0, const int len,
                                             const int nchunks) {
  const int tid = threadIdx.x;   // 0..255 in this role
  // lane-derived values are recomputed every iteration from an opaque copy (see the
  // loop), so the compiler does not hoist address and mask arithmetic out of the loop
  // and keep it in registers across it
  int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  const int H = p.H;
  const uint32_t rs = static_cast<uint32_t>(H) * kD * 2;   // token row stride (bytes)

  // Prefetches are issued every iteration, past the last chunk too (an empty range:
  // every load returns 0 and touches no memory), so that the loop issues the same
  // sequence of loads on every path and the compiler's wait counts stay exact.
  auto rows = [&](const int c, int64_t& base, uint32_t& bytes) {
    const int t0 = tok0 + c * kCh;
    const int nrow = min(kCh, len - c * kCh);
    base = static_cast<int64_t>(t0) * H + h;
    bytes = nrow > 0 ? (nrow - 1) * rs + kD * 2 : 0;   // rows past the end read 0
    return nrow;
  };
  const uint32_t row = (16 * I + l16) * rs;
  auto load_decay = [&](const int c, DecayIn& in) {
    int64_t base;
    uint32_t bytes;
    const int nrow = rows(c, base, bytes);
    const auto rg = make_rsrc(p.g + base * kD, bytes);
#pragma unroll
    for (int b = 0; b < 4; ++b) in.g[b] = buf_ld128(rg, row + (32 * b + 8 * g4) * 2, 0);
    const auto rb = make_rsrc(p.beta + base, nrow > 0 ? (nrow - 1) * H * 2 + 2 : 0);
    in.beta = buf_ld16(rb, (16 * I + l16) * H * 2, 0);
  };
  auto load_keys = [&](const int c, KeyIn& in) {
    int64_t base;
    uint32_t bytes;
    rows(c, base, bytes);
    const auto rq = make_rsrc(p.q + base * kD, bytes);
    const auto rk = make_rsrc(p.k + base * kD, bytes);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      in.k[b] = buf_ld128(rk, row + (32 * b + 8 * g4) * 2, 0);
      if constexpr (OUT) in.q[b] = buf_ld128(rq, row + (32 * b + 8 * g4) * 2, 0);
    }
  };

  // B operands that pick channels 8 (n / 4) + 4 hs + n % 4 of a 32-channel block into
  // column n: the product of a token-major fragment with them lands in accumulator
  // layout with channels as columns, i.e. transposed.
  bf16x8_t sel[2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sel[hs][j] = static_cast<__bf16>(g4 == (l16 >> 2) && j == 4 * hs + (l16 & 3) ? 1.f : 0.f);

  DecayIn dn;
  KeyIn kq;
  float L[4][8];             // inclusive sum of g over the sub-tile's rows up to this one
  float beta_t = 0.f;

  // E1: cumulative log-decay of chunk c from the loaded g, sub-tile totals and beta to
  // LDS.  On the matrix cores: the product of g's fragment with sel[hs] gives, in
  // accumulator layout, g transposed (lane (t, g): tokens 4 g .. +3 of channel
  // 32 b + 8 (l16 / 4) + 4 hs + l16 % 4); read back as a 16-deep A operand that is G^T,
  // and its product with the lower-triangular ones U[s][t] = (s <= t) is L^T, which in
  // accumulator layout puts token l16's channels 32 b + 8 g + 4 hs .. +3 in lane
  // (l16, g) -- the fragment layout.  g is exact in bf16 and the sums are fp32.
  bf16x4_t tri;
#pragma unroll
  for (int i = 0; i < 4; ++i) tri[i] = 4 * g4 + i <= l16 ? 0x3F80 : 0;
  auto e1 = [&](const int c) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bf16x8_t gf = __builtin_bit_cast(bf16x8_t, dn.g[b]);
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const f32x4_t gt = mma(gf, sel[hs], f32x4_t{0.f, 0.f, 0.f, 0.f});
        const f32x4_t lt = mma16(acc_frag4(gt), tri, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) L[b][4 * hs + i] = lt[i];
      }
    }
    beta_t = bf16lo(dn.beta);
    if (l16 == 15) {   // sub-tile totals R_I - R_{I-1}, and times log2 e
      float* tot = reinterpret_cast<float*>(smem + fl::TOT) + I * kD;
      float* totl = reinterpret_cast<float*>(smem + fl::TOTL) + I * kD;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          *reinterpret_cast<float4*>(tot + 32 * b + 8 * g4 + 4 * hh) =
              float4{L[b][4 * hh], L[b][4 * hh + 1], L[b][4 * hh + 2], L[b][4 * hh + 3]};
          *reinterpret_cast<float4*>(totl + 32 * b + 8 * g4 + 4 * hh) =
              float4{L[b][4 * hh] * kLog2e, L[b][4 * hh + 1] * kLog2e, L[b][4 * hh + 2] * kLog2e,
                     L[b][4 * hh + 3] * kLog2e};
        }
    }
    if (g4 == 0) reinterpret_cast<float*>(smem + fl::BETA)[(c & 1) * kCh + 16 * I + l16] = beta_t;
  };


  // E2: decayed operands of chunk c.  Sub-tiles 1-3: rowf = e^{L_t - R_I} >= 1, colf =
  // e^{R_I - L_t} <= 1 (R_I: end of the sub-tile), the sub-tile products' row sides
  // k rowf, q rowf and column side k colf kept in registers, -Kb, Qb, Kt to LDS.
  // Sub-tile 0: ef = e^{L_t} <= 1 and eb = e^{-L_t} <= e^80 (chunk start reference):
  // -Kb and Qb are also its products' row sides and K e^{-L} their column side (LDS too,
  // for the pairs (I, 0) of the other sub-tiles).  One variant per sub-tile (IC = I).
  auto e2_t = [&](auto Ic_, const int c, bf16x8_t (&fKr)[4], bf16x8_t (&fQr)[4], bf16x8_t (&fKc)[4]) {
    constexpr int IC = decltype(Ic_)::value;
    const float* totl = reinterpret_cast<const float*>(smem + fl::TOTL) + IC * kD;
    const float* fac = reinterpret_cast<const float*>(smem + fl::FAC);
    const float* f21 = reinterpret_cast<const float*>(smem + fl::F21);
    const int qb_off = fl::QB + (c & 1) * 16384, kt_off = fl::KTT + (c & 1) * 16384;
    auto frag = [](const uint32_t (&w)[4]) { return __builtin_bit_cast(bf16x8_t, uint4{w[0], w[1], w[2], w[3]}); };
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float4 fo[2];   // e^{R_2 - R_1} (sub-tile 1 only), read ahead of the exponentials
      if (IC == 1) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) fo[hh] = *reinterpret_cast<const float4*>(f21 + 32 * b + 8 * g4 + 4 * hh);
      }
      // results are packed to bf16 pairs as soon as a pair of channels is done, which
      // keeps the fp32 intermediates of only two channels live
      uint32_t pkr[4], pqr[4], pkc[4], pkb[4], pqb[4], pkt[4], p21[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int c0 = 32 * b + 8 * g4 + 4 * hh;
        float tv[4], vK[4], vQ[4], vN[4];
        {
          const float4 fN = *reinterpret_cast<const float4*>(fac + (IC * 3 + 2) * kD + c0);
          vN[0] = fN.x; vN[1] = fN.y; vN[2] = fN.z; vN[3] = fN.w;
        }
        if (IC > 0) {
          const float4 t4 = *reinterpret_cast<const float4*>(totl + c0);
          const float4 fK = *reinterpret_cast<const float4*>(fac + (IC * 3 + 0) * kD + c0);
          const float4 fQ = *reinterpret_cast<const float4*>(fac + (IC * 3 + 1) * kD + c0);
          tv[0] = t4.x; tv[1] = t4.y; tv[2] = t4.z; tv[3] = t4.w;
          vK[0] = fK.x; vK[1] = fK.y; vK[2] = fK.z; vK[3] = fK.w;
          vQ[0] = fQ.x; vQ[1] = fQ.y; vQ[2] = fQ.z; vQ[3] = fQ.w;
        }
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const uint32_t kw = static_cast<uint32_t>(kq.k[b][2 * hh + i2]);
          const uint32_t qw = static_cast<uint32_t>(kq.q[b][2 * hh + i2]);
          const int w = 2 * hh + i2;   // dword of the fragment
          if (IC == 0) {
            float kb[2], qb[2], cs[2], kt[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int i = 2 * i2 + j, e = 4 * hh + i;
              const float kv = j ? bf16hi(kw) : bf16lo(kw);
              const float d = L[b][e] * kLog2e;           // L log2 e <= 0
              const float ef = fast_exp2(d), eb = fast_exp2(-d);
              kb[j] = -(kv * ef);            // -K e^{L}
              if constexpr (OUT) {
                const float qv = j ? bf16hi(qw) : bf16lo(qw);
                qb[j] = (qv * ef) * p.scale;   // scale Q e^{L}
              }
              cs[j] = kv * eb;               // K e^{-L}
              kt[j] = cs[j] * vN[i];         // K e^{Ln - L}
            }
            pkb[w] = pack_bf16x2(kb[0], kb[1]);
            if constexpr (OUT) pqb[w] = pack_bf16x2(qb[0], qb[1]);
            pkc[w] = pack_bf16x2(cs[0], cs[1]);
            pkt[w] = pack_bf16x2(kt[0], kt[1]);
          } else {
            float kr[2], qr[2], kc[2], kb[2], qb[2], kt[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int i = 2 * i2 + j, e = 4 * hh + i;
              const float kv = j ? bf16hi(kw) : bf16lo(kw);
              const float d = __builtin_fmaf(L[b][e], kLog2e, -tv[i]);   // (L - R_I) log2 e >= 0
              const float rowf = fast_exp2(d), colf = fast_exp2(-d);
              kr[j] = kv * rowf;
              if constexpr (OUT) {
                const float qv = j ? bf16hi(qw) : bf16lo(qw);
                qr[j] = qv * rowf;
              }
              kc[j] = kv * colf;
              kb[j] = kr[j] * vK[i];     // -K e^{L}
              if constexpr (OUT) qb[j] = qr[j] * vQ[i];     // scale Q e^{L}
              kt[j] = kc[j] * vN[i];     // K e^{Ln - L}
            }
            pkr[w] = pack_bf16x2(kr[0], kr[1]);
            if constexpr (OUT) pqr[w] = pack_bf16x2(qr[0], qr[1]);
            pkc[w] = pack_bf16x2(kc[0], kc[1]);
            pkb[w] = pack_bf16x2(kb[0], kb[1]);
            if constexpr (OUT) pqb[w] = pack_bf16x2(qb[0], qb[1]);
            pkt[w] = pack_bf16x2(kt[0], kt[1]);
            if (IC == 1) {   // column side of pair (2, 1): K e^{R_2 - L}
              const float f0 = i2 ? fo[hh].z : fo[hh].x, f1 = i2 ? fo[hh].w : fo[hh].y;
              p21[w] = pack_bf16x2(kc[0] * f0, kc[1] * f1);
            }
          }
        }
      }
      fKr[b] = frag(IC == 0 ? pkb : pkr);
      if constexpr (OUT) fQr[b] = frag(IC == 0 ? pqb : pqr);
      fKc[b] = frag(pkc);
      *reinterpret_cast<bf16x8_t*>(smem + fl::KBN + frag_at(IC, b, 4, lane)) = frag(pkb);
      if constexpr (OUT) *reinterpret_cast<bf16x8_t*>(smem + qb_off + frag_at(IC, b, 4, lane)) = frag(pqb);
      // Kt^T: the products with sel[hs] give, in lane (l16, g), tokens 16 I + 4 g .. +3
      // of the channel of state row 16 (2 b + hs) + l16 -- half of that lane's
      // fragment (state tile 2 b + hs, s-block I / 2), elements 4 (I % 2) .. +3
      {
        const bf16x8_t fkt = frag(pkt);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const f32x4_t tr = mma(fkt, sel[hs], f32x4_t{0.f, 0.f, 0.f, 0.f});
          *reinterpret_cast<uint2*>(smem + kt_off + frag_at(2 * b + hs, IC >> 1, 2, lane) + 8 * (IC & 1)) =
              uint2{pack_bf16x2(tr[0], tr[1]), pack_bf16x2(tr[2], tr[3])};
        }
      }
      // column sides for the other sub-tiles' pairs
      if (IC == 0)
        *reinterpret_cast<bf16x8_t*>(smem + fl::CS + 0 * 4096 + frag_at(0, b, 4, lane)) = frag(pkc);
      if (IC == 1) {
        *reinterpret_cast<bf16x8_t*>(smem + fl::CS + 1 * 4096 + frag_at(0, b, 4, lane)) = frag(p21);
        *reinterpret_cast<bf16x8_t*>(smem + fl::CS + 2 * 4096 + frag_at(0, b, 4, lane)) = frag(pkt);
      }
      if (IC == 2)
        *reinterpret_cast<bf16x8_t*>(smem + fl::CS + 3 * 4096 + frag_at(0, b, 4, lane)) = frag(pkt);
    }
  };
  auto e2 = [&](const int c, bf16x8_t (&fKr)[4], bf16x8_t (&fQr)[4], bf16x8_t (&fKc)[4]) {
    switch (I) {
      case 0: e2_t(Ic<0>{}, c, fKr, fQr, fKc); break;
      case 1: e2_t(Ic<1>{}, c, fKr, fQr, fKc); break;
      case 2: e2_t(Ic<2>{}, c, fKr, fQr, fKc); break;
      default: e2_t(Ic<3>{}, c, fKr, fQr, fKc); break;
    }
  };

  // Decayed sub-tile products of chunk c, transposed: C[s, t] = sum_c colside[s, c]
  // rowside[t, c]; lane (t, g) holds s = 16 J + 4 g + i.  Writes M's blocks, -A_IJ
  // (J < I) and the beta-scaled diagonal block A_II (masked to s < t) for its inverse.
  // The ten pairs are spread 3, 2, 2, 3 over the wavefronts: wavefront W takes pairs
  // (PI, PJ)[W] below.  Pairs (I, J >= 1) need the row sides k rowf, q rowf of sub-tile
  // I, which only wavefront I holds; pairs (I, 0) take -Kb and Qb of sub-tile I from
  // LDS (or registers for (0, 0)) and the column side K e^{-L} of sub-tile 0, so any
  // wavefront can run them.  One straight-line variant per wavefront.
  auto products_t = [&](auto Wc, const int c, const bf16x8_t (&fKr)[4], const bf16x8_t (&fQr)[4],
                        const bf16x8_t (&fKc)[4]) {
    constexpr int W = decltype(Wc)::value;
    constexpr int NP = (W == 0 || W == 3) ? 3 : 2;
    constexpr int PI[4][3] = {{0, 2, 3}, {1, 1, 0}, {2, 2, 0}, {3, 3, 3}};
    constexpr int PJ[4][3] = {{0, 0, 0}, {1, 0, 0}, {2, 1, 0}, {3, 1, 2}};
    const int qb_off = fl::QB + (c & 1) * 16384;
    const float* betas = reinterpret_cast<const float*>(smem + fl::BETA) + (c & 1) * kCh;
    f32x4_t pa[NP], pm[NP];
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      pa[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pm[x] = pa[x];
    }
    // The diagonal block first (pair x = 0 on every wavefront; its row and column
    // sides are the wavefront's own registers): A_II goes to the state role's inverse
    // while the other products run.  For (0, 0) the row side is -Kb, so A's sign flips.
    {
      constexpr int I = PI[W][0];
#pragma unroll
      for (int b = 0; b < 4; ++b) pa[0] = mma(fKc[b], fKr[b], pa[0]);
      const float fa_ = I == 0 ? -beta_t : beta_t;
      f32x4_t av;
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = 4 * g4 + i < l16 ? fa_ * pa[0][i] : 0.f;
      *reinterpret_cast<f32x4_t*>(smem + fl::AII + I * 1024 + lane * 16) = av;
      flag_set(smem, fl::AIIF + 4 * I, c + 1);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int x = 0; x < NP; ++x) {
        const int I = PI[W][x], J = PJ[W][x];
        // row sides: registers, except the pairs (I >= 1, 0), which take -Kb and Qb
        const bool rows_lds = J == 0 && I > 0;
        const bf16x8_t rk = rows_lds ? lds_frag(smem, fl::KBN + frag_at(I, b, 4, lane)) : fKr[b];
        bf16x8_t rq;
        if constexpr (OUT) rq = rows_lds ? lds_frag(smem, qb_off + frag_at(I, b, 4, lane)) : fQr[b];
        // column side: the own sub-tile's for the diagonal and, on wavefront 0, for
        // (I, 0); otherwise the region written by the column's owner
        const int cs_id = J == 0 ? 0 : (I == 2 ? 1 : J + 1);   // (2,1) -> 1, (3,1) -> 2, (3,2) -> 3
        const bool cols_reg = J == I || (J == 0 && W == 0);
        const bf16x8_t cs = cols_reg ? fKc[b] : lds_frag(smem, fl::CS + cs_id * 4096 + frag_at(0, b, 4, lane));
        if (x > 0) pa[x] = mma(cs, rk, pa[x]);
        if constexpr (OUT) pm[x] = mma(cs, rq, pm[x]);
      }
    }
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int I = PI[W][x], J = PJ[W][x];
      const float bt = I == W ? beta_t : betas[16 * I + l16];
      // J = 0: the row sides are -Kb (A's sign flips) and Qb (scale included)
      const float fa_ = J == 0 ? -bt : bt, fm_ = J == 0 ? 1.f : p.scale;
      // M[t][s]: fragment (t-tile I, s-block J/2), elements 4 (J%2) .. +3; the
      // diagonal pair's masked to s <= t
      if constexpr (OUT) {
        float mv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mv[i] = fm_ * pm[x][i];
          if (J == I) mv[i] = 4 * g4 + i <= l16 ? mv[i] : 0.f;
        }
        *reinterpret_cast<uint2*>(smem + fl::MF + frag_at(I, J >> 1, 2, lane) + 8 * (J & 1)) =
            uint2{pack_bf16x2(mv[0], mv[1]), pack_bf16x2(mv[2], mv[3])};
      }
      if (J < I) {   // -A_IJ as a 16x16x16 A operand: lane (t, g) holds columns 4 g .. +3
        float av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = fa_ * pa[x][i];
        *reinterpret_cast<uint2*>(smem + fl::AOF + off_id(I, J) * 512 + lane * 8) =
            uint2{pack_bf16x2(-av[0], -av[1]), pack_bf16x2(-av[2], -av[3])};
      }
    }
  };
  auto products = [&](const int c, const bf16x8_t (&fKr)[4], const bf16x8_t (&fQr)[4], const bf16x8_t (&fKc)[4]) {
    switch (I) {
      case 0: products_t(Ic<0>{}, c, fKr, fQr, fKc); break;
      case 1: products_t(Ic<1>{}, c, fKr, fQr, fKc); break;
      case 2: products_t(Ic<2>{}, c, fKr, fQr, fKc); break;
      default: products_t(Ic<3>{}, c, fKr, fQr, fKc); break;
    }
  };

  // prologue: chunk 0's decay and factors
  load_keys(0, kq);
  load_decay(0, dn);
  if (nchunks > 0) e1(0);
  load_decay(1, dn);
  lds_barrier();
  if (nchunks > 0) factor_item(p, smem, 0, tid >> 7, tid & (kD - 1));   // sub-tiles 0, 1
  lds_barrier();

  for (int c = 0; c <= nchunks; ++c) {
    asm volatile("" : "+v"(lane));
    l16 = lane & 15;
    g4 = lane >> 4;
    bf16x8_t fKr[4], fQr[4], fKc[4];
    if (c < nchunks) e2(c, fKr, fQr, fKc);
    load_keys(c + 1, kq);
    lds_barrier();                                                          // A
    if (c < nchunks) products(c, fKr, fQr, fKc);
    if (c + 1 < nchunks) e1(c + 1);
    load_decay(c + 2, dn);
    lds_barrier();                                                          // B
    if (c + 1 < nchunks) factor_item(p, smem, c + 1, tid >> 7, tid & (kD - 1));   // sub-tiles 0, 1
    lds_barrier();                                                          // C
  }
}

// ------------------------------------------------------------------ state role
// Wavefront 4 + j, value columns 32 j .. +31.
__device__ __forceinline__ void state_role(const FusedParams& p, char* smem, const int j,
                                           const int s0_idx, const int sT_idx, const int h,
                                           const int tok0, const int len, const int nchunks) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const int H = p.H;
  const uint32_t rs = static_cast<uint32_t>(H) * kD * 2;   // token row stride (bytes)
  // all ones, or zero when v reads as zero / nothing is written to out (buffer ranges)
  const uint32_t v_mask = p.v_on ? ~0u : 0u, out_mask = p.out_on ? ~0u : 0u;
  const int col0 = 32 * j;

  f32x4_t S[2][8];
  {
    const float* s0 = p.s0_eye ? kEye.v
                      : p.s0 ? p.s0 + (static_cast<int64_t>(s0_idx) * H + h) * kD * kD : nullptr;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[u][ct][i] = s0 ? s0[sigma(16 * ct + 4 * g4 + i) * kD + col0 + 16 * u + l16] : 0.f;
  }

  // B operand of the 16 x 16 identity for 16x16x16 products (lane: column l16, rows
  // 4 g .. +3)
  bf16x4_t eye;
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = 4 * g4 + i == l16 ? 0x3F80 : 0;

  // v of chunk c for this wavefront's value columns: lane (t, g) loads token 16 tt + t,
  // columns col0 + 16 u + 4 g .. +3 (rows past the end read 0)
  i32x2_t vin[2][4];
  // v loads and output stores are issued every iteration (empty ranges outside the
  // sequence), for the same reason as the operand role's prefetches.
  auto load_v = [&](const int c) {
    const int t0 = tok0 + c * kCh;
    const int nrow = min(kCh, len - c * kCh);
    const auto rv = make_rsrc(p.v + (static_cast<int64_t>(t0) * H + h) * kD,
                              (nrow > 0 ? (nrow - 1) * rs + kD * 2 : 0) & v_mask);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        vin[u][tt] = buf_ld64(rv, (16 * tt + l16) * rs + (col0 + 16 * u + 4 * g4) * 2, 0);
  };

  f32x4_t Y[2][4];      // Diag(beta)(V - Kb S) of the chunk being applied
  bf16x8_t Sb[2][4];    // its starting state as bf16 operand fragments

  // X of chunk c: Y = Diag(beta) (V - Kb S) (the stored -Kb makes the product an
  // addition).  V arrives row-major (lane: token l16, value columns 4 g .. +3) and
  // enters the accumulator layout as the product V I_16, exact in fp32; that product
  // (the same 16 x 16 accumulator layout) is the accumulator the -Kb S products add to.
  auto x_step = [&](const int c) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int b = 0; b < 4; ++b) Sb[u][b] = acc_frag(S[u][2 * b], S[u][2 * b + 1]);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        Y[u][tt] = mma16(__builtin_bit_cast(bf16x4_t, vin[u][tt]), eye, f32x4_t{0.f, 0.f, 0.f, 0.f});
    bf16x8_t F[2][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) F[0][tt] = lds_frag(smem, fl::KBN + frag_at(tt, 0, 4, lane));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < 3) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) F[(b + 1) & 1][tt] = lds_frag(smem, fl::KBN + frag_at(tt, b + 1, 4, lane));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) Y[u][tt] = mma(F[b & 1][tt], Sb[u][b], Y[u][tt]);
    }
    const float* betas = reinterpret_cast<const float*>(smem + fl::BETA) + (c & 1) * kCh;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const float4 b4 = *reinterpret_cast<const float4*>(betas + 16 * tt + 4 * g4);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        Y[u][tt][0] *= b4.x;
        Y[u][tt][1] *= b4.y;
        Y[u][tt][2] *= b4.z;
        Y[u][tt][3] *= b4.w;
      }
    }
  };

  // T_II = (I + A_II)^{-1} of chunk c's sub-tile j, written as the A operand of the
  // substitution.  Computed as T^T = (I + B)^{-1} with B = A_II^T, which is strictly
  // lower (B^16 = 0), as (I - B)(I + B^2)(I + B^4)(I + B^8).  This lane holds B in
  // accumulator layout C(B) (rows 4 g + i, column l16).  A 16x16x16 product takes
  // C(X^T) as its A operand and C(Y) as its B operand and returns C(X Y), so the
  // powers are carried in both orientations and nothing is transposed through memory
  // (the first transpose is a product with I).  Each operand is split into bf16 high
  // and low parts, and a product is three matrix-core products (high x high, high x
  // low, low x high): about 16 bits, far finer than the bf16 the inverse is rounded to.
  auto inverse = [&]() {
    const f32x4_t av = *reinterpret_cast<const f32x4_t*>(smem + fl::AII + j * 1024 + lane * 16);
    struct Split {
      bf16x4_t h, l;
    };
    auto split = [](const f32x4_t& x) {
      Split sp;
      sp.h = acc_frag4(x);
      f32x4_t r;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = x[i] - __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(sp.h[i])) << 16);
      sp.l = acc_frag4(r);
      return sp;
    };
    auto mm = [](const Split& xt, const Split& y) {   // C(X Y) from C(X^T), C(Y)
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      return mma16(xt.l, y.h, mma16(xt.h, y.l, mma16(xt.h, y.h, z)));
    };
    const Split sB = split(av);
    const f32x4_t bt = mma16(sB.l, eye, mma16(sB.h, eye, f32x4_t{0.f, 0.f, 0.f, 0.f}));   // C(B^T)
    const Split sBt = split(bt);
    const f32x4_t p1 = mm(sBt, sB), p1t = mm(sB, sBt);           // B^2 and its transpose
    const Split s1 = split(p1), s1t = split(p1t);
    const f32x4_t p2 = mm(s1t, s1), p2t = mm(s1, s1t);           // B^4
    const f32x4_t b3 = mm(sBt, s1), b3t = mm(s1, sBt);           // B^3
    const Split s2 = split(p2), s2t = split(p2t);
    const f32x4_t p3 = mm(s2t, s2);                               // B^8
    f32x4_t t1, t1t;                                              // I - B + B^2 - B^3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = 4 * g4 + i == l16 ? 1.f : 0.f;
      t1[i] = d - av[i] + p1[i] - b3[i];
      t1t[i] = d - bt[i] + p1t[i] - b3t[i];
    }
    const Split sT1t = split(t1t);
    f32x4_t t2 = mm(sT1t, s2), t2t = mm(s2, sT1t);               // T1 (I + B^4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t2[i] += t1[i];
      t2t[i] += t1t[i];
    }
    f32x4_t t3 = mm(split(t2t), split(p3));                       // T2 (I + B^8)
#pragma unroll
    for (int i = 0; i < 4; ++i) t3[i] += t2[i];
    // lane (l16, g) holds T^T[4 g + i][l16] = T[l16][4 g + i]: the A operand
    *reinterpret_cast<uint2*>(smem + fl::TDF + j * 512 + lane * 8) =
        uint2{pack_bf16x2(t3[0], t3[1]), pack_bf16x2(t3[2], t3[3])};
  };

  // Output and state step of chunk cs, whose operands are in LDS; Y holds its X, S and
  // Sb its starting state.  With cs < 0 only the (empty) stores are issued.
  auto apply = [&](const int cs) {
    const bool act = cs >= 0;
    // O^T = S^T Qb^T + Delta^T M^T: lane (t, g) holds value columns 4 g .. +3 of token t
    f32x4_t o[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) o[u][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t Db[2][2];
    const int qb_off = fl::QB + (cs & 1) * 16384, kt_off = fl::KTT + (cs & 1) * 16384;
    if (act) {
      bf16x8_t F[2][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) F[0][tt] = lds_frag(smem, qb_off + frag_at(tt, 0, 4, lane));
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b < 3) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) F[(b + 1) & 1][tt] = lds_frag(smem, qb_off + frag_at(tt, b + 1, 4, lane));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) o[u][tt] = mma(Sb[u][b], F[b & 1][tt], o[u][tt]);
      }
      // Delta_i = T_ii (Y_i - sum_{m<i} A_im Delta_m), both column halves interleaved
      bf16x4_t fa[6], ft[4];
#pragma unroll
      for (int x = 0; x < 6; ++x) fa[x] = lds_frag4(smem, fl::AOF + x * 512 + lane * 8);
#pragma unroll
      for (int x = 0; x < 4; ++x) ft[x] = lds_frag4(smem, fl::TDF + x * 512 + lane * 8);
      bf16x4_t Dq[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f32x4_t w = Y[u][i];
          if (i >= 2)   // A_i0 Delta_0 + A_i1 Delta_1 in one 32-deep product
            w = mma(cat(fa[off_id(i, 0)], fa[off_id(i, 1)]), cat(Dq[u][0], Dq[u][1]), w);
          else if (i == 1)
            w = mma16(fa[off_id(1, 0)], Dq[u][0], w);
          if (i == 3) w = mma16(fa[off_id(3, 2)], Dq[u][2], w);
          Dq[u][i] = acc_frag4(mma16(ft[i], acc_frag4(w), f32x4_t{0.f, 0.f, 0.f, 0.f}));
        }
      }
      // Delta as 32-deep fragments: tiles (2 b, 2 b + 1) side by side
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          Db[u][b] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(Dq[u][2 * b], Dq[u][2 * b + 1], 0, 1, 2, 3, 4, 5, 6, 7));
      // + Delta^T M^T: M fragments (tt, 0) for every tt, (2, 1) and (3, 1)
      {
        bf16x8_t M0[4], M1[2];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) M0[tt] = lds_frag(smem, fl::MF + frag_at(tt, 0, 2, lane));
        M1[0] = lds_frag(smem, fl::MF + frag_at(2, 1, 2, lane));
        M1[1] = lds_frag(smem, fl::MF + frag_at(3, 1, 2, lane));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) o[u][tt] = mma(Db[u][0], M0[tt], o[u][tt]);
          o[u][2] = mma(Db[u][1], M1[0], o[u][2]);
          o[u][3] = mma(Db[u][1], M1[1], o[u][3]);
        }
      }
    }
    // output rows of chunk cs: plain stores, so that the cache joins the wavefronts'
    // pieces of a row into whole lines
    {
      const int t0 = tok0 + cs * kCh;
      const int nrow = act ? min(kCh, len - cs * kCh) : 0;
      const auto ro = make_rsrc(p.out + (static_cast<int64_t>(act ? t0 : tok0) * H + h) * kD,
                                (nrow > 0 ? (nrow - 1) * rs + kD * 2 : 0) & out_mask);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          buf_st64(i32x2_t{static_cast<int>(pack_bf16x2(o[u][tt][0], o[u][tt][1])),
                           static_cast<int>(pack_bf16x2(o[u][tt][2], o[u][tt][3]))},
                   ro, (16 * tt + l16) * rs + (col0 + 16 * u + 4 * g4) * 2, 0);
    }
    if (!act) return;
    // S <- Diag(Lambda) S + Kt^T Delta, Kt fragments one accumulator tile ahead
    const float* lam = reinterpret_cast<const float*>(smem + fl::LAM) + (cs & 1) * kD;
    bf16x8_t K2[2][2];
    K2[0][0] = lds_frag(smem, kt_off + frag_at(0, 0, 2, lane));
    K2[0][1] = lds_frag(smem, kt_off + frag_at(0, 1, 2, lane));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      if (ct < 7) {
        K2[(ct + 1) & 1][0] = lds_frag(smem, kt_off + frag_at(ct + 1, 0, 2, lane));
        K2[(ct + 1) & 1][1] = lds_frag(smem, kt_off + frag_at(ct + 1, 1, 2, lane));
      }
      const float4 l4 = *reinterpret_cast<const float4*>(lam + 16 * ct + 4 * g4);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4_t acc = {S[u][ct][0] * l4.x, S[u][ct][1] * l4.y, S[u][ct][2] * l4.z, S[u][ct][3] * l4.w};
        acc = mma(K2[ct & 1][0], Db[u][0], acc);
        S[u][ct] = mma(K2[ct & 1][1], Db[u][1], acc);
      }
    }
  };

  // The state role's work is a chain of dependent matrix-core products; the operand
  // role on the same SIMD streams independent vector-ALU work.  Issuing the state
  // role's instructions first whenever they are ready keeps its chain moving and lets
  // the operand role fill the gaps.
  __builtin_amdgcn_s_setprio(3);
  load_v(0);
  lds_barrier();
  if (nchunks > 0)   // chunk 0's factors of sub-tiles 2, 3
    factor_item(p, smem, 0, 2 + ((threadIdx.x - 256) >> 7), threadIdx.x & (kD - 1));
  lds_barrier();
  for (int c = 0; c <= nchunks; ++c) {
    apply(c - 1);
    lds_barrier();                                                          // A
    if (c < nchunks) x_step(c);
    load_v(c + 1);
    // this chunk's inverse as soon as its diagonal block is written
    if (c < nchunks) {
      flag_wait(smem, fl::AIIF + 4 * j, c + 1);
      // it shares the window with the operand role's products and decay scan: no
      // precedence over them
      __builtin_amdgcn_s_setprio(0);
      inverse();
      __builtin_amdgcn_s_setprio(3);
    }
    lds_barrier();                                                          // B
    if (c + 1 < nchunks)   // factors of sub-tiles 2, 3
      factor_item(p, smem, c + 1, 2 + ((threadIdx.x - 256) >> 7), threadIdx.x & (kD - 1));
    lds_barrier();                                                          // C
  }

  if (p.sT != nullptr && sT_idx >= 0) {
    float* dst = p.sT + (static_cast<int64_t>(sT_idx) * H + h) * kD * kD;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[sigma(16 * ct + 4 * g4 + i) * kD + col0 + 16 * u + l16] = S[u][ct][i];
  }
}

template <bool OUT>
__global__ __launch_bounds__(kThreadsF, 1) void fused_prefill_kernel(FusedParams p) {
  __shared__ __attribute__((aligned(16))) char smem[fl::BYTES];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H;

  // ---------------------------------------------------------------- which sequence
  const int rank = blockIdx.x / H, h = blockIdx.x % H;
  int n = rank;
  if (p.cu != nullptr && p.N <= 256) {   // longest sequence first
    int* ord = reinterpret_cast<int*>(smem + fl::ORD);
    int mylen = 0;
    if (tid < p.N) {
      int a, l;
      fused_seq(p, tid, a, l);
      mylen = l;
      ord[tid] = l;
    }
    __syncthreads();
    int rk = 0;
    if (tid < p.N)
      for (int m = 0; m < p.N; ++m) {
        const int lm = ord[m];
        rk += (lm > mylen) || (lm == mylen && m < tid);
      }
    __syncthreads();
    if (tid < p.N) ord[rk] = tid;
    __syncthreads();
    n = __builtin_amdgcn_readfirstlane(ord[rank]);   // uniform: keeps addresses scalar
    __syncthreads();
  }
  int tok0, len;
  fused_seq(p, n, tok0, len);
  const int nchunks = (len + kCh - 1) / kCh;

  if (tid < 4) reinterpret_cast<int*>(smem + fl::AIIF)[tid] = 0;
  // M is lower triangular: the upper halves of fragments (0, 0) and (2, 1) are read as
  // zeros and nothing else writes them
  for (int e = tid; e < 8192 / 16; e += kThreadsF)
    *reinterpret_cast<i32x4_t*>(smem + fl::MF + e * 16) = i32x4_t{0, 0, 0, 0};

  if (wave < 4) {
    operand_role<OUT>(p, smem, wave, h, tok0, len, nchunks);
  } else {
    int s0_idx = n, sT_idx = n;
    if (p.segR > 0) {   // n = s segs + r; states indexed r N + s
      const int sq = n / p.segs, r = n % p.segs;
      s0_idx = r * p.N + sq;
      sT_idx = p.sT_last ? (r == p.segR - 1 ? sq : -1) : r * p.N + sq;
    }
    state_role(p, smem, wave - 4, s0_idx, sT_idx, h, tok0, len, nchunks);
  }
}

}  // namespace

bool fused_prefill_supported(const PrefillArgs& a) {
  return !a.dtype_f32 && a.d == kD && !a.prologue && a.snapshots == nullptr;
}

hipError_t launch_fused_prefill(const PrefillArgs& a) {
  FusedParams fp{static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                 static_cast<const bf16_t*>(a.v), static_cast<const bf16_t*>(a.g),
                 static_cast<const bf16_t*>(a.beta), a.initial_state, static_cast<bf16_t*>(a.out),
                 a.final_state, a.cu_seqlens, a.N, a.T, a.total_T, a.H, a.scale};
  hipLaunchKernelGGL(fused_prefill_kernel<true>, dim3(static_cast<unsigned>(a.N) * a.H), dim3(kThreadsF), 0,
                     a.stream, fp);
  return hipGetLastError();
}

bool fused_transition_supported(const TransitionArgs& a) {
  return !a.dtype_f32 && a.d == kD && static_cast<int64_t>(a.B) * a.H >= 256;
}

// A segment's transition with the fused kernel: the run from the identity with v read
// as zero, its exit state written to `transition`; q and v are not read (their
// pointers only stand in for valid addresses), nothing is written but the state.
hipError_t launch_fused_transition(const TransitionArgs& a) {
  const bf16_t* k = static_cast<const bf16_t*>(a.k);
  FusedParams fp{k, k, k, static_cast<const bf16_t*>(a.g), static_cast<const bf16_t*>(a.beta), nullptr,
                 reinterpret_cast<bf16_t*>(a.transition), a.transition, nullptr, a.B, a.T, a.B * a.T, a.H,
                 1.f};
  fp.s0_eye = 1;
  fp.v_on = 0;
  fp.out_on = 0;
  hipLaunchKernelGGL(fused_prefill_kernel<false>, dim3(static_cast<unsigned>(a.B) * a.H), dim3(kThreadsF), 0,
                     a.stream, fp);
  return hipGetLastError();
}

size_t fused_segmented_bytes(const PrefillArgs& a, int R) {
  // exit states and transitions of segments 0 .. R-2, entry states of all R segments
  return static_cast<size_t>(3 * R - 2) * a.N * a.H * kD * kD * sizeof(float);
}

// Few long sequences: every sequence cut into R segments so that N H R workgroups fill
// the machine.  A segment maps its entry state affinely to its exit state, S_exit =
// P S_entry + X (the token rule is linear in (S, v)); X is its exit state from a zero
// entry and P the exit state from the identity with v = 0.  Four launches: X and P
// of segments 0 .. R-2, their composition into every segment's entry state, then the
// output of every segment from its entry state (the last one also writes the final
// state).
hipError_t launch_fused_segmented(const PrefillArgs& a, int R) {
  char* ws = nullptr;
  hipError_t err = ws_acquire(a.workspace, a.workspace_bytes, fused_segmented_bytes(a, R), a.stream, &ws);
  if (err != hipSuccess) return err;
  const size_t per = static_cast<size_t>(a.N) * a.H * kD * kD;
  float* exits = reinterpret_cast<float*>(ws);
  float* trans = exits + (R - 1) * per;
  float* entry = trans + (R - 1) * per;
  // v and out stay valid pointers in every launch; v_on / out_on = 0 make their
  // buffer ranges empty (loads return zero, stores are dropped)
  auto params = [&](int v_on, const float* s0, int out_on, float* sT, int segs, int eye, int last) {
    FusedParams fp{static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                   static_cast<const bf16_t*>(a.v), static_cast<const bf16_t*>(a.g),
                   static_cast<const bf16_t*>(a.beta), s0, static_cast<bf16_t*>(a.out), sT,
                   nullptr, a.N, a.T, a.N * a.T, a.H, a.scale};
    fp.segR = R;
    fp.segs = segs;
    fp.s0_eye = eye;
    fp.sT_last = last;
    fp.v_on = v_on;
    fp.out_on = out_on;
    return fp;
  };
  const unsigned g1 = static_cast<unsigned>(a.N) * (R - 1) * a.H;
  const FusedParams px = params(1, nullptr, 0, exits, R - 1, 0, 0);
  KDA_TRY_LAUNCH(err, fused_prefill_kernel<false>, dim3(g1), dim3(kThreadsF), 0, a.stream, px);
  const FusedParams pp = params(0, nullptr, 0, trans, R - 1, 1, 0);
  KDA_TRY_LAUNCH(err, fused_prefill_kernel<false>, dim3(g1), dim3(kThreadsF), 0, a.stream, pp);
  if (err == hipSuccess)
    err = launch_compose(ComposeArgs{trans, exits, a.initial_state, entry, R - 1, a.N, a.H, kD, a.stream});
  const FusedParams po = params(1, entry, 1, a.final_state, R, 0, 1);
  KDA_TRY_LAUNCH(err, fused_prefill_kernel<true>, dim3(static_cast<unsigned>(a.N) * R * a.H), dim3(kThreadsF), 0,
                 a.stream, po);
  const hipError_t ferr = ws_release(a.workspace, ws, a.stream);
  return err != hipSuccess ? err : ferr;
}

}  // namespace kda
