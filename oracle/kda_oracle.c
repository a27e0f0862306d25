/*
 * Plain CPU oracle for Kimi Delta Attention (KDA): the sequential per-token
 * recurrence in IEEE fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * bench's cpu_baseline leg may load this library.  It shares no code, header
 * or constant with the HIP path and must never be used as a fallback for it.
 *
 * What it computes (one independent problem per (sequence n, head h)):
 *
 *   S = S0[n,h]                (dk x dv, rows = key channels; zero if absent)
 *   for each token t of the sequence, in order:
 *       S[i][:] *= exp(g[t,h,i])                    forget, per key channel
 *       u = S^T k[t,h]                              what the memory recalls
 *       S  += beta[t,h] * k[t,h] (v[t,h] - u)^T     delta-rule write
 *       out[t,h] = S^T (scale * q[t,h])             read the updated state
 *   ST[n,h] = S
 *
 * Sources, by page title and section:
 *  - best.xiaohu.ai "Kimi K3 tech report", section "Sequence length: replacing
 *    most attention layers with fixed-size memory": a fixed-size memory state
 *    that is updated as input arrives while old content decays gradually
 *    across channels (per-key-channel decay, constant-size state).
 *  - same page, section "Key advantage: extending to 1M tokens ...": decay
 *    intensity grows with distance (the decay is cumulative over tokens).
 *  - neurohive.io Kimi K3 review, section "Sequence length: hybrid KDA and
 *    Gated MLA attention": a delta rule that forgets old content and writes new
 *    content, with a per-channel retention factor whose log is bounded below
 *    at -5.
 *  - neurohive.io review, section "Training and inference infrastructure":
 *    one fixed-size recurrent state per request (state in -> state out).
 * The pages never print the update equation.  The reading used here is
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = S_t^T (scale q_t):
 * decay first, the delta correction acts on the decayed state, and the output
 * reads the state after the token's own write.
 *
 * Inputs are read in their stored precision (bf16 as raw uint16 bit patterns,
 * fp32, or fp64) and widened exactly to fp64, so input rounding is not counted
 * as error.  Only the (sequence, head) loop is parallel; the token loop is the
 * definition and stays sequential.  Build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F64 = 2 };

/* Widen element i of a buffer stored in the given precision to double. */
static double widen(const void* p, int dtype, int64_t i) {
  if (dtype == ORC_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16; /* bf16 = top half of fp32 */
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  if (dtype == ORC_F32) return (double)((const float*)p)[i];
  return ((const double*)p)[i];
}

int orc_abi_version(void) { return 1; }

/*
 * Run the recurrence for the listed (sequence, head) pairs.
 *
 *  q,k,g : [total_T, H, dk] in `in_dtype`;  v : [total_T, H, dv];  beta : [total_T, H]
 *  seq_start[n], seq_len[n] : token offset and length of sequence n (0 <= n < N)
 *  s0    : [N, H, dk, dv] in `s0_dtype`, or NULL for a zero initial state
 *  pairs : npairs entries of (n, h) as int32 pairs, or NULL for all N*H pairs
 *  out   : if out_mode == 0, [total_T, H, dv] doubles (only listed pairs written);
 *          if out_mode == 1, the listed pairs' outputs packed one after another,
 *          pair p occupying seq_len[n_p] * dv doubles, in list order;
 *          may be NULL (outputs not stored).
 *  sT    : [npairs, dk, dv] doubles in list order (final state per pair), or NULL.
 *  nthreads : OpenMP threads (<= 0 means the runtime default).
 * Returns 0, or a negative value for a bad argument.
 */
int orc_kda_forward(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, int in_dtype, const void* s0, int s0_dtype,
                    const int64_t* seq_start, const int64_t* seq_len, int N, int H,
                    int dk, int dv, double scale, const int32_t* pairs, int npairs,
                    double* out, int out_mode, double* sT, int nthreads) {
  if (!q || !k || !v || !g || !beta || !seq_start || !seq_len) return -1;
  if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -2;
  if (in_dtype < 0 || in_dtype > 2 || s0_dtype < 0 || s0_dtype > 2) return -3;
  const int P = pairs ? npairs : N * H;
  if (P <= 0) return -4;

  /* Offsets of each pair's packed output block (out_mode == 1). */
  int64_t* packed_off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(P + 1));
  if (!packed_off) return -5;
  packed_off[0] = 0;
  for (int p = 0; p < P; ++p) {
    int n = pairs ? pairs[2 * p] : p / H;
    int h = pairs ? pairs[2 * p + 1] : p % H;
    if (n < 0 || n >= N || h < 0 || h >= H) { free(packed_off); return -6; }
    packed_off[p + 1] = packed_off[p] + seq_len[n] * (int64_t)dv;
  }

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < P; ++p) {
    const int n = pairs ? pairs[2 * p] : p / H;
    const int h = pairs ? pairs[2 * p + 1] : p % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* kv = (double*)malloc(sizeof(double) * (size_t)dk * 3);
    double* vv = (double*)malloc(sizeof(double) * (size_t)dv * 3);
    if (!S || !kv || !vv) {
      free(S); free(kv); free(vv);
#pragma omp atomic write
      status = -5;
      continue;
    }
    double* kt = kv;          /* k_t          */
    double* qt = kv + dk;     /* scale * q_t  */
    double* dec = kv + 2 * dk;/* exp(g_t)     */
    double* vt = vv;          /* v_t          */
    double* u = vv + dv;      /* S^T k_t, then the write vector */
    double* ot = vv + 2 * dv; /* S^T (scale q_t) */

    const int64_t s0_base = ((int64_t)n * H + h) * dk * dv;
    for (int64_t e = 0; e < (int64_t)dk * dv; ++e)
      S[e] = s0 ? widen(s0, s0_dtype, s0_base + e) : 0.0;

    for (int64_t t = 0; t < seq_len[n]; ++t) {
      const int64_t tok = seq_start[n] + t;
      const int64_t qk_base = (tok * H + h) * dk;
      const int64_t v_base = (tok * H + h) * dv;
      const double b = widen(beta, in_dtype, tok * H + h);
      for (int i = 0; i < dk; ++i) {
        kt[i] = widen(k, in_dtype, qk_base + i);
        qt[i] = scale * widen(q, in_dtype, qk_base + i);
        dec[i] = exp(widen(g, in_dtype, qk_base + i));
      }
      for (int j = 0; j < dv; ++j) vt[j] = widen(v, in_dtype, v_base + j);

      /* forget: scale row i (key channel i) by exp(g_i) */
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= dec[i];

      /* recall from the decayed state: u = S^T k */
      for (int j = 0; j < dv; ++j) u[j] = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) u[j] += S[(int64_t)i * dv + j] * kt[i];

      /* write: S += k (beta (v - u))^T */
      for (int j = 0; j < dv; ++j) u[j] = b * (vt[j] - u[j]);
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += kt[i] * u[j];

      /* read the updated state: o = S^T (scale q) */
      if (out) {
        double* o = out_mode == 0 ? out + v_base : out + packed_off[p] + t * dv;
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) ot[j] += S[(int64_t)i * dv + j] * qt[i];
        for (int j = 0; j < dv; ++j) o[j] = ot[j];
      }
    }
    if (sT) memcpy(sT + (int64_t)p * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    free(S); free(kv); free(vv);
  }
  free(packed_off);
  return status;
}
