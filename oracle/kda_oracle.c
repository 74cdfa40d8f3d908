/*
 * KDA forward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64, token-by-token CPU evaluation of the Kimi Delta
 * Attention (KDA) forward recurrence.  Only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load this library; the
 * product path (the HIP library) never does, and the two share no code.
 *
 * Sources (the web pages this project is built from):
 *  - "FlashKDA Delta Attention" skill page (atskills.one, aradotso),
 *    "Tensor shapes and dtypes" table and "Constraints": tensor layouts,
 *    the [.., V, K] orientation of the recurrent state, beta given as logits
 *    with the sigmoid applied inside, int64 cu_seqlens for packed sequences,
 *    initial/final state per sequence.
 *  - "fla-kda" skill listing (skills.rest) and the fla-kda SKILL.md embedded
 *    in the flash-linear-attention skills page (yakaai.com), section
 *    "Gate contracts": the two in-kernel gate activations
 *      softplus form : a = -exp(A_log) * softplus(g + dt_bias)
 *      safe form     : a = lower_bound * sigmoid(exp(A_log) * (g + dt_bias))
 *    and the caller-supplied log-space decay when the gate is not applied in
 *    the kernel.
 *
 * The pages never print the recurrence itself.  The reading used here (the
 * standard gated delta rule with a per-key-channel diagonal decay, state
 * S in R^{V x K}) is, per token t:
 *      S <- S * Diag(exp(a_t))              decay, column c scaled by e^{a_c}
 *      r  = S k_t                           read
 *      S <- S + beta_t (v_t - r) k_t^T      delta-rule write
 *      o_t = scale * S q_t                  read after the write
 * with q, k L2-normalised (eps = 1e-6 inside the square root) when the
 * normalisation flag is set, and beta_t = sigmoid(beta logit) unless the
 * caller passes probabilities.
 *
 * Parity pins: the functions here are checked against closed forms,
 * invariants, library routines and an independent chunked formulation by the
 * CPU tests (tests/test_oracle.py); nothing in them is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_GATE_SOFTPLUS = 0, ORC_GATE_SAFE_SIGMOID = 1, ORC_GATE_PREGATED = 2 };
enum { ORC_FLAG_QK_L2NORM = 1, ORC_FLAG_BETA_IS_PROB = 2 };

#define ORC_L2_EPS 1e-6

/* bf16 bit pattern -> exact double (bf16 is the top half of an IEEE binary32). */
static double bf16_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* softplus(x) = log(1 + e^x), evaluated without overflow. */
static double orc_softplus(double x) {
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

static double orc_sigmoid(double x) {
  return 1.0 / (1.0 + exp(-x));
}

/* Gate activation for one element: x = g + dt_bias (already summed). */
static double orc_gate(int mode, double x, double A_log, double lower_bound) {
  if (mode == ORC_GATE_SOFTPLUS) return -exp(A_log) * orc_softplus(x);
  if (mode == ORC_GATE_SAFE_SIGMOID) return lower_bound * orc_sigmoid(exp(A_log) * x);
  return x; /* pre-gated: the caller passes the log-decay itself */
}

/* Exported for the tests: the activation on n elements. */
void kda_oracle_gate(int mode, int n, const double* x, double A_log, double lower_bound,
                     double* a_out) {
  for (int i = 0; i < n; ++i) a_out[i] = orc_gate(mode, x[i], A_log, lower_bound);
}

/* Exported for the tests: y = x / sqrt(sum x^2 + eps). */
void kda_oracle_l2norm(int n, const double* x, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss + ORC_L2_EPS);
  for (int i = 0; i < n; ++i) y[i] = x[i] * inv;
}

/*
 * Full forward.
 *   q, k  : [B, T, Hqk, K] bf16 bits          v    : [B, T, Hv, V] bf16 bits
 *   g     : [B, T, Hv, K]  bf16 bits          beta : [B, T, Hv]    bf16 bits
 *   A_log : [Hv] float   (unused in pre-gated mode)
 *   dt_bias : [Hv, K] float, or NULL for zero bias
 *   cu_seqlens : [N+1] int64 host array, or NULL (then N == B and sequence n
 *                is batch row n, length T).  With cu_seqlens, B must be 1.
 *   h0    : [N, Hv, V, K] double or NULL (zero initial state)
 *   hT    : [N, Hv, V, K] double or NULL (final state not returned)
 *   out   : [B, T, Hv, V] double or NULL
 * Returns 0, or -1 on an argument error.  Work is split over (sequence,
 * v-head) pairs; nthreads <= 0 uses the OpenMP default.
 */
int kda_oracle_fwd(int B, int T, int Hqk, int Hv, int K, int V, int N,
                   const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* g, const uint16_t* beta,
                   const float* A_log, const float* dt_bias, const int64_t* cu_seqlens,
                   double scale, double lower_bound, int gate_mode, int flags,
                   const double* h0, double* hT, double* out, int nthreads) {
  if (B <= 0 || T < 0 || Hqk <= 0 || Hv <= 0 || K <= 0 || V <= 0) return -1;
  if (Hv % Hqk != 0) return -1;
  if (cu_seqlens) {
    if (B != 1 || N <= 0) return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
    for (int n = 0; n < N; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  } else if (N != B) {
    return -1;
  }
  const int G = Hv / Hqk;
  const long long npairs = (long long)N * Hv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;

#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)V * K);
    double* a = (double*)malloc(sizeof(double) * (size_t)K);
    double* qn = (double*)malloc(sizeof(double) * (size_t)K);
    double* kn = (double*)malloc(sizeof(double) * (size_t)K);
    double* vv = (double*)malloc(sizeof(double) * (size_t)V);
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    if (!S || !a || !qn || !kn || !vv || !r) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long long p = 0; p < npairs; ++p) {
        const int n = (int)(p / Hv), h = (int)(p % Hv), hq = h / G;
        long long bos, eos;
        int b;
        if (cu_seqlens) { b = 0; bos = cu_seqlens[n]; eos = cu_seqlens[n + 1]; }
        else            { b = n; bos = 0; eos = T; }

        /* 1. initial state */
        if (h0) memcpy(S, h0 + ((size_t)n * Hv + h) * V * K, sizeof(double) * (size_t)V * K);
        else    memset(S, 0, sizeof(double) * (size_t)V * K);

        for (long long t = bos; t < eos; ++t) {
          const size_t row = (size_t)b * T + (size_t)t;
          const uint16_t* qt = q + (row * Hqk + hq) * K;
          const uint16_t* kt = k + (row * Hqk + hq) * K;
          const uint16_t* gt = g + (row * Hv + h) * K;
          const uint16_t* vt = v + (row * Hv + h) * V;

          /* 2a. gate activation, per key channel */
          for (int c = 0; c < K; ++c) {
            double x = bf16_to_double(gt[c]) + (dt_bias ? (double)dt_bias[(size_t)h * K + c] : 0.0);
            a[c] = orc_gate(gate_mode, x, A_log ? (double)A_log[h] : 0.0, lower_bound);
          }
          /* 2b. write strength */
          double bt = bf16_to_double(beta[row * Hv + h]);
          if (!(flags & ORC_FLAG_BETA_IS_PROB)) bt = orc_sigmoid(bt);
          /* 2c. query / key normalisation */
          for (int c = 0; c < K; ++c) { qn[c] = bf16_to_double(qt[c]); kn[c] = bf16_to_double(kt[c]); }
          if (flags & ORC_FLAG_QK_L2NORM) {
            kda_oracle_l2norm(K, qn, qn);
            kda_oracle_l2norm(K, kn, kn);
          }
          for (int i = 0; i < V; ++i) vv[i] = bf16_to_double(vt[i]);

          /* 2d. decay: S <- S Diag(e^a) */
          for (int i = 0; i < V; ++i)
            for (int c = 0; c < K; ++c) S[(size_t)i * K + c] *= exp(a[c]);
          /* 2e. read: r = S k */
          for (int i = 0; i < V; ++i) {
            double acc = 0.0;
            for (int c = 0; c < K; ++c) acc += S[(size_t)i * K + c] * kn[c];
            r[i] = acc;
          }
          /* 2f. delta-rule write: S <- S + beta (v - r) k^T */
          for (int i = 0; i < V; ++i) {
            double d = bt * (vv[i] - r[i]);
            for (int c = 0; c < K; ++c) S[(size_t)i * K + c] += d * kn[c];
          }
          /* 2g. output: o = scale S q */
          if (out) {
            double* ot = out + (row * Hv + h) * V;
            for (int i = 0; i < V; ++i) {
              double acc = 0.0;
              for (int c = 0; c < K; ++c) acc += S[(size_t)i * K + c] * qn[c];
              ot[i] = scale * acc;
            }
          }
        }
        /* 3. final state */
        if (hT) memcpy(hT + ((size_t)n * Hv + h) * V * K, S, sizeof(double) * (size_t)V * K);
      }
    }
    free(S); free(a); free(qn); free(kn); free(vv); free(r);
  }
  return err ? -1 : 0;
}
