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

/* ======================================================================
 * Backward (gradients), fp64 inputs -- TEST INFRASTRUCTURE ONLY.
 *
 * The pages list the backward pass among the KDA operations (fla-kda
 * SKILL.md, "Code map": backward passes; "Validation": forward, final state
 * and supported gradients) without printing it.  It is the adjoint of the
 * recurrence above, taken token by token in reverse.  With the state S_{t-1}
 * entering token t, Sd = S_{t-1} Diag(e^a), r = Sd k, u = beta (v - r),
 * S_t = Sd + u k^T and o = scale S_t q, the gradient dS of S_t gives
 *      dS  += scale do q^T            dq  = scale S_t^T do
 *      du   = dS k                    dk  = dS^T u
 *      dbeta= du . (v - r)            dv  = beta du       dr = -beta du
 *      dSd  = dS + dr k^T             dk += Sd^T dr
 *      da_c = e^{a_c} sum_i S_{t-1}[i,c] dSd[i,c]
 *      dS_{t-1} = dSd Diag(e^a)
 * then through the L2 norm, the gate activation and the beta sigmoid to the
 * raw inputs.  States are recomputed from checkpoints every ORC_CK tokens.
 * Inputs are given as doubles (not bf16) so that finite differences of
 * kda_oracle_fwd_f64 can pin these gradients.
 * ====================================================================== */
#define ORC_CK 256

/* One token's derived inputs (channels c < K, rows i < V). */
typedef struct {
  double *a, *ea, *qn, *kn, *vv;
  double bt, braw, rq, rk; /* beta, its raw value, inverse norms (1 when not normalised) */
} orc_tok;

static int orc_tok_alloc(orc_tok* t, int K, int V) {
  t->a = (double*)malloc(sizeof(double) * (size_t)K);
  t->ea = (double*)malloc(sizeof(double) * (size_t)K);
  t->qn = (double*)malloc(sizeof(double) * (size_t)K);
  t->kn = (double*)malloc(sizeof(double) * (size_t)K);
  t->vv = (double*)malloc(sizeof(double) * (size_t)V);
  return t->a && t->ea && t->qn && t->kn && t->vv;
}
static void orc_tok_free(orc_tok* t) { free(t->a); free(t->ea); free(t->qn); free(t->kn); free(t->vv); }

/* Token `row` (flat b*T + t) of v-head h: gate, beta, normalised q and k, v. */
static void orc_tok_load(orc_tok* tk, size_t row, int h, int hq, int Hqk, int Hv, int K, int V,
                         const double* q, const double* k, const double* v, const double* g,
                         const double* beta, const float* A_log, const float* dt_bias,
                         double lower_bound, int gate_mode, int flags) {
  const double* qt = q + (row * Hqk + hq) * K;
  const double* kt = k + (row * Hqk + hq) * K;
  const double* gt = g + (row * Hv + h) * K;
  const double* vt = v + (row * Hv + h) * V;
  for (int c = 0; c < K; ++c) {
    double x = gt[c] + (dt_bias ? (double)dt_bias[(size_t)h * K + c] : 0.0);
    tk->a[c] = orc_gate(gate_mode, x, A_log ? (double)A_log[h] : 0.0, lower_bound);
    tk->ea[c] = exp(tk->a[c]);
  }
  tk->braw = beta[row * Hv + h];
  tk->bt = (flags & ORC_FLAG_BETA_IS_PROB) ? tk->braw : orc_sigmoid(tk->braw);
  double sq = 0.0, sk = 0.0;
  for (int c = 0; c < K; ++c) { sq += qt[c] * qt[c]; sk += kt[c] * kt[c]; }
  tk->rq = (flags & ORC_FLAG_QK_L2NORM) ? 1.0 / sqrt(sq + ORC_L2_EPS) : 1.0;
  tk->rk = (flags & ORC_FLAG_QK_L2NORM) ? 1.0 / sqrt(sk + ORC_L2_EPS) : 1.0;
  for (int c = 0; c < K; ++c) { tk->qn[c] = qt[c] * tk->rq; tk->kn[c] = kt[c] * tk->rk; }
  for (int i = 0; i < V; ++i) tk->vv[i] = vt[i];
}

/* S (V x K) <- the state after the token; o (V) = scale S q if o != NULL. */
static void orc_tok_step(double* S, const orc_tok* tk, int K, int V, double scale, double* o) {
  for (int i = 0; i < V; ++i) {
    double* Si = S + (size_t)i * K;
    double r = 0.0;
    for (int c = 0; c < K; ++c) { Si[c] *= tk->ea[c]; r += Si[c] * tk->kn[c]; }
    const double u = tk->bt * (tk->vv[i] - r);
    for (int c = 0; c < K; ++c) Si[c] += u * tk->kn[c];
    if (o) {
      double acc = 0.0;
      for (int c = 0; c < K; ++c) acc += Si[c] * tk->qn[c];
      o[i] = scale * acc;
    }
  }
}

static int orc_check_shapes(int B, int T, int Hqk, int Hv, int K, int V, int N, const int64_t* cu) {
  if (B <= 0 || T < 0 || Hqk <= 0 || Hv <= 0 || K <= 0 || V <= 0) return -1;
  if (Hv % Hqk != 0) return -1;
  if (cu) {
    if (B != 1 || N <= 0 || cu[0] != 0 || cu[N] != T) return -1;
    for (int n = 0; n < N; ++n)
      if (cu[n + 1] < cu[n]) return -1;
  } else if (N != B) {
    return -1;
  }
  return 0;
}

/* The forward with fp64 inputs (same layouts as kda_oracle_fwd, doubles in
 * place of bf16 bits).  Used as the function whose finite differences pin
 * the gradients; equal to kda_oracle_fwd on bf16-representable inputs. */
int kda_oracle_fwd_f64(int B, int T, int Hqk, int Hv, int K, int V, int N,
                       const double* q, const double* k, const double* v, const double* g,
                       const double* beta, const float* A_log, const float* dt_bias,
                       const int64_t* cu_seqlens, double scale, double lower_bound, int gate_mode,
                       int flags, const double* h0, double* hT, double* out) {
  if (orc_check_shapes(B, T, Hqk, Hv, K, V, N, cu_seqlens)) return -1;
  const int G = Hv / Hqk;
  double* S = (double*)malloc(sizeof(double) * (size_t)V * K);
  orc_tok tk;
  int ok = S && orc_tok_alloc(&tk, K, V);
  if (ok) {
    for (long long p = 0; p < (long long)N * Hv; ++p) {
      const int n = (int)(p / Hv), h = (int)(p % Hv), hq = h / G;
      const int b = cu_seqlens ? 0 : n;
      const long long bos = cu_seqlens ? cu_seqlens[n] : 0, eos = cu_seqlens ? cu_seqlens[n + 1] : T;
      if (h0) memcpy(S, h0 + ((size_t)n * Hv + h) * V * K, sizeof(double) * (size_t)V * K);
      else    memset(S, 0, sizeof(double) * (size_t)V * K);
      for (long long t = bos; t < eos; ++t) {
        const size_t row = (size_t)b * T + (size_t)t;
        orc_tok_load(&tk, row, h, hq, Hqk, Hv, K, V, q, k, v, g, beta, A_log, dt_bias, lower_bound,
                     gate_mode, flags);
        orc_tok_step(S, &tk, K, V, scale, out ? out + (row * Hv + h) * V : NULL);
      }
      if (hT) memcpy(hT + ((size_t)n * Hv + h) * V * K, S, sizeof(double) * (size_t)V * K);
    }
    orc_tok_free(&tk);
  }
  free(S);
  return ok ? 0 : -1;
}

/*
 * Gradients of the forward with respect to every input.
 *   do_   : [B,T,Hv,V] gradient of out          dhT : [N,Hv,V,K] gradient of the
 *           final state, or NULL (zero)
 * Outputs (each may be NULL when not wanted):
 *   dq, dk [B,T,Hqk,K] (summed over the v-heads sharing a q/k head),
 *   dv [B,T,Hv,V], dg [B,T,Hv,K], dbeta [B,T,Hv] (w.r.t. the logits, or the
 *   probabilities with ORC_FLAG_BETA_IS_PROB), dA_log [Hv] (zero when A_log is
 *   NULL or the decay is pre-gated), ddt_bias [Hv,K] (w.r.t. the bias, zero or
 *   not), dh0 [N,Hv,V,K].
 * Work is split over (sequence, v-head) pairs; per-pair partial sums of the
 * shared gradients (dq, dk over grouped heads; dA_log, ddt_bias over
 * sequences) are added up after the parallel loop.
 */
int kda_oracle_bwd(int B, int T, int Hqk, int Hv, int K, int V, int N,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const float* A_log, const float* dt_bias,
                   const int64_t* cu_seqlens, double scale, double lower_bound, int gate_mode,
                   int flags, const double* h0, const double* do_, const double* dhT,
                   double* dq, double* dk, double* dv, double* dg, double* dbeta,
                   double* dA_log, double* ddt_bias, double* dh0, int nthreads) {
  if (orc_check_shapes(B, T, Hqk, Hv, K, V, N, cu_seqlens)) return -1;
  const int G = Hv / Hqk;
  const long long npairs = (long long)N * Hv;
  const size_t VK = (size_t)V * K;
  /* per-v-head q/k gradients and per-pair gate-parameter partials */
  double* dqv = (double*)calloc((size_t)B * T * Hv * K, sizeof(double));
  double* dkv = (double*)calloc((size_t)B * T * Hv * K, sizeof(double));
  double* dAp = (double*)calloc((size_t)npairs, sizeof(double));
  double* ddtp = (double*)calloc((size_t)npairs * K, sizeof(double));
  if (!dqv || !dkv || !dAp || !ddtp) { free(dqv); free(dkv); free(dAp); free(ddtp); return -1; }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;
#pragma omp parallel
  {
    orc_tok tk;
    const int tk_ok = orc_tok_alloc(&tk, K, V);
    double* S = (double*)malloc(sizeof(double) * VK);
    double* Sbuf = (double*)malloc(sizeof(double) * VK * (ORC_CK + 1));
    double* dS = (double*)malloc(sizeof(double) * VK);
    double* Sd = (double*)malloc(sizeof(double) * VK);
    double* r = (double*)malloc(sizeof(double) * V);
    double* du = (double*)malloc(sizeof(double) * V);
    double* dqn = (double*)malloc(sizeof(double) * K);
    double* dkn = (double*)malloc(sizeof(double) * K);
    double* da = (double*)malloc(sizeof(double) * K);
    double* Sck = NULL;
    if (!tk_ok || !S || !Sbuf || !dS || !Sd || !r || !du || !dqn || !dkn || !da) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long long p = 0; p < npairs; ++p) {
        const int n = (int)(p / Hv), h = (int)(p % Hv), hq = h / G;
        const int b = cu_seqlens ? 0 : n;
        const long long bos = cu_seqlens ? cu_seqlens[n] : 0, eos = cu_seqlens ? cu_seqlens[n + 1] : T;
        const long long L = eos - bos, nblk = (L + ORC_CK - 1) / ORC_CK;
        const double Aexp = A_log ? exp((double)A_log[h]) : 1.0;
        /* 1. forward, keeping the state at the start of every block */
        free(Sck);
        Sck = (double*)malloc(sizeof(double) * VK * (size_t)(nblk > 0 ? nblk : 1));
        if (!Sck) {
#pragma omp atomic write
          err = 1;
          continue;
        }
        if (h0) memcpy(S, h0 + ((size_t)n * Hv + h) * VK, sizeof(double) * VK);
        else    memset(S, 0, sizeof(double) * VK);
        for (long long t = bos; t < eos; ++t) {
          if ((t - bos) % ORC_CK == 0) memcpy(Sck + (size_t)((t - bos) / ORC_CK) * VK, S, sizeof(double) * VK);
          orc_tok_load(&tk, (size_t)b * T + (size_t)t, h, hq, Hqk, Hv, K, V, q, k, v, g, beta, A_log, dt_bias,
                       lower_bound, gate_mode, flags);
          orc_tok_step(S, &tk, K, V, scale, NULL);
        }
        /* 2. backward, block by block in reverse */
        if (dhT) memcpy(dS, dhT + ((size_t)n * Hv + h) * VK, sizeof(double) * VK);
        else     memset(dS, 0, sizeof(double) * VK);
        for (long long blk = nblk - 1; blk >= 0; --blk) {
          const long long t0 = bos + blk * ORC_CK, t1 = (t0 + ORC_CK < eos) ? t0 + ORC_CK : eos;
          /* states S_{t0-1} .. S_{t1-1} (Sbuf[j] enters token t0 + j) */
          memcpy(Sbuf, Sck + (size_t)blk * VK, sizeof(double) * VK);
          for (long long t = t0; t < t1; ++t) {
            orc_tok_load(&tk, (size_t)b * T + (size_t)t, h, hq, Hqk, Hv, K, V, q, k, v, g, beta, A_log,
                         dt_bias, lower_bound, gate_mode, flags);
            memcpy(Sbuf + (size_t)(t - t0 + 1) * VK, Sbuf + (size_t)(t - t0) * VK, sizeof(double) * VK);
            orc_tok_step(Sbuf + (size_t)(t - t0 + 1) * VK, &tk, K, V, scale, NULL);
          }
          for (long long t = t1 - 1; t >= t0; --t) {
            const size_t row = (size_t)b * T + (size_t)t;
            orc_tok_load(&tk, row, h, hq, Hqk, Hv, K, V, q, k, v, g, beta, A_log, dt_bias, lower_bound,
                         gate_mode, flags);
            const double* Sp = Sbuf + (size_t)(t - t0) * VK;     /* entering token t */
            const double* St = Sbuf + (size_t)(t - t0 + 1) * VK; /* after token t */
            const double* dot = do_ + (row * Hv + h) * V;
            /* o = scale S_t q */
            for (int c = 0; c < K; ++c) {
              double acc = 0.0;
              for (int i = 0; i < V; ++i) acc += St[(size_t)i * K + c] * dot[i];
              dqn[c] = scale * acc;
            }
            for (int i = 0; i < V; ++i)
              for (int c = 0; c < K; ++c) dS[(size_t)i * K + c] += scale * dot[i] * tk.qn[c];
            /* Sd, r, u */
            for (int i = 0; i < V; ++i) {
              double acc = 0.0;
              for (int c = 0; c < K; ++c) {
                Sd[(size_t)i * K + c] = Sp[(size_t)i * K + c] * tk.ea[c];
                acc += Sd[(size_t)i * K + c] * tk.kn[c];
              }
              r[i] = acc;
            }
            /* S_t = Sd + u k^T */
            double dbt = 0.0;
            for (int c = 0; c < K; ++c) dkn[c] = 0.0;
            for (int i = 0; i < V; ++i) {
              double acc = 0.0;
              for (int c = 0; c < K; ++c) acc += dS[(size_t)i * K + c] * tk.kn[c];
              du[i] = acc;
              const double u = tk.bt * (tk.vv[i] - r[i]);
              for (int c = 0; c < K; ++c) dkn[c] += dS[(size_t)i * K + c] * u;
              dbt += acc * (tk.vv[i] - r[i]);
            }
            /* u = beta (v - r);  r = Sd k */
            double* dvt = dv ? dv + (row * Hv + h) * V : NULL;
            for (int i = 0; i < V; ++i) {
              if (dvt) dvt[i] = tk.bt * du[i];
              const double dr = -tk.bt * du[i];
              for (int c = 0; c < K; ++c) {
                dS[(size_t)i * K + c] += dr * tk.kn[c]; /* dS now holds dSd */
                dkn[c] += Sd[(size_t)i * K + c] * dr;
              }
            }
            /* Sd = S_{t-1} Diag(e^a) */
            for (int c = 0; c < K; ++c) {
              double acc = 0.0;
              for (int i = 0; i < V; ++i) acc += Sp[(size_t)i * K + c] * dS[(size_t)i * K + c];
              da[c] = tk.ea[c] * acc;
            }
            for (int i = 0; i < V; ++i)
              for (int c = 0; c < K; ++c) dS[(size_t)i * K + c] *= tk.ea[c];
            /* beta */
            if (dbeta) dbeta[row * Hv + h] =
                (flags & ORC_FLAG_BETA_IS_PROB) ? dbt : dbt * tk.bt * (1.0 - tk.bt);
            /* L2 norms: y = x r  =>  dx = r (dy - y (y . dy)) */
            double yq = 0.0, yk = 0.0;
            if (flags & ORC_FLAG_QK_L2NORM)
              for (int c = 0; c < K; ++c) { yq += tk.qn[c] * dqn[c]; yk += tk.kn[c] * dkn[c]; }
            double* dqt = dqv + (row * Hv + h) * K;
            double* dkt = dkv + (row * Hv + h) * K;
            for (int c = 0; c < K; ++c) {
              dqt[c] = tk.rq * (dqn[c] - tk.qn[c] * yq);
              dkt[c] = tk.rk * (dkn[c] - tk.kn[c] * yk);
            }
            /* gate: a = f(x), x = g + dt_bias */
            double* dgt = dg ? dg + (row * Hv + h) * K : NULL;
            for (int c = 0; c < K; ++c) {
              const double x = g[(row * Hv + h) * K + c] + (dt_bias ? (double)dt_bias[(size_t)h * K + c] : 0.0);
              double dadx, dadA;
              if (gate_mode == ORC_GATE_SOFTPLUS) {
                dadx = -Aexp * orc_sigmoid(x);
                dadA = tk.a[c];
              } else if (gate_mode == ORC_GATE_SAFE_SIGMOID) {
                const double z = Aexp * x, s = orc_sigmoid(z);
                dadx = lower_bound * s * (1.0 - s) * Aexp;
                dadA = lower_bound * s * (1.0 - s) * z;
              } else {
                dadx = 1.0;
                dadA = 0.0;
              }
              if (dgt) dgt[c] = da[c] * dadx;
              ddtp[(size_t)p * K + c] += da[c] * dadx;
              if (A_log) dAp[p] += da[c] * dadA;
            }
          }
        }
        if (dh0) memcpy(dh0 + ((size_t)n * Hv + h) * VK, dS, sizeof(double) * VK);
      }
    }
    free(Sck);
    orc_tok_free(&tk);
    free(S); free(Sbuf); free(dS); free(Sd); free(r); free(du); free(dqn); free(dkn); free(da);
  }
  /* 3. shared gradients */
  if (dq || dk)
    for (size_t row = 0; row < (size_t)B * T; ++row)
      for (int hq = 0; hq < Hqk; ++hq)
        for (int c = 0; c < K; ++c) {
          double sq = 0.0, sk = 0.0;
          for (int j = 0; j < G; ++j) {
            sq += dqv[(row * Hv + hq * G + j) * K + c];
            sk += dkv[(row * Hv + hq * G + j) * K + c];
          }
          if (dq) dq[(row * Hqk + hq) * K + c] = sq;
          if (dk) dk[(row * Hqk + hq) * K + c] = sk;
        }
  if (dA_log)
    for (int h = 0; h < Hv; ++h) {
      double s = 0.0;
      for (int n = 0; n < N; ++n) s += dAp[(size_t)n * Hv + h];
      dA_log[h] = (gate_mode == ORC_GATE_PREGATED) ? 0.0 : s;
    }
  if (ddt_bias)
    for (int h = 0; h < Hv; ++h)
      for (int c = 0; c < K; ++c) {
        double s = 0.0;
        for (int n = 0; n < N; ++n) s += ddtp[((size_t)n * Hv + h) * K + c];
        ddt_bias[(size_t)h * K + c] = s;
      }
  free(dqv); free(dkv); free(dAp); free(ddtp);
  return err ? -1 : 0;
}
