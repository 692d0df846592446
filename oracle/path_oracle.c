/*
 * Plain fp64 CPU oracle for PaTH attention.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this code.  It shares nothing with the HIP library: no headers,
 * no helpers, no constants.  Every routine below is the slow, obviously
 * correct reading of the defining formulas, written for a reader who holds
 * the source pages next to it.
 *
 * Sources (cited by page title and section):
 *   [P1] "PaTH Attention" technical summary (gist.science 2505.16381)
 *        §2 "Mecanismo Central"  - attention logit k_j^T (prod_{s=j+1..i} H_s) q_i,
 *                                   causal softmax A_ij ∝ exp(logit),
 *                                   H_s = I - beta_s w_s w_s^T, beta_s in (0,2).
 *        §2 "Extensões: PaTH-FoX" - additive data-dependent forget-gate bias.
 *        §3 "Representação de Transformação UT" - a product of the H_s is
 *                                   I - W^T T^{-1} W with T triangular, built
 *                                   from beta (and the Gram matrix W W^T).
 *        §3 "Algoritmo Estilo FlashAttention" - boundary-adjusted Q/K per block.
 *        §3 "Inferência"          - cached keys updated in place with the
 *                                   current step's transition.
 *
 * Readings where the pages are silent (also listed in the design notes):
 *   - the product prod_{s=j+1..i} H_s is H_{j+1} H_{j+2} ... H_i, so H_i is
 *     the first factor to act on q_i; the empty product (j = i) is I;
 *   - softmax is over j <= i, with an explicit logit multiplier `scale`;
 *   - the FoX bias is sum_{s=j+1..i} log f_s, added after `scale`;
 *   - lse is the natural log of the softmax denominator.
 *
 * All arithmetic is fp64 on the exact stored input values; loops run in the
 * order the definitions are written.  OpenMP only spreads independent query
 * rows over threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const double* a, const double* b, int64_t d) {
  double s = 0.0;
  for (int64_t t = 0; t < d; ++t) s += a[t] * b[t];
  return s;
}

/* u <- H_s u = u - beta_s (w_s . u) w_s   [P1 §2 "Mecanismo Central"] */
static void apply_H(double* u, const double* w_s, double beta_s, int64_t d) {
  double c = beta_s * dot(w_s, u, d);
  for (int64_t t = 0; t < d; ++t) u[t] -= c * w_s[t];
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * One head.  For every requested query row i:
 *   u <- q_i
 *   for j = i, i-1, ..., 0:
 *       s_ij = scale * (k_j . u) + sum_{s=j+1..i} log f_s
 *       u <- H_j u                       (so u = H_{j}...H_i q_i next round)
 *   o_i = sum_j softmax_j(s_ij) v_j,  lse_i = log sum_j exp(s_ij)
 * [P1 §2 "Mecanismo Central"; §2 "Extensões: PaTH-FoX" for the bias]
 *
 * q,k,v,w: [L,d] row-major; beta, log_forget: [L] (log_forget may be NULL).
 * rows: n_rows query indices (NULL = all L rows in order).
 * o: [n_rows,d]; lse: [n_rows]; logits (optional, may be NULL): [n_rows,L],
 * entries j > i are set to -INFINITY.
 */
void oracle_path_fwd(int64_t L, int64_t d, const double* q, const double* k,
                     const double* v, const double* w, const double* beta,
                     const double* log_forget, double scale, int64_t n_rows,
                     const int64_t* rows, double* o, double* lse,
                     double* logits) {
  if (rows == NULL) n_rows = L;
#pragma omp parallel
  {
    double* u = (double*)malloc(sizeof(double) * (size_t)d);
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t i = rows ? rows[r] : r;
      memcpy(u, q + i * d, sizeof(double) * (size_t)d);
      double bias = 0.0;
      for (int64_t j = i; j >= 0; --j) {
        s[j] = scale * dot(k + j * d, u, d) + bias;
        apply_H(u, w + j * d, beta[j], d);
        if (log_forget) bias += log_forget[j];
      }
      double m = -INFINITY;
      for (int64_t j = 0; j <= i; ++j) m = s[j] > m ? s[j] : m;
      double l = 0.0;
      for (int64_t j = 0; j <= i; ++j) l += exp(s[j] - m);
      double* oi = o + r * d;
      for (int64_t t = 0; t < d; ++t) oi[t] = 0.0;
      for (int64_t j = 0; j <= i; ++j) {
        double p = exp(s[j] - m) / l;
        for (int64_t t = 0; t < d; ++t) oi[t] += p * v[j * d + t];
      }
      lse[r] = m + log(l);
      if (logits) {
        for (int64_t j = 0; j < L; ++j)
          logits[r * L + j] = (j <= i) ? s[j] : -INFINITY;
      }
    }
    free(u);
    free(s);
  }
}

/*
 * One decode step for one head  [P1 §3 "Inferência"]:
 *   k_j <- H_t k_j  for every cached j < len   (in place, in k_cache)
 *   keys  = [k_0 .. k_{len-1} (updated), k_t],  values = [v_0 .. v_{len-1}, v_t]
 *   s_j = scale * (k_j . q_t) + bias_j;  o = softmax(s) . values;  lse = log sum exp s
 * The new key enters untransformed: its path product is empty.
 * bias is NULL (no bias) or [len + 1].
 * k_cache, v_cache: [len,d]; q_t,k_t,v_t,w_t: [d]; o: [d]; lse: scalar.
 */
static void decode_step(int64_t len, int64_t d, const double* q_t, const double* k_t,
                        const double* v_t, const double* w_t, double beta_t, double* k_cache,
                        const double* v_cache, double scale, const double* bias, double* o,
                        double* lse) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(len + 1));
  for (int64_t j = 0; j < len; ++j) {
    apply_H(k_cache + j * d, w_t, beta_t, d);
    s[j] = scale * dot(k_cache + j * d, q_t, d);
  }
  s[len] = scale * dot(k_t, q_t, d);
  if (bias)
    for (int64_t j = 0; j <= len; ++j) s[j] += bias[j];
  double m = -INFINITY;
  for (int64_t j = 0; j <= len; ++j) m = s[j] > m ? s[j] : m;
  double l = 0.0;
  for (int64_t j = 0; j <= len; ++j) l += exp(s[j] - m);
  for (int64_t t = 0; t < d; ++t) o[t] = 0.0;
  for (int64_t j = 0; j <= len; ++j) {
    double p = exp(s[j] - m) / l;
    const double* vj = (j < len) ? v_cache + j * d : v_t;
    for (int64_t t = 0; t < d; ++t) o[t] += p * vj[t];
  }
  *lse = m + log(l);
  free(s);
}

void oracle_path_decode(int64_t len, int64_t d, const double* q_t,
                        const double* k_t, const double* v_t,
                        const double* w_t, double beta_t, double* k_cache,
                        const double* v_cache, double scale, double* o,
                        double* lse) {
  decode_step(len, d, q_t, k_t, v_t, w_t, beta_t, k_cache, v_cache, scale, NULL, o, lse);
}

/*
 * PaTH-FoX decode step for one head  [P1 §2 "Extensões: PaTH-FoX" with §3
 * "Inferência"]: the forget-gate bias of key j seen from query t is the sum
 * of log f_s over j < s <= t.  With the running prefix c_j = sum_{s<=j} log f_s
 * kept per cached key (cum_cache[j], j < len), the new prefix is
 *   c_t = c_{len-1} + log_f_t   (c_{-1} = 0),
 * the bias of cached key j is c_t - c_j and that of the new key is 0.
 * Everything else is the plain decode step above.  *c_t_out receives c_t.
 */
void oracle_path_decode_fox(int64_t len, int64_t d, const double* q_t,
                            const double* k_t, const double* v_t,
                            const double* w_t, double beta_t, double log_f_t,
                            double* k_cache, const double* v_cache,
                            const double* cum_cache, double scale, double* o,
                            double* lse, double* c_t_out) {
  const double c_t = (len > 0 ? cum_cache[len - 1] : 0.0) + log_f_t;
  double* bias = (double*)malloc(sizeof(double) * (size_t)(len + 1));
  for (int64_t j = 0; j < len; ++j) bias[j] = c_t - cum_cache[j];
  bias[len] = 0.0;
  decode_step(len, d, q_t, k_t, v_t, w_t, beta_t, k_cache, v_cache, scale, bias, o, lse);
  *c_t_out = c_t;
  free(bias);
}

/*
 * UT factor of one block of n tokens  [P1 §3 "Representação de Transformação UT"]:
 * the product H_0 H_1 ... H_{n-1} equals I - W^T T^{-1} W, with W the n x d
 * matrix of rows w_s and T upper triangular, T = diag(1/beta) + strict_upper(W W^T).
 * To stay defined at beta_s = 0 the oracle never forms 1/beta: it solves
 *     (I + diag(beta) strict_upper(W W^T)) X = diag(beta),   X = T^{-1},
 * by plain back substitution, row n-1 first.
 * w: [n,d]; beta: [n]; tinv: [n,n] (upper triangular, zeros below).
 */
void oracle_ut_tinv(int64_t n, int64_t d, const double* w, const double* beta,
                    double* tinv) {
  for (int64_t i = 0; i < n * n; ++i) tinv[i] = 0.0;
  for (int64_t r = n - 1; r >= 0; --r) {
    for (int64_t c = r; c < n; ++c) {
      double acc = (r == c) ? beta[r] : 0.0;
      for (int64_t t = r + 1; t <= c; ++t)
        acc -= beta[r] * dot(w + r * d, w + t * d, d) * tinv[t * n + c];
      tinv[r * n + c] = acc;
    }
  }
}

/*
 * Boundary-adjusted queries and keys of one block and its transition
 * [P1 §3 "Algoritmo Estilo FlashAttention"], taken straight from the
 * definitions, one H at a time (independent of the UT factor above):
 *   qhat_r = H_0 H_1 ... H_r q_r      (apply H_r first, H_0 last)
 *   khat_c = H_{n-1} ... H_{c+1} k_c  (apply H_{c+1} first)
 *   pT     = (H_0 H_1 ... H_{n-1})^T  as an explicit d x d matrix
 * q,k,w: [n,d]; qhat,khat: [n,d]; pT: [d,d].
 */
void oracle_block_adjust(int64_t n, int64_t d, const double* q,
                         const double* k, const double* w, const double* beta,
                         double* qhat, double* khat, double* pT) {
  for (int64_t r = 0; r < n; ++r) {
    double* u = qhat + r * d;
    memcpy(u, q + r * d, sizeof(double) * (size_t)d);
    for (int64_t s = r; s >= 0; --s) apply_H(u, w + s * d, beta[s], d);
  }
  for (int64_t c = 0; c < n; ++c) {
    double* u = khat + c * d;
    memcpy(u, k + c * d, sizeof(double) * (size_t)d);
    for (int64_t s = c + 1; s < n; ++s) apply_H(u, w + s * d, beta[s], d);
  }
  /* P <- I, then P <- P H_s for s = 0..n-1; column t of P is P e_t. */
  double* P = (double*)malloc(sizeof(double) * (size_t)(d * d));
  for (int64_t a = 0; a < d; ++a)
    for (int64_t b = 0; b < d; ++b) P[a * d + b] = (a == b) ? 1.0 : 0.0;
  double* Pw = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t s = 0; s < n; ++s) {
    const double* ws = w + s * d;
    for (int64_t a = 0; a < d; ++a) Pw[a] = dot(P + a * d, ws, d);
    for (int64_t a = 0; a < d; ++a)
      for (int64_t b = 0; b < d; ++b) P[a * d + b] -= beta[s] * Pw[a] * ws[b];
  }
  for (int64_t a = 0; a < d; ++a)
    for (int64_t b = 0; b < d; ++b) pT[a * d + b] = P[b * d + a];
  free(Pw);
  free(P);
}

/* c_i = sum_{s<=i} log f_s, so c_i - c_j is the FoX bias  [P1 §2 "Extensões: PaTH-FoX"] */
void oracle_prefix_sum(int64_t L, const double* x, double* c) {
  double acc = 0.0;
  for (int64_t i = 0; i < L; ++i) {
    acc += x[i];
    c[i] = acc;
  }
}

/*
 * Gradients of the scalar <dO, o> for one head, by reverse-mode
 * differentiation of the defining loop of oracle_path_fwd (lse receives no
 * incoming gradient) [P1 §2 "Mecanismo Central", §2 "Extensões: PaTH-FoX";
 * the pages describe no backward pass, so this is the exact derivative of the
 * forward's definition].  For query i let u^(j) be the transported query the
 * loop holds when it forms s_ij:  u^(i) = q_i,  u^(j-1) = H_j u^(j).
 *   forward:  s_ij = scale k_j.u^(j) + c_i - c_j,  p_ij = softmax_j(s_ij),
 *             o_i = sum_j p_ij v_j
 *   reverse:  dv_j += p_ij dO_i
 *             ds_ij = p_ij (dO_i.v_j - dO_i.o_i)         (softmax adjoint)
 *             dk_j += scale ds_ij u^(j),  dc_i += ds_ij,  dc_j -= ds_ij
 *             the query adjoint g^(j) = dloss/du^(j) runs j = 0 .. i:
 *               g^(j) = scale ds_ij k_j + H_j^T g^(j-1)   (g^(-1) = 0; H_j = H_j^T),
 *               and H_j, which forms u^(j-1) from u^(j), takes with
 *               a = w_j.u^(j), b = w_j.g^(j-1):
 *                 dbeta_j -= a b,   dw_j -= beta_j (b u^(j) + a g^(j-1));
 *             dq_i = g^(i);   dlog_forget_s = sum_{i >= s} dc_i.
 * The u^(j) of one query are kept (i+1 vectors): H may be singular, so they
 * are not rebuilt backwards.  OpenMP spreads the queries over threads (static
 * round robin, so the sums are reproducible for a given thread count); each
 * thread accumulates into its own arrays, summed in thread order at the end.
 * Inputs as oracle_path_fwd plus dO [L,d]; outputs dq, dk, dv, dw [L,d],
 * dbeta [L], dlog_forget [L] (written only when log_forget != NULL).
 */
void oracle_path_bwd(int64_t L, int64_t d, const double* q, const double* k,
                     const double* v, const double* w, const double* beta,
                     const double* log_forget, double scale, const double* dO,
                     double* dq, double* dk, double* dv, double* dw, double* dbeta,
                     double* dlog_forget) {
  int nt = 1;
#ifdef _OPENMP
  nt = omp_get_max_threads();
#endif
  const size_t Ld = (size_t)(L * d);
  /* per-thread accumulators: dk, dv, dw [L,d] and dbeta, dc [L] */
  double* acc = (double*)calloc((size_t)nt * (3 * Ld + 2 * (size_t)L), sizeof(double));
  double* c = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  double bias = 0.0;
  for (int64_t i = 0; i < L; ++i) {
    bias += log_forget ? log_forget[i] : 0.0;
    c[i] = bias;
  }
  for (size_t t = 0; t < Ld; ++t) dq[t] = 0.0;
#pragma omp parallel num_threads(nt)
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* my = acc + (size_t)tid * (3 * Ld + 2 * (size_t)L);
    double *adk = my, *adv = my + Ld, *adw = my + 2 * Ld;
    double *adb = my + 3 * Ld, *adc = my + 3 * Ld + L;
    double* U = (double*)malloc(sizeof(double) * Ld);  /* U[j] = u^(j) */
    double* s = (double*)malloc(sizeof(double) * (size_t)L);
    double* g = (double*)malloc(sizeof(double) * (size_t)d);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static, 1)
    for (int64_t i = 0; i < L; ++i) {
      /* forward of row i, keeping every transported query */
      memcpy(U + i * d, q + i * d, sizeof(double) * (size_t)d);
      for (int64_t j = i; j >= 0; --j) {
        s[j] = scale * dot(k + j * d, U + j * d, d) + (c[i] - c[j]);
        if (j > 0) {
          memcpy(U + (j - 1) * d, U + j * d, sizeof(double) * (size_t)d);
          apply_H(U + (j - 1) * d, w + j * d, beta[j], d);
        }
      }
      double m = -INFINITY;
      for (int64_t j = 0; j <= i; ++j) m = s[j] > m ? s[j] : m;
      double l = 0.0;
      for (int64_t j = 0; j <= i; ++j) l += exp(s[j] - m);
      for (int64_t t = 0; t < d; ++t) o[t] = 0.0;
      for (int64_t j = 0; j <= i; ++j) {
        s[j] = exp(s[j] - m) / l; /* s now holds p_ij */
        for (int64_t t = 0; t < d; ++t) o[t] += s[j] * v[j * d + t];
      }
      const double* dOi = dO + i * d;
      const double Di = dot(dOi, o, d);
      /* reverse of row i */
      for (int64_t t = 0; t < d; ++t) g[t] = 0.0;
      for (int64_t j = 0; j <= i; ++j) {
        const double p = s[j];
        for (int64_t t = 0; t < d; ++t) adv[j * d + t] += p * dOi[t];
        const double ds = p * (dot(dOi, v + j * d, d) - Di);
        adc[i] += ds;
        adc[j] -= ds;
        const double* u = U + j * d;
        if (j > 0) { /* H_j maps u^(j) to u^(j-1), whose adjoint g holds */
          const double a = dot(w + j * d, u, d), b = dot(w + j * d, g, d);
          adb[j] -= a * b;
          for (int64_t t = 0; t < d; ++t) adw[j * d + t] -= beta[j] * (b * u[t] + a * g[t]);
          apply_H(g, w + j * d, beta[j], d);
        }
        for (int64_t t = 0; t < d; ++t) {
          adk[j * d + t] += scale * ds * u[t];
          g[t] += scale * ds * k[j * d + t];
        }
      }
      memcpy(dq + i * d, g, sizeof(double) * (size_t)d);
    }
    free(o);
    free(g);
    free(s);
    free(U);
  }
  for (size_t t = 0; t < Ld; ++t) dk[t] = dv[t] = dw[t] = 0.0;
  for (int64_t i = 0; i < L; ++i) dbeta[i] = 0.0;
  double* dc = c; /* reused: sum of the threads' dc */
  for (int64_t i = 0; i < L; ++i) dc[i] = 0.0;
  for (int th = 0; th < nt; ++th) {
    const double* my = acc + (size_t)th * (3 * Ld + 2 * (size_t)L);
    for (size_t t = 0; t < Ld; ++t) {
      dk[t] += my[t];
      dv[t] += my[Ld + t];
      dw[t] += my[2 * Ld + t];
    }
    for (int64_t i = 0; i < L; ++i) {
      dbeta[i] += my[3 * Ld + i];
      dc[i] += my[3 * Ld + L + i];
    }
  }
  if (dlog_forget) { /* c_i = sum_{s<=i} log f_s: d log f_s = sum_{i>=s} dc_i */
    double run = 0.0;
    for (int64_t s2 = L - 1; s2 >= 0; --s2) {
      run += dc[s2];
      dlog_forget[s2] = log_forget ? run : 0.0;
    }
  }
  free(c);
  free(acc);
}
