/*
 * KDA forward oracle — plain, slow, token-serial CPU reference in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header, table or constant with
 * the HIP implementation.
 *
 * What it computes (Kimi Delta Attention, one recurrence per sequence and
 * head; every (sequence, head) pair is an independent task):
 *
 *   alpha_t = exp(g_t)            per-channel decay, a d_k vector
 *       [core.today "Kimi Linear 특집", ch.4 혁신 1 (channel-wise forget gate);
 *        hnts03 "논문 리뷰: Kimi Delta Attention", section "Kimi Delta Attention"
 *        (scalar gate of Gated DeltaNet replaced by a diagonal, per-channel gate)]
 *
 *   S_t = (Diag(alpha_t) - beta_t k_t (k_t ⊙ alpha_t)^T) S_{t-1} + beta_t k_t v_t^T
 *       [core.today "Kimi Linear 특집", ch.4 혁신 2, state-update equation]
 *
 *   o_t = scale * S_t^T q_t       readout of the d_k x d_v state after the update
 *       [core.today "Kimi Linear 특집", ch.2, linear-attention formula Q(K^T V)]
 *
 * S is d_k x d_v, indexed S[i][j] (i over key channels, j over value
 * channels), so S^T k is the value retrieved by key k, as in the delta rule
 * S <- S + beta k (v - S^T k)^T  [core.today ch.3, delta-rule update].
 *
 * kda_oracle_fwd evaluates the update in the algebraically identical
 * "decay, then delta" order: multiplying out the bracket gives
 *   S~ = Diag(alpha) S_{t-1};  e = v - S~^T k;  S_t = S~ + beta k e^T,
 * because (k ⊙ alpha)^T S_{t-1} = k^T Diag(alpha) S_{t-1} = k^T S~.
 * kda_oracle_fwd_literal evaluates the bracketed matrix exactly as printed
 * (a d_k x d_k transition matrix per token); it is O(d_k^2 d_v) per token and
 * exists only to cross-check the first form on tiny inputs.
 *
 * Memory layout (all row-major, fp64):
 *   q, k, g : [rows][H][DK]      v : [rows][H][DV]      beta : [rows][H]
 *   o       : [rows][H][DV]
 *   S0, S_out : [N][H][DK][DV]   (S0 may be NULL = zero initial state;
 *                                 S_out may be NULL = final state not wanted)
 * Sequence n occupies rows [seq_start[n], seq_start[n] + seq_len[n]); a
 * fixed-length batch of B rows of T tokens is N = B sequences with
 * seq_start[n] = n*T.  A zero-length sequence produces no output rows and
 * returns its initial state unchanged.
 * heads[0..nh) lists the heads to evaluate (NULL = all H heads); output rows
 * and states of other heads are left untouched.
 * Column j of S only ever meets column j of v, of e and of o (the decay scales
 * rows, the error and the write are per column, the readout sums over rows),
 * so a task may cover a block of value columns without changing a single
 * operation: col_block > 0 splits every (sequence, head) into blocks of that
 * many columns; col_block <= 0 keeps whole heads.
 * nthreads > 0 caps the OpenMP threads used across tasks.
 *
 * Returns 0 on success, -1 on invalid sizes, -2 on allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int check_sizes(int64_t N, int64_t H, int64_t DK, int64_t DV, const int64_t* seq_len) {
  if (N < 0 || H <= 0 || DK <= 0 || DV <= 0) return -1;
  for (int64_t n = 0; n < N; ++n)
    if (seq_len[n] < 0) return -1;
  return 0;
}

/* One (sequence, head) task in the decay-then-delta order. */
static void run_task(const double* q, const double* k, const double* v, const double* g,
                     const double* beta, double scale, const double* S0, double* S_out,
                     double* o, int64_t start, int64_t len, int64_t n, int64_t h, int64_t H,
                     int64_t DK, int64_t DV, int64_t j0, int64_t j1, double* S, double* e) {
  const int64_t sdim = DK * DV;
  for (int64_t i = 0; i < DK; ++i)
    for (int64_t j = j0; j < j1; ++j)
      S[i * DV + j] = S0 ? S0[(n * H + h) * sdim + i * DV + j] : 0.0;

  for (int64_t t = start; t < start + len; ++t) {
    const double* qt = q + (t * H + h) * DK;
    const double* kt = k + (t * H + h) * DK;
    const double* vt = v + (t * H + h) * DV;
    const double* gt = g + (t * H + h) * DK;
    const double bt = beta[t * H + h];
    double* ot = o + (t * H + h) * DV;

    /* decay: S <- Diag(exp(g_t)) S  (row i scaled by alpha_i) */
    for (int64_t i = 0; i < DK; ++i) {
      const double a = exp(gt[i]);
      double* Si = S + i * DV;
      for (int64_t j = j0; j < j1; ++j) Si[j] *= a;
    }
    /* error of the decayed memory: e = v - S^T k */
    for (int64_t j = j0; j < j1; ++j) e[j] = vt[j];
    for (int64_t i = 0; i < DK; ++i) {
      const double ki = kt[i];
      const double* Si = S + i * DV;
      for (int64_t j = j0; j < j1; ++j) e[j] -= Si[j] * ki;
    }
    /* rank-1 write: S <- S + beta k e^T */
    for (int64_t i = 0; i < DK; ++i) {
      const double c = bt * kt[i];
      double* Si = S + i * DV;
      for (int64_t j = j0; j < j1; ++j) Si[j] += c * e[j];
    }
    /* readout after the update: o = scale * S^T q */
    for (int64_t j = j0; j < j1; ++j) ot[j] = 0.0;
    for (int64_t i = 0; i < DK; ++i) {
      const double qi = qt[i];
      const double* Si = S + i * DV;
      for (int64_t j = j0; j < j1; ++j) ot[j] += Si[j] * qi;
    }
    for (int64_t j = j0; j < j1; ++j) ot[j] *= scale;
  }
  if (S_out)
    for (int64_t i = 0; i < DK; ++i)
      for (int64_t j = j0; j < j1; ++j) S_out[(n * H + h) * sdim + i * DV + j] = S[i * DV + j];
}

int kda_oracle_fwd(const double* q, const double* k, const double* v, const double* g,
                   const double* beta, double scale, const double* S0, double* S_out, double* o,
                   const int64_t* seq_start, const int64_t* seq_len, int64_t N, int64_t H,
                   int64_t DK, int64_t DV, const int64_t* heads, int64_t nh, int64_t col_block,
                   int nthreads) {
  if (check_sizes(N, H, DK, DV, seq_len)) return -1;
  const int64_t nheads = heads ? nh : H;
  for (int64_t x = 0; heads && x < nh; ++x)
    if (heads[x] < 0 || heads[x] >= H) return -1;
  const int64_t cb = (col_block > 0 && col_block < DV) ? col_block : DV;
  const int64_t ncb = (DV + cb - 1) / cb;
  const int64_t ntask = N * nheads * ncb;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)(DK * DV));
    double* e = (double*)malloc(sizeof(double) * (size_t)DV);
    if (!S || !e) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < ntask; ++task) {
        const int64_t n = task / (nheads * ncb);
        const int64_t hx = (task / ncb) % nheads;
        const int64_t h = heads ? heads[hx] : hx;
        const int64_t j0 = (task % ncb) * cb;
        const int64_t j1 = j0 + cb < DV ? j0 + cb : DV;
        run_task(q, k, v, g, beta, scale, S0, S_out, o, seq_start[n], seq_len[n], n, h, H, DK,
                 DV, j0, j1, S, e);
      }
    }
    free(S);
    free(e);
  }
  return failed ? -2 : 0;
}

/* The update with the bracketed transition matrix formed explicitly:
 *   A_t = Diag(alpha_t) - beta_t k_t (k_t ⊙ alpha_t)^T     (DK x DK)
 *   S_t = A_t S_{t-1} + beta_t k_t v_t^T,   o_t = scale * S_t^T q_t.
 * Same arguments and layout as kda_oracle_fwd (all heads, single thread). */
int kda_oracle_fwd_literal(const double* q, const double* k, const double* v, const double* g,
                           const double* beta, double scale, const double* S0, double* S_out,
                           double* o, const int64_t* seq_start, const int64_t* seq_len, int64_t N,
                           int64_t H, int64_t DK, int64_t DV) {
  if (check_sizes(N, H, DK, DV, seq_len)) return -1;
  const int64_t sdim = DK * DV;
  double* S = (double*)malloc(sizeof(double) * (size_t)sdim);
  double* Sn = (double*)malloc(sizeof(double) * (size_t)sdim);
  double* A = (double*)malloc(sizeof(double) * (size_t)(DK * DK));
  double* alpha = (double*)malloc(sizeof(double) * (size_t)DK);
  if (!S || !Sn || !A || !alpha) {
    free(S); free(Sn); free(A); free(alpha);
    return -2;
  }
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t h = 0; h < H; ++h) {
      if (S0) memcpy(S, S0 + (n * H + h) * sdim, sizeof(double) * sdim);
      else memset(S, 0, sizeof(double) * sdim);
      for (int64_t t = seq_start[n]; t < seq_start[n] + seq_len[n]; ++t) {
        const double* qt = q + (t * H + h) * DK;
        const double* kt = k + (t * H + h) * DK;
        const double* vt = v + (t * H + h) * DV;
        const double* gt = g + (t * H + h) * DK;
        const double bt = beta[t * H + h];
        double* ot = o + (t * H + h) * DV;
        for (int64_t i = 0; i < DK; ++i) alpha[i] = exp(gt[i]);
        for (int64_t r = 0; r < DK; ++r)
          for (int64_t c = 0; c < DK; ++c)
            A[r * DK + c] = (r == c ? alpha[r] : 0.0) - bt * kt[r] * (kt[c] * alpha[c]);
        for (int64_t r = 0; r < DK; ++r)
          for (int64_t j = 0; j < DV; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < DK; ++c) acc += A[r * DK + c] * S[c * DV + j];
            Sn[r * DV + j] = acc + bt * kt[r] * vt[j];
          }
        memcpy(S, Sn, sizeof(double) * sdim);
        for (int64_t j = 0; j < DV; ++j) {
          double acc = 0.0;
          for (int64_t i = 0; i < DK; ++i) acc += S[i * DV + j] * qt[i];
          ot[j] = scale * acc;
        }
      }
      if (S_out) memcpy(S_out + (n * H + h) * sdim, S, sizeof(double) * sdim);
    }
  }
  free(S); free(Sn); free(A); free(alpha);
  return 0;
}

/*
 * Gated DeltaNet (scalar gate), the special case KDA generalises:
 *   alpha_t = exp(g_t)            ONE decay per token and head
 *   S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = scale * S_t^T q_t
 *       [core.today "Kimi Linear 특집", ch.4 혁신 1 (GDN forgets the whole state
 *        with one scalar; KDA makes it a per-channel vector); hnts03 "논문 리뷰:
 *        Kimi Delta Attention", section "Kimi Delta Attention" (previous state times
 *        a scalar decay)]
 * The printed KDA update with Diag(alpha_t) = alpha_t I is exactly this form.
 * Evaluated as: S~ = alpha S (every entry scaled by the same number);
 * e = v - S~^T k; S = S~ + beta k e^T; o = scale S^T q.
 * Layout as kda_oracle_fwd except g: [rows][H] (one gate per token and head).
 * Every (sequence, head) pair is an independent task; nthreads > 0 caps the
 * OpenMP threads.
 */
int gdn_oracle_fwd(const double* q, const double* k, const double* v, const double* g,
                   const double* beta, double scale, const double* S0, double* S_out, double* o,
                   const int64_t* seq_start, const int64_t* seq_len, int64_t N, int64_t H,
                   int64_t DK, int64_t DV, int nthreads) {
  if (check_sizes(N, H, DK, DV, seq_len)) return -1;
  const int64_t sdim = DK * DV;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)sdim);
    double* e = (double*)malloc(sizeof(double) * (size_t)DV);
    if (!S || !e) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < N * H; ++task) {
        const int64_t n = task / H, h = task % H;
        if (S0) memcpy(S, S0 + (n * H + h) * sdim, sizeof(double) * (size_t)sdim);
        else memset(S, 0, sizeof(double) * (size_t)sdim);
        for (int64_t t = seq_start[n]; t < seq_start[n] + seq_len[n]; ++t) {
          const double* qt = q + (t * H + h) * DK;
          const double* kt = k + (t * H + h) * DK;
          const double* vt = v + (t * H + h) * DV;
          const double alpha = exp(g[t * H + h]);
          const double bt = beta[t * H + h];
          double* ot = o + (t * H + h) * DV;
          for (int64_t x = 0; x < sdim; ++x) S[x] *= alpha;
          for (int64_t j = 0; j < DV; ++j) {
            double acc = vt[j];
            for (int64_t i = 0; i < DK; ++i) acc -= S[i * DV + j] * kt[i];
            e[j] = acc;
          }
          for (int64_t i = 0; i < DK; ++i)
            for (int64_t j = 0; j < DV; ++j) S[i * DV + j] += bt * kt[i] * e[j];
          for (int64_t j = 0; j < DV; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < DK; ++i) acc += S[i * DV + j] * qt[i];
            ot[j] = scale * acc;
          }
        }
        if (S_out) memcpy(S_out + (n * H + h) * sdim, S, sizeof(double) * (size_t)sdim);
      }
    }
    free(S);
    free(e);
  }
  return failed ? -2 : 0;
}

/*
 * Backward pass of the KDA recurrence (reverse-mode gradient), fp64, token by
 * token.  For a scalar loss with upstream gradients dO = dL/do_t (same layout as
 * o) and dS_T = dL/dS_final (or NULL = zero), it returns dL/dq, dL/dk, dL/dv,
 * dL/dg, dL/dbeta and dL/dS0 (dS0 may be NULL when not wanted).
 *
 * It differentiates the decay-then-delta evaluation of kda_oracle_fwd step by
 * step, in reverse token order [core.today "Kimi Linear 특집", ch.4 혁신 2,
 * state-update equation; ch.2 readout]:
 *   S~ = Diag(a) S_prev,  a = exp(g);  e = v - S~^T k;  S = S~ + beta k e^T;  o = scale S^T q
 * With dS the gradient arriving at S (from later tokens) the local rules are
 *   dS += scale q do^T;          dq = scale S do
 *   de = beta dS^T k;            dbeta = k^T dS e;       dk  = beta dS e
 *   dS~ = dS - k de^T;           dv = de;                dk -= S~ de
 *   dg_i = a_i sum_j dS~_ij Sprev_ij;                    dS_prev = Diag(a) dS~
 * The forward states of each (sequence, head) are recomputed and kept in full
 * (len + 1 states), so memory is O(len * DK * DV) per running task.
 */
int kda_oracle_bwd(const double* q, const double* k, const double* v, const double* g,
                   const double* beta, double scale, const double* S0, const double* dO,
                   const double* dST, double* dq, double* dk, double* dv, double* dg,
                   double* dbeta, double* dS0, const int64_t* seq_start, const int64_t* seq_len,
                   int64_t N, int64_t H, int64_t DK, int64_t DV, int nthreads) {
  if (check_sizes(N, H, DK, DV, seq_len)) return -1;
  const int64_t sdim = DK * DV;
  int64_t Lmax = 0;
  for (int64_t n = 0; n < N; ++n) Lmax = seq_len[n] > Lmax ? seq_len[n] : Lmax;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* St = (double*)malloc(sizeof(double) * (size_t)((Lmax + 1) * sdim));  /* S_0..S_len */
    double* dS = (double*)malloc(sizeof(double) * (size_t)sdim);
    double* Sd = (double*)malloc(sizeof(double) * (size_t)sdim);                 /* S~ */
    double* e = (double*)malloc(sizeof(double) * (size_t)DV);
    double* de = (double*)malloc(sizeof(double) * (size_t)DV);
    double* a = (double*)malloc(sizeof(double) * (size_t)DK);
    if (!St || !dS || !Sd || !e || !de || !a) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < N * H; ++task) {
        const int64_t n = task / H, h = task % H;
        const int64_t t0 = seq_start[n], len = seq_len[n];
        /* forward, keeping every state */
        if (S0) memcpy(St, S0 + (n * H + h) * sdim, sizeof(double) * (size_t)sdim);
        else memset(St, 0, sizeof(double) * (size_t)sdim);
        for (int64_t s = 0; s < len; ++s) {
          const int64_t t = t0 + s;
          const double* kt = k + (t * H + h) * DK;
          const double* vt = v + (t * H + h) * DV;
          const double* gt = g + (t * H + h) * DK;
          const double bt = beta[t * H + h];
          const double* Sp = St + s * sdim;
          double* Sn = St + (s + 1) * sdim;
          for (int64_t i = 0; i < DK; ++i) {
            const double ai = exp(gt[i]);
            for (int64_t j = 0; j < DV; ++j) Sn[i * DV + j] = ai * Sp[i * DV + j];
          }
          for (int64_t j = 0; j < DV; ++j) {
            double acc = vt[j];
            for (int64_t i = 0; i < DK; ++i) acc -= Sn[i * DV + j] * kt[i];
            e[j] = acc;
          }
          for (int64_t i = 0; i < DK; ++i)
            for (int64_t j = 0; j < DV; ++j) Sn[i * DV + j] += bt * kt[i] * e[j];
        }
        /* backward */
        if (dST) memcpy(dS, dST + (n * H + h) * sdim, sizeof(double) * (size_t)sdim);
        else memset(dS, 0, sizeof(double) * (size_t)sdim);
        for (int64_t s = len - 1; s >= 0; --s) {
          const int64_t t = t0 + s;
          const double* qt = q + (t * H + h) * DK;
          const double* kt = k + (t * H + h) * DK;
          const double* vt = v + (t * H + h) * DV;
          const double* gt = g + (t * H + h) * DK;
          const double* dot = dO + (t * H + h) * DV;
          const double bt = beta[t * H + h];
          const double* Sp = St + s * sdim;        /* S_{t-1} */
          const double* Sc = St + (s + 1) * sdim;  /* S_t */
          double* dqt = dq + (t * H + h) * DK;
          double* dkt = dk + (t * H + h) * DK;
          double* dvt = dv + (t * H + h) * DV;
          double* dgt = dg + (t * H + h) * DK;
          for (int64_t i = 0; i < DK; ++i) a[i] = exp(gt[i]);
          /* readout o = scale S^T q */
          for (int64_t i = 0; i < DK; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < DV; ++j) {
              dS[i * DV + j] += scale * qt[i] * dot[j];
              acc += Sc[i * DV + j] * dot[j];
            }
            dqt[i] = scale * acc;
          }
          /* S~ and e of the forward step */
          for (int64_t i = 0; i < DK; ++i)
            for (int64_t j = 0; j < DV; ++j) Sd[i * DV + j] = a[i] * Sp[i * DV + j];
          for (int64_t j = 0; j < DV; ++j) {
            double acc = vt[j];
            for (int64_t i = 0; i < DK; ++i) acc -= Sd[i * DV + j] * kt[i];
            e[j] = acc;
          }
          /* write S = S~ + beta k e^T */
          double db = 0.0;
          for (int64_t j = 0; j < DV; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < DK; ++i) acc += dS[i * DV + j] * kt[i];
            de[j] = bt * acc;
            db += acc * e[j];
          }
          dbeta[t * H + h] = db;
          for (int64_t i = 0; i < DK; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < DV; ++j) acc += dS[i * DV + j] * e[j];
            dkt[i] = bt * acc;
          }
          /* error e = v - S~^T k */
          for (int64_t j = 0; j < DV; ++j) dvt[j] = de[j];
          for (int64_t i = 0; i < DK; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < DV; ++j) {
              dS[i * DV + j] -= kt[i] * de[j];   /* dS now holds dS~ */
              acc += Sd[i * DV + j] * de[j];
            }
            dkt[i] -= acc;
          }
          /* decay S~ = Diag(a) S_prev */
          for (int64_t i = 0; i < DK; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < DV; ++j) {
              acc += dS[i * DV + j] * Sp[i * DV + j];
              dS[i * DV + j] *= a[i];
            }
            dgt[i] = a[i] * acc;
          }
        }
        if (dS0) memcpy(dS0 + (n * H + h) * sdim, dS, sizeof(double) * (size_t)sdim);
      }
    }
    free(St); free(dS); free(Sd); free(e); free(de); free(a);
  }
  return failed ? -2 : 0;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
