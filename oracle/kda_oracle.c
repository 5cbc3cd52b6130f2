/*
 * Oracle for the Kimi Delta Attention (KDA) recurrence -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, sequential fp64 definition that the GPU path is
 * checked against. It shares no code with the GPU library. Only the tests, the
 * smoke check and the bench's CPU-baseline leg may load it.
 *
 * What it computes, per sequence n and head h, token by token:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T ,   o_t = S_t^T q_t
 *
 * with S in R^{dk x dv} (row i = key channel, column j = value channel),
 * alpha_t = exp(log_alpha_t) one decay per key channel, beta_t one scalar per
 * (token, head). Sources:
 *   - "From GPT-2 to Kimi K3" digest, section "DeltaNet -- 유한한 캐시의 덮어쓰기":
 *     the delta rule reads what the current key retrieves, subtracts it from the
 *     new value and writes the difference back along the key.
 *   - same digest, section "Gated DeltaNet -- 망각을 더하다": a data-dependent
 *     decay alpha in [0,1] on the previous state; alpha = 1 is the pure delta rule.
 *   - same digest, section "Kimi Linear (KDA) -- 채널별 세밀한 게이팅", and the
 *     GeekNews "Kimi Linear" summary, section "Kimi Delta Attention의 세밀한 메모리
 *     제어": the scalar decay becomes a per-channel diagonal Diag(alpha).
 *   - GeekNews "Kimi Linear" summary, section "선형 어텐션에서 Gated DeltaNet까지":
 *     the rank-one update is a generalised Householder transform.
 *
 * The rank-one form used below is the same map written without the dk x dk
 * matrix:  S' = Diag(alpha) S ;  e = v - S'^T k ;  S = S' + beta k e^T ;  o = S^T q.
 * (Expand (I - beta k k^T) S' + beta k v^T = S' + beta k (v - S'^T k)^T.)
 * The output reads the state after the update of its own token.
 *
 * Value columns of S evolve independently (column j only ever reads column j),
 * so the work is split over (sequence, head, column block) with OpenMP; no
 * floating-point operation is reordered by the split, so the result is bitwise
 * identical for any thread count.
 *
 * Layouts (all row-major, contiguous):
 *   q, k, log_alpha : [T_total][H][dk]   float32 (carries bf16 or fp32 values exactly)
 *   v               : [T_total][H][dv]   float32
 *   beta            : [T_total][H]       float32
 *   seq_starts      : [num_seqs + 1]     int64, sequence n = rows [seq_starts[n], seq_starts[n+1])
 *   initial_state   : [num_seqs][H][dk][dv] float64, or NULL for zeros
 * Outputs are written only for the selected heads and the value columns
 * [col_begin, col_end), compactly:
 *   o_sel     : [T_total][n_heads_sel][ncols]          float64 (may be NULL)
 *   final_sel : [num_seqs][n_heads_sel][dk][ncols]     float64 (may be NULL)
 * heads == NULL selects all H heads in order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_COL_BLOCK 16

int kda_oracle_abi_version(void) { return 4; }

/*
 * Optional prologue on the raw projections, as the Kimi Linear layer applies it
 * before the recurrence (GeekNews "Kimi Linear" summary, section "Kimi Linear 모델
 * 구성": q and k get an L2 normalisation for eigenvalue stability; the per-channel
 * decay gate uses a GDN/Mamba-like decay function of a low-rank projection).
 * Readings where the page leaves a step open:
 *   ORACLE_NORM_QK  q_t <- q_t / sqrt(sum_i q_ti^2 + eps), the same for k_t
 *   ORACLE_GATE_PRE log_alpha holds a pre-activation a: log alpha = -softplus(a)
 *   ORACLE_BETA_PRE beta holds a pre-activation b: beta = sigmoid(b)
 */
#define ORACLE_NORM_QK 1
#define ORACLE_GATE_PRE 2
#define ORACLE_BETA_PRE 4

static double softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }
static double sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  const double e = exp(x);
  return e / (1.0 + e);
}

/* One token's inputs in fp64 after the prologue: kd, qd = key and query,
 * alpha = per-channel decay, *b = beta. */
static void token_inputs(const float *k, const float *q, const float *log_alpha, float beta, int dk, int flags,
                         double qk_eps, double *kd, double *qd, double *alpha, double *b) {
  double sk = 0.0, sq = 0.0;
  for (int i = 0; i < dk; ++i) {
    kd[i] = (double)k[i];
    qd[i] = (double)q[i];
    sk += kd[i] * kd[i];
    sq += qd[i] * qd[i];
  }
  if (flags & ORACLE_NORM_QK) {
    const double ik = 1.0 / sqrt(sk + qk_eps), iq = 1.0 / sqrt(sq + qk_eps);
    for (int i = 0; i < dk; ++i) {
      kd[i] *= ik;
      qd[i] *= iq;
    }
  }
  for (int i = 0; i < dk; ++i) {
    const double la = (flags & ORACLE_GATE_PRE) ? -softplus((double)log_alpha[i]) : (double)log_alpha[i];
    alpha[i] = exp(la);
  }
  *b = (flags & ORACLE_BETA_PRE) ? sigmoid((double)beta) : (double)beta;
}

int kda_oracle_forward_ex(const float *q, const float *k, const float *v,
                          const float *log_alpha, const float *beta,
                          const double *initial_state, const int64_t *seq_starts,
                          int num_seqs, int H, int dk, int dv, const int *heads,
                          int n_heads_sel, int col_begin, int col_end,
                          double *o_sel, double *final_sel, int num_threads, int flags, double qk_eps) {
  if (!q || !k || !v || !log_alpha || !beta || !seq_starts) return -1;
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (col_begin < 0 || col_end > dv || col_begin > col_end) return -1;
  if (heads == NULL) n_heads_sel = H;
  if (n_heads_sel <= 0) return -1;
  for (int n = 0; n < num_seqs; ++n)
    if (seq_starts[n + 1] < seq_starts[n]) return -1;
  const int ncols = col_end - col_begin;
  if (ncols == 0 || num_seqs == 0) return 0;
  const int nblk = (ncols + ORACLE_COL_BLOCK - 1) / ORACLE_COL_BLOCK;
  const long long ntask = (long long)num_seqs * n_heads_sel * nblk;

#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (long long task = 0; task < ntask; ++task) {
    const int blk = (int)(task % nblk);
    const int hs = (int)((task / nblk) % n_heads_sel);
    const int n = (int)(task / ((long long)nblk * n_heads_sel));
    const int h = heads ? heads[hs] : hs;
    const int c0 = col_begin + blk * ORACLE_COL_BLOCK;
    const int c1 = (c0 + ORACLE_COL_BLOCK < col_end) ? c0 + ORACLE_COL_BLOCK : col_end;
    const int w = c1 - c0;

    double *S = (double *)malloc(sizeof(double) * (size_t)dk * w);
    double *tok = (double *)malloc(sizeof(double) * (size_t)dk * 3);
    double *kt = tok, *qt = tok + dk, *alpha = tok + 2 * dk;
    double e[ORACLE_COL_BLOCK];

    /* S_0: the given initial state, or zeros */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < w; ++j)
        S[(size_t)i * w + j] =
            initial_state
                ? initial_state[(((size_t)n * H + h) * dk + i) * dv + (c0 + j)]
                : 0.0;

    for (int64_t t = seq_starts[n]; t < seq_starts[n + 1]; ++t) {
      const size_t rk = ((size_t)t * H + h) * dk;
      const size_t rv = ((size_t)t * H + h) * dv;
      double b;
      token_inputs(k + rk, q + rk, log_alpha + rk, beta[(size_t)t * H + h], dk, flags, qk_eps, kt, qt, alpha, &b);
      /* S' = Diag(alpha_t) S_{t-1}: row i scaled by alpha_i */
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < w; ++j) S[(size_t)i * w + j] *= alpha[i];
      /* e = v_t - S'^T k_t: what the key reads back, subtracted from the new value */
      for (int j = 0; j < w; ++j) e[j] = 0.0;
      for (int i = 0; i < dk; ++i) {
        const double ki = kt[i];
        for (int j = 0; j < w; ++j) e[j] += ki * S[(size_t)i * w + j];
      }
      for (int j = 0; j < w; ++j) e[j] = (double)v[rv + c0 + j] - e[j];
      /* S_t = S' + beta_t k_t e^T: the difference written back along the key */
      for (int i = 0; i < dk; ++i) {
        const double bki = b * kt[i];
        for (int j = 0; j < w; ++j) S[(size_t)i * w + j] += bki * e[j];
      }
      /* o_t = S_t^T q_t */
      if (o_sel) {
        double acc[ORACLE_COL_BLOCK];
        for (int j = 0; j < w; ++j) acc[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
          const double qi = qt[i];
          for (int j = 0; j < w; ++j) acc[j] += qi * S[(size_t)i * w + j];
        }
        double *orow = o_sel + ((size_t)t * n_heads_sel + hs) * ncols + (c0 - col_begin);
        for (int j = 0; j < w; ++j) orow[j] = acc[j];
      }
    }

    if (final_sel)
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < w; ++j)
          final_sel[(((size_t)n * n_heads_sel + hs) * dk + i) * ncols + (c0 - col_begin) + j] =
              S[(size_t)i * w + j];
    free(tok);
    free(S);
  }
  return 0;
}

int kda_oracle_forward(const float *q, const float *k, const float *v,
                       const float *log_alpha, const float *beta,
                       const double *initial_state, const int64_t *seq_starts,
                       int num_seqs, int H, int dk, int dv, const int *heads,
                       int n_heads_sel, int col_begin, int col_end,
                       double *o_sel, double *final_sel, int num_threads) {
  return kda_oracle_forward_ex(q, k, v, log_alpha, beta, initial_state, seq_starts, num_seqs, H, dk, dv, heads,
                               n_heads_sel, col_begin, col_end, o_sel, final_sel, num_threads, 0, 0.0);
}

/*
 * One decode step for a batch of independent (sequence, head) states, in place:
 * the same recurrence for a single token. state: [N][H][dk][dv] float64 in/out;
 * q, k, log_alpha: [N][H][dk]; v: [N][H][dv]; beta: [N][H]; o: [N][H][dv] float64.
 */
int kda_oracle_decode_step_ex(const float *q, const float *k, const float *v,
                              const float *log_alpha, const float *beta,
                              double *state, double *o, int N, int H, int dk, int dv,
                              int num_threads, int flags, double qk_eps) {
  if (!q || !k || !v || !log_alpha || !beta || !state || !o) return -1;
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  const long long ntask = (long long)N * H;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(static)
#endif
  for (long long nh = 0; nh < ntask; ++nh) {
    double *S = state + (size_t)nh * dk * dv;
    const float *vv = v + (size_t)nh * dv;
    double *oo = o + (size_t)nh * dv;
    double *tok = (double *)malloc(sizeof(double) * (size_t)dk * 3);
    double *kt = tok, *qt = tok + dk, *alpha = tok + 2 * dk;
    double b;
    token_inputs(k + (size_t)nh * dk, q + (size_t)nh * dk, log_alpha + (size_t)nh * dk, beta[nh], dk, flags, qk_eps,
                 kt, qt, alpha, &b);
    for (int i = 0; i < dk; ++i) {
      const double a = alpha[i];
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
    }
    for (int j = 0; j < dv; ++j) {
      double r = 0.0;
      for (int i = 0; i < dk; ++i) r += kt[i] * S[(size_t)i * dv + j];
      const double ej = (double)vv[j] - r;
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) {
        S[(size_t)i * dv + j] += b * kt[i] * ej;
        acc += qt[i] * S[(size_t)i * dv + j];
      }
      oo[j] = acc;
    }
    free(tok);
  }
  return 0;
}

int kda_oracle_decode_step(const float *q, const float *k, const float *v,
                           const float *log_alpha, const float *beta,
                           double *state, double *o, int N, int H, int dk, int dv,
                           int num_threads) {
  return kda_oracle_decode_step_ex(q, k, v, log_alpha, beta, state, o, N, H, dk, dv, num_threads, 0, 0.0);
}

/*
 * Reverse-mode derivative of the recurrence above (the plain recurrence, no
 * prologue), for training: given the cotangents d_o of every output and d_final
 * of every final state, the gradient of
 *
 *     L = sum_t <o_t, d_o_t> + sum_n <S_final[n], d_final[n]>
 *
 * with respect to q, k, v, log_alpha, beta and the initial state. The pages present
 * the chunked form as the device that makes KDA efficient to train ("From GPT-2 to
 * Kimi K3" digest, section "DeltaNet 병렬화 -- 청크 단위 학습"; GeekNews "Kimi Linear" summary,
 * section "청크 단위 병렬 알고리듬"), so its gradients are the derivatives of this map.
 *
 * One token, forward (as above):  S' = Diag(a) S ;  e = v - S'^T k ;
 * S_t = S' + b k e^T ;  o_t = S_t^T q.  Backward, with L_t the gradient of L with
 * respect to S_t (everything that reads S_t, the output included):
 *     L_t   += q do^T                          (o_t = S_t^T q)
 *     dq     = S_t do
 *     r      = L_t^T k ;  de = b r ;  db = r . e ;  dk = b L_t e
 *     dS'    = L_t - k de^T ;  dk -= S' de ;  dv = de
 *     dlog_a = a o (rowsum of dS' o S)          (S' = Diag(a) S, a = exp(log_a))
 *     L_{t-1} = Diag(a) dS'
 *
 * The states are recomputed forward from checkpoints every ORACLE_BWD_SEG tokens,
 * with the same operations as the forward pass, so memory stays bounded. Work is
 * split over (sequence, head); the gradients of q, k, log_alpha and beta sum over
 * all value columns, so columns are not split here.
 *
 * Layouts as kda_oracle_forward, all heads and columns:
 *   d_o        [T_total][H][dv] float32, or NULL for zeros
 *   d_final    [num_seqs][H][dk][dv] float64, or NULL for zeros
 *   dq, dk_out, dlog_alpha [T_total][H][dk]; dv_out [T_total][H][dv];
 *   dbeta [T_total][H]; d_initial [num_seqs][H][dk][dv] (NULL: not written),
 * all float64 and written in full for every token of every sequence.
 */
#define ORACLE_BWD_SEG 64

static void fwd_token(double *S, const double *kt, const float *v, const double *alpha, double b, int dk, int dv) {
  double e[512];
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[i];
  for (int j = 0; j < dv; ++j) e[j] = 0.0;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) e[j] += kt[i] * S[(size_t)i * dv + j];
  for (int j = 0; j < dv; ++j) e[j] = (double)v[j] - e[j];
  for (int i = 0; i < dk; ++i) {
    const double bk = b * kt[i];
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bk * e[j];
  }
}

int kda_oracle_backward(const float *q, const float *k, const float *v, const float *log_alpha,
                        const float *beta, const double *initial_state, const int64_t *seq_starts,
                        int num_seqs, int H, int dk, int dv, const float *d_o, const double *d_final,
                        double *dq, double *dk_out, double *dv_out, double *dlog_alpha, double *dbeta,
                        double *d_initial, int num_threads) {
  if (!q || !k || !v || !log_alpha || !beta || !seq_starts) return -1;
  if (!dq || !dk_out || !dv_out || !dlog_alpha || !dbeta) return -1;
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || dv > 512) return -1;
  for (int n = 0; n < num_seqs; ++n)
    if (seq_starts[n + 1] < seq_starts[n]) return -1;
  const long long ntask = (long long)num_seqs * H;
  const size_t dd = (size_t)dk * dv;

#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (long long task = 0; task < ntask; ++task) {
    const int h = (int)(task % H);
    const int n = (int)(task / H);
    const int64_t t0 = seq_starts[n], t1 = seq_starts[n + 1];
    const int64_t len = t1 - t0;
    const int64_t nseg = (len + ORACLE_BWD_SEG - 1) / ORACLE_BWD_SEG;
    /* ck[m] = state before token t0 + m * SEG; seg[s] = state before token s of the segment */
    double *ck = (double *)malloc(sizeof(double) * dd * (size_t)(nseg > 0 ? nseg : 1));
    double *seg = (double *)malloc(sizeof(double) * dd * (ORACLE_BWD_SEG + 1));
    double *L = (double *)malloc(sizeof(double) * dd);
    double *dSp = (double *)malloc(sizeof(double) * dd);
    double *tok = (double *)malloc(sizeof(double) * (size_t)dk * 3);
    double *kt = tok, *qt = tok + dk, *alpha = tok + 2 * dk;
    double e[512], r[512], de[512], dov[512];

    double *S = seg;
    for (size_t x = 0; x < dd; ++x) S[x] = initial_state ? initial_state[((size_t)n * H + h) * dd + x] : 0.0;
    for (int64_t m = 0; m < nseg; ++m) {
      memcpy(ck + (size_t)m * dd, S, sizeof(double) * dd);
      const int64_t a0 = t0 + m * ORACLE_BWD_SEG;
      const int64_t a1 = (a0 + ORACLE_BWD_SEG < t1) ? a0 + ORACLE_BWD_SEG : t1;
      for (int64_t t = a0; t < a1; ++t) {
        const size_t rk = ((size_t)t * H + h) * dk;
        double b;
        token_inputs(k + rk, q + rk, log_alpha + rk, beta[(size_t)t * H + h], dk, 0, 0.0, kt, qt, alpha, &b);
        fwd_token(S, kt, v + ((size_t)t * H + h) * dv, alpha, b, dk, dv);
      }
    }
    /* L = gradient with respect to the final state */
    for (size_t x = 0; x < dd; ++x) L[x] = d_final ? d_final[((size_t)n * H + h) * dd + x] : 0.0;

    for (int64_t m = nseg - 1; m >= 0; --m) {
      const int64_t a0 = t0 + m * ORACLE_BWD_SEG;
      const int64_t a1 = (a0 + ORACLE_BWD_SEG < t1) ? a0 + ORACLE_BWD_SEG : t1;
      /* states before every token of the segment, and after its last one */
      memcpy(seg, ck + (size_t)m * dd, sizeof(double) * dd);
      for (int64_t t = a0; t < a1; ++t) {
        const size_t rk = ((size_t)t * H + h) * dk;
        double b;
        token_inputs(k + rk, q + rk, log_alpha + rk, beta[(size_t)t * H + h], dk, 0, 0.0, kt, qt, alpha, &b);
        double *nxt = seg + (size_t)(t - a0 + 1) * dd;
        memcpy(nxt, seg + (size_t)(t - a0) * dd, sizeof(double) * dd);
        fwd_token(nxt, kt, v + ((size_t)t * H + h) * dv, alpha, b, dk, dv);
      }
      for (int64_t t = a1 - 1; t >= a0; --t) {
        const size_t rk = ((size_t)t * H + h) * dk;
        const size_t rv = ((size_t)t * H + h) * dv;
        double b;
        token_inputs(k + rk, q + rk, log_alpha + rk, beta[(size_t)t * H + h], dk, 0, 0.0, kt, qt, alpha, &b);
        const double *Sprev = seg + (size_t)(t - a0) * dd; /* S_{t-1} */
        const double *St = seg + (size_t)(t - a0 + 1) * dd; /* S_t */
        for (int j = 0; j < dv; ++j) dov[j] = d_o ? (double)d_o[rv + j] : 0.0;
        /* e = v - (Diag(a) S_{t-1})^T k, as in the forward step */
        for (int j = 0; j < dv; ++j) e[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) e[j] += kt[i] * (Sprev[(size_t)i * dv + j] * alpha[i]);
        for (int j = 0; j < dv; ++j) e[j] = (double)v[rv + j] - e[j];
        /* the output reads S_t along q */
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] += qt[i] * dov[j];
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += St[(size_t)i * dv + j] * dov[j];
          dq[rk + i] = acc;
        }
        /* S_t = S' + b k e^T */
        for (int j = 0; j < dv; ++j) r[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) r[j] += kt[i] * L[(size_t)i * dv + j];
        double db = 0.0;
        for (int j = 0; j < dv; ++j) {
          de[j] = b * r[j];
          db += r[j] * e[j];
        }
        dbeta[(size_t)t * H + h] = db;
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += L[(size_t)i * dv + j] * e[j];
          dk_out[rk + i] = b * acc;
        }
        /* e = v - S'^T k: dS' = L - k de^T, dk -= S' de, dv = de */
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) dSp[(size_t)i * dv + j] = L[(size_t)i * dv + j] - kt[i] * de[j];
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += (Sprev[(size_t)i * dv + j] * alpha[i]) * de[j];
          dk_out[rk + i] -= acc;
        }
        for (int j = 0; j < dv; ++j) dv_out[rv + j] = de[j];
        /* S' = Diag(a) S_{t-1} */
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += dSp[(size_t)i * dv + j] * Sprev[(size_t)i * dv + j];
          dlog_alpha[rk + i] = alpha[i] * acc;
          for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] = alpha[i] * dSp[(size_t)i * dv + j];
        }
      }
    }
    if (d_initial)
      for (size_t x = 0; x < dd; ++x) d_initial[((size_t)n * H + h) * dd + x] = L[x];
    free(tok);
    free(dSp);
    free(L);
    free(seg);
    free(ck);
  }
  return 0;
}

/*
 * General diagonal-plus-low-rank (DPLR) recurrence -- the comparison point the
 * GeekNews "Kimi Linear" summary measures KDA against (section "일반 DPLR보다 줄어든
 * 연산량": KDA and a general DPLR transition both allow fine-grained decay; KDA ties
 * the transition's two low-rank vectors to the key). The pages do not write the
 * general form out; the reading taken here is the rank-one diagonal-plus-low-rank
 * transition with two free vectors a_t, b_t, and a separate key-value write:
 *
 *     S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T ,   o_t = S_t^T q_t
 *
 * KDA is the case a_t = -beta_t k_t, b_t = alpha_t * k_t (element-wise), with the
 * written key beta_t k_t.
 *
 * Rank-one form used below (no dk x dk matrix is formed):
 *     w = S_{t-1}^T b_t ;  S_t = Diag(alpha_t) S_{t-1} + a_t w^T + k_t v_t^T ;  o_t = S_t^T q_t
 * w reads the state before this token's decay. Columns of S evolve independently,
 * so the same (sequence, head, column block) split as above is exact.
 *
 * Layouts as kda_oracle_forward_ex, with a and b laid out like k.
 */
int dplr_oracle_forward(const float *q, const float *k, const float *v, const float *a, const float *b,
                        const float *log_alpha, const double *initial_state, const int64_t *seq_starts,
                        int num_seqs, int H, int dk, int dv, const int *heads, int n_heads_sel, int col_begin,
                        int col_end, double *o_sel, double *final_sel, int num_threads) {
  if (!q || !k || !v || !a || !b || !log_alpha || !seq_starts) return -1;
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (col_begin < 0 || col_end > dv || col_begin > col_end) return -1;
  if (heads == NULL) n_heads_sel = H;
  if (n_heads_sel <= 0) return -1;
  for (int n = 0; n < num_seqs; ++n)
    if (seq_starts[n + 1] < seq_starts[n]) return -1;
  const int ncols = col_end - col_begin;
  if (ncols == 0 || num_seqs == 0) return 0;
  const int nblk = (ncols + ORACLE_COL_BLOCK - 1) / ORACLE_COL_BLOCK;
  const long long ntask = (long long)num_seqs * n_heads_sel * nblk;

#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (long long task = 0; task < ntask; ++task) {
    const int blk = (int)(task % nblk);
    const int hs = (int)((task / nblk) % n_heads_sel);
    const int n = (int)(task / ((long long)nblk * n_heads_sel));
    const int h = heads ? heads[hs] : hs;
    const int c0 = col_begin + blk * ORACLE_COL_BLOCK;
    const int c1 = (c0 + ORACLE_COL_BLOCK < col_end) ? c0 + ORACLE_COL_BLOCK : col_end;
    const int w = c1 - c0;

    double *S = (double *)malloc(sizeof(double) * (size_t)dk * w);
    double wv[ORACLE_COL_BLOCK];
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < w; ++j)
        S[(size_t)i * w + j] =
            initial_state ? initial_state[(((size_t)n * H + h) * dk + i) * dv + (c0 + j)] : 0.0;

    for (int64_t t = seq_starts[n]; t < seq_starts[n + 1]; ++t) {
      const size_t rk = ((size_t)t * H + h) * dk;
      const size_t rv = ((size_t)t * H + h) * dv;
      /* w = S_{t-1}^T b_t: the low-rank read of the previous state */
      for (int j = 0; j < w; ++j) wv[j] = 0.0;
      for (int i = 0; i < dk; ++i) {
        const double bi = (double)b[rk + i];
        for (int j = 0; j < w; ++j) wv[j] += bi * S[(size_t)i * w + j];
      }
      /* S_t = Diag(alpha_t) S_{t-1} + a_t w^T + k_t v_t^T */
      for (int i = 0; i < dk; ++i) {
        const double al = exp((double)log_alpha[rk + i]);
        const double ai = (double)a[rk + i], ki = (double)k[rk + i];
        for (int j = 0; j < w; ++j)
          S[(size_t)i * w + j] = al * S[(size_t)i * w + j] + ai * wv[j] + ki * (double)v[rv + c0 + j];
      }
      /* o_t = S_t^T q_t */
      if (o_sel) {
        double acc[ORACLE_COL_BLOCK];
        for (int j = 0; j < w; ++j) acc[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
          const double qi = (double)q[rk + i];
          for (int j = 0; j < w; ++j) acc[j] += qi * S[(size_t)i * w + j];
        }
        double *orow = o_sel + ((size_t)t * n_heads_sel + hs) * ncols + (c0 - col_begin);
        for (int j = 0; j < w; ++j) orow[j] = acc[j];
      }
    }
    if (final_sel)
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < w; ++j)
          final_sel[(((size_t)n * n_heads_sel + hs) * dk + i) * ncols + (c0 - col_begin) + j] =
              S[(size_t)i * w + j];
    free(S);
  }
  return 0;
}
