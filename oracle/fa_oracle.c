/*
 * Attention oracle: plain, slow, double-precision CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or table with the HIP
 * library.
 *
 * Sources (the pages this follows):
 *  - "FlashAttention-1: eliminating IO" (deep-learning-notes ch10.2),
 *    section 10.2.1: S = Q K^T, row max m_i, l_i = sum_k exp(S_ik - m_i),
 *    P_ij = exp(S_ij - m_i) / l_i, O_i = sum_j P_ij V_j.  The page leaves the
 *    scale out of the derivation; its forward example of section 10.2.3
 *    multiplies Q K^T by 1/sqrt(d).  Here the scale is an argument.
 *  - Same page, section 10.2.2: the two-partition merge and the tile update
 *    with m~, P~, l~, m', alpha = exp(m - m'), beta = exp(m~ - m'),
 *    l' = alpha l + beta l~, O' = (alpha l O + beta P~ V) / l'.  That form
 *    (normalised O after every tile) is what oracle_tiled_fwd follows.
 *  - Same page, section 10.2.4: dV = P^T dO, dP = dO V^T,
 *    dS = P o (dP - delta), delta_i = dO_i . O_i, dQ = dS K, dK = dS^T Q,
 *    and P recomputed per tile as exp(S - m_i) / l_i.  The scale enters dQ
 *    and dK by the chain rule (S = scale * Q K^T), not dV.
 *  - Same page, section 10.2.5: FA1 loop order, K/V blocks outer and Q
 *    blocks inner, with O_i, m_i, l_i kept between outer iterations.  The
 *    tiled forward and backward here use that order.
 *
 * Causal mask: key j is visible to query i iff j <= i (square attention,
 * N_q = N_k = N).  LSE_i = m_i + ln l_i in the natural log of the scaled
 * scores.
 *
 * Bias and general masks (the explainer's V2 section: mask and bias are
 * merged into the score computation): the *_bias functions add bias_ij to the
 * scaled score, s_ij = scale q_i.k_j + bias_ij, before the softmax; a bias of
 * -inf masks the key (exp(-inf - m) = 0).  A row whose visible scores are all
 * -inf has an empty softmax: its output row is 0, its LSE is -inf (ln of an
 * empty sum) and it contributes nothing to any gradient.
 *
 * Layout: every tensor is a contiguous [B, H, N, d] array of doubles, and
 * LSE / delta are [B, H, N].  All sums are sequential double sums in index
 * order.  No blocking, fusion or reordering beyond what the definitions say.
 *
 * Parity pins: every function here is pinned by the not-gpu tests (brute
 * force, closed forms, invariants, finite differences, torch float64
 * autograd, and the tiled versions against the naive ones).
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* A tiny work pool: threads pull item indices from a shared counter.  */
/* ------------------------------------------------------------------ */
typedef void (*work_fn)(void *ctx, long item, int tid);

typedef struct {
  work_fn fn;
  void *ctx;
  long n_items;
  long next;
  int strided; /* 1: worker t takes items t, t + n, t + 2n, ... (fixed owner) */
  int n_workers;
  pthread_mutex_t lock;
} pool_t;

typedef struct {
  pool_t *pool;
  int tid;
} worker_arg_t;

static void *worker_main(void *p) {
  worker_arg_t *wa = (worker_arg_t *)p;
  pool_t *pool = wa->pool;
  if (pool->strided) {
    long item;
    for (item = wa->tid; item < pool->n_items; item += pool->n_workers)
      pool->fn(pool->ctx, item, wa->tid);
    return NULL;
  }
  for (;;) {
    long item;
    pthread_mutex_lock(&pool->lock);
    item = pool->next++;
    pthread_mutex_unlock(&pool->lock);
    if (item >= pool->n_items) break;
    pool->fn(pool->ctx, item, wa->tid);
  }
  return NULL;
}

static void run_pool_mode(work_fn fn, void *ctx, long n_items, int nthreads, int strided) {
  pool_t pool;
  pthread_t *th;
  worker_arg_t *args;
  int t;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_items) nthreads = (int)(n_items > 0 ? n_items : 1);
  pool.fn = fn;
  pool.ctx = ctx;
  pool.n_items = n_items;
  pool.next = 0;
  pool.strided = strided;
  pool.n_workers = nthreads;
  pthread_mutex_init(&pool.lock, NULL);
  th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  args = (worker_arg_t *)malloc(sizeof(worker_arg_t) * (size_t)nthreads);
  for (t = 0; t < nthreads; ++t) {
    args[t].pool = &pool;
    args[t].tid = t;
  }
  if (nthreads == 1) {
    worker_main(&args[0]);
  } else {
    for (t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, worker_main, &args[t]);
    for (t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  }
  pthread_mutex_destroy(&pool.lock);
  free(th);
  free(args);
}

static void run_pool(work_fn fn, void *ctx, long n_items, int nthreads) {
  run_pool_mode(fn, ctx, n_items, nthreads, 0);
}

static double dot(const double *a, const double *b, long d) {
  double s = 0.0;
  long c;
  for (c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/* Number of keys query i may see: all N, or i + 1 under the causal mask. */
static long visible_keys(long i, long N, int causal) { return causal ? i + 1 : N; }

/* ------------------------------------------------------------------ */
/* Forward, by definition (10.2.1), one query row at a time.           */
/* ------------------------------------------------------------------ */

/* One query row of one head: s_j = scale q.k_j (+ bias_i[j] when bias_i is
 * given), m = max s, l = sum exp(s - m), P_j = exp(s_j - m) / l,
 * o = sum_j P_j v_j, lse = m + ln l; an all -inf row gives o = 0, lse = -inf.
 * s is caller scratch of N doubles. */
static void fwd_row(const double *q_i, const double *K, const double *V, const double *bias_i,
                    long N, long d, double scale, long n_vis, double *s, double *o_i,
                    double *lse_i) {
  long j, c;
  double m = -INFINITY, l = 0.0;
  for (j = 0; j < n_vis; ++j) {
    s[j] = scale * dot(q_i, K + j * d, d);
    if (bias_i) s[j] += bias_i[j];
    if (s[j] > m) m = s[j];
  }
  for (c = 0; c < d; ++c) o_i[c] = 0.0;
  if (m == -INFINITY) { /* no visible key with a finite score */
    *lse_i = -INFINITY;
    return;
  }
  for (j = 0; j < n_vis; ++j) l += exp(s[j] - m);
  for (j = 0; j < n_vis; ++j) {
    const double p = exp(s[j] - m) / l;
    const double *v_j = V + j * d;
    for (c = 0; c < d; ++c) o_i[c] += p * v_j[c];
  }
  *lse_i = m + log(l);
  (void)N;
}

typedef struct {
  const double *q, *k, *v;
  const double *bias; /* [B, H, N, N] or NULL */
  double *o, *lse;
  long N, d, chunk, chunks_per_head;
  double scale;
  int causal;
} fwd_ctx_t;

static void fwd_item(void *p, long item, int tid) {
  fwd_ctx_t *c = (fwd_ctx_t *)p;
  const long bh = item / c->chunks_per_head;
  const long r0 = (item % c->chunks_per_head) * c->chunk;
  const long r1 = r0 + c->chunk < c->N ? r0 + c->chunk : c->N;
  const long hd = c->N * c->d;
  double *s = (double *)malloc(sizeof(double) * (size_t)c->N);
  long i;
  (void)tid;
  for (i = r0; i < r1; ++i)
    fwd_row(c->q + bh * hd + i * c->d, c->k + bh * hd, c->v + bh * hd,
            c->bias ? c->bias + (bh * c->N + i) * c->N : NULL, c->N, c->d, c->scale,
            visible_keys(i, c->N, c->causal), s, c->o + bh * hd + i * c->d,
            c->lse + bh * c->N + i);
  free(s);
}

/* Full forward over [B,H,N,d], with an optional [B,H,N,N] additive bias on the
 * scaled scores (NULL: none).  Returns 0, or -1 on bad sizes. */
int oracle_attn_fwd_bias(const double *q, const double *k, const double *v, const double *bias,
                         double *o, double *lse, long B, long H, long N, long d, double scale,
                         int causal, int nthreads) {
  fwd_ctx_t c;
  if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
  if (B * H * N == 0) return 0;
  c.q = q; c.k = k; c.v = v; c.bias = bias; c.o = o; c.lse = lse;
  c.N = N; c.d = d; c.scale = scale; c.causal = causal;
  c.chunk = 64;
  c.chunks_per_head = (N + c.chunk - 1) / c.chunk;
  run_pool(fwd_item, &c, B * H * c.chunks_per_head, nthreads);
  return 0;
}

/* Full forward over [B,H,N,d] without a bias. */
int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                    long B, long H, long N, long d, double scale, int causal, int nthreads) {
  return oracle_attn_fwd_bias(q, k, v, NULL, o, lse, B, H, N, d, scale, causal, nthreads);
}

typedef struct {
  const double *q, *k, *v;
  const long *rows;
  const double *bias; /* [n_rows, N] or NULL */
  double *o, *lse;
  long N, d;
  double scale;
  int causal;
} rows_ctx_t;

static void rows_item(void *p, long item, int tid) {
  rows_ctx_t *c = (rows_ctx_t *)p;
  const long i = c->rows[item];
  double *s = (double *)malloc(sizeof(double) * (size_t)c->N);
  (void)tid;
  fwd_row(c->q + i * c->d, c->k, c->v, c->bias ? c->bias + item * c->N : NULL, c->N, c->d,
          c->scale, visible_keys(i, c->N, c->causal), s, c->o + item * c->d, c->lse + item);
  free(s);
}

/* Selected query rows of ONE head: q, k, v are [N, d]; rows[r] in [0, N);
 * bias_rows (or NULL) is [n_rows, N], the bias of each selected row;
 * o_rows is [n_rows, d], lse_rows is [n_rows].  Same arithmetic as
 * oracle_attn_fwd_bias, for sampled checks at sizes where the full run is
 * slow. */
int oracle_attn_fwd_rows_bias(const double *q, const double *k, const double *v,
                              const double *bias_rows, long N, long d, double scale, int causal,
                              const long *rows, long n_rows, double *o_rows, double *lse_rows,
                              int nthreads) {
  rows_ctx_t c;
  long r;
  if (N < 1 || d < 1 || n_rows < 0) return -1;
  for (r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return -1;
  c.q = q; c.k = k; c.v = v; c.rows = rows; c.bias = bias_rows; c.o = o_rows; c.lse = lse_rows;
  c.N = N; c.d = d; c.scale = scale; c.causal = causal;
  run_pool(rows_item, &c, n_rows, nthreads);
  return 0;
}

int oracle_attn_fwd_rows(const double *q, const double *k, const double *v, long N, long d,
                         double scale, int causal, const long *rows, long n_rows, double *o_rows,
                         double *lse_rows, int nthreads) {
  return oracle_attn_fwd_rows_bias(q, k, v, NULL, N, d, scale, causal, rows, n_rows, o_rows,
                                   lse_rows, nthreads);
}

/* ------------------------------------------------------------------ */
/* Backward, by definition (10.2.4), one query row at a time.          */
/* ------------------------------------------------------------------ */
/* For row i:  P_ij from the definition, o_i = sum_j P_ij v_j,
 *   dP_ij = dO_i . v_j,  delta_i = sum_j P_ij dP_ij,
 *   dS_ij = P_ij (dP_ij - delta_i),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j += scale dS_ij q_i,  dV_j += P_ij dO_i.
 * delta as rowsum(P o dP) equals dO_i . O_i (the page's form) because
 * O_i = sum_j P_ij v_j; the tiled backward uses the page's form.
 * dK and dV of a head receive contributions from every row, so each worker
 * owns private dK/dV partial sums for the head it is on.  Worker t always
 * takes row chunks t, t + n, t + 2n, ... and the partials are added in worker
 * order, so a run is deterministic for a given thread count. */

typedef struct {
  const double *q, *k, *v, *dout;
  const double *bias; /* [B, H, N, N] or NULL */
  double *dq;
  double *dk_part, *dv_part; /* [nthreads][N][d] for the current head */
  long N, d, chunk, n_chunks;
  long bh;
  double scale;
  int causal;
} bwd_ctx_t;

static void bwd_item(void *p, long item, int tid) {
  bwd_ctx_t *c = (bwd_ctx_t *)p;
  const long N = c->N, d = c->d, hd = N * d;
  const double *Q = c->q + c->bh * hd, *K = c->k + c->bh * hd, *V = c->v + c->bh * hd;
  const double *dO = c->dout + c->bh * hd;
  double *dQ = c->dq + c->bh * hd;
  double *dK = c->dk_part + (long)tid * hd, *dV = c->dv_part + (long)tid * hd;
  const long r0 = item * c->chunk;
  const long r1 = r0 + c->chunk < N ? r0 + c->chunk : N;
  double *s = (double *)malloc(sizeof(double) * (size_t)N);
  double *pr = (double *)malloc(sizeof(double) * (size_t)N);
  double *dp = (double *)malloc(sizeof(double) * (size_t)N);
  long i, j, cc;
  for (i = r0; i < r1; ++i) {
    const long n_vis = visible_keys(i, N, c->causal);
    const double *q_i = Q + i * d, *do_i = dO + i * d;
    const double *bias_i = c->bias ? c->bias + (c->bh * N + i) * N : NULL;
    double m = -INFINITY, l = 0.0, delta = 0.0;
    double *dq_i = dQ + i * d;
    for (j = 0; j < n_vis; ++j) {
      s[j] = c->scale * dot(q_i, K + j * d, d);
      if (bias_i) s[j] += bias_i[j];
      if (s[j] > m) m = s[j];
    }
    for (cc = 0; cc < d; ++cc) dq_i[cc] = 0.0;
    if (m == -INFINITY) continue; /* empty softmax: P = 0, no gradient */
    for (j = 0; j < n_vis; ++j) l += exp(s[j] - m);
    for (j = 0; j < n_vis; ++j) {
      pr[j] = exp(s[j] - m) / l;
      dp[j] = dot(do_i, V + j * d, d);
      delta += pr[j] * dp[j];
    }
    for (j = 0; j < n_vis; ++j) {
      const double ds = pr[j] * (dp[j] - delta);
      const double *k_j = K + j * d;
      double *dk_j = dK + j * d, *dv_j = dV + j * d;
      for (cc = 0; cc < d; ++cc) {
        dq_i[cc] += c->scale * ds * k_j[cc];
        dk_j[cc] += c->scale * ds * q_i[cc];
        dv_j[cc] += pr[j] * do_i[cc];
      }
    }
  }
  free(s);
  free(pr);
  free(dp);
}

/* Full backward over [B,H,N,d] with an optional [B,H,N,N] bias (NULL: none;
 * the bias is an input, no gradient is formed for it): dq, dk, dv out.
 * Returns 0, -1 on bad sizes, -2 if scratch could not be allocated. */
int oracle_attn_bwd_bias(const double *q, const double *k, const double *v, const double *bias,
                         const double *dout, double *dq, double *dk, double *dv, long B, long H,
                         long N, long d, double scale, int causal, int nthreads) {
  bwd_ctx_t c;
  long bh, t, x;
  int nt;
  const long hd = N * d;
  if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
  if (B * H * N == 0) return 0;
  c.chunk = 32;
  c.n_chunks = (N + c.chunk - 1) / c.chunk;
  nt = nthreads < 1 ? 1 : nthreads;
  if (nt > c.n_chunks) nt = (int)c.n_chunks;
  c.dk_part = (double *)malloc(sizeof(double) * (size_t)(nt * hd));
  c.dv_part = (double *)malloc(sizeof(double) * (size_t)(nt * hd));
  if (!c.dk_part || !c.dv_part) {
    free(c.dk_part);
    free(c.dv_part);
    return -2;
  }
  c.q = q; c.k = k; c.v = v; c.bias = bias; c.dout = dout; c.dq = dq;
  c.N = N; c.d = d; c.scale = scale; c.causal = causal;
  for (bh = 0; bh < B * H; ++bh) {
    c.bh = bh;
    memset(c.dk_part, 0, sizeof(double) * (size_t)(nt * hd));
    memset(c.dv_part, 0, sizeof(double) * (size_t)(nt * hd));
    run_pool_mode(bwd_item, &c, c.n_chunks, nt, 1);
    for (x = 0; x < hd; ++x) {
      double sk = 0.0, sv = 0.0;
      for (t = 0; t < nt; ++t) {
        sk += c.dk_part[t * hd + x];
        sv += c.dv_part[t * hd + x];
      }
      dk[bh * hd + x] = sk;
      dv[bh * hd + x] = sv;
    }
  }
  free(c.dk_part);
  free(c.dv_part);
  return 0;
}

int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv, long B, long H, long N, long d,
                    double scale, int causal, int nthreads) {
  return oracle_attn_bwd_bias(q, k, v, NULL, dout, dq, dk, dv, B, H, N, d, scale, causal,
                              nthreads);
}

/* ------------------------------------------------------------------ */
/* Tiled online-softmax forward in the page's FA1 form (10.2.2, 10.2.5) */
/* ------------------------------------------------------------------ */
/* K/V blocks of Bc rows outer, Q blocks of Br rows inner; m, l and the
 * normalised O of every row live between outer iterations.  Inside a tile:
 *   S_ij = scale Q_i K_j^T (masked entries excluded),
 *   m~ = rowmax S_ij, P~ = exp(S_ij - m~), l~ = rowsum P~,
 *   m' = max(m, m~), alpha = exp(m - m'), beta = exp(m~ - m'),
 *   l' = alpha l + beta l~, O' = (alpha l O + beta P~ V_j) / l'.
 * A row with no visible key in a tile skips that tile (its m~ would be
 * -inf).  Output m and l are returned for the tiled backward. */
int oracle_tiled_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                     double *m_out, double *l_out, long B, long H, long N, long d, double scale,
                     int causal, long Br, long Bc) {
  long bh, j0, i0, i, j, c;
  const long hd = N * d;
  double *pt, *acc;
  if (B < 0 || H < 0 || N < 0 || d < 1 || Br < 1 || Bc < 1) return -1;
  pt = (double *)malloc(sizeof(double) * (size_t)Bc);
  acc = (double *)malloc(sizeof(double) * (size_t)d);
  for (bh = 0; bh < B * H; ++bh) {
    const double *Q = q + bh * hd, *K = k + bh * hd, *V = v + bh * hd;
    double *O = o + bh * hd, *m = m_out + bh * N, *l = l_out + bh * N;
    for (i = 0; i < N; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.0;
      for (c = 0; c < d; ++c) O[i * d + c] = 0.0;
    }
    for (j0 = 0; j0 < N; j0 += Bc) {           /* outer: K_j, V_j */
      const long j1 = j0 + Bc < N ? j0 + Bc : N;
      for (i0 = 0; i0 < N; i0 += Br) {         /* inner: Q_i */
        const long i1 = i0 + Br < N ? i0 + Br : N;
        for (i = i0; i < i1; ++i) {
          const long jv = causal ? (i + 1 < j1 ? i + 1 : j1) : j1; /* visible end */
          double mt = -INFINITY, lt = 0.0, mn, alpha, beta, ln;
          if (jv <= j0) continue;
          for (j = j0; j < jv; ++j) {
            pt[j - j0] = scale * dot(Q + i * d, K + j * d, d);
            if (pt[j - j0] > mt) mt = pt[j - j0];
          }
          for (j = j0; j < jv; ++j) {
            pt[j - j0] = exp(pt[j - j0] - mt);
            lt += pt[j - j0];
          }
          mn = m[i] > mt ? m[i] : mt;
          alpha = exp(m[i] - mn);
          beta = exp(mt - mn);
          ln = alpha * l[i] + beta * lt;
          for (c = 0; c < d; ++c) acc[c] = 0.0;
          for (j = j0; j < jv; ++j)
            for (c = 0; c < d; ++c) acc[c] += pt[j - j0] * V[j * d + c];
          for (c = 0; c < d; ++c)
            O[i * d + c] = (alpha * l[i] * O[i * d + c] + beta * acc[c]) / ln;
          m[i] = mn;
          l[i] = ln;
        }
      }
    }
    for (i = 0; i < N; ++i) lse[bh * N + i] = m[i] + log(l[i]);
  }
  free(pt);
  free(acc);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Tiled recompute backward (10.2.4, FA1 loop order of 10.2.5)         */
/* ------------------------------------------------------------------ */
/* Inputs include the forward's O and its saved row statistics m, l.
 *   delta_i = dO_i . O_i                         (once per row)
 *   for K/V block j (outer), Q block i (inner):
 *     S_ij = scale Q_i K_j^T, P_ij = exp(S_ij - m_i) / l_i  (recomputed)
 *     dV_j += P_ij^T dO_i, dP_ij = dO_i V_j^T, dS_ij = P_ij o (dP_ij - delta_i)
 *     dQ_i += scale dS_ij K_j, dK_j += scale dS_ij^T Q_i
 * delta_out ([B,H,N]) receives delta. */
int oracle_tiled_bwd(const double *q, const double *k, const double *v, const double *o,
                     const double *dout, const double *m_in, const double *l_in, double *dq,
                     double *dk, double *dv, double *delta_out, long B, long H, long N, long d,
                     double scale, int causal, long Br, long Bc) {
  long bh, j0, i0, i, j, c;
  const long hd = N * d;
  if (B < 0 || H < 0 || N < 0 || d < 1 || Br < 1 || Bc < 1) return -1;
  for (bh = 0; bh < B * H; ++bh) {
    const double *Q = q + bh * hd, *K = k + bh * hd, *V = v + bh * hd, *O = o + bh * hd;
    const double *dO = dout + bh * hd, *m = m_in + bh * N, *l = l_in + bh * N;
    double *dQ = dq + bh * hd, *dK = dk + bh * hd, *dV = dv + bh * hd;
    double *delta = delta_out + bh * N;
    for (i = 0; i < N; ++i) delta[i] = dot(dO + i * d, O + i * d, d);
    for (i = 0; i < hd; ++i) dQ[i] = dK[i] = dV[i] = 0.0;
    for (j0 = 0; j0 < N; j0 += Bc) {
      const long j1 = j0 + Bc < N ? j0 + Bc : N;
      for (i0 = 0; i0 < N; i0 += Br) {
        const long i1 = i0 + Br < N ? i0 + Br : N;
        for (i = i0; i < i1; ++i) {
          for (j = j0; j < j1; ++j) {
            double p, dp, ds;
            if (causal && j > i) continue;
            p = exp(scale * dot(Q + i * d, K + j * d, d) - m[i]) / l[i];
            dp = dot(dO + i * d, V + j * d, d);
            ds = p * (dp - delta[i]);
            for (c = 0; c < d; ++c) {
              dV[j * d + c] += p * dO[i * d + c];
              dQ[i * d + c] += scale * ds * K[j * d + c];
              dK[j * d + c] += scale * ds * Q[i * d + c];
            }
          }
        }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Exact decoders for the storage formats the GPU receives.            */
/* ------------------------------------------------------------------ */
/* bfloat16: the upper 16 bits of an IEEE binary32. */
void oracle_decode_bf16(const unsigned short *bits, double *out, long n) {
  long i;
  for (i = 0; i < n; ++i) {
    union {
      unsigned int u;
      float f;
    } x;
    x.u = ((unsigned int)bits[i]) << 16;
    out[i] = (double)x.f;
  }
}

/* OCP float8 e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there is
 * no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.  The
 * decoded value is multiplied by the per-tensor scale (exact in double). */
void oracle_decode_e4m3fn(const unsigned char *codes, double scale, double *out, long n) {
  long i;
  for (i = 0; i < n; ++i) {
    const unsigned int c = codes[i];
    const int sign = (c >> 7) & 1, e = (c >> 3) & 15, mant = c & 7;
    double val;
    if (e == 15 && mant == 7)
      val = NAN;
    else if (e == 0)
      val = ldexp((double)mant, -9);
    else
      val = ldexp(1.0 + mant / 8.0, e - 7);
    out[i] = (sign ? -val : val) * scale;
  }
}
