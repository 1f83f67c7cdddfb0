/*
 * moba_ref.c — fp64 CPU oracle for the MoBA prefill forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link or call this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it. It shares no code with the GPU library.
 *
 * What it computes is the plain definition of the method on the PaperTrace
 * page "2.1.3 MoBA" (yayajjiang.github.io), written out row by row in fp64:
 *
 *   - blocks are contiguous and disjoint, block i = rows [iB, (i+1)B)
 *     (section 1, eq. (2), 0-based here);
 *   - block key = mean of the block's keys, gate score s_i = q . kbar_i,
 *     unscaled (section 1, eq. (3));
 *   - blocks after the query's own block are excluded, the own block c is
 *     always selected and never ranked by its (future-leaking) mean, and the
 *     k of top-k counts that own block, so at most k-1 history blocks are
 *     taken (section 2, and section 2.1 on what k counts);
 *   - history blocks rank by (score descending, block index ascending);
 *   - the output is one softmax over the union of the selected tokens, with
 *     the own block causal (j <= p) and history blocks whole
 *     (eqs. (4)-(6)); it is evaluated as a dense masked row over all N keys,
 *     the form of the mask-based reference backend described on the pages.
 *
 * Two more forms exist for the pages' cross-checks: MODE_TWO_BRANCH merges
 * the causal own-block branch and the history branch with (m, l, u)
 * statistics (section 2, eqs. (7)-(8)); MODE_NAIVE adds the two separately
 * normalised branch outputs, the combination section 2 says is wrong.
 *
 * Inputs may be bf16 (uint16 bit patterns, widened exactly) or fp32; all
 * arithmetic is fp64. Rows run in parallel with OpenMP; within a row every
 * sum runs in index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_BF16 = 0, REF_F32 = 1 };
enum { MODE_UNION = 0, MODE_TWO_BRANCH = 1, MODE_NAIVE = 2 };

typedef struct {
  int64_t N;     /* sequence length */
  int32_t Hq;    /* query heads */
  int32_t Hkv;   /* key/value heads; query head h reads KV head h / (Hq/Hkv) */
  int32_t d;     /* head dim */
  int32_t B;     /* block size */
  int32_t k;     /* top-k, counting the query's own block */
  double scale;  /* multiplies the attention logits (not the gate) */
  int32_t dtype; /* REF_BF16 or REF_F32 */
  int32_t routing; /* 0: each query head ranks blocks with its own query;
                      1: the query heads of a KV head share one ranking by the
                         group's summed gate score, sum_h q_h . kbar_i
                         (PaperTrace "2.1.3 MoBA", section 5.5 on GQA) */
} moba_ref_problem;

static inline double ld(const void *base, int dtype, int64_t i) {
  if (dtype == REF_BF16) {
    uint32_t u = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
  }
  return (double)((const float *)base)[i];
}

static int64_t num_blocks(const moba_ref_problem *p) { return (p->N + p->B - 1) / p->B; }

static int check(const moba_ref_problem *p) {
  if (!p || p->N < 1 || p->Hq < 1 || p->Hkv < 1 || p->d < 1 || p->B < 1 || p->k < 1) return 1;
  if (p->Hq % p->Hkv) return 1;
  if (!(p->scale > 0.0) || !isfinite(p->scale)) return 1;
  if (p->dtype != REF_BF16 && p->dtype != REF_F32) return 1;
  if (p->routing != 0 && p->routing != 1) return 1;
  return 0;
}

/*
 * Block keys, eq. (3): kbar[g][i][c] = (1/B) * sum_{j in block i} K[j][g][c],
 * for the n-1 blocks that can ever be history (block n-1 never is: only blocks
 * before a query's own block compete). Returns 0 on success.
 */
int moba_ref_block_means(const moba_ref_problem *p, const void *K, double *kbar) {
  if (check(p) || !K || !kbar) return 1;
  const int64_t nh = num_blocks(p) - 1;
  const int64_t d = p->d;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t g = 0; g < p->Hkv; ++g) {
    for (int64_t i = 0; i < nh; ++i) {
      double *out = kbar + (g * nh + i) * d;
      for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
      for (int64_t j = i * p->B; j < (i + 1) * p->B; ++j)
        for (int64_t c = 0; c < d; ++c) out[c] += ld(K, p->dtype, (j * p->Hkv + g) * d + c);
      for (int64_t c = 0; c < d; ++c) out[c] /= (double)p->B;
    }
  }
  return 0;
}

/* Index of the best remaining candidate: highest score, lowest index on ties. */
static int64_t best_unpicked(const double *s, const unsigned char *picked, int64_t c) {
  int64_t best = -1;
  for (int64_t i = 0; i < c; ++i) {
    if (picked[i]) continue;
    if (best < 0 || s[i] > s[best]) best = i;
  }
  return best;
}

/* Softmax statistics over a set of keys: m = max logit, l = sum e^{z-m}, u = sum e^{z-m} v. */
static void branch_stats(const moba_ref_problem *p, const double *q, const void *K, const void *V,
                         int h, const unsigned char *member, double *m, double *l, double *u,
                         double *z) {
  const int64_t N = p->N, d = p->d;
  const int G = p->Hq / p->Hkv, g = h / G;
  double mx = -INFINITY;
  for (int64_t j = 0; j < N; ++j) {
    if (!member[j]) continue;
    double dot = 0.0;
    const int64_t kb = (j * p->Hkv + g) * d;
    for (int64_t c = 0; c < d; ++c) dot += q[c] * ld(K, p->dtype, kb + c);
    z[j] = p->scale * dot;
    if (z[j] > mx) mx = z[j];
  }
  double sum = 0.0;
  for (int64_t c = 0; c < d; ++c) u[c] = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    if (!member[j]) continue;
    double w = exp(z[j] - mx);
    sum += w;
    const int64_t vb = (j * p->Hkv + g) * d;
    for (int64_t c = 0; c < d; ++c) u[c] += w * ld(V, p->dtype, vb + c);
  }
  *m = mx;
  *l = sum;
}

/*
 * Evaluate nrows (row, head) pairs.
 *
 *  kbar        block keys from moba_ref_block_means, or NULL to compute them here.
 *  forced_sel  NULL, or [nrows][k] selections to use instead of the gate's
 *              ranking: entries b with 0 <= b < the row's own block c are
 *              the history set, a repeated entry counting once and at most
 *              k-1 of them kept in the given order; -1, the own block and
 *              later blocks are skipped; the own block is always attended
 *              causally.
 *  sel_out     [nrows][k]: selected blocks ascending (history, then own block),
 *              padded with -1. May be NULL.
 *  o_out       [nrows][d] fp64 output. May be NULL.
 *  gap_out     [nrows][2]: for rows with more history blocks than k-1 slots
 *              (and k >= 2), the gap between the last selected and the best
 *              unselected history score, and max of their magnitudes; NaN
 *              otherwise. May be NULL.
 *  mode        MODE_UNION, MODE_TWO_BRANCH or MODE_NAIVE.
 *  nthreads    OpenMP threads (<= 0: runtime default).
 */
int moba_ref_rows(const moba_ref_problem *p, const void *Q, const void *K, const void *V,
                  const double *kbar, const int64_t *rows, const int32_t *heads, int64_t nrows,
                  const int32_t *forced_sel, int mode, int32_t *sel_out, double *o_out,
                  double *gap_out, int nthreads) {
  if (check(p) || !Q || !K || !rows || !heads) return 1;
  if ((o_out || mode != MODE_UNION) && !V) return 1;
  const int64_t N = p->N, d = p->d, B = p->B, kk = p->k;
  const int64_t nh = num_blocks(p) - 1;
  const int G = p->Hq / p->Hkv;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N || heads[r] < 0 || heads[r] >= p->Hq) return 1;

  double *own_kbar = NULL;
  if (!kbar && nh > 0) {
    own_kbar = (double *)malloc(sizeof(double) * (size_t)(p->Hkv * nh * d));
    if (!own_kbar) return 2;
    moba_ref_block_means(p, K, own_kbar);
    kbar = own_kbar;
  }
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
  nthreads = 1;
#endif
  int err = 0;
#pragma omp parallel num_threads(nthreads)
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(nh > 0 ? nh : 1));
    unsigned char *picked = (unsigned char *)malloc((size_t)(nh > 0 ? nh : 1));
    int64_t *hist = (int64_t *)malloc(sizeof(int64_t) * (size_t)kk);
    unsigned char *in_union = (unsigned char *)malloc((size_t)N);
    unsigned char *in_own = (unsigned char *)malloc((size_t)N);
    unsigned char *in_hist = (unsigned char *)malloc((size_t)N);
    double *z = (double *)malloc(sizeof(double) * (size_t)N);
    double *ua = (double *)malloc(sizeof(double) * (size_t)d);
    double *ub = (double *)malloc(sizeof(double) * (size_t)d);
    double *qd = (double *)malloc(sizeof(double) * (size_t)d);
    double *qg = (double *)malloc(sizeof(double) * (size_t)d);
    if (!s || !picked || !hist || !in_union || !in_own || !in_hist || !z || !ua || !ub || !qd ||
        !qg) {
#pragma omp atomic write
      err = 2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t row = rows[r];
        const int h = heads[r], g = h / G;
        const int64_t c = row / B; /* the query's own block */
        const int64_t qb = (row * p->Hq + h) * d;
        for (int64_t t = 0; t < d; ++t) qd[t] = ld(Q, p->dtype, qb + t);
        /* the gate's query: this head's, or the sum over the head group */
        for (int64_t t = 0; t < d; ++t) {
          if (p->routing == 1) {
            double acc = 0.0;
            for (int hh = 0; hh < G; ++hh)
              acc += ld(Q, p->dtype, (row * p->Hq + (int64_t)g * G + hh) * d + t);
            qg[t] = acc;
          } else {
            qg[t] = qd[t];
          }
        }

        /* Gate scores over legal history blocks 0..c-1 (eq. (3)). */
        for (int64_t i = 0; i < c; ++i) {
          double dot = 0.0;
          const double *kb = kbar + ((int64_t)g * nh + i) * d;
          for (int64_t t = 0; t < d; ++t) dot += qg[t] * kb[t];
          s[i] = dot;
        }
        /* Selection: up to k-1 history blocks; the own block is forced. */
        int64_t nsel = 0;
        memset(picked, 0, (size_t)(nh > 0 ? nh : 1));
        if (forced_sel) {
          for (int64_t t = 0; t < kk; ++t) {
            int64_t b = forced_sel[r * kk + t];
            if (b >= 0 && b < c && !picked[b] && nsel < kk - 1) {
              picked[b] = 1;
              hist[nsel++] = b;
            }
          }
        } else {
          int64_t want = (kk - 1 < c) ? kk - 1 : c;
          for (int64_t t = 0; t < want; ++t) {
            int64_t b = best_unpicked(s, picked, c);
            picked[b] = 1;
            hist[nsel++] = b;
          }
        }
        if (gap_out) {
          gap_out[2 * r] = NAN;
          gap_out[2 * r + 1] = NAN;
          if (!forced_sel && kk >= 2 && c > kk - 1) {
            double last = s[hist[nsel - 1]];
            int64_t nb = best_unpicked(s, picked, c);
            double next = s[nb];
            gap_out[2 * r] = last - next;
            gap_out[2 * r + 1] = fabs(last) > fabs(next) ? fabs(last) : fabs(next);
          }
        }
        if (sel_out) {
          int64_t t = 0;
          for (int64_t b = 0; b < c; ++b)
            if (picked[b]) sel_out[r * kk + t++] = (int32_t)b;
          sel_out[r * kk + t++] = (int32_t)c;
          for (; t < kk; ++t) sel_out[r * kk + t] = -1;
        }
        if (!o_out) continue;

        /* Candidate set (eqs. (4)-(6)): selected history blocks whole, own block causal. */
        for (int64_t j = 0; j < N; ++j) {
          int64_t bj = j / B;
          in_own[j] = (bj == c && j <= row);
          in_hist[j] = (bj < c && picked[bj]);
          in_union[j] = in_own[j] | in_hist[j];
        }
        double *o = o_out + r * d;
        if (mode == MODE_UNION) {
          double m, l;
          branch_stats(p, qd, K, V, h, in_union, &m, &l, ua, z);
          for (int64_t t = 0; t < d; ++t) o[t] = ua[t] / l;
        } else {
          double ms, ls, mh = -INFINITY, lh = 0.0;
          branch_stats(p, qd, K, V, h, in_own, &ms, &ls, ua, z);
          if (nsel > 0) branch_stats(p, qd, K, V, h, in_hist, &mh, &lh, ub, z);
          if (mode == MODE_TWO_BRANCH) {
            /* eqs. (7)-(8): one softmax over the union from the two branches' statistics */
            double m = ms > mh ? ms : mh;
            double as = exp(ms - m), ah = nsel > 0 ? exp(mh - m) : 0.0;
            double l = as * ls + ah * lh;
            for (int64_t t = 0; t < d; ++t) o[t] = (as * ua[t] + (nsel > 0 ? ah * ub[t] : 0.0)) / l;
          } else {
            for (int64_t t = 0; t < d; ++t) o[t] = ua[t] / ls + (nsel > 0 ? ub[t] / lh : 0.0);
          }
        }
      }
    }
    free(s);
    free(picked);
    free(hist);
    free(in_union);
    free(in_own);
    free(in_hist);
    free(z);
    free(ua);
    free(ub);
    free(qd);
    free(qg);
  }
  free(own_kbar);
  return err;
}

/*
 * Causal full attention, written independently of the routing code above:
 * o[p] = softmax_j<=p(scale q_p . k_j) v_j in fp64 (section 1, eq. (1)).
 * Used as the target the method must reduce to when k covers every block.
 */
int moba_ref_causal_full(const moba_ref_problem *p, const void *Q, const void *K, const void *V,
                         const int64_t *rows, const int32_t *heads, int64_t nrows, double *o_out,
                         int nthreads) {
  if (check(p) || !Q || !K || !V || !rows || !heads || !o_out) return 1;
  const int64_t d = p->d;
  const int G = p->Hq / p->Hkv;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
  nthreads = 1;
#endif
  int err = 0;
#pragma omp parallel num_threads(nthreads)
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)p->N);
    if (!z) {
#pragma omp atomic write
      err = 2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t row = rows[r];
        const int h = heads[r], g = h / G;
        double mx = -INFINITY;
        for (int64_t j = 0; j <= row; ++j) {
          double dot = 0.0;
          for (int64_t t = 0; t < d; ++t)
            dot += ld(Q, p->dtype, (row * p->Hq + h) * d + t) * ld(K, p->dtype, (j * p->Hkv + g) * d + t);
          z[j] = p->scale * dot;
          if (z[j] > mx) mx = z[j];
        }
        double l = 0.0;
        double *o = o_out + r * d;
        for (int64_t t = 0; t < d; ++t) o[t] = 0.0;
        for (int64_t j = 0; j <= row; ++j) {
          double w = exp(z[j] - mx);
          l += w;
          for (int64_t t = 0; t < d; ++t) o[t] += w * ld(V, p->dtype, (j * p->Hkv + g) * d + t);
        }
        for (int64_t t = 0; t < d; ++t) o[t] /= l;
      }
    }
    free(z);
  }
  return err;
}

/*
 * Gradients of the loss L = sum over (row, head) of dO[row,head] . O[row,head]
 * with the block selection held fixed (the hard top-k passes no gradient to
 * the ranking, PaperTrace "2.1.3 MoBA" section 5.3; gradients reach Q, K and
 * V only through attended pairs). For one (row, head) with candidate set I
 * (eq. (4)): z_j = scale q.k_j, P = softmax(z) over I, o = sum_j P_j v_j;
 *   dV_j += P_j dO,
 *   dP_j  = dO . v_j,   D = dO . o = sum_j P_j dP_j,
 *   dZ_j  = P_j (dP_j - D),
 *   dq    = scale sum_j dZ_j k_j,   dK_j += scale dZ_j q.
 * Written out over every (row, head) in fp64; the selection is taken from
 * sel [N][Hq][k] (as moba_ref_rows returns it: history blocks < the row's
 * block, then the own block, -1 padding). dq [N][Hq][d], dk and dv
 * [N][Hkv][d] are overwritten.
 *
 * Every sum runs in the order of the plain loop nest "for row, for head, for
 * key j": dq of a (row, head) adds its keys in ascending j, and dK_j / dV_j
 * add the contributions of the (row, head) pairs in ascending (row, head).
 * Rows are processed in chunks: the per-pair quantities of a chunk (P_j and
 * dZ_j for its attended keys) are computed in parallel over pairs, then each
 * key's dK / dV rows take the chunk's contributions in (row, head) order, in
 * parallel over keys — the same additions in the same order as the serial
 * nest, so the result does not depend on the thread count.
 */
enum { BWD_CHUNK_ROWS = 32 };

int moba_ref_backward(const moba_ref_problem *p, const void *Q, const void *K, const void *V,
                      const double *dO, const int32_t *sel, double *dq, double *dk, double *dv) {
  if (check(p) || !Q || !K || !V || !dO || !sel || !dq || !dk || !dv) return 1;
  const int64_t N = p->N, d = p->d, B = p->B, kk = p->k;
  const int64_t Hq = p->Hq;
  const int G = p->Hq / p->Hkv;
  for (int64_t i = 0; i < N * p->Hq * d; ++i) dq[i] = 0.0;
  for (int64_t i = 0; i < N * p->Hkv * d; ++i) dk[i] = dv[i] = 0.0;
  const int64_t npair = BWD_CHUNK_ROWS * Hq;
  /* per pair of a chunk: membership and P_j, dZ_j over all N keys */
  unsigned char *member = (unsigned char *)malloc((size_t)(npair * N));
  double *pw = (double *)malloc(sizeof(double) * (size_t)(npair * N));
  double *dzw = (double *)malloc(sizeof(double) * (size_t)(npair * N));
  /* the inputs widened to fp64 once (exact) */
  const int64_t nq = N * Hq * d, nk = N * p->Hkv * d;
  double *Qd = (double *)malloc(sizeof(double) * (size_t)nq);
  double *Kd = (double *)malloc(sizeof(double) * (size_t)nk);
  double *Vd = (double *)malloc(sizeof(double) * (size_t)nk);
  if (!member || !pw || !dzw || !Qd || !Kd || !Vd) {
    free(member);
    free(pw);
    free(dzw);
    free(Qd);
    free(Kd);
    free(Vd);
    return 2;
  }
  for (int64_t i = 0; i < nq; ++i) Qd[i] = ld(Q, p->dtype, i);
  for (int64_t i = 0; i < nk; ++i) {
    Kd[i] = ld(K, p->dtype, i);
    Vd[i] = ld(V, p->dtype, i);
  }
  int err = 0;
  for (int64_t r0 = 0; r0 < N && !err; r0 += BWD_CHUNK_ROWS) {
    const int64_t r1 = r0 + BWD_CHUNK_ROWS < N ? r0 + BWD_CHUNK_ROWS : N;
    const int64_t pairs = (r1 - r0) * Hq;
    /* phase 1: softmax weights, D, dZ and dq of each (row, head) of the chunk */
#pragma omp parallel
    {
      double *o = (double *)malloc(sizeof(double) * (size_t)d);
      if (!o) {
#pragma omp atomic write
        err = 2;
      } else {
#pragma omp for schedule(dynamic, 1)
        for (int64_t pi = 0; pi < pairs; ++pi) {
          const int64_t row = r0 + pi / Hq;
          const int h = (int)(pi % Hq), g = h / G;
          const int64_t c = row / B;
          unsigned char *mem = member + pi * N;
          double *z = pw + pi * N, *dz = dzw + pi * N;
          const int32_t *sr = sel + (row * Hq + h) * kk;
          for (int64_t j = 0; j < N; ++j) mem[j] = (j / B == c && j <= row);
          for (int64_t t = 0; t < kk; ++t)
            if (sr[t] >= 0 && sr[t] < c)
              for (int64_t j = sr[t] * B; j < (sr[t] + 1) * B; ++j) mem[j] = 1;
          const int64_t qb = (row * Hq + h) * d;
          double mx = -INFINITY;
          for (int64_t j = 0; j < N; ++j) {
            if (!mem[j]) continue;
            double dot = 0.0;
            for (int64_t t = 0; t < d; ++t)
              dot += Qd[qb + t] * Kd[(j * p->Hkv + g) * d + t];
            z[j] = p->scale * dot;
            if (z[j] > mx) mx = z[j];
          }
          double l = 0.0;
          for (int64_t j = 0; j < N; ++j)
            if (mem[j]) l += exp(z[j] - mx);
          for (int64_t t = 0; t < d; ++t) o[t] = 0.0;
          for (int64_t j = 0; j < N; ++j) {
            if (!mem[j]) continue;
            z[j] = exp(z[j] - mx) / l; /* now P_j */
            for (int64_t t = 0; t < d; ++t) o[t] += z[j] * Vd[(j * p->Hkv + g) * d + t];
          }
          double D = 0.0;
          for (int64_t t = 0; t < d; ++t) D += dO[qb + t] * o[t];
          for (int64_t j = 0; j < N; ++j) {
            if (!mem[j]) continue;
            const int64_t kvb = (j * p->Hkv + g) * d;
            double dp = 0.0;
            for (int64_t t = 0; t < d; ++t) dp += dO[qb + t] * Vd[kvb + t];
            dz[j] = z[j] * (dp - D);
            for (int64_t t = 0; t < d; ++t) dq[qb + t] += p->scale * dz[j] * Kd[kvb + t];
          }
        }
      }
      free(o);
    }
    if (err) break;
    /* phase 2: each key's dV and dK rows, the chunk's pairs in (row, head) order */
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j) {
      for (int64_t pi = 0; pi < pairs; ++pi) {
        if (!member[pi * N + j]) continue;
        const int64_t row = r0 + pi / Hq;
        const int h = (int)(pi % Hq), g = h / G;
        const int64_t qb = (row * Hq + h) * d, kvb = (j * p->Hkv + g) * d;
        const double pj = pw[pi * N + j], dzj = dzw[pi * N + j];
        for (int64_t t = 0; t < d; ++t) {
          dv[kvb + t] += pj * dO[qb + t];
          dk[kvb + t] += p->scale * dzj * Qd[qb + t];
        }
      }
    }
  }
  free(member);
  free(pw);
  free(dzw);
  free(Qd);
  free(Kd);
  free(Vd);
  return err;
}
