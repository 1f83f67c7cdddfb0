/*
 * Seeded synthetic inputs for the MoBA prefill workloads.
 *
 * This module holds no part of the attention method: it only draws the Q, K, V
 * tensors (and row samples) that both the GPU path and the fp64 oracle consume.
 * Every value is a pure function of (seed, tensor id, element index), so any
 * element can be regenerated on its own.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based hash; a pair of
 * 32-bit uniforms feeds the Box-Muller transform (Box & Muller, 1958), whose
 * cosine and sine outputs fill elements 2i and 2i+1 of a tensor.
 *
 * Workload structure (the shape of the pages' experiments):
 *  - Q, K, V i.i.d. N(0, 1);
 *  - every (KV head, block) adds one offset vector, i.i.d. N(0, off_std^2) per
 *    coordinate, to all keys of that block, so block means are well separated;
 *  - optional "needles": per KV head a random unit direction u; a few needle
 *    blocks get +needle_gain*u added to their offset, and a fraction of the
 *    query rows of each head is rotated onto u: q <- q - (q.u)u + sqrt(d)u.
 *
 * Output dtype 0 = bf16 bit patterns (round to nearest even from fp32),
 * 1 = fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { T_Q = 1, T_K = 2, T_V = 3, T_OFF = 4, T_DIR = 5, T_NBLK = 6, T_NROW = 7, T_SAMPLE = 8 };

static inline uint64_t sm64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor) {
  return sm64(seed ^ sm64(tensor * 0xD1B54A32D192ED03ull));
}

/* Standard normal for element idx of the stream keyed by `key`. */
static inline double normal_at(uint64_t key, uint64_t idx) {
  uint64_t r = sm64(key + (idx >> 1) * 0x9E3779B97F4A7C15ull);
  double u1 = ((double)(r >> 32) + 0.5) * (1.0 / 4294967296.0);
  double u2 = ((double)(r & 0xFFFFFFFFull) + 0.5) * (1.0 / 4294967296.0);
  double rad = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (idx & 1) ? rad * sin(th) : rad * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static inline void store(void *out, int dtype, int64_t i, double x) {
  float f = (float)x;
  if (dtype == 0)
    ((uint16_t *)out)[i] = f32_to_bf16_rne(f);
  else
    ((float *)out)[i] = f;
}

typedef struct {
  int64_t N;
  int32_t Hq, Hkv, d, B;
  double off_std;     /* std of the per-(head, block) key offset */
  int32_t n_needle_blocks; /* per KV head; 0 disables needles */
  double needle_gain; /* added along u to a needle block's offset */
  double needle_row_frac; /* fraction of query rows per head rotated onto u */
} synth_cfg;

static int64_t nblocks(const synth_cfg *c) { return (c->N + c->B - 1) / c->B; }

/* Unit direction u_g (fp64) for KV head g. */
static void needle_dir(uint64_t seed, const synth_cfg *c, int g, double *u) {
  uint64_t key = stream_key(seed, T_DIR);
  double nrm = 0.0;
  for (int i = 0; i < c->d; ++i) {
    u[i] = normal_at(key, (uint64_t)g * c->d + i);
    nrm += u[i] * u[i];
  }
  nrm = sqrt(nrm);
  for (int i = 0; i < c->d; ++i) u[i] /= nrm;
}

/* Distinct needle blocks in [0, n-1) for KV head g (n-1 = blocks that can be history). */
int synth_needle_blocks(uint64_t seed, const synth_cfg *c, int g, int32_t *out) {
  int64_t nh = nblocks(c) - 1;
  int want = c->n_needle_blocks;
  if (want > nh) want = (int)nh;
  uint64_t key = stream_key(seed, T_NBLK);
  int got = 0;
  for (uint64_t t = 0; got < want; ++t) {
    int32_t b = (int32_t)(sm64(key + ((uint64_t)g << 32) + t) % (uint64_t)nh);
    int dup = 0;
    for (int i = 0; i < got; ++i) dup |= (out[i] == b);
    if (!dup) out[got++] = b;
  }
  return got;
}

/* Distinct needle rows for query head h; returns the count written. */
int64_t synth_needle_rows(uint64_t seed, const synth_cfg *c, int h, int64_t *out, int64_t cap) {
  int64_t want = (int64_t)llround(c->needle_row_frac * (double)c->N);
  if (want > c->N) want = c->N;
  if (want > cap) want = cap;
  uint64_t key = stream_key(seed, T_NROW);
  unsigned char *taken = (unsigned char *)calloc((size_t)c->N, 1);
  if (!taken) return -1;
  int64_t got = 0;
  for (uint64_t t = 0; got < want; ++t) {
    int64_t p = (int64_t)(sm64(key + ((uint64_t)h << 40) + t) % (uint64_t)c->N);
    if (!taken[p]) {
      taken[p] = 1;
      out[got++] = p;
    }
  }
  free(taken);
  return got;
}

/* Per-(KV head, block) key offsets, fp64 [Hkv][n][d], needles included. */
static double *make_offsets(uint64_t seed, const synth_cfg *c) {
  int64_t n = nblocks(c);
  size_t cnt = (size_t)c->Hkv * (size_t)n * (size_t)c->d;
  double *off = (double *)malloc(cnt * sizeof(double));
  if (!off) return NULL;
  uint64_t key = stream_key(seed, T_OFF);
  for (size_t i = 0; i < cnt; ++i) off[i] = c->off_std * normal_at(key, i);
  if (c->n_needle_blocks > 0 && n > 1) {
    double *u = (double *)malloc(sizeof(double) * c->d);
    int32_t *blk = (int32_t *)malloc(sizeof(int32_t) * (size_t)c->n_needle_blocks);
    for (int g = 0; g < c->Hkv; ++g) {
      needle_dir(seed, c, g, u);
      int nb = synth_needle_blocks(seed, c, g, blk);
      for (int t = 0; t < nb; ++t) {
        double *o = off + ((size_t)g * n + blk[t]) * c->d;
        for (int i = 0; i < c->d; ++i) o[i] += c->needle_gain * u[i];
      }
    }
    free(u);
    free(blk);
  }
  return off;
}

/*
 * Fill Q [N][Hq][d], K [N][Hkv][d], V [N][Hkv][d] (any pointer may be NULL to
 * skip that tensor). Returns 0 on success.
 */
int synth_qkv(uint64_t seed, const synth_cfg *c, int dtype, void *q, void *k, void *v) {
  const int64_t N = c->N, d = c->d;
  if (q) {
    uint64_t key = stream_key(seed, T_Q);
    int64_t cnt = N * c->Hq * d;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < cnt; ++i) store(q, dtype, i, normal_at(key, (uint64_t)i));
    if (c->n_needle_blocks > 0 && c->needle_row_frac > 0.0) {
      int64_t cap = N;
      int G = c->Hq / c->Hkv;
      double *u = (double *)malloc(sizeof(double) * d);
      double *row = (double *)malloc(sizeof(double) * d);
      int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
      for (int h = 0; h < c->Hq; ++h) {
        needle_dir(seed, c, h / G, u);
        int64_t nr = synth_needle_rows(seed, c, h, rows, cap);
        for (int64_t t = 0; t < nr; ++t) {
          int64_t base = (rows[t] * c->Hq + h) * d;
          double dot = 0.0;
          for (int i = 0; i < d; ++i) {
            row[i] = normal_at(key, (uint64_t)(base + i));
            dot += row[i] * u[i];
          }
          double s = sqrt((double)d);
          for (int i = 0; i < d; ++i) store(q, dtype, base + i, row[i] - dot * u[i] + s * u[i]);
        }
      }
      free(u);
      free(row);
      free(rows);
    }
  }
  if (k) {
    double *off = make_offsets(seed, c);
    if (!off) return 1;
    uint64_t key = stream_key(seed, T_K);
    int64_t cnt = N * c->Hkv * d;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < cnt; ++i) {
      int64_t j = i / (c->Hkv * d);
      int64_t g = (i / d) % c->Hkv;
      int64_t ch = i % d;
      int64_t b = j / c->B;
      double x = normal_at(key, (uint64_t)i) + off[((size_t)g * nblocks(c) + b) * d + ch];
      store(k, dtype, i, x);
    }
    free(off);
  }
  if (v) {
    uint64_t key = stream_key(seed, T_V);
    int64_t cnt = N * c->Hkv * d;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < cnt; ++i) store(v, dtype, i, normal_at(key, (uint64_t)i));
  }
  return 0;
}

/*
 * Seeded sample of (row, query head) pairs spread over every block:
 * sample r lands in block r mod n; its offset inside the block is 0 for the
 * first n samples, B-1 for the next n, and hashed after that.
 */
void synth_sample_rows(uint64_t seed, const synth_cfg *c, int64_t count, int64_t *rows, int32_t *heads) {
  int64_t n = nblocks(c);
  uint64_t key = stream_key(seed, T_SAMPLE);
  for (int64_t r = 0; r < count; ++r) {
    uint64_t hsh = sm64(key + (uint64_t)r);
    int64_t blk = r % n;
    int64_t off;
    if (r < n)
      off = 0;
    else if (r < 2 * n)
      off = c->B - 1;
    else
      off = (int64_t)((hsh >> 20) % (uint64_t)c->B);
    int64_t p = blk * c->B + off;
    if (p > c->N - 1) p = c->N - 1;
    rows[r] = p;
    heads[r] = (int32_t)(hsh % (uint64_t)c->Hq);
  }
}
