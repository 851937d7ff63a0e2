/*
 * lsa_oracle.c -- plain, slow, fp64 CPU oracle of the LSA indexer path.
 * TEST INFRASTRUCTURE ONLY (see lsa_oracle.h).  No blocking, no fusion, no
 * reordering beyond what each definition states; OpenMP only splits
 * independent outputs across threads.
 */
#include "lsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int lsa_or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the parallel loops (timing the oracle on one core). */
void lsa_or_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int lsa_or_trigger_due(int64_t t, int tau) {
  if (t < 0 || tau <= 0) return 0;
  return (t % tau) == 0;
}

/* ------------------------------------------------------------------------ */
/* Storage formats                                                          */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32: widen by appending 16 zero bits. */
double lsa_or_bf16_to_double(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* Round a double straight to bf16 (8 significant bits, exponent range of
 * binary32), nearest-even, in a single rounding step. */
uint16_t lsa_or_bf16_from_double(double a) {
  if (isnan(a)) return 0x7FC0;
  uint16_t sign = signbit(a) ? 0x8000 : 0;
  double m = fabs(a);
  if (m == 0.0) return sign;
  if (isinf(m)) return (uint16_t)(sign | 0x7F80);
  int e;
  frexp(m, &e);                 /* m = f * 2^e, f in [0.5, 1) */
  int ulp_exp = e - 8;          /* 8 significant bits */
  if (ulp_exp < -133) ulp_exp = -133;   /* bf16 subnormal spacing 2^-133 */
  double r = nearbyint(ldexp(m, -ulp_exp));   /* ties to even */
  double v = ldexp(r, ulp_exp);
  if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);   /* overflow */
  float f = (float)v;           /* exact: v has <= 8 significant bits */
  uint32_t w;
  memcpy(&w, &f, sizeof w);
  return (uint16_t)(sign | (uint16_t)((w >> 16) & 0x7FFF));
}

/* OCP 8-bit E4M3 "FN" variant: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
 * exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is
 * no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. */
double lsa_or_e4m3_to_double(uint8_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

double lsa_or_softplus(double x) {
  /* log(1 + e^x) written so that it neither overflows nor cancels */
  return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

double lsa_or_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* ------------------------------------------------------------------------ */
/* O1 query encoder                                                          */
/* ------------------------------------------------------------------------ */

void lsa_or_project(int D, int H, int dI, const uint16_t* h,
                    const uint16_t* Wq, const uint16_t* Wg, uint16_t* q,
                    float* g, double* a_out) {
  const int rows = H * dI;
#pragma omp parallel for schedule(static)
  for (int j = 0; j < rows; ++j) {
    double a = 0.0;
    for (int d = 0; d < D; ++d)
      a += lsa_or_bf16_to_double(Wq[(int64_t)j * D + d]) *
           lsa_or_bf16_to_double(h[d]);
    q[j] = lsa_or_bf16_from_double(a);
    if (a_out) a_out[j] = a;
  }
  for (int hh = 0; hh < H; ++hh) {
    double a = 0.0;
    for (int d = 0; d < D; ++d)
      a += lsa_or_bf16_to_double(Wg[(int64_t)hh * D + d]) *
           lsa_or_bf16_to_double(h[d]);
    g[hh] = (float)lsa_or_softplus(a);
  }
}

void lsa_or_query_collapse(int H, int dI, const uint16_t* q, const float* g,
                           double* q_eff) {
  for (int d = 0; d < dI; ++d) {
    double acc = 0.0;
    for (int hh = 0; hh < H; ++hh)
      acc += (double)g[hh] * lsa_or_bf16_to_double(q[hh * dI + d]);
    q_eff[d] = acc;
  }
}

/* ------------------------------------------------------------------------ */
/* O2/O3 score                                                               */
/* ------------------------------------------------------------------------ */

static double key_value(int key_dtype, const void* keys, int64_t off) {
  if (key_dtype == 0) return lsa_or_bf16_to_double(((const uint16_t*)keys)[off]);
  return lsa_or_e4m3_to_double(((const uint8_t*)keys)[off]);
}

void lsa_or_score(int N, int H, int dI, int key_dtype, const void* keys,
                  const float* scale, const uint16_t* q, const float* g,
                  double bias, const int64_t* idx, int64_t n_idx,
                  double* z_out) {
  int64_t n = idx ? n_idx : (int64_t)N;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t s = idx ? idx[i] : i;
    double sigma = (key_dtype == 1 && scale) ? (double)scale[s] : 1.0;
    double z = 0.0;
    for (int hh = 0; hh < H; ++hh) {
      double dot = 0.0;
      for (int d = 0; d < dI; ++d)
        dot += lsa_or_bf16_to_double(q[hh * dI + d]) *
               key_value(key_dtype, keys, s * dI + d);
      z += (double)g[hh] * dot;
    }
    z_out[i] = z * sigma + bias;
  }
}

/* ------------------------------------------------------------------------ */
/* O4 threshold, O5 OR + compaction                                          */
/* ------------------------------------------------------------------------ */

void lsa_or_threshold(int64_t n, const double* z, uint8_t* sel) {
  for (int64_t i = 0; i < n; ++i) sel[i] = (z[i] >= 0.0) ? 1 : 0;
}

int64_t lsa_or_merge_compact(int L, int64_t N, const uint8_t* sel,
                             const double* z, int64_t cap, int32_t* surv_idx,
                             double* surv_z) {
  int64_t count = 0;
  for (int64_t s = 0; s < N; ++s) {
    int any = 0;
    double zmax = NAN;
    for (int l = 0; l < L; ++l) {
      if (sel[(int64_t)l * N + s]) any = 1;
      zmax = fmax(zmax, z[(int64_t)l * N + s]);   /* fmax ignores NaN */
    }
    if (!any) continue;
    if (count < cap) {
      surv_idx[count] = (int32_t)s;
      surv_z[count] = zmax;
    }
    ++count;
  }
  return count;
}

/* ------------------------------------------------------------------------ */
/* O6 top-k                                                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
  double z;
  int32_t idx;
} zi_pair;

static int cmp_score_desc(const void* pa, const void* pb) {
  const zi_pair* a = (const zi_pair*)pa;
  const zi_pair* b = (const zi_pair*)pb;
  int an = isnan(a->z), bn = isnan(b->z);
  if (an != bn) return an ? 1 : -1;           /* NaN ranks last */
  if (!an && a->z != b->z) return (a->z > b->z) ? -1 : 1;
  return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

static int cmp_int_asc(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a < b) ? -1 : (a > b);
}

int64_t lsa_or_topk(int64_t n, const int32_t* surv_idx, const double* surv_z,
                    int64_t k, int32_t* out) {
  zi_pair* p = (zi_pair*)malloc((size_t)(n > 0 ? n : 1) * sizeof(zi_pair));
  for (int64_t i = 0; i < n; ++i) {
    p[i].z = surv_z[i];
    p[i].idx = surv_idx[i];
  }
  qsort(p, (size_t)n, sizeof(zi_pair), cmp_score_desc);
  int64_t kk = n < k ? n : k;
  for (int64_t j = 0; j < kk; ++j) out[j] = p[j].idx;
  qsort(out, (size_t)kk, sizeof(int32_t), cmp_int_asc);
  for (int64_t j = kk; j < k; ++j) out[j] = -1;
  free(p);
  return kk;
}

/* ------------------------------------------------------------------------ */
/* O7 gather                                                                  */
/* ------------------------------------------------------------------------ */

void lsa_or_gather(int64_t N, int64_t row_bytes, const uint8_t* pool,
                   int64_t k, const int32_t* idx, uint8_t* hot) {
  for (int64_t j = 0; j < k; ++j) {
    if (idx[j] >= 0 && idx[j] < N)
      memcpy(hot + j * row_bytes, pool + (int64_t)idx[j] * row_bytes,
             (size_t)row_bytes);
    else
      memset(hot + j * row_bytes, 0, (size_t)row_bytes);
  }
}

/* ------------------------------------------------------------------------ */
/* O10 cold-pool fetch                                                      */
/* ------------------------------------------------------------------------ */

int64_t lsa_or_fetch(int64_t N, int64_t S, int64_t row_bytes, const uint8_t* cold,
                     int64_t n, const int32_t* surv, int32_t* slot_of,
                     int32_t* entry_of, uint8_t* rows) {
  uint8_t* is_surv = (uint8_t*)calloc((size_t)(N > 0 ? N : 1), 1);
  for (int64_t i = 0; i < n; ++i) is_surv[surv[i]] = 1;

  /* rows to copy: survivors not resident now (step 2's order) */
  int64_t need = 0, kept = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (slot_of[surv[i]] < 0) ++need;
    else ++kept;
  }
  if (kept + need > S) {
    free(is_surv);
    return -1;
  }

  /* step 1: evict */
  for (int64_t j = 0; j < S; ++j) {
    int32_t e = entry_of[j];
    if (e >= 0 && !is_surv[e]) {
      slot_of[e] = -1;
      entry_of[j] = -1;
    }
  }

  /* steps 2 and 3: ascending survivors into ascending free slots */
  int64_t j = 0;
  for (int64_t i = 0; i < n; ++i) {
    int32_t s = surv[i];
    if (slot_of[s] >= 0) continue;
    while (j < S && entry_of[j] >= 0) ++j;
    if (j >= S) break; /* unreachable after the capacity check */
    entry_of[j] = s;
    slot_of[s] = (int32_t)j;
    memcpy(rows + j * row_bytes, cold + (int64_t)s * row_bytes, (size_t)row_bytes);
  }
  free(is_surv);
  return need;
}

/* ------------------------------------------------------------------------ */
/* O8 labels                                                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
  float x;
  int64_t idx;
} xi_pair;

static int cmp_logit_desc(const void* pa, const void* pb) {
  const xi_pair* a = (const xi_pair*)pa;
  const xi_pair* b = (const xi_pair*)pb;
  if (a->x != b->x) return (a->x > b->x) ? -1 : 1;
  return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

int64_t lsa_or_nucleus(int64_t N, const float* x, double top_p, uint8_t* sel,
                       double* mass_ahead) {
  if (N <= 0) return 0;
  double m = -INFINITY;
  for (int64_t s = 0; s < N; ++s) m = fmax(m, (double)x[s]);
  double* e = (double*)malloc((size_t)N * sizeof(double));
  double S = 0.0;
  for (int64_t s = 0; s < N; ++s) {
    e[s] = exp((double)x[s] - m);
    S += e[s];
  }
  xi_pair* order = (xi_pair*)malloc((size_t)N * sizeof(xi_pair));
  for (int64_t s = 0; s < N; ++s) {
    order[s].x = x[s];
    order[s].idx = s;
  }
  qsort(order, (size_t)N, sizeof(xi_pair), cmp_logit_desc);
  double A = 0.0;   /* probability mass of the entries already walked */
  int64_t taken = 0;
  for (int64_t j = 0; j < N; ++j) {
    int64_t s = order[j].idx;
    if (mass_ahead) mass_ahead[s] = A;
    if (A < top_p) {
      sel[s] = 1;
      ++taken;
    } else {
      sel[s] = 0;
    }
    A += e[s] / S;
  }
  free(order);
  free(e);
  return taken;
}

void lsa_or_vote(int L, int64_t N, const uint8_t* sel, int theta,
                 uint8_t* count, uint8_t* label) {
  for (int64_t s = 0; s < N; ++s) {
    int c = 0;
    for (int l = 0; l < L; ++l) c += sel[(int64_t)l * N + s] ? 1 : 0;
    count[s] = (uint8_t)c;
    label[s] = (c >= theta) ? 1 : 0;
  }
}

/* ------------------------------------------------------------------------ */
/* O9 student loss + gradient                                                 */
/* ------------------------------------------------------------------------ */

/* Per-element loss terms for logit z and label y (u = margin of the true
 * class, p_t = sigmoid(u)):
 *   BCE = softplus(-u)                 (= softplus(z) - y z)
 *   FL  = (1 - p_t)^gamma * softplus(-u)
 * and d(BCE + FL)/dz. */
static void loss_terms(double z, int y, double gamma, double* bce, double* fl,
                       double* dz) {
  double sgn = y ? 1.0 : -1.0;
  double u = sgn * z;
  double nll = lsa_or_softplus(-u);          /* -log p_t */
  double p = lsa_or_sigmoid(u);
  double one_minus_p = lsa_or_sigmoid(-u);
  double mod = pow(one_minus_p, gamma);
  *bce = nll;
  *fl = mod * nll;
  if (dz) {
    double dbce = lsa_or_sigmoid(z) - (double)y;
    /* d/du [(1-p)^g * nll] with d(1-p)/du = -p(1-p) and d nll/du = -(1-p) */
    double dfl_du = -mod * (gamma * p * nll + one_minus_p);
    *dz = dbce + sgn * dfl_du;
  }
}

static double focal_core(int Q, int64_t N, int D, int H, int dI, double gamma,
                         const double* h, const double* Wq, const double* Wg,
                         double bias, const double* K, const uint8_t* y,
                         double* dWq, double* z_out) {
  const int rows = H * dI;
  double* q = (double*)malloc((size_t)Q * rows * sizeof(double));
  double* g = (double*)malloc((size_t)Q * H * sizeof(double));
  /* query encoder in training precision */
#pragma omp parallel for schedule(static)
  for (int64_t tj = 0; tj < (int64_t)Q * rows; ++tj) {
    int64_t t = tj / rows, j = tj % rows;
    double a = 0.0;
    for (int d = 0; d < D; ++d) a += Wq[j * D + d] * h[t * D + d];
    q[tj] = a;
  }
  for (int t = 0; t < Q; ++t)
    for (int hh = 0; hh < H; ++hh) {
      double a = 0.0;
      for (int d = 0; d < D; ++d) a += Wg[(int64_t)hh * D + d] * h[(int64_t)t * D + d];
      g[t * H + hh] = lsa_or_softplus(a);
    }
  /* logits, loss and dL/dz */
  double* delta = dWq ? (double*)malloc((size_t)Q * N * sizeof(double)) : NULL;
  double loss_sum = 0.0;
  const double inv = 1.0 / ((double)Q * (double)N);
#pragma omp parallel for schedule(static) reduction(+ : loss_sum)
  for (int64_t ts = 0; ts < (int64_t)Q * N; ++ts) {
    int64_t t = ts / N, s = ts % N;
    double z = 0.0;
    for (int hh = 0; hh < H; ++hh) {
      double dot = 0.0;
      for (int d = 0; d < dI; ++d)
        dot += q[t * rows + hh * dI + d] * K[s * dI + d];
      z += g[t * H + hh] * dot;
    }
    z += bias;
    if (z_out) z_out[ts] = z;
    double bce, fl, dz;
    loss_terms(z, y[ts] ? 1 : 0, gamma, &bce, &fl, delta ? &dz : NULL);
    loss_sum += bce + fl;
    if (delta) delta[ts] = dz * inv;
  }
  if (dWq) {
    /* dL/dq_thd = g_th * sum_s delta_ts k_sd ; dL/dWq[(h,d), j] = sum_t dL/dq_thd h_tj */
    double* G = (double*)malloc((size_t)Q * dI * sizeof(double));
#pragma omp parallel for schedule(static)
    for (int64_t td = 0; td < (int64_t)Q * dI; ++td) {
      int64_t t = td / dI, d = td % dI;
      double acc = 0.0;
      for (int64_t s = 0; s < N; ++s) acc += delta[t * N + s] * K[s * dI + d];
      G[td] = acc;
    }
#pragma omp parallel for schedule(static)
    for (int64_t jd = 0; jd < (int64_t)rows * D; ++jd) {
      int64_t j = jd / D, c = jd % D;
      int64_t hh = j / dI, d = j % dI;
      double acc = 0.0;
      for (int t = 0; t < Q; ++t)
        acc += g[t * H + hh] * G[t * dI + d] * h[(int64_t)t * D + c];
      dWq[jd] = acc;
    }
    free(G);
    free(delta);
  }
  free(q);
  free(g);
  return loss_sum * inv;
}

double lsa_or_focal_bce_grad(int Q, int64_t N, int D, int H, int dI,
                             double gamma, const uint16_t* h, const float* Wq,
                             const float* Wg, double bias, const uint16_t* K,
                             const uint8_t* y, double* dWq, double* z_out) {
  const int64_t rows = (int64_t)H * dI;
  double* h64 = (double*)malloc((size_t)Q * D * sizeof(double));
  double* Wq64 = (double*)malloc((size_t)rows * D * sizeof(double));
  double* Wg64 = (double*)malloc((size_t)H * D * sizeof(double));
  double* K64 = (double*)malloc((size_t)N * dI * sizeof(double));
  for (int64_t i = 0; i < (int64_t)Q * D; ++i) h64[i] = lsa_or_bf16_to_double(h[i]);
  for (int64_t i = 0; i < rows * D; ++i) Wq64[i] = (double)Wq[i];
  for (int64_t i = 0; i < (int64_t)H * D; ++i) Wg64[i] = (double)Wg[i];
  for (int64_t i = 0; i < N * dI; ++i) K64[i] = lsa_or_bf16_to_double(K[i]);
  double loss = focal_core(Q, N, D, H, dI, gamma, h64, Wq64, Wg64, bias, K64,
                           y, dWq, z_out);
  free(h64);
  free(Wq64);
  free(Wg64);
  free(K64);
  return loss;
}

double lsa_or_focal_bce_loss64(int Q, int64_t N, int D, int H, int dI,
                               double gamma, const double* h, const double* Wq,
                               const double* Wg, double bias, const double* K,
                               const uint8_t* y) {
  return focal_core(Q, N, D, H, dI, gamma, h, Wq, Wg, bias, K, y, NULL, NULL);
}

/* ------------------------------------------------------------------------ */
/* O11 core attention over the selected rows                                 */
/* ------------------------------------------------------------------------ */

void lsa_or_attention(int64_t n, int D, int H, const uint16_t* q,
                      const uint16_t* rows, double scale, double* out,
                      double* wabs) {
#pragma omp parallel for schedule(static)
  for (int hh = 0; hh < H; ++hh) {
    double* o = out + (int64_t)hh * D;
    double* wa = wabs ? wabs + (int64_t)hh * D : NULL;
    for (int d = 0; d < D; ++d) {
      o[d] = 0.0;
      if (wa) wa[d] = 0.0;
    }
    if (n <= 0) continue;
    double* s = (double*)malloc((size_t)n * sizeof(double));
    /* scores */
    for (int64_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += lsa_or_bf16_to_double(q[(int64_t)hh * D + d]) *
               lsa_or_bf16_to_double(rows[j * D + d]);
      s[j] = scale * dot;
    }
    /* softmax weights, shifted by the maximum score */
    double m = s[0];
    for (int64_t j = 1; j < n; ++j) m = fmax(m, s[j]);
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      s[j] = exp(s[j] - m);
      sum += s[j];
    }
    /* weighted sum of the rows */
    for (int64_t j = 0; j < n; ++j) {
      double p = s[j] / sum;
      for (int d = 0; d < D; ++d) {
        double v = lsa_or_bf16_to_double(rows[j * D + d]);
        o[d] += p * v;
        if (wa) wa[d] += p * fabs(v);
      }
    }
    free(s);
  }
}

/* ------------------------------------------------------------------------ */
/* O13 fine-grained score inside the fetched set                             */
/* ------------------------------------------------------------------------ */

void lsa_or_lightning(int N, int H, int dI, int key_dtype, const void* keys,
                      const float* scale, const uint16_t* q, const float* w,
                      const int32_t* idx, int64_t n, double* out) {
  (void)N;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int64_t s = idx[i];
    const double sigma = (key_dtype == 1 && scale) ? (double)scale[s] : 1.0;
    double acc = 0.0;
    for (int hh = 0; hh < H; ++hh) {
      double dot = 0.0;
      for (int d = 0; d < dI; ++d)
        dot += lsa_or_bf16_to_double(q[hh * dI + d]) * key_value(key_dtype, keys, s * dI + d);
      acc += (double)w[hh] * fmax(0.0, dot * sigma);
    }
    out[i] = acc;
  }
}
