/*
 * HGA reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of what the Hierarchical Global
 * Attention hot path computes.  Only tests/, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no code, header,
 * table or helper with the GPU library; the two meet only through the seeded
 * inputs that synth/ produces.
 *
 * Source of every definition: "Technische Samenvatting: Hierarchical Global
 * Attention (HGA)" (gist.science summary of the HGA paper), section
 * "Kernmechanisme":
 *   item 1  fixed-size chunks (C tokens), each split into groups;
 *   item 2  level-1 routing of the current query against chunk key summaries,
 *           level-2 routing against the group key summaries of the chosen
 *           chunks, and the always-visible current / sink / local chunks;
 *   item 3  RoPE-aware summaries: high-frequency pairs are rotated per token
 *           and then averaged, low-frequency pairs are averaged in raw key
 *           space and then rotated to the chunk's representative position;
 *   item 4  exact softmax attention over the original token K/V of the
 *           selected set (no summary enters the output).
 * Where the page leaves a step open, this file takes the plainest reading:
 *   - RoPE pairs are (x_j, x_{j+d/2}) with omega_j = theta^(-2j/d);
 *   - pair j is high-frequency iff its wavelength 2*pi/omega_j is below a
 *     configured threshold (the chunk size), the same split for chunk and
 *     group summaries;
 *   - a span's representative position is its midpoint a + (n-1)/2;
 *   - group summaries use the same mixed rule over the group's own span;
 *   - routing is per (sequence, KV head) with the query pooled as the mean of
 *     the rotated queries of that KV head's query heads (and query tokens);
 *   - level 2 keeps a single global top-k over all groups of the chosen
 *     chunks; candidates are the complete chunks strictly between the sink
 *     and local windows; ties order by (score descending, id ascending);
 *   - pool keys are stored rotated and rounded once (bf16 RNE, or fp32).
 *
 * Parity pins: every function here is checked in tests/test_oracle_pins.py
 * against closed forms, library routines or brute force.  No function is
 * "parity unpinned".
 *
 * All arithmetic is IEEE fp64 in the order written; loops are plain.  The
 * only library primitives are libm (pow, sin, cos, exp, log, frexp, ldexp,
 * nearbyint) and qsort.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int d;              /* head dim, even */
  int hq;             /* query heads */
  int hkv;            /* key/value heads; hq % hkv == 0 */
  int C;              /* chunk size in tokens */
  int G;              /* groups per chunk; C % G == 0 */
  int n_sink;         /* always-visible leading chunks */
  int n_local;        /* always-visible chunks just before the current one */
  int topk_c;         /* level-1 chunk budget */
  int topk_g;         /* level-2 group budget */
  double theta;       /* RoPE base */
  double hf_wavelength; /* pair j is high-frequency iff 2*pi/omega_j < this */
  int pool_bf16;      /* 1: pool keys stored as bf16 (RNE); 0: as fp32 (RNE) */
  int rep_integer;    /* representative position of a span: 0: a + (n-1)/2; 1: a + n/2 */
  int rope_interleaved; /* RoPE pairs: 0: (x_j, x_{j+d/2}); 1: (x_{2j}, x_{2j+1}) */
  int route_max;      /* routing query of a KV head's query heads: 0: their mean;
                         1: each head's own (mean over the query tokens), a
                         candidate scoring the largest of the heads' scores */
} ora_cfg;

/* ---------------------------------------------------------------- RoPE
 * Pairs are (x_j, x_{j+d/2}) for j < d/2 (half-split convention) or, with
 * rope_interleaved, (x_{2j}, x_{2j+1}) (the interleaved variant; the page
 * does not say which).  Pair j
 * turns at angular frequency omega_j = theta^(-2j/d); at position p it is
 * rotated by the angle p*omega_j:  (a, b) -> (a cos - b sin, a sin + b cos).
 */
/* Dims of the two members of pair j: half-split (j, j + d/2) or, in the
 * interleaved variant, (2j, 2j + 1). */
static int pa(const ora_cfg* c, int j) { return c->rope_interleaved ? 2 * j : j; }
static int pb(const ora_cfg* c, int j) { return c->rope_interleaved ? 2 * j + 1 : j + c->d / 2; }

double ora_omega(const ora_cfg* c, int j) {
  return pow(c->theta, -2.0 * (double)j / (double)c->d);
}

int ora_is_hf(const ora_cfg* c, int j) {
  double wavelength = 2.0 * M_PI / ora_omega(c, j);
  return wavelength < c->hf_wavelength;
}

/* Rotate vector x (length d) to position pos (pos may be fractional). */
void ora_rope(const ora_cfg* c, const double* x, double pos, double* out) {
  int h = c->d / 2;
  for (int j = 0; j < h; ++j) {
    double ang = pos * ora_omega(c, j);
    double cs = cos(ang), sn = sin(ang);
    double a = x[pa(c, j)], b = x[pb(c, j)];
    out[pa(c, j)] = a * cs - b * sn;
    out[pb(c, j)] = a * sn + b * cs;
  }
}

/* --------------------------------------------------------- summaries
 * Summary of the span of n tokens starting at position a (raw, pre-RoPE keys
 * kraw[n][d]).  Representative position r = a + (n-1)/2 (the span midpoint;
 * the page does not fix it), or a + n/2 with rep_integer (the variant).
 *   HF pair j: mean over the span of the per-token rotated pair.
 *   LF pair j: the mean raw pair, rotated to r.
 */
void ora_span_summary(const ora_cfg* c, const double* kraw, long a, int n, double* out) {
  int d = c->d, h = d / 2;
  double r = (double)a + (c->rep_integer ? 0.5 * (double)n : 0.5 * (double)(n - 1));
  for (int j = 0; j < h; ++j) {
    double w = ora_omega(c, j);
    double sa = 0.0, sb = 0.0;
    if (ora_is_hf(c, j)) {
      for (int i = 0; i < n; ++i) {
        double ang = (double)(a + i) * w;
        double ka = kraw[(long)i * d + pa(c, j)], kb = kraw[(long)i * d + pb(c, j)];
        sa += ka * cos(ang) - kb * sin(ang);
        sb += ka * sin(ang) + kb * cos(ang);
      }
      out[pa(c, j)] = sa / n;
      out[pb(c, j)] = sb / n;
    } else {
      for (int i = 0; i < n; ++i) {
        sa += kraw[(long)i * d + pa(c, j)];
        sb += kraw[(long)i * d + pb(c, j)];
      }
      sa /= n;
      sb /= n;
      out[pa(c, j)] = sa * cos(r * w) - sb * sin(r * w);
      out[pb(c, j)] = sa * sin(r * w) + sb * cos(r * w);
    }
  }
}

/* Summaries of every complete chunk and group of one (sequence, KV head):
 * kraw[T][d] -> chunk_sum[T/C][d], group_sum[(T/C)*G][d]. */
void ora_summaries(const ora_cfg* c, const double* kraw, long T, double* chunk_sum, double* group_sum) {
  int d = c->d, g = c->C / c->G;
  long nch = T / c->C;
  for (long ch = 0; ch < nch; ++ch) {
    long a = ch * c->C;
    ora_span_summary(c, kraw + a * d, a, c->C, chunk_sum + ch * d);
    for (int i = 0; i < c->G; ++i) {
      long ga = a + (long)i * g;
      ora_span_summary(c, kraw + ga * d, ga, g, group_sum + (ch * c->G + i) * d);
    }
  }
}

/* -------------------------------------------------------------- pool
 * Round-to-nearest-even of an fp64 value to bf16 (8 significant bits, fp32
 * exponent range), done directly from fp64 so there is no double rounding. */
double ora_round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  double m = frexp(x, &e);        /* x = m * 2^e, 0.5 <= |m| < 1 */
  int q = e - 8;                  /* weight of the last kept bit */
  if (q < -133) q = -133;         /* bf16 subnormal quantum is 2^-133 */
  double s = ldexp(x, -q);
  return ldexp(nearbyint(s), q);  /* default rounding mode: ties to even */
}

void ora_round_bf16_vec(const double* x, long n, double* out) {
  for (long i = 0; i < n; ++i) out[i] = ora_round_bf16(x[i]);
}

/* Rotated pool keys for tokens pos0..pos0+n-1: round(RoPE(k, p)). */
void ora_pool(const ora_cfg* c, const double* kraw, long pos0, long n, double* kpool) {
  int d = c->d;
  for (long i = 0; i < n; ++i) {
    ora_rope(c, kraw + i * d, (double)(pos0 + i), kpool + i * d);
    for (int e = 0; e < d; ++e) {
      double v = kpool[i * d + e];
      kpool[i * d + e] = c->pool_bf16 ? ora_round_bf16(v) : (double)(float)v;
    }
  }
}

/* ------------------------------------------------ windows, candidates
 * For the current chunk ct:
 *   sink chunks   [0, min(n_sink, ct))
 *   local chunks  [max(0, ct - n_local), ct)
 *   candidates    n_sink <= ch < ct - n_local (complete chunks only).
 * Returns the number of window chunks written to win (ascending, no
 * duplicates) and sets *cand_lo, *cand_hi to the candidate range. */
int ora_windows(const ora_cfg* c, long ct, long* win, long* cand_lo, long* cand_hi) {
  int n = 0;
  for (long ch = 0; ch < ct; ++ch) {
    int in_sink = ch < c->n_sink;
    int in_local = ch >= ct - c->n_local;
    if (in_sink || in_local) win[n++] = ch;
  }
  *cand_lo = c->n_sink;
  *cand_hi = ct - c->n_local;
  if (*cand_hi < *cand_lo) *cand_hi = *cand_lo;
  return n;
}

/* ------------------------------------------------------ selection */
typedef struct {
  double s;
  long id;
} ora_item;

static int by_score_desc_id_asc(const void* x, const void* y) {
  const ora_item* a = (const ora_item*)x;
  const ora_item* b = (const ora_item*)y;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

static int by_id(const void* x, const void* y) {
  long a = *(const long*)x, b = *(const long*)y;
  return (a > b) - (a < b);
}

static double dot(const double* x, const double* y, int d) {
  double s = 0.0;
  for (int i = 0; i < d; ++i) s += x[i] * y[i];
  return s;
}

/* Pooled routing query of one KV head: mean over its hg query heads and lq
 * query tokens (positions pos0..pos0+lq-1) of RoPE(q, position).
 * q is [hg][lq][d], raw (pre-RoPE). */
/* ------------------------------------------------------ fp8 pool
 * The FP8 pool variant stores each (token, KV head) row of the rotated keys,
 * and of the values, as OCP E4M3FN codes times one power-of-two scale.
 * E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; normal values
 * (1 + m/8) 2^(e-7) for e = 1..15 (except e = 15, m = 7: NaN), subnormal
 * values m 2^-9; the largest finite value is 448.
 * Scale of a row: the smallest power of two s with max|x| <= 448 s (1 for a
 * zero row); codes: x / s (exact) rounded to nearest even E4M3FN. */
double ora_fp8_scale(double amax) {
  if (!(amax > 0.0)) return 1.0;
  int E;
  double f = 2.0 * frexp(amax, &E);  /* amax = f 2^(E-1), f in [1, 2) */
  E -= 1;
  /* amax <= 1.75 2^(8+k) <=> f 2^(E-8-k) <= 1.75 */
  int k = f <= 1.75 ? E - 8 : E - 7;
  return ldexp(1.0, k);
}

/* |y| <= 448 -> E4M3FN code, rounding to nearest even. */
int ora_fp8_encode(double y) {
  int sign = y < 0.0 ? 0x80 : 0;
  double a = fabs(y);
  if (a == 0.0) return sign;
  int E;
  frexp(a, &E);
  E -= 1;                       /* a in [2^E, 2^(E+1)) */
  if (E < -6) {                 /* subnormal range: quantum 2^-9 */
    double m = rint(a * 512.0);
    if (m >= 8.0) return sign | (1 << 3);  /* rounds up to 2^-6 */
    return sign | (int)m;
  }
  double q = rint(ldexp(a, 3 - E));  /* 8..16 */
  if (q >= 16.0) {
    q = 8.0;
    E += 1;
  }
  return sign | ((E + 7) << 3) | ((int)q - 8);
}

double ora_fp8_decode(int code) {
  int e = (code >> 3) & 15, m = code & 7;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  if (e == 15 && m == 7) v = NAN;
  return (code & 0x80) ? -v : v;
}

/* Quantise rows x[n][d] (fp64): codes[n][d] and scales[n]; deq[n][d] (nullable)
 * receives code values times scale. */
void ora_fp8_rows(const double* x, long n, int d, int* codes, double* scales, double* deq) {
  for (long i = 0; i < n; ++i) {
    double amax = 0.0;
    for (int e = 0; e < d; ++e) amax = fmax(amax, fabs(x[i * d + e]));
    double sc = ora_fp8_scale(amax);
    scales[i] = sc;
    for (int e = 0; e < d; ++e) {
      int cd = ora_fp8_encode(x[i * d + e] / sc);
      codes[i * d + e] = cd;
      if (deq) deq[i * d + e] = ora_fp8_decode(cd) * sc;
    }
  }
}

/* FP8 pool keys: the rotated keys (fp64, unrounded) quantised per row. */
void ora_pool_fp8(const ora_cfg* c, const double* kraw, long pos0, long n, int* codes,
                  double* scales, double* deq) {
  int d = c->d;
  double* rot = (double*)malloc(sizeof(double) * d * n);
  for (long i = 0; i < n; ++i) ora_rope(c, kraw + i * d, (double)(pos0 + i), rot + i * d);
  ora_fp8_rows(rot, n, d, codes, scales, deq);
  free(rot);
}

void ora_pooled_query(const ora_cfg* c, const double* q, int hg, int lq, long pos0, double* qbar) {
  int d = c->d;
  double* tmp = (double*)malloc(sizeof(double) * d);
  for (int e = 0; e < d; ++e) qbar[e] = 0.0;
  for (int h = 0; h < hg; ++h)
    for (int t = 0; t < lq; ++t) {
      ora_rope(c, q + ((long)h * lq + t) * d, (double)(pos0 + t), tmp);
      for (int e = 0; e < d; ++e) qbar[e] += tmp[e];
    }
  for (int e = 0; e < d; ++e) qbar[e] /= (double)(hg * lq);
  free(tmp);
}

/* The routing queries of one KV head from q [hg][lq][d] at positions pos0..
 * into qb: one (route_max = 0: the mean of every rotated query row of the
 * head's query heads and tokens) or hg (route_max = 1: per query head, the
 * mean of its rotated query tokens).  Returns their number. */
static int ora_route_queries(const ora_cfg* c, const double* q, int hg, int lq, long pos0,
                             double* qb) {
  int d = c->d;
  if (!c->route_max) {
    ora_pooled_query(c, q, hg, lq, pos0, qb);
    return 1;
  }
  for (int h = 0; h < hg; ++h) ora_pooled_query(c, q + (long)h * lq * d, 1, lq, pos0, qb + (long)h * d);
  return hg;
}

/* Routing score of a summary row s: the largest of qb[i] . s / sqrt(d) over
 * the nq routing queries (the only one with the mean query). */
static double ora_route_score(const double* qb, int nq, const double* s, int d, double inv_sqrt_d) {
  double best = -INFINITY;
  for (int i = 0; i < nq; ++i) {
    const double v = dot(qb + (long)i * d, s, d) * inv_sqrt_d;
    if (v > best) best = v;
  }
  return best;
}

/* Level-2 routing score of every group id g < n_groups against the routing
 * queries that ora_select forms from q [hg][lq][d] at positions pos0.. (the
 * scores of the groups of the chosen chunks are the ones level 2 ranks). */
void ora_group_scores(const ora_cfg* c, const double* q, int lq, long pos0,
                      const double* group_sum, long n_groups, double* out) {
  int d = c->d, hg = c->hq / c->hkv;
  double* qb = (double*)malloc(sizeof(double) * d * hg);
  const int nq = ora_route_queries(c, q, hg, lq, pos0, qb);
  for (long g = 0; g < n_groups; ++g)
    out[g] = ora_route_score(qb, nq, group_sum + g * d, d, 1.0 / sqrt((double)d));
  free(qb);
}

/* Two-level selection for one (sequence, KV head).
 *   q           [hg][lq][d] raw query of the KV head's query heads
 *   pos0, lq    query tokens pos0..pos0+lq-1, all inside chunk ct
 *   chunk_sum   [>= ct][d], group_sum [>= ct*G][d]
 * Writes the ascending list of selected group ids (window chunks expanded to
 * all their groups, the current chunk's groups up to the last query token,
 * and the routed groups) and returns its length, or -1 if max_sel is too
 * small.  margins[0], margins[1] receive the level-1 and level-2 score gaps
 * between the last kept and first dropped item (INFINITY when nothing is
 * dropped).  cand_scores (optional) receives the level-1 scores of the
 * candidate chunks in chunk order. */
int ora_select(const ora_cfg* c, const double* q, int lq, long pos0, const double* chunk_sum,
               const double* group_sum, int* sel_groups, int max_sel, double* margins,
               double* cand_scores) {
  int d = c->d, G = c->G, g = c->C / c->G, hg = c->hq / c->hkv;
  long ct = pos0 / c->C;
  long last = pos0 + lq - 1;
  double inv_sqrt_d = 1.0 / sqrt((double)d);

  double* qb = (double*)malloc(sizeof(double) * d * hg);
  const int nq = ora_route_queries(c, q, hg, lq, pos0, qb);

  long* win = (long*)malloc(sizeof(long) * (ct + 1));
  long lo, hi;
  int nwin = ora_windows(c, ct, win, &lo, &hi);
  long ncand = hi - lo;

  /* level 1 */
  ora_item* l1 = (ora_item*)malloc(sizeof(ora_item) * (ncand > 0 ? ncand : 1));
  for (long i = 0; i < ncand; ++i) {
    l1[i].id = lo + i;
    l1[i].s = ora_route_score(qb, nq, chunk_sum + (lo + i) * d, d, inv_sqrt_d);
    if (cand_scores) cand_scores[i] = l1[i].s;
  }
  qsort(l1, ncand, sizeof(ora_item), by_score_desc_id_asc);
  long k1 = c->topk_c < ncand ? c->topk_c : ncand;
  margins[0] = (k1 < ncand) ? l1[k1 - 1].s - l1[k1].s : INFINITY;
  if (k1 == 0) margins[0] = INFINITY;

  /* level 2: global top-k over all groups of the chosen chunks */
  long n2 = k1 * G;
  ora_item* l2 = (ora_item*)malloc(sizeof(ora_item) * (n2 > 0 ? n2 : 1));
  for (long i = 0; i < k1; ++i)
    for (int j = 0; j < G; ++j) {
      long gid = l1[i].id * G + j;
      l2[i * G + j].id = gid;
      l2[i * G + j].s = ora_route_score(qb, nq, group_sum + gid * d, d, inv_sqrt_d);
    }
  qsort(l2, n2, sizeof(ora_item), by_score_desc_id_asc);
  long k2 = c->topk_g < n2 ? c->topk_g : n2;
  margins[1] = (k2 < n2) ? l2[k2 - 1].s - l2[k2].s : INFINITY;
  if (k2 == 0) margins[1] = INFINITY;

  /* union with the windows, then sort ascending */
  long cap = (long)nwin * G + (last / g - ct * G + 1) + k2;
  long* ids = (long*)malloc(sizeof(long) * cap);
  long n = 0;
  for (int w = 0; w < nwin; ++w)
    for (int j = 0; j < G; ++j) ids[n++] = win[w] * G + j;
  for (long gid = ct * G; gid <= last / g; ++gid) ids[n++] = gid;
  for (long i = 0; i < k2; ++i) ids[n++] = l2[i].id;
  qsort(ids, n, sizeof(long), by_id);

  int ret = (n <= max_sel) ? (int)n : -1;
  if (ret >= 0)
    for (long i = 0; i < n; ++i) sel_groups[i] = (int)ids[i];

  free(ids);
  free(l2);
  free(l1);
  free(win);
  free(qb);
  return ret;
}

/* ------------------------------------------------- exact attention
 * For each query head of one KV head and each query token tau
 * (pos0..pos0+lq-1): softmax over the selected tokens p <= tau of
 * RoPE(q, tau) . kpool[p] / sqrt(d), applied to vpool.
 *   q [hg][lq][d] raw; kpool/vpool [T][d] for this KV head;
 *   out [hg][lq][d]; lse [hg][lq] (optional) = log sum exp of the logits. */
void ora_attend(const ora_cfg* c, const double* q, int lq, long pos0, const double* kpool,
                const double* vpool, const int* sel_groups, int n_sel, double* out, double* lse) {
  int d = c->d, g = c->C / c->G, hg = c->hq / c->hkv;
  double inv_sqrt_d = 1.0 / sqrt((double)d);
  long ntok = (long)n_sel * g;
  double* qr = (double*)malloc(sizeof(double) * d);
  double* lg = (double*)malloc(sizeof(double) * (ntok > 0 ? ntok : 1));
  for (int h = 0; h < hg; ++h)
    for (int t = 0; t < lq; ++t) {
      long tau = pos0 + t;
      ora_rope(c, q + ((long)h * lq + t) * d, (double)tau, qr);
      double m = -INFINITY;
      for (long i = 0; i < ntok; ++i) {
        long p = (long)sel_groups[i / g] * g + i % g;
        lg[i] = (p <= tau) ? dot(qr, kpool + p * d, d) * inv_sqrt_d : -INFINITY;
        if (lg[i] > m) m = lg[i];
      }
      double den = 0.0;
      double* o = out + ((long)h * lq + t) * d;
      for (int e = 0; e < d; ++e) o[e] = 0.0;
      for (long i = 0; i < ntok; ++i) {
        if (lg[i] == -INFINITY) continue;
        long p = (long)sel_groups[i / g] * g + i % g;
        double w = exp(lg[i] - m);
        den += w;
        for (int e = 0; e < d; ++e) o[e] += w * vpool[p * d + e];
      }
      for (int e = 0; e < d; ++e) o[e] /= den;
      if (lse) lse[(long)h * lq + t] = m + log(den);
    }
  free(lg);
  free(qr);
}

/* Exact merge of two attention results over disjoint token sets, each given
 * as (normalised output, log-sum-exp).  n rows of d values. */
void ora_merge(int d, long n, const double* oa, const double* la, const double* ob,
               const double* lb, double* out, double* lse) {
  for (long r = 0; r < n; ++r) {
    double m = la[r] > lb[r] ? la[r] : lb[r];
    double wa = exp(la[r] - m), wb = exp(lb[r] - m);
    for (int e = 0; e < d; ++e) out[r * d + e] = (wa * oa[r * d + e] + wb * ob[r * d + e]) / (wa + wb);
    if (lse) lse[r] = m + log(wa + wb);
  }
}

/* Gather: copy the selected groups' token rows of one (sequence, KV head)
 * pool [T][d] into a compact working set [n_sel*g][d].  Values are copied,
 * never computed. */
void ora_gather(const ora_cfg* c, const double* pool, const int* sel_groups, int n_sel, double* ws) {
  int d = c->d, g = c->C / c->G;
  for (int s = 0; s < n_sel; ++s)
    memcpy(ws + (long)s * g * d, pool + (long)sel_groups[s] * g * d, sizeof(double) * g * d);
}

/* ----------------------------------------------------------- warm tier
 * "Geheugenarchitectuur": between the hot tier (summaries and the always
 * visible windows in accelerator memory) and the cold tier (the full token
 * K/V history in host memory) sits a bounded least-recently-used cache in
 * accelerator memory of recently routed data.  One call for one unit:
 *   n_warm slots, tags[s] = the cached group id (-1: empty), used[s] = the
 *   step that last used the slot (0: never); routed[0..n) the distinct group
 *   ids the routing chose this step, in list order.
 *   A routed group found among the tags is a hit: its slot's stamp becomes
 *   `step`.  The misses, in list order, take the slots that are not hits in
 *   increasing order of (stamp, slot index) -- the least recently used first,
 *   empty slots (stamp 0) before any used one -- one slot each; a taken
 *   slot's tag becomes the group and its stamp `step`.
 * slot[i] receives the slot holding routed[i] after the call, hit[i] 1 for a
 * hit.  Returns the number of hits, or -1 if the misses outnumber the slots
 * that are not hits (nothing is changed then). */
int ora_warm_step(int n_warm, int* tags, int* used, const int* routed, int n, int step, int* slot,
                  int* hit) {
  int* is_hit = (int*)calloc(n_warm > 0 ? n_warm : 1, sizeof(int));
  int n_hit = 0, n_miss = 0;
  for (int i = 0; i < n; ++i) {
    slot[i] = -1;
    hit[i] = 0;
    for (int s = 0; s < n_warm; ++s)
      if (tags[s] == routed[i]) {
        slot[i] = s;
        hit[i] = 1;
        is_hit[s] = 1;
      }
    if (hit[i]) n_hit += 1;
    else n_miss += 1;
  }
  if (n_miss > n_warm - n_hit) {
    free(is_hit);
    return -1;
  }
  for (int i = 0; i < n; ++i)
    if (hit[i]) used[slot[i]] = step;
  /* each miss in turn takes the least recently used slot still free */
  int* taken = (int*)calloc(n_warm > 0 ? n_warm : 1, sizeof(int));
  for (int i = 0; i < n; ++i) {
    if (hit[i]) continue;
    int best = -1;
    for (int s = 0; s < n_warm; ++s) {
      if (is_hit[s] || taken[s]) continue;
      if (best < 0 || used[s] < used[best]) best = s; /* ties keep the lower slot index */
    }
    taken[best] = 1;
    slot[i] = best;
  }
  for (int i = 0; i < n; ++i)
    if (!hit[i]) {
      tags[slot[i]] = routed[i];
      used[slot[i]] = step;
    }
  free(taken);
  free(is_hit);
  return n_hit;
}

/* ------------------------------------------------ batched driver (timing)
 * One decode/prefill step over nunits independent (sequence, KV head)
 * units: selection then attention, one unit per OpenMP thread.  Per-unit
 * arrays are laid out back to back:
 *   q [nunits][hg][lq][d], pos0 [nunits], chunk_sum [nunits][nch][d],
 *   group_sum [nunits][nch*G][d], kpool/vpool [nunits][T][d],
 *   sel [nunits][max_sel], nsel [nunits], out [nunits][hg][lq][d]. */
int ora_step(const ora_cfg* c, int nunits, const double* q, int lq, const long* pos0,
             const double* chunk_sum, const double* group_sum, long nch, const double* kpool,
             const double* vpool, long T, int* sel, int* nsel, int max_sel, double* out) {
  int d = c->d, hg = c->hq / c->hkv, bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
  for (int u = 0; u < nunits; ++u) {
    double margins[2];
    const double* qu = q + (long)u * hg * lq * d;
    int n = ora_select(c, qu, lq, pos0[u], chunk_sum + (long)u * nch * d,
                       group_sum + (long)u * nch * c->G * d, sel + (long)u * max_sel, max_sel,
                       margins, NULL);
    nsel[u] = n;
    if (n < 0) {
      bad += 1;
      continue;
    }
    ora_attend(c, qu, lq, pos0[u], kpool + (long)u * T * d, vpool + (long)u * T * d,
               sel + (long)u * max_sel, n, out + (long)u * hg * lq * d, NULL);
  }
  return bad;
}

int ora_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the batched driver's parallel loop (timing only; results do
 * not depend on it: each unit is computed by one thread, in the same order). */
void ora_set_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}
