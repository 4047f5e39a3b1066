/*
 * Drives every function of hga_oracle.c once on small inputs, for a build
 * under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
 *   gcc -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all \
 *       -fno-omit-frame-pointer -fopenmp oracle/hga_oracle.c \
 *       oracle/sanitize_check.c -lm -o sanitize_check
 * Any out-of-bounds access, use after free, leak or undefined operation ends
 * the program with a report; a clean run prints "sanitize ok".  Test
 * infrastructure, like the oracle itself.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int d, hq, hkv, C, G, n_sink, n_local, topk_c, topk_g;
  double theta, hf_wavelength;
  int pool_bf16, rep_integer, rope_interleaved, route_max;
} ora_cfg;

double ora_omega(const ora_cfg* c, int j);
int ora_is_hf(const ora_cfg* c, int j);
void ora_rope(const ora_cfg* c, const double* x, double pos, double* out);
void ora_span_summary(const ora_cfg* c, const double* kraw, long a, int n, double* out);
void ora_summaries(const ora_cfg* c, const double* kraw, long T, double* cs, double* gs);
double ora_round_bf16(double x);
void ora_round_bf16_vec(const double* x, long n, double* out);
void ora_pool(const ora_cfg* c, const double* kraw, long pos0, long n, double* kpool);
double ora_fp8_scale(double amax);
int ora_fp8_encode(double y);
double ora_fp8_decode(int code);
void ora_fp8_rows(const double* x, long n, int d, int* codes, double* scales, double* deq);
void ora_pool_fp8(const ora_cfg* c, const double* kraw, long pos0, long n, int* codes,
                  double* scales, double* deq);
int ora_windows(const ora_cfg* c, long ct, long* win, long* cand_lo, long* cand_hi);
void ora_pooled_query(const ora_cfg* c, const double* q, int hg, int lq, long pos0, double* qbar);
void ora_group_scores(const ora_cfg* c, const double* q, int lq, long pos0,
                      const double* group_sum, long n_groups, double* out);
int ora_select(const ora_cfg* c, const double* q, int lq, long pos0, const double* chunk_sum,
               const double* group_sum, int* sel_groups, int max_sel, double* margins,
               double* cand_scores);
void ora_attend(const ora_cfg* c, const double* q, int lq, long pos0, const double* kpool,
                const double* vpool, const int* sel_groups, int n_sel, double* out, double* lse);
void ora_merge(int d, long n, const double* oa, const double* la, const double* ob,
               const double* lb, double* out, double* lse);
void ora_gather(const ora_cfg* c, const double* pool, const int* sel_groups, int n_sel, double* ws);
int ora_warm_step(int n_warm, int* tags, int* used, const int* routed, int n, int step, int* slot,
                  int* hit);
int ora_step(const ora_cfg* c, int nunits, const double* q, int lq, const long* pos0,
             const double* chunk_sum, const double* group_sum, long nch, const double* kpool,
             const double* vpool, long T, int* sel, int* nsel, int max_sel, double* out);
int ora_max_threads(void);

static unsigned long long rng_state = 88172645463325252ull;
static double urand(void) { /* xorshift64, then a uniform in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 4503599627370496.0 - 1.0;
}
static double* randv(long n) {
  double* x = (double*)malloc(sizeof(double) * n);
  for (long i = 0; i < n; ++i) x[i] = urand();
  return x;
}

int main(void) {
  const int d = 64, hq = 4, hkv = 2, hg = 2, T = 1024, C = 64, G = 4;
  const long nch = T / C;
  for (int variant = 0; variant < 4; ++variant) {
    ora_cfg c = {d, hq, hkv, C, G, 1, 2, 3, 6, 1e4, 64.0, variant & 1, variant >> 1, variant & 1,
                 variant >> 1};
    double* kraw = randv((long)T * d);
    double* v = randv((long)T * d);
    double* q = randv((long)hg * 3 * d);
    double* cs = (double*)malloc(sizeof(double) * nch * d);
    double* gs = (double*)malloc(sizeof(double) * nch * G * d);
    double* kp = (double*)malloc(sizeof(double) * T * d);
    double out[64];
    for (int j = 0; j < d / 2; ++j) (void)(ora_omega(&c, j) + ora_is_hf(&c, j));
    ora_rope(&c, kraw, 12.5, out);
    ora_span_summary(&c, kraw, 0, 16, out);
    ora_summaries(&c, kraw, T, cs, gs);
    (void)ora_round_bf16(urand());
    ora_round_bf16_vec(kraw, d, out);
    ora_pool(&c, kraw, 0, T, kp);
    int* codes = (int*)malloc(sizeof(int) * 16 * d);
    double scales[16], deq[16 * 64];
    ora_pool_fp8(&c, kraw, 100, 16, codes, scales, deq);
    ora_fp8_rows(v, 16, d, codes, scales, deq);
    for (int code = 0; code < 256; ++code) (void)ora_fp8_decode(code);
    (void)ora_fp8_encode(0.0);
    (void)ora_fp8_encode(447.9);
    (void)ora_fp8_encode(-1e-4);
    (void)ora_fp8_scale(0.0);
    (void)ora_fp8_scale(3e5);
    long win[16], lo, hi;
    for (long ct = 0; ct < nch; ++ct) (void)ora_windows(&c, ct, win, &lo, &hi);
    double qbar[64], gsc[64], margins[2], cand[16];
    ora_pooled_query(&c, q, hg, 3, 64 * 9 + 5, qbar);
    ora_group_scores(&c, q, 3, 64 * 9 + 5, gs, 9 * G, gsc);
    int sel[64];
    for (long pos = 0; pos < T; pos += 37) {
      int n = ora_select(&c, q, 1, pos, cs, gs, sel, 64, margins, cand);
      if (n < 0) return 1;
      double o[2 * 64], lse[2];
      ora_attend(&c, q, 1, pos, kp, v, sel, n, o, lse);
    }
    if (ora_select(&c, q, 1, 1000, cs, gs, sel, 3, margins, NULL) != -1) return 2;
    double oa[2 * 64], la[2], ob[2 * 64], lb[2], om[2 * 64], lm[2];
    int n = ora_select(&c, q, 1, 900, cs, gs, sel, 64, margins, NULL);
    ora_attend(&c, q, 1, 900, kp, v, sel, n / 2, oa, la);
    ora_attend(&c, q, 1, 900, kp, v, sel + n / 2, n - n / 2, ob, lb);
    ora_merge(d, hg, oa, la, ob, lb, om, lm);
    double* wsb = (double*)malloc(sizeof(double) * n * 16 * d);
    ora_gather(&c, kp, sel, n, wsb);
    int tags[8] = {-1, -1, 3, 9, 4, -1, 7, 2}, used[8] = {0, 0, 2, 1, 3, 0, 1, 2};
    int routed[5] = {9, 11, 2, 30, 31}, slot[5], hit[5];
    if (ora_warm_step(8, tags, used, routed, 5, 4, slot, hit) != 2) return 3;
    int routed2[8] = {40, 41, 42, 43, 44, 45, 46, 47}, slot2[8], hit2[8];
    if (ora_warm_step(8, tags, used, routed2, 8, 5, slot2, hit2) != 0) return 4;
    if (ora_warm_step(4, tags, used, routed2, 8, 6, slot2, hit2) != -1) return 6;
    /* batched driver over 3 units, one thread per unit */
    const int U = 3;
    double* qu = randv((long)U * hg * d);
    long pos0[3] = {1023, 500, 64};
    double* csu = (double*)malloc(sizeof(double) * U * nch * d);
    double* gsu = (double*)malloc(sizeof(double) * U * nch * G * d);
    double* kpu = (double*)malloc(sizeof(double) * U * T * d);
    double* vu = (double*)malloc(sizeof(double) * U * T * d);
    for (int u = 0; u < U; ++u) {
      memcpy(csu + (long)u * nch * d, cs, sizeof(double) * nch * d);
      memcpy(gsu + (long)u * nch * G * d, gs, sizeof(double) * nch * G * d);
      memcpy(kpu + (long)u * T * d, kp, sizeof(double) * T * d);
      memcpy(vu + (long)u * T * d, v, sizeof(double) * T * d);
    }
    int selu[3 * 40], nselu[3];
    double* ou = (double*)malloc(sizeof(double) * U * hg * d);
    if (ora_step(&c, U, qu, 1, pos0, csu, gsu, nch, kpu, vu, T, selu, nselu, 40, ou) != 0) return 5;
    (void)ora_max_threads();
    free(ou); free(vu); free(kpu); free(gsu); free(csu); free(qu); free(wsb); free(codes);
    free(kp); free(gs); free(cs); free(q); free(v); free(kraw);
  }
  printf("sanitize ok\n");
  return 0;
}
