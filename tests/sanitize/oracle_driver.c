/* Drives every entry point of oracle/jbo.c on small shapes, with and without
 * the optional arguments, on one and several threads, and with rejected
 * arguments.  Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitized.py: any out-of-bounds access, leak or undefined
 * operation in the oracle ends the run with a report and a nonzero status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int jbo_gen_taps(int64_t n_tokens, int D, int G, int H, int K, const float* x, const float* W1,
                 const float* b1, const float* W2, const float* b2, double* taps, int nthreads);
int jbo_l2norm(int64_t rows, int d, const float* x, double* out);
int jbo_conv(int B, int T, int H, int dv, int K, const double* taps, const float* v, const float* conv_in,
             double* out);
int jbo_prefill(int B, int T, int H, int dk, int dv, int D, int G, int K, const float* x, const float* q,
                const float* k, const float* v, const float* alpha, const float* beta, const float* W1,
                const float* b1, const float* W2, const float* b2, const float* S0, const float* conv_in,
                double* o, double* S_final, float* conv_out, double* taps_out, int nthreads);
int jbo_decode_step(int B, int H, int dk, int dv, int D, int G, int K, const float* S_in, const float* cache_in,
                    const float* x_t, const float* q_t, const float* k_t, const float* v_t, const float* alpha_t,
                    const float* beta_t, const float* W1, const float* b1, const float* W2, const float* b2,
                    double* o_t, double* S_out, float* cache_out, int nthreads);
int jbo_project(int64_t n_tokens, int D, int H, int dk, int dv, const float* x, const float* Wq, const float* bq,
                const float* Wk, const float* bk, const float* Wv, const float* bv, const float* Wa,
                const float* ba, const float* Wb, const float* bb, float* q, float* k, float* v, double* alpha,
                double* beta, int nthreads);
int jbo_prefill_static(int B, int T, int H, int dk, int dv, int K, const float* q, const float* k, const float* v,
                       const float* alpha, const float* beta, const float* wq, const float* wk, const float* wv,
                       const float* S0, const float* cq_in, const float* ck_in, const float* cv_in, double* o,
                       double* S_final, float* cq_out, float* ck_out, float* cv_out, int nthreads);
int jbo_backward(int B, int T, int H, int dk, int dv, int D, int G, int K, const float* x, const float* q,
                 const float* k, const float* v, const float* alpha, const float* beta, const float* W1,
                 const float* b1, const float* W2, const float* b2, const float* S0, const float* conv_in,
                 const float* dout, const float* dS_final, const float* dconv_out, double* dx, double* dq,
                 double* dk_, double* dv_, double* dalpha, double* dbeta, double* dW1, double* db1, double* dW2,
                 double* db2, double* dS0, double* dconv_in, int nthreads);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static float unif(void) { /* xorshift64*, uniform in (-1, 1) */
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (float)((double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0);
}
static float* fa(size_t n, float scale) {
  float* p = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = scale * unif();
  return p;
}
static float* gates(size_t n, float lo) { /* in [lo, 1) */
  float* p = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = lo + (1.f - lo) * 0.5f * (unif() + 1.f);
  return p;
}
static double* da(size_t n) { return calloc(n, sizeof(double)); }
static float* fz(size_t n) { return calloc(n, sizeof(float)); }

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); ++fails; } } while (0)

int main(void) {
  const int B = 2, T = 67, H = 2, dk = 8, dv = 16, D = 24, G = 4, K = 4;
  const size_t nt = (size_t)B * T;
  float *x = fa(nt * D, 1.f), *q = fa(nt * H * dk, 1.f), *k = fa(nt * H * dk, 1.f), *v = fa(nt * H * dv, 1.f);
  float *al = gates(nt * H, 0.5f), *be = gates(nt * H, 0.f);
  float *W1 = fa((size_t)G * D, 0.3f), *b1 = fa(G, 0.1f), *W2 = fa((size_t)H * K * G, 0.3f), *b2 = fa((size_t)H * K, 0.1f);
  float *S0 = fa((size_t)B * H * dk * dv, 0.1f), *cin = fa((size_t)B * (K - 1) * H * dv, 1.f);
  double *o = da(nt * H * dv), *Sf = da((size_t)B * H * dk * dv), *taps = da(nt * H * K);
  float* cout = fz((size_t)B * (K - 1) * H * dv);
  for (int nth = 1; nth <= 3; nth += 2) {
    EXPECT(jbo_prefill(B, T, H, dk, dv, D, G, K, x, q, k, v, al, be, W1, b1, W2, b2, S0, cin, o, Sf, cout, taps, nth) == 0);
    EXPECT(jbo_prefill(B, T, H, dk, dv, D, G, K, x, q, k, v, al, be, W1, NULL, W2, NULL, NULL, NULL, o, Sf, NULL, NULL, nth) == 0);
    EXPECT(jbo_prefill(B, 0, H, dk, dv, D, G, K, x, q, k, v, al, be, W1, NULL, W2, NULL, S0, cin, o, Sf, cout, NULL, nth) == 0);
  }
  EXPECT(jbo_prefill(-1, T, H, dk, dv, D, G, K, x, q, k, v, al, be, W1, NULL, W2, NULL, NULL, NULL, o, Sf, NULL, NULL, 1) != 0);
  EXPECT(jbo_prefill(B, T, 0, dk, dv, D, G, K, x, q, k, v, al, be, W1, NULL, W2, NULL, NULL, NULL, o, Sf, NULL, NULL, 1) != 0);

  double* tp = da(nt * H * K);
  EXPECT(jbo_gen_taps((int64_t)nt, D, G, H, K, x, W1, b1, W2, b2, tp, 2) == 0);
  double* nrm = da(nt * H * dk);
  EXPECT(jbo_l2norm((int64_t)nt * H, dk, q, nrm) == 0);
  double* cv = da(nt * H * dv);
  EXPECT(jbo_conv(B, T, H, dv, K, tp, v, cin, cv) == 0);
  EXPECT(jbo_conv(B, T, H, dv, K, tp, v, NULL, cv) == 0);

  /* one decode step of the B sequences from the prefill's state */
  float* Sin = fa((size_t)B * H * dk * dv, 0.1f);
  double *ot = da((size_t)B * H * dv), *Sout = da((size_t)B * H * dk * dv);
  float* cache_out = fz((size_t)B * (K - 1) * H * dv);
  EXPECT(jbo_decode_step(B, H, dk, dv, D, G, K, Sin, cin, x, q, k, v, al, be, W1, b1, W2, b2, ot, Sout, cache_out, 2) == 0);

  /* projections */
  float *Wq = fa((size_t)H * dk * D, 0.2f), *Wk = fa((size_t)H * dk * D, 0.2f), *Wv = fa((size_t)H * dv * D, 0.2f);
  float *Wa = fa((size_t)H * D, 0.2f), *Wb = fa((size_t)H * D, 0.2f), *ba = fa(H, 1.f);
  float *pq = fz(nt * H * dk), *pk = fz(nt * H * dk), *pv = fz(nt * H * dv);
  double *pa = da(nt * H), *pb = da(nt * H);
  EXPECT(jbo_project((int64_t)nt, D, H, dk, dv, x, Wq, NULL, Wk, NULL, Wv, NULL, Wa, ba, Wb, NULL, pq, pk, pv, pa, pb, 3) == 0);

  /* the static-conv block */
  float *wq = fa((size_t)H * dk * K, 0.5f), *wk = fa((size_t)H * dk * K, 0.5f), *wv = fa((size_t)H * dv * K, 0.5f);
  float *cq = fa((size_t)B * (K - 1) * H * dk, 1.f), *ck = fa((size_t)B * (K - 1) * H * dk, 1.f);
  float *cqo = fz((size_t)B * (K - 1) * H * dk), *cko = fz((size_t)B * (K - 1) * H * dk), *cvo = fz((size_t)B * (K - 1) * H * dv);
  EXPECT(jbo_prefill_static(B, T, H, dk, dv, K, q, k, v, al, be, wq, wk, wv, S0, cq, ck, cin, o, Sf, cqo, cko, cvo, 2) == 0);
  EXPECT(jbo_prefill_static(B, T, H, dk, dv, K, q, k, v, al, be, wq, wk, wv, NULL, NULL, NULL, NULL, o, Sf, NULL, NULL, NULL, 1) == 0);

  /* the backward pass (crosses the oracle's 64-token checkpoint boundary) */
  float *dout = fa(nt * H * dv, 1.f), *dSf = fa((size_t)B * H * dk * dv, 0.1f), *dco = fa((size_t)B * (K - 1) * H * dv, 1.f);
  double *gx = da(nt * D), *gq = da(nt * H * dk), *gk = da(nt * H * dk), *gv = da(nt * H * dv);
  double *ga = da(nt * H), *gb = da(nt * H), *gW1 = da((size_t)G * D), *gb1 = da(G), *gW2 = da((size_t)H * K * G);
  double *gb2 = da((size_t)H * K), *gS0 = da((size_t)B * H * dk * dv), *gci = da((size_t)B * (K - 1) * H * dv);
  EXPECT(jbo_backward(B, T, H, dk, dv, D, G, K, x, q, k, v, al, be, W1, b1, W2, b2, S0, cin, dout, dSf, dco, gx, gq, gk,
                      gv, ga, gb, gW1, gb1, gW2, gb2, gS0, gci, 3) == 0);
  EXPECT(jbo_backward(B, T, H, dk, dv, D, G, K, x, q, k, v, al, be, W1, NULL, W2, NULL, NULL, NULL, dout, NULL, NULL,
                      gx, gq, gk, gv, ga, gb, gW1, gb1, gW2, gb2, gS0, gci, 1) == 0);
  EXPECT(jbo_backward(B, T, H, dk, dv, D, G, K, NULL, q, k, v, al, be, W1, NULL, W2, NULL, NULL, NULL, dout, NULL, NULL,
                      gx, gq, gk, gv, ga, gb, gW1, gb1, gW2, gb2, gS0, gci, 1) != 0);

  void* all[] = {x, q, k, v, al, be, W1, b1, W2, b2, S0, cin, o, Sf, taps, cout, tp, nrm, cv, Sin, ot, Sout, cache_out,
                 Wq, Wk, Wv, Wa, Wb, ba, pq, pk, pv, pa, pb, wq, wk, wv, cq, ck, cqo, cko, cvo, dout, dSf, dco,
                 gx, gq, gk, gv, ga, gb, gW1, gb1, gW2, gb2, gS0, gci};
  for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
  if (fails) return 1;
  printf("oracle sanitizer run: all calls clean\n");
  return 0;
}
