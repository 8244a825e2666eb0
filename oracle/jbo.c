/*
 * jbo.c -- fp64 sequential CPU oracle for the JetBlock token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library; it is built by gcc from this
 * file alone.
 *
 * What it computes (one token at a time, every quantity in double):
 *
 *   Jet-Nemotron paper (Chinese translation, csdn page), section 2.4 "new
 *   attention block design": a kernel generator takes the same input as the
 *   Q/K/V projections, applies a reducing Linear layer, SiLU, and a final
 *   Linear layer whose outputs are convolution-kernel weights; the dynamic
 *   causal kernels are applied to the value tokens only; the static
 *   convolutions on Q and K are removed; Gated DeltaNet does the time mixing.
 *   The xugj520 blog page, section 2.2, lists kernel size 4 and generator
 *   hidden width 32.
 *
 *   The Gated DeltaNet step with state S (dv x dk):
 *       S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v'_t k_t^T,   o_t = S_t q_t
 *   over L2-normalised q and k, where v'_t is the convolved value.
 *   This oracle stores M = S^T (dk x dv, dv contiguous).
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *   - taps for token t come from x_t; tap j (0..3) multiplies v_{t-3+j}
 *     (j = 3 is the current token); rows before the start come from the
 *     conv cache (raw v rows, oldest first) or are zero;
 *   - one tap set per head (4 taps per head, shared by all dv channels);
 *   - L2 norm: x * (sum x^2 + eps)^(-1/2), eps = 1e-6;
 *   - no 1/sqrt(dk) scaling of q; o uses the updated state S_t;
 *   - generator biases are optional (NULL means zero).
 *
 * Inputs arrive as float arrays holding the exact values handed to the GPU
 * (bf16 values are exactly representable in float); they are widened to
 * double on use.
 *
 * Layouts (row-major, last index contiguous):
 *   x [B][T][D]; q,k [B][T][H][dk]; v [B][T][H][dv]; alpha,beta [B][T][H]
 *   W1 [G][D]; b1 [G]; W2 [H*K][G] (row h*K+j is tap j of head h); b2 [H*K]
 *   S0, S_final [B][H][dk][dv]; conv_in, conv_out [B][K-1][H][dv]
 *   o [B][T][H][dv]; taps [B][T][H][K]
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define JBO_EPS 1e-6

/* ---------------------------------------------------------------- generator */

/* taps for one token: hidden = SiLU(W1 x + b1), taps = W2 hidden + b2. */
static void gen_one(int D, int G, int HK, const float* x, const float* W1,
                    const float* b1, const float* W2, const float* b2,
                    double* hidden, double* taps) {
  for (int g = 0; g < G; ++g) {
    double acc = b1 ? (double)b1[g] : 0.0;
    const float* w = W1 + (int64_t)g * D;
    for (int d = 0; d < D; ++d) acc += (double)w[d] * (double)x[d];
    hidden[g] = acc / (1.0 + exp(-acc)); /* SiLU(h) = h * sigmoid(h) */
  }
  for (int r = 0; r < HK; ++r) {
    double acc = b2 ? (double)b2[r] : 0.0;
    const float* w = W2 + (int64_t)r * G;
    for (int g = 0; g < G; ++g) acc += (double)w[g] * hidden[g];
    taps[r] = acc;
  }
}

typedef struct {
  int64_t n0, n1;
  int D, G, HK;
  const float *x, *W1, *b1, *W2, *b2;
  double* taps;
} gen_job;

static void* gen_worker(void* p) {
  gen_job* j = (gen_job*)p;
  double* hidden = (double*)malloc(sizeof(double) * (size_t)j->G);
  for (int64_t n = j->n0; n < j->n1; ++n)
    gen_one(j->D, j->G, j->HK, j->x + n * j->D, j->W1, j->b1, j->W2, j->b2,
            hidden, j->taps + n * j->HK);
  free(hidden);
  return NULL;
}

/* Kernel generator over n_tokens rows of x.  taps: [n_tokens][H*K]. */
int jbo_gen_taps(int64_t n_tokens, int D, int G, int H, int K, const float* x,
                 const float* W1, const float* b1, const float* W2,
                 const float* b2, double* taps, int nthreads) {
  if (n_tokens < 0 || D <= 0 || G <= 0 || H <= 0 || K <= 0) return 1;
  if (!x || !W1 || !W2 || !taps) return 1;
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > n_tokens) nthreads = n_tokens > 0 ? (int)n_tokens : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  gen_job* jobs = (gen_job*)malloc(sizeof(gen_job) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (gen_job){n_tokens * i / nthreads, n_tokens * (i + 1) / nthreads,
                        D, G, H * K, x, W1, b1, W2, b2, taps};
    if (nthreads == 1) gen_worker(&jobs[i]);
    else pthread_create(&th[i], NULL, gen_worker, &jobs[i]);
  }
  if (nthreads > 1)
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return 0;
}

/* --------------------------------------------------------------- L2 norm */

/* out = x * (sum x^2 + eps)^(-1/2), row by row. */
int jbo_l2norm(int64_t rows, int d, const float* x, double* out) {
  if (rows < 0 || d <= 0 || !x || !out) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += (double)x[r * d + i] * (double)x[r * d + i];
    double s = 1.0 / sqrt(ss + JBO_EPS);
    for (int i = 0; i < d; ++i) out[r * d + i] = (double)x[r * d + i] * s;
  }
  return 0;
}

/* ------------------------------------------------------ dynamic causal conv */

/* Raw value row for token t (may be negative: then it comes from the cache). */
static const float* v_row(int t, int b, int h, int T, int H, int dv, int K,
                          const float* v, const float* conv_in) {
  if (t >= 0) return v + (((int64_t)b * T + t) * H + h) * dv;
  if (!conv_in) return NULL;                /* zero padding */
  int slot = (K - 1) + t;                   /* t = -1 -> newest cache row */
  return conv_in + (((int64_t)b * (K - 1) + slot) * H + h) * dv;
}

/* v'[t][c] = sum_j taps[t][h][j] * v_{t-(K-1)+j}[c] for one (b, t, h). */
static void conv_one(int b, int t, int h, int T, int H, int dv, int K,
                     const double* taps_bth, const float* v,
                     const float* conv_in, double* out) {
  for (int c = 0; c < dv; ++c) out[c] = 0.0;
  for (int j = 0; j < K; ++j) {
    const float* row = v_row(t - (K - 1) + j, b, h, T, H, dv, K, v, conv_in);
    if (!row) continue;
    for (int c = 0; c < dv; ++c) out[c] += taps_bth[j] * (double)row[c];
  }
}

/* Whole convolution: vconv [B][T][H][dv] from taps [B][T][H][K]. */
int jbo_conv(int B, int T, int H, int dv, int K, const double* taps,
             const float* v, const float* conv_in, double* vconv) {
  if (B < 0 || T < 0 || H <= 0 || dv <= 0 || K <= 0) return 1;
  if (!taps || !v || !vconv) return 1;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h) {
        int64_t bth = ((int64_t)b * T + t) * H + h;
        conv_one(b, t, h, T, H, dv, K, taps + bth * K, v, conv_in,
                 vconv + bth * dv);
      }
  return 0;
}

/* ------------------------------------------------- gated delta-rule block */

typedef struct {
  int B, T, H, dk, dv, K;
  const float *q, *k, *v, *alpha, *beta, *S0, *conv_in;
  const double* taps;
  double *o, *S_final;
  int unit0, unit1; /* (b, h) units [unit0, unit1) */
} rec_job;

/* L2 normalisation of one row: out = x (sum x^2 + eps)^(-1/2) */
static void l2n_row(const double* x, int n, double* out) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += x[i] * x[i];
  const double r = 1.0 / sqrt(s + JBO_EPS);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r;
}

/* One token of the recurrence on normalised qh, kh and the convolved value vc:
     S_t = a S_{t-1} (I - b k k^T) + b v' k^T, written for M = S^T:
     M <- a (M - b k (k^T M)) + b k v'^T,   o_t = S_t q = M^T q. */
static void rec_step(double* M, const double* qh, const double* kh, const double* vc,
                     double a, double be, int dk, int dv, double* kM, double* ot) {
  for (int c = 0; c < dv; ++c) {
    double s = 0.0;
    for (int i = 0; i < dk; ++i) s += kh[i] * M[(int64_t)i * dv + c];
    kM[c] = s;
  }
  for (int i = 0; i < dk; ++i)
    for (int c = 0; c < dv; ++c) {
      double* m = &M[(int64_t)i * dv + c];
      *m = a * (*m - be * kh[i] * kM[c]) + be * kh[i] * vc[c];
    }
  for (int c = 0; c < dv; ++c) {
    double s = 0.0;
    for (int i = 0; i < dk; ++i) s += M[(int64_t)i * dv + c] * qh[i];
    ot[c] = s;
  }
}

static void* rec_worker(void* p) {
  rec_job* J = (rec_job*)p;
  const int T = J->T, H = J->H, dk = J->dk, dv = J->dv, K = J->K;
  double* M = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  double* qh = (double*)malloc(sizeof(double) * (size_t)dk);
  double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
  double* vc = (double*)malloc(sizeof(double) * (size_t)dv);
  double* kM = (double*)malloc(sizeof(double) * (size_t)dv);
  for (int u = J->unit0; u < J->unit1; ++u) {
    const int b = u / H, h = u % H;
    const int64_t sbase = ((int64_t)b * H + h) * dk * dv;
    for (int64_t i = 0; i < (int64_t)dk * dv; ++i)
      M[i] = J->S0 ? (double)J->S0[sbase + i] : 0.0;
    for (int t = 0; t < T; ++t) {
      const int64_t bth = ((int64_t)b * T + t) * H + h;
      /* value convolution with the per-token taps */
      conv_one(b, t, h, T, H, dv, K, J->taps + bth * K, J->v, J->conv_in, vc);
      /* L2-normalised query and key */
      for (int i = 0; i < dk; ++i) {
        qh[i] = (double)J->q[bth * dk + i];
        kh[i] = (double)J->k[bth * dk + i];
      }
      l2n_row(qh, dk, qh);
      l2n_row(kh, dk, kh);
      rec_step(M, qh, kh, vc, J->alpha[bth], J->beta[bth], dk, dv, kM, J->o + bth * dv);
    }
    if (J->S_final)
      for (int64_t i = 0; i < (int64_t)dk * dv; ++i) J->S_final[sbase + i] = M[i];
  }
  free(M); free(qh); free(kh); free(vc); free(kM);
  return NULL;
}

/*
 * Full block over B sequences of T tokens.  taps_out (optional) receives the
 * generator output [B][T][H][K].  conv_out (optional) receives the last K-1
 * raw value rows (from v, or from conv_in when T < K-1).  Returns 0 on success.
 */
int jbo_prefill(int B, int T, int H, int dk, int dv, int D, int G, int K,
                const float* x, const float* q, const float* k, const float* v,
                const float* alpha, const float* beta, const float* W1,
                const float* b1, const float* W2, const float* b2,
                const float* S0, const float* conv_in, double* o,
                double* S_final, float* conv_out, double* taps_out,
                int nthreads) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || D <= 0 || G <= 0 || K < 1)
    return 1;
  if (!x || !q || !k || !v || !alpha || !beta || !W1 || !W2 || !o) return 1;
  const int64_t n_tok = (int64_t)B * T;
  double* taps = taps_out;
  if (!taps) taps = (double*)malloc(sizeof(double) * (size_t)(n_tok * H * K + 1));
  if (jbo_gen_taps(n_tok, D, G, H, K, x, W1, b1, W2, b2, taps, nthreads)) {
    if (!taps_out) free(taps);
    return 1;
  }
  const int units = B * H;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = units > 0 ? units : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  rec_job* jobs = (rec_job*)malloc(sizeof(rec_job) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (rec_job){B, T, H, dk, dv, K, q, k, v, alpha, beta, S0, conv_in,
                        taps, o, S_final,
                        (int)((int64_t)units * i / nthreads),
                        (int)((int64_t)units * (i + 1) / nthreads)};
    if (nthreads == 1) rec_worker(&jobs[i]);
    else pthread_create(&th[i], NULL, rec_worker, &jobs[i]);
  }
  if (nthreads > 1)
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  if (conv_out) {
    for (int b = 0; b < B; ++b)
      for (int s = 0; s < K - 1; ++s)
        for (int h = 0; h < H; ++h) {
          const float* row = v_row(T - (K - 1) + s, b, h, T, H, dv, K, v, conv_in);
          float* dst = conv_out + (((int64_t)b * (K - 1) + s) * H + h) * dv;
          for (int c = 0; c < dv; ++c) dst[c] = row ? row[c] : 0.0f;
        }
  }
  if (!taps_out) free(taps);
  return 0;
}

/*
 * One decode step for B sequences: the same block with T = 1.  S_in/S_out are
 * [B][H][dk][dv] (S_out in double), cache_in/cache_out [B][K-1][H][dv],
 * x_t [B][D], q_t,k_t [B][H][dk], v_t [B][H][dv], alpha_t,beta_t [B][H],
 * o_t [B][H][dv].
 */
int jbo_decode_step(int B, int H, int dk, int dv, int D, int G, int K,
                    const float* S_in, const float* cache_in,
                    const float* x_t, const float* q_t, const float* k_t,
                    const float* v_t, const float* alpha_t, const float* beta_t,
                    const float* W1, const float* b1, const float* W2,
                    const float* b2, double* o_t, double* S_out,
                    float* cache_out, int nthreads) {
  return jbo_prefill(B, 1, H, dk, dv, D, G, K, x_t, q_t, k_t, v_t, alpha_t,
                     beta_t, W1, b1, W2, b2, S_in, cache_in, o_t, S_out,
                     cache_out, NULL, nthreads);
}

/* ------------------------------------------------------- input projections */
/*
 * The Linear layers that feed the block.  The csdn translation, section 2.4,
 * says the kernel generator takes the same input as the Q/K/V projection
 * layers; per token x (length D):
 *     q = Wq x + bq,  k = Wk x + bk,  v = Wv x + bv
 *     alpha = sigmoid(Wa x + ba),  beta = sigmoid(Wb x + bb)   (one per head)
 * Readings (the pages describe neither the gate projections nor the
 * activation precision): both gates pass through a sigmoid, which keeps them
 * in (0, 1) as the recurrence needs; q, k and v leave the projections as
 * bf16 activations, the block's input type, i.e. the exact value rounded to
 * the nearest bf16 with ties to even.  Every bias is optional (NULL = 0).
 *
 * Layouts: x [n][D]; Wq, Wk [H*dk][D]; Wv [H*dv][D]; Wa, Wb [H][D];
 * q, k [n][H*dk]; v [n][H*dv]; alpha, beta [n][H].
 */

/* nearest bf16 (8 significant bits, ties to even) of a double, from the
 * definition: scale the value so that the 8 bits are its integer part, round
 * to the nearest integer (the default rounding mode breaks ties to even) and
 * scale back.  Below the smallest normal bf16 (2^-126) the spacing stays
 * 2^-133. */
double jbo_bf16_round(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  frexp(v, &e); /* |v| = f 2^e with f in [0.5, 1) */
  const int sh = e < -125 ? 133 : 8 - e;
  return ldexp(nearbyint(ldexp(v, sh)), -sh);
}

typedef struct {
  int64_t n0, n1;
  int D, H, dk, dv;
  const float *x, *Wq, *bq, *Wk, *bk, *Wv, *bv, *Wa, *ba, *Wb, *bb;
  float *q, *k, *v;
  double *alpha, *beta;
} proj_job;

static double dot_row(const float* w, const float* x, int D) {
  double acc = 0.0;
  for (int i = 0; i < D; ++i) acc += (double)w[i] * (double)x[i];
  return acc;
}

static void* proj_worker(void* p) {
  const proj_job* j = (const proj_job*)p;
  const int D = j->D, nqk = j->H * j->dk, nv = j->H * j->dv;
  for (int64_t n = j->n0; n < j->n1; ++n) {
    const float* x = j->x + n * D;
    for (int r = 0; r < nqk; ++r) {
      j->q[n * nqk + r] = (float)jbo_bf16_round(dot_row(j->Wq + (int64_t)r * D, x, D) + (j->bq ? j->bq[r] : 0.0));
      j->k[n * nqk + r] = (float)jbo_bf16_round(dot_row(j->Wk + (int64_t)r * D, x, D) + (j->bk ? j->bk[r] : 0.0));
    }
    for (int r = 0; r < nv; ++r)
      j->v[n * nv + r] = (float)jbo_bf16_round(dot_row(j->Wv + (int64_t)r * D, x, D) + (j->bv ? j->bv[r] : 0.0));
    for (int h = 0; h < j->H; ++h) {
      const double za = dot_row(j->Wa + (int64_t)h * D, x, D) + (j->ba ? j->ba[h] : 0.0);
      const double zb = dot_row(j->Wb + (int64_t)h * D, x, D) + (j->bb ? j->bb[h] : 0.0);
      j->alpha[n * j->H + h] = 1.0 / (1.0 + exp(-za));
      j->beta[n * j->H + h] = 1.0 / (1.0 + exp(-zb));
    }
  }
  return NULL;
}

int jbo_project(int64_t n_tokens, int D, int H, int dk, int dv, const float* x,
                const float* Wq, const float* bq, const float* Wk, const float* bk,
                const float* Wv, const float* bv, const float* Wa, const float* ba,
                const float* Wb, const float* bb, float* q, float* k, float* v,
                double* alpha, double* beta, int nthreads) {
  if (n_tokens < 0 || D < 1 || H < 1 || dk < 1 || dv < 1 || !x || !Wq || !Wk || !Wv || !Wa || !Wb ||
      !q || !k || !v || !alpha || !beta)
    return 1;
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > n_tokens) nthreads = n_tokens > 0 ? (int)n_tokens : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  proj_job* jobs = (proj_job*)malloc(sizeof(proj_job) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (proj_job){n_tokens * i / nthreads, n_tokens * (i + 1) / nthreads, D, H, dk, dv,
                         x, Wq, bq, Wk, bk, Wv, bv, Wa, ba, Wb, bb, q, k, v, alpha, beta};
    if (nthreads == 1) proj_worker(&jobs[i]);
    else pthread_create(&th[i], NULL, proj_worker, &jobs[i]);
  }
  if (nthreads > 1)
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return 0;
}

/* ------------------------------------------- static-conv Gated DeltaNet block */
/*
 * The block JetBlock replaces (csdn translation, section 2.4: earlier linear
 * attention blocks use static convolution kernels; JetBlock applies a
 * dynamic kernel to V and drops the static ones on Q and K).  Readings (the
 * pages give no detail): a depthwise causal convolution of size K per
 * channel with fixed weights on each of q, k and v, tap j (0..K-1)
 * multiplying token t-(K-1)+j, no activation; q and k are L2-normalised after
 * their convolution; the recurrence is the same.  Rows before the start come
 * from each tensor's own cache (raw rows, oldest first) or are zero.
 *
 * Layouts: q, k [B][T][H][dk]; v [B][T][H][dv]; wq, wk [H*dk][K];
 * wv [H*dv][K]; cq, ck [B][K-1][H][dk]; cv [B][K-1][H][dv] (in and out).
 */

/* raw row of a [B][T][H][d] tensor for token t, or of its cache when t < 0 */
static const float* raw_row(int t, int b, int h, int T, int H, int d, int K, const float* x,
                            const float* cache) {
  if (t >= 0) return x + (((int64_t)b * T + t) * H + h) * d;
  if (!cache) return NULL;
  return cache + (((int64_t)b * (K - 1) + (K - 1) + t) * H + h) * d;
}

/* out[c] = sum_j w[c][j] x_{t-(K-1)+j}[c] for one (b, t, h) */
static void static_conv_one(int b, int t, int h, int T, int H, int d, int K, const float* x,
                            const float* cache, const float* w, double* out) {
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  for (int j = 0; j < K; ++j) {
    const float* row = raw_row(t - (K - 1) + j, b, h, T, H, d, K, x, cache);
    if (!row) continue;
    for (int c = 0; c < d; ++c) out[c] += (double)w[((int64_t)h * d + c) * K + j] * (double)row[c];
  }
}

typedef struct {
  int B, T, H, dk, dv, K;
  const float *q, *k, *v, *alpha, *beta, *wq, *wk, *wv, *S0, *cq, *ck, *cv;
  double *o, *S_final;
  int unit0, unit1;
} rec_static_job;

static void* rec_static_worker(void* p) {
  rec_static_job* J = (rec_static_job*)p;
  const int T = J->T, H = J->H, dk = J->dk, dv = J->dv, K = J->K;
  double* M = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  double* qh = (double*)malloc(sizeof(double) * (size_t)dk);
  double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
  double* vc = (double*)malloc(sizeof(double) * (size_t)dv);
  double* kM = (double*)malloc(sizeof(double) * (size_t)dv);
  for (int u = J->unit0; u < J->unit1; ++u) {
    const int b = u / H, h = u % H;
    const int64_t sbase = ((int64_t)b * H + h) * dk * dv;
    for (int64_t i = 0; i < (int64_t)dk * dv; ++i) M[i] = J->S0 ? (double)J->S0[sbase + i] : 0.0;
    for (int t = 0; t < T; ++t) {
      const int64_t bth = ((int64_t)b * T + t) * H + h;
      static_conv_one(b, t, h, T, H, dk, K, J->q, J->cq, J->wq, qh);
      static_conv_one(b, t, h, T, H, dk, K, J->k, J->ck, J->wk, kh);
      static_conv_one(b, t, h, T, H, dv, K, J->v, J->cv, J->wv, vc);
      l2n_row(qh, dk, qh);
      l2n_row(kh, dk, kh);
      rec_step(M, qh, kh, vc, J->alpha[bth], J->beta[bth], dk, dv, kM, J->o + bth * dv);
    }
    if (J->S_final)
      for (int64_t i = 0; i < (int64_t)dk * dv; ++i) J->S_final[sbase + i] = M[i];
  }
  free(M); free(qh); free(kh); free(vc); free(kM);
  return NULL;
}

/* the last K-1 raw rows of [cache; x] into cache_out */
static void tail_rows(int B, int T, int H, int d, int K, const float* x, const float* cache,
                      float* out) {
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < K - 1; ++s)
      for (int h = 0; h < H; ++h) {
        const float* row = raw_row(T - (K - 1) + s, b, h, T, H, d, K, x, cache);
        float* dst = out + (((int64_t)b * (K - 1) + s) * H + h) * d;
        for (int c = 0; c < d; ++c) dst[c] = row ? row[c] : 0.0f;
      }
}

int jbo_prefill_static(int B, int T, int H, int dk, int dv, int K, const float* q, const float* k,
                       const float* v, const float* alpha, const float* beta, const float* wq,
                       const float* wk, const float* wv, const float* S0, const float* cq_in,
                       const float* ck_in, const float* cv_in, double* o, double* S_final,
                       float* cq_out, float* ck_out, float* cv_out, int nthreads) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || K < 1) return 1;
  if (!q || !k || !v || !alpha || !beta || !wq || !wk || !wv || !o) return 1;
  const int units = B * H;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = units > 0 ? units : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  rec_static_job* jobs = (rec_static_job*)malloc(sizeof(rec_static_job) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (rec_static_job){B, T, H, dk, dv, K, q, k, v, alpha, beta, wq, wk, wv, S0, cq_in, ck_in, cv_in,
                               o, S_final, (int)((int64_t)units * i / nthreads),
                               (int)((int64_t)units * (i + 1) / nthreads)};
    if (nthreads == 1) rec_static_worker(&jobs[i]);
    else pthread_create(&th[i], NULL, rec_static_worker, &jobs[i]);
  }
  if (nthreads > 1)
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  if (cq_out) tail_rows(B, T, H, dk, K, q, cq_in, cq_out);
  if (ck_out) tail_rows(B, T, H, dk, K, k, ck_in, ck_out);
  if (cv_out) tail_rows(B, T, H, dv, K, v, cv_in, cv_out);
  return 0;
}

/* ----------------------------------------------------------------- backward */
/*
 * Reverse-mode gradient of the block (what training it needs: the pages
 * train JetBlock inside the model, csdn translation, sections 2.2 and 3.1).
 * Given the gradients of the outputs -- dout [B][T][H][dv] of o, dS_final
 * [B][H][dk][dv] of S_final and dconv_out [B][K-1][H][dv] of conv_out, the
 * latter two nullable (zero) -- it returns, all in double:
 *   dx [B][T][D], dq, dk [B][T][H][dk], dv [B][T][H][dv],
 *   dalpha, dbeta [B][T][H], dW1 [G][D], db1 [G], dW2 [H*K][G], db2 [H*K],
 *   dS0 [B][H][dk][dv], dconv_in [B][K-1][H][dv]
 * (gradients with respect to S0 and conv_in are returned even when those are
 * NULL, i.e. with respect to the zeros used in their place).
 *
 * Token by token in reverse, with M = S^T and N the state before token t:
 *   forward  a = N^T k,  M_t = alpha (N - beta k a^T) + beta k v'^T,  o = M_t^T q
 *   reverse  dM += q do^T;  dq^ = M_t do;  e = dM^T k;
 *            dv' = beta e;  dbeta = e . (v' - alpha a);
 *            dalpha = sum(dM . N) - beta e . a;
 *            dk^ = beta dM v' - alpha beta (dM a + N e);
 *            dM <- alpha (dM - beta k e^T)          (the gradient of N)
 * then through the L2 norms (q^ = q / n, n = sqrt(sum q^2 + eps):
 * dq = dq^ / n - q (q . dq^) / n^3), the conv (dv'_t spread over the raw rows
 * it read, dtaps_t[j] = dv'_t . raw_{t-3+j}) and the generator
 * (taps = W2 h + b2, h = SiLU(p), p = W1 x + b1,
 * SiLU'(p) = s (1 + p (1 - s)), s = sigmoid(p)).
 * States are recomputed from checkpoints taken every 64 tokens.
 */
#define JBO_CKPT 64

typedef struct {
  int B, T, H, dk, dv, K;
  const float *q, *k, *v, *alpha, *beta, *S0, *conv_in, *dout, *dS_final, *dconv_out;
  const double* taps;
  double *dq, *dk_, *dv_, *dalpha, *dbeta, *dS0, *dconv_in, *dtaps;
  int unit0, unit1;
} bwd_job;

/* the raw-row gradient slot of token t (t < 0: the conv cache) */
static double* draw_row(int t, int b, int h, int T, int H, int dv, int K, double* dv_, double* dconv_in) {
  if (t >= 0) return dv_ + (((int64_t)b * T + t) * H + h) * dv;
  return dconv_in + (((int64_t)b * (K - 1) + (K - 1) + t) * H + h) * dv;
}

static void* bwd_worker(void* p) {
  bwd_job* J = (bwd_job*)p;
  const int T = J->T, H = J->H, dk = J->dk, dv = J->dv, K = J->K;
  const int64_t md = (int64_t)dk * dv;
  const int nblk = (T + JBO_CKPT - 1) / JBO_CKPT;
  double* ck = (double*)malloc(sizeof(double) * (size_t)(md * (nblk > 0 ? nblk : 1)));
  double* Ms = (double*)malloc(sizeof(double) * (size_t)(md * JBO_CKPT));
  double* M = (double*)malloc(sizeof(double) * (size_t)md);
  double* dM = (double*)malloc(sizeof(double) * (size_t)md);
  double *qh = (double*)malloc(sizeof(double) * dk), *kh = (double*)malloc(sizeof(double) * dk);
  double *qr = (double*)malloc(sizeof(double) * dk), *kr = (double*)malloc(sizeof(double) * dk);
  double *dqh = (double*)malloc(sizeof(double) * dk), *dkh = (double*)malloc(sizeof(double) * dk);
  double *vc = (double*)malloc(sizeof(double) * dv), *a = (double*)malloc(sizeof(double) * dv);
  double *e = (double*)malloc(sizeof(double) * dv), *dvc = (double*)malloc(sizeof(double) * dv);
  double* otmp = (double*)malloc(sizeof(double) * dv);
  for (int u = J->unit0; u < J->unit1; ++u) {
    const int b = u / H, h = u % H;
    const int64_t sbase = ((int64_t)b * H + h) * md;
    /* forward to the checkpoints */
    for (int64_t i = 0; i < md; ++i) M[i] = J->S0 ? (double)J->S0[sbase + i] : 0.0;
    for (int t = 0; t < T; ++t) {
      if (t % JBO_CKPT == 0) memcpy(ck + (int64_t)(t / JBO_CKPT) * md, M, sizeof(double) * (size_t)md);
      const int64_t bth = ((int64_t)b * T + t) * H + h;
      conv_one(b, t, h, T, H, dv, K, J->taps + bth * K, J->v, J->conv_in, vc);
      for (int i = 0; i < dk; ++i) { qh[i] = J->q[bth * dk + i]; kh[i] = J->k[bth * dk + i]; }
      l2n_row(qh, dk, qh);
      l2n_row(kh, dk, kh);
      rec_step(M, qh, kh, vc, J->alpha[bth], J->beta[bth], dk, dv, a, otmp);
    }
    /* reverse */
    for (int64_t i = 0; i < md; ++i) dM[i] = J->dS_final ? (double)J->dS_final[sbase + i] : 0.0;
    if (J->dconv_out)
      for (int s = 0; s < K - 1; ++s) {
        double* dst = draw_row(T - (K - 1) + s, b, h, T, H, dv, K, J->dv_, J->dconv_in);
        const float* src = J->dconv_out + (((int64_t)b * (K - 1) + s) * H + h) * dv;
        for (int c = 0; c < dv; ++c) dst[c] += src[c];
      }
    for (int blk = nblk - 1; blk >= 0; --blk) {
      const int t0 = blk * JBO_CKPT, t1 = t0 + JBO_CKPT < T ? t0 + JBO_CKPT : T;
      /* states after each token of the block */
      memcpy(M, ck + (int64_t)blk * md, sizeof(double) * (size_t)md);
      for (int t = t0; t < t1; ++t) {
        const int64_t bth = ((int64_t)b * T + t) * H + h;
        conv_one(b, t, h, T, H, dv, K, J->taps + bth * K, J->v, J->conv_in, vc);
        for (int i = 0; i < dk; ++i) { qh[i] = J->q[bth * dk + i]; kh[i] = J->k[bth * dk + i]; }
        l2n_row(qh, dk, qh);
        l2n_row(kh, dk, kh);
        rec_step(M, qh, kh, vc, J->alpha[bth], J->beta[bth], dk, dv, a, otmp);
        memcpy(Ms + (int64_t)(t - t0) * md, M, sizeof(double) * (size_t)md);
      }
      for (int t = t1 - 1; t >= t0; --t) {
        const int64_t bth = ((int64_t)b * T + t) * H + h;
        const double* Mt = Ms + (int64_t)(t - t0) * md;
        const double* N = t > t0 ? Ms + (int64_t)(t - 1 - t0) * md : ck + (int64_t)blk * md;
        const double al = J->alpha[bth], be = J->beta[bth];
        const float* dot = J->dout + bth * dv;
        conv_one(b, t, h, T, H, dv, K, J->taps + bth * K, J->v, J->conv_in, vc);
        for (int i = 0; i < dk; ++i) { qr[i] = J->q[bth * dk + i]; kr[i] = J->k[bth * dk + i]; }
        l2n_row(qr, dk, qh);
        l2n_row(kr, dk, kh);
        /* output: o = M_t^T q^ */
        for (int i = 0; i < dk; ++i) {
          double s = 0.0;
          for (int c = 0; c < dv; ++c) {
            dM[(int64_t)i * dv + c] += qh[i] * (double)dot[c];
            s += Mt[(int64_t)i * dv + c] * (double)dot[c];
          }
          dqh[i] = s;
        }
        /* the update */
        for (int c = 0; c < dv; ++c) {
          double sa = 0.0, se = 0.0;
          for (int i = 0; i < dk; ++i) {
            sa += N[(int64_t)i * dv + c] * kh[i];
            se += dM[(int64_t)i * dv + c] * kh[i];
          }
          a[c] = sa;
          e[c] = se;
        }
        double dbe = 0.0, dal = 0.0, ea = 0.0;
        for (int c = 0; c < dv; ++c) {
          dvc[c] = be * e[c];
          dbe += e[c] * (vc[c] - al * a[c]);
          ea += e[c] * a[c];
        }
        for (int64_t i = 0; i < md; ++i) dal += dM[i] * N[i];
        dal -= be * ea;
        for (int i = 0; i < dk; ++i) {
          double s1 = 0.0, s2 = 0.0, s3 = 0.0;
          for (int c = 0; c < dv; ++c) {
            s1 += dM[(int64_t)i * dv + c] * vc[c];
            s2 += dM[(int64_t)i * dv + c] * a[c];
            s3 += N[(int64_t)i * dv + c] * e[c];
          }
          dkh[i] = be * s1 - al * be * (s2 + s3);
        }
        for (int i = 0; i < dk; ++i)
          for (int c = 0; c < dv; ++c) {
            double* m = &dM[(int64_t)i * dv + c];
            *m = al * (*m - be * kh[i] * e[c]);
          }
        J->dalpha[bth] = dal;
        J->dbeta[bth] = dbe;
        /* the L2 norms */
        double sq = 0.0, sk = 0.0, qd = 0.0, kd = 0.0;
        for (int i = 0; i < dk; ++i) {
          sq += qr[i] * qr[i]; sk += kr[i] * kr[i];
          qd += qr[i] * dqh[i]; kd += kr[i] * dkh[i];
        }
        const double nq = sqrt(sq + JBO_EPS), nk = sqrt(sk + JBO_EPS);
        for (int i = 0; i < dk; ++i) {
          J->dq[bth * dk + i] = dqh[i] / nq - qr[i] * qd / (nq * nq * nq);
          J->dk_[bth * dk + i] = dkh[i] / nk - kr[i] * kd / (nk * nk * nk);
        }
        /* the conv: v'_t = sum_j taps[j] raw_{t-3+j} */
        for (int j = 0; j < K; ++j) {
          const int tr = t - (K - 1) + j;
          const float* row = v_row(tr, b, h, T, H, dv, K, J->v, J->conv_in);
          double* drow = draw_row(tr, b, h, T, H, dv, K, J->dv_, J->dconv_in);
          double dt = 0.0;
          for (int c = 0; c < dv; ++c) {
            if (row) dt += dvc[c] * (double)row[c];
            drow[c] += J->taps[bth * K + j] * dvc[c];
          }
          J->dtaps[bth * K + j] = dt;
        }
      }
    }
    for (int64_t i = 0; i < md; ++i) J->dS0[sbase + i] = dM[i];
  }
  free(ck); free(Ms); free(M); free(dM); free(qh); free(kh); free(qr); free(kr); free(dqh); free(dkh);
  free(vc); free(a); free(e); free(dvc); free(otmp);
  return NULL;
}

int jbo_backward(int B, int T, int H, int dk, int dv, int D, int G, int K, const float* x, const float* q,
                 const float* k, const float* v, const float* alpha, const float* beta, const float* W1,
                 const float* b1, const float* W2, const float* b2, const float* S0, const float* conv_in,
                 const float* dout, const float* dS_final, const float* dconv_out, double* dx, double* dq,
                 double* dk_, double* dv_, double* dalpha, double* dbeta, double* dW1, double* db1, double* dW2,
                 double* db2, double* dS0, double* dconv_in, int nthreads) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || D <= 0 || G <= 0 || K < 1) return 1;
  if (!x || !q || !k || !v || !alpha || !beta || !W1 || !W2 || !dout) return 1;
  if (!dx || !dq || !dk_ || !dv_ || !dalpha || !dbeta || !dW1 || !db1 || !dW2 || !db2 || !dS0 || !dconv_in)
    return 1;
  const int64_t n_tok = (int64_t)B * T;
  const int HK = H * K;
  double* taps = (double*)malloc(sizeof(double) * (size_t)(n_tok * HK + 1));
  double* dtaps = (double*)calloc((size_t)(n_tok * HK + 1), sizeof(double));
  if (jbo_gen_taps(n_tok, D, G, H, K, x, W1, b1, W2, b2, taps, nthreads)) { free(taps); free(dtaps); return 1; }
  memset(dv_, 0, sizeof(double) * (size_t)(n_tok * H * dv));
  memset(dconv_in, 0, sizeof(double) * (size_t)B * (K - 1) * H * dv);
  const int units = B * H;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = units > 0 ? units : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  bwd_job* jobs = (bwd_job*)malloc(sizeof(bwd_job) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (bwd_job){B, T, H, dk, dv, K, q, k, v, alpha, beta, S0, conv_in, dout, dS_final, dconv_out, taps,
                        dq, dk_, dv_, dalpha, dbeta, dS0, dconv_in, dtaps,
                        (int)((int64_t)units * i / nthreads), (int)((int64_t)units * (i + 1) / nthreads)};
    if (nthreads == 1) bwd_worker(&jobs[i]);
    else pthread_create(&th[i], NULL, bwd_worker, &jobs[i]);
  }
  if (nthreads > 1)
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  /* the generator, token by token */
  memset(dW1, 0, sizeof(double) * (size_t)G * D);
  memset(db1, 0, sizeof(double) * (size_t)G);
  memset(dW2, 0, sizeof(double) * (size_t)HK * G);
  memset(db2, 0, sizeof(double) * (size_t)HK);
  double* pre = (double*)malloc(sizeof(double) * (size_t)G);
  double* hid = (double*)malloc(sizeof(double) * (size_t)G);
  double* dp = (double*)malloc(sizeof(double) * (size_t)G);
  for (int64_t n = 0; n < n_tok; ++n) {
    const float* xr = x + n * D;
    for (int g = 0; g < G; ++g) {
      double acc = b1 ? (double)b1[g] : 0.0;
      for (int d = 0; d < D; ++d) acc += (double)W1[(int64_t)g * D + d] * (double)xr[d];
      pre[g] = acc;
      hid[g] = acc / (1.0 + exp(-acc));
    }
    const double* dt = dtaps + n * HK;
    for (int g = 0; g < G; ++g) {
      double dh = 0.0;
      for (int r = 0; r < HK; ++r) dh += (double)W2[(int64_t)r * G + g] * dt[r];
      const double s = 1.0 / (1.0 + exp(-pre[g]));
      dp[g] = dh * s * (1.0 + pre[g] * (1.0 - s));
    }
    for (int r = 0; r < HK; ++r) {
      db2[r] += dt[r];
      for (int g = 0; g < G; ++g) dW2[(int64_t)r * G + g] += dt[r] * hid[g];
    }
    for (int g = 0; g < G; ++g) {
      db1[g] += dp[g];
      for (int d = 0; d < D; ++d) dW1[(int64_t)g * D + d] += dp[g] * (double)xr[d];
    }
    for (int d = 0; d < D; ++d) {
      double s = 0.0;
      for (int g = 0; g < G; ++g) s += (double)W1[(int64_t)g * D + d] * dp[g];
      dx[n * D + d] = s;
    }
  }
  free(pre); free(hid); free(dp); free(taps); free(dtaps);
  return 0;
}
