/*
 * CPU oracle for the batch-invariant GEMM — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load
 * this library. It shares no code, header or table with the GPU path; it
 * includes no HIP header and is built with plain gcc.
 *
 * What it computes is the plain definition of the matrix product that the
 * nondeterminism blog states in its section on batch-invariant matrix
 * multiplication: C_ij = sum_k A_ik B_kj, with the whole K reduction of one
 * output element done by one worker. Here the reduction is carried out in
 * IEEE binary64 with k ascending, after decoding every operand exactly:
 *
 *   - bf16: the 16 bits are the top half of an IEEE binary32 (exact widening);
 *   - OCP E4M3FN (the element format of MXFP8, the CANN issue's quantised
 *     path): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
 *     infinities, S.1111.111 is NaN, exponent field 0 is subnormal m/8*2^-6;
 *   - E8M0 (the MXFP8 block scale, one per 32 consecutive K elements): the
 *     byte e encodes 2^(e-127), 0xFF is NaN;
 *   - IEEE binary16: 1 sign bit, 5 exponent bits with bias 15, 10 mantissa
 *     bits, exponent field 0 subnormal m/1024*2^-14, field 31 infinity / NaN;
 *   - int8 operands are exact integers; their GEMM is accumulated exactly in
 *     int64 (integer addition is associative: no order question arises).
 *
 * It also holds the blog's RMSNorm in binary64 (section "batch-invariant
 * RMSNorm"), for the batch-invariant RMSNorm kernel.
 *
 * Every product is exact in binary64 (bf16*bf16 has at most 16 significant
 * bits, fp16*fp16 at most 22; a scaled E4M3*E4M3 product has at most 8). The only rounding is the
 * binary64 accumulation, bounded by the blog's sequential-sum bound
 * (section "unit roundoff"): |s_hat - s| <= gamma_{K-1} * sum_k |x_ik w_kj|,
 * gamma_n = n u / (1 - n u), u = 2^-53.
 *
 * The oracle also returns S_ij = sum_k |x_ik w_kj| (exact products, fp64 sum),
 * the scale against which GPU results are judged.
 *
 * Layouts (row-major, leading dimensions in elements):
 *   X[M,K] (ldx), W[K,N] (ldw), Y[M,N] and S[M,N] (ldy) in double,
 *   MX scales: XS[M, K/32] (ldxs), WS[K/32, N] (ldws), one byte each.
 *
 * Threads: OpenMP over output rows; each row's arithmetic is the same
 * sequence whatever the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoders */

double oracle_decode_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* E4M3FN from its definition (exponent bias 7, 3 mantissa bits). */
double oracle_decode_e4m3(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);           /* m/8 * 2^(1-7) */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

double oracle_decode_e8m0(uint8_t code) {
  if (code == 0xFF) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* IEEE binary16 from its definition (exponent bias 15, 10 mantissa bits). */
double oracle_decode_f16(uint16_t bits) {
  int s = bits >> 15;
  int e = (bits >> 10) & 31;
  int m = bits & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);           /* m/1024 * 2^(1-15) */
  else v = ldexp((double)(1024 + m), e - 25);          /* (1 + m/1024) * 2^(e-15) */
  return s ? -v : v;
}

static double e4m3_table[256];
static int e4m3_table_ready = 0;

static void build_e4m3_table(void) {
  if (e4m3_table_ready) return;
  for (int c = 0; c < 256; ++c) e4m3_table[c] = oracle_decode_e4m3((uint8_t)c);
  e4m3_table_ready = 1;
}

/* ---------------------------------------------------------- shared driver */

/*
 * Plain fp64 GEMM over already-decoded operands: for each row i, for k
 * ascending, for each column j: acc[j] += a_ik * b_kj. Y and (optionally) S
 * receive acc and the absolute-value sums. Exposed so the accumulation core
 * can be pinned on fp64 inputs (the blog's unrounded linspace example).
 */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const double* A, int64_t lda,
                    const double* B, int64_t ldb,
                    double* Y, int64_t ldy, double* S, int64_t lds) {
  if (M < 0 || N < 0 || K < 0) return 1;
  if (M == 0 || N == 0) return 0;
  if (!A || !B || !Y) return 1;
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < M; ++i) {
    double* acc = Y + i * ldy;
    double* sabs = S ? S + i * lds : NULL;
    for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
    if (sabs)
      for (int64_t j = 0; j < N; ++j) sabs[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double a = A[i * lda + k];
      const double* brow = B + k * ldb;
      for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
      if (sabs)
        for (int64_t j = 0; j < N; ++j) sabs[j] += fabs(a * brow[j]);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------- bf16 */

int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t* X, int64_t ldx,
                     const uint16_t* W, int64_t ldw,
                     double* Y, int64_t ldy, double* S, int64_t lds) {
  if (M < 0 || N < 0 || K < 0 || ldx < K || ldw < N || ldy < N) return 1;
  if (M == 0 || N == 0) return 0;
  double* A = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
  double* B = (double*)malloc(sizeof(double) * (size_t)(K * N + 1));
  if (!A || !B) { free(A); free(B); return 2; }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) A[i * K + k] = oracle_decode_bf16(X[i * ldx + k]);
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < N; ++j) B[k * N + j] = oracle_decode_bf16(W[k * ldw + j]);
  int rc = oracle_gemm_f64(M, N, K, A, K, B, N, Y, ldy, S, lds);
  free(A);
  free(B);
  return rc;
}

/* ------------------------------------------------------------------- fp16 */

int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t* X, int64_t ldx,
                    const uint16_t* W, int64_t ldw,
                    double* Y, int64_t ldy, double* S, int64_t lds) {
  if (M < 0 || N < 0 || K < 0 || ldx < K || ldw < N || ldy < N) return 1;
  if (M == 0 || N == 0) return 0;
  double* A = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
  double* B = (double*)malloc(sizeof(double) * (size_t)(K * N + 1));
  if (!A || !B) { free(A); free(B); return 2; }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) A[i * K + k] = oracle_decode_f16(X[i * ldx + k]);
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < N; ++j) B[k * N + j] = oracle_decode_f16(W[k * ldw + j]);
  int rc = oracle_gemm_f64(M, N, K, A, K, B, N, Y, ldy, S, lds);
  free(A);
  free(B);
  return rc;
}

/* ------------------------------------------------------------------- int8 */

/* Y_ij = sum_k X_ik W_kj in int64, k ascending (exact). */
int oracle_gemm_i8(int64_t M, int64_t N, int64_t K,
                   const int8_t* X, int64_t ldx,
                   const int8_t* W, int64_t ldw,
                   int64_t* Y, int64_t ldy) {
  if (M < 0 || N < 0 || K < 0 || ldx < K || ldw < N || ldy < N) return 1;
  if (M == 0 || N == 0) return 0;
  if (!X || !W || !Y) return 1;
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < M; ++i) {
    int64_t* acc = Y + i * ldy;
    for (int64_t j = 0; j < N; ++j) acc[j] = 0;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t a = X[i * ldx + k];
      const int8_t* wrow = W + k * ldw;
      for (int64_t j = 0; j < N; ++j) acc[j] += a * (int64_t)wrow[j];
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ MXFP8 */

/*
 * x~_ik = e4m3(X_ik) * 2^(XS[i, k/32] - 127),  w~_kj = e4m3(W_kj) * 2^(WS[k/32, j] - 127),
 * then the fp64 product of the scaled operands. Scaling by a power of two is
 * exact, so this equals applying the two block scales to each block's
 * partial sum.
 */
int oracle_gemm_mxfp8(int64_t M, int64_t N, int64_t K,
                      const uint8_t* X, int64_t ldx,
                      const uint8_t* W, int64_t ldw,
                      const uint8_t* XS, int64_t ldxs,
                      const uint8_t* WS, int64_t ldws,
                      double* Y, int64_t ldy, double* S, int64_t lds) {
  if (M < 0 || N < 0 || K < 0 || (K % 32) != 0 || ldx < K || ldw < N || ldy < N) return 1;
  if (ldxs < K / 32 || ldws < N) return 1;
  if (M == 0 || N == 0) return 0;
  build_e4m3_table();
  double* A = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
  double* B = (double*)malloc(sizeof(double) * (size_t)(K * N + 1));
  if (!A || !B) { free(A); free(B); return 2; }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k)
      A[i * K + k] = e4m3_table[X[i * ldx + k]] * oracle_decode_e8m0(XS[i * ldxs + k / 32]);
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < N; ++j)
      B[k * N + j] = e4m3_table[W[k * ldw + j]] * oracle_decode_e8m0(WS[(k / 32) * ldws + j]);
  int rc = oracle_gemm_f64(M, N, K, A, K, B, N, Y, ldy, S, lds);
  free(A);
  free(B);
  return rc;
}

/* --------------------------------------------------------------- RMSNorm */

/*
 * The blog's batch-invariant RMSNorm section defines
 *   RMSNorm(x_i) = x_i / sqrt((1/d) sum_j x_ij^2 + eps) (.) gamma.
 * Here in binary64: s = sum_j x_ij^2 with j ascending, then
 * y_ij = x_ij / sqrt(s / d + eps) * gamma_j. Operands are decoded exactly
 * (bf16 bits, or binary32 values widened).
 */
static void rmsnorm_rows(int64_t M, int64_t D, const double* X, const double* G, double eps, double* Y,
                         int64_t ldy) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) {
    const double* x = X + i * D;
    double s = 0.0;
    for (int64_t j = 0; j < D; ++j) s += x[j] * x[j];
    const double den = sqrt(s / (double)D + eps);
    for (int64_t j = 0; j < D; ++j) Y[i * ldy + j] = x[j] / den * G[j];
  }
}

int oracle_rmsnorm_bf16(int64_t M, int64_t D, const uint16_t* X, int64_t ldx, const uint16_t* gamma, double eps,
                        double* Y, int64_t ldy) {
  if (M < 0 || D < 1 || ldx < D || ldy < D) return 1;
  if (M == 0) return 0;
  double* A = (double*)malloc(sizeof(double) * (size_t)(M * D));
  double* G = (double*)malloc(sizeof(double) * (size_t)D);
  if (!A || !G) { free(A); free(G); return 2; }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < D; ++j) A[i * D + j] = oracle_decode_bf16(X[i * ldx + j]);
  for (int64_t j = 0; j < D; ++j) G[j] = oracle_decode_bf16(gamma[j]);
  rmsnorm_rows(M, D, A, G, eps, Y, ldy);
  free(A);
  free(G);
  return 0;
}

int oracle_rmsnorm_f32(int64_t M, int64_t D, const float* X, int64_t ldx, const float* gamma, double eps,
                       double* Y, int64_t ldy) {
  if (M < 0 || D < 1 || ldx < D || ldy < D) return 1;
  if (M == 0) return 0;
  double* A = (double*)malloc(sizeof(double) * (size_t)(M * D));
  double* G = (double*)malloc(sizeof(double) * (size_t)D);
  if (!A || !G) { free(A); free(G); return 2; }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < D; ++j) A[i * D + j] = (double)X[i * ldx + j];
  for (int64_t j = 0; j < D; ++j) G[j] = (double)gamma[j];
  rmsnorm_rows(M, D, A, G, eps, Y, ldy);
  free(A);
  free(G);
  return 0;
}

/* ------------------------------------------------------------- attention */

/*
 * The blog's batch-invariant attention section: the query at position i of a
 * sequence attends to that sequence's keys and values at positions j <= i
 * (the causal mask),
 *   o = sum_{j <= i} softmax_j(scale * q . k_j) v_j,
 * where the section's formula has scale = 1/sqrt(d); it is an argument here so
 * that the caller's rounded value is the one used. Decode is a query at the
 * last position of its sequence.
 * Inputs, bf16 bit patterns, row-major:
 *   Q [T][H][D]       query token t, head h;
 *   K, V [nseq][maxlen][Hkv][D]   keys and values of each sequence by logical
 *                     position (what the KV cache holds, in order);
 *   seq[t], pos[t]    the token's sequence and position (pos < maxlen).
 * Query head h reads key/value head h / (H / Hkv) (grouped-query attention).
 * Per (t, h), in binary64 with j ascending:
 *   s_j = scale * sum_e q_e k_je (e ascending), m = max_j s_j,
 *   w_j = exp(s_j - m), O = sum_j w_j v_j / sum_j w_j,
 *   S = sum_j w_j |v_j| / sum_j w_j (the scale of the error metric),
 *   stats = (A, Mabs, R): A = max_j scale * sum_e |q_e k_je|,
 *   Mabs = max_j |s_j|, R = m - min_j s_j (inputs of the error bound).
 * Returns 1 for bad sizes or a token whose seq/pos is out of range.
 */
int oracle_attention(int64_t T, int64_t H, int64_t Hkv, int64_t D, int64_t nseq, int64_t maxlen,
                     const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int32_t* seq,
                     const int32_t* pos, double scale, double* O, double* S, double* stats) {
  if (T < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || D < 1 || nseq < 1 || maxlen < 1) return 1;
  for (int64_t t = 0; t < T; ++t)
    if (seq[t] < 0 || seq[t] >= nseq || pos[t] < 0 || pos[t] >= maxlen) return 1;
  int bad = 0;
  int64_t th;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (th = 0; th < T * H; ++th) {
    const int64_t t = th / H, h = th % H;
    const int64_t sq = seq[t];
    const int64_t p = pos[t];
    const int64_t L = p + 1; /* keys j = 0 .. p */
    const int64_t g = h / (H / Hkv);
    double* q = (double*)malloc(sizeof(double) * (size_t)D);
    double* s = (double*)malloc(sizeof(double) * (size_t)(p + 1));
    double* w = (double*)malloc(sizeof(double) * (size_t)(p + 1));
    if (!q || !s || !w) {
      bad = 1;
      free(q); free(s); free(w);
      continue;
    }
    for (int64_t e = 0; e < D; ++e) q[e] = oracle_decode_bf16(Q[(t * H + h) * D + e]);
    double a_max = 0.0, s_abs = 0.0, m = -INFINITY, s_min = INFINITY;
    for (int64_t j = 0; j < L; ++j) {
      const uint16_t* k = K + ((sq * maxlen + j) * Hkv + g) * D;
      double d = 0.0, da = 0.0;
      for (int64_t e = 0; e < D; ++e) {
        const double prod = q[e] * oracle_decode_bf16(k[e]);
        d += prod;
        da += fabs(prod);
      }
      s[j] = scale * d;
      if (scale * da > a_max) a_max = scale * da;
      if (fabs(s[j]) > s_abs) s_abs = fabs(s[j]);
      if (s[j] > m) m = s[j];
      if (s[j] < s_min) s_min = s[j];
    }
    double den = 0.0;
    for (int64_t j = 0; j < L; ++j) {
      w[j] = exp(s[j] - m);
      den += w[j];
    }
    for (int64_t e = 0; e < D; ++e) {
      double num = 0.0, nabs = 0.0;
      for (int64_t j = 0; j < L; ++j) {
        const double v = oracle_decode_bf16(V[((sq * maxlen + j) * Hkv + g) * D + e]);
        num += w[j] * v;
        nabs += w[j] * fabs(v);
      }
      O[(t * H + h) * D + e] = num / den;
      if (S) S[(t * H + h) * D + e] = nabs / den;
    }
    if (stats) {
      stats[(t * H + h) * 3 + 0] = a_max;
      stats[(t * H + h) * 3 + 1] = s_abs;
      stats[(t * H + h) * 3 + 2] = m - s_min;
    }
    free(q);
    free(s);
    free(w);
  }
  return bad ? 2 : 0;
}

/* ------------------------------------------------------------------ misc */

int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}
