/*
 * oracle.c -- plain, slow, fp64 CPU reference for scaled dot-product
 * attention, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes.  The article "Revolutionizing Web-Based AI: How a Plain
 * JavaScript Prototype Paved the Way for High-Performance WebGPU Flash
 * Attention 2" (section "Translating to WGSL and Optimizing Passes") describes
 * FlashAttention-2 as a blockwise evaluation of softmax attention whose
 * backward pass rebuilds the attention weights from Q, K and a saved
 * log-sum-exp.  Blocking changes only the order of the arithmetic, so the
 * oracle is the plain definition written out with the full N x N matrices
 * materialised, the opposite of what the fast path does:
 *
 *   S_ij  = scale * sum_k q_ik k_jk          (j <= i kept when causal)
 *   LSE_i = m_i + ln sum_j exp(S_ij - m_i),  m_i = max_j S_ij
 *   P_ij  = exp(S_ij - LSE_i)                (0 where masked)
 *   O_i   = sum_j P_ij v_j
 *
 * and, for a scalar loss L with upstream gradient dO = dL/dO,
 *
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = sum_k dO_ik v_jk
 *   D_i   = sum_j P_ij dP_ij                 (softmax-Jacobian form)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * Readings taken where the article is silent (all follow from the plain
 * definition of softmax attention): the scale multiplies the raw dot product;
 * the causal mask keeps j <= i; LSE is the natural-log log-sum-exp of the
 * scaled, masked logits; a row with every key masked gets O = 0,
 * LSE = -inf and zero gradients.
 *
 * Layout: every tensor is a contiguous row-major [B, H, N, d] array of
 * doubles; lse and delta are [B, H, N].  Heads are processed one after the
 * other, so only one head's N x N matrices are alive at a time.  OpenMP
 * parallelises over rows (or over key columns for dK, dV); every sum runs
 * in ascending index order (loops are only interchanged so that the inner
 * loop walks contiguous memory; no blocking and no reassociation).
 *
 * Return value: 0 on success, 1 on a bad argument, 2 when a scratch
 * allocation fails.
 */
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Threads an OpenMP region of this library will use (reported with timings). */
int oracle_max_threads(void) { return omp_get_max_threads(); }

static int bad_args(long B, long H, long N, long d) {
  return B < 0 || H < 0 || N < 0 || d <= 0;
}

/* Scaled, masked logits S (N x N) of one head. */
static void head_logits(const double* q, const double* k, double* S, long N,
                        long d, double scale, int causal) {
  long i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < N; ++i) {
    for (long j = 0; j < N; ++j) {
      if (causal && j > i) {
        S[i * N + j] = -INFINITY;
        continue;
      }
      double acc = 0.0;
      for (long c = 0; c < d; ++c) acc += q[i * d + c] * k[j * d + c];
      S[i * N + j] = scale * acc;
    }
  }
}

/* Row log-sum-exp of S, then S is overwritten by P = exp(S - LSE). */
static void head_softmax(double* S, double* lse, long N) {
  long i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < N; ++i) {
    double* row = S + i * N;
    double m = -INFINITY;
    for (long j = 0; j < N; ++j)
      if (row[j] > m) m = row[j];
    if (m == -INFINITY) { /* every key masked */
      lse[i] = -INFINITY;
      for (long j = 0; j < N; ++j) row[j] = 0.0;
      continue;
    }
    double sum = 0.0;
    for (long j = 0; j < N; ++j) sum += exp(row[j] - m);
    double L = m + log(sum);
    lse[i] = L;
    for (long j = 0; j < N; ++j) row[j] = exp(row[j] - L); /* exp(-inf) = 0 */
  }
}

int oracle_fwd_f64(const double* q, const double* k, const double* v,
                   double* o, double* lse, long B, long H, long N, long d,
                   double scale, int causal) {
  if (bad_args(B, H, N, d)) return 1;
  if (B == 0 || H == 0 || N == 0) return 0;
  double* P = (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
  if (!P) return 2;
  for (long bh = 0; bh < B * H; ++bh) {
    const double* qh = q + bh * N * d;
    const double* kh = k + bh * N * d;
    const double* vh = v + bh * N * d;
    double* oh = o + bh * N * d;
    double* lh = lse + bh * N;
    head_logits(qh, kh, P, N, d, scale, causal);
    head_softmax(P, lh, N);
    long i;
    /* O_i = sum_j P_ij v_j, summed over ascending j for every element. */
#pragma omp parallel for schedule(static)
    for (i = 0; i < N; ++i) {
      double* orow = oh + i * d;
      for (long c = 0; c < d; ++c) orow[c] = 0.0;
      for (long j = 0; j < N; ++j) {
        double p = P[i * N + j];
        for (long c = 0; c < d; ++c) orow[c] += p * vh[j * d + c];
      }
    }
  }
  free(P);
  return 0;
}

int oracle_bwd_f64(const double* q, const double* k, const double* v,
                   const double* dO, double* dq, double* dk, double* dv,
                   double* delta, long B, long H, long N, long d, double scale,
                   int causal) {
  if (bad_args(B, H, N, d)) return 1;
  if (B == 0 || H == 0 || N == 0) return 0;
  size_t nn = (size_t)N * (size_t)N;
  double* P = (double*)malloc(sizeof(double) * nn);
  double* dS = (double*)malloc(sizeof(double) * nn);
  double* lse = (double*)malloc(sizeof(double) * (size_t)N);
  double* D = (double*)malloc(sizeof(double) * (size_t)N);
  if (!P || !dS || !lse || !D) {
    free(P); free(dS); free(lse); free(D);
    return 2;
  }
  for (long bh = 0; bh < B * H; ++bh) {
    const double* qh = q + bh * N * d;
    const double* kh = k + bh * N * d;
    const double* vh = v + bh * N * d;
    const double* gh = dO + bh * N * d;
    double* dqh = dq + bh * N * d;
    double* dkh = dk + bh * N * d;
    double* dvh = dv + bh * N * d;

    /* Recompute P from the definition (the oracle keeps no forward state). */
    head_logits(qh, kh, P, N, d, scale, causal);
    head_softmax(P, lse, N);

    long i, j;
    /* dP_ij = dO_i . v_j, then D_i = sum_j P_ij dP_ij, then dS. */
#pragma omp parallel for schedule(static)
    for (i = 0; i < N; ++i) {
      double Di = 0.0;
      for (long jj = 0; jj < N; ++jj) {
        double acc = 0.0;
        for (long c = 0; c < d; ++c) acc += gh[i * d + c] * vh[jj * d + c];
        dS[i * N + jj] = acc; /* dP for now */
        Di += P[i * N + jj] * acc;
      }
      D[i] = Di;
      for (long jj = 0; jj < N; ++jj)
        dS[i * N + jj] = P[i * N + jj] * (dS[i * N + jj] - Di);
    }
    if (delta) memcpy(delta + bh * N, D, sizeof(double) * (size_t)N);

    /* dQ_i = scale * sum_j dS_ij k_j */
#pragma omp parallel for schedule(static)
    for (i = 0; i < N; ++i) {
      double* grow = dqh + i * d;
      for (long c = 0; c < d; ++c) grow[c] = 0.0;
      for (long jj = 0; jj < N; ++jj) {
        double s = dS[i * N + jj];
        for (long c = 0; c < d; ++c) grow[c] += s * kh[jj * d + c];
      }
      for (long c = 0; c < d; ++c) grow[c] *= scale;
    }
    /* dV_j = sum_i P_ij dO_i ; dK_j = scale * sum_i dS_ij q_i */
#pragma omp parallel for schedule(static)
    for (j = 0; j < N; ++j) {
      double* vrow = dvh + j * d;
      double* krow = dkh + j * d;
      for (long c = 0; c < d; ++c) vrow[c] = krow[c] = 0.0;
      for (long ii = 0; ii < N; ++ii) {
        double p = P[ii * N + j], s = dS[ii * N + j];
        for (long c = 0; c < d; ++c) {
          vrow[c] += p * gh[ii * d + c];
          krow[c] += s * qh[ii * d + c];
        }
      }
      for (long c = 0; c < d; ++c) krow[c] *= scale;
    }
  }
  free(P); free(dS); free(lse); free(D);
  return 0;
}

/*
 * Decoding: N_q new queries against a cache of N_k keys and values.  The
 * article names flash-decoding as a next primitive (section "Next Frontiers
 * in WebGPU ML", "Broader Opset Support") without defining it; it is read as
 * the same softmax attention with a rectangular score matrix,
 *
 *   S_ij  = scale * sum_k q_ik k_jk,  i < N_q, j < N_k
 *   LSE_i = m_i + ln sum_j exp(S_ij - m_i),  P_ij = exp(S_ij - LSE_i)
 *   O_i   = sum_j P_ij v_j
 *
 * where the queries are the last N_q positions of the sequence: with the
 * causal mask, query i sits at position N_k - N_q + i and keeps keys
 * j <= N_k - N_q + i (for N_q = N_k this is the mask of oracle_fwd_f64).
 * Splitting the cache over workgroups and merging their partial results is
 * how the fast path evaluates this; the oracle evaluates the definition.
 *
 * q, o: [B, H, N_q, d]; k, v: [B, H, N_k, d] (one key/value head per query
 * head: grouped heads are expanded by the caller); lse: [B, H, N_q].
 * Requires N_q <= N_k when causal and N_k >= 1 when N_q >= 1.
 */
int oracle_decode_f64(const double* q, const double* k, const double* v,
                      double* o, double* lse, long B, long H, long Nq, long Nk,
                      long d, double scale, int causal) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d <= 0) return 1;
  if (B == 0 || H == 0 || Nq == 0) return 0;
  if (Nk == 0 || (causal && Nq > Nk)) return 1;
  const long off = Nk - Nq; /* position of query 0 in the sequence */
  for (long bh = 0; bh < B * H; ++bh) {
    const double* qh = q + bh * Nq * d;
    const double* kh = k + bh * Nk * d;
    const double* vh = v + bh * Nk * d;
    double* oh = o + bh * Nq * d;
    double* lh = lse + bh * Nq;
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < Nq; ++i) {
      double* S = (double*)malloc(sizeof(double) * (size_t)Nk);
      if (!S) { lh[i] = NAN; continue; }
      const long last = causal ? off + i : Nk - 1; /* last visible key */
      double m = -INFINITY;
      for (long j = 0; j < Nk; ++j) {
        if (j > last) {
          S[j] = -INFINITY;
          continue;
        }
        double acc = 0.0;
        for (long c = 0; c < d; ++c) acc += qh[i * d + c] * kh[j * d + c];
        S[j] = scale * acc;
        if (S[j] > m) m = S[j];
      }
      double sum = 0.0;
      for (long j = 0; j < Nk; ++j) sum += exp(S[j] - m);
      const double L = m + log(sum);
      lh[i] = L;
      double* orow = oh + i * d;
      for (long c = 0; c < d; ++c) orow[c] = 0.0;
      for (long j = 0; j < Nk; ++j) {
        const double p = exp(S[j] - L);
        for (long c = 0; c < d; ++c) orow[c] += p * vh[j * d + c];
      }
      free(S);
    }
  }
  return 0;
}
