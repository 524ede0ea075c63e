/*
 * oracle.c -- plain, slow, fp64 CPU reference for exact scaled-dot-product
 * attention (forward O and per-row log-sum-exp, and the backward dQ/dK/dV).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU path and must never be used as a
 * fallback for it.
 *
 * What it computes.  The pages about FlashAttention-4 (QbitAI's news piece
 * "英伟达最强B200算力浪费60%", and the Tencent Cloud article "AI Infra 系列
 * 第六章 GPU 性能工程（二）", section 7 on FA4's four techniques) describe a
 * fused *exact* attention kernel whose speed tricks (online softmax that is
 * rescaled only when the running maximum threatens stability; a polynomial
 * exp2 on the FMA units) leave the mathematical result unchanged.  The
 * result they reach is the textbook definition, written out here directly
 * and with no blocking, fusion or reordering:
 *
 *   s_ij  = scale * sum_d Q_id K_jd           for visible j
 *   m_i   = max_j s_ij,   l_i = sum_j exp(s_ij - m_i)
 *   P_ij  = exp(s_ij - m_i) / l_i
 *   O_i   = sum_j P_ij V_j,       LSE_i = m_i + ln(l_i)   (natural log)
 *
 * Visible keys: all j, or j <= i when causal (the query and key sequences
 * have the same length, so the top-left and bottom-right diagonals agree).
 *
 * Backward (closed-form gradient of the same definition; the backward pass
 * recomputes P from the log-sum-exp rather than storing it, the
 * recomputation lever in section 5 of the Tencent Cloud article):
 *
 *   Delta_i = sum_d dO_id O_id
 *   dV_j    = sum_i P_ij dO_i
 *   dP_ij   = dO_i . V_j,          dS_ij = P_ij (dP_ij - Delta_i)
 *   dQ_i    = scale * sum_j dS_ij K_j,   dK_j = scale * sum_i dS_ij Q_i
 *
 * Every tensor is fp64, contiguous [B][H][S][D] (LSE: [B][H][S]).  The
 * callers upcast the bf16 inputs exactly.  OpenMP splits independent rows
 * (or key columns) across threads; each output element is produced by one
 * thread with a fixed summation order, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <omp.h>

/* Number of threads the parallel loops use (OpenMP's current setting). */
int oracle_max_threads(void) { return omp_get_max_threads(); }

void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

/* Number of keys visible to query row `pos` in a sequence of S keys. */
static long visible_keys(long pos, long S, int causal) {
  return causal ? pos + 1 : S;
}

/*
 * One query row against the keys/values of one head.
 *   q[D]        the query row
 *   pos         its position in the sequence (only used when causal)
 *   k, v        [S][D] keys and values of the same (batch, head)
 *   s_buf[S]    scratch for the scaled logits
 *   o[D], *lse  outputs
 */
static void fwd_one_row(const double* q, long pos, const double* k,
                        const double* v, long S, long D, double scale,
                        int causal, double* s_buf, double* o, double* lse) {
  const long n = visible_keys(pos, S, causal);
  double m = -INFINITY;
  for (long j = 0; j < n; ++j) {
    double dot = 0.0;
    for (long d = 0; d < D; ++d) dot += q[d] * k[j * D + d];
    s_buf[j] = scale * dot;
    if (s_buf[j] > m) m = s_buf[j];
  }
  double l = 0.0;
  for (long j = 0; j < n; ++j) {
    s_buf[j] = exp(s_buf[j] - m); /* unnormalised probability */
    l += s_buf[j];
  }
  for (long d = 0; d < D; ++d) o[d] = 0.0;
  for (long j = 0; j < n; ++j) {
    const double p = s_buf[j] / l;
    for (long d = 0; d < D; ++d) o[d] += p * v[j * D + d];
  }
  *lse = m + log(l);
}

/*
 * Forward for an arbitrary set of query rows of ONE head (used to sample a
 * few rows of a large problem).
 *   q_rows[n][D]  the query rows, pos[n] their sequence positions (0..S-1)
 *   k, v [S][D]   keys and values of that head
 *   o_rows[n][D], lse_rows[n]  outputs
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attn_fwd_rows(const double* q_rows, const long* pos, long n,
                         const double* k, const double* v, long S, long D,
                         double scale, int causal, double* o_rows,
                         double* lse_rows) {
  if (n < 0 || S <= 0 || D <= 0) return -1;
  for (long r = 0; r < n; ++r)
    if (pos[r] < 0 || pos[r] >= S) return -1;
  int err = 0;
#pragma omp parallel
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)S);
    if (!s_buf) {
#pragma omp atomic write
      err = -1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (long r = 0; r < n; ++r)
        fwd_one_row(q_rows + r * D, pos[r], k, v, S, D, scale, causal, s_buf,
                    o_rows + r * D, lse_rows + r);
      free(s_buf);
    }
  }
  return err;
}

/*
 * Full forward over [B][H][S][D].  Every row of every head is independent.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attn_fwd(const double* q, const double* k, const double* v,
                    long B, long H, long S, long D, double scale, int causal,
                    double* o, double* lse) {
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0) return -1;
  const long rows = B * H * S;
  int err = 0;
#pragma omp parallel
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)S);
    if (!s_buf) {
#pragma omp atomic write
      err = -1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (long r = 0; r < rows; ++r) {
        const long head = r / S, i = r % S;
        const double* kh = k + head * S * D;
        const double* vh = v + head * S * D;
        fwd_one_row(q + r * D, i, kh, vh, S, D, scale, causal, s_buf,
                    o + r * D, lse + r);
      }
      free(s_buf);
    }
  }
  return err;
}

/*
 * Backward for ONE head, all inputs [S][D].  The oracle computes its own
 * fp64 forward (O and LSE) first, then the closed-form gradients above.
 *   pass 1 (parallel over query rows i):  LSE_i, O_i, Delta_i, dQ_i
 *   pass 2 (parallel over key rows j):    dK_j, dV_j, summing over the
 *                                         queries i that see key j
 * Outputs dq, dk, dv [S][D]; o_out [S][D] and lse_out [S] may be NULL.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attn_bwd_head(const double* q, const double* k, const double* v,
                         const double* dout, long S, long D, double scale,
                         int causal, double* dq, double* dk, double* dv,
                         double* o_out, double* lse_out) {
  if (S <= 0 || D <= 0) return -1;
  double* o = (double*)malloc(sizeof(double) * (size_t)(S * D));
  double* lse = (double*)malloc(sizeof(double) * (size_t)S);
  double* delta = (double*)malloc(sizeof(double) * (size_t)S);
  if (!o || !lse || !delta) {
    free(o); free(lse); free(delta);
    return -1;
  }
  int err = 0;
  /* pass 1: forward row, Delta_i and dQ_i */
#pragma omp parallel
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)S);
    if (!s_buf) {
#pragma omp atomic write
      err = -1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (long i = 0; i < S; ++i) {
        const double* qi = q + i * D;
        const double* doi = dout + i * D;
        fwd_one_row(qi, i, k, v, S, D, scale, causal, s_buf, o + i * D,
                    lse + i);
        double dl = 0.0;
        for (long d = 0; d < D; ++d) dl += doi[d] * o[i * D + d];
        delta[i] = dl;
        double* dqi = dq + i * D;
        for (long d = 0; d < D; ++d) dqi[d] = 0.0;
        const long n = visible_keys(i, S, causal);
        for (long j = 0; j < n; ++j) {
          double dot = 0.0;
          for (long d = 0; d < D; ++d) dot += qi[d] * k[j * D + d];
          const double p = exp(scale * dot - lse[i]);
          double dp = 0.0;
          for (long d = 0; d < D; ++d) dp += doi[d] * v[j * D + d];
          const double ds = p * (dp - delta[i]);
          for (long d = 0; d < D; ++d) dqi[d] += ds * k[j * D + d];
        }
        for (long d = 0; d < D; ++d) dqi[d] *= scale;
      }
      free(s_buf);
    }
  }
  /* pass 2: dK_j and dV_j over the queries that see key j */
  if (!err) {
#pragma omp parallel for schedule(dynamic, 4)
    for (long j = 0; j < S; ++j) {
      const double* kj = k + j * D;
      const double* vj = v + j * D;
      double* dkj = dk + j * D;
      double* dvj = dv + j * D;
      for (long d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
      const long i0 = causal ? j : 0;
      for (long i = i0; i < S; ++i) {
        const double* qi = q + i * D;
        const double* doi = dout + i * D;
        double dot = 0.0;
        for (long d = 0; d < D; ++d) dot += qi[d] * kj[d];
        const double p = exp(scale * dot - lse[i]);
        double dp = 0.0;
        for (long d = 0; d < D; ++d) dp += doi[d] * vj[d];
        const double ds = p * (dp - delta[i]);
        for (long d = 0; d < D; ++d) {
          dvj[d] += p * doi[d];
          dkj[d] += ds * qi[d];
        }
      }
      for (long d = 0; d < D; ++d) dkj[d] *= scale;
    }
  }
  if (!err && o_out)
    for (long x = 0; x < S * D; ++x) o_out[x] = o[x];
  if (!err && lse_out)
    for (long x = 0; x < S; ++x) lse_out[x] = lse[x];
  free(o); free(lse); free(delta);
  return err;
}

/* Backward over [B][H][S][D]: one head after another. */
int oracle_attn_bwd(const double* q, const double* k, const double* v,
                    const double* dout, long B, long H, long S, long D,
                    double scale, int causal, double* dq, double* dk,
                    double* dv) {
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0) return -1;
  for (long hd = 0; hd < B * H; ++hd) {
    const long off = hd * S * D;
    int rc = oracle_attn_bwd_head(q + off, k + off, v + off, dout + off, S, D,
                                  scale, causal, dq + off, dk + off, dv + off,
                                  NULL, NULL);
    if (rc) return rc;
  }
  return 0;
}

/*
 * Causal backward restricted to the last n positions of ONE head (used to
 * check the end of a sequence too long for a whole-head oracle).  With the
 * causal mask, key j >= S-n is seen only by queries i >= j, all of them in
 * the last n rows, so dK_j and dV_j of those keys need the forward of just
 * those rows; dQ_i of those rows sums over every key j <= i.  Same
 * definitions as oracle_attn_bwd_head, evaluated for these rows and keys.
 *   q_tail[n][D], do_tail[n][D]  query and dO rows S-n .. S-1
 *   k, v [S][D]                  all keys and values of the head
 *   dq_tail, dk_tail, dv_tail [n][D]  gradients of rows / keys S-n .. S-1
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attn_bwd_causal_tail(const double* q_tail, const double* do_tail,
                                long n, const double* k, const double* v,
                                long S, long D, double scale, double* dq_tail,
                                double* dk_tail, double* dv_tail) {
  if (n <= 0 || n > S || D <= 0) return -1;
  const long t0 = S - n;
  double* o = (double*)malloc(sizeof(double) * (size_t)(n * D));
  double* lse = (double*)malloc(sizeof(double) * (size_t)n);
  double* delta = (double*)malloc(sizeof(double) * (size_t)n);
  if (!o || !lse || !delta) {
    free(o); free(lse); free(delta);
    return -1;
  }
  int err = 0;
  /* rows S-n .. S-1: forward, Delta_i and dQ_i over keys 0 .. i */
#pragma omp parallel
  {
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)S);
    if (!s_buf) {
#pragma omp atomic write
      err = -1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long r = 0; r < n; ++r) {
        const long i = t0 + r;
        const double* qi = q_tail + r * D;
        const double* doi = do_tail + r * D;
        fwd_one_row(qi, i, k, v, S, D, scale, 1, s_buf, o + r * D, lse + r);
        double dl = 0.0;
        for (long d = 0; d < D; ++d) dl += doi[d] * o[r * D + d];
        delta[r] = dl;
        double* dqi = dq_tail + r * D;
        for (long d = 0; d < D; ++d) dqi[d] = 0.0;
        for (long j = 0; j <= i; ++j) {
          double dot = 0.0;
          for (long d = 0; d < D; ++d) dot += qi[d] * k[j * D + d];
          const double p = exp(scale * dot - lse[r]);
          double dp = 0.0;
          for (long d = 0; d < D; ++d) dp += doi[d] * v[j * D + d];
          const double ds = p * (dp - delta[r]);
          for (long d = 0; d < D; ++d) dqi[d] += ds * k[j * D + d];
        }
        for (long d = 0; d < D; ++d) dqi[d] *= scale;
      }
      free(s_buf);
    }
  }
  /* keys S-n .. S-1: dK_j and dV_j over the queries i = j .. S-1 */
  if (!err) {
#pragma omp parallel for schedule(dynamic, 1)
    for (long c = 0; c < n; ++c) {
      const long j = t0 + c;
      const double* kj = k + j * D;
      const double* vj = v + j * D;
      double* dkj = dk_tail + c * D;
      double* dvj = dv_tail + c * D;
      for (long d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
      for (long r = c; r < n; ++r) {
        const double* qi = q_tail + r * D;
        const double* doi = do_tail + r * D;
        double dot = 0.0;
        for (long d = 0; d < D; ++d) dot += qi[d] * kj[d];
        const double p = exp(scale * dot - lse[r]);
        double dp = 0.0;
        for (long d = 0; d < D; ++d) dp += doi[d] * vj[d];
        const double ds = p * (dp - delta[r]);
        for (long d = 0; d < D; ++d) {
          dvj[d] += p * doi[d];
          dkj[d] += ds * qi[d];
        }
      }
      for (long d = 0; d < D; ++d) dkj[d] *= scale;
    }
  }
  free(o); free(lse); free(delta);
  return err;
}
