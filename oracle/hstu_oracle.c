/*
 * hstu_oracle.c -- plain, slow, fp64 CPU definition of the HSTU layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no source with the GPU path.
 *
 * Every value is widened to double on entry and nothing is rounded in
 * between: the result is the exact real-valued definition up to fp64
 * summation order.  Loops are written in the most direct form on purpose.
 *
 * Sources (page title, section):
 *  [AS]  "Actions Speak Louder than Words" reading notes (paper-archivist.com),
 *        §3.1 eqs. (1)-(3) and the list under them, §3.2 pointwise aggregated
 *        attention.
 *  [SC]  "4.4 推荐模型的 Scaling" (llm-learning-path), section "HSTU 层" and the
 *        toy HSTULayer in section "代码" (chunk order u,v,q,k; per-head split;
 *        lower-triangular mask including the diagonal; SiLU then mask).
 *  [GR]  GenRank article (joto.ai), "工业场景中的高效生成式排序GenRank",
 *        part (2): ALiBi as the relative position/time bias.
 *  The bucketed rab^{p,t} form (position offset table + log2 time-delta
 *  table) is the one the workload definition states; the pages only say the
 *  real implementation buckets relative position and time ([SC], remark after
 *  the toy code).
 *
 * Readings where the pages are silent (also listed in the design notes):
 *  - alpha multiplies Q K^T inside the SiLU; out_scale multiplies the sum
 *    afterwards (1 by default, 1/n reproduces the toy's division).
 *  - time delta < 0 falls in bucket 0; the bucket is floor(log2(1+dt))
 *    clipped to [0, NT-1], computed on integers.
 *  - ALiBi bias is -slope_h * (i - j).
 *  - positions i, j are 0-based and local to the user's sequence.
 */
#include <stdint.h>
#include <stdlib.h>
#include <math.h>
#include <string.h>

enum { ORACLE_BIAS_NONE = 0, ORACLE_BIAS_RAB_PT = 1, ORACLE_BIAS_ALIBI = 2 };

/* SiLU(x) = x * sigmoid(x) = x / (1 + e^{-x})   [AS §3.1: phi1 = phi2 = SiLU] */
static double silu(double x) { return x / (1.0 + exp(-x)); }

/* Position bucket: the offset i - j clipped to [0, P-1]. */
int32_t oracle_pos_bucket(int64_t i_minus_j, int32_t num_pos_buckets) {
  if (i_minus_j < 0) return 0;
  if (i_minus_j > (int64_t)num_pos_buckets - 1) return num_pos_buckets - 1;
  return (int32_t)i_minus_j;
}

/* Time bucket: floor(log2(1 + dt)) clipped to [0, NT-1], on integers.
 * floor(log2(u)) for an integer u >= 1 is the number of times u can be halved
 * before it reaches 1. */
int32_t oracle_time_bucket(int64_t dt, int32_t num_time_buckets) {
  if (dt < 0) dt = 0;
  uint64_t u = (uint64_t)dt + 1u;
  int32_t e = 0;
  while (u > 1u) { u >>= 1; e++; }
  if (e > num_time_buckets - 1) e = num_time_buckets - 1;
  return e;
}

/* Bucket histograms of every row: for user b's local row i, pos_counts[t][p] and
 * time_counts[t][k] (t = offsets[b] + i) count the keys j <= i whose position bucket is p and
 * whose time bucket is k.  Used to check the integer bucket indexing of the attention. */
void oracle_bucket_counts(int32_t B, const int64_t* offsets, const int64_t* ts, int32_t num_pos,
                          int32_t num_time, int32_t* pos_counts, int32_t* time_counts) {
  for (int32_t b = 0; b < B; ++b) {
    const int64_t base = offsets[b], n = offsets[b + 1] - offsets[b];
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
      int32_t* pc = pos_counts + (base + i) * num_pos;
      int32_t* tc = time_counts + (base + i) * num_time;
      for (int64_t j = 0; j <= i; ++j) {
        pc[oracle_pos_bucket(i - j, num_pos)]++;
        tc[oracle_time_bucket(ts[base + i] - ts[base + j], num_time)]++;
      }
    }
  }
}

typedef struct {
  int32_t kind;
  const int64_t* ts;      /* [T] timestamps (RAB_PT)                        */
  const double* w_pos;    /* [H_tab * stride_p] position table              */
  const double* w_time;   /* [H_tab * stride_t] time table                  */
  int32_t num_pos, num_time;
  int64_t head_stride_pos, head_stride_time; /* 0 = one table for all heads */
  const double* slopes;   /* [H] ALiBi slopes                               */
} oracle_bias;

/* rab^{p,t}(i, j) for head h of a user whose first token is token `base`. */
static double bias_value(const oracle_bias* bs, int h, int64_t base, int64_t i, int64_t j) {
  if (bs->kind == ORACLE_BIAS_RAB_PT) {
    int32_t pb = oracle_pos_bucket(i - j, bs->num_pos);
    int32_t tb = oracle_time_bucket(bs->ts[base + i] - bs->ts[base + j], bs->num_time);
    return bs->w_pos[h * bs->head_stride_pos + pb] + bs->w_time[h * bs->head_stride_time + tb];
  }
  if (bs->kind == ORACLE_BIAS_ALIBI) {
    return -bs->slopes[h] * (double)(i - j);
  }
  return 0.0;
}

/* One output row of eq. (2) for user b, head h, local row i:
 *   O[i,:] = out_scale * sum_{j <= i} SiLU(alpha * <q_i, k_j> + rab(i,j)) * v_j
 * q, k, v are [T, H, d] with token row strides (in elements). */
/* Mirror mode only: w rounded to the nearest bfloat16 (8 significant bits, ties to even). */
static double round_bf16(double w) {
  int e;
  const double m = frexp(w, &e);
  return ldexp(nearbyint(m * 256.0), e - 8);
}

static void attn_row(int64_t base, int h, int64_t i, int H, int dqk, int dv,
                     const double* q, int64_t qs, const double* k, int64_t ks,
                     const double* v, int64_t vs, const oracle_bias* bs,
                     double alpha, double out_scale, double weight_unit, double* out /* [dv] */) {
  for (int c = 0; c < dv; c++) out[c] = 0.0;
  const double* qi = q + (base + i) * qs + (int64_t)h * dqk;
  for (int64_t j = 0; j <= i; j++) {
    const double* kj = k + (base + j) * ks + (int64_t)h * dqk;
    const double* vj = v + (base + j) * vs + (int64_t)h * dv;
    double s = 0.0;
    for (int c = 0; c < dqk; c++) s += qi[c] * kj[c];
    double a = silu(alpha * s + bias_value(bs, h, base, i, j));
    /* mirror mode: the weight kept as a bf16 multiple of weight_unit */
    if (weight_unit != 0.0) a = weight_unit * round_bf16(a / weight_unit);
    for (int c = 0; c < dv; c++) out[c] += a * vj[c];
  }
  for (int c = 0; c < dv; c++) out[c] *= out_scale;
  (void)H;
}

/* Full jagged attention: o is [T, H, dv] contiguous.  weight_unit != 0 is the mirror mode
 * (each SiLU weight kept as weight_unit times a bf16 value); 0 is the exact definition. */
void oracle_attention_mirror(int32_t B, int32_t H, int32_t dqk, int32_t dv,
                             const int64_t* offsets, const double* q, int64_t q_stride,
                             const double* k, int64_t k_stride, const double* v, int64_t v_stride,
                             int32_t bias_kind, const int64_t* ts, const double* w_pos,
                             int32_t num_pos, int64_t head_stride_pos, const double* w_time,
                             int32_t num_time, int64_t head_stride_time, const double* slopes,
                             double alpha, double out_scale, double weight_unit, double* o) {
  oracle_bias bs = {bias_kind, ts, w_pos, w_time, num_pos, num_time,
                    head_stride_pos, head_stride_time, slopes};
  int64_t n_items = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t it = 0; it < n_items; it++) {
    int32_t b = (int32_t)(it / H), h = (int32_t)(it % H);
    int64_t base = offsets[b], n = offsets[b + 1] - offsets[b];
    for (int64_t i = 0; i < n; i++)
      attn_row(base, h, i, H, dqk, dv, q, q_stride, k, k_stride, v, v_stride, &bs, alpha,
               out_scale, weight_unit, o + ((base + i) * H + h) * (int64_t)dv);
  }
}

void oracle_attention(int32_t B, int32_t H, int32_t dqk, int32_t dv, const int64_t* offsets,
                      const double* q, int64_t q_stride, const double* k, int64_t k_stride,
                      const double* v, int64_t v_stride, int32_t bias_kind, const int64_t* ts,
                      const double* w_pos, int32_t num_pos, int64_t head_stride_pos,
                      const double* w_time, int32_t num_time, int64_t head_stride_time,
                      const double* slopes, double alpha, double out_scale, double* o) {
  oracle_attention_mirror(B, H, dqk, dv, offsets, q, q_stride, k, k_stride, v, v_stride,
                          bias_kind, ts, w_pos, num_pos, head_stride_pos, w_time, num_time,
                          head_stride_time, slopes, alpha, out_scale, 0.0, o);
}

/* Selected rows only: rows[r] = (token t, head h); out is [R, dv].
 * Used to check outputs at full workload sizes one row at a time. */
void oracle_attention_rows(int32_t B, int32_t H, int32_t dqk, int32_t dv, const int64_t* offsets,
                           const double* q, int64_t q_stride, const double* k, int64_t k_stride,
                           const double* v, int64_t v_stride, int32_t bias_kind, const int64_t* ts,
                           const double* w_pos, int32_t num_pos, int64_t head_stride_pos,
                           const double* w_time, int32_t num_time, int64_t head_stride_time,
                           const double* slopes, double alpha, double out_scale, int64_t R,
                           const int64_t* row_token, const int32_t* row_head, double* out) {
  oracle_bias bs = {bias_kind, ts, w_pos, w_time, num_pos, num_time,
                    head_stride_pos, head_stride_time, slopes};
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < R; r++) {
    int64_t t = row_token[r];
    int32_t b = 0;
    while (b < B && offsets[b + 1] <= t) b++; /* user that owns token t */
    int64_t base = offsets[b];
    attn_row(base, row_head[r], t - base, H, dqk, dv, q, q_stride, k, k_stride, v, v_stride,
             &bs, alpha, out_scale, 0.0, out + r * (int64_t)dv);
  }
}

/* Gradients of eq. (2) ("Actions Speak Louder than Words" reading notes §3.1 eq. (2), §3.2)
 * for an upstream gradient dO of O, by the chain rule on each term a_ij v_j of row i:
 *   x_ij = alpha <q_i, k_j> + rab(i, j),  a_ij = SiLU(x_ij),  SiLU'(x) = s (1 + x (1 - s)),
 *   s = 1 / (1 + e^-x)   (product rule on x * s(x));
 *   dV_j += out_scale a_ij dO_i;   g_ij = out_scale <dO_i, v_j> SiLU'(x_ij);
 *   dQ_i += alpha g_ij k_j;   dK_j += alpha g_ij q_i;
 *   d w_pos[h][pos bucket(i, j)] += g_ij;   d w_time[h][time bucket(i, j)] += g_ij   (rab_pt).
 * dq, dk, dv are [T, H, d] contiguous; dw_pos / dw_time have the tables' shapes (head stride
 * 0 = one table shared by the heads, which then sums over heads).  All outputs are
 * overwritten. */
void oracle_attention_bwd(int32_t B, int32_t H, int32_t dqk, int32_t dv, const int64_t* offsets,
                          const double* q, const double* k, const double* v, const double* dO,
                          int32_t bias_kind, const int64_t* ts, const double* w_pos,
                          int32_t num_pos, int64_t head_stride_pos, const double* w_time,
                          int32_t num_time, int64_t head_stride_time, const double* slopes,
                          double alpha, double out_scale, double* dq, double* dk, double* dvo,
                          double* dw_pos, double* dw_time) {
  oracle_bias bs = {bias_kind, ts, w_pos, w_time, num_pos, num_time,
                    head_stride_pos, head_stride_time, slopes};
  const int64_t T = offsets[B];
  for (int64_t t = 0; t < T * H * (int64_t)dqk; t++) dq[t] = dk[t] = 0.0;
  for (int64_t t = 0; t < T * H * (int64_t)dv; t++) dvo[t] = 0.0;
  const int rab = bias_kind == ORACLE_BIAS_RAB_PT;
  const int64_t np_tab = rab ? (head_stride_pos ? (int64_t)H * head_stride_pos : num_pos) : 0;
  const int64_t nt_tab = rab ? (head_stride_time ? (int64_t)H * head_stride_time : num_time) : 0;
  for (int64_t t = 0; t < np_tab; t++) dw_pos[t] = 0.0;
  for (int64_t t = 0; t < nt_tab; t++) dw_time[t] = 0.0;
  /* per-(user, head) partial table gradients, summed serially afterwards (no races) */
  int64_t n_items = (int64_t)B * H;
  int64_t per = rab ? (int64_t)num_pos + num_time : 0;
  double* part = per ? (double*)calloc((size_t)(n_items * per), sizeof(double)) : NULL;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t it = 0; it < n_items; it++) {
    int32_t b = (int32_t)(it / H), h = (int32_t)(it % H);
    int64_t base = offsets[b], n = offsets[b + 1] - offsets[b];
    for (int64_t i = 0; i < n; i++) {
      const double* qi = q + ((base + i) * H + h) * (int64_t)dqk;
      const double* doi = dO + ((base + i) * H + h) * (int64_t)dv;
      double* dqi = dq + ((base + i) * H + h) * (int64_t)dqk;
      for (int64_t j = 0; j <= i; j++) {
        const double* kj = k + ((base + j) * H + h) * (int64_t)dqk;
        const double* vj = v + ((base + j) * H + h) * (int64_t)dv;
        double s = 0.0, dov = 0.0;
        for (int c = 0; c < dqk; c++) s += qi[c] * kj[c];
        for (int c = 0; c < dv; c++) dov += doi[c] * vj[c];
        double x = alpha * s + bias_value(&bs, h, base, i, j);
        double sg = 1.0 / (1.0 + exp(-x));
        double a = x * sg;
        double g = out_scale * dov * sg * (1.0 + x * (1.0 - sg));
        double* dvj = dvo + ((base + j) * H + h) * (int64_t)dv;
        double* dkj = dk + ((base + j) * H + h) * (int64_t)dqk;
        /* dV_j and dK_j are shared by the rows i >= j of this (user, head) only */
        for (int c = 0; c < dv; c++) dvj[c] += out_scale * a * doi[c];
        for (int c = 0; c < dqk; c++) {
          dqi[c] += alpha * g * kj[c];
          dkj[c] += alpha * g * qi[c];
        }
        if (rab) {
          part[it * per + oracle_pos_bucket(i - j, num_pos)] += g;
          part[it * per + num_pos + oracle_time_bucket(ts[base + i] - ts[base + j], num_time)] += g;
        }
      }
    }
  }
  if (rab) {
    for (int64_t it = 0; it < n_items; it++) {
      int32_t h = (int32_t)(it % H);
      for (int p = 0; p < num_pos; p++) dw_pos[h * head_stride_pos + p] += part[it * per + p];
      for (int p = 0; p < num_time; p++)
        dw_time[h * head_stride_time + p] += part[it * per + num_pos + p];
    }
    free(part);
  }
}

/* Candidate scoring over a user history [AS §3.6 M-FALCON; GenRank part (2): the candidates of
 * one request share one position].  User b: history rows [hist_off[b], hist_off[b+1]) of
 * k_h, v_h with timestamps ts_h, positions 0 .. n_b - 1; candidate rows [cand_off[b],
 * cand_off[b+1]) of q_c, k_c, v_c with timestamps ts_c, every candidate at position n_b.
 * Candidate c attends to the whole history and to itself, to no other candidate:
 *   O[c] = out_scale * ( sum_{j < n_b} SiLU(alpha <q_c,k_j> + rab(n_b - j, t_c - t_j)) v_j
 *                        + SiLU(alpha <q_c,k_c> + rab(0, 0)) v_c ).
 * o is [Tc, H, dv]. */
static double cand_bias(const oracle_bias* bs, int h, int64_t pos_delta, int64_t dt) {
  if (bs->kind == ORACLE_BIAS_RAB_PT) {
    int32_t pb = oracle_pos_bucket(pos_delta, bs->num_pos);
    int32_t tb = oracle_time_bucket(dt, bs->num_time);
    return bs->w_pos[h * bs->head_stride_pos + pb] + bs->w_time[h * bs->head_stride_time + tb];
  }
  if (bs->kind == ORACLE_BIAS_ALIBI) return -bs->slopes[h] * (double)pos_delta;
  return 0.0;
}

void oracle_attention_candidates(int32_t B, int32_t H, int32_t dqk, int32_t dv,
                                 const int64_t* hist_off, const int64_t* cand_off,
                                 const double* q_c, const double* k_c, const double* v_c,
                                 const double* k_h, const double* v_h, int32_t bias_kind,
                                 const int64_t* ts_h, const int64_t* ts_c, const double* w_pos,
                                 int32_t num_pos, int64_t head_stride_pos, const double* w_time,
                                 int32_t num_time, int64_t head_stride_time,
                                 const double* slopes, double alpha, double out_scale,
                                 double* o) {
  oracle_bias bs = {bias_kind, ts_h, w_pos, w_time, num_pos, num_time,
                    head_stride_pos, head_stride_time, slopes};
  int64_t n_items = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t it = 0; it < n_items; it++) {
    int32_t b = (int32_t)(it / H), h = (int32_t)(it % H);
    int64_t hb = hist_off[b], n = hist_off[b + 1] - hist_off[b];
    for (int64_t c = cand_off[b]; c < cand_off[b + 1]; c++) {
      const double* qi = q_c + (c * H + h) * (int64_t)dqk;
      double* out = o + (c * H + h) * (int64_t)dv;
      for (int e = 0; e < dv; e++) out[e] = 0.0;
      for (int64_t j = 0; j <= n; j++) {  /* j == n: the candidate itself */
        const double* kj = j < n ? k_h + ((hb + j) * H + h) * (int64_t)dqk : k_c + (c * H + h) * (int64_t)dqk;
        const double* vj = j < n ? v_h + ((hb + j) * H + h) * (int64_t)dv : v_c + (c * H + h) * (int64_t)dv;
        double s = 0.0;
        for (int e = 0; e < dqk; e++) s += qi[e] * kj[e];
        int64_t dt = bias_kind == ORACLE_BIAS_RAB_PT ? ts_c[c] - (j < n ? ts_h[hb + j] : ts_c[c]) : 0;
        double a = silu(alpha * s + cand_bias(&bs, h, n - j, dt));
        for (int e = 0; e < dv; e++) out[e] += a * vj[e];
      }
      for (int e = 0; e < dv; e++) out[e] *= out_scale;
    }
  }
}

/* One HSTU layer [AS §3.1 eqs. (1)-(3)]:
 *   Z = SiLU(X W1^T + b1);  U | V | Q | K = column blocks of Z (widths H*dv, H*dv,
 *       H*dqk, H*dqk; head h owns columns [h*d, (h+1)*d) of each block);
 *   O = eq. (2) on Q, K, V;
 *   Y = (LayerNorm(O) * U) W2^T + b2   (+ X when residual != 0)
 * LayerNorm runs over the H*dv features of a token, biased variance, then
 * gamma/beta.  W1 is [2H(dqk+dv), D], W2 is [D, H*dv] (row = output feature).
 * z_out [T, 2H(dqk+dv)] and o_out [T, H*dv] are optional (may be NULL). */
void oracle_layer(int32_t B, int32_t D, int32_t H, int32_t dqk, int32_t dv, const int64_t* offsets,
                  const double* x, const double* w1, const double* b1, const double* gamma,
                  const double* beta, double ln_eps, const double* w2, const double* b2,
                  int32_t bias_kind, const int64_t* ts, const double* w_pos, int32_t num_pos,
                  int64_t head_stride_pos, const double* w_time, int32_t num_time,
                  int64_t head_stride_time, const double* slopes, double alpha, int32_t residual,
                  double* y, double* z_out, double* o_out) {
  int64_t T = offsets[B];
  int64_t N1 = 2LL * H * (dqk + dv);
  int64_t HV = (int64_t)H * dv;
  double* z = z_out ? z_out : (double*)malloc(sizeof(double) * (size_t)(T * N1 + 1));
  double* o = o_out ? o_out : (double*)malloc(sizeof(double) * (size_t)(T * HV + 1));

  /* eq. (1): pointwise projection with SiLU */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    for (int64_t n = 0; n < N1; n++) {
      double acc = b1[n];
      for (int64_t c = 0; c < D; c++) acc += x[t * D + c] * w1[n * D + c];
      z[t * N1 + n] = silu(acc);
    }
  }
  /* Split: U = cols [0, HV), V = [HV, 2HV), Q = [2HV, 2HV + H dqk), K = rest */
  const double* U = z;
  const double* V = z + HV;
  const double* Q = z + 2 * HV;
  const double* K = z + 2 * HV + (int64_t)H * dqk;

  /* eq. (2) */
  oracle_attention(B, H, dqk, dv, offsets, Q, N1, K, N1, V, N1, bias_kind, ts, w_pos, num_pos,
                   head_stride_pos, w_time, num_time, head_stride_time, slopes, alpha, 1.0, o);

  /* eq. (3) */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    const double* ot = o + t * HV;
    double mean = 0.0, var = 0.0;
    for (int64_t c = 0; c < HV; c++) mean += ot[c];
    mean /= (double)HV;
    for (int64_t c = 0; c < HV; c++) var += (ot[c] - mean) * (ot[c] - mean);
    var /= (double)HV;
    double rstd = 1.0 / sqrt(var + ln_eps);
    double* g = (double*)malloc(sizeof(double) * (size_t)HV);
    for (int64_t c = 0; c < HV; c++)
      g[c] = ((ot[c] - mean) * rstd * gamma[c] + beta[c]) * U[t * N1 + c];
    for (int64_t n = 0; n < D; n++) {
      double acc = b2[n];
      for (int64_t c = 0; c < HV; c++) acc += g[c] * w2[n * HV + c];
      if (residual) acc += x[t * D + n];
      y[t * D + n] = acc;
    }
    free(g);
  }
  if (!z_out) free(z);
  if (!o_out) free(o);
}

/* Threads the OpenMP loops above run with (reported beside timings). */
#ifdef _OPENMP
#include <omp.h>
int32_t oracle_num_threads(void) { return (int32_t)omp_get_max_threads(); }
#else
int32_t oracle_num_threads(void) { return 1; }
#endif
