/*
 * msa_oracle.c -- plain, slow, fp64 CPU reference of the MiniMax Sparse
 * Attention (MSA) forward pass.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library.  It shares no code with the
 * HIP path and the HIP path never calls it.
 *
 * What it follows (all on the page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出
 * MiniMax-M3 模型", the MarkTechPost repost):
 *   - section 什么是 MSA ("what is MSA"): blocks of Bk tokens, k blocks kept per
 *     query and GQA group, a fixed budget of k*Bk key/value tokens;
 *   - section 两个分支如何工作 ("how the two branches work"): one index-query
 *     head per group against one shared index-key head, scores over the visible
 *     keys, max-pooled to blocks; top-k per query and group with the query's own
 *     (local) block always included; the main branch gathers the causally
 *     visible tokens of the chosen blocks and runs scaled dot-product softmax
 *     per query head;
 *   - section 内核协同设计 ("kernel co-design"): softmax keeps the order, so the
 *     top-k is taken on raw scores (no max/exp/sum).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   R1 index score = raw dot product (no scale, activation or bias);
 *   R2 key j is visible to the query at position p iff j <= p;
 *   R4 a block's pooled score is the max over its visible tokens only; blocks
 *      after the local block are not candidates;
 *   R5 the local block takes one of the k slots: S = {l} U top_(k-1) of the
 *      other visible blocks;
 *   R6 with at most k visible blocks, all are selected; unused slots are -1;
 *   R7 equal pooled scores: the lower block index wins (-0 equals +0);
 *   R8 the selected indices are emitted in ascending order;
 *   R13 FP8 index inputs are OCP E4M3 (see oracle_pool_f8);
 *   R14 the KL student is the softmax of the raw index scores over the
 *       teacher's token set (see oracle_kl).
 *
 * Every function works on a batch of independent "rows" (one query position of
 * one sequence and one GQA group); the caller slices the tensors.  bf16 inputs
 * are passed as their 16-bit patterns and widened exactly to double.
 * Return value: 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * Index branch, scores and block max-pool.
 *   iq     [nrows][d_idx]  index query of each row (its group's head)
 *   pos    [nrows]         position p of each row's query, 0 <= p < n_kv
 *   ik     [n_kv][d_idx]   the shared index-key head of the row's sequence
 *   pooled [nrows][ld]     out: pooled[r][t] for t = 0 .. floor(p/bk);
 *                          entries after the local block are left untouched.
 * pooled[r][t] = max over j in block t with j <= p of sum_c iq[r][c]*ik[j][c].
 */
int oracle_pool(const uint16_t* iq, int64_t nrows, const int64_t* pos, const uint16_t* ik,
                int64_t n_kv, int32_t d_idx, int32_t bk, double* pooled, int64_t ld) {
  if (nrows < 0 || d_idx <= 0 || bk <= 0 || ld < (n_kv + bk - 1) / bk) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] >= n_kv) return -1;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t p = pos[r];
    const int64_t local = p / bk;
    for (int64_t t = 0; t <= local; ++t) {
      const int64_t j_end = (t + 1) * bk < p + 1 ? (t + 1) * bk : p + 1;
      double best = -INFINITY;
      for (int64_t j = t * bk; j < j_end; ++j) {
        double s = 0.0;
        for (int32_t c = 0; c < d_idx; ++c) s += bf(iq[r * d_idx + c]) * bf(ik[j * d_idx + c]);
        if (s > best) best = s;
      }
      pooled[r * ld + t] = best;
    }
  }
  return 0;
}

/*
 * FP8 index inputs.  The released kernels take FP8 as well as BF16 (page
 * "MiniMax lança MSA…", section "Kernel open source e MiniMax-M3"; page
 * "MiniMax 发布 MSA…", section 内核协同设计, the paragraph on the open-source
 * kernel).  The pages do not name the 8-bit format; the reading taken (R13) is
 * OCP E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, NaN only for exponent and mantissa all ones, largest finite
 * value 448; exponent field 0 holds the subnormals m/8 * 2^-6.
 */
static double e4m3(uint8_t c) {
  const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m, -9)          /* (m/8) * 2^(1-7) */
                            : ldexp(8.0 + (double)m, e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

/* Decode n E4M3 codes (exposed so that the decoder can be pinned on its own). */
int oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
  if (n < 0) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3(codes[i]);
  return 0;
}

/*
 * The index scores and block max-pool of oracle_pool with E4M3 index inputs:
 * the same definition on the decoded values (R1: raw dot product, no scale).
 *   iq [nrows][d_idx] and ik [n_kv][d_idx] are E4M3 codes; the rest as above.
 */
int oracle_pool_f8(const uint8_t* iq, int64_t nrows, const int64_t* pos, const uint8_t* ik,
                   int64_t n_kv, int32_t d_idx, int32_t bk, double* pooled, int64_t ld) {
  if (nrows < 0 || d_idx <= 0 || bk <= 0 || ld < (n_kv + bk - 1) / bk) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] >= n_kv) return -1;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t p = pos[r];
    const int64_t local = p / bk;
    for (int64_t t = 0; t <= local; ++t) {
      const int64_t j_end = (t + 1) * bk < p + 1 ? (t + 1) * bk : p + 1;
      double best = -INFINITY;
      for (int64_t j = t * bk; j < j_end; ++j) {
        double s = 0.0;
        for (int32_t c = 0; c < d_idx; ++c) s += e4m3(iq[r * d_idx + c]) * e4m3(ik[j * d_idx + c]);
        if (s > best) best = s;
      }
      pooled[r * ld + t] = best;
    }
  }
  return 0;
}

typedef struct {
  double score;
  int32_t block;
} cand_t;

/* Larger score first; among equal scores the lower block index first. */
static int cand_order(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->block > y->block) - (x->block < y->block);
}

static int int_order(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * Index branch, block top-k with the forced local block (exp-free: the raw
 * pooled scores are ranked directly).
 *   pooled [nrows][ld], pos [nrows] as above
 *   sel    [nrows][k]  out: ascending block ids, the local block included,
 *                      padded with -1 when fewer than k blocks are visible.
 */
int oracle_select(const double* pooled, int64_t ld, int64_t nrows, const int64_t* pos, int32_t bk,
                  int32_t k, int32_t* sel) {
  if (nrows < 0 || bk <= 0 || k < 1) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] / bk >= ld) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < nrows; ++r) {
    const int32_t local = (int32_t)(pos[r] / bk);
    int32_t* out = sel + r * k;
    int32_t n = 0;
    if (local + 1 <= k) {
      for (int32_t t = 0; t <= local; ++t) out[n++] = t;
    } else {
      cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)local);
      for (int32_t t = 0; t < local; ++t) {
        c[t].score = pooled[r * ld + t];
        c[t].block = t;
      }
      qsort(c, (size_t)local, sizeof(cand_t), cand_order);
      for (int32_t s = 0; s < k - 1; ++s) out[n++] = c[s].block;
      out[n++] = local;
      free(c);
      qsort(out, (size_t)n, sizeof(int32_t), int_order);
    }
    for (int32_t s = n; s < k; ++s) out[s] = -1;
  }
  return 0;
}

/*
 * Main branch: exact softmax attention of each query head over the causally
 * visible tokens of the row's selected blocks.
 *   q    [nrows][G][d]  the G query heads of the row's group
 *   sel  [nrows][k]     block ids (-1 = unused; duplicates count once)
 *   K, V [n_kv][d]      the row's KV head
 *   out  [nrows][G][d], lse [nrows][G] (natural log of the softmax denominator)
 * T = { j : floor(j/bk) in sel, j <= p, j < n_kv };
 * z_j = scale * q.k_j;  out = sum_j e^(z_j - m) v_j / sum_j e^(z_j - m);
 * lse = m + ln(sum_j e^(z_j - m)), m = max_j z_j.
 */
int oracle_attend(const uint16_t* q, int64_t nrows, const int64_t* pos, const int32_t* sel, int32_t k,
                  int32_t G, const uint16_t* K, const uint16_t* V, int64_t n_kv, int32_t d, int32_t bk,
                  double scale, double* out, double* lse) {
  if (nrows < 0 || k < 1 || G < 1 || d <= 0 || bk <= 0) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] >= n_kv) return -1;
  const int64_t n_blk = (n_kv + bk - 1) / bk;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t p = pos[r];
    int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    memcpy(blocks, sel + r * k, sizeof(int32_t) * (size_t)k);
    qsort(blocks, (size_t)k, sizeof(int32_t), int_order);
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)k * (size_t)bk);
    int64_t nt = 0;
    for (int32_t s = 0; s < k; ++s) {
      const int32_t t = blocks[s];
      if (t < 0 || t >= n_blk || (s > 0 && t == blocks[s - 1])) continue;
      for (int64_t j = (int64_t)t * bk; j < ((int64_t)t + 1) * bk && j < n_kv && j <= p; ++j) tok[nt++] = j;
    }
    double* z = (double*)malloc(sizeof(double) * (size_t)(nt > 0 ? nt : 1));
    for (int32_t h = 0; h < G; ++h) {
      const uint16_t* qh = q + (r * G + h) * d;
      double* oh = out + (r * G + h) * d;
      double m = -INFINITY;
      for (int64_t a = 0; a < nt; ++a) {
        double s = 0.0;
        for (int32_t c = 0; c < d; ++c) s += bf(qh[c]) * bf(K[tok[a] * d + c]);
        z[a] = scale * s;
        if (z[a] > m) m = z[a];
      }
      double l = 0.0;
      for (int32_t c = 0; c < d; ++c) oh[c] = 0.0;
      for (int64_t a = 0; a < nt; ++a) {
        const double w = exp(z[a] - m);
        l += w;
        for (int32_t c = 0; c < d; ++c) oh[c] += w * bf(V[tok[a] * d + c]);
      }
      for (int32_t c = 0; c < d; ++c) oh[c] /= l;
      lse[r * G + h] = m + log(l);
    }
    free(z);
    free(tok);
    free(blocks);
  }
  return 0;
}

/*
 * KL alignment of the Index Branch to the Main Branch, the training signal of
 * the index projections (page "MiniMax 发布 MSA…", section MSA 如何训练: the
 * loss matches the Index Branch's distribution to the Main Branch's attention,
 * the teacher being the Main Branch's distribution over the selected tokens
 * averaged over the group's heads; page "MiniMax lança MSA…", section
 * "Treinamento com KL Divergence").  Per row, over T (the visible tokens of the
 * selected blocks, as in oracle_attend):
 *   teacher  p_j = (1/G) sum_h softmax_j(scale * q_h . k_j),
 *   student  s_j = softmax_j(iq . ik_j)            (R14: raw index scores, R1),
 *   kl = sum_j p_j ln(p_j / s_j),  terms with p_j = 0 contribute 0.
 *   q [nrows][G][d], iq [nrows][d_idx], pos [nrows], sel [nrows][k];
 *   K [n_kv][d], ik [n_kv][d_idx]  ->  kl [nrows]
 */
int oracle_kl(const uint16_t* q, int64_t nrows, const int64_t* pos, const int32_t* sel, int32_t k, int32_t G,
              const uint16_t* K, int64_t n_kv, int32_t d, const uint16_t* iq, const uint16_t* ik, int32_t d_idx,
              int32_t bk, double scale, double* kl) {
  if (nrows < 0 || k < 1 || G < 1 || d <= 0 || d_idx <= 0 || bk <= 0) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] >= n_kv) return -1;
  const int64_t n_blk = (n_kv + bk - 1) / bk;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t p = pos[r];
    int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    memcpy(blocks, sel + r * k, sizeof(int32_t) * (size_t)k);
    qsort(blocks, (size_t)k, sizeof(int32_t), int_order);
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)k * (size_t)bk);
    int64_t nt = 0;
    for (int32_t s = 0; s < k; ++s) {
      const int32_t t = blocks[s];
      if (t < 0 || t >= n_blk || (s > 0 && t == blocks[s - 1])) continue;
      for (int64_t j = (int64_t)t * bk; j < ((int64_t)t + 1) * bk && j < n_kv && j <= p; ++j) tok[nt++] = j;
    }
    const size_t n = (size_t)(nt > 0 ? nt : 1);
    double* teach = (double*)calloc(n, sizeof(double));
    double* w = (double*)malloc(sizeof(double) * n);
    /* teacher: each head's softmax over T, averaged over the group */
    for (int32_t h = 0; h < G; ++h) {
      const uint16_t* qh = q + (r * G + h) * d;
      double m = -INFINITY;
      for (int64_t a = 0; a < nt; ++a) {
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) dot += bf(qh[c]) * bf(K[tok[a] * d + c]);
        w[a] = scale * dot;
        if (w[a] > m) m = w[a];
      }
      double l = 0.0;
      for (int64_t a = 0; a < nt; ++a) l += exp(w[a] - m);
      for (int64_t a = 0; a < nt; ++a) teach[a] += exp(w[a] - m) / l / G;
    }
    /* student: softmax of the raw index scores over the same tokens */
    double m = -INFINITY;
    for (int64_t a = 0; a < nt; ++a) {
      double dot = 0.0;
      for (int32_t c = 0; c < d_idx; ++c) dot += bf(iq[r * d_idx + c]) * bf(ik[tok[a] * d_idx + c]);
      w[a] = dot;
      if (w[a] > m) m = w[a];
    }
    double l = 0.0;
    for (int64_t a = 0; a < nt; ++a) l += exp(w[a] - m);
    const double log_norm = m + log(l);
    double acc = 0.0;
    for (int64_t a = 0; a < nt; ++a)
      if (teach[a] > 0.0) acc += teach[a] * (log(teach[a]) - (w[a] - log_norm));
    kl[r] = acc;
    free(w);
    free(teach);
    free(tok);
    free(blocks);
  }
  return 0;
}

/*
 * The teacher of oracle_kl on its own (the distribution the KL backward
 * holds fixed): teach[r][j] = (1/G) sum_h softmax_j(scale * q_h . k_j) for j
 * in T, 0 for every other key.  Rows as in oracle_kl -> teach [nrows][n_kv].
 */
int oracle_kl_teacher(const uint16_t* q, int64_t nrows, const int64_t* pos, const int32_t* sel, int32_t k, int32_t G,
                      const uint16_t* K, int64_t n_kv, int32_t d, int32_t bk, double scale, double* teach) {
  if (nrows < 0 || k < 1 || G < 1 || d <= 0 || bk <= 0) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] >= n_kv) return -1;
  const int64_t n_blk = (n_kv + bk - 1) / bk;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t p = pos[r];
    double* tr = teach + r * n_kv;
    for (int64_t j = 0; j < n_kv; ++j) tr[j] = 0.0;
    int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    memcpy(blocks, sel + r * k, sizeof(int32_t) * (size_t)k);
    qsort(blocks, (size_t)k, sizeof(int32_t), int_order);
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)k * (size_t)bk);
    int64_t nt = 0;
    for (int32_t s = 0; s < k; ++s) {
      const int32_t t = blocks[s];
      if (t < 0 || t >= n_blk || (s > 0 && t == blocks[s - 1])) continue;
      for (int64_t j = (int64_t)t * bk; j < ((int64_t)t + 1) * bk && j < n_kv && j <= p; ++j) tok[nt++] = j;
    }
    double* w = (double*)malloc(sizeof(double) * (size_t)(nt > 0 ? nt : 1));
    for (int32_t h = 0; h < G; ++h) {
      const uint16_t* qh = q + (r * G + h) * d;
      double m = -INFINITY;
      for (int64_t a = 0; a < nt; ++a) {
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) dot += bf(qh[c]) * bf(K[tok[a] * d + c]);
        w[a] = scale * dot;
        if (w[a] > m) m = w[a];
      }
      double l = 0.0;
      for (int64_t a = 0; a < nt; ++a) l += exp(w[a] - m);
      for (int64_t a = 0; a < nt; ++a) tr[tok[a]] += exp(w[a] - m) / l / G;
    }
    free(w);
    free(tok);
    free(blocks);
  }
  return 0;
}

/*
 * Gradient of the KL alignment term with respect to the index projections'
 * outputs, the teacher held fixed (page "MiniMax 发布 MSA…", section MSA 如何训练:
 * gradient detach stops the KL gradient at the Index Branch's inputs, so it
 * trains only the index projections; the teacher comes from the Main Branch).
 * With z_j = iq . ik_j, student s_j = softmax_j(z_j) and teacher t_j over T
 * as in oracle_kl, d kl / d z_j = s_j - t_j, so for a row weight w (the
 * gradient of the loss with respect to the row's kl):
 *   d_iq = w sum_j (s_j - t_j) ik_j,   d_ik_j += w (s_j - t_j) iq.
 *   rows as in oracle_kl; w [nrows] -> d_iq [nrows][d_idx];
 *   d_ik [n_kv][d_idx] accumulated over every row (the caller zeroes it).
 */
int oracle_kl_bwd(const uint16_t* q, int64_t nrows, const int64_t* pos, const int32_t* sel, int32_t k, int32_t G,
                  const uint16_t* K, int64_t n_kv, int32_t d, const uint16_t* iq, const uint16_t* ik, int32_t d_idx,
                  int32_t bk, double scale, const double* w, double* d_iq, double* d_ik) {
  if (nrows < 0 || k < 1 || G < 1 || d <= 0 || d_idx <= 0 || bk <= 0) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] >= n_kv) return -1;
  const int64_t n_blk = (n_kv + bk - 1) / bk;
  int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)k * (size_t)bk);
  const size_t cap = (size_t)k * (size_t)bk;
  double* teach = (double*)malloc(sizeof(double) * cap);
  double* zz = (double*)malloc(sizeof(double) * cap);
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t p = pos[r];
    memcpy(blocks, sel + r * k, sizeof(int32_t) * (size_t)k);
    qsort(blocks, (size_t)k, sizeof(int32_t), int_order);
    int64_t nt = 0;
    for (int32_t s = 0; s < k; ++s) {
      const int32_t t = blocks[s];
      if (t < 0 || t >= n_blk || (s > 0 && t == blocks[s - 1])) continue;
      for (int64_t j = (int64_t)t * bk; j < ((int64_t)t + 1) * bk && j < n_kv && j <= p; ++j) tok[nt++] = j;
    }
    /* teacher */
    for (int64_t a = 0; a < nt; ++a) teach[a] = 0.0;
    for (int32_t h = 0; h < G; ++h) {
      const uint16_t* qh = q + (r * G + h) * d;
      double m = -INFINITY;
      for (int64_t a = 0; a < nt; ++a) {
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) dot += bf(qh[c]) * bf(K[tok[a] * d + c]);
        zz[a] = scale * dot;
        if (zz[a] > m) m = zz[a];
      }
      double l = 0.0;
      for (int64_t a = 0; a < nt; ++a) l += exp(zz[a] - m);
      for (int64_t a = 0; a < nt; ++a) teach[a] += exp(zz[a] - m) / l / G;
    }
    /* student and the gradient */
    double m = -INFINITY;
    for (int64_t a = 0; a < nt; ++a) {
      double dot = 0.0;
      for (int32_t c = 0; c < d_idx; ++c) dot += bf(iq[r * d_idx + c]) * bf(ik[tok[a] * d_idx + c]);
      zz[a] = dot;
      if (dot > m) m = dot;
    }
    double l = 0.0;
    for (int64_t a = 0; a < nt; ++a) l += exp(zz[a] - m);
    for (int32_t c = 0; c < d_idx; ++c) d_iq[r * d_idx + c] = 0.0;
    for (int64_t a = 0; a < nt; ++a) {
      const double gz = w[r] * (exp(zz[a] - m) / l - teach[a]);
      for (int32_t c = 0; c < d_idx; ++c) {
        d_iq[r * d_idx + c] += gz * bf(ik[tok[a] * d_idx + c]);
        d_ik[tok[a] * d_idx + c] += gz * bf(iq[r * d_idx + c]);
      }
    }
  }
  free(zz);
  free(teach);
  free(tok);
  free(blocks);
  return 0;
}

/*
 * Gradient of the Main Branch (the backward pass of oracle_attend), from the
 * definition of softmax attention over the row's token set T:
 *   P_hj = softmax_j(scale q_h . k_j),  o_h = sum_j P_hj v_j,
 *   given dO_h:  dv_j += P_hj dO_h,
 *                dP_hj = dO_h . v_j,  dS_hj = P_hj (dP_hj - dO_h . o_h),
 *                dq_h  = scale sum_j dS_hj k_j,   dk_j += scale dS_hj q_h.
 *   q, dO [nrows][G][d]; pos, sel [nrows][k] as in oracle_attend;
 *   K, V [n_kv][d] -> dQ [nrows][G][d]; dK, dV [n_kv][d] accumulated over every
 *   row and head of the call (the caller zeroes them).  Rows run one after the
 *   other (dK, dV are shared).
 */
int oracle_attend_bwd(const uint16_t* q, int64_t nrows, const int64_t* pos, const int32_t* sel, int32_t k,
                      int32_t G, const uint16_t* K, const uint16_t* V, int64_t n_kv, int32_t d, int32_t bk,
                      double scale, const uint16_t* dO, double* dQ, double* dK, double* dV) {
  if (nrows < 0 || k < 1 || G < 1 || d <= 0 || bk <= 0) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] >= n_kv) return -1;
  const int64_t n_blk = (n_kv + bk - 1) / bk;
  int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)k * (size_t)bk);
  double* P = (double*)malloc(sizeof(double) * (size_t)k * (size_t)bk);
  double* o = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t p = pos[r];
    memcpy(blocks, sel + r * k, sizeof(int32_t) * (size_t)k);
    qsort(blocks, (size_t)k, sizeof(int32_t), int_order);
    int64_t nt = 0;
    for (int32_t s = 0; s < k; ++s) {
      const int32_t t = blocks[s];
      if (t < 0 || t >= n_blk || (s > 0 && t == blocks[s - 1])) continue;
      for (int64_t j = (int64_t)t * bk; j < ((int64_t)t + 1) * bk && j < n_kv && j <= p; ++j) tok[nt++] = j;
    }
    for (int32_t h = 0; h < G; ++h) {
      const uint16_t* qh = q + (r * G + h) * d;
      const uint16_t* gh = dO + (r * G + h) * d;
      double* dqh = dQ + (r * G + h) * d;
      /* probabilities and the output of this head */
      double m = -INFINITY;
      for (int64_t a = 0; a < nt; ++a) {
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) dot += bf(qh[c]) * bf(K[tok[a] * d + c]);
        P[a] = scale * dot;
        if (P[a] > m) m = P[a];
      }
      double l = 0.0;
      for (int64_t a = 0; a < nt; ++a) {
        P[a] = exp(P[a] - m);
        l += P[a];
      }
      for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
      for (int64_t a = 0; a < nt; ++a) {
        P[a] /= l;
        for (int32_t c = 0; c < d; ++c) o[c] += P[a] * bf(V[tok[a] * d + c]);
      }
      double delta = 0.0; /* dO_h . o_h */
      for (int32_t c = 0; c < d; ++c) delta += bf(gh[c]) * o[c];
      for (int32_t c = 0; c < d; ++c) dqh[c] = 0.0;
      for (int64_t a = 0; a < nt; ++a) {
        const int64_t j = tok[a];
        double dp = 0.0;
        for (int32_t c = 0; c < d; ++c) dp += bf(gh[c]) * bf(V[j * d + c]);
        const double ds = P[a] * (dp - delta);
        for (int32_t c = 0; c < d; ++c) {
          dV[j * d + c] += P[a] * bf(gh[c]);
          dqh[c] += scale * ds * bf(K[j * d + c]);
          dK[j * d + c] += scale * ds * bf(qh[c]);
        }
      }
    }
  }
  free(o);
  free(P);
  free(tok);
  free(blocks);
  return 0;
}

/*
 * Dense causal GQA softmax attention (every key j <= p), written separately
 * from oracle_attend; with k*Bk >= n_kv the sparse result must equal it.
 */
int oracle_dense_gqa(const uint16_t* q, int64_t nrows, const int64_t* pos, int32_t G, const uint16_t* K,
                     const uint16_t* V, int64_t n_kv, int32_t d, double scale, double* out, double* lse) {
  if (nrows < 0 || G < 1 || d <= 0) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (pos[r] < 0 || pos[r] >= n_kv) return -1;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t p = pos[r];
    double* w = (double*)malloc(sizeof(double) * (size_t)(p + 1));
    for (int32_t h = 0; h < G; ++h) {
      const uint16_t* qh = q + (r * G + h) * d;
      double zmax = -INFINITY;
      for (int64_t j = 0; j <= p; ++j) {
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) dot += bf(qh[c]) * bf(K[j * d + c]);
        w[j] = dot * scale;
        zmax = w[j] > zmax ? w[j] : zmax;
      }
      double den = 0.0;
      for (int64_t j = 0; j <= p; ++j) {
        w[j] = exp(w[j] - zmax);
        den += w[j];
      }
      for (int32_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j <= p; ++j) acc += w[j] * bf(V[j * d + c]);
        out[(r * G + h) * d + c] = acc / den;
      }
      lse[r * G + h] = zmax + log(den);
    }
    free(w);
  }
  return 0;
}

/*
 * Merge of partial attention results over disjoint token sets (the merge
 * stage of the two-stage forward on the same page, section 内核协同设计):
 *   LSE = ln sum_s e^(lse_s);   o = sum_s e^(lse_s - LSE) o_s.
 * Parts with lse_s = -inf (empty sets) contribute nothing.
 *   o_parts [nrows][nparts][d], lse_parts [nrows][nparts] -> o [nrows][d], lse [nrows]
 */
int oracle_merge(const double* o_parts, const double* lse_parts, int64_t nrows, int32_t nparts, int32_t d,
                 double* o, double* lse) {
  if (nrows < 0 || nparts < 1 || d <= 0) return -1;
  for (int64_t r = 0; r < nrows; ++r) {
    const double* ls = lse_parts + r * nparts;
    double m = -INFINITY;
    for (int32_t s = 0; s < nparts; ++s) m = ls[s] > m ? ls[s] : m;
    double sum = 0.0;
    for (int32_t s = 0; s < nparts; ++s)
      if (ls[s] > -INFINITY) sum += exp(ls[s] - m);
    const double total = m + log(sum);
    for (int32_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int32_t s = 0; s < nparts; ++s)
        if (ls[s] > -INFINITY) acc += exp(ls[s] - total) * o_parts[(r * nparts + s) * d + c];
      o[r * d + c] = acc;
    }
    lse[r] = total;
  }
  return 0;
}
