/*
 * rattn_oracle.c -- plain fp64 CPU oracle for relative-bias grouped-query attention.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header or helper with the HIP library; it reads the same raw input bytes.
 *
 * What it computes (the plain definition, nothing blocked, fused or reordered):
 *
 *   vLLM recipes page "thinkingmachines/Inkling", Overview > Architectural highlights >
 *   Attention: grouped-query attention with head size 128; instead of RoPE the logits
 *   carry a trained bias that depends on the query-key distance; 11 full
 *   attention layers and 55 sliding-window layers.  The exact form of that term is fixed
 *   here as a per-query-head table r[h, d] indexed by the distance d = i - j and clamped
 *   at R-1:
 *
 *       logit[i, j] = (q_i . k_j) / sqrt(head_dim) + r[h, min(i - j, R - 1)]
 *
 *   Same page, Overview > MTP: up to 9 query tokens per step; Client Usage: paged KV
 *   cache with block size 128.
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *   - query t of a sequence with ctx keys sits at absolute position p = ctx - n_q + t
 *     (bottom-right alignment: the queries are the last n_q tokens, their own K/V are in
 *     the cache);
 *   - key j is visible iff 0 <= p - j, and additionally p - j <= W - 1 when W > 0
 *     (the window counts W keys including the query itself);
 *   - query head h reads KV head floor(h / (Hq / Hkv)) (contiguous groups);
 *   - the 1/sqrt(head_dim) scale applies to q.k only; the softmax is base e; LSE is the
 *     natural-log log-sum-exp of the logits.
 *
 * Per query row, two passes: first every visible logit and their maximum m, then
 * w_j = exp(s_j - m), Z = sum_j w_j, out = sum_j (w_j / Z) v_j, lse = m + log Z.
 * All arithmetic is double.  bf16 and fp32 inputs widen to double exactly.
 */
#include "rattn_oracle.h" /* include/rattn_oracle.h */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* widen n elements of a bf16 (bit pattern), fp32 or fp64 array to double */
static void widen(const void* src, size_t offset, int n, int dtype, double* dst) {
  int e;
  if (dtype == RATTN_ORACLE_BF16) {
    const uint16_t* s = (const uint16_t*)src + offset;
    for (e = 0; e < n; ++e) {
      uint32_t u = (uint32_t)s[e] << 16;
      float f;
      memcpy(&f, &u, sizeof f);
      dst[e] = (double)f;
    }
  } else if (dtype == RATTN_ORACLE_FP32) {
    const float* s = (const float*)src + offset;
    for (e = 0; e < n; ++e) dst[e] = (double)s[e];
  } else {
    const double* s = (const double*)src + offset;
    for (e = 0; e < n; ++e) dst[e] = s[e];
  }
}

/* element offset of row (b, j, kvh) of K or V, contiguous or paged */
static size_t kv_offset(const int* block_table, int b, int j, int kvh, int Lk_max, int Hkv,
                        int head_dim, int block_size, int max_blocks_per_seq) {
  if (block_table == NULL)
    return (((size_t)b * Lk_max + j) * Hkv + kvh) * head_dim;
  {
    int phys = block_table[(size_t)b * max_blocks_per_seq + j / block_size];
    return (((size_t)phys * block_size + j % block_size) * Hkv + kvh) * head_dim;
  }
}

/* bias_per_row = 0: bias is [Hq, R], the table of head h; 1: bias is [B, n_q, Hq, R], one
   table per query row (the row (b, t, h) reads its own R entries) */
static int ref_forward(const void* q, const void* k, const void* v, const int* block_table,
                       const int* ctx_lens, const int* windows, const double* bias, int bias_per_row,
                       double* out, double* lse, double* probs, int B, int n_q, int Lk_max, int Hq,
                       int Hkv, int head_dim, int block_size, int R, int max_blocks_per_seq, int dtype,
                       int num_threads) {
  long long rows, row;
  int b;
  int bad = 0;
  if (q == NULL || k == NULL || v == NULL || ctx_lens == NULL || bias == NULL || out == NULL)
    return 1;
  if (B < 0 || n_q < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || head_dim < 1 || R < 1)
    return 1;
  if (dtype != RATTN_ORACLE_BF16 && dtype != RATTN_ORACLE_FP32 && dtype != RATTN_ORACLE_FP64)
    return 1;
  if (block_table != NULL && (block_size < 1 || max_blocks_per_seq < 1)) return 1;
  for (b = 0; b < B; ++b) {
    if (ctx_lens[b] < n_q) bad = 1;
    if (block_table == NULL && ctx_lens[b] > Lk_max) bad = 1;
    if (block_table != NULL && ctx_lens[b] > (long long)max_blocks_per_seq * block_size) bad = 1;
    if (probs != NULL && ctx_lens[b] > Lk_max) bad = 1;
  }
  if (bad) return 1;

  rows = (long long)B * n_q * Hq;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif

#pragma omp parallel
  {
    double* qrow = (double*)malloc(sizeof(double) * head_dim);
    double* krow = (double*)malloc(sizeof(double) * head_dim);
    double* acc = (double*)malloc(sizeof(double) * head_dim);
    double* s = NULL;
    size_t s_cap = 0;

#pragma omp for schedule(dynamic, 1)
    for (row = 0; row < rows; ++row) {
      const int h = (int)(row % Hq);
      const int t = (int)((row / Hq) % n_q);
      const int bb = (int)(row / ((long long)Hq * n_q));
      const int group = Hq / Hkv;
      const int kvh = h / group;
      const int ctx = ctx_lens[bb];
      const int p = ctx - n_q + t;                       /* absolute query position */
      const int W = windows ? windows[bb] : 0;
      const int lo = (W > 0 && p - W + 1 > 0) ? p - W + 1 : 0;
      const int hi = p;                                  /* causal: keys 0..p */
      const double scale = 1.0 / sqrt((double)head_dim);
      const double* r = bias + (size_t)(bias_per_row ? row : h) * R;
      double m = -INFINITY, Z = 0.0;
      int j, e;
      const size_t orow = (size_t)row * head_dim;

      if ((size_t)(hi - lo + 1) > s_cap) {
        s_cap = (size_t)(hi - lo + 1);
        free(s);
        s = (double*)malloc(sizeof(double) * s_cap);
      }
      widen(q, (((size_t)bb * n_q + t) * Hq + h) * head_dim, head_dim, dtype, qrow);

      /* pass 1: logits of the visible keys and their maximum */
      for (j = lo; j <= hi; ++j) {
        double dot = 0.0;
        int dist = p - j;
        widen(k, kv_offset(block_table, bb, j, kvh, Lk_max, Hkv, head_dim, block_size,
                           max_blocks_per_seq), head_dim, dtype, krow);
        for (e = 0; e < head_dim; ++e) dot += qrow[e] * krow[e];
        s[j - lo] = dot * scale + r[dist < R - 1 ? dist : R - 1];
        if (s[j - lo] > m) m = s[j - lo];
      }

      /* pass 2: weights, normaliser and the weighted sum of V rows */
      for (e = 0; e < head_dim; ++e) acc[e] = 0.0;
      for (j = lo; j <= hi; ++j) {
        double w = exp(s[j - lo] - m);
        Z += w;
        widen(v, kv_offset(block_table, bb, j, kvh, Lk_max, Hkv, head_dim, block_size,
                           max_blocks_per_seq), head_dim, dtype, krow);
        for (e = 0; e < head_dim; ++e) acc[e] += w * krow[e];
      }
      for (e = 0; e < head_dim; ++e) out[orow + e] = acc[e] / Z;
      if (lse != NULL) lse[row] = m + log(Z);
      if (probs != NULL) {
        double* pr = probs + (size_t)row * Lk_max;
        for (j = 0; j < Lk_max; ++j) pr[j] = 0.0;
        for (j = lo; j <= hi; ++j) pr[j] = exp(s[j - lo] - m) / Z;
      }
    }
    free(qrow);
    free(krow);
    free(acc);
    free(s);
  }
  return 0;
}

int rattn_ref_cpu(const void* q, const void* k, const void* v, const int* block_table,
                  const int* ctx_lens, const int* windows, const double* bias, double* out,
                  double* lse, double* probs, int B, int n_q, int Lk_max, int Hq, int Hkv,
                  int head_dim, int block_size, int R, int max_blocks_per_seq, int dtype,
                  int num_threads) {
  return ref_forward(q, k, v, block_table, ctx_lens, windows, bias, 0, out, lse, probs, B, n_q, Lk_max, Hq,
                     Hkv, head_dim, block_size, R, max_blocks_per_seq, dtype, num_threads);
}

int rattn_ref_cpu_tokbias(const void* q, const void* k, const void* v, const int* block_table,
                          const int* ctx_lens, const int* windows, const double* bias,
                          double* out, double* lse, double* probs, int B, int n_q, int Lk_max,
                          int Hq, int Hkv, int head_dim, int block_size, int R,
                          int max_blocks_per_seq, int dtype, int num_threads) {
  return ref_forward(q, k, v, block_table, ctx_lens, windows, bias, 1, out, lse, probs, B, n_q, Lk_max, Hq,
                     Hkv, head_dim, block_size, R, max_blocks_per_seq, dtype, num_threads);
}

int rattn_oracle_version(void) { return 2; }

