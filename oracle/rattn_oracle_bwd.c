/*
 * rattn_oracle_bwd.c -- plain fp64 CPU oracle of the backward pass of relative-bias
 * grouped-query attention (gradients of the forward pass in rattn_oracle.c).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite and the benchmark may load
 * this library.  It shares no source, header or helper with the HIP library.
 *
 * vLLM recipes page "thinkingmachines/Inkling", Overview > Architectural highlights >
 * Attention defines the forward pass (GQA, head size 128, a trained bias on the logits that
 * depends on the query-key distance, in place of RoPE; the term fixed as
 * r[h, min(i - j, R - 1)]); the page lists training and LoRA among the model's uses.
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

/*
 * Backward pass (test infrastructure, like the forward above).
 *
 * The forward pass is the definition above; the gradients are its plain chain rule for an
 * output gradient dout (the recipes page lists training and LoRA among the model's uses and
 * prints no gradient formulas):
 *     P_j = softmax_j(s_j),  dP_j = dout . v_j,  D = sum_j P_j dP_j,  dS_j = P_j (dP_j - D),
 *     dq = sum_j dS_j k_j / sqrt(d),  dk_j += dS_j q / sqrt(d),  dv_j += P_j dout,
 *     dbias[h, min(p - j, R - 1)] += dS_j,
 * one query row at a time, over its visible keys, in double.  Each query head accumulates
 * into its own dk, dv buffers (heads run in parallel); the heads of a KV head are summed
 * afterwards in head order.  With a forward output `out` given, D is instead
 * sum_e dout_e out_e, the row sum the backward kernels take from the forward's output.
 * The magnitude sums take every term by absolute value, with dS replaced by
 *     P_j (|dP_j - D| + w (a_j + D_abs)),   a_j = sum_e |dout_e v_j,e| (dP_j's terms),
 * D_abs the size of D's terms (sum_j P_j a_j, or sum_e |dout_e out_e| with `out`).
 */
int rattn_ref_cpu_backward(const void* q, const void* k, const void* v, const void* dout,
                           const void* out, const double* bias, double* dq, double* dk, double* dv,
                           double* dbias, double* dq_abs, double* dk_abs, double* dv_abs,
                           double* dbias_abs, double abs_weight, int B, int Lq, int Lk, int Hq,
                           int Hkv, int head_dim, int R, int window, int dtype, int num_threads) {
  const int want_abs = dq_abs != NULL && dk_abs != NULL && dv_abs != NULL && dbias_abs != NULL;
  const size_t kv_elems = (size_t)B * Lk * Hkv * head_dim;
  const size_t head_kv = (size_t)B * Lk * head_dim; /* one query head's dk (or dv) buffer */
  double *dk_h, *dv_h, *dka_h = NULL, *dva_h = NULL;
  int h, g;
  size_t x;
  if (q == NULL || k == NULL || v == NULL || dout == NULL || bias == NULL || dq == NULL || dk == NULL ||
      dv == NULL || dbias == NULL)
    return 1;
  if (B < 0 || Lq < 0 || Lk < Lq || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || head_dim < 1 || R < 1) return 1;
  if (dtype != RATTN_ORACLE_BF16 && dtype != RATTN_ORACLE_FP32 && dtype != RATTN_ORACLE_FP64) return 1;
  dk_h = (double*)calloc((size_t)Hq * head_kv + 1, sizeof(double));
  dv_h = (double*)calloc((size_t)Hq * head_kv + 1, sizeof(double));
  if (want_abs) {
    dka_h = (double*)calloc((size_t)Hq * head_kv + 1, sizeof(double));
    dva_h = (double*)calloc((size_t)Hq * head_kv + 1, sizeof(double));
  }
  if (dk_h == NULL || dv_h == NULL || (want_abs && (dka_h == NULL || dva_h == NULL))) {
    free(dk_h);
    free(dv_h);
    free(dka_h);
    free(dva_h);
    return 1;
  }
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif

#pragma omp parallel
  {
    const double scale = 1.0 / sqrt((double)head_dim);
    double* qrow = (double*)malloc(sizeof(double) * head_dim);
    double* grow = (double*)malloc(sizeof(double) * head_dim); /* dout row */
    double* orow = (double*)malloc(sizeof(double) * head_dim); /* out row, when given */
    double* acc = (double*)malloc(sizeof(double) * head_dim);
    double* acca = (double*)malloc(sizeof(double) * head_dim);
    double* kb = (double*)malloc(sizeof(double) * ((size_t)Lk * head_dim + 1)); /* K of (b, kvh) */
    double* vb = (double*)malloc(sizeof(double) * ((size_t)Lk * head_dim + 1)); /* V of (b, kvh) */
    double* s = (double*)malloc(sizeof(double) * ((size_t)Lk + 1));
    double* dp = (double*)malloc(sizeof(double) * ((size_t)Lk + 1));
    double* av = (double*)malloc(sizeof(double) * ((size_t)Lk + 1)); /* sum_e |dout_e v_j,e| */
    int hh;

#pragma omp for schedule(dynamic, 1)
    for (hh = 0; hh < Hq; ++hh) {
      const int kvh = hh / (Hq / Hkv);
      const double* r = bias + (size_t)hh * R;
      double* dkq = dk_h + (size_t)hh * head_kv;
      double* dvq = dv_h + (size_t)hh * head_kv;
      double* dkaq = want_abs ? dka_h + (size_t)hh * head_kv : NULL;
      double* dvaq = want_abs ? dva_h + (size_t)hh * head_kv : NULL;
      double* dr = dbias + (size_t)hh * R;
      double* dra = want_abs ? dbias_abs + (size_t)hh * R : NULL;
      int b, t, j, e;
      for (j = 0; j < R; ++j) {
        dr[j] = 0.0;
        if (dra) dra[j] = 0.0;
      }
      for (b = 0; b < B; ++b) {
        for (j = 0; j < Lk; ++j) {
          const size_t off = (((size_t)b * Lk + j) * Hkv + kvh) * head_dim;
          widen(k, off, head_dim, dtype, kb + (size_t)j * head_dim);
          widen(v, off, head_dim, dtype, vb + (size_t)j * head_dim);
        }
        for (t = 0; t < Lq; ++t) {
          const int p = Lk - Lq + t; /* absolute query position */
          const int lo = (window > 0 && p - window + 1 > 0) ? p - window + 1 : 0;
          const size_t qoff = (((size_t)b * Lq + t) * Hq + hh) * head_dim;
          double m = -INFINITY, Z = 0.0, D = 0.0, Dabs = 0.0;
          widen(q, qoff, head_dim, dtype, qrow);
          widen(dout, qoff, head_dim, dtype, grow);
          if (out != NULL) widen(out, qoff, head_dim, dtype, orow);
          /* logits and their maximum */
          for (j = lo; j <= p; ++j) {
            const double* kj = kb + (size_t)j * head_dim;
            const int dist = p - j;
            double dot = 0.0;
            for (e = 0; e < head_dim; ++e) dot += qrow[e] * kj[e];
            s[j] = dot * scale + r[dist < R - 1 ? dist : R - 1];
            if (s[j] > m) m = s[j];
          }
          /* P (stored over s), dP and D */
          for (j = lo; j <= p; ++j) {
            s[j] = exp(s[j] - m);
            Z += s[j];
          }
          for (j = lo; j <= p; ++j) {
            const double* vj = vb + (size_t)j * head_dim;
            double d1 = 0.0, d2 = 0.0;
            s[j] /= Z;
            for (e = 0; e < head_dim; ++e) {
              d1 += grow[e] * vj[e];
              d2 += fabs(grow[e] * vj[e]);
            }
            dp[j] = d1;
            av[j] = d2;
            D += s[j] * d1;
            Dabs += s[j] * d2;
          }
          if (out != NULL) { /* D from the given forward output */
            D = Dabs = 0.0;
            for (e = 0; e < head_dim; ++e) {
              D += grow[e] * orow[e];
              Dabs += fabs(grow[e] * orow[e]);
            }
          }
          /* dS and the four gradients */
          for (e = 0; e < head_dim; ++e) acc[e] = acca[e] = 0.0;
          for (j = lo; j <= p; ++j) {
            const double* kj = kb + (size_t)j * head_dim;
            const int dist = p - j;
            const int c = dist < R - 1 ? dist : R - 1;
            const double ds = s[j] * (dp[j] - D);
            const double dsa = s[j] * (fabs(dp[j] - D) + abs_weight * (av[j] + Dabs));
            double* dkj = dkq + ((size_t)b * Lk + j) * head_dim;
            double* dvj = dvq + ((size_t)b * Lk + j) * head_dim;
            for (e = 0; e < head_dim; ++e) {
              acc[e] += ds * kj[e];
              dkj[e] += ds * qrow[e] * scale;
              dvj[e] += s[j] * grow[e];
            }
            dr[c] += ds;
            if (want_abs) {
              double* dkaj = dkaq + ((size_t)b * Lk + j) * head_dim;
              double* dvaj = dvaq + ((size_t)b * Lk + j) * head_dim;
              for (e = 0; e < head_dim; ++e) {
                acca[e] += dsa * fabs(kj[e]);
                dkaj[e] += dsa * fabs(qrow[e]) * scale;
                dvaj[e] += s[j] * fabs(grow[e]);
              }
              dra[c] += dsa;
            }
          }
          for (e = 0; e < head_dim; ++e) {
            dq[qoff + e] = acc[e] * scale;
            if (want_abs) dq_abs[qoff + e] = acca[e] * scale;
          }
        }
      }
    }
    free(qrow);
    free(grow);
    free(orow);
    free(acc);
    free(acca);
    free(kb);
    free(vb);
    free(s);
    free(dp);
    free(av);
  }

  /* dk, dv: the query heads of each KV head, summed in head order */
  for (x = 0; x < kv_elems; ++x) {
    dk[x] = dv[x] = 0.0;
    if (want_abs) dk_abs[x] = dv_abs[x] = 0.0;
  }
  for (h = 0; h < Hq; ++h) {
    const int kvh = h / (Hq / Hkv);
    int b, j;
    for (b = 0; b < B; ++b)
      for (j = 0; j < Lk; ++j) {
        const size_t src = ((size_t)h * B * Lk + (size_t)b * Lk + j) * head_dim;
        const size_t dst = (((size_t)b * Lk + j) * Hkv + kvh) * head_dim;
        for (g = 0; g < head_dim; ++g) {
          dk[dst + g] += dk_h[src + g];
          dv[dst + g] += dv_h[src + g];
          if (want_abs) {
            dk_abs[dst + g] += dka_h[src + g];
            dv_abs[dst + g] += dva_h[src + g];
          }
        }
      }
  }
  free(dk_h);
  free(dv_h);
  free(dka_h);
  free(dva_h);
  return 0;
}
