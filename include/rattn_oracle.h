/*
 * rattn_oracle.h -- interface of the CPU oracle library oracle/librattn_oracle.so.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This header belongs to the oracle library only:
 * the HIP library (librattn.so, include/rattn.h) neither includes it nor links the oracle,
 * and the two share no source, header, helper or constant.
 *
 * Relative-bias grouped-query attention, vLLM recipes page "thinkingmachines/Inkling",
 * Overview > Architectural highlights > Attention (GQA, head size 128, a trained bias on the
 * logits that depends on the query-key distance, in place of RoPE), with the term fixed as
 * r[h, min(i - j, R - 1)].  Computed in fp64 from the plain definition.
 *
 * Bias tables are passed as double: the fp32 tables of the HIP library widen to double
 * exactly, and the pins also feed tables that fp32 cannot hold.
 */
#ifndef RATTN_ORACLE_H
#define RATTN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

#define RATTN_ORACLE_BF16 0 /* inputs are bfloat16 bit patterns (uint16) */
#define RATTN_ORACLE_FP32 1
#define RATTN_ORACLE_FP64 2

/*
 * Forward pass.  All pointers are HOST pointers; the call is synchronous and touches no
 * device.
 *
 * q      [B, n_q, Hq, head_dim]                        (dtype)
 * k, v   contiguous: [B, Lk_max, Hkv, head_dim]        when block_table == NULL
 *        paged:      [num_blocks, block_size, Hkv, head_dim]  otherwise   (dtype)
 * block_table [B, max_blocks_per_seq] int32 physical block ids, or NULL
 * ctx_lens    [B] keys of each sequence, including its n_q query tokens
 * windows     [B] window per sequence (<= 0: full causal), or NULL for all full
 * bias        [Hq, R] double
 * out         [B, n_q, Hq, head_dim] double
 * lse         [B, n_q, Hq] double natural log, or NULL
 * probs       [B, n_q, Hq, Lk_max] double attention weights (0 where not visible), or NULL
 * Query t of sequence b sits at position ctx_lens[b] - n_q + t.
 * num_threads <= 0 keeps the OpenMP default.
 * Returns 0 on success, 1 on an invalid argument (nothing written).
 */
int rattn_ref_cpu(const void* q, const void* k, const void* v, const int* block_table,
                  const int* ctx_lens, const int* windows, const double* bias, double* out,
                  double* lse, double* probs, int B, int n_q, int Lk_max, int Hq, int Hkv,
                  int head_dim, int block_size, int R, int max_blocks_per_seq, int dtype,
                  int num_threads);

/*
 * Forward pass with a token-dependent bias: every query row has its own table, so the
 * logit of query t (position p) of sequence b, head h, and key j is
 *     q . k_j / sqrt(head_dim) + bias[b, t, h, min(p - j, R - 1)],
 * bias being [B, n_q, Hq, R] double.  Everything else as rattn_ref_cpu.
 */
int rattn_ref_cpu_tokbias(const void* q, const void* k, const void* v, const int* block_table,
                          const int* ctx_lens, const int* windows, const double* bias,
                          double* out, double* lse, double* probs, int B, int n_q, int Lk_max,
                          int Hq, int Hkv, int head_dim, int block_size, int R,
                          int max_blocks_per_seq, int dtype, int num_threads);

/*
 * Backward pass of a prefill over contiguous K/V (every sequence has Lk keys; query t at
 * position Lk - Lq + t; window <= 0 full causal), for an output gradient dout:
 *     P = softmax over the visible keys,  dP = dout V^T,  D = sum_j P_j dP_j (per row),
 *     dS = P (dP - D),  dq = dS K / sqrt(d),  dk = dS^T Q / sqrt(d),  dv = P^T dout,
 *     dbias[h, c] = sum of dS over the visible pairs with min(p - j, R - 1) = c,
 * dk and dv summed over the query heads of each KV head.
 *
 * q, dout [B, Lq, Hq, head_dim], k, v [B, Lk, Hkv, head_dim] (dtype); bias [Hq, R] double;
 * dq [B, Lq, Hq, head_dim], dk, dv [B, Lk, Hkv, head_dim], dbias [Hq, R] double, written.
 *
 * out: NULL, or a forward output [B, Lq, Hq, head_dim] (dtype): then D = sum_e dout_e out_e
 * per row, the row sum a backward implementation takes from the forward's (rounded) output,
 * in place of sum_j P_j dP_j.
 *
 * Optional magnitude sums (NULL to skip), the same sums with every term replaced by its
 * absolute value and dS by dS_abs = P_j (|dP_j - D| + w (a_j + D_abs)), where
 * a_j = sum_e |dout_e v_j,e| is the size of dP_j's terms, D_abs the size of D's terms
 * (sum_j P_j a_j, or sum_e |dout_e out_e| with out) and w = abs_weight: dq_abs, dk_abs,
 * dv_abs (dv_abs = P^T |dout|), dbias_abs.  They bound rounding errors of an
 * implementation element by element.
 * Returns 0 on success, 1 on an invalid argument (nothing written).
 */
int rattn_ref_cpu_backward(const void* q, const void* k, const void* v, const void* dout,
                           const void* out, const double* bias, double* dq, double* dk, double* dv,
                           double* dbias, double* dq_abs, double* dk_abs, double* dv_abs,
                           double* dbias_abs, double abs_weight, int B, int Lq, int Lk, int Hq,
                           int Hkv, int head_dim, int R, int window, int dtype, int num_threads);

int rattn_oracle_version(void);

#ifdef __cplusplus
}
#endif
#endif
