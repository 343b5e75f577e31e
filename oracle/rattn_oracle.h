/*
 * rattn_oracle.h -- the CPU oracle's own interface (test infrastructure, not product).
 *
 * Relative-bias grouped-query attention, vLLM recipes page "thinkingmachines/Inkling",
 * Overview > Architectural highlights > Attention (GQA, head size 128, a trained bias on the
 * logits that depends on the query-key distance, in place of RoPE), with the term fixed as
 * r[h, min(i - j, R - 1)].  Computed in fp64 from the plain definition.
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
 * All pointers are HOST pointers; the call is synchronous and touches no device.
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

int rattn_oracle_version(void);

#ifdef __cplusplus
}
#endif
#endif
