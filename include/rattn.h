/*
 * rattn.h -- relative-bias grouped-query attention for AMD Instinct MI355X (gfx950).
 *
 * The operation (vLLM recipes page "thinkingmachines/Inkling", Overview > Architectural
 * highlights > Attention): grouped-query attention with head size 128 without RoPE; the
 * logits instead carry a trained bias that depends on the distance between query and key.
 * The term is a per-query-head table r indexed by the clamped distance, so for a query at
 * absolute position i and a key at position j:
 *
 *     logit[i, j] = (q_i . k_j) / sqrt(128) + r[h, min(i - j, R - 1)]
 *     out_i       = sum_j softmax_j(logit[i, :]) v_j,   lse_i = log sum_j exp(logit[i, j])
 *
 * over the visible keys: 0 <= i - j (causal) and, for a sliding-window layer with window
 * W > 0, i - j <= W - 1 (W keys including the query itself).  The page names both full and
 * sliding-window layers, multi-token (MTP) verification of up to 9 tokens per step
 * (Overview > MTP), and a paged KV cache with 128-token blocks (Client Usage,
 * "--block-size 128").
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, innermost dimension last; the head dimension is 128.
 *   - Query head h reads KV head h / (Hq / Hkv) (contiguous groups); Hq % Hkv == 0.
 *   - bf16 data is IEEE bfloat16 bit patterns.  Accumulation is fp32.  bf16 outputs are
 *     rounded to nearest even from fp32.
 *   - lse is fp32, natural logarithm.
 *   - Device pointers must be valid on the current HIP device; `stream` is a hipStream_t
 *     passed as void* (NULL = the null stream).  Calls only enqueue work: they neither
 *     allocate nor synchronise, and the caller owns every buffer.
 *   - Status: RATTN_OK or an error code; on error rattn_last_error() returns a
 *     thread-local message.  Argument errors are detected on the host before any HIP call,
 *     so nothing is enqueued and no output is written.
 *   - Results are deterministic: fixed arguments give bitwise-identical outputs.
 */
#ifndef RATTN_H
#define RATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RATTN_ABI_VERSION 9

enum rattn_status {
  RATTN_OK = 0,
  RATTN_ERR_INVALID_ARG = 1, /* null pointer, inconsistent sizes */
  RATTN_ERR_UNSUPPORTED = 2, /* head_dim != 128, block_size != 128, dtype not handled */
  RATTN_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  RATTN_ERR_HIP = 4          /* a HIP launch failed; message holds hipGetErrorString */
};

enum rattn_dtype { RATTN_BF16 = 0, RATTN_FP32 = 1 };

/*
 * Device workspace, in bytes, that rattn_prefill uses for these arguments: for bf16, a
 * 256-byte job queue, plus, where the plan splits the key range of its heaviest query
 * tiles, per-tile counters and the pieces' partial results; for fp32, 0.  kv_splits as
 * for rattn_prefill.  The plan is a pure function of the arguments.  Returns 0 for
 * invalid sizes.
 *
 * Why a queue: one workgroup fits on a compute unit (its K/V ring fills the LDS), so a
 * grid of one workgroup per query tile leaves each unit idle while a finished workgroup's
 * stores drain and the next one starts (~6 us per hand-over, measured).  With the queue
 * the launch has one workgroup per compute unit, each taking the next query tile (or
 * piece) as it finishes one.
 * Why a split: the query tiles of a long sliding-window (or long causal) prefill all walk
 * about as many keys as the longest one, and with about two tiles per compute unit the
 * last ones to start finish late.  Splitting the keys of the heaviest tiles into pieces
 * that merge by log-sum-exp evens the work out (the key-range split the decode path uses
 * for every sequence, applied to prefill tiles).
 */
size_t rattn_prefill_workspace_bytes(int B, int Lq, int Lk, int Hq, int Hkv, int window, int dtype,
                                     int kv_splits);

/*
 * Prefill / chunked prefill over contiguous K/V.
 *
 *   q    [B, Lq, Hq, 128]   dtype    device, read
 *   k    [B, Lk, Hkv, 128]  dtype    device, read
 *   v    [B, Lk, Hkv, 128]  dtype    device, read
 *   bias [Hq, R]            fp32     device, read   (r above; R >= 1)
 *   out  [B, Lq, Hq, 128]   dtype    device, written
 *   lse  [B, Lq, Hq]        fp32     device, written; may be NULL
 *   workspace               device scratch of workspace_bytes >=
 *                           rattn_prefill_workspace_bytes(...) bytes, or NULL with
 *                           workspace_bytes = 0 (then one workgroup per query tile,
 *                           nothing split: slower, same result)
 *
 * Query t of every sequence sits at absolute position Lk - Lq + t (bottom-right alignment:
 * a chunk of Lq new tokens whose own keys are the last Lq of the Lk keys), so Lq <= Lk.
 * window <= 0 selects full causal attention; window > 0 a sliding window of that many keys.
 * dtype RATTN_BF16: bf16 in/out.  RATTN_FP32: fp32 in/out; q.k is formed without rounding
 * the inputs to bf16 (three-term bf16 split), likewise p.v (never key-split).
 * kv_splits: 0 = the library's plan (a split only where it shortens the launch), 1 = no
 * split, n in 2..8 = split every query tile with at least 2n key tiles of 64 into n pieces.
 * A split changes only the summation order of the result.
 * Workspace: its first 256 bytes + 256 KB hold the job queue and the per-tile split
 * counters (at the same place for every plan), which must be zero when the workspace is
 * first used; every completed call leaves them zero again, so a workspace zero-filled
 * once can be reused by later calls of any size and plan it is large enough for.  Calls that share a workspace must not run concurrently.  With or without a
 * workspace, and whichever workgroup runs which tile, the result is the same bit for bit
 * for a given plan.
 * B == 0 or Lq == 0 is a no-op returning RATTN_OK (pointers may then be NULL).
 * Status: INVALID_ARG for a null required pointer, negative sizes, Hq % Hkv != 0, Lq > Lk,
 * R < 1, kv_splits outside 0..8, workspace_bytes > 0 with a NULL workspace; WORKSPACE if
 * workspace_bytes is below rattn_prefill_workspace_bytes(...); UNSUPPORTED for head_dim !=
 * 128 or an unknown dtype; HIP if the launch fails.
 */
int rattn_prefill(const void* q, const void* k, const void* v, const float* bias, void* out,
                  float* lse, int B, int Lq, int Lk, int Hq, int Hkv, int head_dim, int R,
                  int window, int dtype, int kv_splits, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Prefill / chunked prefill with a token-dependent relative-bias table.  The recipes page
 * "thinkingmachines/Inkling" keeps the "qkvr" linears in BF16 (Variants) and names a
 * sheared-bias attention kernel for relative attention (Performance); read here as the
 * projection producing, for every query token t, its own table r_t (bf16), so that
 *     logit[t, j] = (q_t . k_j) / sqrt(128) + r_t[h, min(p - j, R - 1)]
 * for the query at position p = Lk - Lq + t.  Everything else (positions, causal / window
 * visibility, GQA mapping, outputs, workspace and split plan) is that of rattn_prefill with
 * dtype RATTN_BF16.
 *
 *   bias_tok [B, Lq, Hq, R]  bf16  device, read; row (b, t, h) is r_t[h, :] of query t;
 *            4-byte aligned; R >= 4.  Entries at distances that no visible key of the row
 *            has (d > p, or d >= window) are never used and may hold anything (NaN
 *            included); the clamp entry r_t[h, R - 1] is used when the row sees a key at
 *            distance >= R - 1.
 *
 * Status: as rattn_prefill; INVALID_ARG also for a misaligned bias_tok, UNSUPPORTED for R < 4.
 */
int rattn_prefill_tokbias(const void* q, const void* k, const void* v, const void* bias_tok,
                          void* out, float* lse, int B, int Lq, int Lk, int Hq, int Hkv,
                          int head_dim, int R, int window, int kv_splits, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Chunked prefill against a paged KV cache (prefix caching: vLLM recipes page
 * "thinkingmachines/Inkling", Overview, lists prefix caching among the supported features;
 * Client Usage serves with 128-token cache blocks).  Sequence b has ctx_lens[b] keys in
 * the cache, the chunk's own K/V included; its n_b queries (n_b = Lq, or with packed
 * queries cu_seqlens_q[b + 1] - cu_seqlens_q[b]) are its last n_b tokens, query t at
 * position ctx_lens[b] - n_b + t, with the relative-bias attention and causal / window
 * rule of rattn_prefill.
 *
 *   q           [B, Lq, Hq, 128]                  bf16   device, read; with cu_seqlens_q,
 *               packed [cu_seqlens_q[B], Hq, 128]: sequence b's queries are rows
 *               cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1 (out and lse likewise)
 *   cu_seqlens_q [B + 1]                          int32  device, read, or NULL (Lq queries
 *               per sequence); non-decreasing from 0, with 0 <= n_b <= Lq the caller's
 *               guarantee (Lq is then the longest chunk)
 *   k_cache     [num_blocks, 128, Hkv, 128]       bf16   device, read
 *   v_cache     [num_blocks, 128, Hkv, 128]       bf16   device, read
 *   block_table [B, max_blocks_per_seq]           int32  device, read (physical block ids)
 *   ctx_lens    [B]                               int32  device, read; n_b <= ctx_lens[b] <=
 *               min(max_ctx_len, 128 * max_blocks_per_seq) is the caller's guarantee
 *   bias        [Hq, R]                           fp32   device, read
 *   out         [B, Lq, Hq, 128]                  bf16   device, written
 *   lse         [B, Lq, Hq]                       fp32   device, written (natural log); may be NULL
 *   window      <= 0 full causal, else the sliding window (as in rattn_prefill)
 *
 * Only blocks holding a key visible to some query of the chunk are read; other block-table
 * entries are never dereferenced.  Cache slots before the first query's window, and at or
 * past ctx_lens[b], may hold anything (NaN included): they are zero-filled on load.
 * A job is (sequence, KV head, head group, 32 (8 / query heads per workgroup) tokens of
 * the chunk, up to Lq); jobs run sequence by sequence, longest context first.  workspace: NULL (one workgroup per job) or at least
 * RATTN_PREFILL_PAGED_WORKSPACE_BYTES of device memory, zero-filled before its first use,
 * holding a job queue (one workgroup per compute unit takes jobs until none is left); every
 * completed call leaves it zero, and calls sharing it must not run concurrently (the
 * first 256 bytes of a rattn_prefill workspace serve as well).  Either way the result is
 * the same bit for bit.  B == 0 or Lq == 0 is a no-op.  Status: INVALID_ARG (null pointer,
 * sizes, Hq % Hkv, R < 1, num_blocks < 1, max_ctx_len < Lq or beyond the block table,
 * workspace_bytes > 0 with a NULL workspace), WORKSPACE (a workspace smaller than
 * RATTN_PREFILL_PAGED_WORKSPACE_BYTES), UNSUPPORTED (head_dim or block_size != 128), HIP
 * (launch failure).
 */
#define RATTN_PREFILL_PAGED_WORKSPACE_BYTES 256

int rattn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                        const int* block_table, const int* ctx_lens, const int* cu_seqlens_q,
                        const float* bias, void* out, float* lse, int B, int Lq, int Hq, int Hkv,
                        int head_dim, int block_size, int R, int window, int num_blocks,
                        int max_blocks_per_seq, int max_ctx_len,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Short convolution of the new keys and values as they enter the paged caches (vLLM recipes
 * page "thinkingmachines/Inkling", Overview > Architectural highlights > Short convolution:
 * four-tap short convolutions over the token axis of the attention keys and values, among
 * others, with their state kept in paged storage).  Read as the causal depthwise convolution over
 * tokens with four taps and a weight per tap and channel, no bias, no activation:
 *     y[p, c] = sum_{s=0..3} w[s, c] * x[p - s, c],   x[p] = 0 for p < 0.
 * Sequence b has n_b = cu_seqlens[b + 1] - cu_seqlens[b] new tokens at positions
 * ctx_lens[b] - n_b .. ctx_lens[b] - 1: y (rounded to bf16, nearest even) is written to the
 * attention caches and the raw x to the state caches at those positions; the raw x of up to
 * three earlier positions is read from the state caches (written by earlier calls).
 *
 *   k_new, v_new    [cu_seqlens[B], Hkv, 128]          bf16  device, read (packed new tokens)
 *   w_k, w_v        [4, Hkv, 128]                      fp32  device, read (tap s multiplies x[p - s])
 *   k_cache, v_cache [num_blocks, 128, Hkv, 128]       bf16  device, written at the new positions
 *   k_state, v_state [num_blocks, 128, Hkv, 128]       bf16  device, read before each chunk,
 *                    written at the new positions (the caches share the block table)
 *   block_table     [B, max_blocks_per_seq]            int32 device, read
 *   ctx_lens        [B]                                int32 device, read: keys after the write
 *   cu_seqlens      [B + 1]                            int32 device, read: non-decreasing from 0
 *
 * Caller's guarantees: 0 <= n_b <= max_new, n_b <= ctx_lens[b] <= 128 * max_blocks_per_seq,
 * block-table entries of the positions written or read are valid, and no two sequences write
 * the same physical slot.  Only those slots are touched.  Bitwise reproducible.  B == 0 or
 * max_new == 0 is a no-op.  Status: INVALID_ARG (null pointer, sizes, B > 65535),
 * UNSUPPORTED (head_dim or block_size != 128, Hkv > 8), HIP (launch failure).
 */
int rattn_kv_sconv_write(const void* k_new, const void* v_new, const float* w_k, const float* w_v,
                         void* k_cache, void* v_cache, void* k_state, void* v_state,
                         const int* block_table, const int* ctx_lens, const int* cu_seqlens, int B,
                         int Hkv, int head_dim, int block_size, int num_blocks,
                         int max_blocks_per_seq, int max_new, void* stream);

/*
 * Device workspace, in bytes, that rattn_prefill_backward needs: two fp32 per query row
 * (rowsum(dout * out) and lse * log2(e), B * Lq * Hq rows), then, for each of two chunks of
 * a key block's queries and each pair of query heads of a KV head (ceil(G / 2) pairs,
 * G = Hq / Hkv), a partial dK and a partial dV ([B, Lk, Hkv, 128] fp32 each), then two
 * partial dq per query row and head for token tiles cut in two (2 * B * Hq * (Lq rounded up
 * to 256) * 128 fp32), then the bias table scaled to score units (Hq * Lk fp32:
 * at most Lk entries per head are reachable), then B * Hq * ceil(Lq / 32) int counters, every
 * part rounded up to 256 bytes.  Returns 0 for invalid sizes.
 */
size_t rattn_prefill_backward_workspace_bytes(int B, int Lq, int Lk, int Hq, int Hkv);

/*
 * Gradients of rattn_prefill (bf16, contiguous K/V) for an output gradient dout.
 * vLLM recipes page "thinkingmachines/Inkling", Overview > Architectural highlights >
 * Attention defines the forward pass (GQA, head size 128, a distance-dependent bias on the
 * logits); the same page lists training and LoRA among the model's uses.  With
 * s = q.k / sqrt(128) + r[h, min(p - j, R - 1)] over the visible keys (the visibility and
 * positions of rattn_prefill), P = softmax(s) recomputed from lse, D = rowsum(dout * out):
 *   dS = P * (dout V^T - D),  dq = dS K / sqrt(128),  dk = dS^T Q / sqrt(128),
 *   dv = P^T dout,  dbias[h, d] = sum of dS over the pairs at clamped distance d,
 * dk and dv summed over the query heads of each KV head.
 *
 *   q, out, dout  [B, Lq, Hq, 128]    bf16   device, read (out and lse: rattn_prefill's
 *   k, v          [B, Lk, Hkv, 128]   bf16   device, read  results for these inputs)
 *   bias          [Hq, R]             fp32   device, read
 *   lse           [B, Lq, Hq]         fp32   device, read (natural log)
 *   dq            [B, Lq, Hq, 128]    fp32   device, written
 *   dk, dv        [B, Lk, Hkv, 128]   fp32   device, written (every entry, once)
 *   dbias         [Hq, R]             fp32   device, written (zeroed, then accumulated)
 *   workspace     device scratch of at least rattn_prefill_backward_workspace_bytes(...)
 *   window        <= 0 full causal, > 0 sliding window of that many keys
 *
 * The caller owns every buffer; the call enqueues its kernels on `stream` and returns.
 * dq, dk and dv are deterministic (dk and dv: per-pair partials summed in pair order);
 * dbias is a sum of fp32 atomic adds, so its last bits may differ from run to run.
 * A non-finite dout or out row makes the gradients that depend on it non-finite, and may do
 * so for dk, dv and dbias entries of the same query head's 32 x 32 (query, key) tiles that it
 * does not reach (a product with a zero probability is still non-finite); nothing is ever
 * written outside dq, dk, dv, dbias and the workspace.  Status: INVALID_ARG (null
 * pointer, sizes, Lq > Lk, B or Hq > 65535), UNSUPPORTED (head_dim != 128), WORKSPACE
 * (missing or too small), HIP (launch failure).
 */
int rattn_prefill_backward(const void* q, const void* k, const void* v, const float* bias,
                           const void* out, const void* dout, const float* lse, float* dq,
                           float* dk, float* dv, float* dbias, int B, int Lq, int Lk, int Hq,
                           int Hkv, int head_dim, int R, int window, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Number of split workgroups rattn_decode_paged will use for these arguments.  The
 * visible keys of the whole batch form one stream of 64-token units that is divided
 * evenly among them.  num_splits > 0 asks for exactly that many (fewer when the batch has
 * fewer units); 0 selects the default, one per compute unit of the current device (256 on
 * an MI355X; 256 too when no device answers the query).  Returns
 * 0 for invalid sizes.  The choice changes only the summation order of the result.
 */
int rattn_decode_num_splits(int B, int n_q, int Hq, int Hkv, int max_ctx_len, int num_splits);

/*
 * Device workspace, in bytes, that rattn_decode_paged needs for these arguments (one
 * partial output and log-sum-exp per split workgroup and per segment it touches).  It is
 * an upper bound for any max_blocks_per_seq.  Returns 0 for invalid sizes.
 */
size_t rattn_decode_workspace_bytes(int B, int n_q, int Hq, int Hkv, int max_ctx_len,
                                    int num_splits);

/*
 * Paged decode with multi-query (MTP) verification: n_q query tokens per sequence attend
 * to the sequence's paged KV cache.  The visible keys are split among the workgroups
 * (rattn_decode_num_splits) and the partial results are merged by log-sum-exp.
 *
 *   q           [B, n_q, Hq, 128]                 bf16   device, read
 *   k_cache     [num_blocks, 128, Hkv, 128]       bf16   device, read
 *   v_cache     [num_blocks, 128, Hkv, 128]       bf16   device, read
 *   block_table [B, max_blocks_per_seq]           int32  device, read (physical block ids)
 *   ctx_lens    [B]                               int32  device, read; keys in the cache
 *               for the sequence INCLUDING its n_q query tokens; 1 <= n_q <= ctx_lens[b]
 *               <= min(max_ctx_len, 128 * max_blocks_per_seq) is the caller's guarantee
 *   windows     [B]                               int32  device, read; <= 0 full causal,
 *               > 0 sliding window; NULL means every sequence is full causal
 *   bias        [Hq, R]                           fp32   device, read
 *   out         [B, n_q, Hq, 128]                 bf16   device, written
 *   lse         [B, n_q, Hq]                      fp32   device, written; may be NULL
 *   workspace   device scratch of at least rattn_decode_workspace_bytes(...) bytes
 *
 * Query t of sequence b sits at position ctx_lens[b] - n_q + t and sees keys per the
 * causal / window rule above (the n_q queries are causal among themselves).
 * Only blocks holding a key visible to some query of the sequence are read; other
 * block-table entries are never dereferenced and may hold anything.  Cache slots outside
 * [max(0, ctx - n_q - W + 1), ctx) (W the window, 0 if full) may hold anything, NaN
 * included: they are zero-filled on load and never reach an output.
 * block_size and head_dim must be 128.  num_splits: 0 = automatic, else the number of split
 * workgroups.  Batches are processed in launches of at most 2048 sequences.
 * B == 0 is a no-op.  Status: INVALID_ARG (null pointer, sizes, Hq % Hkv, n_q < 1, R < 1,
 * num_blocks < 1), UNSUPPORTED (head_dim, block_size, n_q > 128),
 * WORKSPACE (workspace NULL or smaller than required), HIP (launch failure).
 */
int rattn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                       const int* block_table, const int* ctx_lens, const int* windows,
                       const float* bias, void* out, float* lse, int B, int n_q, int Hq,
                       int Hkv, int head_dim, int block_size, int R, int num_blocks,
                       int max_blocks_per_seq, int max_ctx_len, int num_splits,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free paged decode, for callers that cannot allocate device memory on the call
 * path: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, computation and result as rattn_decode_paged (the same
 * kernels and split plan: the output is bit-identical), minus the workspace: the split
 * partials go to a static device array of rattn_decode_paged_noalloc_max_scratch_bytes()
 * bytes (64 MiB) that the library holds on every device it runs on until the process ends.
 * The call allocates and frees nothing (no hipMalloc, hipFree or allocating library
 * routine); its first call on a device looks the array's address up on that device.
 * The array holds only partial results that each call writes before it reads them, so
 * nothing in it has to start at zero; it keeps the last call's contents.
 * Every call on one device shares that device's array: calls that overlap on one device
 * (on different streams, or from different threads without ordering) race and may return
 * wrong results; calls on one stream are ordered and safe.
 * Status: as rattn_decode_paged, and WORKSPACE when rattn_decode_workspace_bytes(...) for
 * these sizes exceeds the static size (checked on the host before any launch; use
 * rattn_decode_paged with a workspace, or fewer sequences per call); HIP if the array's
 * address cannot be obtained.
 */
size_t rattn_decode_paged_noalloc_max_scratch_bytes(void);

int rattn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                               const int* block_table, const int* ctx_lens, const int* windows,
                               const float* bias, void* out, float* lse, int B, int n_q, int Hq,
                               int Hkv, int head_dim, int block_size, int R, int num_blocks,
                               int max_blocks_per_seq, int max_ctx_len, int num_splits,
                               void* stream);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* rattn_last_error(void);

/* RATTN_ABI_VERSION of the loaded library. */
int rattn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RATTN_H */
