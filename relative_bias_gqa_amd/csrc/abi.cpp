// abi.cpp -- the C-ABI entry points declared in include/rattn.h.
//
// Host-side only: argument validation (always before any HIP call), the work
// decomposition of each launch, the split plan of the paged decode, and the thread-local
// error message.  No allocation and no synchronisation happen here: every call enqueues
// its kernels on the caller's stream and returns.
#include <stdarg.h>
#include <stdio.h>

#include "launch.hpp"
#include "rattn.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return RATTN_OK;
}

int largest_divisor_at_most(int n, int cap) {
  for (int d = cap; d > 1; --d)
    if (n % d == 0) return d;
  return 1;
}

constexpr int kMaxPosition = (1 << 30) - 1;  // positions stay clear of the kernels' window sentinel
constexpr float kScaleLog2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)

// ---- paged-decode plan ---------------------------------------------------------------
// Segment = (sequence, KV head, subgroup of gs query heads); rows = n_q * gs.  The unit
// stream (64-token units of every segment) is divided among P workgroups; sequences are
// processed in launches of at most `batch` sequences, each reusing the same workspace.
constexpr int kAutoWorkgroups = 256;  // one per compute unit of an MI355X

struct DecodePlan {
  int gs, n_hs, KH, rows, SL, P, batch, KS;
  size_t lse_off, total;
};

bool plan_decode(int B, int n_q, int Hq, int Hkv, int max_ctx_len, int max_blocks, int num_splits, DecodePlan* pl) {
  if (B < 1 || n_q < 1 || n_q > rattn::kDecodeMaxRows || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      max_ctx_len < 1 || max_ctx_len > kMaxPosition || max_blocks < 1 || num_splits < 0)
    return false;
  const int G = Hq / Hkv;
  const int SL = rattn::kDecodeUnit - 1 + n_q;
  // query heads per segment: the largest divisor of G whose rows fit four waves and whose
  // bias slices fit the per-unit staging buffer
  int gs = 0;
  for (int d = G; d >= 1; --d) {
    if (G % d == 0 && n_q * d <= rattn::kDecodeMaxRows && d * SL <= rattn::kDecodeBiasFloats) {
      gs = d;
      break;
    }
  }
  if (gs == 0) return false;
  const int n_hs = G / gs;
  const long long KH = (long long)Hkv * n_hs;
  // units per launch must stay below 2^31 (a sequence has at most 2 units per block-table
  // entry, whatever ctx_lens holds: the kernels clamp it to the table)
  (void)max_ctx_len;
  const long long max_units_per_seq = 2LL * max_blocks + 1;
  long long batch = B < rattn::kDecodeMaxBatch ? B : rattn::kDecodeMaxBatch;
  const long long cap = 0x7fffffffLL / (max_units_per_seq * KH);
  if (cap < 1) return false;
  if (batch > cap) batch = cap;
  const int P = num_splits > 0 ? num_splits : kAutoWorkgroups;
  const long long rows = (long long)n_q * gs;
  // up to two row blocks of 32: the two 32-key halves of a unit go to different waves
  const int KS = rows <= 64 ? 2 : 1;
  const long long slots = (P + batch * KH) * KS;
  if (batch * KH * rows > 0x7fffffffLL) return false;
  pl->gs = gs;
  pl->n_hs = n_hs;
  pl->KH = (int)KH;
  pl->rows = (int)rows;
  pl->SL = SL;
  pl->P = P;
  pl->batch = (int)batch;
  pl->KS = KS;
  const size_t o_bytes = (size_t)slots * (size_t)rows * 128 * sizeof(float);
  pl->lse_off = (o_bytes + 255) & ~(size_t)255;
  pl->total = pl->lse_off + (size_t)slots * (size_t)rows * sizeof(float);
  return true;
}

}  // namespace

extern "C" {

const char* rattn_last_error(void) { return g_err; }

int rattn_abi_version(void) { return RATTN_ABI_VERSION; }

int rattn_prefill(const void* q, const void* k, const void* v, const float* bias, void* out,
                  float* lse, int B, int Lq, int Lk, int Hq, int Hkv, int head_dim, int R,
                  int window, int dtype, void* stream) {
  if (B < 0 || Lq < 0 || Lk < 0 || Hq < 0 || Hkv < 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill: negative size (B=%d Lq=%d Lk=%d Hq=%d Hkv=%d)", B, Lq,
                Lk, Hq, Hkv);
  if (head_dim != 128) return fail(RATTN_ERR_UNSUPPORTED, "rattn_prefill: head_dim %d (only 128)", head_dim);
  if (dtype != RATTN_BF16 && dtype != RATTN_FP32)
    return fail(RATTN_ERR_UNSUPPORTED, "rattn_prefill: unknown dtype %d", dtype);
  if (B == 0 || Lq == 0) return ok();
  if (!q || !k || !v || !bias || !out) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill: null pointer argument");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill: Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (Lq > Lk) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill: Lq=%d > Lk=%d", Lq, Lk);
  if (Lk > kMaxPosition) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill: Lk=%d too large", Lk);
  if (R < 1) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill: R=%d < 1", R);

  rattn::PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.bias = bias;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.Lq = Lq;
  p.Lk = Lk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.R = R;
  p.window = window > 0 ? window : 0;
  p.G = Hq / Hkv;
  p.hpw = largest_divisor_at_most(p.G, 8);
  while (8 % p.hpw != 0) p.hpw = largest_divisor_at_most(p.G, p.hpw - 1);
  p.tsub = 8 / p.hpw;
  p.n_hg = p.G / p.hpw;
  p.n_tok_tiles = (Lq + 32 * p.tsub - 1) / (32 * p.tsub);
  p.scale_log2 = kScaleLog2;
  const long long grid = (long long)p.n_tok_tiles * B * Hkv * p.n_hg;
  if (grid > 0x7fffffffLL) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill: problem too large for one launch");

  hipError_t e = dtype == RATTN_BF16 ? rattn::launch_prefill_bf16(p, (hipStream_t)stream)
                                     : rattn::launch_prefill_fp32(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RATTN_ERR_HIP, "rattn_prefill: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int rattn_decode_num_splits(int B, int n_q, int Hq, int Hkv, int max_ctx_len, int num_splits) {
  DecodePlan pl;
  if (!plan_decode(B, n_q, Hq, Hkv, max_ctx_len, (max_ctx_len + 127) / 128, num_splits, &pl)) return 0;
  return pl.P;
}

size_t rattn_decode_workspace_bytes(int B, int n_q, int Hq, int Hkv, int max_ctx_len, int num_splits) {
  DecodePlan pl;
  if (!plan_decode(B, n_q, Hq, Hkv, max_ctx_len, (max_ctx_len + 127) / 128, num_splits, &pl)) return 0;
  return pl.total;
}

int rattn_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                       const int* ctx_lens, const int* windows, const float* bias, void* out, float* lse,
                       int B, int n_q, int Hq, int Hkv, int head_dim, int block_size, int R, int num_blocks,
                       int max_blocks_per_seq, int max_ctx_len, int num_splits, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_ctx_len < 0 || num_splits < 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: negative size");
  if (head_dim != 128) return fail(RATTN_ERR_UNSUPPORTED, "rattn_decode_paged: head_dim %d (only 128)", head_dim);
  if (block_size != 128)
    return fail(RATTN_ERR_UNSUPPORTED, "rattn_decode_paged: block_size %d (only 128)", block_size);
  if (n_q < 1) return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: n_q=%d < 1", n_q);
  if (n_q > rattn::kDecodeMaxRows)
    return fail(RATTN_ERR_UNSUPPORTED, "rattn_decode_paged: n_q=%d > %d", n_q, rattn::kDecodeMaxRows);
  if (B == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !bias || !out)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: null pointer argument");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (R < 1) return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: R=%d < 1", R);
  if (num_blocks < 1 || max_blocks_per_seq < 1)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: num_blocks=%d, max_blocks_per_seq=%d", num_blocks,
                max_blocks_per_seq);
  if (max_ctx_len < n_q)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: max_ctx_len=%d < n_q=%d", max_ctx_len, n_q);
  if ((long long)max_ctx_len > 128LL * max_blocks_per_seq || max_ctx_len > kMaxPosition)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: max_ctx_len=%d exceeds the block table (%d blocks)",
                max_ctx_len, max_blocks_per_seq);
  DecodePlan pl;
  if (!plan_decode(B, n_q, Hq, Hkv, max_ctx_len, max_blocks_per_seq, num_splits, &pl))
    return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: problem too large for one launch");
  if (!workspace || workspace_bytes < pl.total)
    return fail(RATTN_ERR_WORKSPACE, "rattn_decode_paged: workspace %zu bytes at %p, need %zu", workspace_bytes,
                workspace, pl.total);

  rattn::DecodeParams p;
  p.k_cache = (const uint16_t*)k_cache;
  p.v_cache = (const uint16_t*)v_cache;
  p.bias = bias;
  p.ws_o = (float*)workspace;
  p.ws_lse = (float*)((char*)workspace + pl.lse_off);
  p.n_q = n_q;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.R = R;
  p.num_blocks = num_blocks;
  p.mbps = max_blocks_per_seq;
  p.G = Hq / Hkv;
  p.gs = pl.gs;
  p.n_hs = pl.n_hs;
  p.KH = pl.KH;
  p.rows = pl.rows;
  p.SL = pl.SL;
  p.KS = pl.KS;
  p.P = pl.P;
  p.scale_log2 = kScaleLog2;
  const size_t q_rows = (size_t)n_q * Hq;
  for (int b0 = 0; b0 < B; b0 += pl.batch) {
    p.B = B - b0 < pl.batch ? B - b0 : pl.batch;
    p.q = (const uint16_t*)q + (size_t)b0 * q_rows * 128;
    p.out = (uint16_t*)out + (size_t)b0 * q_rows * 128;
    p.lse = lse ? lse + (size_t)b0 * q_rows : nullptr;
    p.block_table = block_table + (size_t)b0 * max_blocks_per_seq;
    p.ctx_lens = ctx_lens + b0;
    p.windows = windows ? windows + b0 : nullptr;
    hipError_t e = rattn::launch_decode(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(RATTN_ERR_HIP, "rattn_decode_paged: launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // extern "C"
