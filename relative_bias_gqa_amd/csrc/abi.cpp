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

// ---- paged-decode split plan ---------------------------------------------------------
struct DecodePlan {
  int gs, n_hs, rows, S, SB;
  size_t o_bytes, lse_off, total;
};

bool plan_decode(int B, int n_q, int Hq, int Hkv, int max_ctx_len, int num_splits, DecodePlan* pl) {
  if (B < 0 || n_q < 1 || n_q > rattn::kDecodeMaxRows || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      max_ctx_len < 1 || max_ctx_len > kMaxPosition || num_splits < 0)
    return false;
  const int G = Hq / Hkv;
  // query heads per workgroup: as many of the group as fit the row and bias-slice limits
  int gs = 1;
  for (int d = G; d >= 1; --d) {
    if (G % d != 0) continue;
    if (n_q * d <= rattn::kDecodeMaxRows && d * (127 + n_q) <= rattn::kDecodeBiasFloats) {
      gs = d;
      break;
    }
  }
  const int rows = n_q * gs;
  const int n_hs = G / gs;
  const long long max_blocks = (max_ctx_len + 127) / 128;
  long long SB;
  if (num_splits > 0) {
    const long long S = num_splits < max_blocks ? num_splits : max_blocks;
    SB = (max_blocks + S - 1) / S;
  } else {
    // (a) each split reads at least 64x the bytes of partial results it writes
    //     (rows x 129 floats against SB blocks of 32 KB K + 32 KB V);
    // (b) the grid offers about 8192 workgroups at the longest context.
    const long long min_sb = ((long long)rows * 129 * 4 * 64 + 65535) / 65536;
    const long long fill_sb = ((long long)B * Hkv * n_hs * max_blocks + 8191) / 8192;
    SB = min_sb > fill_sb ? min_sb : fill_sb;
    if (SB < 1) SB = 1;
  }
  const long long S = (max_blocks + SB - 1) / SB;
  const long long nrows = (long long)B * n_q * Hq;
  const long long grid = (long long)B * Hkv * n_hs * S;
  if (grid > 0x7fffffffLL || nrows > 0x7fffffffLL) return false;
  pl->gs = gs;
  pl->n_hs = n_hs;
  pl->rows = rows;
  pl->S = (int)S;
  pl->SB = (int)SB;
  pl->o_bytes = (size_t)nrows * (size_t)S * 128 * sizeof(float);
  pl->lse_off = (pl->o_bytes + 255) & ~(size_t)255;
  pl->total = pl->lse_off + (size_t)nrows * (size_t)S * sizeof(float);
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
  if (!plan_decode(B, n_q, Hq, Hkv, max_ctx_len, num_splits, &pl)) return 0;
  return pl.S;
}

size_t rattn_decode_workspace_bytes(int B, int n_q, int Hq, int Hkv, int max_ctx_len, int num_splits) {
  DecodePlan pl;
  if (!plan_decode(B, n_q, Hq, Hkv, max_ctx_len, num_splits, &pl)) return 0;
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
  if (!plan_decode(B, n_q, Hq, Hkv, max_ctx_len, num_splits, &pl))
    return fail(RATTN_ERR_INVALID_ARG, "rattn_decode_paged: problem too large for one launch");
  if (!workspace || workspace_bytes < pl.total)
    return fail(RATTN_ERR_WORKSPACE, "rattn_decode_paged: workspace %zu bytes at %p, need %zu", workspace_bytes,
                workspace, pl.total);

  rattn::DecodeParams p;
  p.q = (const uint16_t*)q;
  p.k_cache = (const uint16_t*)k_cache;
  p.v_cache = (const uint16_t*)v_cache;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.windows = windows;
  p.bias = bias;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.ws_o = (float*)workspace;
  p.ws_lse = (float*)((char*)workspace + pl.lse_off);
  p.B = B;
  p.n_q = n_q;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.R = R;
  p.num_blocks = num_blocks;
  p.mbps = max_blocks_per_seq;
  p.G = Hq / Hkv;
  p.gs = pl.gs;
  p.n_hs = pl.n_hs;
  p.rows = pl.rows;
  p.S = pl.S;
  p.SB = pl.SB;
  p.scale_log2 = kScaleLog2;
  hipError_t e = rattn::launch_decode(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RATTN_ERR_HIP, "rattn_decode_paged: launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
