// abi.cpp -- the C-ABI entry points declared in include/rattn.h.
//
// Host-side only: argument validation (always before any HIP call), the work
// decomposition of each launch, the split plan of the paged decode, and the thread-local
// error message.  No allocation and no synchronisation happen here: every call enqueues
// its kernels on the caller's stream and returns.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <functional>
#include <queue>
#include <vector>

#include "backward.hpp"
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

// compute units of the current device (queried once per device; 256, an MI355X's count,
// when no device answers)
int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---- paged-decode plan ---------------------------------------------------------------
// Segment = (sequence, KV head, subgroup of gs query heads); rows = n_q * gs.  The unit
// stream (64-token units of every segment) is divided among P workgroups; sequences are
// processed in launches of at most `batch` sequences, each reusing the same workspace.
// The default P is one workgroup per compute unit of the current device.

struct DecodePlan {
  int gs, n_hs, KH, rows, SL, P, batch, KS, NW;
  size_t lse_off, total;
};

bool plan_decode(int B, int n_q, int Hq, int Hkv, int max_ctx_len, int max_blocks, int num_splits, DecodePlan* pl) {
  if (B < 1 || n_q < 1 || n_q > rattn::kDecodeMaxRows || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      max_ctx_len < 1 || max_ctx_len > kMaxPosition || max_blocks < 1 || num_splits < 0)
    return false;
  const int G = Hq / Hkv;
  const int SL = rattn::kDecodeUnit - 1 + n_q;
  // query heads per segment: the largest divisor of G whose rows fit four 32-row blocks and whose
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
  const int P = num_splits > 0 ? num_splits : compute_units();
  const long long rows = (long long)n_q * gs;
  // the two 32-key halves of a unit go to different waves, one wave per (32-row block, key
  // half): four waves up to two row blocks, eight (two per SIMD) up to four
  const int KS = 2;
  const int NW = rows <= 64 ? 4 : 8;
  const long long slots = (P + batch * KH) * KS;
  if (batch * KH * rows * rattn::kDecodeMergeSlices > 0x7fffffffLL) return false;
  pl->gs = gs;
  pl->n_hs = n_hs;
  pl->KH = (int)KH;
  pl->rows = (int)rows;
  pl->SL = SL;
  pl->P = P;
  pl->batch = (int)batch;
  pl->KS = KS;
  pl->NW = NW;
  const size_t o_bytes = (size_t)slots * (size_t)rows * 128 * sizeof(float);
  pl->lse_off = (o_bytes + 255) & ~(size_t)255;
  pl->total = pl->lse_off + (size_t)slots * (size_t)rows * sizeof(float);
  return true;
}

// ---- prefill work decomposition and key-range split plan -----------------------------
// A workgroup takes one KV head, hpw of its query heads and 32 * tsub tokens (hpw * tsub
// = 8 waves).  Workgroups go to compute units in index order as units free up, heaviest
// token tiles first.  When the heaviest tiles are long compared with a unit's share of the
// work (a sliding window: every tile past the window costs the same), the last ones to
// start finish late; splitting the key range of the heaviest tiles into `parts` pieces,
// merged through the workspace, evens this out.  The plan simulates the in-order dispatch
// for the grid without a split and for a few splits and keeps the fastest.
void prefill_shape(int B, int Lq, int Lk, int Hq, int Hkv, int window, rattn::PrefillParams* p) {
  p->B = B;
  p->Lq = Lq;
  p->Lk = Lk;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->window = window > 0 ? window : 0;
  p->G = Hq / Hkv;
  p->hpw = largest_divisor_at_most(p->G, 8);
  while (8 % p->hpw != 0) p->hpw = largest_divisor_at_most(p->G, p->hpw - 1);
  p->tsub = 8 / p->hpw;
  p->n_hg = p->G / p->hpw;
  p->n_tok_tiles = (Lq + 32 * p->tsub - 1) / (32 * p->tsub);
  p->n_split = 0;
  p->parts = 1;
  p->ws_o = nullptr;
  p->ws_lse = nullptr;
  p->ws_cnt = nullptr;
  p->queue = nullptr;
  p->queue_workgroups = 0;
  p->block_table = nullptr;
  p->ctx_lens = nullptr;
  p->cu_q = nullptr;
  p->mbps = 0;
  p->num_blocks = 0;
  p->bias_tok = nullptr;
}

// 64-key tiles walked by token tile `tile` (the same range as the kernel computes)
int prefill_tile_keys(const rattn::PrefillParams& p, int tile) {
  const long long rows = 32LL * p.tsub, off = (long long)p.Lk - p.Lq;
  const long long T0 = tile * rows, T1 = std::min<long long>(p.Lq, T0 + rows);
  const long long weff = p.window > 0 ? p.window : (1LL << 30);
  const long long kb = std::max(0LL, off + T0 - weff + 1) / 64, ke = (off + T1 - 1) / 64 + 1;
  return (int)(ke - kb);
}

// Workspace of a bf16 prefill: [256 B: job queue] [256 KB: split counters] [partial lse]
// [partial O].  The counters sit at the same place for every plan, so a workspace reused
// by calls of different plans never finds one call's partial results under another's
// counters (which must start at zero; every call leaves the queue and counters at zero).
struct PrefillSplit {
  int n_split = 0, parts = 1, n_big = 0;
  size_t cnt_off = 0, lse_off = 0, o_off = 0, ws_bytes = 0;
};
constexpr size_t kQueueBytes = 256;
constexpr size_t kCounterBytes = 256 * 1024;
constexpr long long kMaxSplitJobs = kCounterBytes / sizeof(int);

// With a queue, a launch has one workgroup per compute unit and each takes the next job
// slot when it finishes one: the plan simulates that on the compute units of the device.
// fixed costs in key-tile times: a job's start (Q and the first tiles in flight) and
// output; a piece's, including writing its partial and its share of the merge (measured
// per job on sliding-window prefill on an MI355X: ~3 tile-times in the piece itself; the
// rest stands for what the simulation leaves out -- partial-store and merge traffic of
// concurrent pieces -- fitted so the plan matches the fastest measured split counts)
constexpr double kWgOverhead = 1.5;
constexpr double kPieceOverhead = 7.0;

// finish time of the last job, jobs started in order on the least-loaded unit
double simulate_dispatch(const std::vector<double>& jobs, int n_units) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> units;
  for (int i = 0; i < n_units; ++i) units.push(0.0);
  double end = 0.0;
  for (double j : jobs) {
    const double t = units.top() + j;
    units.pop();
    units.push(t);
    end = std::max(end, t);
  }
  return end;
}

PrefillSplit split_layout(const rattn::PrefillParams& p, int n_split, int parts) {
  PrefillSplit sp;
  sp.cnt_off = kQueueBytes;
  sp.ws_bytes = kQueueBytes;
  if (n_split <= 0 || parts < 2) return sp;
  sp.n_split = n_split;
  sp.parts = parts;
  const size_t per_tile = (size_t)p.B * p.Hkv * p.n_hg;
  const size_t jobs = (size_t)n_split * per_tile, pieces = jobs * parts;
  sp.lse_off = sp.cnt_off + kCounterBytes;
  sp.o_off = (sp.lse_off + pieces * 256 * sizeof(float) + 255) & ~(size_t)255;
  sp.ws_bytes = sp.o_off + pieces * 256 * 128 * sizeof(float);
  return sp;
}

PrefillSplit plan_prefill_split_uncached(const rattn::PrefillParams& p, int dtype, int kv_splits, int n_units) {
  if (dtype != RATTN_BF16) return PrefillSplit{};
  if (kv_splits == 1) return split_layout(p, 0, 1);
  const int nt = p.n_tok_tiles;
  std::vector<int> keys(nt);
  for (int t = 0; t < nt; ++t) keys[t] = prefill_tile_keys(p, t);  // non-decreasing in t
  const long long per_tile = (long long)p.B * p.Hkv * p.n_hg;
  const int max_split = (int)std::min<long long>(nt, kMaxSplitJobs / per_tile);  // counters
  // Job order: the unsplit tiles longer than the longest piece, the pieces, the other
  // unsplit tiles (each list from the heaviest down), so the queue starts the longest
  // jobs first.
  auto big_of = [&](int n_split, int parts) {
    if (n_split == 0) return 0;
    const int longest_piece = (keys[nt - 1] + parts - 1) / parts;
    int n_big = 0;
    while (n_split + n_big < nt && keys[nt - 1 - n_split - n_big] > longest_piece) ++n_big;
    return n_big;
  };
  if (kv_splits >= 2) {
    // split every token tile with at least 2 * kv_splits key tiles (the heaviest ones
    // while the counters last)
    int n_split = 0;
    while (n_split < max_split && keys[nt - 1 - n_split] >= 2 * kv_splits) ++n_split;
    PrefillSplit sp = split_layout(p, n_split, kv_splits);
    sp.n_big = big_of(n_split, kv_splits);
    return sp;
  }
  if ((long long)nt * per_tile * rattn::kMaxPieces > 0x7fffffffLL) return split_layout(p, 0, 1);
  // job sizes in queue order, pieces mapped to slots as the kernel does
  auto jobs_of = [&](int n_split, int parts) {
    std::vector<double> jobs;
    const int n_big = big_of(n_split, parts);
    for (int t = nt - 1 - n_split; t >= nt - n_split - n_big; --t)
      for (long long r = 0; r < per_tile; ++r) jobs.push_back(keys[t] + kWgOverhead);
    const long long n_jobs = (long long)n_split * per_tile;
    for (long long w = 0; w < n_jobs * parts; ++w) {
      int job, piece;
      rattn::prefill_piece_of(w, n_jobs, parts, &job, &piece);
      const int k = keys[nt - 1 - (int)(job / per_tile)];
      jobs.push_back(k * (piece + 1) / parts - k * piece / parts + kPieceOverhead);
    }
    for (int t = nt - 1 - n_split - n_big; t >= 0; --t)
      for (long long r = 0; r < per_tile; ++r) jobs.push_back(keys[t] + kWgOverhead);
    return jobs;
  };
  double total = 0.0;
  for (int t = 0; t < nt; ++t) total += (keys[t] + kWgOverhead) * per_tile;
  double best = simulate_dispatch(jobs_of(0, 1), n_units);
  // a grid that already finishes within 5 % of an even spread is left alone
  if (best <= 1.05 * total / n_units) return split_layout(p, 0, 1);
  int best_split = 0, best_parts = 1;
  // candidates: the tiles with at least some number of key tiles (2 parts, and fractions
  // of the longest), and the heaviest n tiles for n a multiple of nt / 16 (the tiles of a
  // sliding-window prefill past its window all have the same length, and splitting only
  // some of them can balance better than splitting all)
  const int kmax = keys[nt - 1];
  std::vector<int> counts;
  for (int frac = 0; frac <= 3; ++frac) {
    const int thr = std::max(4, kmax * frac / 4);
    int n_split = 0;
    while (n_split < nt && keys[nt - 1 - n_split] >= thr) ++n_split;
    counts.push_back(n_split);
  }
  for (int k = 1; k <= 16; ++k) counts.push_back((int)((long long)nt * k / 16));
  // the fastest split plan (within 0.5 %, the one with fewer pieces), if it beats the
  // unsplit launch by at least 3 %
  double best_m = 0.0;
  long long best_pieces = 0;
  for (int parts = 2; parts <= 4; ++parts)
    for (int n_split : counts) {
      n_split = std::min(n_split, max_split);
      while (n_split > 0 && keys[nt - n_split] < 2 * parts) --n_split;  // pieces of >= 2 key tiles
      if (n_split == 0) continue;
      const double m = simulate_dispatch(jobs_of(n_split, parts), n_units);
      const long long pieces = (long long)n_split * parts;
      if (best_split == 0 || m < 0.995 * best_m || (m <= 1.005 * best_m && pieces < best_pieces)) {
        best_m = m;
        best_pieces = pieces;
        best_split = n_split;
        best_parts = parts;
      }
    }
  if (best_split == 0 || best_m >= 0.97 * best) return split_layout(p, 0, 1);
  PrefillSplit sp = split_layout(p, best_split, best_parts);
  sp.n_big = big_of(best_split, best_parts);
  return sp;
}


// the plan of the last few shapes (calls repeat their shapes)
PrefillSplit plan_prefill_split(const rattn::PrefillParams& p, int dtype, int kv_splits) {
  struct Entry {
    int key[9];
    PrefillSplit plan;
  };
  thread_local Entry cache[8];
  thread_local int filled = 0, next = 0;
  const int n_units = compute_units();
  const int key[9] = {p.B, p.Lq, p.Lk, p.Hq, p.Hkv, p.window, dtype, kv_splits, n_units};
  for (int i = 0; i < filled; ++i)
    if (std::equal(key, key + 9, cache[i].key)) return cache[i].plan;
  const PrefillSplit sp = plan_prefill_split_uncached(p, dtype, kv_splits, n_units);
  std::copy(key, key + 9, cache[next].key);
  cache[next].plan = sp;
  next = (next + 1) % 8;
  filled = std::min(filled + 1, 8);
  return sp;
}

}  // namespace

extern "C" {

const char* rattn_last_error(void) { return g_err; }

int rattn_abi_version(void) { return RATTN_ABI_VERSION; }

}  // extern "C"

namespace {

// Contiguous prefill with the per-head table (bias [Hq, R] fp32, bias_tok null) or the
// token-dependent one (bias_tok [B, Lq, Hq, R] bf16, bias null).
int prefill_contiguous(const char* fn, bool token, const void* q, const void* k, const void* v, const float* bias,
                       const void* bias_tok, void* out, float* lse, int B, int Lq, int Lk, int Hq, int Hkv,
                       int head_dim, int R, int window, int dtype, int kv_splits, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (B < 0 || Lq < 0 || Lk < 0 || Hq < 0 || Hkv < 0)
    return fail(RATTN_ERR_INVALID_ARG, "%s: negative size (B=%d Lq=%d Lk=%d Hq=%d Hkv=%d)", fn, B, Lq, Lk, Hq,
                Hkv);
  if (head_dim != 128) return fail(RATTN_ERR_UNSUPPORTED, "%s: head_dim %d (only 128)", fn, head_dim);
  if (dtype != RATTN_BF16 && dtype != RATTN_FP32) return fail(RATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (kv_splits < 0 || kv_splits > rattn::kMaxPieces)
    return fail(RATTN_ERR_INVALID_ARG, "%s: kv_splits=%d outside 0..%d", fn, kv_splits, rattn::kMaxPieces);
  if (B == 0 || Lq == 0) return ok();
  if (!q || !k || !v || !(token ? bias_tok : (const void*)bias) || !out)
    return fail(RATTN_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(RATTN_ERR_INVALID_ARG, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, Hq, Hkv);
  if (Lq > Lk) return fail(RATTN_ERR_INVALID_ARG, "%s: Lq=%d > Lk=%d", fn, Lq, Lk);
  if (Lk > kMaxPosition) return fail(RATTN_ERR_INVALID_ARG, "%s: Lk=%d too large", fn, Lk);
  if (R < 1) return fail(RATTN_ERR_INVALID_ARG, "%s: R=%d < 1", fn, R);
  if (token) {
    if (R < 4) return fail(RATTN_ERR_UNSUPPORTED, "%s: R=%d (the token-dependent table needs R >= 4)", fn, R);
    if (((uintptr_t)bias_tok & 3) != 0)
      return fail(RATTN_ERR_INVALID_ARG, "%s: bias_tok must be 4-byte aligned", fn);
    if ((long long)B * Lq * Hq * (long long)R > 0x3fffffffffffLL)
      return fail(RATTN_ERR_INVALID_ARG, "%s: token table too large", fn);
  }
  if (workspace == nullptr && workspace_bytes != 0)
    return fail(RATTN_ERR_INVALID_ARG, "%s: workspace_bytes=%zu with a null workspace", fn, workspace_bytes);

  rattn::PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.bias = bias;
  p.out = out;
  p.lse = lse;
  p.R = R;
  prefill_shape(B, Lq, Lk, Hq, Hkv, window, &p);
  p.bias_tok = (const uint16_t*)bias_tok;
  p.scale_log2 = kScaleLog2;
  // no workspace: one workgroup per job, never split
  const PrefillSplit sp = workspace == nullptr ? PrefillSplit{} : plan_prefill_split(p, dtype, kv_splits);
  if (sp.ws_bytes > workspace_bytes)
    return fail(RATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, sp.ws_bytes);
  p.n_split = sp.n_split;
  p.n_big = sp.n_big;
  p.parts = sp.parts;
  p.queue = sp.ws_bytes ? (int*)workspace : nullptr;
  p.queue_workgroups = p.queue ? compute_units() : 0;
  p.ws_cnt = sp.ws_bytes ? (int*)((char*)workspace + sp.cnt_off) : nullptr;
  p.ws_lse = sp.n_split ? (float*)((char*)workspace + sp.lse_off) : nullptr;
  p.ws_o = sp.n_split ? (float*)((char*)workspace + sp.o_off) : nullptr;
  const long long per_tile = (long long)B * Hkv * p.n_hg;
  const long long grid = ((long long)p.n_tok_tiles - p.n_split) * per_tile + (long long)p.n_split * per_tile * p.parts;
  if (grid > 0x7fffffffLL) return fail(RATTN_ERR_INVALID_ARG, "%s: problem too large for one launch", fn);

  hipError_t e = dtype == RATTN_BF16 ? rattn::launch_prefill_bf16(p, (hipStream_t)stream)
                                     : rattn::launch_prefill_fp32(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int rattn_prefill(const void* q, const void* k, const void* v, const float* bias, void* out,
                  float* lse, int B, int Lq, int Lk, int Hq, int Hkv, int head_dim, int R,
                  int window, int dtype, int kv_splits, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return prefill_contiguous("rattn_prefill", false, q, k, v, bias, nullptr, out, lse, B, Lq, Lk, Hq, Hkv, head_dim, R,
                            window, dtype, kv_splits, workspace, workspace_bytes, stream);
}

int rattn_prefill_tokbias(const void* q, const void* k, const void* v, const void* bias_tok, void* out,
                          float* lse, int B, int Lq, int Lk, int Hq, int Hkv, int head_dim, int R,
                          int window, int kv_splits, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return prefill_contiguous("rattn_prefill_tokbias", true, q, k, v, nullptr, bias_tok, out, lse, B, Lq, Lk, Hq, Hkv,
                            head_dim, R, window, RATTN_BF16, kv_splits, workspace, workspace_bytes, stream);
}

int rattn_prefill_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                        const int* ctx_lens, const int* cu_seqlens_q, const float* bias, void* out, float* lse,
                        int B, int Lq, int Hq, int Hkv, int head_dim, int block_size, int R, int window,
                        int num_blocks,
                        int max_blocks_per_seq, int max_ctx_len, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (B < 0 || Lq < 0 || Hq < 0 || Hkv < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_ctx_len < 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: negative size");
  if (head_dim != 128) return fail(RATTN_ERR_UNSUPPORTED, "rattn_prefill_paged: head_dim %d (only 128)", head_dim);
  if (block_size != 128)
    return fail(RATTN_ERR_UNSUPPORTED, "rattn_prefill_paged: block_size %d (only 128)", block_size);
  if (B == 0 || Lq == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !bias || !out)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: null pointer argument");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: Hq=%d must be a positive multiple of Hkv=%d", Hq,
                Hkv);
  if (R < 1) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: R=%d < 1", R);
  if (num_blocks < 1 || max_blocks_per_seq < 1)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: num_blocks=%d, max_blocks_per_seq=%d", num_blocks,
                max_blocks_per_seq);
  if (max_ctx_len < Lq)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: max_ctx_len=%d < Lq=%d", max_ctx_len, Lq);
  if ((long long)max_ctx_len > 128LL * max_blocks_per_seq || max_ctx_len > kMaxPosition)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: max_ctx_len=%d exceeds the block table (%d blocks)",
                max_ctx_len, max_blocks_per_seq);
  if (workspace == nullptr && workspace_bytes != 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: workspace_bytes=%zu with a null workspace",
                workspace_bytes);
  if (workspace != nullptr && workspace_bytes < RATTN_PREFILL_PAGED_WORKSPACE_BYTES)
    return fail(RATTN_ERR_WORKSPACE, "rattn_prefill_paged: workspace of %zu bytes, %d needed", workspace_bytes,
                RATTN_PREFILL_PAGED_WORKSPACE_BYTES);

  rattn::PrefillParams p;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.bias = bias;
  p.out = out;
  p.lse = lse;
  p.R = R;
  prefill_shape(B, Lq, max_ctx_len, Hq, Hkv, window, &p);
  p.scale_log2 = kScaleLog2;
  p.n_big = 0;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.cu_q = cu_seqlens_q;
  p.mbps = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  // with a workspace: the job queue (one workgroup per compute unit), else one per job
  p.queue = workspace != nullptr ? (int*)workspace : nullptr;
  p.queue_workgroups = p.queue ? compute_units() : 0;
  const long long grid = (long long)p.n_tok_tiles * B * Hkv * p.n_hg;
  if (grid > 0x7fffffffLL) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_paged: problem too large for one launch");
  hipError_t e = rattn::launch_prefill_bf16(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RATTN_ERR_HIP, "rattn_prefill_paged: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int rattn_kv_sconv_write(const void* k_new, const void* v_new, const float* w_k, const float* w_v, void* k_cache,
                         void* v_cache, void* k_state, void* v_state, const int* block_table, const int* ctx_lens,
                         const int* cu_seqlens, int B, int Hkv, int head_dim, int block_size, int num_blocks,
                         int max_blocks_per_seq, int max_new, void* stream) {
  if (B < 0 || Hkv < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_new < 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_kv_sconv_write: negative size");
  if (head_dim != 128) return fail(RATTN_ERR_UNSUPPORTED, "rattn_kv_sconv_write: head_dim %d (only 128)", head_dim);
  if (block_size != 128)
    return fail(RATTN_ERR_UNSUPPORTED, "rattn_kv_sconv_write: block_size %d (only 128)", block_size);
  if (Hkv > 8) return fail(RATTN_ERR_UNSUPPORTED, "rattn_kv_sconv_write: Hkv=%d > 8", Hkv);
  if (B == 0 || max_new == 0) return ok();
  if (!k_new || !v_new || !w_k || !w_v || !k_cache || !v_cache || !k_state || !v_state || !block_table ||
      !ctx_lens || !cu_seqlens)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_kv_sconv_write: null pointer argument");
  if (Hkv < 1) return fail(RATTN_ERR_INVALID_ARG, "rattn_kv_sconv_write: Hkv=%d < 1", Hkv);
  if (num_blocks < 1 || max_blocks_per_seq < 1)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_kv_sconv_write: num_blocks=%d, max_blocks_per_seq=%d", num_blocks,
                max_blocks_per_seq);
  if (B > 65535) return fail(RATTN_ERR_INVALID_ARG, "rattn_kv_sconv_write: B=%d > 65535", B);
  rattn::SconvParams p;
  p.k_new = (const uint16_t*)k_new;
  p.v_new = (const uint16_t*)v_new;
  p.w_k = w_k;
  p.w_v = w_v;
  p.k_cache = (uint16_t*)k_cache;
  p.v_cache = (uint16_t*)v_cache;
  p.k_state = (uint16_t*)k_state;
  p.v_state = (uint16_t*)v_state;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.cu = cu_seqlens;
  p.B = B;
  p.Hkv = Hkv;
  p.mbps = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.max_new = max_new;
  hipError_t e = rattn::launch_sconv_write(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RATTN_ERR_HIP, "rattn_kv_sconv_write: launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Backward workspace: D and lse * log2(e) per query row ([B, Hq, Lq] each), then the partial
// dK and dV of each pair of query heads for each of the (at most) two query-step chunks of a
// key block ([2, ceil(G / 2), B, Lk, Hkv, 128] each), then the second key-tile chunk's dq
// ([B, Lq, Hq, 128]); each part 256-aligned.
struct BackwardLayout {
  size_t l2_off, pk_off, pv_off, dqp_off, bias_off, cnt_off, total;
  int n_pairs;
};

bool backward_layout(int B, int Lq, int Lk, int Hq, int Hkv, BackwardLayout* lay) {
  if (B < 0 || Lq < 0 || Lk < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return false;
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)B * Lq * Hq;
  const size_t plane = (size_t)B * Lk * Hkv * 128;
  lay->n_pairs = (Hq / Hkv + 1) / 2;
  lay->l2_off = align(rows * sizeof(float));
  lay->pk_off = lay->l2_off + align(rows * sizeof(float));
  lay->pv_off = lay->pk_off + align(2 * (size_t)lay->n_pairs * plane * sizeof(float));
  lay->dqp_off = lay->pv_off + align(2 * (size_t)lay->n_pairs * plane * sizeof(float));
  // the dq pass's split partials: two slots per unit (256 query x head rows of 128 fp32 each);
  // the units of a chunk cover B * Hq * (Lq rounded up to 256) rows at most
  const size_t unit_rows = (size_t)B * Hq * (((size_t)Lq + 255) / 256 * 256);
  lay->bias_off = lay->dqp_off + align(2 * unit_rows * 128 * sizeof(float));
  lay->cnt_off = lay->bias_off + align((size_t)Hq * Lk * sizeof(float));
  // counters of the dq pass's split token tiles: at most one per 32 queries and query head
  lay->total = std::max<size_t>(256, lay->cnt_off + align((size_t)B * Hq * ((Lq + 31) / 32) * sizeof(int)));
  return true;
}

// Query steps (32-query tiles) that see key block blk of the key-stationary pass, key tiles
// (32 keys) that token tile t of the query-stationary pass walks; the kernels' counts.
long long bwd_kv_block_steps(int Lq, int Lk, int window, int blk) {
  const long long off = (long long)Lk - Lq, weff = window > 0 ? window : 0x40000000LL;
  const long long J0 = 128LL * blk, q_lo = std::max(0LL, J0 - off);
  const long long q_hi = std::min((long long)Lq - 1, J0 + 127 + weff - 1 - off);
  return q_lo <= q_hi ? q_hi / 32 - q_lo / 32 + 1 : 0;
}

// Makespan of a launch whose units (in launch order) take w[i] (in steps), for the way the
// hardware hands out workgroups: workgroup i to XCD i % 8, within it to shader engine
// (i / 8) % 4, and to whichever compute unit of that engine frees up first.  A model used
// only to choose between plans.
double dispatch_makespan(const std::vector<double>& w, int cus) {
  const int per_pool = std::max(1, cus / 32);
  std::vector<std::priority_queue<double, std::vector<double>, std::greater<double>>> pools(32);
  for (auto& q : pools)
    for (int c = 0; c < per_pool; ++c) q.push(0.0);
  double end = 0.0;
  for (size_t i = 0; i < w.size(); ++i) {
    auto& q = pools[(i % 8) * 4 + (i / 8) % 4];
    const double t = q.top() + w[i];
    q.pop();
    q.push(t);
    end = std::max(end, t);
  }
  return end;
}

struct ChunkPlan {
  int chunks, chunk;
};

// Units of segments with the given walks (in launch order), each repeated `inner` times (head
// groups, KV heads, sequences), cut into `chunks` chunks, chunk-major: a unit weighs its steps
// plus the steps it spends on loads before its first one, times `cost`.
std::vector<double> chunk_units(const std::vector<long long>& walk, long long inner, int chunks, double cost) {
  long long most = 1;
  for (long long x : walk) most = std::max(most, x);
  const long long chunk = (most + chunks - 1) / chunks;
  const double overhead = 3.0;
  std::vector<double> w;
  w.reserve(walk.size() * chunks * inner);
  for (int c = 0; c < chunks; ++c)
    for (long long x : walk) {
      const long long steps = std::max(0LL, std::min(chunk, x - c * chunk));
      const double t = steps > 0 ? (double)steps + overhead : (c == 0 ? overhead : 0.1);
      for (long long g = 0; g < inner; ++g) w.push_back(t * cost);
    }
  return w;
}

ChunkPlan chunk_plan(const std::vector<long long>& walk, int chunks) {
  long long most = 1;
  for (long long x : walk) most = std::max(most, x);
  return ChunkPlan{chunks, (int)std::min<long long>((most + chunks - 1) / chunks, 0x7fffffff)};
}

// One or two chunks per segment of each of the two passes of one grid (the key-stationary
// units `a` first, then the query-stationary ones `b`; a step of `a` costs `cost_a` steps of
// `b`): the plan that the dispatch model finishes first.
void plan_chunks_joint(const std::vector<long long>& wa, long long inner_a, double cost_a,
                       const std::vector<long long>& wb, long long inner_b, ChunkPlan* pa, ChunkPlan* pb) {
  *pa = chunk_plan(wa, 1);
  *pb = chunk_plan(wb, 1);
  if (wa.empty() || wb.empty() || inner_a <= 0 || inner_b <= 0 ||
      (double)wa.size() * inner_a + (double)wb.size() * inner_b > 4e6)
    return;
  double best_t = 0.0;
  for (int ca = 1; ca <= 2; ++ca)
    for (int cb = 1; cb <= 2; ++cb) {
      std::vector<double> w = chunk_units(wa, inner_a, ca, cost_a);
      const std::vector<double> b = chunk_units(wb, inner_b, cb, 1.0);
      w.insert(w.end(), b.begin(), b.end());
      const double t = dispatch_makespan(w, compute_units());
      if ((ca == 1 && cb == 1) || t < best_t) {
        best_t = t;
        *pa = chunk_plan(wa, ca);
        *pb = chunk_plan(wb, cb);
      }
    }
}

long long bwd_dq_tile_keys(int Lq, int Lk, int window, int tsub, int t) {
  const long long off = (long long)Lk - Lq, weff = window > 0 ? window : 0x40000000LL;
  const long long T0 = 32LL * tsub * t, T1 = std::min<long long>(Lq, T0 + 32LL * tsub);
  return (off + T1 - 1) / 32 + 1 - std::max(0LL, off + T0 - weff + 1) / 32;
}

}  // namespace

extern "C" {

size_t rattn_prefill_backward_workspace_bytes(int B, int Lq, int Lk, int Hq, int Hkv) {
  BackwardLayout lay;
  return backward_layout(B, Lq, Lk, Hq, Hkv, &lay) ? lay.total : 0;
}

int rattn_prefill_backward(const void* q, const void* k, const void* v, const float* bias, const void* out,
                           const void* dout, const float* lse, float* dq, float* dk, float* dv, float* dbias, int B,
                           int Lq, int Lk, int Hq, int Hkv, int head_dim, int R, int window, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (B < 0 || Lq < 0 || Lk < 0 || Hq < 0 || Hkv < 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_backward: negative size (B=%d Lq=%d Lk=%d Hq=%d Hkv=%d)", B,
                Lq, Lk, Hq, Hkv);
  if (head_dim != 128)
    return fail(RATTN_ERR_UNSUPPORTED, "rattn_prefill_backward: head_dim %d (only 128)", head_dim);
  if (!q || !k || !v || !bias || !out || !dout || !lse || !dq || !dk || !dv || !dbias)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_backward: null pointer argument");
  if (Hkv < 1 || Hq < Hkv || Hq % Hkv != 0)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_backward: Hq=%d must be a positive multiple of Hkv=%d", Hq,
                Hkv);
  if (Lq > Lk) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_backward: Lq=%d > Lk=%d", Lq, Lk);
  if (Lk > kMaxPosition) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_backward: Lk=%d too large", Lk);
  if (R < 1) return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_backward: R=%d < 1", R);
  if (B > 65535 || Hq > 65535)
    return fail(RATTN_ERR_INVALID_ARG, "rattn_prefill_backward: B=%d or Hq=%d > 65535", B, Hq);
  BackwardLayout lay;
  backward_layout(B, Lq, Lk, Hq, Hkv, &lay);
  const size_t need = lay.total;
  if (!workspace || workspace_bytes < need)
    return fail(RATTN_ERR_WORKSPACE, "rattn_prefill_backward: workspace of %zu bytes, %zu needed",
                workspace ? workspace_bytes : (size_t)0, need);
  rattn::BackwardParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.bias = bias;
  p.out = out;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dbias = dbias;
  p.D = (float*)workspace;
  p.L2 = (float*)((char*)workspace + lay.l2_off);
  p.part_dk = (float*)((char*)workspace + lay.pk_off);
  p.part_dv = (float*)((char*)workspace + lay.pv_off);
  p.dq_part = (float*)((char*)workspace + lay.dqp_off);
  p.bias_s = (float*)((char*)workspace + lay.bias_off);
  p.dq_cnt = (int*)((char*)workspace + lay.cnt_off);
  p.Rs = std::min(R, Lk);
  p.n_pairs = lay.n_pairs;
  {
    rattn::PrefillParams shape;  // the forward's head / token grouping
    prefill_shape(B, Lq, Lk, Hq, Hkv, window, &shape);
    p.hpw = shape.hpw;
    p.tsub = shape.tsub;
    p.n_hg = shape.n_hg;
    p.n_tok_tiles = shape.n_tok_tiles;
  }
  {
    // walk of every key block / token tile, then one or two chunks each, whichever plan the
    // dispatch model finishes sooner for the two passes' grid (a key-stationary step and a
    // query-stationary one both cover 8192 query-key pairs; the first takes about 1.1 times
    // as long)
    ChunkPlan kv, qp;
    // the plans of the last few shapes (training repeats its shapes; a plan simulates every unit)
    struct Entry {
      int key[7];
      ChunkPlan kv, qp;
    };
    thread_local Entry cache[8];
    thread_local int filled = 0, next = 0;
    const int key[7] = {B, Lq, Lk, Hq, Hkv, window, compute_units()};
    int hit = -1;
    for (int i = 0; i < filled && hit < 0; ++i)
      if (std::equal(key, key + 7, cache[i].key)) hit = i;
    if (hit >= 0) {
      kv = cache[hit].kv;
      qp = cache[hit].qp;
    } else {
      const int n_blk = (Lk + 127) / 128;
      std::vector<long long> kw(n_blk), qw(p.n_tok_tiles);
      for (int blk = 0; blk < n_blk; ++blk) kw[blk] = bwd_kv_block_steps(Lq, Lk, window, blk);
      for (int t = 0; t < p.n_tok_tiles; ++t) qw[p.n_tok_tiles - 1 - t] = bwd_dq_tile_keys(Lq, Lk, window, p.tsub, t);
      plan_chunks_joint(kw, (long long)B * Hkv * lay.n_pairs, 1.1, qw, (long long)B * Hkv * p.n_hg, &kv, &qp);
      std::copy(key, key + 7, cache[next].key);
      cache[next].kv = kv;
      cache[next].qp = qp;
      next = (next + 1) % 8;
      filled = std::min(filled + 1, 8);
    }
    p.kv_chunks = kv.chunks;
    p.kv_chunk = kv.chunk;
    p.q_chunks = qp.chunks;
    p.q_chunk = qp.chunk;
  }
  p.B = B;
  p.Lq = Lq;
  p.Lk = Lk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.R = R;
  p.window = window;
  p.scale_log2 = kScaleLog2;
  const hipError_t e = rattn::launch_backward(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RATTN_ERR_HIP, "rattn_prefill_backward: launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t rattn_prefill_workspace_bytes(int B, int Lq, int Lk, int Hq, int Hkv, int window, int dtype,
                                     int kv_splits) {
  if (B < 1 || Lq < 1 || Lk < Lq || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Lk > kMaxPosition ||
      (dtype != RATTN_BF16 && dtype != RATTN_FP32) || kv_splits < 0 || kv_splits > rattn::kMaxPieces)
    return 0;
  rattn::PrefillParams p;
  prefill_shape(B, Lq, Lk, Hq, Hkv, window, &p);
  return plan_prefill_split(p, dtype, kv_splits).ws_bytes;
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

}  // extern "C"

namespace {

// The paged decode of both entry points.  from_scratch: the workspace is the device's static
// scratch (looked up after validation), workspace / workspace_bytes are ignored.
int decode_paged(const char* fn, const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                 const int* ctx_lens, const int* windows, const float* bias, void* out, float* lse, int B, int n_q,
                 int Hq, int Hkv, int head_dim, int block_size, int R, int num_blocks, int max_blocks_per_seq,
                 int max_ctx_len, int num_splits, void* workspace, size_t workspace_bytes, bool from_scratch,
                 void* stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_ctx_len < 0 || num_splits < 0)
    return fail(RATTN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (head_dim != 128) return fail(RATTN_ERR_UNSUPPORTED, "%s: head_dim %d (only 128)", fn, head_dim);
  if (block_size != 128) return fail(RATTN_ERR_UNSUPPORTED, "%s: block_size %d (only 128)", fn, block_size);
  if (n_q < 1) return fail(RATTN_ERR_INVALID_ARG, "%s: n_q=%d < 1", fn, n_q);
  if (n_q > rattn::kDecodeMaxRows)
    return fail(RATTN_ERR_UNSUPPORTED, "%s: n_q=%d > %d", fn, n_q, rattn::kDecodeMaxRows);
  if (B == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !bias || !out)
    return fail(RATTN_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(RATTN_ERR_INVALID_ARG, "%s: Hq=%d must be a positive multiple of Hkv=%d", fn, Hq, Hkv);
  if (R < 1) return fail(RATTN_ERR_INVALID_ARG, "%s: R=%d < 1", fn, R);
  if (num_blocks < 1 || max_blocks_per_seq < 1)
    return fail(RATTN_ERR_INVALID_ARG, "%s: num_blocks=%d, max_blocks_per_seq=%d", fn, num_blocks,
                max_blocks_per_seq);
  if (max_ctx_len < n_q) return fail(RATTN_ERR_INVALID_ARG, "%s: max_ctx_len=%d < n_q=%d", fn, max_ctx_len, n_q);
  if ((long long)max_ctx_len > 128LL * max_blocks_per_seq || max_ctx_len > kMaxPosition)
    return fail(RATTN_ERR_INVALID_ARG, "%s: max_ctx_len=%d exceeds the block table (%d blocks)", fn, max_ctx_len,
                max_blocks_per_seq);
  DecodePlan pl;
  if (!plan_decode(B, n_q, Hq, Hkv, max_ctx_len, max_blocks_per_seq, num_splits, &pl))
    return fail(RATTN_ERR_INVALID_ARG, "%s: problem too large for one launch", fn);
  if (from_scratch) {
    if (pl.total > rattn::kDecodeScratchBytes)
      return fail(RATTN_ERR_WORKSPACE,
                  "%s: these sizes need %zu bytes of split scratch, more than the static %zu; use "
                  "rattn_decode_paged with a workspace, or fewer sequences or splits per call",
                  fn, pl.total, rattn::kDecodeScratchBytes);
    const hipError_t e = rattn::decode_scratch(&workspace);
    if (e != hipSuccess) return fail(RATTN_ERR_HIP, "%s: scratch address: %s", fn, hipGetErrorString(e));
    workspace_bytes = rattn::kDecodeScratchBytes;
  }
  if (!workspace || workspace_bytes < pl.total)
    return fail(RATTN_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", fn, workspace_bytes, workspace,
                pl.total);

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
  p.NW = pl.NW;
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
    if (e != hipSuccess) return fail(RATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

int rattn_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                       const int* ctx_lens, const int* windows, const float* bias, void* out, float* lse,
                       int B, int n_q, int Hq, int Hkv, int head_dim, int block_size, int R, int num_blocks,
                       int max_blocks_per_seq, int max_ctx_len, int num_splits, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return decode_paged("rattn_decode_paged", q, k_cache, v_cache, block_table, ctx_lens, windows, bias, out, lse, B,
                      n_q, Hq, Hkv, head_dim, block_size, R, num_blocks, max_blocks_per_seq, max_ctx_len, num_splits,
                      workspace, workspace_bytes, false, stream);
}

size_t rattn_decode_paged_noalloc_max_scratch_bytes(void) { return rattn::kDecodeScratchBytes; }

int rattn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                               const int* ctx_lens, const int* windows, const float* bias, void* out, float* lse,
                               int B, int n_q, int Hq, int Hkv, int head_dim, int block_size, int R, int num_blocks,
                               int max_blocks_per_seq, int max_ctx_len, int num_splits, void* stream) {
  return decode_paged("rattn_decode_paged_noalloc", q, k_cache, v_cache, block_table, ctx_lens, windows, bias, out,
                      lse, B, n_q, Hq, Hkv, head_dim, block_size, R, num_blocks, max_blocks_per_seq, max_ctx_len,
                      num_splits, nullptr, 0, true, stream);
}

}  // extern "C"
