// launch.hpp -- internal interface between the C-ABI host layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rattn {

// Prefill / chunked prefill over contiguous K/V (all sizes already validated).
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const float* bias;
  void* out;
  float* lse;
  int B, Lq, Lk, Hq, Hkv, R, window;
  int G;            // Hq / Hkv
  int hpw;          // query heads per workgroup (divides G, at most 8)
  int tsub;         // 32-token sub-tiles per workgroup (8 / hpw)
  int n_tok_tiles;  // ceil(Lq / (32 * tsub))
  int n_hg;         // G / hpw head groups per KV head
  float scale_log2; // log2(e) / sqrt(128)
  // Key-range split of the heaviest token tiles (bf16 path): the last n_split token tiles
  // are each computed by `parts` workgroups over consecutive shares of their key tiles,
  // which merge through the workspace (n_split = 0, parts = 1: no split).
  int n_split;
  int parts;
  int n_big;      // unsplit token tiles (the heaviest ones) scheduled before the pieces
  float* ws_o;    // [n_split * B * Hkv * n_hg * parts, 256 rows, 128] normalised partials
  float* ws_lse;  // [same, 256 rows] log2-sum-exp of each partial
  int* ws_cnt;    // [n_split * B * Hkv * n_hg] finished pieces; zero between calls
  int* queue;            // [2] job queue and done counter (zero before and after a call), or null
  int queue_workgroups;  // workgroups of a launch with a queue
  // paged K/V (bf16 path, no split, no queue): k / v are caches [num_blocks, 128, Hkv, 128],
  // block_table [B, mbps], ctx_lens [B] keys per sequence (Lk is their maximum); null when
  // K and V are contiguous [B, Lk, Hkv, 128]
  const int* block_table;
  const int* ctx_lens;
  const int* cu_q;  // paged: [B + 1] packed query offsets (q, out, lse [total, Hq, ...]), or null: [B, Lq, ...]
  int mbps;
  int num_blocks;
  // token-dependent table (contiguous bf16 path): bf16 [B, Lq, Hq, R], row (b, t, h) the table
  // of query t, head h (bias unused); null for the per-head table bias [Hq, R]
  const uint16_t* bias_tok;
};

constexpr int kMaxPieces = 8;
constexpr int kMaxSortedSeqs = 1024;  // paged prefill: sequences ordered by context length in LDS

// Piece slot w (< n_jobs * parts) of a split prefill takes piece *piece of job *job.  In
// each group of 8 * parts slots (8 jobs), slot x + 8 k takes piece k of job x: the pieces
// of a job are 8 slots apart, so in the first round of workgroups (workgroup i runs on
// XCD i % 8) they share an XCD, and the merges (done by whichever piece of a job finishes
// last) spread over all XCDs.  A last, partial group keeps the pieces of a job adjacent.
__host__ __device__ inline void prefill_piece_of(long long w, long long n_jobs, int parts, int* job, int* piece) {
  const long long full = n_jobs / 8 * 8 * parts;
  if (w < full) {
    const long long g = w / (8 * parts);
    const int r = (int)(w - g * 8 * parts);
    *job = (int)(g * 8 + r % 8);
    *piece = r / 8;
  } else {
    const long long r = w - full;
    *job = (int)(n_jobs / 8 * 8 + r / parts);
    *piece = (int)(r % parts);
  }
}  // largest `parts` of a prefill key-range split

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream);
hipError_t launch_prefill_fp32(const PrefillParams& p, hipStream_t stream);

// Paged decode (sizes validated by the host).  The visible keys of every (sequence, KV
// head, query-head subgroup) "segment" are cut into 64-token units; the concatenated unit
// stream of the whole batch is divided evenly among P workgroups, each of which writes
// one partial result per segment it touches (slot = workgroup + segment).
struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int* block_table;
  const int* ctx_lens;
  const int* windows;
  const float* bias;
  uint16_t* out;
  float* lse;
  float* ws_o;    // [P + B * KH, KS, rows, 128] partial outputs (normalised per piece)
  float* ws_lse;  // [P + B * KH, KS, rows] partial log2-sum-exp
  int B, n_q, Hq, Hkv, R, mbps;
  int num_blocks; // physical blocks in each cache
  int G;          // Hq / Hkv
  int gs;         // query heads per segment
  int n_hs;       // G / gs
  int KH;         // Hkv * n_hs segments per sequence
  int rows;       // n_q * gs query rows per segment
  int SL;         // bias entries per head staged for one unit: 63 + n_q
  int KS;         // waves sharing a unit's keys: 2, one 32-key half each
  int NW;         // waves per split workgroup (4, or 8 when rows > 64)
  int P;          // split workgroups
  float scale_log2;
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// Static device scratch of the allocation-free decode (per device, kDecodeScratchBytes):
// its address on the current device, looked up once per device.
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(void** ptr);

// Short convolution of new K/V tokens written into the paged caches.
struct SconvParams {
  const uint16_t* k_new;   // [T, Hkv, 128] bf16, packed new tokens (rows cu[b] .. cu[b + 1] - 1)
  const uint16_t* v_new;
  const float* w_k;        // [4, Hkv, 128] fp32: tap s multiplies x[p - s]
  const float* w_v;
  uint16_t* k_cache;       // [num_blocks, 128, Hkv, 128] bf16: conv outputs at the new positions
  uint16_t* v_cache;
  uint16_t* k_state;       // same layout: raw K/V, read before a chunk, written at its positions
  uint16_t* v_state;
  const int* block_table;  // [B, mbps]
  const int* ctx_lens;     // [B] keys after the write
  const int* cu;           // [B + 1]
  int B, Hkv, mbps, num_blocks, max_new;
};

hipError_t launch_sconv_write(const SconvParams& p, hipStream_t stream);

// Decode limits the host must respect.
constexpr int kDecodeMaxRows = 128;       // n_q * gs (four blocks of 32 rows)
constexpr int kDecodeBiasFloats = 1024;   // gs * (63 + n_q) per unit
constexpr int kDecodeMaxBatch = 2048;     // sequences per launch (prefix table in LDS)
constexpr int kDecodeUnit = 64;           // tokens per unit
constexpr int kDecodeMergeSlices = 4;     // merge workgroups per (segment, row), 32 outputs each

}  // namespace rattn
