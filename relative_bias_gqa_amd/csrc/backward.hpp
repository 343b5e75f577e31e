// backward.hpp -- launch parameters of the prefill backward pass (host <-> device).
#pragma once

#include <hip/hip_runtime.h>

namespace rattn {

// Gradients of a contiguous bf16 prefill (layouts of PrefillParams; outputs fp32).
struct BackwardParams {
  const void* q;      // [B, Lq, Hq, 128] bf16
  const void* k;      // [B, Lk, Hkv, 128] bf16
  const void* v;      // [B, Lk, Hkv, 128] bf16
  const float* bias;  // [Hq, R]
  const void* out;    // [B, Lq, Hq, 128] bf16, the forward's output
  const void* dout;   // [B, Lq, Hq, 128] bf16
  const float* lse;   // [B, Lq, Hq], natural log, the forward's
  float* dq;          // [B, Lq, Hq, 128]
  float* dk;          // [B, Lk, Hkv, 128]
  float* dv;          // [B, Lk, Hkv, 128]
  float* dbias;       // [Hq, R]
  float* D;           // [B, Hq, Lq] workspace: rowsum(dout * out) (head-major)
  float* L2;          // [B, Hq, Lq] workspace: lse * log2(e)
  // key-stationary pass: a key block's query steps in kv_chunks chunks of kv_chunk;
  // partials [chunk][pair] (chunk-1 planes are written and read only for two-chunk blocks)
  float* part_dk;     // [2, n_pairs, B, Lk, Hkv, 128] workspace: dK of each pair (unscaled)
  float* part_dv;     // [2, n_pairs, B, Lk, Hkv, 128] workspace: dV of each pair
  int n_pairs;        // ceil(G / 2)
  int kv_chunk;       // steps per chunk (a block's steps when kv_chunks == 1)
  // query-stationary pass: a token tile's key tiles in q_chunks chunks of q_chunk; for a
  // two-chunk tile each chunk's dq goes to its slot of dq_part, and whichever chunk finishes
  // second adds the other's partial (dq_cnt: one counter per tile and head group)
  float* dq_part;     // [units, 2, 8 waves, 64, 64] workspace
  int* dq_cnt;        // [n_tok_tiles * B * Hkv * n_hg] workspace, zeroed by the row pass
  // sqrt(128) * bias[h, i] for i < Rs = min(R, Lk) (the entries any visible pair can reach):
  // the seed of every S accumulator, as in the forward pass
  float* bias_s;      // [Hq, Rs] workspace
  int Rs;
  int q_chunk;        // key tiles per chunk (a tile's when q_chunks == 1)
  int kv_chunks, q_chunks;  // chunks per key block / token tile: 1 or 2 (host's plan)
  // query-stationary pass: a workgroup takes hpw query heads x 32 * tsub queries (hpw * tsub
  // = 8 waves), n_hg = G / hpw head groups per KV head, n_tok_tiles token tiles
  int hpw, tsub, n_hg, n_tok_tiles;
  int B, Lq, Lk, Hq, Hkv, G, R, window;
  float scale_log2;   // log2(e) / sqrt(128)
};

// All launches of the backward pass, in order on `stream`.
hipError_t launch_backward(const BackwardParams& p, hipStream_t stream);

}  // namespace rattn
