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
};

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream);
hipError_t launch_prefill_fp32(const PrefillParams& p, hipStream_t stream);

// Paged split-KV decode (sizes validated, split plan fixed by the host).
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
  float* ws_o;    // [B, n_q, Hq, S, 128] partial outputs (normalised per split)
  float* ws_lse;  // [B, n_q, Hq, S] partial log2-sum-exp
  int B, n_q, Hq, Hkv, R, mbps;
  int num_blocks; // physical blocks in each cache
  int G;          // Hq / Hkv
  int gs;         // query heads per workgroup
  int n_hs;       // G / gs
  int rows;       // n_q * gs query rows per workgroup
  int S;          // splits per sequence
  int SB;         // cache blocks per split
  float scale_log2;
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// Decode limits the host must respect.
constexpr int kDecodeMaxRows = 128;       // n_q * gs
constexpr int kDecodeBiasFloats = 1152;   // gs * (127 + n_q)

}  // namespace rattn
