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
  float* D;           // [B, Lq, Hq] workspace: rowsum(dout * out)
  int B, Lq, Lk, Hq, Hkv, G, R, window;
  float scale_log2;   // log2(e) / sqrt(128)
};

hipError_t launch_backward(const BackwardParams& p, hipStream_t stream);

}  // namespace rattn
