// sconv.hip -- the key/value short convolution written into the paged caches, gfx950.
//
// vLLM recipes page "thinkingmachines/Inkling", Overview > Architectural highlights > Short
// convolution: each layer runs four-tap short convolutions over the token axis of, among
// others, the attention keys and values, with their state kept in paged storage.  Read
// here as the causal depthwise convolution over tokens with four taps and a weight per tap
// and channel (no bias, no activation):
//     y[p, c] = sum_{s=0..3} w[s, c] x[p - s, c],   x[p] = 0 for p < 0,
// computed for a chunk of new tokens of every sequence as they enter the caches: y goes to
// the attention cache and the raw x to the state cache, both at the new positions, and the
// raw x of the three positions before a chunk come from the state cache.  It is the step
// right before attention on the same tensors.
//
// Bound by HBM bytes (per new token: its raw K and V read once, four cache rows written), so
// the kernel is a plain streaming one: a thread takes 8 channels (16 bytes) of one token of
// K or V; consecutive threads take consecutive channels, so every load and store of a wave
// covers whole 256-byte rows.  The rows of the three earlier tokens a thread also reads are
// its neighbours' own rows (served by the caches), except before a chunk, where they come
// from the state cache.  fp32 accumulation, bf16 output rounded to nearest even.
#include "device_common.hpp"
#include "launch.hpp"

namespace rattn {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = 16;

__global__ __launch_bounds__(kThreads) void sconv_write_kernel(SconvParams p) {
  const int b = blockIdx.y;
  const int r0 = p.cu[b];
  const int n = min(max(p.cu[b + 1] - r0, 0), p.max_new);
  const int t_begin = blockIdx.x * kTokensPerBlock;
  if (t_begin >= n) return;  // uniform
  const int ctx = min(max(p.ctx_lens[b], n), 128 * p.mbps);
  const int start = ctx - n;  // position of the first new token
  const int chunks = p.Hkv * 16;              // 16-byte chunks of one token's row (K or V)
  const int per_pass = kThreads / (2 * chunks);  // tokens per pass of the workgroup
  const int tid = threadIdx.x;
  const int c = tid % chunks;
  const int tensor = (tid / chunks) & 1;  // 0: K, 1: V
  const int tok_in_pass = tid / (2 * chunks);
  if (tok_in_pass >= per_pass) return;
  const size_t ch = (size_t)c * 8;  // first channel of this thread (h * 128 + d)
  const uint16_t* xnew = tensor ? p.v_new : p.k_new;
  const uint16_t* state_in = tensor ? p.v_state : p.k_state;
  uint16_t* cache = tensor ? p.v_cache : p.k_cache;
  uint16_t* state = tensor ? p.v_state : p.k_state;
  const float* w = tensor ? p.w_v : p.w_k;
  const size_t row = (size_t)p.Hkv * 128;  // channels per token
  // weights of the four taps for these 8 channels
  float wt[4][8];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f32x4_t a = *(const f32x4_t*)(w + s * row + ch);
    const f32x4_t bq = *(const f32x4_t*)(w + s * row + ch + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wt[s][i] = a[i];
      wt[s][4 + i] = bq[i];
    }
  }
  const int* bt = p.block_table + (size_t)b * p.mbps;
  auto slot_of = [&](int pos) -> size_t {  // element offset of position pos's row in a cache
    const int phys = min(max(bt[pos >> 7], 0), p.num_blocks - 1);
    return ((size_t)phys * 128 + (pos & 127)) * row;
  };
  const int t_end = min(n, t_begin + kTokensPerBlock);
  // two tokens per iteration keep twice the loads in flight (measured 3 % faster; 4 was slower)
#pragma unroll 2
  for (int t = t_begin + tok_in_pass; t < t_end; t += per_pass) {
    const int pos = start + t;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    u32x4_t x0 = zero_u32x4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int q = pos - s;
      u32x4_t x = zero_u32x4();
      if (q >= start) x = *(const u32x4_t*)(xnew + (size_t)(r0 + q - start) * row + ch);
      else if (q >= 0) x = *(const u32x4_t*)(state_in + slot_of(q) + ch);
      if (s == 0) x0 = x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wt[s][2 * i], bf16_lo_to_f32(x[i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wt[s][2 * i + 1], bf16_hi_to_f32(x[i]), acc[2 * i + 1]);
      }
    }
    const size_t dst = slot_of(pos) + ch;
    *(u32x4_t*)(cache + dst) = u32x4_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    // the state row is read again only by a later call (the three rows before its chunk):
    // stream it past the caches (non-temporal, measured 1.5 % faster)
    __builtin_nontemporal_store(x0, (u32x4_t*)(state + dst));
  }
}

}  // namespace

hipError_t launch_sconv_write(const SconvParams& p, hipStream_t stream) {
  if (p.B <= 0 || p.max_new <= 0) return hipSuccess;
  // a pass of the workgroup covers at least one token's K and V rows: at most 8 KV heads
  if (p.Hkv < 1 || 2 * p.Hkv * 16 > kThreads) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((p.max_new + kTokensPerBlock - 1) / kTokensPerBlock), (unsigned)p.B);
  hipLaunchKernelGGL(sconv_write_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rattn
