// decode.hip -- paged split-KV decode with multi-query (MTP) verification for gfx950.
//
// Each sequence b has ctx_lens[b] keys in a paged cache of 128-token blocks (vLLM recipes
// page "thinkingmachines/Inkling", Client Usage: "--block-size 128") and n_q query tokens
// at positions ctx - n_q .. ctx - 1 (Overview > MTP: up to 9 tokens per step with eight
// MTP heads).  Every query row computes the relative-bias attention of Overview >
// Architectural highlights > Attention:
//   softmax_j(q.k_j / sqrt(128) + r[h, min(p - j, R - 1)]) . V over the causal (and, for a
//   sliding-window sequence, windowed) keys.
//
// Pass 1 (split kernel): workgroup = (sequence, KV head, query-head subgroup, split of SB
// consecutive cache blocks).  Its query rows are the n_q tokens x gs query heads that
// share the KV head (GQA packing: every K/V block is read from HBM once for all of them).
// Waves own 32 rows each.  Per cache block the workgroup gathers K and V (32 KB each per KV
// head) through the block table into LDS -- the next block's loads are in flight while the
// current one is computed -- and each wave does S^T = K Q^T, bias + mask, an online
// softmax and O^T += V^T P^T.  Slots outside the sequence's visible range are zero-filled
// on load, so poisoned (NaN) cache contents never reach the arithmetic.  The split writes
// its normalised partial output and log2-sum-exp to the workspace.
// Pass 2 (merge kernel): per query row, LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s, written as bf16 (+ natural-log lse).
#include "device_common.hpp"
#include "launch.hpp"

namespace rattn {
namespace {

constexpr int kThreads = 256;   // 4 waves
constexpr int kBlock = 128;     // tokens per cache block
constexpr int kKStride = 136;   // bf16 per K row in LDS
constexpr int kVStride = 160;   // bf16 per V row in LDS
constexpr float kRescaleSlack = 8.0f;

struct SeqRange {
  int ctx, Weff, blk_lo, blk_hi, vis_lo;
};

__device__ __forceinline__ SeqRange seq_range(const DecodeParams& p, int b) {
  SeqRange r;
  r.ctx = p.ctx_lens[b];
  const int W = p.windows ? p.windows[b] : 0;
  r.Weff = W > 0 ? W : 0x40000000;
  r.vis_lo = W > 0 ? max(0, r.ctx - p.n_q - W + 1) : 0;
  r.blk_lo = r.vis_lo / kBlock;
  // never index past the sequence's block-table row or the planned splits, whatever
  // ctx_lens holds
  r.blk_hi = min(min((r.ctx - 1) / kBlock + 1, p.mbps), p.S * p.SB);
  return r;
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *(const u32x4_t*)p; }

__global__ __launch_bounds__(kThreads, 1) void decode_split_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBlock * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kBlock * kVStride];
  __shared__ __attribute__((aligned(16))) float b_lds[kDecodeBiasFloats];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int hf = lane >> 5;

  // ---- job --------------------------------------------------------------------------
  const int s = (int)blockIdx.x % p.S;
  const int rest = (int)blockIdx.x / p.S;
  const int hs = rest % p.n_hs;
  const int hk = (rest / p.n_hs) % p.Hkv;
  const int b = rest / (p.n_hs * p.Hkv);

  const SeqRange sr = seq_range(p, b);
  const int blk_begin = max(s * p.SB, sr.blk_lo);
  const int blk_end = min((s + 1) * p.SB, sr.blk_hi);
  if (blk_begin >= blk_end) return;  // no visible key in this split (uniform exit)

  const int p0 = sr.ctx - p.n_q;     // position of query 0
  const int p_last = sr.ctx - 1;
  const int SL = kBlock - 1 + p.n_q; // bias slice length per head and block

  // ---- this lane's query row ---------------------------------------------------------
  const int c = 32 * wave + col;
  const bool wave_active = 32 * wave < p.rows;
  const bool row_ok = c < p.rows;
  const int tq = row_ok ? c / p.gs : 0;
  const int gi = row_ok ? c % p.gs : 0;
  const int h = hk * p.G + hs * p.gs + gi;
  u32x4_t qr[8];
  {
    const size_t qbase = (((size_t)b * p.n_q + tq) * p.Hq + h) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qr[ks] = row_ok ? ld16(p.q + qbase + 16 * ks + 8 * hf) : zero_u32x4();
  }
  const float bias_sat = p.bias[(size_t)h * p.R + (p.R - 1)] * kLog2e;

  // ---- block loads (gather through the block table, zero-fill invisible slots) --------
  u32x4_t kreg[8], vreg[8];
  float breg[(kDecodeBiasFloats + kThreads - 1) / kThreads];
  const int* bt_row = p.block_table + (size_t)b * p.mbps;
  auto issue_block = [&](int blk) {
    // ids outside [0, num_blocks) are clamped so a bad table entry cannot address memory
    // beyond the caches
    const int phys = min(max(bt_row[blk], 0), p.num_blocks - 1);
    const int r0 = tid >> 4, chunk = tid & 15;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int row = r0 + 16 * cc;
      const int j = blk * kBlock + row;
      if (j >= sr.vis_lo && j < sr.ctx) {
        const size_t a = (((size_t)phys * kBlock + row) * p.Hkv + hk) * kHeadDim + chunk * 8;
        kreg[cc] = ld16(p.k_cache + a);
        vreg[cc] = ld16(p.v_cache + a);
      } else {
        kreg[cc] = zero_u32x4();
        vreg[cc] = zero_u32x4();
      }
    }
    const int j0 = blk * kBlock;
    if (p0 - (j0 + kBlock - 1) < p.R - 1) {  // block not entirely beyond R - 1: stage slices
      const int d0 = p0 - j0 - (kBlock - 1);
#pragma unroll
      for (int i = 0; i < (kDecodeBiasFloats + kThreads - 1) / kThreads; ++i) {
        const int idx = tid + kThreads * i;
        float val = 0.f;
        if (idx < p.gs * SL) {
          const int g = idx / SL, x = idx % SL;
          const int d = min(max(d0 + x, 0), p.R - 1);
          val = p.bias[(size_t)(hk * p.G + hs * p.gs + g) * p.R + d] * kLog2e;
        }
        breg[i] = val;
      }
    }
  };
  auto store_block = [&](int blk) {
    const int r0 = tid >> 4, chunk = tid & 15;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      *(u32x4_t*)&k_lds[(r0 + 16 * cc) * kKStride + chunk * 8] = kreg[cc];
      *(u32x4_t*)&v_lds[(r0 + 16 * cc) * kVStride + chunk * 8] = vreg[cc];
    }
    const int j0 = blk * kBlock;
    if (p0 - (j0 + kBlock - 1) < p.R - 1) {
#pragma unroll
      for (int i = 0; i < (kDecodeBiasFloats + kThreads - 1) / kThreads; ++i) {
        const int idx = tid + kThreads * i;
        if (idx < p.gs * SL) b_lds[idx] = breg[i];
      }
    }
  };

  // ---- running state ---------------------------------------------------------------
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = zero_f32x16();
  float m_run = kNegInf;
  float l_run = 0.f;

  auto compute_block = [&](int blk) {
    if (!wave_active) return;
    const int j0 = blk * kBlock;
    const bool saturated = p0 - (j0 + kBlock - 1) >= p.R - 1;
    const bool need_mask = (j0 + kBlock - 1 > p0) || (j0 < p_last - sr.Weff + 1);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {  // two halves of 64 keys
      f32x16_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero_f32x16();
        const uint16_t* krow = &k_lds[(64 * kh + 32 * kb + col) * kKStride + 8 * hf];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) sacc[kb] = mfma_32x32x16(*(const u32x4_t*)(krow + 16 * ks), qr[ks], sacc[kb]);
      }
      float t[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 64 * kh + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);  // key offset in block
          const float bv = saturated ? bias_sat : b_lds[gi * SL + (tq + kBlock - 1 - kk)];
          t[kb][r] = sacc[kb][r] * p.scale_log2 + bv;
        }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 64 * kh + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            const int d = p0 + tq - j0 - kk;
            t[kb][r] = (d >= 0 && d < sr.Weff) ? t[kb][r] : kNegInf;
          }
      }
      float mx = t[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, t[kb][r]);
      mx = half_swap_max(mx);
      const bool raise = mx > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float alpha = raise ? fast_exp2(m_run - mx) : 1.f;
        m_run = raise ? mx : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      const float msub = (m_run == kNegInf) ? 0.f : m_run;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          t[kb][r] = fast_exp2(t[kb][r] - msub);
          lsum += t[kb][r];
        }
      l_run += lsum;
      u32x4_t pk[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) pk[kb][half] = pack_p_operand(&t[kb][8 * half]);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const u32x4_t a = load_vt_operand(v_lds, kVStride, 64 * kh + 32 * kb + 16 * half, 32 * db, lane);
            o[db] = mfma_32x32x16(a, pk[kb][half], o[db]);
          }
    }
  };

  // ---- block loop ------------------------------------------------------------------
  issue_block(blk_begin);
  store_block(blk_begin);
  __syncthreads();
  for (int blk = blk_begin; blk < blk_end; ++blk) {
    const bool has_next = blk + 1 < blk_end;
    if (has_next) issue_block(blk + 1);
    compute_block(blk);
    __syncthreads();
    if (has_next) {
      store_block(blk + 1);
      __syncthreads();
    }
  }

  // ---- partial result of this split ------------------------------------------------
  const float l_tot = half_swap_sum(l_run);
  if (!row_ok) return;
  const size_t row_id = ((size_t)b * p.n_q + tq) * p.Hq + h;
  const size_t slot = row_id * p.S + s;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* dst = p.ws_o + slot * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * db + 8 * q + 4 * hf;
      *(f32x4_t*)(dst + d) = f32x4_t{o[db][4 * q] * inv, o[db][4 * q + 1] * inv, o[db][4 * q + 2] * inv,
                                     o[db][4 * q + 3] * inv};
    }
  if (hf == 0) p.ws_lse[slot] = l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;
}

// One workgroup per query row: merge the partial results of its sequence's splits.
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeParams p) {
  __shared__ float red[kThreads];
  __shared__ f32x4_t acc_lds[8][32];
  const int tid = threadIdx.x;
  const size_t row_id = blockIdx.x;
  const int b = (int)(row_id / ((size_t)p.n_q * p.Hq));
  const SeqRange sr = seq_range(p, b);
  const int s_lo = sr.blk_lo / p.SB;
  const int s_hi = (sr.blk_hi - 1) / p.SB + 1;
  const float* lse_s = p.ws_lse + row_id * p.S;

  float m = kNegInf;
  for (int s = s_lo + tid; s < s_hi; s += kThreads) m = fmaxf(m, lse_s[s]);
  red[tid] = m;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float z = 0.f;
  for (int s = s_lo + tid; s < s_hi; s += kThreads) z += fast_exp2(lse_s[s] - M);
  red[tid] = z;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float Z = red[0];

  const int d4 = tid & 31, grp = tid >> 5;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = s_lo + grp; s < s_hi; s += 8) {
    const float w = fast_exp2(lse_s[s] - M);
    const f32x4_t x = *(const f32x4_t*)(p.ws_o + (row_id * p.S + s) * kHeadDim + 4 * d4);
    acc += w * x;
  }
  acc_lds[grp][d4] = acc;
  __syncthreads();
  if (grp == 0) {
    f32x4_t tot = acc_lds[0][d4];
#pragma unroll
    for (int g = 1; g < 8; ++g) tot += acc_lds[g][d4];
    const float inv = 1.f / Z;
    *(u32x2_t*)(p.out + row_id * kHeadDim + 4 * d4) =
        u32x2_t{pack_bf16x2(tot[0] * inv, tot[1] * inv), pack_bf16x2(tot[2] * inv, tot[3] * inv)};
  }
  if (tid == 0 && p.lse != nullptr) p.lse[row_id] = (M + __log2f(Z)) * kLn2;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const long long grid1 = (long long)p.B * p.Hkv * p.n_hs * p.S;
  const long long grid2 = (long long)p.B * p.n_q * p.Hq;
  if (grid1 <= 0) return hipSuccess;
  if (grid1 > 0x7fffffffLL || grid2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_split_kernel, dim3((unsigned)grid1), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)grid2), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rattn
