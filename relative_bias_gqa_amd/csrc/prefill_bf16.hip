// prefill_bf16.hip -- relative-bias GQA prefill / chunked prefill, bf16 inputs, gfx950.
//
// Computes, for every query row (b, t, h) at absolute position p = Lk - Lq + t,
//   out = softmax_j(q.k_j / sqrt(128) + r[h, min(p - j, R - 1)]) . V,  lse = log-sum-exp,
// over keys 0 <= p - j (and p - j <= W - 1 for a sliding window): the relative attention
// of the vLLM recipes page "thinkingmachines/Inkling" (Overview > Architectural
// highlights > Attention: a learned relative-position term added to the pre-softmax
// logits of GQA with head size 128, full and sliding-window layers).  Its Performance
// section names a "sheared-bias" kernel: the bias a query tile meets against a key tile
// is one diagonal band of r, which is what each wave stages per tile.
//
// Work decomposition (one workgroup = 8 waves = 512 threads, one workgroup per CU):
//   - a workgroup owns one KV head of one sequence, `hpw` query heads of that head's group
//     and 32 * tsub consecutive query tokens (hpw * tsub = 8); each wave owns one query
//     head x 32 tokens = the 32 columns of its MFMA accumulators;
//   - it walks 64-key tiles from the first key any of its rows can see to the last, so
//     tiles before the window or after the diagonal are never loaded;
//   - K and V tiles go from global memory straight into LDS (global_load_lds_dwordx4) in a
//     ring of four stages, three tiles ahead of the one computed, and serve all of the
//     workgroup's query heads (GQA packing: one K/V read per head group).  K/V rows are
//     stored with a 16-byte-chunk XOR swizzle so the MFMA operand reads are conflict free;
//   - each wave also loads its own 95-entry diagonal slice of r for the tile into the
//     stage, scales it by sqrt(128) in place and seeds its S accumulators with it, so the
//     MFMA adds q.k onto the bias; a tile entirely beyond distance R - 1 seeds one scalar;
//   - per tile and wave: S^T = sqrt(128) r + K Q^T on v_mfma_f32_32x32x16_bf16 (Q resident
//     in registers), logits in log2 units with the running maximum in the same FMA,
//     the causal / window mask only on edge tiles, an online softmax whose maximum is only
//     raised when a row's maximum grows by more than 8 (log2 units), and O^T += V^T P^T
//     with P rounded to bf16 and V read transposed from LDS (ds_read_b64_tr_b16).
#include "device_common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace rattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;                           // keys per tile
constexpr int kStages = 4;
constexpr int kKVBytes = kBK * kHeadDim * 2;      // 16 KB of K (or V) per stage
constexpr int kSliceFloats = 128;                 // per wave: 95 distances used
constexpr int kBiasBytes = kWaves * kSliceFloats * 4;
constexpr int kStageBytes = 2 * kKVBytes + kBiasBytes;  // 36 KB
constexpr int kLoadsPerStage = 6;                 // per wave: 2 K + 2 V + 2 bias
constexpr float kRescaleSlack = 8.0f;             // log2 units: P entries stay below 2^8
constexpr float kSqrtD = 11.313708498984761f;     // sqrt(128)

// 256 bytes of zeros: the source of every K/V row past the end of the sequence.
__device__ __attribute__((aligned(256))) const uint32_t kZeroRowP[64] = {0};

// V^T operand (32 d-rows x 16 keys) from a swizzled V tile: LDS row = key, 256 B, the
// 16-byte chunk c of row r stored at chunk c ^ (2 (r & 7)).  Lane half hf supplies keys
// kbase + 4 hf + 0..3 and kbase + 8 + 4 hf + 0..3, the register order of the S^T block.
__device__ __forceinline__ u32x4_t vt_operand(const unsigned char* v_stage, int kbase, int dcol0, int lane) {
  const int m = lane & 15;
  const int hf = lane >> 5;
  const int row = kbase + 4 * hf + (m >> 2);
  const int col = dcol0 + 16 * ((lane >> 4) & 1) + 4 * (m & 3);
  const int off = (((col >> 3) ^ ((row & 7) << 1)) << 4) + ((col & 7) << 1);
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v_stage + row * 256 + off));
  const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v_stage + (row + 8) * 256 + off));
  const u32x2_t ua = __builtin_bit_cast(u32x2_t, a);
  const u32x2_t ub = __builtin_bit_cast(u32x2_t, b);
  return u32x4_t{ua[0], ua[1], ub[0], ub[1]};
}

__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // accumulator column = query token within the wave
  const int hf = lane >> 5;   // which half of the key rows this lane holds

  // ---- job: heaviest (last) token tiles first ---------------------------------------
  const int per_tile = p.B * p.Hkv * p.n_hg;
  const int tile = p.n_tok_tiles - 1 - (int)blockIdx.x / per_tile;
  const int rem = (int)blockIdx.x % per_tile;
  const int hg = rem % p.n_hg;
  const int hk = (rem / p.n_hg) % p.Hkv;
  const int b = rem / (p.n_hg * p.Hkv);

  const int h = hk * p.G + hg * p.hpw + (wave % p.hpw);
  const int T0 = tile * 32 * p.tsub;
  const int T1 = min(p.Lq, T0 + 32 * p.tsub);
  const int tw0 = T0 + (wave / p.hpw) * 32;  // first token of this wave
  const int off = p.Lk - p.Lq;               // position of token 0
  const int pw0 = off + tw0;                 // position of this wave's column 0
  const int wvalid = min(32, p.Lq - tw0);    // valid columns of this wave (may be <= 0)
  const bool wave_active = wvalid > 0;
  const int pw_last = pw0 + max(wvalid, 1) - 1;
  const int Weff = p.window > 0 ? p.window : 0x40000000;

  // keys the workgroup needs, in whole tiles, and the keys this wave needs
  const int kt_begin = max(0, off + T0 - Weff + 1) / kBK;
  const int kt_end = (off + T1 - 1) / kBK + 1;
  const int n_tiles = kt_end - kt_begin;
  const int wkmin = max(0, pw0 - Weff + 1);
  const int wkmax = pw_last;

  // ---- Q^T operand, resident for the whole key loop -------------------------------
  u32x4_t qr[8];
  {
    const int tq = tw0 + col;
    const bool ok = wave_active && tq < p.Lq;
    const size_t qbase = (((size_t)b * p.Lq + (ok ? tq : 0)) * p.Hq + h) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qr[ks] = ok ? *(const u32x4_t*)((const uint16_t*)p.q + qbase + 16 * ks + 8 * hf) : zero_u32x4();
  }
  // bias in score units (multiplied by sqrt(128)), so that it can seed the S accumulator:
  // (q.k + sqrt(128) r) * log2(e) / sqrt(128) = q.k * log2(e) / sqrt(128) + r * log2(e)
  float bias_sat_v = p.bias[(size_t)h * p.R + (p.R - 1)] * kSqrtD;
  // pin the waits for these loads here, before any LDS-bound load is in flight
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(qr[ks]));
  asm volatile("" : "+v"(bias_sat_v));

  // ---- tile loads -------------------------------------------------------------------
  // K/V: wave w issues keys 8 w .. 8 w + 7 of the tile, four keys (1 KB) per instruction;
  // lane i fetches 16-byte chunk (i & 15) ^ swz(key) of key 4 m + i / 16.
  uint32_t koff[2], voff[2], kz[2], vz[2];
  int ktok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tok = 8 * wave + 4 * i + (lane >> 4);
    const int slot = lane & 15;
    const int ck = slot ^ (tok & 15);
    const int cv = slot ^ ((tok & 7) << 1);
    ktok[i] = tok;
    koff[i] = (uint32_t)(tok * p.Hkv) * 256u + ck * 16;
    voff[i] = (uint32_t)(tok * p.Hkv) * 256u + cv * 16;
    kz[i] = ck * 16;
    vz[i] = cv * 16;
  }
  const unsigned char* kc_bytes = (const unsigned char*)p.k + ((size_t)b * p.Lk * p.Hkv + hk) * 256;
  const unsigned char* vc_bytes = (const unsigned char*)p.v + ((size_t)b * p.Lk * p.Hkv + hk) * 256;
  const unsigned char* zero_bytes = (const unsigned char*)kZeroRowP;
  const float* bias_row = p.bias + (size_t)h * p.R;
  const uint32_t ring_base = lds_addr(ring);

  auto issue_tile = [&](int kt, int st) {
    const int j0 = kt * kBK;
    const size_t base = (size_t)j0 * p.Hkv * 256;
    const uint32_t kdst = ring_base + st * kStageBytes + wave * 2048;
    const uint32_t vdst = kdst + kKVBytes;
    const uint32_t bdst = ring_base + st * kStageBytes + 2 * kKVBytes + wave * (kSliceFloats * 4);
    const bool tail = j0 + kBK > p.Lk;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const unsigned char* gk = kc_bytes + base + koff[i];
      const unsigned char* gv = vc_bytes + base + voff[i];
      if (tail && j0 + ktok[i] >= p.Lk) {
        gk = zero_bytes + kz[i];
        gv = zero_bytes + vz[i];
      }
      dma16(gk, kdst + i * 1024);
      dma16(gv, vdst + i * 1024);
    }
    // this wave's bias slice: entry x = r[h, clamp(pw0 - j0 - 63 + x, 0, R - 1)]
    const int d0 = pw0 - j0 - (kBK - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = min(max(d0 + 64 * i + lane, 0), p.R - 1);
      dma4(bias_row + d, bdst + i * 256);
    }
  };

  // ---- running state ---------------------------------------------------------------
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = zero_f32x16();
  float m_run = kNegInf;  // running max (log2 units), identical in both lane halves
  float l_run = 0.f;      // this lane's share of the running normaliser

  // bias entry of key kk (0..63) for this lane's column: slice[63 + col - kk]
  const int bias_lane = col - 4 * hf + 4;  // slice[bias_lane + 59 - (kk - 4 hf)]

  auto wave_sees = [&](int kt) {
    const int j0 = kt * kBK;
    return wave_active && j0 <= wkmax && j0 + kBK - 1 >= wkmin;
  };

  // S^T = sqrt(128) r + K Q^T for the two 32-key blocks of tile kt (stage st): the
  // accumulators start from this wave's bias slice (or the saturated scalar)
  auto score_tile = [&](int kt, int st, f32x16_t* s) {
    const int j0 = kt * kBK;
    const unsigned char* k_st = ring + st * kStageBytes;
    float* b_st = (float*)(k_st + 2 * kKVBytes + wave * (kSliceFloats * 4));
    if (pw0 - (j0 + kBK - 1) >= p.R - 1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = bias_sat_v;
    } else {
      // scale the slice to score units in place (only this wave reads it)
#pragma unroll
      for (int i = 0; i < 2; ++i) b_st[64 * i + lane] *= kSqrtD;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = b_st[bias_lane + 59 - (32 * kb + 8 * (r >> 2) + (r & 3))];
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int krow = 32 * kb + col;
      const unsigned char* kr = k_st + krow * 256;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        u32x4_t ka[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ka[i] = *(const u32x4_t*)(kr + (((2 * (4 * g + i) + hf) ^ (krow & 15)) << 4));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[kb] = mfma_32x32x16(ka[i], qr[4 * g + i], s[kb]);
        }
      }
    }
  };

  // mask and online softmax of tile kt from its scores: P as bf16
  auto softmax = [&](int kt, f32x16_t* s, u32x4_t (*pk)[2]) {
    const int j0 = kt * kBK;
    const bool need_mask = (j0 + kBK - 1 > pw0) || (j0 < pw_last - Weff + 1);

    // logits relative to the running maximum, in log2 units
    const bool fresh = m_run == kNegInf;
    const float m_ref = fresh ? 0.f : m_run;
    f32x16_t* t = s;  // the logits overwrite the scores
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) t[kb][r] = fmaf(s[kb][r], p.scale_log2, -m_ref);
    if (need_mask) {
      const int dl = pw0 + col - j0 - 4 * hf;  // distance of this lane's first key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = dl - (32 * kb + 8 * (r >> 2) + (r & 3));
          t[kb][r] = (uint32_t)d < (uint32_t)Weff ? t[kb][r] : kNegInf;
        }
    }
    // row maximum: a tree of three-input maxima over the 32 values, then the lane pair
    float m8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kb = i >> 2, r = (i & 3) * 4;
      m8[i] = fmaxf(fmaxf(t[kb][r], t[kb][r + 1]), fmaxf(t[kb][r + 2], t[kb][r + 3]));
    }
    float mx = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])), fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
    mx = half_swap_max(mx);

    // raise the running maximum when a row's new maximum exceeds it by the slack
    const bool raise = fresh ? (mx > kNegInf) : (mx > kRescaleSlack);
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float delta = raise ? mx : 0.f;
      const float m_new = m_ref + delta;
      const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;
      m_run = raise ? m_new : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) t[kb][r] -= delta;
    }

    // P = exp2(t); the normaliser sums it in fp32 (the log-sum-exp needs that accuracy),
    // the P.V product takes it rounded to bf16
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * half + 2 * e;
          const float e0 = fast_exp2(t[kb][r]), e1 = fast_exp2(t[kb][r + 1]);
          lsum += e0 + e1;
          w[e] = pack_bf16x2(e0, e1);
        }
        pk[kb][half] = w;
      }
    l_run += lsum;
  };

  // O^T += V^T P^T for tile kt (stage st)
  auto pv = [&](int st, const u32x4_t (*pk)[2]) {
    const unsigned char* v_st = ring + st * kStageBytes + kKVBytes;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4_t va[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          va[db] = vt_operand(v_st, 32 * kb + 16 * half, 32 * db, lane);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = mfma_32x32x16(va[db], pk[kb][half], o[db]);
      }
  };

  // ---- key loop: tile t computed from stage t % 4 while tiles t+1..t+3 load -------------
  f32x16_t s_cur[2];
  u32x4_t pk[2][2];
  const int prologue = min(kStages - 1, n_tiles);
  for (int i = 0; i < prologue; ++i) issue_tile(kt_begin + i, i);
  for (int t = 0; t < n_tiles; ++t) {
    const int ahead = min(kStages - 2, n_tiles - 1 - t);  // tiles issued after this one
    if (ahead >= 2) vm_wait<2 * kLoadsPerStage>();
    else if (ahead == 1) vm_wait<kLoadsPerStage>();
    else vm_wait<0>();
    wg_barrier();  // tile t is in LDS; every wave is done with tile t - 1
    if (t + kStages - 1 < n_tiles) issue_tile(kt_begin + t + kStages - 1, (t + kStages - 1) % kStages);
    if (wave_sees(kt_begin + t)) {
      score_tile(kt_begin + t, t % kStages, s_cur);
      softmax(kt_begin + t, s_cur, pk);
      pv(t % kStages, pk);
    }
  }

  // ---- epilogue --------------------------------------------------------------------
  const float l_tot = half_swap_sum(l_run);
  const int tq = tw0 + col;
  if (!wave_active || tq >= p.Lq) return;
  const float inv = 1.f / l_tot;
  const size_t obase = (((size_t)b * p.Lq + tq) * p.Hq + h) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * db + 8 * q + 4 * hf;
      const float x0 = o[db][4 * q + 0] * inv, x1 = o[db][4 * q + 1] * inv;
      const float x2 = o[db][4 * q + 2] * inv, x3 = o[db][4 * q + 3] * inv;
      *(u32x2_t*)((uint16_t*)p.out + obase + d) = u32x2_t{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
    }
  if (hf == 0 && p.lse != nullptr)
    p.lse[((size_t)b * p.Lq + tq) * p.Hq + h] = (m_run + __log2f(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  const long long grid = (long long)p.n_tok_tiles * p.B * p.Hkv * p.n_hg;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rattn
