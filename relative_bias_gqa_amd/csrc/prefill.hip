// prefill.hip -- relative-bias GQA prefill / chunked prefill for gfx950, fp32 inputs.
// (bf16 inputs use prefill_bf16.hip.)
//
// Computes, for every query row (b, t, h) at absolute position p = Lk - Lq + t,
//   out = softmax_j(q.k_j / sqrt(128) + r[h, min(p - j, R - 1)]) . V,  lse = log-sum-exp,
// over keys 0 <= p - j (and p - j <= W - 1 for a sliding window).  This is the relative
// attention of the vLLM recipes page "thinkingmachines/Inkling" (Overview >
// Architectural highlights > Attention: GQA with head size 128, a trained bias on the
// logits that depends on the query-key distance, full and sliding-window layers).  The
// page's Performance section names a "sheared-bias" attention kernel: the bias a query
// tile meets against a key tile is one diagonal slice of r, which is what is staged here.
//
// Work decomposition (one workgroup = 8 waves = 512 threads):
//   - a workgroup owns one KV head of one sequence, `hpw` query heads of that KV head's
//     group and 32 * tsub consecutive query tokens (hpw * tsub = 8); each wave owns one
//     query head x 32 tokens, i.e. 32 accumulator columns;
//   - it walks 64-key tiles from the first key any of its rows can see to the last, so
//     tiles entirely before the window or after the diagonal are never loaded;
//   - each K and V tile is read from HBM/L2 once per workgroup and serves all of its query
//     heads (GQA packing);
//   - per tile and wave: S^T = K Q^T on MFMA (K from LDS, Q resident in registers), logits
//     in the log2 domain with the staged bias slice (or one scalar when the whole tile is
//     beyond R - 1), the causal / window mask only on edge tiles, an online softmax whose
//     running maximum is only raised when it grows by more than kRescaleSlack (so the
//     O rescale is rare), then O^T += V^T P^T with V read transposed from LDS.
//   - the fp32 inputs are never rounded to bf16: K and V sit in LDS as hi/lo bf16 planes
//     (hi = bf16(x), lo = bf16(x - hi)), Q as hi/lo registers, and each product takes the
//     three terms hi.hi + hi.lo + lo.hi; one LDS stage, the next tile's loads in registers.
#include "device_common.hpp"
#include "launch.hpp"

namespace rattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;              // keys per tile
constexpr int kKStride = 136;        // bf16 per K row in LDS (272 B: conflict-free b128 reads)
constexpr int kVStride = 160;        // bf16 per V row in LDS (320 B: conflict-free tr reads)
constexpr int kBiasSlice = kBK + 32 - 1;  // distances one wave tile meets (95)
constexpr int kBiasCopy = 100;       // floats per shifted copy (95 + 3 shift, padded)
constexpr int kBiasWave = 4 * kBiasCopy;
constexpr float kRescaleSlack = 8.0f;  // log2 units: P entries stay below 2^8

constexpr int kPlanes = 2;           // bf16 hi and lo planes of the fp32 K and V
constexpr int kKElems = kBK * kKStride;
constexpr int kVElems = kBK * kVStride;

struct TileRegs {  // 64 x 128 fp32 K and V: four 16-byte chunks each per thread
  f32x4_t k[4], v[4];
};

__device__ __forceinline__ f32x4_t ld16f(const void* p) { return *(const f32x4_t*)p; }

// hi = bf16(x), lo = bf16(x - hi) for four floats, packed as 4 bf16 each.
__device__ __forceinline__ void split4(f32x4_t x, u32x2_t& hi, u32x2_t& lo) {
  const uint32_t h01 = pack_bf16x2(x[0], x[1]);
  const uint32_t h23 = pack_bf16x2(x[2], x[3]);
  hi[0] = h01;
  hi[1] = h23;
  lo[0] = pack_bf16x2(x[0] - bf16_lo_to_f32(h01), x[1] - bf16_hi_to_f32(h01));
  lo[1] = pack_bf16x2(x[2] - bf16_lo_to_f32(h23), x[3] - bf16_hi_to_f32(h23));
}

__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kPlanes][kKElems];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kPlanes][kVElems];
  __shared__ __attribute__((aligned(16))) float b_lds[kWaves][kBiasWave];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // keys the workgroup needs, in whole tiles
  const int kmin = max(0, off + T0 - Weff + 1);
  const int kmax = off + T1 - 1;
  const int kt_begin = kmin / kBK;
  const int kt_end = kmax / kBK + 1;
  // keys this wave needs
  const int wkmin = max(0, pw0 - Weff + 1);
  const int wkmax = pw_last;

  // ---- Q^T operand, resident for the whole key loop -------------------------------
  u32x4_t qh[8], ql[8];
  {
    const int tq = tw0 + col;
    const bool ok = wave_active && tq < p.Lq;
    const size_t qbase = (((size_t)b * p.Lq + (ok ? tq : 0)) * p.Hq + h) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int d = 16 * ks + 8 * hf;
      f32x4_t x0, x1;
      if (ok) {
        x0 = ld16f((const float*)p.q + qbase + d);
        x1 = ld16f((const float*)p.q + qbase + d + 4);
      } else {
        x0 = x1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      u32x2_t h0, l0, h1, l1;
      split4(x0, h0, l0);
      split4(x1, h1, l1);
      qh[ks] = u32x4_t{h0[0], h0[1], h1[0], h1[1]};
      ql[ks] = u32x4_t{l0[0], l0[1], l1[0], l1[1]};
    }
  }

  // ---- tile loads: global -> registers -> LDS -------------------------------------
  TileRegs tr;
  float breg[2];
  const size_t kv_seq = (size_t)b * p.Lk;
  auto issue_tile = [&](int kt) {
    const int j0 = kt * kBK;
    const int r0 = tid >> 5, chunk = tid & 31;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + r0 + 16 * c;
      if (j < p.Lk) {
        const size_t a = ((kv_seq + j) * p.Hkv + hk) * kHeadDim + chunk * 4;
        tr.k[c] = ld16f((const float*)p.k + a);
        tr.v[c] = ld16f((const float*)p.v + a);
      } else {
        tr.k[c] = tr.v[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    // bias slice for this wave: distances pw0 - j0 - 63 + c, c = 0..94, clamped to [0, R-1]
    const int d0 = pw0 - j0 - (kBK - 1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = lane + 64 * c;
      const int d = min(max(d0 + idx, 0), p.R - 1);
      breg[c] = (idx < kBiasSlice) ? p.bias[(size_t)h * p.R + d] * kLog2e : 0.f;
    }
  };
  auto store_tile = [&]() {
    const int r0 = tid >> 5, chunk = tid & 31;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x2_t hi, lo;
      split4(tr.k[c], hi, lo);
      *(u32x2_t*)&k_lds[0][(r0 + 16 * c) * kKStride + chunk * 4] = hi;
      *(u32x2_t*)&k_lds[1][(r0 + 16 * c) * kKStride + chunk * 4] = lo;
      split4(tr.v[c], hi, lo);
      *(u32x2_t*)&v_lds[0][(r0 + 16 * c) * kVStride + chunk * 4] = hi;
      *(u32x2_t*)&v_lds[1][(r0 + 16 * c) * kVStride + chunk * 4] = lo;
    }
    // four copies shifted by 0..3 so every lane can fetch its four biases with one
    // aligned 16-byte read (copy s holds slice[c] at index c + s)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = lane + 64 * c;
      if (idx < kBiasSlice) {
#pragma unroll
        for (int s = 0; s < 4; ++s) b_lds[wave][s * kBiasCopy + idx + s] = breg[c];
      }
    }
  };

  // ---- running state ---------------------------------------------------------------
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = zero_f32x16();
  float m_run = kNegInf;  // running max (log2 domain), identical in both lane halves
  float l_run = 0.f;      // this lane's share of the running normaliser

  const float bias_sat = p.bias[(size_t)h * p.R + (p.R - 1)] * kLog2e;
  const int bsel = (4 - (col & 3)) & 3;  // which shifted bias copy is aligned for this lane

  auto compute_tile = [&](int kt) {
    const int j0 = kt * kBK;
    if (!wave_active || j0 > wkmax || j0 + kBK - 1 < wkmin) return;
    const bool need_mask = (j0 + kBK - 1 > pw0) || (j0 < pw_last - Weff + 1);
    const bool saturated = pw0 - (j0 + kBK - 1) >= p.R - 1;

    // S^T = K Q^T : two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero_f32x16();
      const uint16_t* krow = &k_lds[0][(32 * kb + col) * kKStride + 8 * hf];
      const uint16_t* krow_lo = &k_lds[1][(32 * kb + col) * kKStride + 8 * hf];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4_t a = *(const u32x4_t*)(krow + 16 * ks);
        const u32x4_t al = *(const u32x4_t*)(krow_lo + 16 * ks);
        s[kb] = mfma_32x32x16(a, qh[ks], s[kb]);
        s[kb] = mfma_32x32x16(a, ql[ks], s[kb]);
        s[kb] = mfma_32x32x16(al, qh[ks], s[kb]);
      }
    }

    // logits in log2 units: s * log2(e)/sqrt(128) + r * log2(e)
    float t[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4_t bv;
        if (saturated) {
          bv = f32x4_t{bias_sat, bias_sat, bias_sat, bias_sat};
        } else {
          // element (col, key 32kb + 8q + 4hf + e) reads slice[col - 32kb - 8q - 4hf - e + 63]
          const int a = col - 32 * kb - 8 * q - 4 * hf + 60;
          bv = *(const f32x4_t*)&b_lds[wave][bsel * kBiasCopy + a + bsel];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) t[kb][4 * q + e] = s[kb][4 * q + e] * p.scale_log2 + bv[3 - e];
      }
    }
    if (need_mask) {
      const int dl = pw0 + col - j0 - 4 * hf;  // distance of this lane's first key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = dl - 32 * kb - 8 * (r >> 2) - (r & 3);
          t[kb][r] = (d >= 0 && d < Weff) ? t[kb][r] : kNegInf;
        }
    }

    // online softmax with a lazily raised maximum
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

    // O^T += V^T P^T
    u32x4_t ph[2][2], pl[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        ph[kb][half] = pack_p_operand(&t[kb][8 * half]);
        float rest[8];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t w = ph[kb][half][e >> 1];
          rest[e] = t[kb][8 * half + e] - bf16_lo_to_f32(w);
          rest[e + 1] = t[kb][8 * half + e + 1] - bf16_hi_to_f32(w);
        }
        pl[kb][half] = pack_p_operand(rest);
      }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kbase = 32 * kb + 16 * half;
          const u32x4_t a = load_vt_operand(&v_lds[0][0], kVStride, kbase, 32 * db, lane);
          const u32x4_t al = load_vt_operand(&v_lds[1][0], kVStride, kbase, 32 * db, lane);
          o[db] = mfma_32x32x16(a, ph[kb][half], o[db]);
          o[db] = mfma_32x32x16(al, ph[kb][half], o[db]);
          o[db] = mfma_32x32x16(a, pl[kb][half], o[db]);
        }
  };

  // ---- key loop ----------------------------------------------------------------------
  issue_tile(kt_begin);
  store_tile();
  __syncthreads();
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const bool has_next = kt + 1 < kt_end;
    if (has_next) issue_tile(kt + 1);  // into registers, while this tile is computed
    compute_tile(kt);
    __syncthreads();  // every wave is done with this tile's LDS
    if (has_next) store_tile();
    __syncthreads();
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
      *(f32x4_t*)((float*)p.out + obase + d) = f32x4_t{x0, x1, x2, x3};
    }
  if (hf == 0 && p.lse != nullptr)
    p.lse[((size_t)b * p.Lq + tq) * p.Hq + h] = (m_run + __log2f(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_prefill_fp32(const PrefillParams& p, hipStream_t stream) {
  const long long grid = (long long)p.n_tok_tiles * p.B * p.Hkv * p.n_hg;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rattn
