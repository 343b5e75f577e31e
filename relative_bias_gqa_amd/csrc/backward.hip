// backward.hip -- gradients of the relative-bias GQA prefill (bf16 inputs), gfx950.
//
// The forward pass (vLLM recipes page "thinkingmachines/Inkling", Overview > Architectural
// highlights > Attention: GQA with head size 128, a trained distance-dependent bias on the
// logits in place of RoPE; the page also lists training and LoRA among the model's uses)
// is s = q.k / sqrt(128) + r[h, min(p - j, R - 1)] over the visible keys, P = softmax(s),
// O = P V.  Its gradients for an output gradient dO, with D = rowsum(dO * O):
//   dS = P * (dO V^T - D),  dQ = dS K / sqrt(128),  dK = dS^T Q / sqrt(128),  dV = P^T dO,
//   dr[h, d] = sum of dS over the (query, key) pairs at clamped distance d,
// dK and dV summed over the query heads of a KV head.  P is recomputed from the forward's
// log-sum-exp, never stored.
//
// Three launches on the caller's stream:
//   1. D = rowsum(dout * out) and lse * log2(e) per query row (fp32, head-major), plus the
//      preparation: dr zeroed, the bias table scaled to score units (sqrt(128) r, the seed of
//      every S accumulator, as in the forward pass), the split counters zeroed;
//   2. both passes in one grid (neither reads the other's results, so each fills the compute
//      units the other leaves idle; the key-stationary units, the longer ones, come first):
//      - key-stationary dK, dV: a workgroup owns 128 keys of a KV head and a pair of its
//        query heads (8 waves = 4 blocks of 32 keys x 2 heads); K and V stay in LDS, the query
//        tiles that see them stream in by direct-to-LDS DMA; S = Q K^T and dP = dO V^T come
//        out with one key per lane, the A-operand layout of dV += P^T dO and dK += dS^T Q, so
//        P and dS feed those MFMAs from registers (dO and Q read transposed from LDS); each
//        pair writes a partial dK, dV;
//      - query-stationary dQ and dr: the forward's decomposition (8 waves, one query head x
//        32 queries each, Q^T and dO^T resident in registers), K and V streamed through an LDS
//        ring; S^T and dP^T come out with one query per lane, the B-operand layout of
//        dQ^T += K^T dS^T, so dQ stays in registers and is stored once (a token tile whose key
//        tiles two workgroups share is merged by the one that finishes second); dS is also
//        summed per distance through a skewed table in LDS and added into dr (fp32 atomics:
//        dr's last bits may change from run to run);
//   3. dK, dV = the pairs' partials summed in pair order (deterministic).
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS are rounded to
// bf16 as MFMA operands.
#include <algorithm>

#include "backward.hpp"
#include "device_common.hpp"

namespace rattn {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kRsqrtD = 0.08838834764831845f;  // 1 / sqrt(128)
constexpr float kSqrtD = 11.313708498984761f;     // sqrt(128)
constexpr int kDiagStride = 34;            // floats per row of the diagonal table (conflict free)

// 256 bytes of zeros: the source of every K/V row past Lk and query row past Lq.
__device__ __attribute__((aligned(256))) const uint32_t kZeroRowB[64] = {0};
// The masks live in the data: a bias-slice entry at a distance no visible pair has
// (negative, or >= the window) is loaded as -inf, and lse * log2(e) of a query row past Lq as
// +inf, so exp2 gives P = 0 (hence dS = 0) for every invisible pair with no select.
__device__ const float kNegInfF = -__builtin_inff();
__device__ const float kPosInfF = __builtin_inff();

// Keeps the compiler from moving memory accesses across this point.  Used between LDS
// accesses of one wave, which the LDS performs in the wave's order.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

__global__ __launch_bounds__(256) void bwd_fill_zero_kernel(float* a, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) a[i] = 0.f;
}

// dbias = 0, and bias_s[h, i] = sqrt(128) * bias[h, i] for i < Rs: the table in score units
// that seeds the S accumulators of both passes (the forward pass seeds its own the same way);
// the dq pass's n_cnt split counters = 0.  Elements i0, i0 + stride, ... of each.
__device__ __forceinline__ void prep_work(const BackwardParams& p, size_t n_r, size_t n_cnt, size_t i0, size_t stride) {
  for (size_t i = i0; i < n_r; i += stride) {
    p.dbias[i] = 0.f;
    const size_t h = i / p.R;
    const int j = (int)(i - h * p.R);
    if (j < p.Rs) p.bias_s[h * p.Rs + j] = p.bias[i] * kSqrtD;
  }
  for (size_t i = i0; i < n_cnt; i += stride) p.dq_cnt[i] = 0;
}

// The same work alone (when there is no query row to run bwd_rowdot_kernel for).
__global__ __launch_bounds__(256) void bwd_prep_kernel(BackwardParams p, size_t n_r, size_t n_cnt) {
  prep_work(p, n_r, n_cnt, (size_t)blockIdx.x * 256 + threadIdx.x, (size_t)gridDim.x * 256);
}

// D = sum_d dout[b, t, h, d] * out[b, t, h, d] and L2 = lse[b, t, h] * log2(e) for every row,
// in fp32, stored head-major ([B, Hq, Lq]) so that a query tile of one head is contiguous.
// A workgroup takes one (batch, head) pair and kRowdotRows consecutive query positions, so its
// D and L2 stores fill whole cache lines from one XCD.  Sixteen lanes share a row, each reading
// one 16-byte chunk of dout and of out; the sixteen partial sums are then added across those
// lanes.
constexpr int kRowdotPasses = 2;
constexpr int kRowdotRows = 16 * kRowdotPasses;  // query positions per workgroup: one 128 B line of D

// The launch also does prep_work over its whole grid (one launch fewer).
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(BackwardParams p, int n_tb, size_t n_r, size_t n_cnt) {
  const uint16_t* const out = (const uint16_t*)p.out;
  const uint16_t* const dout = (const uint16_t*)p.dout;
  const float* const lse = p.lse;
  float* const D = p.D;
  float* const L2 = p.L2;
  const int Lq = p.Lq, Hq = p.Hq;
  const int c = threadIdx.x & 15;
  const int tb = blockIdx.x % n_tb;
  const size_t bh = blockIdx.x / n_tb;
  const size_t b = bh / Hq, h = bh % Hq;
  const int t0 = tb * kRowdotRows + (threadIdx.x >> 4);
  u32x4_t x[kRowdotPasses], y[kRowdotPasses];
#pragma unroll
  for (int j = 0; j < kRowdotPasses; ++j) {
    const int t = t0 + 16 * j;
    x[j] = u32x4_t{0, 0, 0, 0};
    y[j] = u32x4_t{0, 0, 0, 0};
    if (t < Lq) {
      const size_t row = (b * Lq + t) * Hq + h;
      x[j] = ((const u32x4_t*)(out + row * kHeadDim))[c];
      y[j] = ((const u32x4_t*)(dout + row * kHeadDim))[c];
    }
  }
#pragma unroll
  for (int j = 0; j < kRowdotPasses; ++j) {
    const int t = t0 + 16 * j;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo_to_f32(x[j][i]), bf16_lo_to_f32(y[j][i]), acc);
      acc = fmaf(bf16_hi_to_f32(x[j][i]), bf16_hi_to_f32(y[j][i]), acc);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (t < Lq && c == 0) {
      const size_t dst = bh * Lq + t;
      D[dst] = acc;
      L2[dst] = lse[(b * Lq + t) * Hq + h] * kLog2e;
    }
  }
  prep_work(p, n_r, n_cnt, (size_t)blockIdx.x * 256 + threadIdx.x, (size_t)gridDim.x * 256);
}

// ---- key-stationary pass (dK, dV) -----------------------------------------------------
// A workgroup owns 128 keys (four 32-key blocks) of one KV head and one pair of its query
// heads: 8 waves, wave w = key block w & 3 for head slot w >> 2.  K and V of the 128 keys sit
// in LDS for the whole pass; the query tiles that see them stream through a two-stage LDS
// ring, one step ahead, straight from global memory (global_load_lds_dwordx4): per step
// the Q and dO tiles (32 queries) of both heads, their D and lse*log2(e), and each wave's
// 63-entry slice of the bias table in score units (the seeds of its S).  Per step a wave computes S = Q K^T and dP = dO V^T with one key per
// lane (the accumulator column), then P and dS, then dV += P^T dO and dK += dS^T Q (P and dS
// as A operands straight from registers, dO and Q read transposed from LDS).  At the end the
// two slots of a key block add up through LDS and slot 0 writes the pair's partial dK, dV;
// the pairs are summed in pair order afterwards (no atomics: the result is deterministic).
//
// Tiles in LDS have 256-byte rows; 16-byte chunk c of row r is stored at chunk c ^ swz(r),
// swz(r) = 4 (r & 3) + ((r >> 2) & 3): the sixteen rows a 16-lane group reads row-wise get
// sixteen different chunks, and the four rows x four chunks of a transposed read
// (ds_read_b64_tr_b16) land in sixteen different chunks as well.
constexpr int kKvBlocks = 4;                // 32-key blocks per workgroup
constexpr int kKvKeys = 32 * kKvBlocks;     // 128
constexpr int kKvWaves = 2 * kKvBlocks;     // two head slots
constexpr int kTileBytes = 32 * 256;        // 32 rows of 128 bf16
constexpr int kRingQ = 0;                   // Q of slot 0, slot 1
constexpr int kRingG = 2 * kTileBytes;      // dO of slot 0, slot 1
constexpr int kRingD = 4 * kTileBytes;      // D: slot 0 (32 floats), slot 1
constexpr int kRingL = kRingD + 256;        // lse * log2(e), likewise
constexpr int kRingBias = kRingL + 256;     // 64 floats per wave
constexpr int kRingStage = kRingBias + kKvWaves * 256;

__device__ __forceinline__ int swz(int r) { return lds_swz(r); }

// a ^ k computed where it is used (k a constant).  Left to itself the compiler computes such
// loop-invariant lane addresses once, keeps them in registers the kernel does not have, and
// reloads them from scratch inside the loop, whose wait also waits for the DMA in flight.
__device__ __forceinline__ uint32_t xor_at(uint32_t a, uint32_t k) {
  uint32_t r;
  asm volatile("v_xor_b32_e32 %0, %1, %2" : "=v"(r) : "i"(k), "v"(a));
  return r;
}

// A wave-uniform value held in a scalar register at this point, so that the vector
// instruction using it reads it there rather than from a hoisted (and spilled) vector copy.
__device__ __forceinline__ uint32_t sgpr_at(uint32_t x) {
  x = __builtin_amdgcn_readfirstlane(x);
  asm volatile("" : "+s"(x));
  return x;
}

// Query steps (32-query tiles) that see key block blk of the key-stationary pass.
__device__ __forceinline__ int kv_block_steps(const BackwardParams& p, int blk) {
  const int off = p.Lk - p.Lq;
  const int Weff = p.window > 0 ? p.window : 0x40000000;
  const int J0 = blk * kKvKeys;
  const int q_lo = max(0, J0 - off);
  const int q_hi = (int)min((long long)p.Lq - 1, (long long)J0 + kKvKeys - 1 + Weff - 1 - off);
  return q_lo <= q_hi ? q_hi / 32 - q_lo / 32 + 1 : 0;
}

// base + off computed here, as one value: the compiler would otherwise fold a per-tile scalar
// base into every per-lane address separately (two vector operations per address).
__device__ __forceinline__ uint32_t base_at(uint32_t base, uint32_t off) {
  uint32_t r;
  asm volatile("v_add_u32_e32 %0, %1, %2" : "=v"(r) : "s"(__builtin_amdgcn_readfirstlane(base)), "v"(off));
  return r;
}

// The lane's index, read where it is used (a value the compiler cannot keep across a loop).
__device__ __forceinline__ uint32_t lane_now() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Direct-to-LDS load of bias-slice entries: lane i stores at LDS byte lds + 4 i the entry at
// table offset idx (bytes, from `table`) when ok, else -inf.  Both loads take a scalar base.
__device__ __forceinline__ void dma4_bias_or_neginf(const float* table, uint32_t idx_bytes, bool ok, uint32_t lds) {
  if (ok) dma4s(table, idx_bytes, lds);
  else dma4s(&kNegInfF, 0u, lds);
}

// Unit u0 of the key-stationary pass (workgroup u0 of the grid); kv_lds holds K then V of its
// 128 keys (64 KB), ring the two stages of query tiles.
__device__ __forceinline__ void dkdv_work(const BackwardParams& p, const int u0, unsigned char* kv_lds,
                                          unsigned char* ring) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wave & 3, slot = wave >> 2;
  const int col = lane & 31, hf = lane >> 5;
  // One workgroup per unit: a key block's query steps, for one head pair and KV head, cut
  // into kv_chunks (1 or 2) chunks of kv_chunk steps.  Launch order: chunk, then key block,
  // then the head pairs and KV heads.  Workgroup i runs on XCD i % 8 and, within it, on a
  // shader engine fixed by its position, only the compute unit being picked as one frees up;
  // this order gives every shader engine the same mix of units, heaviest first (later blocks
  // see fewer queries, second chunks are lighter); the host picks the number of chunks.
  const int per_block = p.n_pairs * p.Hkv * p.B;
  const int n_blk = (p.Lk + kKvKeys - 1) / kKvKeys;
  auto unit = [&](const int u) {
  const int chunk = __builtin_amdgcn_readfirstlane(u / (n_blk * per_block));
  const int blk = __builtin_amdgcn_readfirstlane((u / per_block) % n_blk);
  const int rem = u % per_block;
  const int hp = __builtin_amdgcn_readfirstlane(rem % p.n_pairs);
  const int hk = __builtin_amdgcn_readfirstlane((rem / p.n_pairs) % p.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(rem / (p.n_pairs * p.Hkv));
  const int J0 = blk * kKvKeys;
  const int j0w = J0 + 32 * kb;
  const int Lq = p.Lq, Lk = p.Lk, off = Lk - Lq;
  const int Weff = p.window > 0 ? p.window : 0x40000000;
  const bool has_head = 2 * hp + slot < p.G;
  const int h = hk * p.G + min(2 * hp + slot, p.G - 1);  // a wave without a head loads slot 0's
  const int h_slot0 = hk * p.G + 2 * hp;
  const int h_slot1 = hk * p.G + min(2 * hp + 1, p.G - 1);
  // query tiles that see a key of the workgroup: positions J0 .. J0 + 127 + W - 1
  const int q_lo = max(0, J0 - off);
  const int q_hi = (int)min((long long)Lq - 1, (long long)J0 + kKvKeys - 1 + Weff - 1 - off);
  // this chunk's query tiles: t_lo .. t_lo + n_steps - 1 (wave-uniform; scalar registers)
  const int all_steps = q_lo <= q_hi ? q_hi / 32 - q_lo / 32 + 1 : 0;
  if (chunk == 1 && all_steps <= p.kv_chunk) return;  // the block has one chunk
  const int t_lo = __builtin_amdgcn_readfirstlane(q_lo / 32 + chunk * p.kv_chunk);
  const int n_steps = __builtin_amdgcn_readfirstlane(min(all_steps - chunk * p.kv_chunk, p.kv_chunk));
  const size_t q_row = (size_t)p.Hq * 256;   // bytes between queries of a head
  const size_t kv_row = (size_t)p.Hkv * 256;
  const unsigned char* zero_bytes = (const unsigned char*)kZeroRowB;
  const uint32_t kv_base = lds_addr(kv_lds);
  const uint32_t ring_base = lds_addr(ring);

  // ---- K and V of the workgroup's keys (keys past Lk: zero rows) --------------------
  {
    const unsigned char* kg = (const unsigned char*)p.k + (((size_t)b * Lk + J0) * p.Hkv + hk) * 256;
    const unsigned char* vg = (const unsigned char*)p.v + (((size_t)b * Lk + J0) * p.Hkv + hk) * 256;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = 8 * wave + i;  // instruction g of 64: K rows 4 g .. (g < 32), else V
      const int m = g & 31;
      const int r = 4 * m + (lane >> 4);
      const int c = (lane & 15) ^ swz(r);
      const unsigned char* src = (g < 32 ? kg : vg) + (size_t)r * kv_row + 16 * c;
      if (J0 + r >= Lk) src = zero_bytes + 16 * c;
      dma16(src, kv_base + (g < 32 ? 0 : kKvKeys * 256) + m * 1024);
    }
  }

  // ---- per-step loads ---------------------------------------------------------------
  // Q / dO tiles: wave w issues rows 16 (w & 1) .. + 15 of tile T = w >> 1 (Q slot 0, Q slot
  // 1, dO slot 0, dO slot 1), four rows per instruction; lane i of instruction n fetches
  // logical chunk (i & 15) ^ swz(row) of row 16 (w & 1) + 4 n + i / 16.
  // Row 16 (w & 1) + 4 n + i / 16 has swizzle 4 (i / 16) + n, so instruction n's lane offset
  // is voff0 ^ 16 n plus the uniform 4 n rows.
  const int T = wave >> 1;
  const uint32_t voff0 = (uint32_t)(16 * (wave & 1) + (lane >> 4)) * (uint32_t)q_row +
                         16u * (uint32_t)((lane & 15) ^ ((lane >> 4) << 2));
  const int hT = (T & 1) ? h_slot1 : h_slot0;
  // this wave's tile rows of step 0; step s adds s * 32 rows (kept scalar)
  const unsigned char* tsrc0 = (const unsigned char*)uniform_ptr(
      (const unsigned char*)(T < 2 ? p.q : p.dout) + (size_t)hT * 256 + ((size_t)b * Lq + t_lo * 32) * q_row);
  const size_t step_bytes = 32 * q_row;
  // D / lse * log2(e) rows of slot 0's head (waves 0, 1); lanes 32-63 read slot 1's head,
  // Lq rows further when it is another head
  const float* drow0 = (const float*)uniform_ptr((wave == 0 ? p.D : p.L2) + ((size_t)b * p.Hq + h_slot0) * Lq);
  const uint32_t d_half = __builtin_amdgcn_readfirstlane(h_slot1 != h_slot0 ? (uint32_t)Lq : 0u);
  const float* bias_h = (const float*)uniform_ptr(p.bias_s + (size_t)h * p.Rs);
  auto issue_step = [&](int s, int st) {
    const int q0 = (t_lo + s) * 32;
    const uint32_t stage = ring_base + st * kRingStage;
    const unsigned char* src = tsrc0 + (size_t)s * step_bytes;
    const uint32_t dst = stage + (T < 2 ? kRingQ : kRingG) + (T & 1) * kTileBytes + (wave & 1) * 4096;
    if (q0 + 32 <= Lq) {
#pragma unroll
      for (int n = 0; n < 4; ++n) dma16s(src + (size_t)(4 * n) * q_row, xor_at(voff0, 16u * n), dst + n * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int r = 16 * (wave & 1) + 4 * n + (lane >> 4);
        const unsigned char* a = src + (size_t)(4 * n) * q_row + (voff0 ^ (16u * n));
        if (q0 + r >= Lq) a = zero_bytes + 16 * ((lane & 15) ^ swz(r));
        dma16(a, dst + n * 1024);
      }
    }
    if (wave < 2) {
      // D (wave 0) or lse * log2(e) (wave 1) of the tile's 32 queries, for both slots; rows
      // past Lq: D = 0, lse * log2(e) = +inf
      const uint32_t l = lane_now();
      const uint32_t d_lane = 4u * ((l & 31) + (l >> 5) * sgpr_at(d_half));
      if (q0 + 32 <= Lq) {
        dma4s(uniform_ptr(drow0 + q0), d_lane, stage + (wave == 0 ? kRingD : kRingL));
      } else {
        const int t = q0 + (int)(l & 31);
        const float* a = (const float*)((const unsigned char*)(drow0 + q0) + d_lane);
        if (t >= Lq) a = wave == 0 ? (const float*)kZeroRowB : &kPosInfF;
        dma4(a, stage + (wave == 0 ? kRingD : kRingL));
      }
    }
    // this wave's bias slice in score units: entry e = sqrt(128) r[h, min(d, R - 1)] at
    // distance d = dbase + e, the distance of query e - 31 + jj of the tile to key jj of the
    // block; -inf where no visible pair has distance d (entries past the table's Rs hold no
    // pair's distance: clamped into it)
    const int d = off + q0 - j0w - 31 + (int)lane_now();
    dma4_bias_or_neginf(bias_h, 4u * (uint32_t)min(d, (int)sgpr_at(p.Rs - 1)), (uint32_t)d < sgpr_at(Weff),
                        stage + kRingBias + wave * 256);
  };

  // ---- per-lane LDS operand addresses -----------------------------------------------
  // row read (A and B operands): row (lane & 31), logical chunk 2 ks + hf, at
  // rowA ^ (32 ks) from the tile base
  const uint32_t rowA = (uint32_t)col * 256u + 16u * (uint32_t)(hf ^ swz(lane & 15));
  // transposed read (B operand of dV and dK): rows 16 qs + 4 hf + (m >> 2) (+ 8), columns
  // 32 db + 16 u + 4 (m & 3), at (tr1 or tr2) ^ (64 db) + 4096 qs from the tile base
  uint32_t tr1, tr2;
  {
    const int m = lane & 15, u = (lane >> 4) & 1;
    const int y = 2 * u + ((m & 3) >> 1);
    const int r1 = 4 * hf + (m >> 2), r2 = r1 + 8;
    tr1 = (uint32_t)(r1 * 256 + 16 * (y ^ swz(r1)) + 8 * (m & 1));
    tr2 = (uint32_t)(r2 * 256 + 16 * (y ^ swz(r2)) + 8 * (m & 1));
  }
  const uint32_t ka = kv_base + 32u * 256u * kb + rowA;  // this wave's K rows; V 32 KB further

  f32x16_t dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dk[db] = dv[db] = zero_f32x16();

  auto compute_step = [&](int s, int st) {
    const int q0 = (t_lo + s) * 32;
    const int pq0 = off + q0;  // position of the tile's query 0
    // does any query of the tile see a key of this wave's block?
    if (!has_head || pq0 + 31 < j0w || pq0 - (Weff - 1) > j0w + 31) return;
    const uint32_t stage = ring_base + st * kRingStage;
    const uint32_t qt = stage + kRingQ + slot * kTileBytes;
    const uint32_t gt = stage + kRingG + slot * kTileBytes;
    // Four phases, each kept together by a scheduling barrier so that no phase's operand
    // loads are hoisted into an earlier one (the wave has no registers to spare), while each
    // phase's vector work overlaps its own products:
    //   1. S = Q K^T;  2. dP = dO V^T, with P from S;  3. dV += P^T dO, with dS from dP;
    //   4. dK += dS^T Q.
    // S and dP have the tile's queries as rows and the lane's key as column: register r holds
    // query qq = 8 (r >> 2) + 4 hf + (r & 3), whose bias entry is slice entry qq - col + 31.
    // Tile and block bases are multiples of 256 bytes, so (base + lane offset) ^ (32 ks) is the
    // swizzled address of chunk 2 ks + hf; dO sits 16 KB after Q, V 32 KB after K.
    // S starts from the bias in score units (register r: slice entry qq - col + 31, ascending
    // in r, so consecutive registers load in pairs straight into the accumulator).
    const uint32_t qa = qt + rowA;
    const uint32_t bsl = stage + kRingBias + wave * 256 + 4u * (uint32_t)(4 * hf - col + 31);
    f32x16_t sacc, dpacc = zero_f32x16();
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = lds_ldf(bsl + 4u * (8 * (r >> 2) + (r & 3)));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      sacc = mfma_32x32x16(lds_ld16(qa ^ (32u * ks)), lds_ld16(xor_at(ka, 32u * ks)), sacc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      dpacc = mfma_32x32x16(lds_ld16((qa ^ (32u * ks)) + 2 * kTileBytes),
                            lds_ld16(xor_at(ka, 32u * ks) + kKvKeys * 256), dpacc);
    const uint32_t ll_addr = stage + kRingL + slot * 128 + 16 * hf;
    float pr[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4_t lq4 = __builtin_bit_cast(f32x4_t, lds_ld16(ll_addr + 32 * g));
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) pr[4 * g + c4] = fast_exp2(fmaf(sacc[4 * g + c4], p.scale_log2, -lq4[c4]));
    }
    const u32x4_t ap0 = pack_p_operand(pr), ap1 = pack_p_operand(pr + 8);
    __builtin_amdgcn_sched_barrier(0);
    // dV += P^T dO (rows: keys, the lane's P; columns: dims, dO read transposed).  All sixteen
    // transposed reads of a phase go out before its products (S and dP, dead by now, leave the
    // registers), instead of one product ahead.
    const uint32_t t1 = qt + tr1, t2 = qt + tr2;
    u32x4_t top[8];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t o1 = (t1 ^ (64u * db)) + 4096u * qs + 2 * kTileBytes;
        const uint32_t o2 = (t2 ^ (64u * db)) + 4096u * qs + 2 * kTileBytes;
        const u32x2_t g1 = lds_tr8(o1), g2 = lds_tr8(o2);
        top[4 * qs + db] = u32x4_t{g1[0], g1[1], g2[0], g2[1]};
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int db = 0; db < 4; ++db) dv[db] = mfma_32x32x16(qs ? ap1 : ap0, top[4 * qs + db], dv[db]);
    const uint32_t dl_addr = stage + kRingD + slot * 128 + 16 * hf;
    float ds[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4_t dq4 = __builtin_bit_cast(f32x4_t, lds_ld16(dl_addr + 32 * g));
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) ds[4 * g + c4] = pr[4 * g + c4] * (dpacc[4 * g + c4] - dq4[c4]);
    }
    const u32x4_t as0 = pack_p_operand(ds), as1 = pack_p_operand(ds + 8);
    __builtin_amdgcn_sched_barrier(0);
    // dK += dS^T Q (Q read transposed)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t o1 = (t1 ^ (64u * db)) + 4096u * qs, o2 = (t2 ^ (64u * db)) + 4096u * qs;
        const u32x2_t x1 = lds_tr8(o1), x2 = lds_tr8(o2);
        top[4 * qs + db] = u32x4_t{x1[0], x1[1], x2[0], x2[1]};
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int db = 0; db < 4; ++db) dk[db] = mfma_32x32x16(qs ? as1 : as0, top[4 * qs + db], dk[db]);
  };

  // ---- the query-tile loop: step s computed from stage s & 1 while step s + 1 loads ----
  if (n_steps > 0) issue_step(0, 0);
  for (int s = 0; s < n_steps; ++s) {
    vm_wait<0>();  // this wave's loads of step s (and, on the first step, of K and V)
    wg_barrier();  // every wave's loads of step s are in LDS; every wave is done with step s - 1
    if (s + 1 < n_steps) issue_step(s + 1, (s + 1) & 1);
    compute_step(s, s & 1);
  }
  vm_wait<0>();

  // ---- slot 1 hands its sums to slot 0; slot 0 writes the pair's partial ---------------
  // accumulator register 4 i + c of block db: key 8 i + 4 hf + c of the block, dim 32 db + col
  float* red = (float*)ring;
  const size_t part_row = (((size_t)chunk * p.n_pairs + hp) * p.B + b) * Lk;
  auto hand_over = [&](f32x16_t (&acc)[4], float* part) {
    __syncthreads();  // every wave is done with the ring
    if (slot == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((kb * 4 + db) * 16 + r) * 64 + lane] = acc[db][r];
    }
    __syncthreads();
    if (slot == 0) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0w + 8 * (r >> 2) + 4 * hf + (r & 3);
          const float x = acc[db][r] + red[((kb * 4 + db) * 16 + r) * 64 + lane];
          if (j < Lk) part[((part_row + j) * p.Hkv + hk) * kHeadDim + 32 * db + col] = x;
        }
    }
  };
  hand_over(dk, p.part_dk);
  hand_over(dv, p.part_dv);
  };
  unit(u0);
}

// dk = (sum over head pairs of the partial dK) / sqrt(128), dv = sum of the partial dV, in
// pair order, a pair's second chunk (blocks walked in two) right after its first; four
// consecutive floats per thread.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BackwardParams p, size_t n4) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const size_t plane = (size_t)p.B * p.Lk * p.Hkv * kHeadDim;
  const int j = (int)((i / ((size_t)p.Hkv * 32)) % (size_t)p.Lk);
  const bool two = kv_block_steps(p, j / kKvKeys) > p.kv_chunk;
  f32x4_t a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
  for (int hp = 0; hp < p.n_pairs; ++hp) {
    a += ((const f32x4_t*)(p.part_dk + (size_t)hp * plane))[i];
    c += ((const f32x4_t*)(p.part_dv + (size_t)hp * plane))[i];
    if (two) {
      a += ((const f32x4_t*)(p.part_dk + (size_t)(p.n_pairs + hp) * plane))[i];
      c += ((const f32x4_t*)(p.part_dv + (size_t)(p.n_pairs + hp) * plane))[i];
    }
  }
  ((f32x4_t*)p.dk)[i] = a * kRsqrtD;
  ((f32x4_t*)p.dv)[i] = c;
}

// ---- query-stationary pass (dQ, dr) -----------------------------------------------------
// The forward's decomposition: a workgroup of 8 waves owns one KV head, hpw of its query heads
// and 32 * tsub queries (hpw * tsub = 8); each wave owns one query head x 32 queries, its Q^T
// and dO^T operands resident in registers, and walks the 32-key tiles its workgroup sees.
// K, V and each wave's 64-entry slice of the bias table in score units are loaded straight
// into LDS (global_load_lds) through a ring of three stages, two tiles ahead, and serve every
// wave (GQA packing).  Per tile a wave computes dP^T = V dO^T and S^T = K Q^T (seeded with the
// bias) with one query per lane (the accumulator column), P and dS, dQ^T += K^T dS^T (K read
// transposed; dQ stays in registers and is stored once), and sums dS along the tile's 63
// diagonals through a skewed table in LDS (row = diagonal, column = the lane's query, 34 floats
// per row) into dr: a diagonal that continues into the next key tile carries its sum there,
// and each finished diagonal is one fp32 atomic add.  K rows are read both row-wise and
// transposed: the tile uses the swizzle of the key-stationary pass.
constexpr int kDqWaves = 8;
constexpr int kDqStages = 3;
constexpr int kDqKV = 32 * 256;                       // a K (or V) tile: 32 keys x 256 B
constexpr int kDqBias = 2 * kDqKV;                    // bias slices: 64 floats per wave
constexpr int kDqStage = kDqBias + kDqWaves * 256;
constexpr int kDqLoads = 3;

constexpr int kDqRing = kDqStages * kDqStage;
constexpr int kDqDiag = kDqWaves * 63 * kDiagStride * 4;

// Unit u0 of the query-stationary pass (workgroup kv_units + u0 of the grid); ring holds the
// three stages of K/V tiles and bias slices, diag_w a distance table per wave, merges the flag
// of a workgroup that finishes a split token tile second.
__device__ __forceinline__ void dq_work(const BackwardParams& p, const int u0, unsigned char* ring,
                                        float (*diag_w)[63 * kDiagStride], int& merges) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  // dS of a tile by diagonal: row e = col - jj + 31 (distance dbase + e), column col (the
  // query).  The cells of row e that no pair maps to (columns outside e - 31 .. e) are the
  // same in every tile and never written: zeroed once, they let a row sum take all 32 columns.
  float* diag = diag_w[wave];
  for (int i = lane; i < 63 * kDiagStride; i += 64) diag[i] = 0.f;  // this wave's own table
  // One workgroup per unit: a token tile's key tiles, for one head group and KV head, cut into
  // q_chunks (1 or 2) chunks of q_chunk; a tile cut in two is merged by whichever of its chunks
  // finishes second (at the end of the unit).  Launch order: chunk, then token tile (heaviest,
  // last, first), then the head groups and KV heads (see the key-stationary pass for why).
  const int per_tile = p.B * p.Hkv * p.n_hg;
  auto unit = [&](const int u) {
  const int chunk = __builtin_amdgcn_readfirstlane(u / (p.n_tok_tiles * per_tile));
  const int tile = __builtin_amdgcn_readfirstlane(p.n_tok_tiles - 1 - (u / per_tile) % p.n_tok_tiles);
  const int rem = __builtin_amdgcn_readfirstlane(u % per_tile);
  const int hg = rem % p.n_hg;
  const int hk = (rem / p.n_hg) % p.Hkv;
  const int b = rem / (p.n_hg * p.Hkv);
  const int h = hk * p.G + hg * p.hpw + (wave % p.hpw);
  const int Lq = p.Lq, Lk = p.Lk, off = Lk - Lq;
  const int T0 = tile * 32 * p.tsub;
  const int T1 = min(Lq, T0 + 32 * p.tsub);
  const int q0 = T0 + (wave / p.hpw) * 32;  // this wave's first query
  const int nq = min(32, Lq - q0);         // its queries (may be <= 0)
  const int Weff = p.window > 0 ? p.window : 0x40000000;
  const bool qvalid = col < nq;
  const size_t q_row = (size_t)p.Hq * kHeadDim;
  const size_t row0 = ((size_t)b * Lq + q0) * p.Hq + h;
  // Q^T and dO^T operands (lane: its query, dims 16 ks + 8 hf ..), resident for the key loop
  u32x4_t qr[8], gr[8];
  {
    const size_t rq = row0 + (size_t)(qvalid ? col : 0) * p.Hq;
    const uint16_t* qs = (const uint16_t*)p.q + rq * kHeadDim + 8 * hf;
    const uint16_t* gs = (const uint16_t*)p.dout + rq * kHeadDim + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qr[ks] = qvalid ? *(const u32x4_t*)(qs + 16 * ks) : zero_u32x4();
      gr[ks] = qvalid ? *(const u32x4_t*)(gs + 16 * ks) : zero_u32x4();
    }
  }
  const size_t drow = ((size_t)b * p.Hq + h) * Lq + q0 + col;  // D and lse * log2(e): head-major
  // a lane past Lq: lse * log2(e) = +inf makes its P (hence dS) zero
  float lse2 = qvalid ? p.L2[drow] : __builtin_inff();
  float dd = qvalid ? p.D[drow] : 0.f;
  // pin the waits for these loads here, before any LDS-bound load is in flight
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(qr[ks]), "+v"(gr[ks]));
  asm volatile("" : "+v"(lse2), "+v"(dd));
  const int pq = off + q0 + col;  // this lane's query position
  float* dbias_h = p.dbias + (size_t)h * p.R;
  // key tiles of the workgroup's chunk, and of this wave
  const int all_tiles = (off + T1 - 1) / 32 + 1 - max(0, off + T0 - Weff + 1) / 32;
  if (chunk == 1 && all_tiles <= p.q_chunk) return;  // the tile has one chunk
  const int kt_begin = __builtin_amdgcn_readfirstlane(max(0, off + T0 - Weff + 1) / 32 + chunk * p.q_chunk);
  const int n_tiles = __builtin_amdgcn_readfirstlane(min(all_tiles - chunk * p.q_chunk, p.q_chunk));
  const int wj_lo = max(0, off + q0 - Weff + 1), wj_hi = off + q0 + max(nq, 1) - 1;

  // ---- tile loads: waves 0-3 issue K, waves 4-7 V, two instructions of 4 keys each ----
  const size_t kv_row = (size_t)p.Hkv * 256;  // bytes between keys
  const unsigned char* kvg = (const unsigned char*)(wave < 4 ? p.k : p.v) + ((size_t)b * Lk * p.Hkv + hk) * 256;
  const unsigned char* zero_bytes = (const unsigned char*)kZeroRowB;
  const uint32_t ring_base = lds_addr(ring);
  uint32_t koff[2];
  int krow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * (2 * (wave & 3) + i) + (lane >> 4);
    krow[i] = r;
    koff[i] = (uint32_t)r * (uint32_t)kv_row + 16u * (uint32_t)((lane & 15) ^ swz(r));
  }
  auto issue_tile = [&](int kt, int st) {
    const int j0 = kt * 32;
    const uint32_t stage = ring_base + st * kDqStage;
    const uint32_t dst = stage + (wave < 4 ? 0 : kDqKV) + (wave & 3) * 2048;
    const unsigned char* base = uniform_ptr(kvg + (size_t)j0 * kv_row);
    if (j0 + 32 <= Lk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16s(base, koff[i], dst + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const unsigned char* a = base + koff[i];
        if (j0 + krow[i] >= Lk) a = zero_bytes + 16 * ((lane & 15) ^ swz(krow[i]));
        dma16(a, dst + i * 1024);
      }
    }
    // this wave's bias slice in score units, reversed: position 63 - e holds entry
    // e = sqrt(128) r[h, min(d, R - 1)] at distance d = dbase + e; -inf where no visible pair has
    // distance d (entries past the table's Rs hold no pair's distance: clamped into it)
    const int d = off + q0 - j0 - 31 + (63 - lane);
    dma4((uint32_t)d < (uint32_t)Weff ? p.bias_s + (size_t)h * p.Rs + min(d, p.Rs - 1) : &kNegInfF,
         stage + kDqBias + wave * 256);
  };

  // ---- per-lane LDS operand addresses (tile-relative, as in the key-stationary pass) ----
  const uint32_t rowA = (uint32_t)col * 256u + 16u * (uint32_t)(hf ^ swz(lane & 15));
  uint32_t tr1, tr2;
  {
    const int m = lane & 15, u = (lane >> 4) & 1;
    const int y = 2 * u + ((m & 3) >> 1);
    const int r1 = 4 * hf + (m >> 2), r2 = r1 + 8;
    tr1 = (uint32_t)(r1 * 256 + 16 * (y ^ swz(r1)) + 8 * (m & 1));
    tr2 = (uint32_t)(r2 * 256 + 16 * (y ^ swz(r2)) + 8 * (m & 1));
  }

  f32x16_t dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dq[db] = zero_f32x16();
  // dr sums carried from one key tile to the next (lanes 32..62), at distance carry_base + lane
  float carry = 0.f;
  int carry_base = 0;

  auto compute_tile = [&](int kt, int st) {
    const int j0 = kt * 32;
    if (!(nq > 0) || j0 > wj_hi || j0 + 31 < wj_lo) return;
    const uint32_t stage = ring_base + st * kDqStage;  // (wave-uniform)
    const uint32_t kt_lds = stage;
    // S^T starts from the bias in score units.  Register r of an accumulator holds key j0 + jj,
    // jj = 8 (r >> 2) + 4 hf + (r & 3); its seed is slice entry col - jj + 31, at position
    // 32 - col + jj = (32 - col + 4 hf) + x_r, x_r = 8 (r >> 2) + (r & 3): ascending in r, so
    // consecutive registers load in pairs straight into the accumulator.  The seeds go out
    // first; dP^T runs before S^T, so that their latency is spent on its products.
    const uint32_t bsl = base_at(stage + kDqBias + wave * 256, 4u * (uint32_t)(32 - col + 4 * hf));
    f32x16_t st_acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) st_acc[r] = lds_ldf(bsl + 4u * (8 * (r >> 2) + (r & 3)));
    // dP^T = V dO^T, then S^T = K Q^T: rows are keys, the lane's column is its query.  The
    // stage base is a multiple of 256 bytes, so (base + lane offset) ^ (32 ks) is the swizzled
    // address of chunk 2 ks + hf; V sits 8 KB after K.  The eight V operands are read ahead of
    // their products and each register takes its K operand once its product has issued
    // (scheduling barriers hold this order; left to itself the scheduler fed every product
    // through one register, a full LDS latency each).
    const uint32_t ka = base_at(kt_lds, rowA);
    f32x16_t dpt = zero_f32x16();
    u32x4_t op[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) op[ks] = lds_ld16((ka ^ (32u * ks)) + kDqKV);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) dpt = mfma_32x32x16(op[ks], gr[ks], dpt);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) op[ks] = lds_ld16(ka ^ (32u * ks));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) st_acc = mfma_32x32x16(op[ks], qr[ks], st_acc);
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      ds[r] = fast_exp2(fmaf(st_acc[r], p.scale_log2, -lse2)) * (dpt[r] - dd);
    // table cell (row col - jj + 31, column col): from the cell of x_r = 27, 34 (27 - x_r) further
    float* const dcell = diag + (col - 4 * hf + 4) * kDiagStride + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) dcell[kDiagStride * (27 - (8 * (r >> 2) + (r & 3)))] = ds[r];
    // dr: lane e < 63 sums row e of the table (the pairs at distance dbase + e; invisible pairs
    // hold zero), with its reads free to overlap the dQ products below.  The table is this
    // wave's own and the LDS serves a wave's requests in order, so only the compiler's order
    // is kept here.
    lds_order();
    float x;
    {
      const float* row = diag + min(lane, 62) * kDiagStride;
      f32x2_t acc = {0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 32; c += 2) acc += *(const f32x2_t*)(row + c);
      x = lane < 63 ? acc[0] + acc[1] : 0.f;
    }
    // dQ^T += K^T dS^T: rows are dims (K read transposed), the lane's column its query
    const uint32_t t1 = base_at(kt_lds, tr1), t2 = base_at(kt_lds, tr2);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t bs = pack_p_operand(ds + 8 * ks);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t o1 = (t1 ^ (64u * db)) + 4096u * ks, o2 = (t2 ^ (64u * db)) + 4096u * ks;
        const u32x2_t a1 = lds_tr8(o1), a2 = lds_tr8(o2);
        dq[db] = mfma_32x32x16(u32x4_t{a1[0], a1[1], a2[0], a2[1]}, bs, dq[db]);
      }
    }
    lds_order();  // the next tile's table stores come after the row reads
    const int dbase = off + q0 - j0 - 31;
    // Key tiles advance by 32, so the diagonals of rows e <= 30 (tile distance c = e - 31 < 0)
    // continue as rows e + 32 of the next tile: lanes 0..30 hand their sums to lanes 32..62,
    // and only rows 31..62, which no later tile reaches, are added to dr.
    const float tot = x + carry;
    // rows of the table at negative distances hold only invisible pairs: never added
    if (lane >= 31 && lane < 63 && dbase + lane >= 0 && tot != 0.f)
      unsafeAtomicAdd(dbias_h + min(dbase + lane, p.R - 1), tot);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    carry = lane >= 32 && lane < 63 ? __uint_as_float(sw[0]) : 0.f;  // lane l >= 32: row l - 32's sum
    carry_base = dbase - 32;                                           // lane l: distance carry_base + l
  };

  // ---- key loop: tile t computed from stage t % 3 while tiles t + 1, t + 2 load ----------
  const int prologue = min(2, n_tiles);
  for (int i = 0; i < prologue; ++i) issue_tile(kt_begin + i, i);
  for (int t = 0; t < n_tiles; ++t) {
    // tile t's loads are done; tile t + 1's (and at most one dr atomic) may be in flight
    if (t + 1 < n_tiles) vm_wait<kDqLoads>();
    else vm_wait<0>();
    wg_barrier();  // tile t is in LDS for every wave; every wave is done with tile t - 1
    if (t + 2 < n_tiles) issue_tile(kt_begin + t + 2, (t + 2) % kDqStages);
    compute_tile(kt_begin + t, t % kDqStages);
  }
  // the last computed tile's carried rows (the visible key tiles of a wave are contiguous, so
  // no tile it skipped lies between two it computed)
  if (lane >= 32 && lane < 63 && carry_base + lane >= 0 && carry != 0.f)
    unsafeAtomicAdd(dbias_h + min(carry_base + lane, p.R - 1), carry);
  // accumulator register 4 i + c of block db: dim 32 db + 8 i + 4 hf + c of query q0 + col
  const size_t qoff = (row0 + (size_t)col * p.Hq) * kHeadDim + 4 * hf;
  if (all_tiles <= p.q_chunk) {  // one chunk: this workgroup's dq is the result
    if (!qvalid) return;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4_t x;
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = dq[db][4 * i + c] * kRsqrtD;
        *(f32x4_t*)(p.dq + qoff + 32 * db + 8 * i) = x;
      }
    return;
  }
  // Two chunks: each writes its partial into its own slot of the workspace with device-coherent
  // stores (relaxed agent-scope atomic stores carry the sc1 bit on this target and go to the
  // coherence point, past this XCD's L2), waits for them and counts; the one that counts
  // second reads the other's slot the same way and writes dq = part 0 + part 1, the same sum
  // whichever chunk that is.  Slot layout: element e = 16 db + 4 i + c of lane l of wave w at
  // (64 w + e) * 64 + l, so each access of a wave covers 256 consecutive bytes.
  const size_t unit_c = (size_t)(u % (p.n_tok_tiles * per_tile));  // the unit within its chunk
  float* const slot = p.dq_part + (unit_c * 2 + chunk) * (kDqWaves * 64 * 64) + wave * 64 * 64 + lane;
#pragma unroll
  for (int e = 0; e < 64; ++e)
    __hip_atomic_store(slot + 64 * e, dq[e >> 4][e & 15] * kRsqrtD, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial has landed
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(p.dq_cnt + unit_c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merges = old == 1;
  }
  __syncthreads();
  if (!merges || !qvalid) return;
  const float* const other = slot + (chunk ? -1 : 1) * (kDqWaves * 64 * 64);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4_t x;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float mine = dq[db][4 * i + c] * kRsqrtD;
        const float theirs =
            __hip_atomic_load(other + 64 * (16 * db + 4 * i + c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        x[c] = chunk ? theirs + mine : mine + theirs;
      }
      *(f32x4_t*)(p.dq + qoff + 32 * db + 8 * i) = x;
    }
  };
  unit(u0);
}

constexpr int kKvLds = 2 * kKvKeys * 256 + 2 * kRingStage;
constexpr int kDqLds = kDqRing + kDqDiag + 16;
constexpr int kPassLds = kKvLds > kDqLds ? kKvLds : kDqLds;
static_assert(64 * kKvWaves == 64 * kDqWaves, "one workgroup size for both passes");

// One workgroup per unit of either pass: the kv_units key-stationary units first (they take
// about 1.1 times as long per step), then the query-stationary ones, each in its own launch
// order.  LDS holds one pass's buffers at a time: K, V and the query ring, or the K/V ring,
// the distance tables and the split flag.
__global__ __launch_bounds__(64 * kDqWaves, 1) void bwd_passes_kernel(BackwardParams p, int kv_units) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kPassLds];
  const int i = blockIdx.x;
  if (i < kv_units) {
    dkdv_work(p, i, lds, lds + kKvKeys * 512);
  } else {
    dq_work(p, i - kv_units, lds, (float(*)[63 * kDiagStride])(lds + kDqRing), *(int*)(lds + kDqRing + kDqDiag));
  }
}

}  // namespace

hipError_t launch_backward(const BackwardParams& p, hipStream_t stream) {
  const size_t n_kv = (size_t)p.B * p.Lk * p.Hkv * kHeadDim;
  const size_t n_r = (size_t)p.Hq * p.R;
  auto fill = [&](float* a, size_t n) {
    if (n == 0) return;
    const size_t blocks = std::min((n + 255) / 256, (size_t)4096);
    hipLaunchKernelGGL(bwd_fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n);
  };
  const size_t n_cnt = (size_t)std::max(p.n_tok_tiles, 0) * std::max(p.B, 0) * p.Hkv * p.n_hg;
  if (p.B <= 0 || p.Lq <= 0 || p.Lk <= 0) {
    if (n_r > 0 || n_cnt > 0) {
      const size_t blocks = std::max<size_t>(1, std::min((std::max(n_r, n_cnt) + 255) / 256, (size_t)4096));
      hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n_r, n_cnt);
    }
    fill(p.dk, n_kv);
    fill(p.dv, n_kv);
    return hipGetLastError();
  }
  const int n_tb = (p.Lq + kRowdotRows - 1) / kRowdotRows;
  const size_t rowdot_blocks = (size_t)p.B * p.Hq * n_tb;
  if (rowdot_blocks > 0x7fffffffULL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_rowdot_kernel, dim3((unsigned)rowdot_blocks), dim3(256), 0, stream, p, n_tb, n_r, n_cnt);
  const long long kv_units = (long long)((p.Lk + kKvKeys - 1) / kKvKeys) * p.kv_chunks * p.Hkv * p.n_pairs * p.B;
  const long long q_units = (long long)p.n_tok_tiles * p.q_chunks * p.B * p.Hkv * p.n_hg;
  const size_t n4 = n_kv / 4;
  if (kv_units + q_units > 0x7fffffffLL || (n4 + 255) / 256 > 0x7fffffffULL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_passes_kernel, dim3((unsigned)(kv_units + q_units)), dim3(64 * kDqWaves), 0, stream, p,
                     (int)kv_units);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, p, n4);
  return hipGetLastError();
}

}  // namespace rattn
