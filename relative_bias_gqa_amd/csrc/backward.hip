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
// Three passes on the caller's stream, after a fill that zeroes dk, dv and dr:
//   1. D per query row (fp32, from the bf16 out and dout);
//   2. key-stationary: one wave per (32 keys, query head), two heads of a KV head per
//      workgroup sharing the K/V tiles, walks the query tiles that see its keys; S = Q K^T
//      and dP = dO V^T come out with one key per lane (the accumulator column), which is
//      the register layout the A operand of dV += P^T dO and dK += dS^T Q needs, so P and
//      dS feed the MFMAs straight from registers; dO and Q are read transposed from LDS for
//      the B operand.  dK and dV of the wave's head are added into dk, dv at the end (fp32
//      atomics, one add per element per query head);
//   3. query-stationary: one wave per (32 queries, query head), paired the same way, walks
//      the key tiles its queries see; S^T and dP^T come out with one query per lane, the
//      B-operand layout of dQ^T += K^T dS^T, so dQ is accumulated in registers and stored
//      once; dS is also summed per distance through a skewed table in LDS (one row per
//      diagonal of the 32 x 32 tile) and the 63 row sums added into dr.
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS are rounded to
// bf16 as MFMA operands.  Tiles sit in LDS with 272-byte rows (256 bytes of data and 16 of
// padding) so that the row-wise operand reads of 32 consecutive rows spread over the banks.
#include <algorithm>

#include "backward.hpp"
#include "device_common.hpp"

namespace rattn {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRows = 32;                  // keys or queries per wave tile
constexpr int kStride = 136;               // LDS row stride of a 128-wide bf16 tile (elements)
constexpr int kTileElems = kRows * kStride;
constexpr float kRsqrtD = 0.08838834764831845f;  // 1 / sqrt(128)
constexpr int kDiagStride = 34;            // floats per row of the diagonal table (conflict free)

// The 63 bias entries a 32 x 32 tile meets: entry e = r[h, clamp(dbase + e, 0, R - 1)] for the
// pairs at distance dbase + e, dbase = (distance of query 0 to key 31).  Lanes 0..62 load one.
__device__ __forceinline__ void stage_bias(float* band, const float* bias_h, int dbase, int R, int lane) {
  if (lane < 63) band[lane] = bias_h[min(max(dbase + lane, 0), R - 1)];
}

// 32 rows of 128 bf16 from global memory (row r at src + r * row_stride) into an LDS tile;
// rows at or past n_valid are zero.  One wave, 16 bytes per lane per pass.
__device__ __forceinline__ void load_tile(uint16_t* tile, const uint16_t* src, size_t row_stride, int n_valid,
                                          int lane) {
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const int idx = pass * 64 + lane;
    const int row = idx >> 4, c = idx & 15;
    u32x4_t x = zero_u32x4();
    if (row < n_valid) x = *(const u32x4_t*)(src + row * row_stride + c * 8);
    *(u32x4_t*)(tile + row * kStride + c * 8) = x;
  }
}

// Operand of k-step ks read along rows: lane l gets row (l & 31), elements 16 ks + 8 (l >> 5)
// .. + 7.  The A operand (rows of the product) and the B operand (columns) of
// v_mfma_f32_32x32x16_bf16 both take this form when the tile is stored row by row.
__device__ __forceinline__ u32x4_t row_operand(const uint16_t* tile, int ks, int lane) {
  return *(const u32x4_t*)(tile + (lane & 31) * kStride + 16 * ks + 8 * (lane >> 5));
}

// Keeps the compiler from moving memory accesses across this point.  Used between LDS
// accesses of one wave, which the LDS performs in the wave's order.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// Work item of this workgroup.  Workgroup i of a launch runs on XCD i mod 8 (each XCD has its
// own L2), so consecutive work items (neighbouring tiles of one head pair, which read mostly
// the same Q / dO or K / V tiles at the same time) are given to one XCD: XCD x takes a
// contiguous range of the items, in launch order.  A bijection for any grid size.
struct WorkItem {
  int tile, pair, b;
};
__device__ __forceinline__ WorkItem xcd_work_item() {
  const int n = gridDim.x * gridDim.y * gridDim.z;
  const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int per = n / 8, rem = n % 8, x = L % 8;
  const int w = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + L / 8;
  WorkItem it;
  it.tile = w % gridDim.x;
  it.pair = (w / gridDim.x) % gridDim.y;
  it.b = w / (gridDim.x * gridDim.y);
  return it;
}
// The work item in launch order (consecutive tiles on consecutive XCDs).
__device__ __forceinline__ WorkItem launch_order_work_item() {
  WorkItem it;
  it.tile = blockIdx.x;
  it.pair = blockIdx.y;
  it.b = blockIdx.z;
  return it;
}

__global__ __launch_bounds__(256) void bwd_fill_zero_kernel(float* a, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) a[i] = 0.f;
}

// D[row] = sum_d dout[row, d] * out[row, d] for every (b, t, h) row, in fp32.
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t* out, const uint16_t* dout, float* D,
                                                         size_t rows) {
  const size_t row = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const u32x4_t* o = (const u32x4_t*)(out + row * kHeadDim);
  const u32x4_t* g = (const u32x4_t*)(dout + row * kHeadDim);
  float acc = 0.f;
#pragma unroll 4
  for (int c = 0; c < 16; ++c) {
    const u32x4_t x = o[c], y = g[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo_to_f32(x[i]), bf16_lo_to_f32(y[i]), acc);
      acc = fmaf(bf16_hi_to_f32(x[i]), bf16_hi_to_f32(y[i]), acc);
    }
  }
  D[row] = acc;
}

// Key-stationary pass: dK and dV.  Grid (key tiles, Hkv * ceil(G / 2), B); a workgroup is
// two waves, each one query head of the same KV head, sharing the K and V tiles.  With an odd
// G the second wave of the last pair has no head: it runs along (for the barriers) and
// writes nothing.
__global__ __launch_bounds__(2 * 64) void bwd_dkdv_kernel(BackwardParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t qt_w[2][kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t gt_w[2][kTileElems];  // dO
  __shared__ float lse_w[2][kRows];
  __shared__ float d_w[2][kRows];
  __shared__ float bias_w[2][64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  uint16_t* qt = qt_w[wave];
  uint16_t* gt = gt_w[wave];
  float* lse_s = lse_w[wave];
  float* d_s = d_w[wave];
  float* bias_s = bias_w[wave];
  const int col = lane & 31, hf = lane >> 5;
  const WorkItem it = xcd_work_item();
  const int j0 = it.tile * kRows;
  const int npair = (p.G + 1) / 2;
  const int hk = it.pair / npair;
  const int hg = 2 * (it.pair % npair) + wave;
  const bool has_head = hg < p.G;
  const int h = hk * p.G + (has_head ? hg : hg - 1);
  const int b = it.b;
  const int Lq = p.Lq, Lk = p.Lk, off = Lk - Lq;
  const int Weff = p.window > 0 ? p.window : 0x40000000;
  // queries that see a key of this tile: positions j0 .. j0 + 31 + Weff - 1
  const int q_lo = max(0, j0 - off);
  const int q_hi = (int)min((long long)Lq - 1, (long long)j0 + kRows - 1 + Weff - 1 - off);
  const size_t kv_row = (size_t)p.Hkv * kHeadDim;
  const size_t q_row = (size_t)p.Hq * kHeadDim;
  const uint16_t* kg = (const uint16_t*)p.k + ((size_t)b * Lk + j0) * kv_row + (size_t)hk * kHeadDim;
  const uint16_t* vg = (const uint16_t*)p.v + ((size_t)b * Lk + j0) * kv_row + (size_t)hk * kHeadDim;
  load_tile(wave == 0 ? kt : vt, wave == 0 ? kg : vg, kv_row, min(kRows, Lk - j0), lane);
  const float* bias_h = p.bias + (size_t)h * p.R;
  f32x16_t dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dk[db] = dv[db] = zero_f32x16();
  const int j = j0 + col;  // this lane's key (accumulator column of S and dP)
  for (int qi = q_lo / kRows; q_lo <= q_hi && qi <= q_hi / kRows; ++qi) {
    const int q0 = qi * kRows;
    const int nq = min(kRows, Lq - q0);
    // One barrier per query tile keeps the two waves together (and, on the first tile, makes
    // the other wave's K or V tile visible).  Everything else in LDS here (Q, dO, lse, D and
    // the bias band) belongs to this wave alone, and the LDS serves one wave's requests in
    // order, so between those only the compiler's order has to be kept (lds_order).
    __syncthreads();
    const size_t row0 = ((size_t)b * Lq + q0) * p.Hq + h;
    const int dbase = off + q0 - j0 - (kRows - 1);
    stage_bias(bias_s, bias_h, dbase, p.R, lane);
    load_tile(qt, (const uint16_t*)p.q + row0 * kHeadDim, q_row, nq, lane);
    load_tile(gt, (const uint16_t*)p.dout + row0 * kHeadDim, q_row, nq, lane);
    if (lane < kRows) {
      lse_s[lane] = lane < nq ? p.lse[row0 + (size_t)lane * p.Hq] * kLog2e : 0.f;
      d_s[lane] = lane < nq ? p.D[row0 + (size_t)lane * p.Hq] : 0.f;
    }
    lds_order();
    // S = Q K^T and dP = dO V^T: rows are queries, the lane's column is key j
    f32x16_t s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s = mfma_32x32x16(row_operand(qt, ks, lane), row_operand(kt, ks, lane), s);
      dp = mfma_32x32x16(row_operand(gt, ks, lane), row_operand(vt, ks, lane), dp);
    }
    // register r holds query 8 (r >> 2) + 4 hf + (r & 3) of the tile
    float pr[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = 8 * (r >> 2) + 4 * hf + (r & 3);
      const int dist = off + q0 + qq - j;
      const bool vis = qq < nq && dist >= 0 && dist < Weff;
      const float lg = fmaf(s[r], p.scale_log2, fmaf(bias_s[qq - col + 31], kLog2e, -lse_s[qq]));
      pr[r] = vis ? fast_exp2(lg) : 0.f;
      // select, not multiply: an invisible pair stays zero even if dP - D is not finite
      ds[r] = vis ? pr[r] * (dp[r] - d_s[qq]) : 0.f;
    }
    // dV += P^T dO and dK += dS^T Q: rows are keys (the lane's P and dS), columns dims
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const u32x4_t ap = pack_p_operand(pr + 8 * qs);
      const u32x4_t as = pack_p_operand(ds + 8 * qs);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dv[db] = mfma_32x32x16(ap, load_vt_operand(gt, kStride, 16 * qs, 32 * db, lane), dv[db]);
        dk[db] = mfma_32x32x16(as, load_vt_operand(qt, kStride, 16 * qs, 32 * db, lane), dk[db]);
      }
    }
  }
  if (!has_head) return;
  // accumulator register 4 i + c of block db: key 8 i + 4 hf + c, dim 32 db + col
  float* dkg = p.dk + ((size_t)b * Lk + j0) * kv_row + (size_t)hk * kHeadDim;
  float* dvg = p.dv + ((size_t)b * Lk + j0) * kv_row + (size_t)hk * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
      if (j0 + key < Lk) {
        const size_t o = (size_t)key * kv_row + 32 * db + col;
        unsafeAtomicAdd(dkg + o, dk[db][r] * kRsqrtD);
        unsafeAtomicAdd(dvg + o, dv[db][r]);
      }
    }
}

// Query-stationary pass: dQ and dr.  Grid (query tiles, Hkv * ceil(G / 2), B); a workgroup is two
// waves, each one query head of the same KV head, sharing the K and V tiles (wave 0 loads
// K, wave 1 V).  With an odd G the second wave of the last pair runs along and stores nothing.
__global__ __launch_bounds__(2 * 64) void bwd_dq_kernel(BackwardParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kTileElems];
  __shared__ float bias_w[2][64];
  // dS of the tile by diagonal: row e = col - jj + 31 (distance dbase + e), column col (the
  // query); the cells of row e that no pair maps to (columns outside e - 31 .. e) are skipped
  __shared__ __attribute__((aligned(16))) float diag_w[2][63 * kDiagStride];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  float* bias_s = bias_w[wave];
  float* diag = diag_w[wave];
  const int col = lane & 31, hf = lane >> 5;
  // (the XCD-contiguous order measured 15 % slower here than launch order: every XCD then
  // walks one head pair's tiles from light to heavy and the heaviest come last)
  const WorkItem it = launch_order_work_item();
  const int q0 = it.tile * kRows;
  const int npair = (p.G + 1) / 2;
  const int hk = it.pair / npair;
  const int hg = 2 * (it.pair % npair) + wave;
  const bool has_head = hg < p.G;
  const int h = hk * p.G + (has_head ? hg : hg - 1);
  const int b = it.b;
  const int Lq = p.Lq, Lk = p.Lk, off = Lk - Lq;
  const int nq = min(kRows, Lq - q0);
  const int Weff = p.window > 0 ? p.window : 0x40000000;
  const size_t kv_row = (size_t)p.Hkv * kHeadDim;
  const size_t q_row = (size_t)p.Hq * kHeadDim;
  const size_t row0 = ((size_t)b * Lq + q0) * p.Hq + h;
  // this lane's query (accumulator column of S^T and dP^T)
  const bool qvalid = col < nq;
  // Q^T and dO^T operands (lane: its query, dims 16 ks + 8 hf ..), resident for the key loop
  u32x4_t qr[8], gr[8];
  {
    const uint16_t* qs = (const uint16_t*)p.q + (row0 + (size_t)(qvalid ? col : 0) * p.Hq) * kHeadDim + 8 * hf;
    const uint16_t* gs = (const uint16_t*)p.dout + (row0 + (size_t)(qvalid ? col : 0) * p.Hq) * kHeadDim + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qr[ks] = qvalid ? *(const u32x4_t*)(qs + 16 * ks) : zero_u32x4();
      gr[ks] = qvalid ? *(const u32x4_t*)(gs + 16 * ks) : zero_u32x4();
    }
  }
  const int pq = off + q0 + col;
  const float lse2 = qvalid ? p.lse[row0 + (size_t)col * p.Hq] * kLog2e : 0.f;
  const float dd = qvalid ? p.D[row0 + (size_t)col * p.Hq] : 0.f;
  const float* bias_h = p.bias + (size_t)h * p.R;
  float* dbias_h = p.dbias + (size_t)h * p.R;
  // keys the tile's queries see: positions off + q0 - Weff + 1 .. off + q0 + 31
  const int j_lo = max(0, off + q0 - Weff + 1);
  const int j_hi = min(Lk - 1, off + q0 + nq - 1);
  const uint16_t* kg = (const uint16_t*)p.k + (size_t)b * Lk * kv_row + (size_t)hk * kHeadDim;
  const uint16_t* vg = (const uint16_t*)p.v + (size_t)b * Lk * kv_row + (size_t)hk * kHeadDim;
  f32x16_t dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dq[db] = zero_f32x16();
  for (int kti = j_lo / kRows; j_lo <= j_hi && kti <= j_hi / kRows; ++kti) {
    const int j0 = kti * kRows;
    __syncthreads();  // the previous tile's reads of kt, vt and bias_s are done
    load_tile(wave == 0 ? kt : vt, (wave == 0 ? kg : vg) + (size_t)j0 * kv_row, kv_row, min(kRows, Lk - j0), lane);
    const int dbase = off + q0 - j0 - (kRows - 1);
    stage_bias(bias_s, bias_h, dbase, p.R, lane);
    __syncthreads();
    // S^T = K Q^T and dP^T = V dO^T: rows are keys, the lane's column is its query
    f32x16_t st = zero_f32x16(), dpt = zero_f32x16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      st = mfma_32x32x16(row_operand(kt, ks, lane), qr[ks], st);
      dpt = mfma_32x32x16(row_operand(vt, ks, lane), gr[ks], dpt);
    }
    // register r holds key j0 + 8 (r >> 2) + 4 hf + (r & 3)
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jj = 8 * (r >> 2) + 4 * hf + (r & 3);
      const int dist = pq - (j0 + jj);
      const bool vis = qvalid && dist >= 0 && dist < Weff;
      const float lg = fmaf(st[r], p.scale_log2, fmaf(bias_s[col - jj + 31], kLog2e, -lse2));
      const float pr = vis ? fast_exp2(lg) : 0.f;
      ds[r] = vis ? pr * (dpt[r] - dd) : 0.f;
      diag[(col - jj + 31) * kDiagStride + col] = ds[r];
    }
    // dQ^T += K^T dS^T: rows are dims (K read transposed), the lane's column its query
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t bs = pack_p_operand(ds + 8 * ks);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        dq[db] = mfma_32x32x16(load_vt_operand(kt, kStride, 16 * ks, 32 * db, lane), bs, dq[db]);
    }
    // dr: lane e < 63 sums row e of the table (the pairs at distance dbase + e; invisible pairs
    // hold zero).  The table is this wave's own and the
    // LDS serves a wave's requests in order, so only the compiler's order is kept here.
    lds_order();
    if (lane < 63) {
      float x = 0.f;
#pragma unroll
      for (int c = 0; c < kRows; c += 2) {
        const f32x2_t y = *(const f32x2_t*)(diag + lane * kDiagStride + c);
        const int jj0 = c - lane + 31;  // key of column c
        x += ((unsigned)jj0 < (unsigned)kRows ? y[0] : 0.f) + ((unsigned)(jj0 + 1) < (unsigned)kRows ? y[1] : 0.f);
      }
      // rows of the table at negative distances hold only invisible pairs: never added
      if (has_head && dbase + lane >= 0 && x != 0.f) unsafeAtomicAdd(dbias_h + min(dbase + lane, p.R - 1), x);
    }
    lds_order();  // the next tile's table stores come after these reads
  }
  if (!qvalid || !has_head) return;
  // accumulator register 4 i + c of block db: dim 32 db + 8 i + 4 hf + c of query q0 + col
  float* dqg = p.dq + (row0 + (size_t)col * p.Hq) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4_t x;
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = dq[db][4 * i + c] * kRsqrtD;
      *(f32x4_t*)(dqg + 32 * db + 8 * i + 4 * hf) = x;
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
  fill(p.dk, n_kv);
  fill(p.dv, n_kv);
  fill(p.dbias, n_r);
  if (p.B <= 0 || p.Lq <= 0 || p.Lk <= 0) return hipGetLastError();
  const size_t rows = (size_t)p.B * p.Lq * p.Hq;
  hipLaunchKernelGGL(bwd_rowdot_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t*)p.out, (const uint16_t*)p.dout, p.D, rows);
  const unsigned pairs = (unsigned)(p.Hkv * ((p.G + 1) / 2));
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)((p.Lk + kRows - 1) / kRows), pairs, (unsigned)p.B), dim3(128),
                     0, stream, p);
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((p.Lq + kRows - 1) / kRows), pairs, (unsigned)p.B), dim3(128), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace rattn
