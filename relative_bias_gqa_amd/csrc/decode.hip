// decode.hip -- paged decode with multi-query (MTP) verification for gfx950.
//
// Each sequence b has ctx_lens[b] keys in a paged cache of 128-token blocks (vLLM recipes
// page "thinkingmachines/Inkling", Client Usage: "--block-size 128") and n_q query tokens
// at positions ctx - n_q .. ctx - 1 (Overview > MTP: up to 9 tokens per step with eight
// MTP heads).  Every query row computes the relative-bias attention of Overview >
// Architectural highlights > Attention:
//   softmax_j(q.k_j / sqrt(128) + r[h, min(p - j, R - 1)]) . V over the causal (and, for a
//   sliding-window sequence, windowed) keys.
//
// The operation streams the visible K/V of the batch once, so it is bound by HBM bytes.
// Work decomposition: a segment is (sequence, KV head, query-head subgroup); its rows are
// the n_q tokens x gs query heads that share the KV head (GQA packing: each K/V byte is
// read from HBM once for all of them).  A segment's visible keys are cut into 64-token
// units; the units of all segments, in order, form one stream that is divided among P
// workgroups (one per CU) in contiguous runs, each of its workgroup's share of the cost (a
// unit that needs per-key bias entries weighing 6 against 5 for one whose keys all take the
// clamp entry; with four waves, a share of 9 parts on an odd XCD against 10 on an even one),
// so every CU finishes at about the same time whatever the context lengths.  A workgroup walks its run
// in order and writes one normalised partial output and log2-sum-exp per segment it touches
// (slot = workgroup + segment); the merge kernel combines the pieces of each segment.
//
// Split kernel pipeline (4 waves, or 8 when a segment has more than two 32-row blocks, the
// loading waves at raised priority): K and V rows of a unit are gathered through the block
// table straight into LDS (global_load_lds_dwordx4, no register staging) into a ring of
// four stages, three units ahead of the one being computed, so about 96 KB per CU are
// always in flight.  Slots outside a sequence's visible range are loaded from a zero row
// instead of the cache, so poisoned (NaN) cache contents never reach the arithmetic and
// invisible block-table entries are never dereferenced.  K and V rows are stored with a
// 16-byte-chunk XOR swizzle (LDS rows are 256 B, no padding) so the MFMA operand reads
// are bank-conflict free.  The relative-bias slice of every unit (63 + n_q distances per
// head) is staged the same way.  Per unit, each computing wave (32 query rows) does
// S^T = K Q^T on MFMA, bias + mask, an online softmax and O^T += V^T P^T.
#include "device_common.hpp"
#include "launch.hpp"

#include <atomic>
#include <type_traits>

namespace rattn {

// Scratch of the allocation-free decode entry point: the split partials that the allocating
// entry point keeps in its caller's workspace.  Each device the library runs on holds its
// own copy for the life of the process; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (decode_scratch), never by this name.
__device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* a = addr[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    // once per device, with that device current (two threads may both ask: the runtime
    // returns the same address to both)
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(a, std::memory_order_release);
  }
  *ptr = a;
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;  // merge kernel: 4 waves
constexpr int kUnit = kDecodeUnit;  // 64 tokens per unit / pipeline stage
constexpr int kStages = 4;
constexpr int kKVBytes = kUnit * kHeadDim * 2;           // 16 KB of K (or V) per stage
constexpr int kBiasBytes = kDecodeBiasFloats * 4;        // 4 KB of bias per stage
constexpr int kStageBytes = 2 * kKVBytes + kBiasBytes;   // 36 KB
constexpr float kRescaleSlack = 8.0f;

// 256 bytes of zeros: the source of every invisible K/V row.
__device__ __attribute__((aligned(256))) const uint32_t kZeroRow[64] = {0};

struct SeqInfo {
  int ctx;     // keys in the cache (clamped into [1, 128 * max_blocks_per_seq])
  int weff;    // window, or a huge value for full attention
  int vis_lo;  // first key any query of the sequence can see
  int clo;     // first unit (64-token chunk index) of the visible range
  int nch;     // units of the visible range
};

__device__ __forceinline__ SeqInfo seq_info_of(const DecodeParams& p, int ctx_len, int W) {
  SeqInfo s;
  s.ctx = min(max(ctx_len, 1), p.mbps * 128);
  s.weff = W > 0 ? W : 0x40000000;
  s.vis_lo = W > 0 ? max(0, s.ctx - p.n_q - W + 1) : 0;
  s.clo = s.vis_lo / kUnit;
  s.nch = (s.ctx - 1) / kUnit + 1 - s.clo;
  return s;
}

__device__ __forceinline__ SeqInfo seq_info(const DecodeParams& p, int b) {
  return seq_info_of(p, p.ctx_lens[b], p.windows ? p.windows[b] : 0);
}

// The same for a sequence index that every lane of the wave holds: read through the scalar
// cache, so that a loading wave's read does not wait behind its global -> LDS loads.
__device__ __forceinline__ SeqInfo seq_info_u(const DecodeParams& p, int b) {
  return seq_info_of(p, uniform_load_i32(p.ctx_lens + b), p.windows ? uniform_load_i32(p.windows + b) : 0);
}

// Position in the unit stream: sequence, segment within the sequence, absolute chunk.
struct Cursor {
  int b, kh, c;
  SeqInfo si;
};

__device__ __forceinline__ Cursor cursor_at(const DecodeParams& p, const int* pre, int u) {
  // last b with pre[b] * KH <= u
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] * p.KH <= u) lo = mid;
    else hi = mid - 1;
  }
  Cursor c;
  c.b = lo;
  c.si = seq_info_u(p, lo);
  const int r = u - pre[lo] * p.KH;
  c.kh = r / c.si.nch;
  c.c = c.si.clo + (r - c.kh * c.si.nch);
  return c;
}

__device__ __forceinline__ void cursor_next(const DecodeParams& p, Cursor& c) {
  if (++c.c == c.si.clo + c.si.nch) {
    if (++c.kh == p.KH) {
      c.kh = 0;
      if (c.b + 1 < p.B) {
        ++c.b;
        c.si = seq_info_u(p, c.b);
      }
    }
    c.c = c.si.clo;
  }
}

// ---- division of the unit stream among the workgroups ----------------------------------
// Units do not cost the same: a unit whose keys are all at distance >= R - 1 from every
// query of its sequence adds the single clamp entry r[h, R - 1], any other one stages a
// slice of r per head and adds it element by element, about 1.2 times the time.  With C(k)
// the cost of the units before unit k and C their total, each workgroup gets a contiguous run
// of units whose cost is its share of C (shares below).
constexpr int kCostSat = 5;
constexpr int kCostUnsat = 6;

// leading units of the visible range whose keys are all at distance >= R - 1
__device__ __forceinline__ int seq_nsat(const DecodeParams& p, const SeqInfo& s) {
  // unit c (keys 64 c .. 64 c + 63) qualifies iff (ctx - n_q) - (64 c + 63) >= R - 1
  const long long lim = (long long)s.ctx - p.n_q - p.R - (kUnit - 2);
  if (lim < 0) return 0;
  return (int)min(max(lim / kUnit + 1 - s.clo, 0LL), (long long)s.nch);
}

// cost of one segment (one KV head's share) of a sequence
__device__ __forceinline__ long long seg_cost(int nch, int nsat) {
  return (long long)nsat * kCostSat + (long long)(nch - nsat) * kCostUnsat;
}

// Shares by XCD.  Workgroup w runs on XCD w % 8.  With four waves (segments of up to 64 rows:
// the kernel waits on its K/V loads) workgroups on odd XCDs took ~10 % longer for the same
// units (per-workgroup timelines), so there a share is 10 parts on an even XCD and 9 on an
// odd one; with eight waves (more rows: compute and loads overlap) the XCDs ran alike and
// every share is one part.  K(w) = the parts of the workgroups before w.
struct Caps {
  int even, odd;
};
__device__ __forceinline__ Caps share_caps(const DecodeParams& p) { return p.NW == 4 ? Caps{10, 9} : Caps{1, 1}; }
__device__ __forceinline__ long long cap_prefix(long long w, Caps c) {
  const int j = (int)(w & 7);
  return (w >> 3) * (4LL * (c.even + c.odd)) + (long long)((j + 1) >> 1) * c.even + (long long)(j >> 1) * c.odd;
}
// the last workgroup w with cap_prefix(w) <= x
__device__ __forceinline__ long long cap_owner(long long x, Caps c) {
  const long long c8 = 4LL * (c.even + c.odd);
  const long long a = x / c8;
  const long long r = x - a * c8;
  int j = 0;
#pragma unroll
  for (int i = 1; i < 8; ++i) j += (long long)((i + 1) >> 1) * c.even + (long long)(i >> 1) * c.odd <= r ? 1 : 0;
  return 8 * a + j;
}

// Workgroups that take part: few enough that every workgroup's cost range (at least
// C min(part) / (P max(part)) wide) holds the start of some unit, so that no workgroup is left
// empty: at most one per cost kCostUnsat (scaled by the largest to the smallest share, plus
// one for rounding, when they differ).
__device__ __forceinline__ int split_count(const DecodeParams& p, long long ctot) {
  const Caps c = share_caps(p);
  const int lo = min(c.even, c.odd), hi = max(c.even, c.odd);
  const long long per = lo == hi ? kCostUnsat : (kCostUnsat * hi + lo - 1) / lo + 1;
  return (int)max(1LL, min((long long)p.P, ctot / per));
}

struct SplitRange {
  int P;        // workgroups that take part
  int n_units;  // this workgroup's units
  Cursor c0;    // its first unit
};

// This workgroup's share of the unit stream, computed by the whole workgroup (NT threads)
// with `lds` as scratch (at least NT / 4 + 12 (B + 1) bytes, not yet in use by any load).
template <int NT>
__device__ SplitRange split_range(const DecodeParams& p, unsigned char* lds) {
  long long* wave_u = (long long*)lds;     // [NT / 64]: units of each wave's sequences
  long long* wave_c = wave_u + NT / 64;    // [NT / 64]: their cost
  long long* pre_c = wave_c + NT / 64;     // [B + 1]: cost of the sequences before b (all segments)
  int* pre_u = (int*)(pre_c + p.B + 1);    // [B + 1]: units per segment of the sequences before b
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int per = (p.B + NT - 1) / NT;
  long long lu = 0, lc = 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < p.B) {
      const SeqInfo si = seq_info(p, b);
      lu += si.nch;
      lc += seg_cost(si.nch, seq_nsat(p, si));
    }
  }
  // inclusive scan within the wave, then the totals of the waves before this one
  long long su = lu, sc = lc;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long tu = __shfl_up(su, off), tc = __shfl_up(sc, off);
    if (lane >= off) {
      su += tu;
      sc += tc;
    }
  }
  if (lane == 63) {
    wave_u[wave] = su;
    wave_c[wave] = sc;
  }
  __syncthreads();
  for (int v = 0; v < wave; ++v) {
    su += wave_u[v];
    sc += wave_c[v];
  }
  long long ru = su - lu, rc = sc - lc;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < p.B) {
      const SeqInfo si = seq_info(p, b);
      pre_u[b] = (int)ru;
      pre_c[b] = rc * p.KH;
      ru += si.nch;
      rc += seg_cost(si.nch, seq_nsat(p, si));
    }
  }
  if (tid == NT - 1) {
    pre_u[p.B] = (int)su;
    pre_c[p.B] = sc * p.KH;
  }
  __syncthreads();
  const long long ctot = pre_c[p.B];
  const int units = pre_u[p.B] * p.KH;
  SplitRange sr;
  sr.P = split_count(p, ctot);
  sr.n_units = 0;
  const int w = blockIdx.x;
  // index of the first unit whose cost prefix is >= T (units if there is none)
  auto first_unit = [&](long long T) {
    if (T >= ctot) return units;
    int lo = 0, hi = p.B - 1;  // last b with pre_c[b] <= T
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre_c[mid] <= T) lo = mid;
      else hi = mid - 1;
    }
    const SeqInfo si = seq_info_u(p, lo);
    const int nsat = seq_nsat(p, si);
    const long long sc = seg_cost(si.nch, nsat);
    const long long r = T - pre_c[lo];
    const int kh = (int)(r / sc);
    const long long r2 = r - kh * sc, sat_cost = (long long)nsat * kCostSat;
    const int k = r2 <= sat_cost ? (int)((r2 + kCostSat - 1) / kCostSat)
                                 : nsat + (int)((r2 - sat_cost + kCostUnsat - 1) / kCostUnsat);
    return pre_u[lo] * p.KH + kh * si.nch + k;
  };
  if (w < sr.P) {
    const Caps caps = share_caps(p);
    const long long ktot = cap_prefix(sr.P, caps);
    const int u0 = first_unit((cap_prefix(w, caps) * ctot + ktot - 1) / ktot);
    sr.n_units = first_unit((cap_prefix(w + 1, caps) * ctot + ktot - 1) / ktot) - u0;
    sr.c0 = cursor_at(p, pre_u, u0);
  }
  __syncthreads();  // every wave is done with the scratch before any load reaches it
  return sr;
}

// NW: waves per workgroup (4, or 8 = two per SIMD, so that one wave's softmax overlaps
// its partner's MFMAs).  Every computing wave owns one 32-row block and one 32-key half of
// each unit (KS = 2 waves share a unit's keys, KB = 1 key block per wave).  NL: waves that
// issue the loads, the last NL of the workgroup (NL = NW: every wave; NL < NW: waves
// without a computing role, so that the computing waves spend no instructions on
// addresses, block-table reads and load issue).  NB: bias loads per loading wave and unit
// (64 floats each), NB * 64 * NL >= gs * SL.
template <int NW, int NL, int NB>
__global__ __launch_bounds__(64 * NW, 1) void decode_split_kernel(DecodeParams p) {
  constexpr int NT = 64 * NW;
  constexpr int KS = 2;            // waves sharing the keys of a unit
  constexpr int KB = 2 / KS;       // 32-key blocks per computing wave and unit
  constexpr int TPW = kUnit / NL;  // tokens of a unit loaded by one loading wave
  constexpr int NI = TPW / 4;      // K (and V) load instructions per loading wave and unit
  constexpr int kLoadsPerStage = 2 * NI + NB;
  static_assert(NL >= 1 && NL <= NW && NI >= 1 && NI * 4 * NL == kUnit, "load split");
  static_assert(2 * kLoadsPerStage < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages * kStageBytes];
  static_assert(NT / 4 + 12 * (kDecodeMaxBatch + 1) <= kStages * kStageBytes, "split scratch");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hf = lane >> 5;
  const int li = wave - (NW - NL);  // index among the loading waves, < 0 for the others
  const bool loader = li >= 0;

  const SplitRange sr = split_range<NT>(p, ring);
  const int w = blockIdx.x;
  if (w >= sr.P) return;  // uniform
  const int n_units = sr.n_units;

  // ---- loads of one unit into a stage -------------------------------------------------
  // K/V: loading wave li issues tokens TPW li .. TPW li + TPW - 1 of the 64-token unit,
  // four tokens (1 KB) per instruction; lane i of instruction m fetches 16-byte chunk
  // (i & 15) ^ swz(tok) of token tok = 4 m + i / 16, which lands at LDS chunk i & 15.
  // Per-lane byte offsets are fixed; a unit only adds its block base.
  // Per-lane offsets are the same for every unit; they are recomputed inside each issue
  // (from an opaque copy of the lane index) instead of being kept in registers, so that
  // they do not occupy registers across the computing waves' code.
  // Bias: NB * 64 * NL floats per stage; entry g * SL + x = r[h_g, clamp(d0 + x, 0, R - 1)].
  const unsigned char* kc_bytes = (const unsigned char*)p.k_cache;
  const unsigned char* vc_bytes = (const unsigned char*)p.v_cache;
  const unsigned char* zero_bytes = (const unsigned char*)kZeroRow;
  const uint32_t ring_base = lds_addr(ring);

  auto issue_unit = [&](const Cursor& ic, int st) {
    const int kvh = ic.kh / p.n_hs;
    const int hs = ic.kh - kvh * p.n_hs;
    const int j0 = ic.c * kUnit;
    int phys = uniform_load_i32(p.block_table + (size_t)ic.b * p.mbps + (ic.c >> 1));
    phys = min(max(phys, 0), p.num_blocks - 1);
    const size_t base = (((size_t)phys * 128 + (ic.c & 1) * kUnit) * p.Hkv + kvh) * 256;
    const unsigned char* kb_ = kc_bytes + base;
    const unsigned char* vb_ = vc_bytes + base;
    const uint32_t kdst = ring_base + st * kStageBytes + li * (TPW * 256);
    const uint32_t vdst = kdst + kKVBytes;
    const uint32_t bdst = ring_base + st * kStageBytes + 2 * kKVBytes + li * (NB * 256);
    const bool interior = j0 >= ic.si.vis_lo && j0 + kUnit <= ic.si.ctx;
    int lt = lane;
    asm volatile("" : "+v"(lt));
    const int slot = lt & 15;
    const int tok0 = TPW * li + (lt >> 4);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = tok0 + 4 * i;
      const uint32_t ck16 = (uint32_t)(slot ^ (tok & 15)) * 16u;
      const uint32_t cv16 = (uint32_t)(slot ^ ((tok & 7) << 1)) * 16u;
      const uint32_t row = (uint32_t)(tok * p.Hkv) * 256u;
      const unsigned char* gk = kb_ + row + ck16;
      const unsigned char* gv = vb_ + row + cv16;
      if (!interior) {
        const int j = j0 + tok;
        const bool vis = j >= ic.si.vis_lo && j < ic.si.ctx;
        gk = vis ? gk : zero_bytes + ck16;
        gv = vis ? gv : zero_bytes + cv16;
      }
      dma16nt(gk, kdst + i * 1024);
      dma16nt(gv, vdst + i * 1024);
    }
    const int p0 = ic.si.ctx - p.n_q;
    const bool saturated = p0 - (j0 + kUnit - 1) >= p.R - 1;
    const int d0 = p0 - j0 - (kUnit - 1);
    const int hbase = kvh * p.G + hs * p.gs;
    // entry 64 (NB li + i) + lane = (head g, distance offset x); x steps by 64 < SL + 1
    int g = 0, x = 0;
    if (!saturated) {
      const int idx0 = 64 * NB * li + lt;
      g = idx0 / p.SL;
      x = idx0 - g * p.SL;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float* src = p.bias;
      if (!saturated) {
        if (i > 0) {
          x += 64;
          if (x >= p.SL) {
            x -= p.SL;
            ++g;
          }
        }
        if (g < p.gs) src = p.bias + (size_t)(hbase + g) * p.R + min(max(d0 + x, 0), p.R - 1);
      }
      dma4(src, bdst + i * 256);
    }
  };

  // ---- this wave's role: row block rb (32 rows) and key half ks of every unit ----------
  // Wave w takes row block w % n_rb and key half w / n_rb (waves past 2 n_rb compute
  // nothing); the two halves keep separate online-softmax states (separate pieces for the
  // merge kernel).
  const int n_rb = (p.rows + 31) / 32;
  const int rb = wave % n_rb;
  const int ks_w = wave / n_rb;
  const bool wave_active = rb < n_rb && ks_w < KS;
  const int kb_lo = ks_w;
  // The loading waves issue first whenever they are ready: with more computing waves than
  // SIMDs a loading wave shares its SIMD with a computing one, and at equal priority its
  // load issue after each barrier queues behind that wave's MFMA and softmax instructions
  // (1M-token MTP verify: 3.5 % shorter split kernel).
  if (loader) __builtin_amdgcn_s_setprio(3);
  // LDS operand bases (stage 0).  K rows are 256 B with 16-byte chunk c of key j at chunk
  // c ^ (j & 15): the A operand of k-step k8 (key 32 kb + col, chunk 2 k8 + hf) sits at
  // kx0 ^ (32 k8).  V rows have chunk c of key j at c ^ (2 (j & 7)): the transposed read
  // of d block db, keys kbase.. is at vz0 ^ (64 db) + 256 kbase (and 8 rows on).
  const uint32_t kx0 = ring_base + 8192u * kb_lo + col * 256 + 32 * ((col & 15) >> 1) + 16 * (hf ^ (col & 1));
  uint32_t vz0;
  {
    const int m = lane & 15, u = (lane >> 4) & 1;
    const int vrow = 4 * hf + (m >> 2);
    const int y = (2 * u + ((m & 3) >> 1)) ^ (2 * (vrow & 7));
    vz0 = ring_base + kKVBytes + 8192u * kb_lo + vrow * 256 + 16 * y + 8 * (m & 1);
  }
  const int r_row = 32 * rb + col;
  const bool row_ok = r_row < p.rows;
  const int tq = row_ok ? r_row / p.gs : 0;
  const int gq = row_ok ? r_row - tq * p.gs : 0;
  // bias entry of key kk for this lane: bs[bias_lane + 59 - (kk - 4 hf - 32 kb_lo)]
  const int bias_lane = gq * p.SL + tq + 4 - 4 * hf - 32 * kb_lo;

  f32x16_t o[4];
  u32x4_t qr[8];
  float m_run = kNegInf, l_run = 0.f, bias_sat = 0.f;

  auto begin_segment = [&](const Cursor& cc) {
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = zero_f32x16();
    m_run = kNegInf;
    l_run = 0.f;
    if (!wave_active) return;
    const int kvh = cc.kh / p.n_hs;
    const int hs = cc.kh - kvh * p.n_hs;
    const int h = kvh * p.G + hs * p.gs + gq;
    const size_t qbase = (((size_t)cc.b * p.n_q + tq) * p.Hq + h) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qr[ks] = row_ok ? *(const u32x4_t*)(p.q + qbase + 16 * ks + 8 * hf) : zero_u32x4();
    bias_sat = p.bias[(size_t)h * p.R + (p.R - 1)] * kLog2e;
    // take the loaded values through an opaque definition here, so the compiler's wait for
    // them sits at this point and not in front of the first MFMA, behind later LDS loads
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(qr[ks]));
    asm volatile("" : "+v"(bias_sat));
  };

  auto flush_segment = [&](int seg) {
    if (!wave_active) return;
    const float l_tot = half_swap_sum(l_run);
    if (!row_ok) return;
    const size_t slot_row = ((size_t)(w + seg) * KS + ks_w) * p.rows + r_row;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* dst = p.ws_o + slot_row * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 32 * db + 8 * q + 4 * hf;
        *(f32x4_t*)(dst + d) = f32x4_t{o[db][4 * q] * inv, o[db][4 * q + 1] * inv, o[db][4 * q + 2] * inv,
                                       o[db][4 * q + 3] * inv};
      }
    if (hf == 0) p.ws_lse[slot_row] = l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;
  };

  // logits of this wave's 32-key blocks into t, in log2 units relative to m_ref (the
  // running maximum, or 0 before the row's first visible key): the bias and the
  // reference in one FMA.  Returns the row maximum over this lane and its partner.
  auto logits = [&](auto sat_c, auto mask_c, const f32x16_t* sacc, const float* bs_lds, float (*t)[16],
                    int dl, int weff, float m_ref) {
    constexpr bool SAT = decltype(sat_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    float bb[KB][16];
    if constexpr (!SAT) {
#pragma unroll
      for (int i = 0; i < KB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) bb[i][r] = bs_lds[bias_lane + 59 - (32 * i + 8 * (r >> 2) + (r & 3))];
    }
    const float c_sat = bias_sat - m_ref;
#pragma unroll
    for (int i = 0; i < KB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x;
        if constexpr (SAT) x = fmaf(sacc[i][r], p.scale_log2, c_sat);
        else x = fmaf(bb[i][r], kLog2e, fmaf(sacc[i][r], p.scale_log2, -m_ref));
        if constexpr (MASK) {
          // distance of this key from the lane's query; visible iff 0 <= d < weff
          const int d = dl - (32 * i + 8 * (r >> 2) + (r & 3));
          x = (uint32_t)d < (uint32_t)weff ? x : kNegInf;
        }
        t[i][r] = x;
      }
    float mb[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      float m = max3f(t[i][0], t[i][1], t[i][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) m = max3f(m, t[i][r], t[i][r + 1]);
      mb[i] = m;
    }
    if constexpr (KB == 1) return half_swap_max3(mb[0], t[0][15]);
    else return half_swap_max3(max3f(mb[0], mb[1], t[0][15]), t[1][15]);
  };

  auto compute_unit = [&](const Cursor& cc, int st) {
    if (!wave_active) return;
    const unsigned char* ks_lds = ring + st * kStageBytes;
    const unsigned char* vs_lds = ks_lds + kKVBytes;
    const float* bs_lds = (const float*)(vs_lds + kKVBytes);
    // this unit's operand bases: one register each, the reads differ by an XOR with a
    // constant and an immediate offset (kept opaque so the compiler does not precompute
    // every read address of every stage)
    uint32_t kx = kx0 + st * kStageBytes, vz = vz0 + st * kStageBytes;
    asm volatile("" : "+v"(kx), "+v"(vz));
    const int j0 = cc.c * kUnit;
    const int p0 = cc.si.ctx - p.n_q;  // position of query 0
    const bool saturated = p0 - (j0 + kUnit - 1) >= p.R - 1;
    const bool need_mask = (j0 + kUnit - 1 > p0) || (j0 < cc.si.ctx - cc.si.weff);

    // the K operands of this wave's 32-key blocks first, then S^T = K Q^T; the V operands
    // are read after the score MFMAs are issued, so that their latency overlaps the
    // softmax and the K and V operands are never live together (which would push the
    // wave past 256 VGPRs into AGPR accumulators and copies)
    u32x4_t ka[KB][8];
#pragma unroll
    for (int i = 0; i < KB; ++i)
#pragma unroll
      for (int k8 = 0; k8 < 8; ++k8) ka[i][k8] = lds_ld16((kx ^ (32u * k8)) + 8192u * i);
    f32x16_t sacc[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      sacc[i] = zero_f32x16();
#pragma unroll
      for (int k8 = 0; k8 < 8; ++k8) sacc[i] = mfma_32x32x16(ka[i][k8], qr[k8], sacc[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // V^T operands of 32-key block i (the first block's are read now, overlapping the
    // softmax; a second block's while the first block's P.V MFMAs run)
    u32x4_t va[4][2];
    auto load_v = [&](int i) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t a = (vz ^ (64u * db)) + 256u * (32 * i + 16 * half);
          const u32x2_t lo = lds_tr8(a), hi = lds_tr8(a + 2048u);
          va[db][half] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
    };
    load_v(0);
    float t[KB][16];
    const int dl = p0 + tq - j0 - 4 * hf - 32 * kb_lo;  // distance of this lane's first key
    const int weff = cc.si.weff;
    const bool fresh = m_run == kNegInf;
    const float m_ref = fresh ? 0.f : m_run;
    float mx;
    if (saturated) {
      mx = need_mask ? logits(std::true_type{}, std::true_type{}, sacc, bs_lds, t, dl, weff, m_ref)
                     : logits(std::true_type{}, std::false_type{}, sacc, bs_lds, t, dl, weff, m_ref);
    } else {
      mx = need_mask ? logits(std::false_type{}, std::true_type{}, sacc, bs_lds, t, dl, weff, m_ref)
                     : logits(std::false_type{}, std::false_type{}, sacc, bs_lds, t, dl, weff, m_ref);
    }
    // online softmax: the running maximum is raised only when a row's maximum exceeds it
    // by more than the slack (or on the row's first visible key), rescaling O, the
    // normaliser and this unit's logits
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
      for (int i = 0; i < KB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) t[i][r] -= delta;
    }
    float lsum = 0.f;
    u32x4_t pk[KB][2];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        t[i][r] = fast_exp2(t[i][r]);
        lsum += t[i][r];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) pk[i][half] = pack_p_operand(&t[i][8 * half]);
    }
    l_run += lsum;
    // O^T += V^T P^T
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (i > 0) load_v(i);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) o[db] = mfma_32x32x16(va[db][half], pk[i][half], o[db]);
    }
  };

  // ---- main loop: unit t computed from stage t % 4 while units t+1..t+3 load ------------
  Cursor cc = sr.c0;
  Cursor ic = cc;
  begin_segment(cc);  // before any LDS load is in flight
  const int prologue = min(kStages - 1, n_units);
  if (loader) {
    for (int i = 0; i < prologue; ++i) {
      issue_unit(ic, i);
      cursor_next(p, ic);
    }
  }
  int seg = cc.b * p.KH + cc.kh;
  for (int t = 0; t < n_units; ++t) {
    if (loader) {
      const int ahead = min(kStages - 2, n_units - 1 - t);  // units issued after this one
      if (ahead >= 2) vm_wait<2 * kLoadsPerStage>();
      else if (ahead == 1) vm_wait<kLoadsPerStage>();
      else vm_wait<0>();
    }
    wg_barrier();  // unit t is in LDS; every wave is done with unit t - 1
    if (loader && t + kStages - 1 < n_units) {
      issue_unit(ic, (t + kStages - 1) % kStages);
      cursor_next(p, ic);
    }
    const int cseg = cc.b * p.KH + cc.kh;
    if (cseg != seg) {
      flush_segment(seg);
      begin_segment(cc);
      seg = cseg;
    }
    compute_unit(cc, t % kStages);
    cursor_next(p, cc);
  }
  flush_segment(seg);
}

// Merge: one workgroup per (segment, row, slice of the 128 outputs; SLICES = 4 when a
// segment has many pieces, else 1).  Its threads form groups of 32 / SLICES (one float4
// each of the slice); group g takes pieces g, g + groups, ..., eight at a time with all
// eight pieces' loads in flight, and keeps a running maximum, sum and weighted output (one
// pass: a piece's weight is 2^(lse - max) against the running max).  The groups' partial
// results are then combined through LDS in group order.
constexpr int kMergeBatch = 8;  // pieces per group and round

template <int SLICES>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeParams p) {
  constexpr int kMergeLanes = kHeadDim / SLICES / 4;  // float4 lanes per piece
  constexpr int kMergeGroups = kThreads / kMergeLanes;
  __shared__ long long cred[2][kThreads / 64];
  __shared__ float gm[kMergeGroups], gz[kMergeGroups];
  __shared__ f32x4_t gacc[kMergeGroups][kMergeLanes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int slice = blockIdx.x % SLICES;
  const int sr = blockIdx.x / SLICES;
  const int seg = sr / p.rows;
  const int r_row = sr - seg * p.rows;
  const int b = seg / p.KH;
  const int kh = seg - b * p.KH;

  // cost of the sequences before b, and in total
  long long before = 0, total = 0;
  for (int bb = tid; bb < p.B; bb += kThreads) {
    const SeqInfo si = seq_info(p, bb);
    const long long c = seg_cost(si.nch, seq_nsat(p, si));
    total += c;
    if (bb < b) before += c;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    before += __shfl_xor(before, off);
    total += __shfl_xor(total, off);
  }
  if (lane == 0) {
    cred[0][wave] = before;
    cred[1][wave] = total;
  }
  __syncthreads();
  before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    before += cred[0][w];
    total += cred[1][w];
  }
  const long long ctot = total * p.KH;
  const long long P = split_count(p, ctot);
  // the workgroups that hold this segment's first and last units
  const SeqInfo sb = seq_info_u(p, b);
  const int nsat = seq_nsat(p, sb);
  const long long sc = seg_cost(sb.nch, nsat);
  const long long c_first = before * p.KH + kh * sc;
  const long long c_last = c_first + sc - (nsat == sb.nch ? kCostSat : kCostUnsat);
  const Caps caps = share_caps(p);
  const long long ktot = cap_prefix(P, caps);
  const int w_first = (int)min(cap_owner(c_first * ktot / ctot, caps), P - 1);
  const int w_last = (int)min(cap_owner(c_last * ktot / ctot, caps), P - 1);
  // piece i = (workgroup w_first + i / KS, key half i % KS)
  const int n_pieces = (w_last - w_first + 1) * p.KS;
  auto slot_row = [&](int i) {
    return ((size_t)(w_first + i / p.KS + seg) * p.KS + (i % p.KS)) * p.rows + r_row;
  };

  const int d4 = tid % kMergeLanes, grp = tid / kMergeLanes;
  const int col = slice * (kHeadDim / SLICES) + 4 * d4;
  float m = kNegInf, z = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = grp; i0 < n_pieces; i0 += kMergeGroups * kMergeBatch) {
    float l[kMergeBatch];
    f32x4_t x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int i = i0 + kMergeGroups * u;
      l[u] = kNegInf;
      x[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (i < n_pieces) {
        const size_t sr_i = slot_row(i);
        l[u] = p.ws_lse[sr_i];
        x[u] = *(const f32x4_t*)(p.ws_o + sr_i * kHeadDim + col);
      }
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) mb = fmaxf(mb, l[u]);
    if (mb != kNegInf) {
      const float scale = fast_exp2(m - mb);  // 0 while m is still -inf
      acc *= scale;
      z *= scale;
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float wt = fast_exp2(l[u] - mb);  // 0 for an empty piece (lse -inf)
        acc += wt * x[u];
        z += wt;
      }
      m = mb;
    }
  }
  if (d4 == 0) {
    gm[grp] = m;
    gz[grp] = z;
  }
  gacc[grp][d4] = acc;
  __syncthreads();
  if (tid < kMergeLanes) {
    float M = kNegInf;
#pragma unroll
    for (int g = 0; g < kMergeGroups; ++g) M = fmaxf(M, gm[g]);
    float Z = 0.f;
    f32x4_t tot = {0.f, 0.f, 0.f, 0.f};
    if (M != kNegInf) {
#pragma unroll
      for (int g = 0; g < kMergeGroups; ++g) {
        const float wt = fast_exp2(gm[g] - M);
        Z += wt * gz[g];
        tot += wt * gacc[g][tid];
      }
    }
    const float inv = Z > 0.f ? 1.f / Z : 0.f;
    const int kvh = kh / p.n_hs;
    const int hs = kh - kvh * p.n_hs;
    const int tq = r_row / p.gs;
    const int h = kvh * p.G + hs * p.gs + (r_row - tq * p.gs);
    const size_t out_row = ((size_t)b * p.n_q + tq) * p.Hq + h;
    *(u32x2_t*)(p.out + out_row * kHeadDim + slice * (kHeadDim / SLICES) + 4 * tid) =
        u32x2_t{pack_bf16x2(tot[0] * inv, tot[1] * inv), pack_bf16x2(tot[2] * inv, tot[3] * inv)};
    if (tid == 0 && slice == 0 && p.lse != nullptr) p.lse[out_row] = Z > 0.f ? (M + __log2f(Z)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.B <= 0) return hipSuccess;
  if (p.KH < 1) return hipErrorInvalidConfiguration;
  // merge slices: 4 when a segment averages 64 or more pieces (KS per workgroup that
  // touches it), so that a row's pieces are read by four workgroups at once
  const long long segs = (long long)p.B * p.KH;
  const int slices = (long long)p.KS * (p.P / segs + 2) >= 64 ? kDecodeMergeSlices : 1;
  const long long grid2 = segs * p.rows * slices;
  if (grid2 > 0x7fffffffLL || p.P < 1) return hipErrorInvalidConfiguration;
  if ((p.NW != 4 && p.NW != 8) || p.KS != 2) return hipErrorInvalidConfiguration;
  // every computing role (32-row block, key half) needs a wave of its own; the waves left
  // over issue the loads (two of them), else every wave does
  const int roles = (p.rows + 31) / 32 * 2;
  if (roles > p.NW) return hipErrorInvalidConfiguration;
  const int NL = p.NW - roles >= 2 ? 2 : p.NW;
  const int nb = (p.gs * p.SL + 64 * NL - 1) / (64 * NL);  // bias loads per loading wave and unit
  if (nb < 1 || nb * 64 * NL > kDecodeBiasFloats) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)p.P);
#define RATTN_SPLIT(NW_, NL_, NB_) \
  hipLaunchKernelGGL((decode_split_kernel<NW_, NL_, NB_>), grid, dim3(64 * NW_), 0, stream, p)
  if (NL == 2) {
    // bias loads of up to 1024 floats spread over two waves
    switch (nb) {
      case 1: case 2: if (p.NW == 8) RATTN_SPLIT(8, 2, 2); else RATTN_SPLIT(4, 2, 2); break;
      case 3: case 4: if (p.NW == 8) RATTN_SPLIT(8, 2, 4); else RATTN_SPLIT(4, 2, 4); break;
      case 5: case 6: if (p.NW == 8) RATTN_SPLIT(8, 2, 6); else RATTN_SPLIT(4, 2, 6); break;
      default: if (p.NW == 8) RATTN_SPLIT(8, 2, 8); else RATTN_SPLIT(4, 2, 8); break;
    }
  } else if (p.NW == 8) {
    if (nb == 1) RATTN_SPLIT(8, 8, 1);
    else RATTN_SPLIT(8, 8, 2);
  } else {
    switch (nb) {
      case 1: RATTN_SPLIT(4, 4, 1); break;
      case 2: RATTN_SPLIT(4, 4, 2); break;
      case 3: RATTN_SPLIT(4, 4, 3); break;
      default: RATTN_SPLIT(4, 4, 4); break;
    }
  }
#undef RATTN_SPLIT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (slices == 1) hipLaunchKernelGGL(decode_merge_kernel<1>, dim3((unsigned)grid2), dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL(decode_merge_kernel<kDecodeMergeSlices>, dim3((unsigned)grid2), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rattn
