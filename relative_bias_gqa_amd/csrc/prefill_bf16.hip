// prefill_bf16.hip -- relative-bias GQA prefill / chunked prefill, bf16 inputs, gfx950.
//
// Computes, for every query row (b, t, h) at absolute position p = Lk - Lq + t,
//   out = softmax_j(q.k_j / sqrt(128) + r[h, min(p - j, R - 1)]) . V,  lse = log-sum-exp,
// over keys 0 <= p - j (and p - j <= W - 1 for a sliding window): the relative attention
// of the vLLM recipes page "thinkingmachines/Inkling" (Overview > Architectural
// highlights > Attention: GQA with head size 128, a trained bias on the logits that
// depends on the query-key distance, full and sliding-window layers).  Its Performance
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
//     ring of four stages, two tiles ahead, and serve all of the workgroup's query heads
//     (GQA packing: one K/V read per head group).  K/V rows carry a 16-byte-chunk XOR
//     swizzle so the MFMA operand reads are conflict free, and every operand address is
//     one register XORed with a constant;
//   - each wave also loads its own diagonal slice of r for the tile (distances clamped to
//     R - 1) into the stage and seeds its S accumulators with it, scaled by sqrt(128), so
//     the MFMA adds q.k onto the bias;
//   - TOK (a token-dependent table, every query row with its own r_t[h, :]): no slice is
//     staged; a wave tile whose distances all clamp to R - 1 adds each row's r_t[h, R - 1]
//     in the logit FMA; other tiles load each lane's 32 entries (8 runs of 4 consecutive
//     distances) into registers at the start of the MFMA half-step, the rows' lines having
//     been pulled into L2 two tiles earlier by one extra DMA per wave issued with K and V;
//   - the two halves of the workgroup (one wave of each on every SIMD) run in ping-pong,
//     half a tile apart: while one wave of a SIMD runs its MFMA half-step (O^T += V^T P^T
//     of the previous tile, then S^T = sqrt(128) r + K Q^T on v_mfma_f32_32x32x16_bf16,
//     Q resident in registers), the other runs its softmax half-step on the vector ALU:
//     logits in log2 units with the running maximum in the same FMA, the causal / window
//     mask only on edge tiles, an online softmax whose maximum is only raised when a row's
//     maximum grows by more than 8 (log2 units), P rounded to bf16; one workgroup
//     barrier per tile.  V is read transposed from LDS (ds_read_b64_tr_b16).
#include "device_common.hpp"
#include "launch.hpp"

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
constexpr int kWgRows = 32 * kWaves;              // query rows of a workgroup
constexpr float kRescaleSlack = 8.0f;             // log2 units: P entries stay below 2^8
constexpr float kSqrtD = 11.313708498984761f;     // sqrt(128)

// 256 bytes of zeros: the source of every K/V row past the end of the sequence.
__device__ __attribute__((aligned(256))) const uint32_t kZeroRowP[64] = {0};

// PAGED: K and V come from paged caches [num_blocks, 128, Hkv, 128] through the block
// table (chunked prefill over a cached prefix), and sequence b has its own context length
// ctx_lens[b] (its Lq queries are its last Lq tokens).  A 64-key tile is always one half of
// one 128-token block, laid out like 64 rows of a contiguous K/V, so only the tile's base
// address (one scalar block-table read per tile) and the key count per sequence differ.
// Keys that no query of the chunk can see (before the first query's window, or at or past
// the context) are loaded from a zero row: the cache may hold anything there.  Jobs go
// sequence by sequence, longest context first (each workgroup ranks the sequences by
// ctx_lens in LDS, up to kMaxSortedSeqs of them), last token tile first: with the job
// queue that is close to longest-first whatever the mix of context lengths.
template <bool PAGED, bool TOK>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillParams p) {
  static_assert(!(PAGED && TOK), "the token-dependent table is for contiguous K/V");
  // DMA loads per wave and stage: 2 K + 2 V, and 2 bias-slice loads (static table) or one
  // L2 warm-up load of the rows' table entries (token-dependent table)
  constexpr int kLPS = TOK ? 5 : kLoadsPerStage;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages * kStageBytes];
  __shared__ int last_piece;
  __shared__ int next_slot;
  __shared__ int seq_key[PAGED ? kMaxSortedSeqs : 1];    // ctx_lens
  __shared__ int seq_order[PAGED ? kMaxSortedSeqs : 1];  // sequences, longest context first

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // accumulator column = query token within the wave
  const int hf = lane >> 5;   // which half of the key rows this lane holds

  // ---- jobs: longest first -------------------------------------------------------------
  // Slots: the n_big heaviest unsplit token tiles (longer than any piece), then the
  // `parts` pieces of the key ranges of the n_split heaviest token tiles, then the other
  // unsplit tiles, each list from the heaviest tile down.  A workgroup runs slot
  // blockIdx.x, then (with a queue) the next unclaimed slot, until none is left: the
  // output stores of one job drain while the next one runs.
  const int per_tile = p.B * p.Hkv * p.n_hg;
  const int n_piece_slots = p.n_split * per_tile * p.parts;
  const int n_slots = n_piece_slots + (p.n_tok_tiles - p.n_split) * per_tile;
  const int n_big_slots = p.n_big * per_tile;
  const bool sorted = PAGED && p.B <= kMaxSortedSeqs;
  if constexpr (PAGED) {
    if (sorted) {
      for (int i = tid; i < p.B; i += kThreads) seq_key[i] = p.ctx_lens[i];
      __syncthreads();
      // rank of sequence i: the sequences with a longer context, or as long and lower index
      for (int i = tid; i < p.B; i += kThreads) {
        const int ki = seq_key[i];
        int r = 0;
        for (int j = 0; j < p.B; ++j) r += (seq_key[j] > ki || (seq_key[j] == ki && j < i)) ? 1 : 0;
        seq_order[r] = i;
      }
      __syncthreads();
    }
  }
  for (int slot = blockIdx.x; slot < n_slots;) {
    const bool is_piece = slot >= n_big_slots && slot < n_big_slots + n_piece_slots;
    int job, piece = 0;
    if (is_piece)
      prefill_piece_of(slot - n_big_slots, (long long)p.n_split * per_tile, p.parts, &job, &piece);
    else
      job = p.n_split * per_tile + (slot < n_big_slots ? slot : slot - n_piece_slots);
    int tile, hg, hk, b;
    if constexpr (PAGED) {
      // sequence-major: job = ((rank * n_tok_tiles + (n_tok_tiles - 1 - tile)) * Hkv + hk) * n_hg + hg
      const int per_seq = p.n_tok_tiles * p.Hkv * p.n_hg;
      const int r = job / per_seq, within = job - r * per_seq;
      tile = p.n_tok_tiles - 1 - within / (p.Hkv * p.n_hg);
      const int rem = within % (p.Hkv * p.n_hg);
      hg = rem % p.n_hg;
      hk = rem / p.n_hg;
      b = sorted ? seq_order[r] : r;
    } else {
      tile = p.n_tok_tiles - 1 - job / per_tile;
      const int rem = job % per_tile;
      hg = rem % p.n_hg;
      hk = (rem / p.n_hg) % p.Hkv;
      b = rem / (p.n_hg * p.Hkv);
    }

    const int h = hk * p.G + hg * p.hpw + (wave % p.hpw);
    const int T0 = tile * 32 * p.tsub;
    // this job's sequence: its queries (paged with packed queries: cu_q[b] .. cu_q[b + 1] - 1,
    // at most Lq) and the row of its first query
    const int qlen = PAGED && p.cu_q != nullptr ? min(max(p.cu_q[b + 1] - p.cu_q[b], 0), p.Lq) : p.Lq;
    const size_t qrow0 = PAGED && p.cu_q != nullptr ? (size_t)p.cu_q[b] : (size_t)b * p.Lq;
    const int T1 = min(qlen, T0 + 32 * p.tsub);
    const int tw0 = T0 + (wave / p.hpw) * 32;  // first token of this wave
    // keys of this job's sequence
    const int Lk = PAGED ? min(max(p.ctx_lens[b], qlen), 128 * p.mbps) : p.Lk;
    const int off = Lk - qlen;                 // position of token 0
    const int pw0 = off + tw0;                 // position of this wave's column 0
    const int wvalid = min(32, qlen - tw0);    // valid columns of this wave (may be <= 0)
    const bool wave_active = wvalid > 0;
    const int pw_last = pw0 + max(wvalid, 1) - 1;
    const int Weff = p.window > 0 ? p.window : 0x40000000;

    // keys the workgroup needs, in whole tiles (a piece: its share of them)
    int kt_begin = max(0, off + T0 - Weff + 1) / kBK;
    int kt_end = (off + T1 - 1) / kBK + 1;
    if (is_piece) {
      const int nt = kt_end - kt_begin;
      const int first = kt_begin;
      kt_begin = first + (nt * piece) / p.parts;
      kt_end = first + (nt * (piece + 1)) / p.parts;
    }
    // (a paged job past its sequence's queries has no work)
    const int n_tiles = PAGED ? (T0 < qlen ? max(kt_end - kt_begin, 0) : 0) : kt_end - kt_begin;

    // ---- Q^T operand, resident for the whole key loop -------------------------------
    u32x4_t qr[8];
    {
      const int tq = tw0 + col;
      const bool ok = wave_active && tq < qlen;
      const size_t qbase = ((qrow0 + (ok ? tq : 0)) * p.Hq + h) * kHeadDim;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qr[ks] = ok ? *(const u32x4_t*)((const uint16_t*)p.q + qbase + 16 * ks + 8 * hf) : zero_u32x4();
    }
    // token-dependent table: this lane's row r_t[h, :] (bf16 [B, Lq, Hq, R]; a row past the
    // chunk reads row 0 of the sequence, never stored) and its clamp entry r_t[h, R - 1]
    const uint16_t* tok_row = nullptr;
    float tok_sat = 0.f;
    if constexpr (TOK) {
      const int tq = tw0 + col;
      const bool ok = wave_active && tq < qlen;
      tok_row = p.bias_tok + ((qrow0 + (ok ? tq : 0)) * p.Hq + h) * (size_t)p.R;
      tok_sat = __uint_as_float((uint32_t)tok_row[p.R - 1] << 16);
      asm volatile("" : "+v"(tok_sat));
    }
    // pin the waits for these loads here, before any LDS-bound load is in flight
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(qr[ks]));

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
    const size_t seq_base = PAGED ? 0 : (size_t)b * p.Lk * p.Hkv;
    const unsigned char* kc_bytes = (const unsigned char*)p.k + (seq_base + hk) * 256;
    const unsigned char* vc_bytes = (const unsigned char*)p.v + (seq_base + hk) * 256;
    // first key any query of the sequence's chunk can see (keys before it may hold anything
    // in a paged cache)
    const int vis_lo = PAGED ? max(0, off - Weff + 1) : 0;
    const unsigned char* zero_bytes = (const unsigned char*)kZeroRowP;
    const float* bias_row = p.bias + (size_t)h * p.R;
    const uint32_t ring_base = lds_addr(ring);

    // Interior tiles issue from a scalar base plus fixed per-lane offsets (no vector ALU
    // work); the last tile (keys past Lk read a zero row) and bias halves that are only
    // partly clamped compute per-lane addresses.
    const uint32_t boff = 4u * (63 - lane);  // bias entry lo + 63 - lane of a 64-entry half
    const uint32_t zoff = 0;
    auto issue_tile = [&](int kt, int st) {
      const int j0 = kt * kBK;
      size_t base;
      if constexpr (PAGED) {
        int phys = uniform_load_i32(p.block_table + (size_t)b * p.mbps + (j0 >> 7));
        phys = min(max(phys, 0), p.num_blocks - 1);
        base = ((size_t)phys * 128 + (j0 & 127)) * p.Hkv * 256;
      } else {
        base = (size_t)j0 * p.Hkv * 256;
      }
      const uint32_t kdst = ring_base + st * kStageBytes + wave * 2048;
      const uint32_t vdst = kdst + kKVBytes;
      const uint32_t bdst = ring_base + st * kStageBytes + 2 * kKVBytes + wave * (kSliceFloats * 4);
      if (j0 + kBK <= Lk && (!PAGED || j0 >= vis_lo)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          dma16s(kc_bytes + base, koff[i], kdst + i * 1024);
          dma16s(vc_bytes + base, voff[i], vdst + i * 1024);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const unsigned char* gk = kc_bytes + base + koff[i];
          const unsigned char* gv = vc_bytes + base + voff[i];
          if (j0 + ktok[i] >= Lk || (PAGED && j0 + ktok[i] < vis_lo)) {
            gk = zero_bytes + kz[i];
            gv = zero_bytes + vz[i];
          }
          dma16(gk, kdst + i * 1024);
          dma16(gv, vdst + i * 1024);
        }
      }
      if constexpr (!TOK) {
        // this wave's bias slice, stored by decreasing distance:
        // entry y = r[h, clamp(pw0 - j0 + 31 - y, 0, R - 1)]; half i holds y = 64 i + lane,
        // distances lo + 63 - lane with lo = pw0 - j0 - 32 - 64 i
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int lo = pw0 - j0 - 32 - 64 * i;
          if (lo >= 0 && lo + 63 <= p.R - 1) {
            dma4s(bias_row + lo, boff, bdst + i * 256);
          } else if (lo >= p.R - 1) {
            dma4s(bias_row + (p.R - 1), zoff, bdst + i * 256);
          } else {
            const int d = min(max(lo + 63 - lane, 0), p.R - 1);
            dma4(bias_row + d, bdst + i * 256);
          }
        }
      } else {
        // L2 warm-up of the table entries this tile's rows will load (distances pw0 + col -
        // j0 - 63 .. + 0: 128 bytes per row, the two halves from lanes col and col + 32); the
        // bytes land in this wave's unused slice area of the stage and are never read
        // (d <= R - 2: the 4 aligned bytes around entry d stay inside the row)
        const int d = min(max(pw0 + col - j0 - 63 + 32 * hf, 0), p.R - 2);
        dma4((const void*)((uintptr_t)(tok_row + d) & ~(uintptr_t)3), bdst);
      }
    };

    // ---- per-lane LDS operand addresses (stage 0) ----------------------------------------
    // K tile rows are 256 B with 16-byte chunk c of key j stored at chunk c ^ (j & 15).  The
    // A operand of k-step i (key row 32 kb + col, chunk 2 i + hf) then sits at byte
    //   row base + ((32 i) ^ L),  L = 32 ((col & 15) >> 1) + 16 (hf ^ (col & 1)),
    // i.e. at kx0 ^ (32 i) (+ 8192 for kb = 1), the row base being 256-byte aligned.
    const uint32_t kx0 = ring_base + col * 256 + 32 * ((col & 15) >> 1) + 16 * (hf ^ (col & 1));
    // V tile rows are 256 B with chunk c of key j at chunk c ^ (2 (j & 7)).  Lane (m = lane
    // & 15, u = bit 4, hf) of the transposed read for d block db, keys kbase.. reads key row
    // kbase + 4 hf + (m >> 2) (and 8 rows on) at column 32 db + 16 u + 4 (m & 3): with
    // Y = (2 u + ((m & 3) >> 1)) ^ (2 (row & 7)) that is vz0 ^ (64 db) + 256 kbase.
    uint32_t vz0;
    {
      const int m = lane & 15, u = (lane >> 4) & 1;
      const int vrow = 4 * hf + (m >> 2);
      const int y = (2 * u + ((m & 3) >> 1)) ^ (2 * (vrow & 7));
      vz0 = ring_base + kKVBytes + vrow * 256 + 16 * y + 8 * (m & 1);
    }
    // this wave's bias slice: seeds at sb0 + 4 (32 kb + 8 (r >> 2) + (r & 3))
    const uint32_t sb0 = ring_base + 2 * kKVBytes + wave * (kSliceFloats * 4) + 4 * (31 - col + 4 * hf);
    const uint32_t sl0 = ring_base + 2 * kKVBytes + wave * (kSliceFloats * 4) + 8 * lane;

    // ---- running state ---------------------------------------------------------------
    f32x16_t o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = zero_f32x16();
    float m_run = kNegInf;  // running max (log2 units), identical in both lane halves
    float l_run = 0.f;      // this lane's share of the running normaliser
    f32x16_t s[2];          // S^T of the tile in flight (two 32-key blocks)
    u32x4_t pk[2][2];       // its P^T as bf16 MFMA operands

    // The S accumulators of the tile in stage st start from the wave's bias slice (scaled
    // to score units in the MFMA half-step).  Distances beyond R - 1 are clamped in the
    // slice, so a tile entirely past them is seeded with r[h, R - 1] like any other.
    // The seeds of the tile in stage st: this wave's whole slice is first scaled by sqrt(128)
    // in place (two entries per lane: two multiplies instead of one per seed), then the 32
    // seeds are read; the LDS serves one wave's requests in order, so the reads see the
    // scaled entries.  Runs once per tile, inside the MFMA half-step: the slice read goes
    // out before the first operand reads, the rest after the second group of MFMAs.
    float sl_e0, sl_e1;
    uint32_t sl_addr;
    auto seeds_begin = [&](int st) {
      sl_addr = sl0 + st * kStageBytes;
      asm volatile("" : "+v"(sl_addr));
      const lds_f32_t* ps = (const lds_f32_t*)(size_t)sl_addr;
      sl_e0 = ps[0];
      sl_e1 = ps[1];
    };
    auto seeds_end = [&](int st) {
      lds_f32_t* ps = (lds_f32_t*)(size_t)sl_addr;
      ps[0] = sl_e0 * kSqrtD;
      ps[1] = sl_e1 * kSqrtD;
      // one base register per call, the rest immediate offsets (kept from being hoisted
      // out of the loop as 32 separate addresses)
      uint32_t base = sb0 + st * kStageBytes;
      asm volatile("" : "+v"(base));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = lds_ldf(base + 4 * (32 * kb + 8 * (r >> 2) + (r & 3)));
    };

    // MFMA half-step: O^T += V^T P^T for the previous tile (stage st_prev), then
    // S^T = sqrt(128) r + K Q^T for the tile in stage st on the seeded accumulators.  The
    // 32 MFMAs run as eight groups of four (P.V keys 16 G.., then S k-steps in pairs); each
    // group's operands are read from LDS two groups ahead.
    // Token-dependent table: this wave's tile is SAT (every distance >= R - 1: the rows'
    // clamp entries), INNER (every distance in 0 .. R - 1: lane runs straight from the rows)
    // or MIXED (runs clamped into the row, entries chosen per element).  tb[4 kb + g]: the
    // run of 4 consecutive distances for keys 32 kb + 8 g + 4 hf .. + 3.
    u32x2_t tb[8];
    auto tok_class = [&](int kt) {
      const int j0 = kt * kBK;
      const int dmin = pw0 - j0 - (kBK - 1), dmax = pw0 + 31 - j0;
      return dmin >= p.R - 1 ? 0 : (dmin >= 0 && dmax <= p.R - 1 ? 1 : 2);
    };
    auto tok_load = [&](int kt) {
      const int cls = tok_class(kt);
      if (cls == 0) return;
      const int d0 = pw0 + col - kt * kBK - 4 * hf;  // distance of the lane's first key
      if (cls == 1) {
        const uint16_t* base = tok_row + (d0 - 3);
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_memcpy(&tb[i], base - (32 * (i >> 2) + 8 * (i & 3)), 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int a = min(max(d0 - (32 * (i >> 2) + 8 * (i & 3)) - 3, 0), p.R - 4);
          __builtin_memcpy(&tb[i], tok_row + a, 8);
        }
      }
    };

    auto mfma_half = [&](int st, int st_prev, int kt) {
      const uint32_t so = st * kStageBytes;
      const uint32_t kx = kx0 + so;
      const uint32_t vz = vz0 + st_prev * kStageBytes;
      // operands of group gi: P.V (gi < 4) keys 16 gi.., or S k-steps 2 (gi - 4) and
      // 2 (gi - 4) + 1 of both key blocks
      auto load = [&](int gi, u32x4_t* op) {
        if (gi < 4) {
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const uint32_t a = (vz ^ (64u * db)) + 256u * (16 * gi);
            const u32x2_t lo = lds_tr8(a), hi = lds_tr8(a + 2048u);
            op[db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          }
        } else {
          // k-steps 2 (gi - 4) and 2 (gi - 4) + 1 of both key blocks
#pragma unroll
          for (int i = 0; i < 4; ++i) op[i] = lds_ld16((kx ^ (32u * (2 * (gi - 4) + (i >> 1)))) + 8192u * (i & 1));
        }
      };
      u32x4_t op[3][4];
      if constexpr (!TOK) seeds_begin(st);
      else tok_load(kt);
      __builtin_amdgcn_sched_barrier(0);
      load(0, op[0]);
      load(1, op[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        if (gi + 2 < 8) load(gi + 2, op[(gi + 2) % 3]);
        const u32x4_t* cur = op[gi % 3];
        if (gi < 4) {
#pragma unroll
          for (int db = 0; db < 4; ++db) o[db] = mfma_32x32x16(cur[db], pk[gi >> 1][gi & 1], o[db]);
          // the seeds (needed from group 4 on); the slice read went out before the operands
          // of groups 0 and 1, so it has arrived
          if (gi == 1) {
            if constexpr (!TOK) {
              seeds_end(st);
            } else {
              s[0] = zero_f32x16();
              s[1] = zero_f32x16();
            }
          }
        } else {
          // alternate the two key blocks so that consecutive MFMAs are independent
#pragma unroll
          for (int i = 0; i < 4; ++i) s[i & 1] = mfma_32x32x16(cur[i], qr[2 * (gi - 4) + (i >> 1)], s[i & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads two groups ahead
      }
      if constexpr (TOK) {
        // the table runs have arrived before the next barrier (the loads are the wave's
        // youngest compiler-visible ones; the group passing its barrier next issues more
        // K/V loads, which the compiler's own wait would otherwise include)
        if (tok_class(kt) != 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(tb[i]));
        }
      }
    };

    // Token-dependent table: logits of tile kt in log2 units relative to m_ref (bias, scale
    // and reference in two FMAs), the causal / window mask applied after the bias, so a
    // table entry at a distance no visible key has never reaches the result.
    auto tok_logits = [&](int kt, float m_ref) {
      const int j0 = kt * kBK;
      const int cls = tok_class(kt);
      const int dl = pw0 + col - j0 - 4 * hf;  // distance of the lane's first key
      if (cls == 0) {
        const float c = fmaf(tok_sat, kLog2e, -m_ref);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], p.scale_log2, c);
      } else if (cls == 1) {
        // run [d0 - 3, d0 - 2, d0 - 1, d0]: key k of the run (distance d0 - k) is element 3 - k
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const u32x2_t w = tb[4 * kb + (r >> 2)];
            const int k = r & 3;
            const uint32_t word = k < 2 ? w[1] : w[0];
            const float bv = (k & 1) ? __uint_as_float(word << 16) : __uint_as_float(word & 0xffff0000u);
            s[kb][r] = fmaf(bv, kLog2e, fmaf(s[kb][r], p.scale_log2, -m_ref));
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int d0 = dl - 32 * kb - 8 * (r >> 2);
            const int a = min(max(d0 - 3, 0), p.R - 4);
            const int dist = d0 - (r & 3);
            const int idx = min(max(dist - a, 0), 3);
            const u32x2_t w = tb[4 * kb + (r >> 2)];
            const uint32_t word = idx >= 2 ? w[1] : w[0];
            float bv = (idx & 1) ? __uint_as_float(word & 0xffff0000u) : __uint_as_float(word << 16);
            bv = dist >= p.R - 1 ? tok_sat : bv;
            bv = dist < 0 ? 0.f : bv;
            s[kb][r] = fmaf(bv, kLog2e, fmaf(s[kb][r], p.scale_log2, -m_ref));
          }
      }
      if (j0 + kBK - 1 > pw0 || j0 < pw_last - Weff + 1) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
            s[kb][r] = (uint32_t)(dl - c) < (uint32_t)Weff ? s[kb][r] : kNegInf;
          }
      }
    };

    // Softmax half-step of tile kt: logits in log2 units relative to the running maximum
    // (the bias and the max in one FMA), the causal / window mask on edge tiles, the row
    // maximum, a lazy raise of the running maximum (only when a row's maximum grows by
    // more than the slack, rescaling O and the normaliser), then P = exp2 in fp32 for the
    // normaliser (the log-sum-exp needs that accuracy) and rounded to bf16 for P.V.
    auto softmax_half = [&](int kt) {
      const int j0 = kt * kBK;
      if (!TOK && (j0 + kBK - 1 > pw0 || j0 < pw_last - Weff + 1)) {
        // edge tile: mask the raw scores (in place; -inf stays -inf through the logit FMA).
        // Key 32 kb + 8 (r >> 2) + 4 hf + (r & 3) is at distance dl - c(kb, r) from this
        // lane's query; visible iff 0 <= distance < Weff (Weff is huge without a window).
        const int dl = pw0 + col - j0 - 4 * hf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
            s[kb][r] = (uint32_t)(dl - c) < (uint32_t)Weff ? s[kb][r] : kNegInf;
          }
      }
      const bool fresh = m_run == kNegInf;
      const float m_ref = fresh ? 0.f : m_run;
      const float raise_above = fresh ? kNegInf : kRescaleSlack;
      if constexpr (!TOK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], p.scale_log2, -m_ref);
      } else {
        tok_logits(kt, m_ref);
      }
      float ma = max3f(s[0][0], s[0][1], s[0][2]);
      float mb = max3f(s[1][0], s[1][1], s[1][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) {
        ma = max3f(ma, s[0][r], s[0][r + 1]);
        mb = max3f(mb, s[1][r], s[1][r + 1]);
      }
      const float mx = half_swap_max3(max3f(ma, mb, s[0][15]), s[1][15]);
      const bool raise = mx > raise_above;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float delta = raise ? mx : 0.f;
        const float m_new = m_ref + delta;
        const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;
        m_run = raise ? m_new : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
        s[0] -= delta;
        s[1] -= delta;
      }
      float lsum;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * half + 2 * e;
            const float e0 = fast_exp2(s[kb][r]), e1 = fast_exp2(s[kb][r + 1]);
            lsum = (kb | half | e) ? lsum + (e0 + e1) : e0 + e1;
            w[e] = pack_bf16x2(e0, e1);
          }
          pk[kb][half] = w;
        }
      l_run += lsum;
    };

    // ---- key loop: two wave groups in ping-pong -------------------------------------
    // Waves 0-3 and 4-7 (one of each on every SIMD) run the same code per tile t: read the
    // seeds of tile t, an MFMA half-step (P.V of tile t - 1, then S of tile t), a softmax
    // half-step (tile t).  There is one workgroup barrier per tile; barrier t means "tile t
    // is whole in LDS" (every wave waited for its share of it first), and right after it
    // each wave starts its share of tile t + 2, into the stage of tile t - 2.  Group 0
    // passes barrier t before its MFMA half of tile t, group 1 after it (and barrier 0 ahead
    // of everything), so between barriers t and t + 1 group 0 runs MFMA(t) then softmax(t)
    // while group 1 runs softmax(t - 1) then MFMA(t): the two waves of a SIMD take turns on
    // the matrix cores and the vector ALU.  Every read of a stage falls between the barrier
    // that completes its tile and the barrier that refills it, two tiles later.
    const bool g1 = wave >= kWaves / 2;
    const int prologue = min(2, n_tiles);
    for (int i = 0; i < prologue; ++i) issue_tile(kt_begin + i, i);
    // P of "tile -1" is zero and the V rows of the last stage are zeroed, so that the first
    // MFMA half-step can run its P.V like every other (it adds nothing)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) pk[kb][half] = zero_u32x4();
    {
      u32x4_t* vlast = (u32x4_t*)(ring + (kStages - 1) * kStageBytes + kKVBytes);
      vlast[tid] = zero_u32x4();
      vlast[tid + kThreads] = zero_u32x4();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // before the first barrier
    }
    auto tile_barrier = [&](int j) {
      if (j + 1 < n_tiles) vm_wait<kLPS>();  // tile j; tile j + 1 may still be loading
      else vm_wait<0>();
      wg_barrier_reads_in_flight();
      if (j + 2 < n_tiles) issue_tile(kt_begin + j + 2, (j + 2) % kStages);
    };
    if (g1 && n_tiles > 0) tile_barrier(0);
    for (int t = 0; t < n_tiles; ++t) {
      if (!g1) tile_barrier(t);
      mfma_half(t % kStages, (t + kStages - 1) % kStages, kt_begin + t);
      if (g1 && t + 1 < n_tiles) tile_barrier(t + 1);
      softmax_half(kt_begin + t);
    }
    // claim the next job now: the atomic's round trip overlaps the epilogue
    int claimed = n_slots;
    if (tid == 0 && p.queue != nullptr)
      claimed = (int)gridDim.x + __hip_atomic_fetch_add(p.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n_tiles > 0) {
      // P.V of the last tile
      const uint32_t vz = vz0 + ((n_tiles - 1) % kStages) * kStageBytes;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        u32x4_t va[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint32_t a = (vz ^ (64u * db)) + 256u * (16 * G);
          const u32x2_t lo = lds_tr8(a), hi = lds_tr8(a + 2048u);
          va[db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = mfma_32x32x16(va[db], pk[G >> 1][G & 1], o[db]);
      }
    }

    // ---- epilogue --------------------------------------------------------------------
    const float l_tot = half_swap_sum(l_run);
    const int tq = tw0 + col;
    const bool row_ok = wave_active && tq < qlen;
    const size_t obase = ((qrow0 + (row_ok ? tq : 0)) * p.Hq + h) * kHeadDim;
    if (!is_piece) {
      if (row_ok) {
        const float inv = 1.f / l_tot;
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
          p.lse[(qrow0 + tq) * p.Hq + h] = (m_run + __log2f(l_tot)) * kLn2;
      }
    } else {

      // A piece: its normalised output and log2-sum-exp per row go to the workspace (a row
      // that saw no key of this piece: zeros and -inf).  The piece that finishes last merges
      // all pieces of the tile from the workspace (its own included), in piece order (so the
      // result does not depend on which one that is), and writes the output.
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;
      // Partial layout (per piece, per wave): 16-byte chunk c = 4 db + q of every lane, then
      // the lane -- each 16-byte store or load of a wave covers 1 KB of consecutive bytes.
      const int wrow = wave * 32 + col;  // row of the workgroup, 0..255
      const size_t my_slot = (size_t)job * p.parts + piece;  // piece j of a job: slot job * parts + j
      auto part_o = [&](size_t sl) { return p.ws_o + ((sl * kWaves + wave) * 32 * kHeadDim + 4 * lane); };
      // The partials are written and read with device-coherent accesses (the sc1 bit, as a
      // relaxed agent-scope atomic access of this target has it), which go to the coherence
      // point directly: a device-scope fence instead would write back and invalidate this
      // XCD's whole L2, and with it the K/V tiles of every other workgroup.
      auto st_dev = [](float* a, float v) { __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
      auto ld_dev = [](const float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
      {
        float* wo = part_o(my_slot);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t v = {o[db][4 * q] * inv, o[db][4 * q + 1] * inv, o[db][4 * q + 2] * inv,
                               o[db][4 * q + 3] * inv};
            // A VALU write to a register that an in-flight store of more than 8 bytes still
            // reads as data needs wait states; the compiler does not insert them after inline
            // assembly (without them the partials came out corrupted whenever the next
            // store's values reused these registers), so the store brings its own.
            asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 4"
                         :
                         : "v"(wo + (4 * db + q) * 256), "v"(v)
                         : "memory");
          }
        if (hf == 0) st_dev(p.ws_lse + my_slot * kWgRows + wrow, lse2);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partials have landed
      __syncthreads();
      if (tid == 0) {
        const int old = __hip_atomic_fetch_add(p.ws_cnt + job, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_piece = old == p.parts - 1;
        // every piece of this tile has counted: leave the counter at zero for the next call
        if (last_piece) __hip_atomic_store(p.ws_cnt + job, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (last_piece && row_ok) {
        const size_t slot0 = (size_t)job * p.parts;  // workgroup index of piece 0 of this tile
        float lse_j[kMaxPieces];
        float mmax = kNegInf;
#pragma unroll
        for (int j = 0; j < kMaxPieces; ++j) {
          lse_j[j] = j >= p.parts ? kNegInf : ld_dev(p.ws_lse + (slot0 + j) * kWgRows + wrow);
          mmax = fmaxf(mmax, lse_j[j]);
        }
        f32x16_t acc[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = zero_f32x16();
        float wsum = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxPieces; ++j) {
          if (j >= p.parts) break;
          const float w = lse_j[j] == kNegInf ? 0.f : fast_exp2(lse_j[j] - mmax);
          wsum += w;
          {
            const float* src = part_o(slot0 + j);
            f32x4_t x[16];
#pragma unroll
            for (int c = 0; c < 16; ++c)
              asm volatile("global_load_dwordx4 %0, %1, off sc1" : "=v"(x[c]) : "v"(src + c * 256) : "memory");
            asm volatile("s_waitcnt vmcnt(0)"
                         : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                           "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]),
                           "+v"(x[14]), "+v"(x[15])
                         :
                         : "memory");
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[db][4 * q + i] = fmaf(w, x[4 * db + q][i], acc[db][4 * q + i]);
          }
        }
        const float winv = 1.f / wsum;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d = 32 * db + 8 * q + 4 * hf;
            const float x0 = acc[db][4 * q + 0] * winv, x1 = acc[db][4 * q + 1] * winv;
            const float x2 = acc[db][4 * q + 2] * winv, x3 = acc[db][4 * q + 3] * winv;
            *(u32x2_t*)((uint16_t*)p.out + obase + d) = u32x2_t{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          }
        if (hf == 0 && p.lse != nullptr)
          p.lse[(qrow0 + tq) * p.Hq + h] = (mmax + __log2f(wsum)) * kLn2;
      }  // last piece
    }  // piece
    // next job: every wave is done with this one's LDS stages and shared flags
    if (tid == 0) next_slot = claimed;
    __syncthreads();
    slot = next_slot;
  }  // jobs
  // The workgroup that finishes last leaves the queue at zero for the next call.  Each
  // workgroup counts after its last claim has returned, so the last count comes after
  // every claim.
  if (tid == 0 && p.queue != nullptr) {
    const int done = __hip_atomic_fetch_add(p.queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1) {
      __hip_atomic_store(p.queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  const long long per_tile = (long long)p.B * p.Hkv * p.n_hg;
  long long grid = ((long long)p.n_tok_tiles - p.n_split) * per_tile + (long long)p.n_split * per_tile * p.parts;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // with a queue: one workgroup per compute unit, each running jobs until none is left
  if (p.queue != nullptr && grid > p.queue_workgroups) grid = p.queue_workgroups;
  if (p.block_table != nullptr)
    hipLaunchKernelGGL((prefill_bf16_kernel<true, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  else if (p.bias_tok != nullptr)
    hipLaunchKernelGGL((prefill_bf16_kernel<false, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<false, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rattn
