// Host driver of the sanitizer build: calls every entry point of include/rattn.h through the
// C-ABI layer (kernel launches stubbed, device pointers fake: the layer never dereferences
// them) and the CPU oracle of include/rattn_oracle.h on small inputs.  Checks the status
// codes, and that every buffer the layer derives from a caller's workspace lies inside it.
// Any out-of-bounds access, use of freed memory or undefined behaviour in the host code
// aborts the run with a sanitizer report; a failed check exits with status 1.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "rattn.h"
#include "rattn_oracle.h"
#include "stubs.hpp"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

// distinct, aligned, never-dereferenced device addresses
static void* dev(uintptr_t i) { return (void*)(uintptr_t)(0x100000000ULL + i * 0x10000000ULL); }

// [p, p + bytes) inside [ws, ws + ws_bytes)?
static bool inside(const void* p, size_t bytes, const void* ws, size_t ws_bytes) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)ws;
  return a >= b && a + bytes <= b + ws_bytes && a + bytes >= a;
}

static void prefill_cases() {
  struct Case { int B, Lq, Lk, Hq, Hkv, R, window, dtype, splits; };
  const Case cases[] = {
      {1, 8192, 8192, 16, 2, 4096, 4096, RATTN_BF16, 0}, {1, 8192, 32768, 16, 2, 4096, 0, RATTN_BF16, 0},
      {2, 300, 300, 8, 2, 40, 0, RATTN_BF16, 0},         {1, 500, 1500, 16, 2, 300, 0, RATTN_BF16, 3},
      {3, 1, 77, 4, 4, 5, 1, RATTN_BF16, 0},             {1, 129, 400, 4, 4, 33, 0, RATTN_FP32, 0},
      {1, 96, 96, 32, 2, 64, 0, RATTN_BF16, 2},          {1, 8192, 8192, 16, 2, 4096, 4096, RATTN_BF16, 7}};
  for (const Case& c : cases) {
    const size_t need = rattn_prefill_workspace_bytes(c.B, c.Lq, c.Lk, c.Hq, c.Hkv, c.window, c.dtype, c.splits);
    void* ws = need ? dev(50) : nullptr;
    const int before = stub::rec.prefill_bf16_calls + stub::rec.prefill_fp32_calls;
    int st = rattn_prefill(dev(1), dev(2), dev(3), (const float*)dev(4), dev(5), (float*)dev(6), c.B, c.Lq, c.Lk, c.Hq,
                           c.Hkv, 128, c.R, c.window, c.dtype, c.splits, ws, need, nullptr);
    CHECK(st == RATTN_OK);
    CHECK(stub::rec.prefill_bf16_calls + stub::rec.prefill_fp32_calls == before + 1);
    const rattn::PrefillParams& p = stub::rec.prefill;
    CHECK(p.hpw * p.tsub == 8 && p.G % p.hpw == 0 && p.n_hg * p.hpw == p.G);
    CHECK(p.n_tok_tiles == (c.Lq + 32 * p.tsub - 1) / (32 * p.tsub));
    if (p.queue) CHECK(inside(p.queue, 2 * sizeof(int), ws, need));
    const size_t groups = (size_t)p.n_split * c.B * c.Hkv * p.n_hg;
    if (p.ws_cnt && p.n_split) CHECK(inside(p.ws_cnt, groups * sizeof(int), ws, need));
    if (p.n_split) {
      const size_t pieces = groups * p.parts;
      CHECK(inside(p.ws_lse, pieces * 256 * sizeof(float), ws, need));
      CHECK(inside(p.ws_o, pieces * 256 * 128 * sizeof(float), ws, need));
    }
    if (need) {  // one byte short
      st = rattn_prefill(dev(1), dev(2), dev(3), (const float*)dev(4), dev(5), (float*)dev(6), c.B, c.Lq, c.Lk, c.Hq,
                         c.Hkv, 128, c.R, c.window, c.dtype, c.splits, ws, need - 1, nullptr);
      CHECK(st == RATTN_ERR_WORKSPACE);
    }
    // token-dependent bias (bf16 only)
    if (c.dtype == RATTN_BF16 && c.R >= 4) {
      st = rattn_prefill_tokbias(dev(1), dev(2), dev(3), dev(4), dev(5), (float*)dev(6), c.B, c.Lq, c.Lk, c.Hq, c.Hkv,
                                 128, c.R, c.window, c.splits, ws, need, nullptr);
      CHECK(st == RATTN_OK);
      CHECK(stub::rec.prefill.bias_tok == dev(4));
    }
  }
  // invalid arguments: nothing launched, a status and a message
  const int before = stub::rec.prefill_bf16_calls;
  CHECK(rattn_prefill(nullptr, dev(2), dev(3), (const float*)dev(4), dev(5), nullptr, 1, 8, 8, 2, 1, 128, 4, 0,
                      RATTN_BF16, 0, dev(50), 1 << 20, nullptr) == RATTN_ERR_INVALID_ARG);
  CHECK(rattn_prefill(dev(1), dev(2), dev(3), (const float*)dev(4), dev(5), nullptr, 1, 9, 8, 2, 1, 128, 4, 0,
                      RATTN_BF16, 0, dev(50), 1 << 20, nullptr) == RATTN_ERR_INVALID_ARG);  // Lq > Lk
  CHECK(rattn_prefill(dev(1), dev(2), dev(3), (const float*)dev(4), dev(5), nullptr, 1, 8, 8, 3, 2, 128, 4, 0,
                      RATTN_BF16, 0, dev(50), 1 << 20, nullptr) == RATTN_ERR_INVALID_ARG);  // Hq % Hkv
  CHECK(rattn_prefill(dev(1), dev(2), dev(3), (const float*)dev(4), dev(5), nullptr, 1, 8, 8, 2, 1, 64, 4, 0,
                      RATTN_BF16, 0, dev(50), 1 << 20, nullptr) == RATTN_ERR_UNSUPPORTED);  // head_dim
  CHECK(rattn_prefill_tokbias(dev(1), dev(2), dev(3), (const void*)((uintptr_t)dev(4) + 2), dev(5), nullptr, 1, 8, 8,
                              2, 1, 128, 8, 0, 0, dev(50), 1 << 20, nullptr) == RATTN_ERR_INVALID_ARG);  // alignment
  CHECK(stub::rec.prefill_bf16_calls == before);
  CHECK(std::strlen(rattn_last_error()) > 0);
  CHECK(rattn_prefill_workspace_bytes(-1, 8, 8, 2, 1, 0, RATTN_BF16, 0) == 0);
}

static void paged_prefill_cases() {
  const int B = 4, Lq = 700, Hq = 16, Hkv = 2, mbps = 64, nblocks = 256;
  const size_t need = 1 << 20;
  int st = rattn_prefill_paged(dev(1), dev(2), dev(3), (const int*)dev(7), (const int*)dev(8), (const int*)dev(9),
                               (const float*)dev(4), dev(5), (float*)dev(6), B, Lq, Hq, Hkv, 128, 128, 512, 0,
                               nblocks, mbps, 8192, dev(50), need, nullptr);
  CHECK(st == RATTN_OK || st == RATTN_ERR_WORKSPACE);
  CHECK(rattn_prefill_paged(dev(1), dev(2), dev(3), (const int*)dev(7), (const int*)dev(8), nullptr,
                            (const float*)dev(4), dev(5), (float*)dev(6), B, Lq, Hq, Hkv, 128, 64, 512, 0, nblocks,
                            mbps, 8192, dev(50), need, nullptr) != RATTN_OK);  // block size 64
}

static void decode_cases() {
  struct Case { int B, n_q, Hq, Hkv, ctx, splits; };
  const Case cases[] = {{64, 1, 16, 2, 8192, 0}, {1, 9, 16, 2, 1 << 20, 0}, {3000, 2, 8, 1, 300, 5},
                        {5, 16, 32, 2, 5000, 1}, {1, 1, 1, 1, 1, 0},        {2, 128, 1, 1, 777, 5000}};
  for (const Case& c : cases) {
    const int mbps = (c.ctx + 127) / 128;
    const int P = rattn_decode_num_splits(c.B, c.n_q, c.Hq, c.Hkv, c.ctx, c.splits);
    CHECK(P >= 1);
    const size_t need = rattn_decode_workspace_bytes(c.B, c.n_q, c.Hq, c.Hkv, c.ctx, c.splits);
    CHECK(need > 0);
    void* ws = dev(60);
    stub::rec.on_decode = [&](const rattn::DecodeParams& p) {
      const size_t slots = (size_t)(p.P + (size_t)p.B * p.KH) * p.KS;
      return p.B >= 1 && p.rows == c.n_q * p.gs && p.rows <= 128 && p.gs * p.n_hs == p.G &&
             inside(p.ws_o, slots * p.rows * 128 * sizeof(float), ws, need) &&
             inside(p.ws_lse, slots * p.rows * sizeof(float), ws, need);
    };
    int st = rattn_decode_paged(dev(1), dev(2), dev(3), (const int*)dev(7), (const int*)dev(8), nullptr,
                                (const float*)dev(4), dev(5), (float*)dev(6), c.B, c.n_q, c.Hq, c.Hkv, 128, 128, 4096,
                                c.B * mbps, mbps, c.ctx, c.splits, ws, need, nullptr);
    CHECK(st == RATTN_OK);
    CHECK(rattn_decode_paged(dev(1), dev(2), dev(3), (const int*)dev(7), (const int*)dev(8), nullptr,
                             (const float*)dev(4), dev(5), (float*)dev(6), c.B, c.n_q, c.Hq, c.Hkv, 128, 128, 4096,
                             c.B * mbps, mbps, c.ctx, c.splits, ws, need - 1, nullptr) == RATTN_ERR_WORKSPACE);
    // allocation-free variant: the partials must fit the static scratch, or the call is refused
    const void* sc = stub::scratch_base();
    const size_t sc_bytes = rattn_decode_paged_noalloc_max_scratch_bytes();
    stub::rec.on_decode = [&](const rattn::DecodeParams& p) {
      const size_t slots = (size_t)(p.P + (size_t)p.B * p.KH) * p.KS;
      return inside(p.ws_o, slots * p.rows * 128 * sizeof(float), sc, sc_bytes) &&
             inside(p.ws_lse, slots * p.rows * sizeof(float), sc, sc_bytes);
    };
    st = rattn_decode_paged_noalloc(dev(1), dev(2), dev(3), (const int*)dev(7), (const int*)dev(8), nullptr,
                                    (const float*)dev(4), dev(5), (float*)dev(6), c.B, c.n_q, c.Hq, c.Hkv, 128, 128,
                                    4096, c.B * mbps, mbps, c.ctx, c.splits, nullptr);
    CHECK(st == (need <= sc_bytes ? RATTN_OK : RATTN_ERR_WORKSPACE));
  }
  stub::rec.on_decode = [](const rattn::DecodeParams&) { return true; };
  CHECK(rattn_decode_num_splits(0, 1, 8, 2, 10, 0) <= 0 || rattn_decode_workspace_bytes(0, 1, 8, 2, 10, 0) == 0);
  CHECK(rattn_decode_workspace_bytes(1, 129, 1, 1, 10, 0) == 0);  // too many rows
}

static void sconv_cases() {
  int st = rattn_kv_sconv_write(dev(1), dev(2), (const float*)dev(3), (const float*)dev(4), dev(5), dev(6), dev(7),
                                dev(8), (const int*)dev(9), (const int*)dev(10), (const int*)dev(11), 4, 2, 128, 128,
                                64, 16, 3000, nullptr);
  CHECK(st == RATTN_OK);
  CHECK(stub::rec.sconv.max_new == 3000 && stub::rec.sconv.B == 4);
  CHECK(rattn_kv_sconv_write(dev(1), dev(2), (const float*)dev(3), (const float*)dev(4), dev(5), dev(6), dev(7),
                             dev(8), (const int*)dev(9), (const int*)dev(10), (const int*)dev(11), 4, 2, 96, 128, 64,
                             16, 3000, nullptr) != RATTN_OK);
}

static long long kv_steps(int Lq, int Lk, int window, int blk) {
  const long long off = (long long)Lk - Lq, weff = window > 0 ? window : 0x40000000LL;
  const long long J0 = 128LL * blk, lo = J0 - off > 0 ? J0 - off : 0;
  const long long hi = (long long)Lq - 1 < J0 + 127 + weff - 1 - off ? (long long)Lq - 1 : J0 + 127 + weff - 1 - off;
  return lo <= hi ? hi / 32 - lo / 32 + 1 : 0;
}

static void backward_cases() {
  struct Case { int B, Lq, Lk, Hq, Hkv, R, window; };
  const Case cases[] = {{1, 8192, 8192, 16, 2, 4096, 4096}, {2, 300, 300, 8, 2, 40, 0}, {1, 150, 700, 8, 2, 77, 120},
                        {1, 96, 96, 48, 3, 64, 0},          {1, 1, 5, 1, 1, 3, 1},     {1, 0, 300, 8, 2, 32, 0},
                        {1, 2048, 32768, 16, 2, 512, 0}, {1, 1024, 1024, 16, 2, 300, 0}};
  for (const Case& c : cases) {
    const size_t need = rattn_prefill_backward_workspace_bytes(c.B, c.Lq, c.Lk, c.Hq, c.Hkv);
    CHECK(need >= 256);
    void* ws = dev(70);
    const int before = stub::rec.backward_calls;
    int st = rattn_prefill_backward(dev(1), dev(2), dev(3), (const float*)dev(4), dev(5), dev(6), (const float*)dev(7),
                                    (float*)dev(8), (float*)dev(9), (float*)dev(10), (float*)dev(11), c.B, c.Lq, c.Lk,
                                    c.Hq, c.Hkv, 128, c.R, c.window, ws, need, nullptr);
    CHECK(st == RATTN_OK);
    CHECK(stub::rec.backward_calls == before + 1);
    const rattn::BackwardParams& p = stub::rec.backward;
    const size_t rows = (size_t)c.B * c.Lq * c.Hq, plane = (size_t)c.B * c.Lk * c.Hkv * 128;
    CHECK(p.n_pairs == (c.Hq / c.Hkv + 1) / 2);
    CHECK(inside(p.D, rows * 4, ws, need) && inside(p.L2, rows * 4, ws, need));
    CHECK(inside(p.part_dk, 2 * p.n_pairs * plane * 4, ws, need));
    CHECK(inside(p.part_dv, 2 * p.n_pairs * plane * 4, ws, need));
    // the dq pass's units (a token tile x head group x KV head x sequence): two partial slots of
    // 8 waves x 64 x 64 fp32 each, and one split counter each
    const size_t units = (size_t)p.n_tok_tiles * c.B * c.Hkv * p.n_hg;
    CHECK(p.hpw * p.tsub == 8 && p.n_hg * p.hpw == c.Hq / c.Hkv);
    CHECK(inside(p.dq_part, units * 2 * 8 * 64 * 64 * 4, ws, need));
    CHECK(inside(p.dq_cnt, units * 4, ws, need));
    // the bias table in score units: Rs = min(R, Lk) entries per head
    CHECK(p.Rs == (c.R < c.Lk ? c.R : c.Lk));
    CHECK(inside(p.bias_s, (size_t)c.Hq * p.Rs * 4, ws, need));
    CHECK((p.kv_chunks == 1 || p.kv_chunks == 2) && (p.q_chunks == 1 || p.q_chunks == 2));
    // the plans on 256 compute units: the 8K-token window-4096 workload uncut (its 512 + 512
    // units fill the grid; measured 0.847 ms against 0.880 with both passes cut in two), and a
    // causal 1024-token prefill, whose 64 + 64 units would leave most compute units idle, with
    // both passes cut in two
    if (stub::rec.compute_units == 256 && c.Lq == 8192 && c.Lk == 8192 && c.window == 4096)
      CHECK(p.kv_chunks == 1 && p.q_chunks == 1);
    if (stub::rec.compute_units == 256 && c.Lq == 1024 && c.Lk == 1024 && c.window == 0)
      CHECK(p.kv_chunks == 2 && p.q_chunks == 2);
    long long most = 1;
    for (int blk = 0; blk < (c.Lk + 127) / 128; ++blk) {
      const long long s = kv_steps(c.Lq, c.Lk, c.window, blk);
      most = s > most ? s : most;
    }
    CHECK((long long)p.kv_chunk * p.kv_chunks >= most && p.kv_chunk >= 1);
    CHECK(p.q_chunk >= 1);
    CHECK(rattn_prefill_backward(dev(1), dev(2), dev(3), (const float*)dev(4), dev(5), dev(6), (const float*)dev(7),
                                 (float*)dev(8), (float*)dev(9), (float*)dev(10), (float*)dev(11), c.B, c.Lq, c.Lk,
                                 c.Hq, c.Hkv, 128, c.R, c.window, ws, need - 1, nullptr) == RATTN_ERR_WORKSPACE);
  }
  CHECK(rattn_prefill_backward_workspace_bytes(1, 1, 1, 3, 2) == 0);
  CHECK(rattn_prefill_backward(dev(1), dev(2), dev(3), (const float*)dev(4), dev(5), dev(6), (const float*)dev(7),
                               (float*)dev(8), (float*)dev(9), (float*)dev(10), (float*)dev(11), 1, 9, 8, 2, 1, 128, 4,
                               0, dev(70), 1 << 20, nullptr) == RATTN_ERR_INVALID_ARG);
}

// ---- the CPU oracle on small inputs ------------------------------------------------------
static uint16_t to_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (uint16_t)((u + 0x7FFF + ((u >> 16) & 1)) >> 16);
}

static void oracle_cases() {
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 1.f);
  const int B = 2, n_q = 5, Lk = 37, Hq = 4, Hkv = 2, D = 128, R = 9, bs = 16, mbps = 3;
  std::vector<uint16_t> q((size_t)B * n_q * Hq * D), k((size_t)B * Lk * Hkv * D), v(k.size());
  for (auto* a : {&q, &k, &v})
    for (auto& x : *a) x = to_bf16(nd(rng));
  std::vector<double> bias((size_t)Hq * R), bias_tok((size_t)B * n_q * Hq * R);
  for (auto& x : bias) x = 0.5 * nd(rng);
  for (auto& x : bias_tok) x = 0.5 * nd(rng);
  std::vector<int> ctx = {37, 20}, windows = {0, 7};
  std::vector<double> out((size_t)B * n_q * Hq * D), lse((size_t)B * n_q * Hq), probs((size_t)B * n_q * Hq * Lk);
  for (int threads : {1, 2}) {
    CHECK(rattn_ref_cpu(q.data(), k.data(), v.data(), nullptr, ctx.data(), windows.data(), bias.data(), out.data(),
                        lse.data(), probs.data(), B, n_q, Lk, Hq, Hkv, D, 0, R, 0, RATTN_ORACLE_BF16, threads) == 0);
    for (double x : out) CHECK(std::isfinite(x));
    CHECK(rattn_ref_cpu_tokbias(q.data(), k.data(), v.data(), nullptr, ctx.data(), nullptr, bias_tok.data(),
                                out.data(), lse.data(), nullptr, B, n_q, Lk, Hq, Hkv, D, 0, R, 0, RATTN_ORACLE_BF16,
                                threads) == 0);
    for (double x : lse) CHECK(std::isfinite(x));
  }
  // paged: blocks of 16 tokens, a scrambled table
  std::vector<int> table = {4, 1, 3, 0, 5, 2};
  std::vector<uint16_t> kc((size_t)6 * bs * Hkv * D), vc(kc.size());
  for (auto* a : {&kc, &vc})
    for (auto& x : *a) x = to_bf16(nd(rng));
  CHECK(rattn_ref_cpu(q.data(), kc.data(), vc.data(), table.data(), ctx.data(), windows.data(), bias.data(), out.data(),
                      lse.data(), nullptr, B, n_q, Lk, Hq, Hkv, D, bs, R, mbps, RATTN_ORACLE_BF16, 0) == 0);
  // invalid: a context shorter than the queries
  std::vector<int> bad = {3, 20};
  CHECK(rattn_ref_cpu(q.data(), k.data(), v.data(), nullptr, bad.data(), nullptr, bias.data(), out.data(), lse.data(),
                      nullptr, B, n_q, Lk, Hq, Hkv, D, 0, R, 0, RATTN_ORACLE_BF16, 0) != 0);
  // backward: contiguous, Lq = n_q queries over Lk keys, with and without the forward output
  const int Lq = n_q;
  std::vector<uint16_t> dout((size_t)B * Lq * Hq * D), fo(dout.size());
  for (auto* a : {&dout, &fo})
    for (auto& x : *a) x = to_bf16(nd(rng));
  std::vector<double> dq(dout.size()), dk(k.size()), dv(k.size()), db(bias.size());
  std::vector<double> dqa(dq.size()), dka(dk.size()), dva(dv.size()), dba(db.size());
  for (const void* o : {(const void*)nullptr, (const void*)fo.data()}) {
    CHECK(rattn_ref_cpu_backward(q.data(), k.data(), v.data(), dout.data(), o, bias.data(), dq.data(), dk.data(),
                                 dv.data(), db.data(), dqa.data(), dka.data(), dva.data(), dba.data(), 0.25, B, Lq, Lk,
                                 Hq, Hkv, D, R, 6, RATTN_ORACLE_BF16, 2) == 0);
    for (double x : dk) CHECK(std::isfinite(x));
    for (size_t i = 0; i < db.size(); ++i) CHECK(std::fabs(db[i]) <= dba[i] * (1 + 1e-12) + 1e-300);
  }
  CHECK(rattn_ref_cpu_backward(q.data(), k.data(), v.data(), dout.data(), nullptr, bias.data(), dq.data(), dk.data(),
                               dv.data(), db.data(), nullptr, nullptr, nullptr, nullptr, 1.0, B, Lk + 1, Lk, Hq, Hkv, D,
                               R, 0, RATTN_ORACLE_BF16, 1) != 0);  // Lq > Lk
}

int main() {
  CHECK(rattn_abi_version() == RATTN_ABI_VERSION);
  int device = 0;
  for (int cus : {256, 304, 80}) {
    stub::rec.compute_units = cus;
    stub::rec.device = device++;
    prefill_cases();
    paged_prefill_cases();
    decode_cases();
    sconv_cases();
    backward_cases();
  }
  oracle_cases();
  // every stubbed launch was reached
  CHECK(stub::rec.prefill_bf16_calls > 0 && stub::rec.prefill_fp32_calls > 0 && stub::rec.decode_calls > 0);
  CHECK(stub::rec.sconv_calls > 0 && stub::rec.backward_calls > 0);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer driver: all checks passed\n");
  return 0;
}
