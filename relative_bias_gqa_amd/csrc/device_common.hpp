// device_common.hpp -- gfx950 building blocks shared by the attention kernels.
//
// MFMA operand layouts (v_mfma_f32_32x32x16_bf16, wave64), as used throughout:
//   A (32 x 16):  lane l holds A[l % 32][8 * (l / 32) + e],  e = 0..7
//   B (16 x 32):  lane l holds B[8 * (l / 32) + e][l % 32]
//   C (32 x 32):  lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// The kernels compute S^T = K Q^T and O^T = V^T P^T, so a lane's accumulator column
// is one query row and the softmax statistics of that row live in the lane and its
// partner lane l ^ 32.
//
// ds_read_b64_tr_b16 (LDS transpose read): within each group of 16 lanes, if lane m
// supplies the address of four consecutive 16-bit elements M[m][0..3], lane i receives
// M[4 e + i / 4][i % 4] for e = 0..3.  With lane m pointing at V[row0 + m / 4][col0 +
// 4 (m % 4)] this hands lane i the column V[row0 + 0..3][col0 + i] of a row-major tile,
// which is the V^T operand of the P.V product without any transposed store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap: lane l < 32 gets
// its partner's value in the second result, lane l >= 32 in the first).
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Maxima on v_max3_f32 / v_max_f32 directly: the operands here are results of FMAs or
// -inf, never signalling NaNs, so the quieting that fmaxf adds in IEEE mode is not needed.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// max(x, y) over this lane and lane l ^ 32
__device__ __forceinline__ float half_swap_max3(float x, float y) {
  const float m = max2f(x, y);
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return max2f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// V^T operand (32 d-rows x 16 keys) of one MFMA from a row-major bf16 V tile in LDS.
// Key order within the 16-key step: lane half hf supplies keys kbase + 4 hf + 0..3 and
// kbase + 8 + 4 hf + 0..3, matching the register order of the S^T accumulator.
__device__ __forceinline__ u32x4_t load_vt_operand(const uint16_t* v_tile, int stride, int kbase,
                                                   int dcol0, int lane) {
  const int m = lane & 15;
  const int hf = lane >> 5;
  const int row = kbase + 4 * hf + (m >> 2);
  const int col = dcol0 + 16 * ((lane >> 4) & 1) + 4 * (m & 3);
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v_tile + row * stride + col));
  const s16x4_t b =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v_tile + (row + 8) * stride + col));
  const u32x2_t ua = __builtin_bit_cast(u32x2_t, a);
  const u32x2_t ub = __builtin_bit_cast(u32x2_t, b);
  u32x4_t r;
  r[0] = ua[0];
  r[1] = ua[1];
  r[2] = ub[0];
  r[3] = ub[1];
  return r;
}

// P^T operand for one 16-key step from eight probabilities (accumulator registers
// 8*half .. 8*half+7 of a 32-key block), packed to bf16.
__device__ __forceinline__ u32x4_t pack_p_operand(const float* p8) {
  u32x4_t r;
  r[0] = pack_bf16x2(p8[0], p8[1]);
  r[1] = pack_bf16x2(p8[2], p8[3]);
  r[2] = pack_bf16x2(p8[4], p8[5]);
  r[3] = pack_bf16x2(p8[6], p8[7]);
  return r;
}

// LDS accesses through plain 32-bit byte addresses, so that the per-lane part of every
// operand address is one register and the rest is an immediate offset or an XOR with a
// constant (the K/V tile swizzles of the kernels are chosen to allow this).
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) float lds_f32_t;
__device__ __forceinline__ u32x4_t lds_ld16(uint32_t a) { return *(const lds_u32x4_t*)(size_t)a; }
__device__ __forceinline__ float lds_ldf(uint32_t a) { return *(const lds_f32_t*)(size_t)a; }
// 16-byte-chunk swizzle of LDS tiles with 256-byte rows: chunk c of row r is stored at chunk
// c ^ lds_swz(r), lds_swz(r) = 4 (r & 3) + ((r >> 2) & 3).  Sixteen consecutive rows read at one
// logical chunk (a row-wise MFMA operand, 16 lanes x 16 B) hit sixteen different chunks, and
// the rows x columns a transposed read (ds_read_b64_tr_b16) gathers in each half-wave hit all
// 64 banks.  Rows r and r + 8 differ by chunk bit 1 (byte address bit 5).  (The forward
// kernels keep their own V layout: this one measured no faster there.)
__device__ __forceinline__ int lds_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ u32x2_t lds_tr8(uint32_t a) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(size_t)a));
}

// ---- direct global -> LDS loads (global_load_lds_dword{,x4}) --------------------------
// Lane i of the issuing wave writes its 4 (or 16) bytes at LDS byte address
// M0 + 4 i (or 16 i); lanes that are switched off write nothing.  The loads are issued
// from inline assembly so that the compiler does not pair every later LDS read with a
// wait for all of them; the caller orders them explicitly with vm_wait<n>() (they count
// in vmcnt like any vector-memory load) and a workgroup barrier.  M0 is saved and restored
// around each load, and one wait state separates the M0 write from the load.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void dma16(const void* g, uint32_t lds_byte_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte_addr);
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(g), "s"(m0v)
      : "memory");
}

// The same as dma16 with the non-temporal cache policy, for data read exactly once (the
// paged KV stream of decode): measured 7 % faster on a 2.3 GB batch-64 decode than the
// default policy, which keeps the streamed lines in the caches.
__device__ __forceinline__ void dma16nt(const void* g, uint32_t lds_byte_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte_addr);
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(g), "s"(m0v)
      : "memory");
}

__device__ __forceinline__ void dma4(const void* g, uint32_t lds_byte_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte_addr);
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(g), "s"(m0v)
      : "memory");
}

// The same with a wave-uniform base address in SGPRs and a 32-bit per-lane byte offset,
// so that issuing a load needs no vector ALU work.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_byte_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte_addr);
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(off), "s"(base), "s"(m0v)
      : "memory");
}

__device__ __forceinline__ void dma4s(const void* base, uint32_t off, uint32_t lds_byte_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte_addr);
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(off), "s"(base), "s"(m0v)
      : "memory");
}

// A pointer that is the same in every lane, made provably so (SGPR pair) for the scalar
// base operand of dma16s / dma4s.
__device__ __forceinline__ const unsigned char* uniform_ptr(const void* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const unsigned char*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// Wave-uniform 32-bit load through the scalar cache (lgkmcnt), so that it does not wait
// behind the LDS-bound loads in flight.
__device__ __forceinline__ int uniform_load_i32(const int* ptr) {
  // readfirstlane returns a signed int: widen each half as unsigned
  const uint64_t a = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t ua = ((uint64_t)hi << 32) | (uint64_t)lo;
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=&s"(v) : "s"(ua) : "memory");
  return v;
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that is also a compiler fence for memory operations.  The wave's own
// LDS accesses complete first (lgkmcnt 0); outstanding global loads are not waited for.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that leaves the wave's own LDS reads in flight: for loops whose LDS
// reads all complete before their results are used (the compiler waits for them there),
// so that a wave never reaches a barrier that precedes a refill of the data it reads
// with such a read still pending.  Global -> LDS loads are ordered separately (vm_wait).
__device__ __forceinline__ void wg_barrier_reads_in_flight() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ u32x4_t zero_u32x4() {
  u32x4_t z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

__device__ __forceinline__ f32x16_t zero_f32x16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

}  // namespace rattn
