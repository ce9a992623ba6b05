// zl_device.h -- gfx950 device primitives shared by the decode kernels.
//
// Lane layouts used throughout (64-lane wavefront, lane = 16*g + n, g = lane/16):
//   v_mfma_f32_16x16x32_{f16,bf16}  D = A(16x32) * B(32x16) + C
//     A operand: lane holds A[row n][k 8g .. 8g+7]
//     B operand: lane holds B[k 8g .. 8g+7][col n]
//     C/D      : lane holds C[rows 4g .. 4g+3][col n]
//   ds_read_b64_tr_b16: inside each 16-lane group, lane m supplies the address
//     of 4 consecutive 16-bit values; lane 4a+b receives value b of the rows
//     given by lanes a, a+4, a+8, a+12 (a 4x16 -> 16x4 transpose).
// These were confirmed on the device with a one-instruction probe before the
// kernels were built on them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zl {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ZL_LDS __attribute__((address_space(3)))

enum DType { kF16 = 0, kBF16 = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit MFMA 16x16x32 with fp32 accumulation; operands are raw 16-bit lanes.
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(i16x8 a, i16x8 b, f32x4 c) {
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round-to-nearest-even conversion of fp32 to the 16-bit storage type.
template <int DT>
__device__ __forceinline__ uint16_t to16(float x) {
  if constexpr (DT == kF16)
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  else
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Two values rounded to nearest-even and packed (lo in bits 0-15): one
// v_cvt_pk_{f16,bf16}_f32 on gfx950.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  if constexpr (DT == kF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Hardware 2^x (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane (lane ^ mask) (a general exchange through the LDS crossbar).
__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = __lane_id();
  const int v = __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x));
  return __builtin_bit_cast(float, v);
}

// Sum of x over lanes 0 .. lane (an inclusive scan across the wave), in six
// doubling steps through the LDS crossbar.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute((lane >= d ? lane - d : lane) << 2, x);
    x += lane >= d ? y : 0;
  }
  return x;
}

// Reductions over the four 16-lane groups (lanes n, n+16, n+32, n+48) with
// the gfx950 lane-swap instructions, entirely in the VALU (no LDS round
// trip).  Given two registers that both hold x, v_permlane16_swap leaves the
// values of lanes l and l^16 in lane l of the two registers (one in each);
// v_permlane32_swap does the same for l and l^32.  Every lane of a head gets
// the bitwise same result (each stage combines the same two values, and max
// and + commute).  The swaps are written as inline asm: the compiler's
// builtin returns the pair, and when both halves feed one expression it has
// been seen to use the first half twice.  s_nop 1 gives the two wait states
// a lane swap needs after a VALU write of its operands.
__device__ __forceinline__ void lane_swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lane_swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// v_max_f32 written out: fmaxf on values that come out of inline asm costs
// two extra canonicalising maxes (IEEE mode quiets signalling NaNs), which
// the scores and maxima here (finite or -inf) never need.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float max_over_groups(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  lane_swap16(a, b);
  x = vmax(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  lane_swap32(a, b);
  return vmax(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// max_over_groups of four independent values at once: the four swaps of each
// stage go out back to back after one s_nop, so the four reductions overlap.
// The asm has no side effects beyond its operands (not volatile), so the
// scheduler may move other work around it.
__device__ __forceinline__ void max_over_groups4(float (&x)[4]) {
  uint32_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = b[i] = __builtin_bit_cast(uint32_t, x[i]);
  asm(
      "s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\t"
      "v_permlane16_swap_b32 %4, %5\n\tv_permlane16_swap_b32 %6, %7"
      : "+v"(a[0]), "+v"(b[0]), "+v"(a[1]), "+v"(b[1]), "+v"(a[2]), "+v"(b[2]), "+v"(a[3]), "+v"(b[3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = vmax(__builtin_bit_cast(float, a[i]), __builtin_bit_cast(float, b[i]));
    a[i] = b[i] = __builtin_bit_cast(uint32_t, x[i]);
  }
  asm(
      "s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\t"
      "v_permlane32_swap_b32 %4, %5\n\tv_permlane32_swap_b32 %6, %7"
      : "+v"(a[0]), "+v"(b[0]), "+v"(a[1]), "+v"(b[1]), "+v"(a[2]), "+v"(b[2]), "+v"(a[3]), "+v"(b[3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = vmax(__builtin_bit_cast(float, a[i]), __builtin_bit_cast(float, b[i]));
}

// The same for two values.
__device__ __forceinline__ void max_over_groups2(float (&x)[2]) {
  uint32_t a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) a[i] = b[i] = __builtin_bit_cast(uint32_t, x[i]);
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3"
      : "+v"(a[0]), "+v"(b[0]), "+v"(a[1]), "+v"(b[1]));
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    x[i] = vmax(__builtin_bit_cast(float, a[i]), __builtin_bit_cast(float, b[i]));
    a[i] = b[i] = __builtin_bit_cast(uint32_t, x[i]);
  }
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3"
      : "+v"(a[0]), "+v"(b[0]), "+v"(a[1]), "+v"(b[1]));
#pragma unroll
  for (int i = 0; i < 2; ++i) x[i] = vmax(__builtin_bit_cast(float, a[i]), __builtin_bit_cast(float, b[i]));
}

__device__ __forceinline__ float sum_over_groups(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  lane_swap16(a, b);
  x = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  lane_swap32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// 16 bytes from global memory straight into LDS: lane i's bytes land at
// lds_base + 16*i (lds_base must be wave-uniform).
__device__ __forceinline__ void dma16(const void* gptr, ZL_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 16, 0, 0);
}

// The same with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (the instruction's SADDR form): no vector address
// arithmetic per instruction.  Written as inline asm because the compiler
// widens the offset to a 64-bit vector address.  The compiler does not see
// this load, so it must be waited for explicitly (wait_vmcnt) before its LDS
// bytes are read, as every DMA here is; the s_nop separates the M0 write from
// the load.
__device__ __forceinline__ void dma16_saddr(const void* base, uint32_t off, ZL_LDS void* lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_base) : "memory");
}

// 16 bytes from global memory into registers, marked non-temporal: key/value
// rows are streamed once, so their lines need not stay in the caches.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}

// 16 bytes of registers into LDS.
__device__ __forceinline__ void lds_write_b128(ZL_LDS char* p, u32x4 v) { *(ZL_LDS u32x4*)p = v; }

// Wait until at most N vector-memory operations of this wave are outstanding.
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt/lgkmcnt left at max.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ u32x4 lds_read_b128(const ZL_LDS char* p) {
  return *(const ZL_LDS u32x4*)p;
}

// Transposing LDS read issued as inline asm: the compiler's builtin carries
// no memory information, so the compiler would make every such read wait for
// all in-flight global->LDS DMA (vmcnt(0)), serialising the load pipeline.
// The result is NOT ready until lds_wait<N>() has been passed with it.
template <int OFFSET = 0>
__device__ __forceinline__ i16x4 lds_read_tr16(const ZL_LDS char* p) {
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(p), "i"(OFFSET) : "memory");
  return r;
}

// Wait until at most N LDS operations of this wave are outstanding, and tie
// the eight given registers to that point so no use of them is scheduled
// earlier.
#define ZL_LGKM_WAIT8(NSTR)                                                            \
  asm volatile("s_waitcnt lgkmcnt(" NSTR ")"                                          \
               : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6), \
                 "+v"(r7))
template <int N>
__device__ __forceinline__ void lds_wait(i16x4& r0, i16x4& r1, i16x4& r2, i16x4& r3, i16x4& r4,
                                         i16x4& r5, i16x4& r6, i16x4& r7) {
  static_assert(N == 0 || N == 8, "supported lgkmcnt values");
  if constexpr (N == 0)
    ZL_LGKM_WAIT8("0");
  else
    ZL_LGKM_WAIT8("8");
}
#undef ZL_LGKM_WAIT8

// Workgroup barrier that orders LDS only (finished LDS reads/writes of every
// wave before any wave continues).  Unlike __syncthreads it does not wait for
// this wave's outstanding global loads, so DMA prefetches stay in flight.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Make the compiler wait for (and consider complete) registers loaded from
// global memory, at this point.
template <typename T>
__device__ __forceinline__ void touch(T& r) {
  asm volatile("" : "+v"(r));
}

__device__ __forceinline__ int readfirstlane(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace zl
