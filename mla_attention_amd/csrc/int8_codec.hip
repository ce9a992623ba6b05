// int8_codec.hip -- per-chunk INT8 coding of an all-reduce payload, the
// single-GPU half of ZhiLight's INT8 all-reduce (first page, section 1 on
// dual streams and the INT8 all-reduce; second page, section "Dual streams,
// host all-reduce and the memory model"): the 16-bit payload that a
// tensor-parallel all-reduce would move is coded to one byte per element plus
// one fp32 scale per chunk of consecutive elements, and one hop of a ring
// all-reduce adds its own values to a received coded chunk and codes the sum
// again.  Per chunk (symmetric, 127 levels per sign):
//   amax = max |x|,  r = 127 / amax (0 when amax = 0),
//   code = rint(x * r) (ties to even),  scale = amax / 127,
//   hop:  y = code_in * scale_in + local.
// Codes are integers decided by floating point, so every step is an fp32
// operation rounded on its own: the file is compiled without contraction and
// the divisions are the correctly rounded ones.
//
// Layout: one wavefront per group of 1, 2 or 4 consecutive chunks of 64*E
// elements (E = 4, 8 or 16: chunks of 256, 512 or 1024), lane l holding
// elements l*E .. l*E+E-1 of each, so that every lane moves one 8-to-32-byte
// piece of each array; a group's loads are all issued before any arithmetic;
// the chunk maximum is a wave reduction in the vector unit.  Every byte is
// touched once, so the full-width loads and stores are non-temporal (the
// lines need not stay in the caches; measured 3-7% faster).  HBM-bound:
// 2 bytes in and 1 out per element to code, 1 in and 2 out to decode, 3 in
// and 1 to 3 out for a hop; the scales add 4 bytes per chunk.
#include "zl_device.h"
#include "zl_kernels.h"

#pragma clang fp contract(off)

namespace zl {
namespace {

template <int DT>
__device__ __forceinline__ float from16(uint16_t h) {
  if constexpr (DT == kF16)
    return (float)__builtin_bit_cast(_Float16, h);
  else
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Maximum over the wave of a non-negative, non-NaN value, whose bit pattern
// then orders like the value: DPP rotations by 8, 4, 2 and 1 lanes within
// each row of 16, then the lane swaps across the rows (all in the vector
// unit; through the LDS crossbar the six steps cost the coding kernels 2-4%).
// Call with all 64 lanes active.
__device__ __forceinline__ float wave_max(float v) {
  int x = __builtin_bit_cast(int, v);
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));  // row_ror:8
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false));  // row_ror:4
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false));  // row_ror:2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false));  // row_ror:1
  return max_over_groups(__builtin_bit_cast(float, x));
}

// E consecutive 16-bit values (valid of them; the rest read as 0).
template <int DT, int E>
__device__ __forceinline__ void load16(const uint16_t* p, int valid, float (&v)[E]) {
  if (valid == E) {
    uint16_t h[E];
    if constexpr (E == 4) {
      *(u32x2*)h = __builtin_nontemporal_load((const u32x2*)p);
    } else {
#pragma unroll
      for (int i = 0; i < E / 8; ++i) *(u32x4*)(h + 8 * i) = __builtin_nontemporal_load((const u32x4*)(p + 8 * i));
    }
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = from16<DT>(h[e]);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = e < valid ? from16<DT>(p[e]) : 0.f;
  }
}

template <int DT, int E>
__device__ __forceinline__ void store16(uint16_t* p, int valid, const float (&v)[E]) {
  uint16_t h[E];
#pragma unroll
  for (int e = 0; e < E; ++e) h[e] = to16<DT>(v[e]);
  if (valid == E) {
    if constexpr (E == 4) {
      __builtin_nontemporal_store(*(const u32x2*)h, (u32x2*)p);
    } else {
#pragma unroll
      for (int i = 0; i < E / 8; ++i) __builtin_nontemporal_store(*(const u32x4*)(h + 8 * i), (u32x4*)(p + 8 * i));
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e < valid) p[e] = h[e];
  }
}

template <int E>
__device__ __forceinline__ void load_codes(const int8_t* p, int valid, float (&v)[E]) {
  int8_t c[E];
  if (valid == E) {
    if constexpr (E == 4)
      *(uint32_t*)c = __builtin_nontemporal_load((const uint32_t*)p);
    else if constexpr (E == 8)
      *(u32x2*)c = __builtin_nontemporal_load((const u32x2*)p);
    else
      *(u32x4*)c = __builtin_nontemporal_load((const u32x4*)p);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) c[e] = e < valid ? p[e] : (int8_t)0;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = (float)c[e];
}

template <int E>
__device__ __forceinline__ void store_codes(int8_t* p, int valid, const int8_t (&c)[E]) {
  if (valid == E) {
    if constexpr (E == 4)
      __builtin_nontemporal_store(*(const uint32_t*)c, (uint32_t*)p);
    else if constexpr (E == 8)
      __builtin_nontemporal_store(*(const u32x2*)c, (u32x2*)p);
    else
      __builtin_nontemporal_store(*(const u32x4*)c, (u32x4*)p);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e < valid) p[e] = c[e];
  }
}

// Chunks a wave loads before coding any of them (memory-level parallelism),
// measured per operation on a cold 256 MiB payload with the non-temporal
// accesses: decoding gains from four (71 against 75-85 us with fewer), the
// hop, which moves four arrays, runs best with two (130 against 139 us with
// one and 145 with four), coding is indifferent.
template <int OP>
constexpr int chunks_per_wave() {
  return OP == kCodecDequantize ? 4 : 2;
}

// Most workgroups per launch (the waves stride over the groups beyond), also
// measured on a cold 256 MiB payload: coding and the hop run 2-3% faster with
// 32768 than with 8192, decoding 3% slower.
template <int OP>
constexpr long long max_blocks() {
  return OP == kCodecDequantize ? 8192 : 32768;
}

template <int OP, int DT, int E>
__global__ __launch_bounds__(256) void codec_kernel(CodecArgs a) {
  constexpr int C = 64 * E;
  constexpr int U = chunks_per_wave<OP>();
  const int lane = __lane_id();
  const int wave = (int)threadIdx.x >> 6;
  const long long nchunks = (a.n + C - 1) / C;
  const long long ngroups = (nchunks + U - 1) / U;
  for (long long gi = (long long)blockIdx.x * 4 + wave; gi < ngroups; gi += (long long)gridDim.x * 4) {
    // Chunks gi*U .. gi*U+U-1: all loads first, then the arithmetic.
    float v[U][E];
    int valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long c = gi * U + u;
      const long long left = a.n - (c * C + (long long)lane * E);
      valid[u] = left <= 0 ? 0 : (left >= E ? E : (int)left);
      const long long e0 = c * C + (long long)lane * E;
      if constexpr (OP == kCodecQuantize) {
        load16<DT, E>(a.x + e0, valid[u], v[u]);
      } else {
        load_codes<E>(a.codes_in + e0, valid[u], v[u]);
      }
    }
    if constexpr (OP != kCodecQuantize) {
      float l[U][E];
      if constexpr (OP == kCodecReduce) {
#pragma unroll
        for (int u = 0; u < U; ++u) load16<DT, E>(a.x + (gi * U + u) * C + (long long)lane * E, valid[u], l[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const long long c = gi * U + u;
        const float s = c < nchunks ? a.scales_in[c] : 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          v[u][e] = v[u][e] * s;
          if constexpr (OP == kCodecReduce) v[u][e] = v[u][e] + l[u][e];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long c = gi * U + u;
      const long long e0 = c * C + (long long)lane * E;
      if (OP != kCodecQuantize && a.out16) store16<DT, E>(a.out16 + e0, valid[u], v[u]);
      if (OP == kCodecDequantize || !a.codes_out || c >= nchunks) continue;
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(v[u][e]));  // absent elements are 0
      m = wave_max(m);
      const float r = m > 0.f ? 127.f / m : 0.f;
      int8_t q[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float t = rintf(v[u][e] * r);
        q[e] = (int8_t)(t > 127.f ? 127.f : (t < -127.f ? -127.f : t));
      }
      store_codes<E>(a.codes_out + e0, valid[u], q);
      if (lane == 0) a.scales_out[c] = m / 127.f;
    }
  }
}

template <int OP, int DT>
hipError_t launch_op(const CodecArgs& a, int chunk, hipStream_t stream) {
  const long long nchunks = (a.n + chunk - 1) / chunk;
  constexpr int U = chunks_per_wave<OP>();
  const long long want = (nchunks + 4 * U - 1) / (4 * U);
  const unsigned blocks = (unsigned)(want < max_blocks<OP>() ? want : max_blocks<OP>());
  if (blocks == 0) return hipSuccess;
  if (chunk == 256)
    hipLaunchKernelGGL((codec_kernel<OP, DT, 4>), dim3(blocks), dim3(256), 0, stream, a);
  else if (chunk == 512)
    hipLaunchKernelGGL((codec_kernel<OP, DT, 8>), dim3(blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((codec_kernel<OP, DT, 16>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int OP>
hipError_t launch_dt(const CodecArgs& a, int chunk, int dtype, hipStream_t stream) {
  return dtype == kF16 ? launch_op<OP, kF16>(a, chunk, stream) : launch_op<OP, kBF16>(a, chunk, stream);
}

}  // namespace

hipError_t launch_codec(const CodecArgs& a, int op, int chunk, int dtype, hipStream_t stream) {
  if (op == kCodecQuantize) return launch_dt<kCodecQuantize>(a, chunk, dtype, stream);
  if (op == kCodecDequantize) return launch_dt<kCodecDequantize>(a, chunk, dtype, stream);
  return launch_dt<kCodecReduce>(a, chunk, dtype, stream);
}

}  // namespace zl
