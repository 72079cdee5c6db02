// Shared device helpers for the gfx950 kernels: element types, conversions,
// vector loads/stores and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llama {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
// float -> bfloat16 with round-to-nearest-even (the IEEE conversion rule).
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }

// 4 consecutive elements <-> float4
__device__ __forceinline__ f32x4 load4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  bf16x4 v = *(const bf16x4*)p;
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *(bf16x4*)p = o;
}
// 8 consecutive values (lo, hi) as one 16-byte store; p 16-byte aligned
__device__ __forceinline__ void store8(bf16* p, f32x4 lo, f32x4 hi) {
  bf16x8 o = {(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3], (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
  *(bf16x8*)p = o;
}
__device__ __forceinline__ bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// 16-byte load with the non-temporal hint, for data read exactly once (weights
// streamed by the one-token projections, the KV rows of a decode step): it does
// not displace reusable lines in L2 / MALL, and streams measured faster with it.
__device__ __forceinline__ bf16x8 load_stream8(const bf16* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)p));
}

// Sum over the 64 lanes of a wavefront (every lane receives the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Reductions over lane pairs (l, l ^ 16) and (l, l ^ 32) with the gfx950 lane
// swaps: each returns op(v[l], v[l ^ off]) on every lane, from VALU
// instructions instead of an LDS permute.  A swap of v with itself leaves, in
// its two results, v[l] and v[l ^ off] (in an order that depends on the lane),
// and both ops are symmetric, so every lane of a pair gets the same value.
// Lane rows (16 lanes each) 0/1 and 2/3 trade halves of two 4-vectors: a lane
// of row r gets, as lo and hi, the values of rows r & ~1 and r | 1 of x (r even)
// or of y (r odd).  With x, y holding 4 consecutive columns per lane row of two
// 16-column tiles (row r: columns 4r..4r+3), lo/hi become 8 consecutive columns:
// row 0 tile x columns 0-7, row 1 tile y 0-7, row 2 tile x 8-15, row 3 tile y 8-15.
__device__ __forceinline__ void pair_transpose16(const f32x4& x, const f32x4& y, f32x4& lo, f32x4& hi) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[v]), __float_as_uint(y[v]), false, false);
    lo[v] = __uint_as_float(r[0]);
    hi[v] = __uint_as_float(r[1]);
  }
}
__device__ __forceinline__ float pair_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup id remapping so that consecutive logical tiles land on the same
// XCD (the dispatcher deals workgroups round-robin over the 8 XCDs, each with
// its own L2).  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  if (nblocks % 8) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

}  // namespace llama
