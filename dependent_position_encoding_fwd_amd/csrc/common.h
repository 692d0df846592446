// Shared device helpers for the gfx950 PaTH kernels: storage-type loads and
// stores, bf16 rounding, wave reductions and the block geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace path {

// Tokens per UT block.  The pages fix no block size; 64 matches the wave width
// and the MFMA tiles (results do not depend on it).
constexpr int kBlk = 64;

// Start of query row r of a block's in-block logits (padded lower triangle of
// kDiagTri floats, see launch.h).
__host__ __device__ constexpr int diag_row(int r) {
  return 8 * (r >> 2) * ((r >> 2) + 1) + 4 * (r & 3) * ((r >> 2) + 1);
}
static_assert(diag_row(kBlk - 1) + kBlk == kDiagTri, "padded triangle size");

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(p->bits);
}

template <typename T>
__device__ __forceinline__ void store_f32(T* p, float x);
template <>
__device__ __forceinline__ void store_f32<float>(float* p, float x) {
  *p = x;
}
template <>
__device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, float x) {
  p->bits = f32_to_bf16(x);
}

// Sum over the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

}  // namespace path
