// Matrix-core helpers shared by the gfx950 scan kernels: 16-bit vector types,
// the 16x16x32 MFMA, fp32 -> fp16 packing (with the lo part of an fp16 hi/lo
// split) and reductions over the four 16-lane groups of a wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace path {
namespace mfma {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f4 mma16(const h8& a, const h8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mmb16(const b8& a, const b8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

union H8 {
  h8 v;
  h2 p[4];
};
union B8 {
  b8 v;
  b2 p[4];
  uint4 u;
};

__device__ __forceinline__ h8 pack_h8(const f4& x, const f4& y) {
  H8 r;
  r.p[0] = __builtin_convertvector(f2{x[0], x[1]}, h2);
  r.p[1] = __builtin_convertvector(f2{x[2], x[3]}, h2);
  r.p[2] = __builtin_convertvector(f2{y[0], y[1]}, h2);
  r.p[3] = __builtin_convertvector(f2{y[2], y[3]}, h2);
  return r.v;
}
__device__ __forceinline__ h8 pack_lo(const f4& x, const f4& y, const h8& hi) {
  f4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = x[i] - static_cast<float>(hi[i]);
    b[i] = y[i] - static_cast<float>(hi[4 + i]);
  }
  return pack_h8(a, b);
}
__device__ __forceinline__ b8 pack_b8(const f4& x, const f4& y) {
  B8 r;
  r.p[0] = __builtin_convertvector(f2{x[0], x[1]}, b2);
  r.p[1] = __builtin_convertvector(f2{x[2], x[3]}, b2);
  r.p[2] = __builtin_convertvector(f2{y[0], y[1]}, b2);
  r.p[3] = __builtin_convertvector(f2{y[2], y[3]}, b2);
  return r.v;
}

// Reductions over the 4 lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float grp_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float grp_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Direct-to-LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at lds + 16 l.  Issued from asm: the compiler's wait insertion
// treats an LDS DMA it can see as unordered with LDS reads and then waits for
// every outstanding LDS read at each use (lgkmcnt(0)) until the DMA is waited
// for.  Here the caller waits for the data (s_waitcnt vmcnt(0), then a
// barrier) before any wave reads them, and compiler-counted waits on its own
// loads stay safe because they only ever over-wait.
__device__ __forceinline__ void lds_dma16(const void* g, const void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(base) : "memory");
}

// Max over the 64 lanes of a wave with no address registers: the four lane
// groups through the lane swaps above, then the 16 lanes of a row through DPP
// moves (neighbours within a quad, then the half-row and row mirrors).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = grp_max(x);
  x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp_mov<0x140>(x));  // row_mirror
}

}  // namespace mfma
}  // namespace path
