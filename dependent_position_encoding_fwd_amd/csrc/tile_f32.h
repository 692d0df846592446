// Tile products on the fp32 matrix cores (16x16x4 MFMA, fp32 in and out) for
// workgroups whose first four waves compute them: the shared building block of
// the fp32 kernels (block prepare, backward).
#pragma once

#include <hip/hip_runtime.h>

namespace path {
namespace f32tile {

typedef float f4 __attribute__((ext_vector_type(4)));

// For an M x N product, wave wv owns the 16-row tiles wv, wv + 4, ... and every
// 16-column tile: acc[r][c] is rows 16 (wv + 4 r) .., columns 16 c ...  In one
// MFMA lane l supplies A[l % 16][k] and B[k][l % 16] with k = l / 16 and holds
// D[4 (l / 16) + i][l % 16] in element i.  The reduction index is visited in
// chunks of 16, lane group g taking k = 16 c + 4 g + j in MFMA j of chunk c, so
// each lane reads 4 consecutive k of its row.  a(m, k) and b(k, n) are read
// through accessors; emit(m, n, value) receives each output element once.
template <int M, int N>
using Acc = f4[M / 64][N / 16];

template <int M, int N, int K, typename FA, typename FB>
__device__ __forceinline__ void tile_acc(const FA& a, const FB& b, Acc<M, N>& acc) {
  static_assert(M % 64 == 0 && N % 16 == 0 && K % 16 == 0, "tile shape");
  constexpr int R = M / 64, NC = N / 16;
  const int wv = threadIdx.x >> 6, lr = threadIdx.x & 15, lk = (threadIdx.x >> 4) & 3;
#pragma unroll 2
  for (int c = 0; c < K / 16; ++c) {
    float av[4][R], bv[4][NC];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = 16 * c + 4 * lk + j;
#pragma unroll
      for (int r = 0; r < R; ++r) av[j][r] = a(16 * (wv + 4 * r) + lr, kk);
#pragma unroll
      for (int n = 0; n < NC; ++n) bv[j][n] = b(kk, 16 * n + lr);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int n = 0; n < NC; ++n)
          acc[r][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j][r], bv[j][n], acc[r][n], 0, 0, 0);
  }
}

template <int M, int N>
__device__ __forceinline__ void tile_zero(Acc<M, N>& acc) {
#pragma unroll
  for (int r = 0; r < M / 64; ++r)
#pragma unroll
    for (int n = 0; n < N / 16; ++n) acc[r][n] = f4{0.f, 0.f, 0.f, 0.f};
}

template <int M, int N, typename FE>
__device__ __forceinline__ void tile_emit(const Acc<M, N>& acc, const FE& emit) {
  const int wv = threadIdx.x >> 6, lr = threadIdx.x & 15, lk = (threadIdx.x >> 4) & 3;
#pragma unroll
  for (int r = 0; r < M / 64; ++r)
#pragma unroll
    for (int n = 0; n < N / 16; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) emit(16 * (wv + 4 * r) + 4 * lk + i, 16 * n + lr, acc[r][n][i]);
}

template <int M, int N, int K, typename FA, typename FB, typename FE>
__device__ __forceinline__ void tile_mm(const FA& a, const FB& b, const FE& emit) {
  Acc<M, N> acc;
  tile_zero<M, N>(acc);
  tile_acc<M, N, K>(a, b, acc);
  tile_emit<M, N>(acc, emit);
}

}  // namespace f32tile
}  // namespace path
