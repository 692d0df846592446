// Projection prologue of PaTH attention on the bf16 matrix cores.
//
// [PaTH Attention summary (gist.science 2505.16381), §2 "Mecanismo Central"]:
// the transition vector w_s and the factor beta_s are functions of the input
// token x_s, with beta_s = 2 sigmoid(u^T x_s + b).  The pages give no formula
// for w_s; here it is a per-head linear map scaled to unit length,
//     w_s = W_h x_s / max(|W_h x_s|, 1e-12),
// and [§6 "Limitações"]'s clipping of beta is an optional upper bound.
//
// One GEMM over all heads: tokens x [T, Dm] (T = B L, bf16) against the rows
// of Ww [H d, Dm] (head h owns rows h d .. h d + d - 1) and of u [H, Dm].  A
// workgroup takes 128 tokens and one group of 128 columns: either the rows of
// 128 / d whole heads (so each head's vector w_s is in the tile and is
// normalised in the epilogue) or the u rows of 128 consecutive heads (their
// beta logits).
// Products are 16x16x32 bf16 MFMAs with fp32 accumulation; the reduction over
// Dm runs in chunks of 64 through two LDS stages, fed from registers that hold
// the next 3 chunks' global loads.
// Workgroup ids are dealt to the 8 XCDs round robin; all column groups of a
// token tile are given ids on one XCD, so its L2 fetches the tile once.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "mfma_util.h"

namespace path {

namespace {

constexpr int kPT = 256;     // threads: four waves
constexpr int kPM = 128;     // tokens per workgroup (32 per wave)
constexpr int kPK = 64;      // reduction chunk
constexpr int kPKP = kPK + 8;  // LDS row pitch (bf16 elements): 144 bytes, spreads the 16-byte reads
constexpr int kPN = 128;     // columns per workgroup

using mfma::b8;
using mfma::f4;

template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over a row of 16 lanes, the same bits in every lane of the row.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_row<0xB1>(x);
  x += dpp_row<0x4E>(x);
  x += dpp_row<0x141>(x);
  x += dpp_row<0x140>(x);
  return x;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kPT, 2) void project_kernel(
    int64_t T, int64_t L, int64_t H, int64_t Dm, int ntiles, int ncol, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ Ww, const uint16_t* __restrict__ u, const float* __restrict__ bias,
    float beta_max, uint16_t* __restrict__ w_out, float* __restrict__ beta_out) {
  constexpr int NC = kPN / 16;         // column tiles
  constexpr int HT = D / 16;           // column tiles per head
  constexpr int P = 3;                 // chunks of global loads in flight
  constexpr int BL = kPN * kPK / 8 / kPT;  // 16-byte weight loads per thread per chunk
  constexpr int AL = kPM * kPK / 8 / kPT;  // 16-byte token loads per thread per chunk
  __shared__ __align__(16) uint16_t As[2][kPM][kPKP];
  __shared__ __align__(16) uint16_t Bs[2][kPN][kPKP];

  // XCD-aware map: ids i, i + 8, i + 16, ... run on one XCD; consecutive ids of
  // that stream walk the column groups of one token tile.
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int col = j % ncol;
  const int tile = (j / ncol) * 8 + xcd;
  if (tile >= ntiles) return;  // whole workgroup: no barrier reached
  const int64_t t0 = static_cast<int64_t>(tile) * kPM;
  const int64_t nwg = (H * D + kPN - 1) / kPN;  // column groups of w
  const bool beta_group = col >= nwg;
  const int64_t r0 = (beta_group ? col - nwg : col) * static_cast<int64_t>(kPN);
  const int64_t nrows = beta_group ? H : H * D;  // rows of the matrix this group reads
  const uint16_t* Wm = beta_group ? u : Ww;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  uint4 ra[P][AL], rb[P][BL];  // chunk c is held in set c % P
  const int nchunks = static_cast<int>(Dm / kPK);
  auto gload = [&](int c, uint4 (&a)[AL], uint4 (&b)[BL]) {
#pragma unroll
    for (int p = 0; p < AL; ++p) {
      const int idx = tid + kPT * p;
      const int row = idx >> 3, seg = idx & 7;
      const int64_t t = t0 + row;
      a[p] = make_uint4(0u, 0u, 0u, 0u);
      if (t < T) a[p] = *reinterpret_cast<const uint4*>(x + t * Dm + c * kPK + 8 * seg);
    }
#pragma unroll
    for (int p = 0; p < BL; ++p) {
      const int idx = tid + kPT * p;
      const int row = idx >> 3, seg = idx & 7;
      const int64_t r = r0 + row;
      b[p] = make_uint4(0u, 0u, 0u, 0u);
      if (r < nrows) b[p] = *reinterpret_cast<const uint4*>(Wm + r * Dm + c * kPK + 8 * seg);
    }
  };
  auto lstore = [&](int s, const uint4 (&a)[AL], const uint4 (&b)[BL]) {
#pragma unroll
    for (int p = 0; p < AL; ++p) {
      const int idx = tid + kPT * p;
      *reinterpret_cast<uint4*>(&As[s][idx >> 3][8 * (idx & 7)]) = a[p];
    }
#pragma unroll
    for (int p = 0; p < BL; ++p) {
      const int idx = tid + kPT * p;
      *reinterpret_cast<uint4*>(&Bs[s][idx >> 3][8 * (idx & 7)]) = b[p];
    }
  };

  f4 acc[2][NC];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) acc[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int q = 0; q < P; ++q)
    if (q < nchunks) gload(q, ra[q], rb[q]);
  lstore(0, ra[0], rb[0]);
  __syncthreads();
  for (int c0 = 0; c0 < nchunks; c0 += P) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int c = c0 + q;
      if (c >= nchunks) break;
      const int s = c & 1;
      // set q was written to LDS one step ago: it takes chunk c + P
      if (c + P < nchunks) gload(c + P, ra[q], rb[q]);
#pragma unroll
      for (int ks = 0; ks < kPK / 32; ++ks) {
        // lane (lg, lr): row lr of each 16-row tile, reduction elements 32 ks + 8 lg .. + 7
        b8 af[2], bf[NC];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          af[rt] = *reinterpret_cast<const b8*>(&As[s][32 * wv + 16 * rt + lr][32 * ks + 8 * lg]);
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) bf[ct] = *reinterpret_cast<const b8*>(&Bs[s][16 * ct + lr][32 * ks + 8 * lg]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int ct = 0; ct < NC; ++ct) acc[rt][ct] = mfma::mmb16(af[rt], bf[ct], acc[rt][ct]);
      }
      if (c + 1 < nchunks) lstore(s ^ 1, ra[(q + 1) % P], rb[(q + 1) % P]);
      __syncthreads();
    }
  }

  // Epilogue.  acc[rt][ct][i] is token 32 wv + 16 rt + 4 lg + i, column 16 ct + lr.
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + 32 * wv + 16 * rt + 4 * lg + i;
      const bool live = t < T;
      const int64_t bi = t / L, li = t - bi * L;
      if (!beta_group) {
#pragma unroll
        for (int hh = 0; hh < kPN / D; ++hh) {  // the heads of the group
          float n2 = 0.f;
#pragma unroll
          for (int ct = HT * hh; ct < HT * (hh + 1); ++ct) n2 = fmaf(acc[rt][ct][i], acc[rt][ct][i], n2);
          n2 = sum16(n2);
          const float inv = 1.f / fmaxf(sqrtf(n2), 1e-12f);
          const int64_t h = r0 / D + hh;
          if (live && h < H) {
            uint16_t* dst = w_out + ((bi * H + h) * L + li) * D;
#pragma unroll
            for (int ct = HT * hh; ct < HT * (hh + 1); ++ct)
              dst[16 * (ct - HT * hh) + lr] = f32_to_bf16(acc[rt][ct][i] * inv);
          }
        }
      } else if (live) {
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          const int64_t h = r0 + 16 * ct + lr;
          if (h < H) {
            const float z = acc[rt][ct][i] + bias[h];
            float beta = 2.f / (1.f + expf(-z));
            if (beta_max > 0.f) beta = fminf(beta, beta_max);
            beta_out[(bi * H + h) * L + li] = beta;
          }
        }
      }
    }
  }
}

hipError_t launch_project(int64_t B, int64_t L, int64_t Dm, int64_t H, int64_t d, const void* x, const void* Ww,
                          const void* u, const float* bias, float beta_max, void* w_out, float* beta_out,
                          hipStream_t stream) {
  const int64_t T = B * L;
  const int ntiles = static_cast<int>((T + kPM - 1) / kPM);
  const int ncol = static_cast<int>((H * d + kPN - 1) / kPN + (H + kPN - 1) / kPN);
  const int64_t per_xcd = (ntiles + 7) / 8;
  const dim3 grid(static_cast<unsigned>(8 * per_xcd * ncol));
  const auto* xs = static_cast<const uint16_t*>(x);
  const auto* ws = static_cast<const uint16_t*>(Ww);
  const auto* us = static_cast<const uint16_t*>(u);
  auto* wo = static_cast<uint16_t*>(w_out);
  if (d == 64)
    hipLaunchKernelGGL(project_kernel<64>, grid, dim3(kPT), 0, stream, T, L, H, Dm, ntiles, ncol, xs, ws, us, bias,
                       beta_max, wo, beta_out);
  else
    hipLaunchKernelGGL(project_kernel<128>, grid, dim3(kPT), 0, stream, T, L, H, Dm, ntiles, ncol, xs, ws, us, bias,
                       beta_max, wo, beta_out);
  return hipGetLastError();
}

}  // namespace path
