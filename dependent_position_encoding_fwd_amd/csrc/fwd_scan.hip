// Right-to-left block scan forward of PaTH attention, fp32 on the vector ALUs.
//
// [PaTH Attention summary (gist.science 2505.16381), §2 "Mecanismo Central"]
//     s_ij = scale * k_j^T (H_{j+1} ... H_i) q_i (+ FoX bias), softmax over j <= i.
// [§3 "Algoritmo Estilo FlashAttention"] One workgroup owns one 64-query block
// m.  Each thread carries its query's transported vector u.  Inside block m it
// walks keys c = r, r-1, ..., 0 applying one H at a time, which leaves
// u = qhat_r (the boundary-adjusted query).  It then scans the key blocks
// n = m-1, ..., 0 right to left: logits against the adjusted keys khat_n,
// an online softmax step, and u <- P_n u through the block transition P_n^T.
// [§2 "Extensões: PaTH-FoX"] bias = cum_i - cum_j with cum the prefix sum of
// log f.  Every thread works on its own LDS rows, so no barriers are needed.
//
// This kernel is the fp32 path (fp32 inputs) and a readable baseline; the
// bf16 path runs on the matrix cores.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace path {

template <typename T, int D, bool FOX>
__global__ __launch_bounds__(64) void fwd_scan_f32_kernel(
    int64_t L, int Nb, float scale, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ w, const float* __restrict__ beta,
    const float* __restrict__ cum, const float* __restrict__ khat, const float* __restrict__ pT,
    T* __restrict__ o, float* __restrict__ lse) {
  constexpr int C = kBlk;
  constexpr int DP = D + 1;
  __shared__ float U[C][DP];
  __shared__ float U2[C][DP];
  __shared__ float Os[C][DP];
  __shared__ float S[C][C + 1];

  const int m = Nb - 1 - static_cast<int>(blockIdx.x % Nb);  // longest rows first
  const int64_t bh = blockIdx.x / Nb;
  const int r = threadIdx.x;
  const int64_t i = static_cast<int64_t>(m) * C + r;
  if (i >= L) return;  // no barriers below: idle rows may leave

  const int64_t base = bh * L * D;
  float* u = U[r];
  float* u2 = U2[r];
  float* acc = Os[r];
  float* srow = S[r];
  for (int e = 0; e < D; ++e) {
    u[e] = load_f32(q + base + i * D + e);
    acc[e] = 0.f;
  }
  const float ci = FOX ? cum[bh * L + i] : 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  auto accumulate = [&](int n, int cnt) {
    float mb = -INFINITY;
    for (int c = 0; c < cnt; ++c) mb = fmaxf(mb, srow[c]);
    const float mnew = fmaxf(mrun, mb);
    const float alpha = expf(mrun - mnew);
    lrun *= alpha;
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
    for (int c = 0; c < cnt; ++c) {
      const float p = expf(srow[c] - mnew);
      lrun += p;
      const T* vc = v + base + (static_cast<int64_t>(n) * C + c) * D;
      for (int e = 0; e < D; ++e) acc[e] += p * load_f32(vc + e);
    }
    mrun = mnew;
  };

  // Diagonal block: keys c = r .. 0, one transition at a time.
  for (int c = r; c >= 0; --c) {
    const int64_t j = static_cast<int64_t>(m) * C + c;
    const T* kj = k + base + j * D;
    const T* wj = w + base + j * D;
    float s = 0.f, a = 0.f;
    for (int e = 0; e < D; ++e) {
      s += load_f32(kj + e) * u[e];
      a += load_f32(wj + e) * u[e];
    }
    srow[c] = scale * s + (FOX ? ci - cum[bh * L + j] : 0.f);
    a *= beta[bh * L + j];
    for (int e = 0; e < D; ++e) u[e] -= a * load_f32(wj + e);
  }
  accumulate(m, r + 1);

  // Off-diagonal key blocks, right to left.
  for (int n = m - 1; n >= 0; --n) {
    for (int c = 0; c < C; ++c) {
      const int64_t j = static_cast<int64_t>(n) * C + c;
      const float* kj = khat + base + j * D;
      float s = 0.f;
      for (int e = 0; e < D; ++e) s += kj[e] * u[e];
      srow[c] = scale * s + (FOX ? ci - cum[bh * L + j] : 0.f);
    }
    accumulate(n, C);
    if (n > 0) {
      const float* P = pT + (bh * Nb + n) * static_cast<int64_t>(D) * D;
      for (int b = 0; b < D; ++b) u2[b] = 0.f;
      for (int a = 0; a < D; ++a) {
        const float ua = u[a];
        for (int b = 0; b < D; ++b) u2[b] += ua * P[a * D + b];
      }
      for (int b = 0; b < D; ++b) u[b] = u2[b];
    }
  }

  const float inv = 1.f / lrun;
  for (int e = 0; e < D; ++e) store_f32(o + base + i * D + e, acc[e] * inv);
  lse[bh * L + i] = mrun + logf(lrun);
}

template <typename T, int D>
static hipError_t launch_t(int64_t B, int64_t H, int64_t L, float scale, const void* q,
                           const void* k, const void* v, const void* w, const float* beta,
                           const float* cum, const float* khat, const float* pT, void* o,
                           float* lse, hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  dim3 grid(static_cast<unsigned>(B * H * Nb));
  if (cum) {
    hipLaunchKernelGGL((fwd_scan_f32_kernel<T, D, true>), grid, dim3(64), 0, stream, L, Nb, scale,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       static_cast<const T*>(w), beta, cum, khat, pT, static_cast<T*>(o), lse);
  } else {
    hipLaunchKernelGGL((fwd_scan_f32_kernel<T, D, false>), grid, dim3(64), 0, stream, L, Nb, scale,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       static_cast<const T*>(w), beta, cum, khat, pT, static_cast<T*>(o), lse);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_scan_f32(int dtype, int64_t B, int64_t H, int64_t L, int64_t d, float scale,
                               const void* q, const void* k, const void* v, const void* w,
                               const float* beta, const float* cum, const float* khat,
                               const float* pT, void* o, float* lse, hipStream_t stream) {
  if (dtype == 0) {
    return d == 64 ? launch_t<float, 64>(B, H, L, scale, q, k, v, w, beta, cum, khat, pT, o, lse, stream)
                   : launch_t<float, 128>(B, H, L, scale, q, k, v, w, beta, cum, khat, pT, o, lse, stream);
  }
  return d == 64 ? launch_t<bf16_t, 64>(B, H, L, scale, q, k, v, w, beta, cum, khat, pT, o, lse, stream)
                 : launch_t<bf16_t, 128>(B, H, L, scale, q, k, v, w, beta, cum, khat, pT, o, lse, stream);
}

}  // namespace path
