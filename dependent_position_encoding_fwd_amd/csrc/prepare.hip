// Per-block UT transform for PaTH attention in fp32: products on the fp32
// matrix cores, the triangular solve on the vector ALUs.
//
// [PaTH Attention summary (gist.science 2505.16381), §3 "Representação de
// Transformação UT"]: the product of the transitions of one block,
// H_0 H_1 ... H_63 with H_s = I - beta_s w_s w_s^T, equals I - W^T T^{-1} W
// where W stacks the w_s and T is upper triangular,
//     T = diag(1/beta) + strict_upper(W W^T).
// T^{-1} is formed without dividing by beta (beta = 0 must give H = I): the
// unit upper triangular M = (I + diag(beta) strict_upper(W W^T))^{-1} by back
// substitution, and T^{-1} = M diag(beta).  M itself is an output too (the
// backward's in-block gradients use it).
// [§3 "Algoritmo Estilo FlashAttention"]: the boundary-adjusted query of local
// row r carries the block's transitions up to r, and the adjusted key of row c
// the transitions after c:
//     qhat_r = H_0 ... H_r q_r       = q_r - W^T T^{-1} (W q_r masked to s <= r)
//     khat_c = (H_{c+1}...H_63)^T k_c = k_c - W^T T^{-T} (W k_c masked to s > c)
// These use that a contiguous principal block of the inverse of a triangular
// matrix is the inverse of the same block of the matrix.  The block's
// transition is also produced in row-update form, pT = P^T = I - W^T T^{-T} W.
#include "common.h"
#include "launch.h"
#include "tile_f32.h"

namespace path {
namespace {

// Position p of a row holds reduction index unperm32(p): index k = 32c + 16h +
// 4g + r sits at 32c + 8g + 4h + r, the order in which the 16-bit backward's
// matrix-core operands take a 32-wide slice.
__device__ constexpr int unperm32(int p) {
  return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}

// Writes a 64 x 64 fp32 matrix held in LDS (pitch 65) as split bf16 rows,
// hi = bf16(x) then lo = bf16(x - hi), the columns in unperm32 order:
// out[row][p] = src(row, unperm32(p)).
typedef float pk_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 pk_b2 __attribute__((ext_vector_type(2)));

template <typename F>
__device__ __forceinline__ void pack_split(const F& src, uint16_t* __restrict__ out) {
  constexpr int N = kBlk;
  for (int grp = threadIdx.x; grp < N * N / 4; grp += blockDim.x) {
    const int row = grp / (N / 4), pos = 4 * (grp % (N / 4));
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const pk_f2 x = {src(row, unperm32(pos + 2 * h)), src(row, unperm32(pos + 2 * h + 1))};
      const pk_b2 xh = __builtin_convertvector(x, pk_b2);  // round to nearest even
      const pk_f2 r = x - pk_f2{static_cast<float>(xh[0]), static_cast<float>(xh[1])};
      hi[h] = __builtin_bit_cast(uint32_t, xh);
      lo[h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, pk_b2));
    }
    *reinterpret_cast<uint2*>(out + row * N + pos) = make_uint2(hi[0], hi[1]);
    *reinterpret_cast<uint2*>(out + N * N + row * N + pos) = make_uint2(lo[0], lo[1]);
  }
}

}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(256) void prepare_f32_kernel(
    int64_t L, int Nb, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ w, const float* __restrict__ beta, float* __restrict__ tinv_out,
    float* __restrict__ minv_out, float* __restrict__ qhat_out, float* __restrict__ khat_out,
    float* __restrict__ pT_out, uint16_t* __restrict__ packed_out) {
  constexpr int C = kBlk;
  constexpr int CP = C + 1;
  constexpr int DP = D + 1;
  __shared__ float Ws[C][DP];  // rows w_s of the block (zero past L)
  __shared__ float Xs[C][DP];  // k rows, then q rows, then F = T^{-T} W
  __shared__ float Gs[C][CP];  // strict_upper(W W^T), then masked W k / W q products, then Y
  __shared__ float Ts[C][CP];  // M (T^{-1} = M diag(beta))
  __shared__ float bs[C];      // (67 KB at d = 64: two workgroups per CU)

  const int tid = threadIdx.x;
  const int n = blockIdx.x % Nb;
  const int64_t bh = blockIdx.x / Nb;
  const int64_t t0 = static_cast<int64_t>(n) * C;
  const int valid = static_cast<int>(L - t0 < C ? L - t0 : C);
  const int64_t base = bh * L * D;

  for (int idx = tid; idx < C * D; idx += 256) {
    int r = idx / D, e = idx % D;
    Ws[r][e] = r < valid ? load_f32(w + base + (t0 + r) * D + e) : 0.f;
  }
  if (tid < C) bs[tid] = tid < valid ? beta[bh * L + t0 + tid] : 0.f;
  __syncthreads();

  using f32tile::Acc;
  using f32tile::tile_acc;
  using f32tile::tile_emit;
  using f32tile::tile_mm;
  using f32tile::tile_zero;
  // Y = Z M, written over Z in Gs once every wave has read Z
  const auto gs_times = [&](const auto& b) {
    Acc<C, C> acc;
    tile_zero<C, C>(acc);
    tile_acc<C, C, C>([&](int r, int t) { return Gs[r][t]; }, b, acc);
    __syncthreads();
    tile_emit<C, C>(acc, [&](int r, int a, float x) { Gs[r][a] = x; });
  };
  // G = strict_upper(W W^T)
  tile_mm<C, C, D>([&](int r, int e) { return Ws[r][e]; }, [&](int e, int t) { return Ws[t][e]; },
                   [&](int r, int t, float x) { Gs[r][t] = t > r ? x : 0.f; });
  __syncthreads();

  // Back substitution, last row first:
  // M[r][c] = delta_rc - beta_r * sum_{r<t<=c} G[r][t] M[t][c].
  // Four lanes (a quad of one wave) per column c: lane qq sums the terms
  // t = qq (mod 4) and the quad adds its four partial sums; the lane that owns
  // t = r writes M[r][c], so each lane reads back only its own writes.
  {
    const int c = tid >> 2, qq = tid & 3;
    for (int r = C - 1; r >= 0; --r) {
      float acc = 0.f;
      for (int t = r + 1 + ((qq - r - 1) & 3); t <= c; t += 4) acc += Gs[r][t] * Ts[t][c];
      acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xF, 0xF, false));
      acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xF, 0xF, false));
      if ((r & 3) == qq) Ts[r][c] = r <= c ? (r == c ? 1.f : 0.f) - bs[r] * acc : 0.f;
    }
  }
  __syncthreads();

  if (tinv_out) {
    float* dst = tinv_out + (bh * Nb + n) * (C * C);
    for (int idx = tid; idx < C * C; idx += 256) dst[idx] = Ts[idx / C][idx % C] * bs[idx % C];
  }
  if (minv_out) {
    float* dst = minv_out + (bh * Nb + n) * (C * C);
    for (int idx = tid; idx < C * C; idx += 256) dst[idx] = Ts[idx / C][idx % C];
  }

  // packed_out (d = 64 only): instead of khat_out and pT_out, each block's
  // Khat and P_n as split bf16 rows for the 16-bit backward, eight 64 x 64
  // matrices: Khat rows j (columns e), Khat^T rows a (columns j), P_n rows a
  // (columns b), P_n^T rows a (columns b), each hi then lo, columns in
  // unperm32 order.
  uint16_t* const pk = (D == kBlk && packed_out) ? packed_out + (bh * Nb + n) * int64_t(8 * C * C) : nullptr;

  if (khat_out || pk) {
    for (int idx = tid; idx < C * D; idx += 256) {
      int r = idx / D, e = idx % D;
      Xs[r][e] = r < valid ? load_f32(k + base + (t0 + r) * D + e) : 0.f;
    }
    __syncthreads();
    // Z[c][s] = (w_s . k_c) for s > c, else 0
    tile_mm<C, C, D>([&](int c, int e) { return Xs[c][e]; }, [&](int e, int s2) { return Ws[s2][e]; },
                     [&](int c, int s2, float x) { Gs[c][s2] = s2 > c ? x : 0.f; });
    __syncthreads();
    // Y = Z T^{-1}: Y[c][a] = sum_{c<s<=a} Z[c][s] T^{-1}[s][a] (= (T^{-T} z_c)_a; both factors
    // vanish outside that range, so the full product is the same sum), into Gs
    gs_times([&](int s2, int a) { return Ts[s2][a] * bs[a]; });
    __syncthreads();
    // khat = K - Y W  (Y[c][a] = 0 for a <= c)
    tile_mm<C, D, C>([&](int c, int a) { return Gs[c][a]; }, [&](int a, int e) { return Ws[a][e]; },
                     [&](int c, int e, float x) {
                       if (pk) {
                         Xs[c][e] -= x;  // each element read and written by one lane
                       } else if (c < valid) {
                         khat_out[base + (t0 + c) * D + e] = Xs[c][e] - x;
                       }
                     });
    __syncthreads();
    if constexpr (D == kBlk) {
      if (pk) {
        pack_split([&](int j, int e) { return Xs[j][e]; }, pk);
        pack_split([&](int a, int j) { return Xs[j][a]; }, pk + 2 * C * C);
        __syncthreads();
      }
    }
  }

  if (qhat_out) {
    for (int idx = tid; idx < C * D; idx += 256) {
      int r = idx / D, e = idx % D;
      Xs[r][e] = r < valid ? load_f32(q + base + (t0 + r) * D + e) : 0.f;
    }
    __syncthreads();
    // A[r][t] = (w_t . q_r) for t <= r, else 0
    tile_mm<C, C, D>([&](int r, int e) { return Xs[r][e]; }, [&](int e, int t) { return Ws[t][e]; },
                     [&](int r, int t, float x) { Gs[r][t] = t <= r ? x : 0.f; });
    __syncthreads();
    // Y = A T^{-T}: Y[r][a] = sum_{a<=t<=r} T^{-1}[a][t] A[r][t] (= (T^{-1} a_r)_a, 0 for a > r), into Gs
    gs_times([&](int t, int a) { return Ts[a][t] * bs[t]; });
    __syncthreads();
    // qhat = Q - Y W
    tile_mm<C, D, C>([&](int r, int a) { return Gs[r][a]; }, [&](int a, int e) { return Ws[a][e]; },
                     [&](int r, int e, float x) {
                       if (r < valid) qhat_out[base + (t0 + r) * D + e] = Xs[r][e] - x;
                     });
    __syncthreads();
  }

  if (pT_out || pk) {
    // F = T^{-T} W: F[s][e] = sum_{t<=s} T^{-1}[t][s] W[t][e]
    tile_mm<C, D, C>([&](int s2, int t) { return Ts[t][s2] * bs[s2]; }, [&](int t, int e) { return Ws[t][e]; },
                     [&](int s2, int e, float x) { Xs[s2][e] = x; });
    __syncthreads();
    // P^T = I - W^T F (into Gs for packing: Y's last reader passed the barrier above)
    float* dst = pT_out ? pT_out + (bh * Nb + n) * (static_cast<int64_t>(D) * D) : nullptr;
    tile_mm<D, D, C>([&](int a, int s2) { return Ws[s2][a]; }, [&](int s2, int b) { return Xs[s2][b]; },
                     [&](int a, int b, float x) {
                       const float v = (a == b ? 1.f : 0.f) - x;
                       if (pk) {
                         Gs[a][b] = v;
                       } else {
                         dst[a * D + b] = v;
                       }
                     });
    if constexpr (D == kBlk) {
      if (pk) {
        __syncthreads();
        pack_split([&](int a, int b) { return Gs[b][a]; }, pk + 4 * C * C);  // P_n[a][b] = P^T[b][a]
        pack_split([&](int a, int b) { return Gs[a][b]; }, pk + 6 * C * C);
      }
    }
  }
}

// One workgroup per (b,h): fp64 prefix sum of log forget gates.
__global__ __launch_bounds__(256) void prefix_sum_kernel(int64_t L, const float* __restrict__ x,
                                                         float* __restrict__ c) {
  __shared__ double part[256];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t per = (L + 255) / 256;
  const int64_t lo = tid * per;
  const int64_t hi = lo + per < L ? lo + per : L;
  const float* xs = x + bh * L;
  double acc = 0.0;
  for (int64_t i = lo; i < hi; ++i) acc += static_cast<double>(xs[i]);
  part[tid] = acc;
  __syncthreads();
  if (tid == 0) {
    double run = 0.0;
    for (int t = 0; t < 256; ++t) {
      double v = part[t];
      part[t] = run;
      run += v;
    }
  }
  __syncthreads();
  double run = part[tid];
  float* cs = c + bh * L;
  for (int64_t i = lo; i < hi; ++i) {
    run += static_cast<double>(xs[i]);
    cs[i] = static_cast<float>(run);
  }
}

// One workgroup per (b,h): the fp64-accumulated prefix sum of log f times
// `mult`, padded to Nb*64 entries by repeating the last value.  Each thread
// sums a contiguous run of the gates, the runs' totals are scanned in order,
// and each thread then writes its run from its starting total.
__global__ __launch_bounds__(256) void cum_padded_kernel(int64_t L, int Nb, const float* __restrict__ x,
                                                         float mult, float* __restrict__ c) {
  __shared__ double part[256];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t Lp = static_cast<int64_t>(Nb) * kBlk;
  const int64_t per = (L + 255) / 256;
  const int64_t lo = tid * per;
  const int64_t hi = lo + per < L ? lo + per : L;
  double acc = 0.0;
  for (int64_t i = lo; i < hi; ++i) acc += static_cast<double>(x[bh * L + i]);
  part[tid] = acc;
  __syncthreads();
  if (tid == 0) {
    double run = 0.0;
    for (int t = 0; t < 256; ++t) {
      double v = part[t];
      part[t] = run;
      run += v;
    }
  }
  __syncthreads();
  double run = part[tid];
  float* cs = c + bh * Lp;
  for (int64_t i = lo; i < hi; ++i) {
    run += static_cast<double>(x[bh * L + i]);
    cs[i] = static_cast<float>(run * mult);
  }
  __syncthreads();
  const float last = cs[L - 1];
  for (int64_t i = L + tid; i < Lp; i += 256) cs[i] = last;
}

hipError_t launch_cum_padded(int64_t BH, int64_t L, const float* log_forget, float mult, float* cum,
                             hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  hipLaunchKernelGGL(cum_padded_kernel, dim3(static_cast<unsigned>(BH)), dim3(256), 0, stream, L, Nb,
                     log_forget, mult, cum);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_prepare_t(int64_t B, int64_t H, int64_t L, const void* q, const void* k,
                                   const void* w, const float* beta, float* tinv, float* minv, float* qhat,
                                   float* khat, float* pT, uint16_t* packed, hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  dim3 grid(static_cast<unsigned>(B * H * Nb));
  hipLaunchKernelGGL((prepare_f32_kernel<T, D>), grid, dim3(256), 0, stream, L, Nb,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(w),
                     beta, tinv, minv, qhat, khat, pT, packed);
  return hipGetLastError();
}

hipError_t launch_prepare_f32(int dtype, int64_t B, int64_t H, int64_t L, int64_t d,
                              const void* q, const void* k, const void* w, const float* beta,
                              float* tinv, float* minv, float* qhat, float* khat, float* pT, void* packed,
                              hipStream_t stream) {
  uint16_t* pk = static_cast<uint16_t*>(packed);
  if (dtype == 0) {
    return d == 64 ? launch_prepare_t<float, 64>(B, H, L, q, k, w, beta, tinv, minv, qhat, khat, pT, pk, stream)
                   : launch_prepare_t<float, 128>(B, H, L, q, k, w, beta, tinv, minv, qhat, khat, pT, pk, stream);
  }
  return d == 64 ? launch_prepare_t<bf16_t, 64>(B, H, L, q, k, w, beta, tinv, minv, qhat, khat, pT, pk, stream)
                 : launch_prepare_t<bf16_t, 128>(B, H, L, q, k, w, beta, tinv, minv, qhat, khat, pT, pk, stream);
}

hipError_t launch_prefix_sum(int64_t BH, int64_t L, const float* x, float* c, hipStream_t stream) {
  hipLaunchKernelGGL(prefix_sum_kernel, dim3(static_cast<unsigned>(BH)), dim3(256), 0, stream, L, x, c);
  return hipGetLastError();
}

}  // namespace path
