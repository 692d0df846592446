// Backward pass of PaTH attention: gradients of <dO, o> with respect to q, k,
// v, w, beta and the log forget gates, in fp32 arithmetic: tile products on
// the fp32 matrix cores, Householder chains on the vector ALUs.
//
// The forward [PaTH Attention summary (gist.science 2505.16381), §2 "Mecanismo
// Central", §2 "Extensões: PaTH-FoX"; blockwise as in §3 "Representação de
// Transformação UT" and §3 "Algoritmo Estilo FlashAttention"] gives, for query
// i in block m and key j in block n < m,
//     s_ij = scale * khat_j . Qt_i^(n) + (c_i - c_j),
//     Qt^(m-1) = Qhat_m,   Qt^(n-1) = P_n Qt^(n),   P_n = H_{64n} ... H_{64n+63},
// and inside a block the logit of keys c <= r is scale * k_c . (H_{c+1}...H_r q_r).
// The pages say nothing about training; this file differentiates that forward.
//
// Cross-block part (bwd_pair_kernel for fp32 storage, one workgroup per query
// block m; bwd_pair16.hip splits the same two passes over kernels for bf16):
//   pass 1, right to left: Qt^(n) for n = m-1..0, kept in a scratch buffer;
//   pass 2, left to right: with dS_ij = p_ij (dO_i . v_j - D_i), D_i = dO_i . o_i,
//     the adjoint of the transported queries obeys
//       Lam^(n) = P_n^T Lam^(n-1) + scale Khat_n^T dS_n,   Lam^(-1) = 0,
//     so Lam^(m-1) is the gradient reaching Qhat_m, P_n receives Lam^(n-1) Qt^(n)^T,
//     Khat_n receives scale dS_n Qt^(n)^T and V_n receives p_n dO_m; the last
//     three are summed over query blocks with fp32 atomics.
// In-block part (bwd_block_kernel, one workgroup per block): every Householder
// chain of the block is replayed by 16 lanes of a wave (four chains per wave)
// and then differentiated in reverse:
// query chains x <- H_t x from q_r down to qhat_r (they meet the in-block keys
// on the way), key chains from k_c up to khat_c, and one chain per column of
// P_n.  Running a chain backwards needs its states in the opposite order; each
// state is rebuilt from the next one as x^(t+1) = x^(t) + beta_t a_t w_t, where
// a_t = w_t . x^(t+1) is the one scalar the forward replay keeps per step.  For
// H_t = I - beta_t w_t w_t^T receiving dH_t = sum xbar x^T over its uses,
//     dw_t = -beta_t (dH_t + dH_t^T) w_t,   dbeta_t = -w_t^T dH_t w_t.
// Gate gradient: dc_i = sum_{j<i} dS_ij - sum_{i'>i} dS_i'i, and
// d log f_s = sum_{i>=s} dc_i (fp64 suffix sums).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tile_f32.h"

namespace path {
namespace {

using f32tile::Acc;
using f32tile::f4;
using f32tile::tile_acc;
using f32tile::tile_emit;
using f32tile::tile_mm;
using f32tile::tile_zero;

constexpr int kT = 256;    // threads per workgroup: 4 waves

// DPP lane move within a row of 16 lanes (row_mask and bank_mask full).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// A operands held in registers: af[r][4 c + j] = a(16 (wv + 4 r) + lr, 16 c + 4 lk + j),
// the values lane (lk, lr) of wave wv feeds to the MFMAs of tile_acc.  Only the
// wave's own rows are held, so a fragment can be fetched from global memory
// one iteration ahead of its use.
template <int M, int K>
using Frag = float[M / 64][K / 4];

template <int M, int K, typename FA>
__device__ __forceinline__ void frag_load(const FA& a, Frag<M, K>& af) {
  const int wv = threadIdx.x >> 6, lr = threadIdx.x & 15, lk = (threadIdx.x >> 4) & 3;
#pragma unroll
  for (int r = 0; r < M / 64; ++r)
#pragma unroll
    for (int c = 0; c < K / 16; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) af[r][4 * c + j] = a(16 * (wv + 4 * r) + lr, 16 * c + 4 * lk + j);
}

template <int M, int N, int K, typename FB>
__device__ __forceinline__ void tile_acc_ra(const Frag<M, K>& af, const FB& b, Acc<M, N>& acc) {
  constexpr int R = M / 64, NC = N / 16;
  const int lr = threadIdx.x & 15, lk = (threadIdx.x >> 4) & 3;
#pragma unroll
  for (int c = 0; c < K / 16; ++c) {
    float bv[4][NC];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int n = 0; n < NC; ++n) bv[j][n] = b(16 * c + 4 * lk + j, 16 * n + lr);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int n = 0; n < NC; ++n)
          acc[r][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[r][4 * c + j], bv[j][n], acc[r][n], 0, 0, 0);
  }
}

// Sum over the 16 lanes of a row, the same bits in every lane of the row:
// pairwise sums within quads, 8-lane halves and the row (each step adds two
// partial sums held by two lanes, and addition is commutative).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return x;
}


}  // namespace

// Eight consecutive elements as fp32 (16-byte aligned: one or two vector loads).
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t wd[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(wd[e] << 16);
    x[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
  }
}

// D_i = dO_i . o_i: D/8 consecutive lanes per row, 8 elements each (one
// 16- or 32-byte load per operand), summed across the lanes by shuffles.
template <typename T, int D>
__global__ __launch_bounds__(kT) void bwd_rowdot_kernel(int64_t rows, const T* __restrict__ dO,
                                                        const T* __restrict__ o, float* __restrict__ out) {
  constexpr int G = D / 8;  // lanes per row
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kT + threadIdx.x;
  const int64_t r = idx / G;
  const int part = static_cast<int>(idx % G);
  float s = 0.f;
  if (r < rows) {
    float x[8], y[8];
    load8(dO + r * D + 8 * part, x);
    load8(o + r * D + 8 * part, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(x[e], y[e], s);
  }
#pragma unroll
  for (int off = 1; off < G; off <<= 1) s += __shfl_xor(s, off, 64);
  if (r < rows && part == 0) out[r] = s;
}

__global__ __launch_bounds__(kT) void bwd_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kT + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kT)
    p[i] = 0.f;
}

// out[s] = sum_{i >= s} dc[i] per head, accumulated in fp64.
__global__ __launch_bounds__(kT) void bwd_suffix_kernel(int64_t L, const float* __restrict__ dc,
                                                        float* __restrict__ out) {
  __shared__ double tot[kT];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * L;
  const int64_t chunk = (L + kT - 1) / kT;
  const int64_t lo = threadIdx.x * chunk;
  const int64_t hi = lo + chunk < L ? lo + chunk : L;
  double s = 0.0;
  for (int64_t i = lo; i < hi; ++i) s += dc[base + i];
  tot[threadIdx.x] = s;
  __syncthreads();
  double run = 0.0;
  for (int t = threadIdx.x + 1; t < kT; ++t) run += tot[t];
  for (int64_t i = hi - 1; i >= lo; --i) {
    run += dc[base + i];
    out[base + i] = static_cast<float>(run);
  }
}

template <typename T, int D, bool FOX>
__global__ __launch_bounds__(kT, D == 64 ? 2 : 1) void bwd_pair_kernel(
    int64_t L, int Nb, int64_t BH, float scale, const T* __restrict__ v, const T* __restrict__ dO,
    const float* __restrict__ qhat, const float* __restrict__ khat, const float* __restrict__ pT,
    const float* __restrict__ cum, const float* __restrict__ lse, const float* __restrict__ Dv,
    float* __restrict__ qt_scratch, float* __restrict__ dqh, float* __restrict__ rsum,
    float* __restrict__ dkh, float* __restrict__ dPacc, float* __restrict__ dVacc,
    float* __restrict__ csum) {
  constexpr int C = kBlk, CQ = C + 1, CA = C + 4, DP = D + 1, NQ = D * C / kT;
  __shared__ float Qt[D][CQ];   // transported queries of the block, column i = query i
  __shared__ float Lam[D][CA];  // their adjoint; in the first pass the transport's output
  __shared__ float X[C][CA];    // [key j][query i]: p, then dS
  __shared__ float dOs[C][DP];  // dO of the query block (rows past the end are 0)
  __shared__ float sD[C], sL[C], sCm[C], sCn[C], sRs[C];

  const int tid = threadIdx.x;
  const int lr = tid & 15, lk = (tid >> 4) & 3, wv = tid >> 6;
  const int m = Nb - 1 - static_cast<int>(blockIdx.x / BH);  // longest query blocks first
  const int64_t bh = blockIdx.x % BH;
  const int64_t i0 = static_cast<int64_t>(m) * C;
  const int valid = static_cast<int>(L - i0 < C ? L - i0 : C);
  const int64_t hb = bh * L;
  const T* dOm = dO + (hb + i0) * D;

  if (tid < C) {
    const bool ok = tid < valid;
    sD[tid] = ok ? Dv[hb + i0 + tid] : 0.f;
    sL[tid] = ok ? lse[hb + i0 + tid] : 0.f;
    sCm[tid] = (FOX && ok) ? cum[hb + i0 + tid] : 0.f;
    sRs[tid] = 0.f;
  }
  for (int idx = tid; idx < C * D; idx += kT) {
    const int i = idx / D, e = idx % D;
    const bool ok = i < valid;
    Qt[e][i] = ok ? qhat[(hb + i0 + i) * D + e] : 0.f;
    dOs[i][e] = ok ? load_f32(dOm + idx) : 0.f;
  }

  const int64_t npairs = static_cast<int64_t>(Nb) * (Nb - 1) / 2;
  float* scr = qt_scratch + (bh * npairs + static_cast<int64_t>(m) * (m - 1) / 2) * (D * C);
  // P_n as stored: pT[(bh Nb + n) D^2 + b D + a] = P_n[a][b]
  const auto Pblk = [&](int n) { return pT + (bh * Nb + n) * D * D; };

  // Pass 1: Qt^(n) for n = m-1 .. 0, each kept in the scratch buffer.
  Frag<D, D> pf;  // P_n[a][b] for the wave's rows a
  if (m >= 2) {
    const float* P = Pblk(m - 1);
    frag_load<D, D>([&](int a, int b) { return P[b * D + a]; }, pf);
  }
  __syncthreads();
  for (int n = m - 1; n >= 0; --n) {
    float* dst = scr + static_cast<int64_t>(n) * (D * C);
    for (int idx = tid; idx < D * C; idx += kT) dst[idx] = Qt[idx / C][idx % C];
    if (n == 0) break;
    Acc<D, C> acc;
    tile_zero<D, C>(acc);
    tile_acc_ra<D, C, D>(pf, [&](int b, int i) { return Qt[b][i]; }, acc);
    if (n >= 2) {
      const float* P = Pblk(n - 1);
      frag_load<D, D>([&](int a, int b) { return P[b * D + a]; }, pf);
    }
    tile_emit<D, C>(acc, [&](int a, int i, float x) { Lam[a][i] = x; });
    __syncthreads();
    for (int idx = tid; idx < D * C; idx += kT) Qt[idx / C][idx % C] = Lam[idx / C][idx % C];
    __syncthreads();
  }

  // Pass 2: key blocks left to right.  Operands of block n + 1 are fetched into
  // registers while block n is computed, each right after its last use:
  //   qn  - Qt^(n) from the scratch buffer (written to LDS at the top);
  //   kf  - khat_n rows (A of S = Khat Qt), vf - value rows (A of V dO^T);
  //   ktf - scale * Khat_n^T and ptf - P_n^T (A operands of the adjoint update).
  float qn[NQ];
  Frag<C, D> kf, vf;
  Frag<D, C> ktf;
  Frag<D, D> ptf;
  float cn = 0.f;
  const auto loadA = [&](int n) {
    const float* src = scr + static_cast<int64_t>(n) * (D * C);
#pragma unroll
    for (int u = 0; u < NQ; ++u) qn[u] = src[tid + kT * u];
    const float* kb = khat + (hb + static_cast<int64_t>(n) * C) * D;
    const T* vb = v + (hb + static_cast<int64_t>(n) * C) * D;  // a whole block: n < m
    frag_load<C, D>([&](int j, int e) { return kb[j * D + e]; }, kf);
    frag_load<C, D>([&](int j, int e) { return load_f32(vb + j * D + e); }, vf);
    if (FOX && tid < C) cn = cum[hb + static_cast<int64_t>(n) * C + tid];
  };
  const auto loadB = [&](int n) {
    const float* kb = khat + (hb + static_cast<int64_t>(n) * C) * D;
    frag_load<D, C>([&](int a, int j) { return scale * kb[j * D + a]; }, ktf);
    if (n >= 1) {
      const float* P = Pblk(n);
      frag_load<D, D>([&](int a, int b) { return P[a * D + b]; }, ptf);
    }
  };
  if (m >= 1) {
    loadA(0);
    loadB(0);
  }
  for (int n = 0; n < m; ++n) {
    const int64_t j0 = static_cast<int64_t>(n) * C;
    // Qt's readers of block n - 1 passed the barrier before the adjoint emit
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int idx = tid + kT * u;
      Qt[idx / C][idx % C] = qn[u];
    }
    if (FOX && tid < C) sCn[tid] = cn;
    __syncthreads();

    // p_ij = exp(scale Khat_n Qt + c_i - c_j - lse_i), kept in registers
    Acc<C, C> ps;
    tile_zero<C, C>(ps);
    tile_acc_ra<C, C, D>(kf, [&](int e, int i) { return Qt[e][i]; }, ps);
    // dP_ij = dO_i . v_j
    Acc<C, C> pd;
    tile_zero<C, C>(pd);
    tile_acc_ra<C, C, D>(vf, [&](int e, int i) { return dOs[i][e]; }, pd);
    if (n + 1 < m) loadA(n + 1);
#pragma unroll
    for (int c = 0; c < C / 16; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = 16 * wv + 4 * lk + t, i = 16 * c + lr;
        const float sv = scale * ps[0][c][t] + (FOX ? sCm[i] - sCn[j] : 0.f);
        const float p = i < valid ? expf(sv - sL[i]) : 0.f;
        ps[0][c][t] = p;
        X[j][i] = p;
      }
    // dV_n += p dO_m (the wave's own rows of X: no barrier)
    tile_mm<C, D, C>([&](int j, int i) { return X[j][i]; }, [&](int i, int e) { return dOs[i][e]; },
                     [&](int j, int e, float x) { unsafeAtomicAdd(dVacc + (hb + j0 + j) * D + e, x); });
    // dS = p (dO . v - D), over the same elements
    float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C / 16; ++c) {
      float colp = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = 16 * wv + 4 * lk + t, i = 16 * c + lr;
        const float ds = ps[0][c][t] * (pd[0][c][t] - sD[i]);
        X[j][i] = ds;
        rowp[t] += ds;
        colp += ds;
      }
      if (FOX) atomicAdd(&sRs[16 * c + lr], colp);
    }
    if (FOX) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float r = row16_sum(rowp[t]);
        if (lr == 0) unsafeAtomicAdd(csum + hb + j0 + 16 * wv + 4 * lk + t, r);
      }
    }
    // dKhat_n += scale dS Qt^T
    tile_mm<C, D, C>([&](int j, int i) { return X[j][i]; }, [&](int i, int e) { return Qt[e][i]; },
                     [&](int j, int e, float x) { unsafeAtomicAdd(dkh + (hb + j0 + j) * D + e, scale * x); });
    // dP_n += Lam^(n-1) Qt^(n)^T
    if (n >= 1)
      tile_mm<D, D, C>([&](int a, int i) { return Lam[a][i]; }, [&](int i, int b) { return Qt[b][i]; },
                       [&](int a, int b, float x) { unsafeAtomicAdd(dPacc + ((bh * Nb + n) * D + a) * D + b, x); });
    __syncthreads();  // every wave's dS rows are in X
    // Lam <- P_n^T Lam + scale Khat_n^T dS
    Acc<D, C> acc;
    tile_zero<D, C>(acc);
    if (n >= 1) tile_acc_ra<D, C, D>(ptf, [&](int b, int i) { return Lam[b][i]; }, acc);
    tile_acc_ra<D, C, C>(ktf, [&](int j, int i) { return X[j][i]; }, acc);
    if (n + 1 < m) loadB(n + 1);
    __syncthreads();
    tile_emit<D, C>(acc, [&](int a, int i, float x) { Lam[a][i] = x; });
  }
  __syncthreads();
  for (int idx = tid; idx < C * D; idx += kT) {
    const int i = idx / D, e = idx % D;
    // the first block has no earlier key blocks: nothing reaches its qhat
    if (i < valid) dqh[(hb + i0 + i) * D + e] = m > 0 ? Lam[e][i] : 0.f;
  }
  if (FOX && tid < valid) rsum[hb + i0 + tid] = sRs[tid];
}

// Reduce-scatter over the four 16-lane rows of a wave: each lane passes four
// values v[0..3] and receives, in row s, the sum over the four rows of v[s]
// (lane l16 of every row contributing its own v).  Two permlane32 swaps pair
// rows s and s ^ 2 (rows 0-1 keep v0, v1; rows 2-3 keep v2, v3), one
// permlane16 swap pairs rows s and s ^ 1.  Every lane takes part.
__device__ __forceinline__ float rows_reduce_scatter(float v0, float v1, float v2, float v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
  const float r02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // rows 0-1: v0, rows 2-3: v2
  const float r13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // rows 0-1: v1, rows 2-3: v3
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(r02), __float_as_uint(r13), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48),
// the same bits in every lane.
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Waves of the in-block kernel: 16 at d = 64, 8 at d = 128 (LDS holds the
// block's w, k rows and their gradient sums, 32 or 64 KB each).
template <int D>
constexpr int block_waves() { return D == 64 ? 16 : 8; }

template <typename T, int D, bool FOX>
__global__ __launch_bounds__(64 * block_waves<D>()) void bwd_block_kernel(
    int64_t L, int Nb, int64_t BH, float scale, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ w, const float* __restrict__ beta,
    const T* __restrict__ dO, const float* __restrict__ cum, const float* __restrict__ lse,
    const float* __restrict__ Dv, const float* __restrict__ dqh, const float* __restrict__ dkh,
    const float* __restrict__ dPacc, const float* __restrict__ dVacc, const float* __restrict__ rsum,
    const float* __restrict__ csum, T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv,
    T* __restrict__ dw, float* __restrict__ dbeta, float* __restrict__ dc) {
  constexpr int C = kBlk, CP = C + 1, NW = block_waves<D>(), NT = 64 * NW;
  constexpr int NU = D / 16;  // elements of a chain's vector per lane
  constexpr int G = D == 64 ? 2 : 1;  // groups of four chains a wave runs in lockstep
  __shared__ float Ws[C][D], Ks[C][D], gW[C][D], gK[C][D];
  __shared__ float PD[C][CP];     // [key c][query r]: dO_r . v_c, then p
  __shared__ float sA[NW][G][4][C];  // a_t = w_t . x^(t+1) of each chain a wave runs
  __shared__ float sB[C], sL[C], sD[C], sC[C], gB[C], cs[C], rs[C];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = (tid >> 4) & 3, l16 = tid & 15;  // chain of the wave, lane in the chain
  const int n = static_cast<int>(blockIdx.x / BH);
  const int64_t bh = blockIdx.x % BH;
  const int64_t t0 = static_cast<int64_t>(n) * C;
  const int valid = static_cast<int>(L - t0 < C ? L - t0 : C);
  const int64_t hb = bh * L;
  const int64_t rb = (hb + t0) * D;  // first element of the block's rows

  for (int idx = tid; idx < C * D; idx += NT) {
    const int r = idx / D, e = idx % D;
    const bool ok = r < valid;
    Ws[r][e] = ok ? load_f32(w + rb + idx) : 0.f;
    Ks[r][e] = ok ? load_f32(k + rb + idx) : 0.f;
    gW[r][e] = 0.f;
    gK[r][e] = 0.f;
  }
  if (tid < C) {
    const bool ok = tid < valid;
    sB[tid] = ok ? beta[hb + t0 + tid] : 0.f;
    sL[tid] = ok ? lse[hb + t0 + tid] : 0.f;
    sD[tid] = ok ? Dv[hb + t0 + tid] : 0.f;
    sC[tid] = (FOX && ok) ? cum[hb + t0 + tid] : 0.f;
    gB[tid] = 0.f;
    cs[tid] = 0.f;
    rs[tid] = 0.f;
  }
  const auto dO_at = [&](int r, int e) { return r < valid ? load_f32(dO + rb + static_cast<int64_t>(r) * D + e) : 0.f; };
  if (wave < kT / 64)  // the tile products run on the first four waves
    tile_mm<C, C, D>([&](int c, int e) { return c < valid ? load_f32(v + rb + static_cast<int64_t>(c) * D + e) : 0.f; },
                     [&](int e, int r) { return dO_at(r, e); },
                     [&](int c, int r, float x) { PD[c][r] = c <= r ? x : 0.f; });  // p = 0 above the causal edge
  __syncthreads();

  // Householder chains, four per wave and G groups of four in lockstep: chain
  // `sub` of group gi owns lanes 16 sub .. 16 sub + 15, each holding elements
  // e = l16 + 16 u of the chain's vector.  Dot products are sums over the
  // chain's 16 lanes (DPP moves within a row, so chains never mix).  A chain's
  // earlier state is rebuilt from the next as x^(t+1) = x^(t) + beta_t a_t w_t.
  // Groups hold four consecutive indices: query chains r, key chains c, then
  // (when P_n takes part in a transport) columns of P_n.  The contributions of
  // the G x 4 chains to a gradient row are summed in registers over the groups
  // and across the wave's rows (reduce-scatter) before one LDS atomic per lane:
  // the atomic rate, not the arithmetic, bounds this kernel.
  const auto dotw = [&](int t, const float (&x)[NU]) {
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) s = fmaf(Ws[t][l16 + 16 * u], x[u], s);
    return row16_sum(s);
  };
  const auto add_rows = [&](float (*dst)[D], int t, const float (&c)[NU]) {
#pragma unroll
    for (int h = 0; h < NU / 4; ++h)
      atomicAdd(&dst[t][l16 + 16 * (4 * h + sub)],
                rows_reduce_scatter(c[4 * h], c[4 * h + 1], c[4 * h + 2], c[4 * h + 3]));
  };
  const int ngq = (valid + 3) / 4;
  const int nsq = (ngq + G - 1) / G;  // lockstep sets of query (and of key) groups
  const bool haveP = n >= 1 && n <= Nb - 2;
  const int nsets = 2 * nsq + (haveP ? D / 4 / G : 0);
  for (int set = wave; set < nsets; set += NW) {
    float x[G][NU], xb[G][NU];
    if (set < nsq) {
      // Query chain r: x^(t+1) = H_{t+1}...H_r q_r meets key t, then takes H_t.
      int r[G];
      bool live[G];
      float lr[G], dr[G], cr[G], rsum_r[G];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        r[gi] = 4 * (G * set + gi) + sub;  // < 64: G nsq <= 16 groups
        live[gi] = r[gi] < valid;
#pragma unroll
        for (int u = 0; u < NU; ++u)
          x[gi][u] = live[gi] ? load_f32(q + rb + static_cast<int64_t>(r[gi]) * D + l16 + 16 * u) : 0.f;
      }
      const int tmax = min(4 * (G * set + G - 1) + 3, valid - 1);
      for (int t = tmax; t >= 0; --t) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const bool act = live[gi] && t <= r[gi];
          const float a = dotw(t, x[gi]);
          if (act && l16 == 0) sA[wave][gi][sub][t] = a;
          const float ba = act ? sB[t] * a : 0.f;
#pragma unroll
          for (int u = 0; u < NU; ++u) x[gi][u] = fmaf(-ba, Ws[t][l16 + 16 * u], x[gi][u]);
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
          xb[gi][u] = live[gi] ? dqh[rb + static_cast<int64_t>(r[gi]) * D + l16 + 16 * u] : 0.f;
        lr[gi] = live[gi] ? sL[r[gi]] : 0.f;
        dr[gi] = live[gi] ? sD[r[gi]] : 0.f;
        cr[gi] = live[gi] ? sC[r[gi]] : 0.f;
        rsum_r[gi] = 0.f;
      }
      for (int t = 0; t <= tmax; ++t) {
        const float bt = sB[t];
        float cw[NU], ck[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) cw[u] = ck[u] = 0.f;
        float gb = 0.f, cst = 0.f;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const bool act = live[gi] && t <= r[gi];
          const float a = act ? sA[wave][gi][sub][t] : 0.f;
          float xn[NU];
#pragma unroll
          for (int u = 0; u < NU; ++u) xn[u] = fmaf(bt * a, Ws[t][l16 + 16 * u], x[gi][u]);
          float kx = 0.f;
#pragma unroll
          for (int u = 0; u < NU; ++u) kx = fmaf(Ks[t][l16 + 16 * u], xn[u], kx);
          kx = row16_sum(kx);
          const float g = dotw(t, xb[gi]);
          const float sv = scale * kx + (FOX ? cr[gi] - sC[t] : 0.f);
          const float p = act ? expf(sv - lr[gi]) : 0.f;
          const float ds = act ? p * (PD[t][r[gi]] - dr[gi]) : 0.f;
          const float E = scale * ds;
          const float bta = act ? bt : 0.f;  // an idle chain adds exact zeros
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            cw[u] = fmaf(-bta, fmaf(a, xb[gi][u], g * xn[u]), cw[u]);
            ck[u] = fmaf(E, xn[u], ck[u]);
          }
          gb -= g * a;
          if (FOX && t < r[gi]) cst += ds;
          if (act) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
              xb[gi][u] = fmaf(-bt * g, Ws[t][l16 + 16 * u], xb[gi][u]);
              xb[gi][u] = fmaf(E, Ks[t][l16 + 16 * u], xb[gi][u]);
              x[gi][u] = xn[u];
            }
            if (l16 == 0) {
              PD[t][r[gi]] = p;
              if (FOX && t < r[gi]) rsum_r[gi] += ds;
            }
          }
        }
        add_rows(gW, t, cw);
        add_rows(gK, t, ck);
        // dbeta_t and gate terms of the chains (idle chains give 0), one lane adds
        const float gbt = rows_sum(gb);
        const float cs4 = FOX ? rows_sum(cst) : 0.f;
        if (lane == 0) {
          atomicAdd(&gB[t], gbt);
          if (FOX) atomicAdd(&cs[t], cs4);
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
        if (live[gi]) {
#pragma unroll
          for (int u = 0; u < NU; ++u)
            store_f32(dq + rb + static_cast<int64_t>(r[gi]) * D + l16 + 16 * u, xb[gi][u]);
          if (FOX && l16 == 0) rs[r[gi]] = rsum_r[gi];
        }
    } else if (set < 2 * nsq) {
      // Key chain c: y = H_t...H_{c+1} k_c, from k_c up to khat_c.
      const int s0 = set - nsq;
      int c[G];
      bool live[G];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        c[gi] = 4 * (G * s0 + gi) + sub;
        live[gi] = c[gi] < valid;
#pragma unroll
        for (int u = 0; u < NU; ++u) x[gi][u] = live[gi] ? Ks[c[gi]][l16 + 16 * u] : 0.f;
      }
      const int tmin = 4 * G * s0 + 1;  // smallest c + 1 of the set
      for (int t = tmin; t < valid; ++t) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const bool act = live[gi] && t > c[gi];
          const float a = dotw(t, x[gi]);
          if (act && l16 == 0) sA[wave][gi][sub][t] = a;
          const float ba = act ? sB[t] * a : 0.f;
#pragma unroll
          for (int u = 0; u < NU; ++u) x[gi][u] = fmaf(-ba, Ws[t][l16 + 16 * u], x[gi][u]);
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int u = 0; u < NU; ++u)
          xb[gi][u] = live[gi] ? dkh[rb + static_cast<int64_t>(c[gi]) * D + l16 + 16 * u] : 0.f;
      for (int t = valid - 1; t >= tmin; --t) {
        const float bt = sB[t];
        float cw[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) cw[u] = 0.f;
        float gb = 0.f;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const bool act = live[gi] && t > c[gi];
          const float a = act ? sA[wave][gi][sub][t] : 0.f;
          float xp[NU];
#pragma unroll
          for (int u = 0; u < NU; ++u) xp[u] = fmaf(bt * a, Ws[t][l16 + 16 * u], x[gi][u]);
          const float g = dotw(t, xb[gi]);
          const float bta = act ? bt : 0.f;
#pragma unroll
          for (int u = 0; u < NU; ++u) cw[u] = fmaf(-bta, fmaf(a, xb[gi][u], g * xp[u]), cw[u]);
          gb -= g * a;
          if (act) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
              xb[gi][u] = fmaf(-bt * g, Ws[t][l16 + 16 * u], xb[gi][u]);
              x[gi][u] = xp[u];
            }
          }
        }
        add_rows(gW, t, cw);
        const float gbt = rows_sum(gb);
        if (lane == 0) atomicAdd(&gB[t], gbt);
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
        if (live[gi]) {
#pragma unroll
          for (int u = 0; u < NU; ++u) atomicAdd(&gK[c[gi]][l16 + 16 * u], xb[gi][u]);
        }
    } else {
      // Column col of P_n = H_0 ... H_63: x = H_t...H_63 e_col.
      const int s0 = set - 2 * nsq;
      int col[G];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        col[gi] = 4 * (G * s0 + gi) + sub;
#pragma unroll
        for (int u = 0; u < NU; ++u) x[gi][u] = (l16 + 16 * u == col[gi]) ? 1.f : 0.f;
      }
      for (int t = valid - 1; t >= 0; --t) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const float a = dotw(t, x[gi]);
          if (l16 == 0) sA[wave][gi][sub][t] = a;
          const float ba = sB[t] * a;
#pragma unroll
          for (int u = 0; u < NU; ++u) x[gi][u] = fmaf(-ba, Ws[t][l16 + 16 * u], x[gi][u]);
        }
      }
      const float* gP = dPacc + (bh * Nb + n) * D * D;
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int u = 0; u < NU; ++u) xb[gi][u] = gP[(l16 + 16 * u) * D + col[gi]];
      for (int t = 0; t < valid; ++t) {
        const float bt = sB[t];
        float cw[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) cw[u] = 0.f;
        float gb = 0.f;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const float a = sA[wave][gi][sub][t];
          float xn[NU];
#pragma unroll
          for (int u = 0; u < NU; ++u) xn[u] = fmaf(bt * a, Ws[t][l16 + 16 * u], x[gi][u]);
          const float g = dotw(t, xb[gi]);
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            cw[u] = fmaf(-bt, fmaf(a, xb[gi][u], g * xn[u]), cw[u]);
            xb[gi][u] = fmaf(-bt * g, Ws[t][l16 + 16 * u], xb[gi][u]);
            x[gi][u] = xn[u];
          }
          gb -= g * a;
        }
        add_rows(gW, t, cw);
        const float gbt = rows_sum(gb);
        if (lane == 0) atomicAdd(&gB[t], gbt);
      }
    }
  }
  __syncthreads();

  for (int idx = tid; idx < C * D; idx += NT) {
    const int r = idx / D, e = idx % D;
    if (r < valid) {
      store_f32(dk + rb + idx, gK[r][e]);
      store_f32(dw + rb + idx, gW[r][e]);
    }
  }
  if (tid < valid) {
    dbeta[hb + t0 + tid] = gB[tid];
    if (FOX) dc[hb + t0 + tid] = rsum[hb + t0 + tid] + rs[tid] - csum[hb + t0 + tid] - cs[tid];
  }
  // dv_c = cross-block part + sum_r p_cr dO_r
  if (wave < kT / 64)
    tile_mm<C, D, C>([&](int c, int r) { return PD[c][r]; }, dO_at, [&](int c, int e, float x) {
      if (c < valid) store_f32(dv + rb + static_cast<int64_t>(c) * D + e, x + dVacc[rb + static_cast<int64_t>(c) * D + e]);
    });
}

template <typename T, int D, bool FOX>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int64_t BH = a.BH, L = a.L;
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  const T* v = static_cast<const T*>(a.v);
  const T* dO = static_cast<const T*>(a.dout);
  hipLaunchKernelGGL((bwd_rowdot_kernel<T, D>), dim3(static_cast<unsigned>((BH * L * (D / 8) + kT - 1) / kT)),
                     dim3(kT), 0, stream, BH * L, dO, static_cast<const T*>(a.o), a.ws.Dv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_zero_kernel, dim3(2048), dim3(kT), 0, stream, a.ws.zero_begin, a.ws.zero_count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(BH * Nb));
  if constexpr (std::is_same_v<T, bf16_t>) {
    if ((e = launch_bwd_pair16(D, a, stream)) != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((bwd_pair_kernel<T, D, FOX>), grid, dim3(kT), 0, stream, L, Nb, BH, a.scale, v, dO,
                       a.ws.qhat, a.ws.khat, a.ws.pT, a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dqh, a.ws.rsum,
                       a.ws.dkh, a.ws.dP, a.ws.dV, a.ws.csum);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const BwdBlockArgs b{BH, L, a.scale, a.q, a.k, a.v, a.w, a.dout, a.beta, a.ws.cum, a.lse, a.ws.Dv, a.ws.minv,
                       a.ws.dqh, a.ws.dkh, a.ws.dP, a.ws.dV, a.ws.rsum, a.ws.csum, a.dq, a.dk, a.dv, a.dw,
                       a.dbeta, a.ws.dc};
  if constexpr (D == 64) {
    if ((e = launch_bwd_block_ut(std::is_same_v<T, float> ? 0 : 1, b, stream)) != hipSuccess) return e;
  } else if constexpr (std::is_same_v<T, bf16_t>) {
    if ((e = launch_bwd_block_ut128(b, stream)) != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((bwd_block_kernel<T, D, FOX>), grid, dim3(64 * block_waves<D>()), 0, stream, L, Nb, BH,
                       a.scale, static_cast<const T*>(a.q), static_cast<const T*>(a.k), v, static_cast<const T*>(a.w),
                       a.beta, dO, a.ws.cum, a.lse, a.ws.Dv, a.ws.dqh, a.ws.dkh, a.ws.dP, a.ws.dV, a.ws.rsum,
                       a.ws.csum, static_cast<T*>(a.dq), static_cast<T*>(a.dk), static_cast<T*>(a.dv),
                       static_cast<T*>(a.dw), a.dbeta, a.ws.dc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (FOX) {
    hipLaunchKernelGGL(bwd_suffix_kernel, dim3(static_cast<unsigned>(BH)), dim3(kT), 0, stream, L, a.ws.dc,
                       a.dlog_forget);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd(int dtype, int64_t d, const BwdArgs& a, hipStream_t stream) {
  const bool fox = a.ws.cum != nullptr;
  if (dtype == 0) {
    if (d == 64) return fox ? launch_bwd_t<float, 64, true>(a, stream) : launch_bwd_t<float, 64, false>(a, stream);
    return fox ? launch_bwd_t<float, 128, true>(a, stream) : launch_bwd_t<float, 128, false>(a, stream);
  }
  if (d == 64) return fox ? launch_bwd_t<bf16_t, 64, true>(a, stream) : launch_bwd_t<bf16_t, 64, false>(a, stream);
  return fox ? launch_bwd_t<bf16_t, 128, true>(a, stream) : launch_bwd_t<bf16_t, 128, false>(a, stream);
}

}  // namespace path
