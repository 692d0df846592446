// In-block part of the PaTH backward for head dimension 64, in matrix form.
//
// [PaTH Attention summary (gist.science 2505.16381), §3 "Representação de
// Transformação UT"]: for the 64 tokens of one block (rows w_s, k_s, q_s of
// W, K, Q and the factors beta_s), with
//     G = W W^T,  N = strict_upper(G),  M = (I + diag(beta) N)^{-1},
//     X = M diag(beta)                       (the UT factor T^{-1})
//     Z = strict_upper(K W^T)                (Z[c][a] = k_c . w_a, a > c)
//     Y = Z X,  F = X^T W,  Ut = upper(W Q^T) (Ut[b][r] = w_b . q_r, b <= r)
// the block's outputs are
//     Khat = K - Y W                  (k_c carried through H_{c+1} .. H_63)
//     P    = I - F^T W                (= H_0 H_1 ... H_63)
//     Qhat = Q - Ut^T F               (q_r carried through H_r .. H_0)
//     S^T  = upper(K Q^T - Y Ut)      (in-block logits k_c . H_{c+1}..H_r q_r, c <= r)
// The cross-block kernel hands over the gradients reaching Khat, P and Qhat
// (summed over the other blocks); the in-block attention adds the logits'
// gradient, scale * p (dO . v - D) per key c <= query r.  This kernel runs
// reverse mode through the formulas above (writing  A' for the gradient of A):
//     K' = S' Q + Khat' + Zm' W            Q' = S'^T K + Qhat' + U'^T W
//     Y' = -S' Ut^T - Khat' W^T            Ut' = -Y^T S' - F Qhat'^T,  U' = upper(Ut')
//     F' = -Ut Qhat' - W P'^T              X' = W F'^T + Z^T Y'
//     Z' = Y' X^T,  Zm' = strict_upper(Z')
//     W' = -Y^T Khat' - F P' + U' Q + X F' + Zm'^T K + (G' + G'^T) W
//     beta'_j = sum_i M[i][j] X'[i][j] + sum_b T'[j][b] N[j][b]
//     T' = -M^T (X' X^T),   G' = strict_upper(diag(beta) T')
// which are thirty 64 x 64 x 64 products on the fp32 matrix cores.
//
// Layout: 16 waves (four per SIMD); each 64 x 64 matrix lives in registers,
// wave w holding its 16 x 16 tile (w & 3, w >> 2) (4 floats per lane; with
// PATH_UT_TPW = 2, 8 waves of two tiles each, which measured 10 % slower).
// W, K, Q and M stay in LDS; the other operands of a product are
// staged into four LDS slots between two barriers.  A slot row has 68 floats,
// which keeps both the row reads (16 rows x 4 consecutive floats) and the
// column reads (4 rows x 16 consecutive floats) of the products on distinct
// banks.
#include "common.h"
#include "launch.h"

namespace path {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kC = kBlk;     // tokens per block
constexpr int kD = 64;       // head dimension
constexpr int kSP = 68;      // slot row pitch (floats)
constexpr int kSlot = kC * kSP;
#ifndef PATH_UT_TPW
#define PATH_UT_TPW 1
#endif
constexpr int kTPW = PATH_UT_TPW;  // 16 x 16 tiles of a 64 x 64 matrix per wave
constexpr int kUW = 16 / kTPW;     // waves
constexpr int kUT = 64 * kUW;
constexpr int kEPT = kC * kD / kUT;  // elements per thread of a 64 x 64 row copy

// This wave's share of a 64 x 64 matrix: element i of t[j] is row
// 16 rt + 4 lk + i, column 32 ch + 16 j + lr.
struct Mat {
  f4 t[kTPW];
};

struct Lane {
  int rt, ch, lr, lk;
  __device__ int row(int i) const { return 16 * rt + 4 * lk + i; }
  __device__ int col(int j) const { return 16 * (kTPW * ch + j) + lr; }
};

__device__ __forceinline__ Mat zero_mat() {
  Mat m;
#pragma unroll
  for (int j = 0; j < kTPW; ++j) m.t[j] = f4{0.f, 0.f, 0.f, 0.f};
  return m;
}

// Operand reads.  A(m, k): Row reads S[m][k] (one 16-byte read per lane and
// chunk), Col reads S[k][m] (A = S^T).  B(k, n): Col reads S[k][n] (B = S),
// Tr reads S[n][k] (B = S^T), optionally times beta_k.
enum { kRow = 0, kCol = 1 };
enum { kBCol = 0, kBTr = 1, kBTrBeta = 2 };

template <int AK, int BK>
__device__ __forceinline__ void mm(Mat& acc, const Lane& L, const float* A, const float* B,
                                   const float* beta) {
#pragma unroll
  for (int c = 0; c < kC / 16; ++c) {
    const int k0 = 16 * c + 4 * L.lk;
    float av[4], bv[kTPW][4];
    if constexpr (AK == kRow) {
      const f4 v = *reinterpret_cast<const f4*>(A + (16 * L.rt + L.lr) * kSP + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = v[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = A[(k0 + j) * kSP + 16 * L.rt + L.lr];
    }
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
      const int n = 16 * (kTPW * L.ch + t) + L.lr;
      if constexpr (BK == kBCol) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[t][j] = B[(k0 + j) * kSP + n];
      } else {
        f4 v = *reinterpret_cast<const f4*>(B + n * kSP + k0);
        if constexpr (BK == kBTrBeta) v *= *reinterpret_cast<const f4*>(beta + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[t][j] = v[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < kTPW; ++t) acc.t[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[t][j], acc.t[t], 0, 0, 0);
  }
}

// A with its columns scaled by beta (A = M diag(beta) read as rows of M).
__device__ __forceinline__ void mm_xrow_bcol(Mat& acc, const Lane& L, const float* A, const float* B,
                                             const float* beta) {
#pragma unroll
  for (int c = 0; c < kC / 16; ++c) {
    const int k0 = 16 * c + 4 * L.lk;
    const f4 v = *reinterpret_cast<const f4*>(A + (16 * L.rt + L.lr) * kSP + k0) *
                 *reinterpret_cast<const f4*>(beta + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < kTPW; ++t)
        acc.t[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[j], B[(k0 + j) * kSP + 16 * (kTPW * L.ch + t) + L.lr], acc.t[t],
                                                        0, 0, 0);
  }
}

__device__ __forceinline__ void stage(const Mat& m, const Lane& L, float* S) {
#pragma unroll
  for (int j = 0; j < kTPW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) S[L.row(i) * kSP + L.col(j)] = m.t[j][i];
}

__device__ __forceinline__ Mat from_slot(const Lane& L, const float* S) {
  Mat m;
#pragma unroll
  for (int j = 0; j < kTPW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) m.t[j][i] = S[L.row(i) * kSP + L.col(j)];
  return m;
}

// Element-wise update with the element's (row, column).
template <typename F>
__device__ __forceinline__ void each(Mat& m, const Lane& L, const F& f) {
#pragma unroll
  for (int j = 0; j < kTPW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = m.t[j][i];
      f(L.row(i), L.col(j), x);
      m.t[j][i] = x;
    }
}

// 64 rows of a [*, 64] row-major tensor into a slot as fp32 (rows >= valid are 0).
template <typename T>
__device__ __forceinline__ void load_rows(float* S, const T* src, int valid) {
  const int tid = threadIdx.x;
  const int r = tid / (kD / kEPT), c0 = kEPT * (tid % (kD / kEPT));  // kEPT consecutive elements of row r
  float x[kEPT];
  if (r < valid) {
#pragma unroll
    for (int e = 0; e < kEPT; ++e) x[e] = load_f32(src + r * kD + c0 + e);
  } else {
#pragma unroll
    for (int e = 0; e < kEPT; ++e) x[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < kEPT; e += 4) *reinterpret_cast<f4*>(S + r * kSP + c0 + e) = f4{x[e], x[e + 1], x[e + 2], x[e + 3]};
}

// Sum over the 16 lanes of a row (the same bits in every lane of the row).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp_row<0xB1>(x);
  x += dpp_row<0x4E>(x);
  x += dpp_row<0x141>(x);
  x += dpp_row<0x140>(x);
  return x;
}
// Sum over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float sum4rows(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

}  // namespace

template <typename T, bool FOX>
__global__ __launch_bounds__(kUT) void bwd_block_ut_kernel(
    int64_t L, int Nb, int64_t BH, float scale, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ w, const float* __restrict__ beta,
    const T* __restrict__ dO, const float* __restrict__ cum, const float* __restrict__ lse,
    const float* __restrict__ Dv, const float* __restrict__ minv, const float* __restrict__ dqh,
    const float* __restrict__ dkh, const float* __restrict__ dPacc, const float* __restrict__ dVacc,
    const float* __restrict__ rsum, const float* __restrict__ csum, T* __restrict__ dq, T* __restrict__ dk,
    T* __restrict__ dv, T* __restrict__ dw, float* __restrict__ dbeta, float* __restrict__ dc) {
  constexpr int C = kC, D = kD;
  __shared__ __attribute__((aligned(16))) float PW[kSlot], PK[kSlot], PQ[kSlot], PM[kSlot];
  __shared__ __attribute__((aligned(16))) float S0[kSlot], S1[kSlot], S2[kSlot], S3[kSlot];
  __shared__ __attribute__((aligned(16))) float sb[C];
  __shared__ float slse[C], sD[C], scum[C], gB[C], rs[C], cs[C];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const Lane Ln{wave & 3, wave >> 2, lane & 15, lane >> 4};
  const int n = static_cast<int>(blockIdx.x / BH);
  const int64_t bh = blockIdx.x % BH;
  const int64_t t0 = static_cast<int64_t>(n) * C;
  const int valid = static_cast<int>(L - t0 < C ? L - t0 : C);
  const int64_t hb = bh * L;
  const int64_t rb = (hb + t0) * D;  // first element of the block's rows
  const float* Mg = minv + (bh * Nb + n) * (C * C);
  const float* dPg = dPacc + (bh * Nb + n) * (D * D);

  // ---- inputs: W, K, Q rows and M (fp32) into LDS, the per-row scalars
  load_rows(PW, w + rb, valid);
  load_rows(PK, k + rb, valid);
  load_rows(PQ, q + rb, valid);
  load_rows(PM, Mg, C);
  if (tid < C) {
    const bool ok = tid < valid;
    sb[tid] = ok ? beta[hb + t0 + tid] : 0.f;
    slse[tid] = ok ? lse[hb + t0 + tid] : 0.f;
    sD[tid] = ok ? Dv[hb + t0 + tid] : 0.f;
    scum[tid] = (FOX && ok) ? cum[hb + t0 + tid] : 0.f;
    gB[tid] = rs[tid] = cs[tid] = 0.f;
  }
  __syncthreads();

  // ---- forward quantities of the block
  Mat N = zero_mat(), Z = zero_mat(), Ut = zero_mat(), Sd = zero_mat(), F = zero_mat();
  mm<kRow, kBTr>(N, Ln, PW, PW, sb);   // G = W W^T
  each(N, Ln, [&](int r, int c, float& x) { x = c > r ? x : 0.f; });
  mm<kRow, kBTr>(Z, Ln, PK, PW, sb);   // K W^T
  each(Z, Ln, [&](int r, int c, float& x) { x = c > r ? x : 0.f; });
  mm<kRow, kBTr>(Ut, Ln, PW, PQ, sb);  // W Q^T
  each(Ut, Ln, [&](int r, int c, float& x) { x = c >= r ? x : 0.f; });
  mm<kRow, kBTr>(Sd, Ln, PK, PQ, sb);  // K Q^T
  mm<kCol, kBCol>(F, Ln, PM, PW, sb);  // M^T W, then F = diag(beta) M^T W
  each(F, Ln, [&](int r, int, float& x) { x *= sb[r]; });

  stage(Z, Ln, S0);
  __syncthreads();
  Mat Y = zero_mat();
  mm<kRow, kBCol>(Y, Ln, S0, PM, sb);  // Z M, then Y = Z M diag(beta)
  each(Y, Ln, [&](int, int c, float& x) { x *= sb[c]; });

  __syncthreads();
  stage(Y, Ln, S1);
  stage(Ut, Ln, S2);
  __syncthreads();
  {
    Mat yu = zero_mat();
    mm<kRow, kBCol>(yu, Ln, S1, S2, sb);  // Y Ut
#pragma unroll
    for (int j = 0; j < kTPW; ++j) Sd.t[j] -= yu.t[j];
    each(Sd, Ln, [&](int r, int c, float& x) { x = c >= r ? x : 0.f; });  // S^T[c][r], c <= r
  }

  // ---- in-block attention: p, dS, the value gradient
  __syncthreads();
  load_rows(S3, v + rb, valid);
  load_rows(S0, dO + rb, valid);
  __syncthreads();
  Mat Pm = zero_mat(), Sb = zero_mat();
  {
    Mat pd = zero_mat();
    mm<kRow, kBTr>(pd, Ln, S3, S0, sb);  // PD[c][r] = v_c . dO_r
    float csum_l[4] = {0.f, 0.f, 0.f, 0.f};
    float rsum_l[kTPW] = {};
#pragma unroll
    for (int j = 0; j < kTPW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = Ln.row(i), r = Ln.col(j);
        const bool act = c <= r && r < valid;
        const float sv = scale * Sd.t[j][i] + (FOX ? scum[r] - scum[c] : 0.f);
        const float p = act ? expf(sv - slse[r]) : 0.f;
        const float ds = act ? p * (pd.t[j][i] - sD[r]) : 0.f;
        Pm.t[j][i] = p;
        Sb.t[j][i] = scale * ds;
        if (FOX && c < r) {
          csum_l[i] += ds;  // key c, summed over queries r > c
          rsum_l[j] += ds;  // query r, summed over keys c < r
        }
      }
    if (FOX) {
      // key sums over this wave's columns (16 lanes of each of its tiles), query
      // sums over its 16 rows (4 in-lane x 4 lane rows), then across waves
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = sum16(csum_l[i]);
        if (Ln.lr == 0) atomicAdd(&cs[Ln.row(i)], s);
      }
#pragma unroll
      for (int j = 0; j < kTPW; ++j) {
        const float s = sum4rows(rsum_l[j]);
        if (Ln.lk == 0) atomicAdd(&rs[Ln.col(j)], s);
      }
    }
  }
  __syncthreads();
  stage(Pm, Ln, S3);
  __syncthreads();
  {
    Mat dvm = zero_mat();
    mm<kRow, kBCol>(dvm, Ln, S3, S0, sb);  // dv_c = sum_r p[r][c] dO_r
    each(dvm, Ln, [&](int c, int e, float& x) {
      if (c < valid) store_f32(dv + rb + c * D + e, x + dVacc[rb + c * D + e]);
    });
  }

  // ---- gradients
  __syncthreads();
  stage(Sb, Ln, S0);
  load_rows(S3, dkh + rb, valid);
  __syncthreads();
  Mat Kb = from_slot(Ln, S3), Qb = zero_mat(), Yb = zero_mat(), Wb = zero_mat(), Utb = zero_mat();
  mm<kRow, kBCol>(Kb, Ln, S0, PQ, sb);  // + S' Q
  mm<kCol, kBCol>(Qb, Ln, S0, PK, sb);  // S'^T K
  mm<kRow, kBTr>(Yb, Ln, S0, S2, sb);   // S' Ut^T
  mm<kRow, kBTr>(Yb, Ln, S3, PW, sb);   // + Khat' W^T   (Y' is the negation)
  mm<kCol, kBCol>(Wb, Ln, S1, S3, sb);  // Y^T Khat'     (subtracted from W')
  mm<kCol, kBCol>(Utb, Ln, S1, S0, sb); // Y^T S'        (subtracted from Ut')
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    Yb.t[j] = -Yb.t[j];
    Wb.t[j] = -Wb.t[j];
    Utb.t[j] = -Utb.t[j];
  }

  __syncthreads();
  stage(F, Ln, S1);
  load_rows(S3, dqh + rb, valid);
  load_rows(S0, dPg, D);
  __syncthreads();
  {
    const Mat qh = from_slot(Ln, S3);
#pragma unroll
    for (int j = 0; j < kTPW; ++j) Qb.t[j] += qh.t[j];
  }
  Mat Fb = zero_mat();
  {
    Mat t1 = zero_mat(), t3 = zero_mat();
    mm<kRow, kBTr>(t1, Ln, S1, S3, sb);   // F Qhat'^T
    mm<kRow, kBCol>(Fb, Ln, S2, S3, sb);  // Ut Qhat'
    mm<kRow, kBTr>(Fb, Ln, PW, S0, sb);   // + W P'^T     (F' is the negation)
    mm<kRow, kBCol>(t3, Ln, S1, S0, sb);  // F P'
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      Utb.t[j] -= t1.t[j];
      Fb.t[j] = -Fb.t[j];
      Wb.t[j] -= t3.t[j];
    }
  }
  each(Utb, Ln, [&](int r, int c, float& x) { x = c >= r ? x : 0.f; });  // U' = upper(Ut')

  __syncthreads();
  stage(Utb, Ln, S2);
  stage(Fb, Ln, S1);
  stage(Yb, Ln, S3);
  stage(Z, Ln, S0);
  __syncthreads();
  Mat Xb = zero_mat(), Zb = zero_mat();
  mm<kRow, kBCol>(Wb, Ln, S2, PQ, sb);  // + U' Q
  mm<kCol, kBCol>(Qb, Ln, S2, PW, sb);  // + U'^T W
  mm<kRow, kBTr>(Xb, Ln, PW, S1, sb);   // W F'^T
  mm<kCol, kBCol>(Xb, Ln, S0, S3, sb);  // + Z^T Y'
  mm_xrow_bcol(Wb, Ln, PM, S1, sb);     // + X F'   (X = M diag(beta))
  mm<kRow, kBTrBeta>(Zb, Ln, S3, PM, sb);  // Z' = Y' X^T
  each(Zb, Ln, [&](int r, int c, float& x) { x = c > r ? x : 0.f; });

  __syncthreads();
  stage(Zb, Ln, S0);
  stage(Xb, Ln, S1);
  __syncthreads();
  mm<kRow, kBCol>(Kb, Ln, S0, PW, sb);  // + Zm' W
  mm<kCol, kBCol>(Wb, Ln, S0, PK, sb);  // + Zm'^T K
  {
    // beta'_j += sum_i M[i][j] X'[i][j]: this wave's 16 rows, then across waves
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s += PM[Ln.row(i) * kSP + Ln.col(j)] * Xb.t[j][i];
      s = sum4rows(s);
      if (Ln.lk == 0) atomicAdd(&gB[Ln.col(j)], s);
    }
  }
  Mat R = zero_mat();
  mm<kRow, kBTrBeta>(R, Ln, S1, PM, sb);  // R = X' X^T

  __syncthreads();
  stage(R, Ln, S2);
  __syncthreads();
  Mat Tb = zero_mat();
  mm<kCol, kBCol>(Tb, Ln, PM, S2, sb);  // M^T R; T' = -M^T R
  {
    // beta'_a += sum_b T'[a][b] N[a][b]: this wave's columns, then across waves
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = 0.f;
#pragma unroll
      for (int j = 0; j < kTPW; ++j) s[i] -= Tb.t[j][i] * N.t[j][i];
      s[i] = sum16(s[i]);
    }
    if (Ln.lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&gB[Ln.row(i)], s[i]);
    }
  }
  each(Tb, Ln, [&](int r, int c, float& x) { x = c > r ? -sb[r] * x : 0.f; });  // G' = strict_upper(diag(beta) T')

  __syncthreads();
  stage(Tb, Ln, S3);
  __syncthreads();
  mm<kRow, kBCol>(Wb, Ln, S3, PW, sb);  // + G' W
  mm<kCol, kBCol>(Wb, Ln, S3, PW, sb);  // + G'^T W

  // ---- outputs (rows through LDS, 16-byte row segments)
  __syncthreads();
  stage(Qb, Ln, S0);
  stage(Kb, Ln, S1);
  stage(Wb, Ln, S2);
  __syncthreads();
  {
    const int r = tid / (kD / kEPT), c0 = kEPT * (tid % (kD / kEPT));
    if (r < valid) {
#pragma unroll
      for (int e = 0; e < kEPT; ++e) {
        store_f32(dq + rb + r * D + c0 + e, S0[r * kSP + c0 + e]);
        store_f32(dk + rb + r * D + c0 + e, S1[r * kSP + c0 + e]);
        store_f32(dw + rb + r * D + c0 + e, S2[r * kSP + c0 + e]);
      }
    }
  }
  if (tid < valid) {
    dbeta[hb + t0 + tid] = gB[tid];
    if (FOX) dc[hb + t0 + tid] = rsum[hb + t0 + tid] + rs[tid] - csum[hb + t0 + tid] - cs[tid];
  }
}

template <typename T, bool FOX>
static hipError_t launch_ut_t(const BwdBlockArgs& a, hipStream_t stream) {
  const int Nb = static_cast<int>((a.L + kBlk - 1) / kBlk);
  hipLaunchKernelGGL((bwd_block_ut_kernel<T, FOX>), dim3(static_cast<unsigned>(a.BH * Nb)), dim3(kUT), 0, stream,
                     a.L, Nb, a.BH, a.scale, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<const T*>(a.w), a.beta, static_cast<const T*>(a.dO),
                     a.cum, a.lse, a.Dv, a.minv, a.dqh, a.dkh, a.dP, a.dV, a.rsum, a.csum, static_cast<T*>(a.dq),
                     static_cast<T*>(a.dk), static_cast<T*>(a.dv), static_cast<T*>(a.dw), a.dbeta, a.dc);
  return hipGetLastError();
}

hipError_t launch_bwd_block_ut(int dtype, const BwdBlockArgs& a, hipStream_t stream) {
  const bool fox = a.cum != nullptr;
  if (dtype == 0) return fox ? launch_ut_t<float, true>(a, stream) : launch_ut_t<float, false>(a, stream);
  return fox ? launch_ut_t<bf16_t, true>(a, stream) : launch_ut_t<bf16_t, false>(a, stream);
}

}  // namespace path
