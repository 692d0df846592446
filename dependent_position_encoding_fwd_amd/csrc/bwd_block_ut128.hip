// In-block part of the PaTH backward for head dimension 128 with bf16 storage,
// in matrix form.
//
// [PaTH Attention summary (gist.science 2505.16381), §3 "Representação de
// Transformação UT"]: for the 64 tokens of one block (rows w_s, k_s, q_s of
// W, K, Q and the factors beta_s), with
//     G = W W^T,  N = strict_upper(G),  M = (I + diag(beta) N)^{-1},
//     X = M diag(beta),  Z = strict_upper(K W^T),  Y = Z X,  F = X^T W,
//     Ut = upper(W Q^T)
// the block's outputs are Khat = K - Y W, P = I - F^T W, Qhat = Q - Ut^T F and
// the in-block logits S^T = upper(K Q^T - Y Ut).  Reverse mode through these
// formulas, from the gradients reaching Khat, P and Qhat from the other blocks
// and the in-block logits' gradient scale * p (dO . v - D):
//     K' = S' Q + Khat' + Zm' W            Q' = S'^T K + Qhat' + U'^T W
//     Y' = -S' Ut^T - Khat' W^T            Ut' = -Y^T S' - F Qhat'^T,  U' = upper(Ut')
//     F' = -Ut Qhat' - W P'^T              X' = W F'^T + Z^T Y'
//     Z' = Y' X^T,  Zm' = strict_upper(Z')
//     W' = -Y^T Khat' - F P' + U' Q + X F' + Zm'^T K + (G' + G'^T) W
//     beta'_j = sum_i M[i][j] X'[i][j] + sum_b T'[j][b] N[j][b]
//     T' = -M^T (X' X^T),   G' = strict_upper(diag(beta) T')
// (the head-dimension-64 kernel, bwd_block_ut.hip, runs the same formulas).
// Every product runs on the fp32 matrix cores (16x16x4 MFMA).
//
// Layout: 16 waves; wave w holds tile (w & 3, w >> 2) of every 64 x 64 matrix
// and tiles (w & 3, w >> 2) and (w & 3, (w >> 2) + 4) of every 64 x 128 one
// (16 x 16 tiles, 4 floats per lane each).  LDS is nine units of 17 KB: five
// work units, then W, K and Q as bf16 rows of 136 halves (one unit each; the
// inputs are bf16, so this is exact) and M as fp32 rows of 68 floats.  A
// 64 x 64 fp32 operand takes one work unit (rows of 68 floats), a 64 x 128 one
// two adjacent units (rows of 132 floats); the 128 x 128 gradient of P_n is
// fed in two halves of 64 rows.  Row pitches of 4 mod 64 words keep the row
// reads (16 rows x 4 consecutive elements) and the column reads (4 rows x 16
// consecutive elements) of the products on distinct banks.
#include "common.h"
#include "launch.h"

namespace path {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kC = kBlk;              // tokens per block
constexpr int kD = 128;               // head dimension
constexpr int kNT = 1024;             // 16 waves
constexpr int kPc = 68;               // fp32 row pitch of a 64-column operand (floats)
constexpr int kPd = 132;              // fp32 row pitch of a 128-column operand (floats)
constexpr int kPh = 136;              // bf16 row pitch of a 128-column operand (halves)
constexpr int kUnit = kC * kPc * 4;   // bytes of one LDS unit
static_assert(kC * kPh * 2 == kUnit, "a bf16 64 x 128 operand fills one unit");
static_assert(kC * kPd * 4 <= 2 * kUnit, "an fp32 64 x 128 operand fits two units");

// Operands in LDS: fp32 rows of P floats, or bf16 rows of kPh halves.
template <int P>
struct F32 {
  const float* p;
  __device__ f4 vec4(int r, int c) const { return *reinterpret_cast<const f4*>(p + r * P + c); }
  __device__ float at(int r, int c) const { return p[r * P + c]; }
};
struct B16 {
  const uint16_t* p;
  __device__ f4 vec4(int r, int c) const {
    const uint2 u = *reinterpret_cast<const uint2*>(p + r * kPh + c);
    return f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
              __uint_as_float(u.y & 0xffff0000u)};
  }
  __device__ float at(int r, int c) const { return __uint_as_float(static_cast<uint32_t>(p[r * kPh + c]) << 16); }
};

// This wave's share of a 64 x 64 (NT = 1) or 64 x 128 (NT = 2) matrix: element
// i of t[j] is row 16 rt + 4 lk + i, column 16 (ch + 4 j) + lr.
template <int NT>
struct Mat {
  f4 t[NT];
};
using MatC = Mat<1>;
using MatD = Mat<2>;

struct Lane {
  int rt, ch, lr, lk;
  __device__ int row(int i) const { return 16 * rt + 4 * lk + i; }
  __device__ int col(int j) const { return 16 * (ch + 4 * j) + lr; }
};

template <int NT>
__device__ __forceinline__ Mat<NT> zero() {
  Mat<NT> m;
#pragma unroll
  for (int j = 0; j < NT; ++j) m.t[j] = f4{0.f, 0.f, 0.f, 0.f};
  return m;
}

// acc += A B over the reduction index k = 0 .. KL-1 (each term times beta_k
// when BETA).  A(m, k): Row reads S[m][k], Col reads S[k][m].  B(k, n): Col
// reads S[k][n], Tr reads S[n][k].
enum { kRow = 0, kCol = 1 };
enum { kBCol = 0, kBTr = 1 };

template <int AK, int BK, int KL, bool BETA = false, int NT, class OA, class OB>
__device__ __forceinline__ void mm(Mat<NT>& acc, const Lane& L, const OA& A, const OB& B, const float* beta) {
  const int m = 16 * L.rt + L.lr;
  // two chunks at a time: unrolled further, the hoisted reads spill at 16 waves
#pragma unroll 2
  for (int c = 0; c < KL / 16; ++c) {
    const int k0 = 16 * c + 4 * L.lk;
    f4 av;
    if constexpr (AK == kRow) {
      av = A.vec4(m, k0);
    } else {
      av = f4{A.at(k0, m), A.at(k0 + 1, m), A.at(k0 + 2, m), A.at(k0 + 3, m)};
    }
    if constexpr (BETA) av *= *reinterpret_cast<const f4*>(beta + k0);
    f4 bv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = L.col(t);
      if constexpr (BK == kBTr) {
        bv[t] = B.vec4(n, k0);
      } else {
        bv[t] = f4{B.at(k0, n), B.at(k0 + 1, n), B.at(k0 + 2, n), B.at(k0 + 3, n)};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc.t[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[t][j], acc.t[t], 0, 0, 0);
  }
}

template <int P, int NT>
__device__ __forceinline__ void stage(const Mat<NT>& m, const Lane& L, float* S) {
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) S[L.row(i) * P + L.col(j)] = m.t[j][i];
}

template <int P, int NT>
__device__ __forceinline__ Mat<NT> from_slot(const Lane& L, const float* S) {
  Mat<NT> m;
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) m.t[j][i] = S[L.row(i) * P + L.col(j)];
  return m;
}

template <int NT>
__device__ __forceinline__ void add(Mat<NT>& a, const Mat<NT>& b, float s) {
#pragma unroll
  for (int j = 0; j < NT; ++j) a.t[j] += s * b.t[j];
}

// Element-wise update with the element's (row, column).
template <int NT, typename F>
__device__ __forceinline__ void each(Mat<NT>& m, const Lane& L, const F& f) {
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = m.t[j][i];
      f(L.row(i), L.col(j), x);
      m.t[j][i] = x;
    }
}

// 64 rows of a [*, 128] bf16 tensor into a unit (rows >= valid are zeros):
// thread t copies 16 bytes of row t / 16.
__device__ __forceinline__ void load_b16(uint16_t* S, const bf16_t* src, int valid) {
  const int tid = threadIdx.x, r = tid >> 4, c0 = 8 * (tid & 15);
  uint4 x = {0u, 0u, 0u, 0u};
  if (r < valid) x = *reinterpret_cast<const uint4*>(src + r * kD + c0);
  *reinterpret_cast<uint4*>(S + r * kPh + c0) = x;
}

// 64 rows of a [*, 128] fp32 tensor into two units (rows >= valid are zeros).
__device__ __forceinline__ void load_f32d(float* S, const float* src, int valid) {
  const int tid = threadIdx.x, r = tid >> 4, c0 = 8 * (tid & 15);
  f4 a = f4{0.f, 0.f, 0.f, 0.f}, b = a;
  if (r < valid) {
    a = *reinterpret_cast<const f4*>(src + r * kD + c0);
    b = *reinterpret_cast<const f4*>(src + r * kD + c0 + 4);
  }
  *reinterpret_cast<f4*>(S + r * kPd + c0) = a;
  *reinterpret_cast<f4*>(S + r * kPd + c0 + 4) = b;
}

// The block's 64 x 64 fp32 M into a unit.
__device__ __forceinline__ void load_m(float* S, const float* src) {
  const int tid = threadIdx.x, r = tid >> 4, c0 = 4 * (tid & 15);
  *reinterpret_cast<f4*>(S + r * kPc + c0) = *reinterpret_cast<const f4*>(src + r * kC + c0);
}

// Rows < valid of an fp32 64 x 128 operand (two units) to bf16 rows of dst,
// rounded to nearest even; 16 bytes per thread.
__device__ __forceinline__ void store_rows(bf16_t* dst, const float* S, int valid) {
  const int tid = threadIdx.x, r = tid >> 4, c0 = 8 * (tid & 15);
  if (r >= valid) return;
  const f4 a = *reinterpret_cast<const f4*>(S + r * kPd + c0);
  const f4 b = *reinterpret_cast<const f4*>(S + r * kPd + c0 + 4);
  const auto pk = [](float x, float y) {
    return static_cast<uint32_t>(f32_to_bf16(x)) | (static_cast<uint32_t>(f32_to_bf16(y)) << 16);
  };
  *reinterpret_cast<uint4*>(dst + r * kD + c0) = uint4{pk(a[0], a[1]), pk(a[2], a[3]), pk(b[0], b[1]), pk(b[2], b[3])};
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

template <bool FOX>
__global__ __launch_bounds__(kNT) void bwd_block_ut128_kernel(
    int64_t L, int Nb, int64_t BH, float scale, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ w, const float* __restrict__ beta,
    const bf16_t* __restrict__ dO, const float* __restrict__ cum, const float* __restrict__ lse,
    const float* __restrict__ Dv, const float* __restrict__ minv, const float* __restrict__ dqh,
    const float* __restrict__ dkh, const float* __restrict__ dPacc, const float* __restrict__ dVacc,
    const float* __restrict__ rsum, const float* __restrict__ csum, bf16_t* __restrict__ dq,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, bf16_t* __restrict__ dw, float* __restrict__ dbeta,
    float* __restrict__ dc) {
  constexpr int C = kC, D = kD;
  __shared__ __attribute__((aligned(16))) char sm[9 * kUnit];
  __shared__ __attribute__((aligned(16))) float sb[C];
  __shared__ float slse[C], sD[C], scum[C], gB[C], rs[C], cs[C];
  float* const u0 = reinterpret_cast<float*>(sm);
  float* const u1 = reinterpret_cast<float*>(sm + kUnit);
  float* const u2 = reinterpret_cast<float*>(sm + 2 * kUnit);
  float* const u3 = reinterpret_cast<float*>(sm + 3 * kUnit);
  float* const u4 = reinterpret_cast<float*>(sm + 4 * kUnit);
  uint16_t* const pw = reinterpret_cast<uint16_t*>(sm + 5 * kUnit);
  uint16_t* const pk = reinterpret_cast<uint16_t*>(sm + 6 * kUnit);
  uint16_t* const pq = reinterpret_cast<uint16_t*>(sm + 7 * kUnit);
  float* const pm = reinterpret_cast<float*>(sm + 8 * kUnit);
  const B16 W{pw}, K{pk}, Q{pq};
  const F32<kPc> M{pm};

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

  // ---- inputs: W, K, Q (bf16) and M into LDS, the per-row scalars
  load_b16(pw, w + rb, valid);
  load_b16(pk, k + rb, valid);
  load_b16(pq, q + rb, valid);
  load_m(pm, Mg);
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
  MatC N = zero<1>(), Z = zero<1>(), Ut = zero<1>(), Sd = zero<1>();
  MatD F = zero<2>();
  mm<kRow, kBTr, D>(N, Ln, W, W, sb);   // G = W W^T
  each(N, Ln, [&](int r, int c, float& x) { x = c > r ? x : 0.f; });
  mm<kRow, kBTr, D>(Z, Ln, K, W, sb);   // K W^T
  each(Z, Ln, [&](int r, int c, float& x) { x = c > r ? x : 0.f; });
  mm<kRow, kBTr, D>(Ut, Ln, W, Q, sb);  // W Q^T
  each(Ut, Ln, [&](int r, int c, float& x) { x = c >= r ? x : 0.f; });
  mm<kRow, kBTr, D>(Sd, Ln, K, Q, sb);  // K Q^T
  mm<kCol, kBCol, C>(F, Ln, M, W, sb);  // M^T W, then F = diag(beta) M^T W
  each(F, Ln, [&](int r, int, float& x) { x *= sb[r]; });

  stage<kPc>(Z, Ln, u0);
  __syncthreads();
  MatC Y = zero<1>();
  mm<kRow, kBCol, C>(Y, Ln, F32<kPc>{u0}, M, sb);  // Z M, then Y = Z M diag(beta)
  each(Y, Ln, [&](int, int c, float& x) { x *= sb[c]; });

  __syncthreads();
  stage<kPc>(Y, Ln, u1);
  stage<kPc>(Ut, Ln, u2);
  __syncthreads();
  const F32<kPc> Ys{u1}, Uts{u2};
  {
    MatC yu = zero<1>();
    mm<kRow, kBCol, C>(yu, Ln, Ys, Uts, sb);  // Y Ut
    add(Sd, yu, -1.f);
    each(Sd, Ln, [&](int r, int c, float& x) { x = c >= r ? x : 0.f; });  // S^T[c][r], c <= r
  }

  // ---- in-block attention: p, dS, the value gradient
  __syncthreads();
  load_b16(reinterpret_cast<uint16_t*>(u3), v + rb, valid);
  load_b16(reinterpret_cast<uint16_t*>(u0), dO + rb, valid);
  __syncthreads();
  const B16 dOs{reinterpret_cast<const uint16_t*>(u0)};
  MatC Pm = zero<1>(), Sb = zero<1>();
  {
    MatC pd = zero<1>();
    mm<kRow, kBTr, D>(pd, Ln, B16{reinterpret_cast<const uint16_t*>(u3)}, dOs, sb);  // PD[c][r] = v_c . dO_r
    float csum_l[4] = {0.f, 0.f, 0.f, 0.f};
    float rsum_l = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = Ln.row(i), r = Ln.col(0);
      const bool act = c <= r && r < valid;
      const float sv = scale * Sd.t[0][i] + (FOX ? scum[r] - scum[c] : 0.f);
      const float p = act ? expf(sv - slse[r]) : 0.f;
      const float ds = act ? p * (pd.t[0][i] - sD[r]) : 0.f;
      Pm.t[0][i] = p;
      Sb.t[0][i] = scale * ds;
      if (FOX && c < r) {
        csum_l[i] += ds;  // key c, summed over queries r > c
        rsum_l += ds;     // query r, summed over keys c < r
      }
    }
    if (FOX) {
      // key sums over this wave's 16 columns, query sums over its 16 rows
      // (4 in-lane x 4 lane rows), then across waves
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = sum16(csum_l[i]);
        if (Ln.lr == 0) atomicAdd(&cs[Ln.row(i)], s);
      }
      const float s = sum4rows(rsum_l);
      if (Ln.lk == 0) atomicAdd(&rs[Ln.col(0)], s);
    }
  }
  __syncthreads();
  stage<kPc>(Pm, Ln, u3);
  __syncthreads();
  {
    MatD dvm = zero<2>();
    mm<kRow, kBCol, C>(dvm, Ln, F32<kPc>{u3}, dOs, sb);  // dv_c = sum_r p[r][c] dO_r
    each(dvm, Ln, [&](int c, int e, float& x) {
      if (c < valid) store_f32(dv + rb + c * D + e, x + dVacc[rb + c * D + e]);
    });
  }

  // ---- gradients
  __syncthreads();
  stage<kPc>(Sb, Ln, u0);
  load_f32d(u3, dkh + rb, valid);  // units 3, 4
  __syncthreads();
  const F32<kPc> Sbs{u0};
  const F32<kPd> Khs{u3};
  MatD Kb = from_slot<kPd, 2>(Ln, u3), Qb = zero<2>(), Wb = zero<2>();
  MatC Yb = zero<1>(), Utb = zero<1>();
  mm<kRow, kBCol, C>(Kb, Ln, Sbs, Q, sb);    // + S' Q
  mm<kCol, kBCol, C>(Qb, Ln, Sbs, K, sb);    // S'^T K
  mm<kRow, kBTr, C>(Yb, Ln, Sbs, Uts, sb);   // S' Ut^T
  mm<kRow, kBTr, D>(Yb, Ln, Khs, W, sb);     // + Khat' W^T   (Y' is the negation)
  mm<kCol, kBCol, C>(Wb, Ln, Ys, Khs, sb);   // Y^T Khat'     (subtracted from W')
  mm<kCol, kBCol, C>(Utb, Ln, Ys, Sbs, sb);  // Y^T S'        (subtracted from Ut')
  Yb.t[0] = -Yb.t[0];
  Wb.t[0] = -Wb.t[0];
  Wb.t[1] = -Wb.t[1];
  Utb.t[0] = -Utb.t[0];

  __syncthreads();
  stage<kPd>(F, Ln, u0);           // units 0, 1
  load_f32d(u3, dqh + rb, valid);  // units 3, 4
  __syncthreads();
  const F32<kPd> Fs{u0}, Qhs{u3};
  add(Qb, from_slot<kPd, 2>(Ln, u3), 1.f);
  MatD Fb = zero<2>(), t3 = zero<2>();
  {
    MatC t1 = zero<1>();
    mm<kRow, kBTr, D>(t1, Ln, Fs, Qhs, sb);  // F Qhat'^T
    add(Utb, t1, -1.f);
  }
  mm<kRow, kBCol, C>(Fb, Ln, Uts, Qhs, sb);  // Ut Qhat'
  // dP_n in two halves of 64 rows (units 2, 3): row half h holds P'[64h + e][*]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
    load_f32d(u2, dPg + h * 64 * D, 64);
    __syncthreads();
    {
      // + W P'^T on this wave's column tile in half h (columns 64h .. 64h + 63)
      MatC f1;
      f1.t[0] = Fb.t[h];
      Lane Lh = Ln;
      Lh.ch += 4 * h;
      mm<kRow, kBTr, D>(f1, Lh, W, F32<kPd>{u2 - 64 * h * kPd}, sb);
      Fb.t[h] = f1.t[0];
    }
    mm<kRow, kBCol, C>(t3, Ln, F32<kPd>{u0 + 64 * h}, F32<kPd>{u2}, sb);  // F P' over reduction rows of half h
  }
  add(Wb, t3, -1.f);
  Fb.t[0] = -Fb.t[0];
  Fb.t[1] = -Fb.t[1];
  each(Utb, Ln, [&](int r, int c, float& x) { x = c >= r ? x : 0.f; });  // U' = upper(Ut')

  __syncthreads();
  stage<kPd>(Fb, Ln, u0);  // units 0, 1
  stage<kPc>(Utb, Ln, u2);
  stage<kPc>(Yb, Ln, u3);
  stage<kPc>(Z, Ln, u4);
  __syncthreads();
  const F32<kPd> Fbs{u0};
  const F32<kPc> Ubs{u2}, Ybs{u3}, Zs{u4};
  MatC Xb = zero<1>(), Zb = zero<1>();
  mm<kRow, kBCol, C>(Wb, Ln, Ubs, Q, sb);        // + U' Q
  mm<kCol, kBCol, C>(Qb, Ln, Ubs, W, sb);        // + U'^T W
  mm<kRow, kBTr, D>(Xb, Ln, W, Fbs, sb);         // W F'^T
  mm<kCol, kBCol, C>(Xb, Ln, Zs, Ybs, sb);       // + Z^T Y'
  mm<kRow, kBCol, C, true>(Wb, Ln, M, Fbs, sb);  // + X F'   (X = M diag(beta))
  mm<kRow, kBTr, C, true>(Zb, Ln, Ybs, M, sb);   // Z' = Y' X^T
  each(Zb, Ln, [&](int r, int c, float& x) { x = c > r ? x : 0.f; });

  __syncthreads();
  stage<kPc>(Zb, Ln, u0);
  stage<kPc>(Xb, Ln, u1);
  __syncthreads();
  const F32<kPc> Zbs{u0}, Xbs{u1};
  mm<kRow, kBCol, C>(Kb, Ln, Zbs, W, sb);  // + Zm' W
  mm<kCol, kBCol, C>(Wb, Ln, Zbs, K, sb);  // + Zm'^T K
  {
    // beta'_j += sum_i M[i][j] X'[i][j]: this wave's 16 rows, then across waves
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += pm[Ln.row(i) * kPc + Ln.col(0)] * Xb.t[0][i];
    s = sum4rows(s);
    if (Ln.lk == 0) atomicAdd(&gB[Ln.col(0)], s);
  }
  MatC R = zero<1>();
  mm<kRow, kBTr, C, true>(R, Ln, Xbs, M, sb);  // R = X' X^T

  __syncthreads();
  stage<kPc>(R, Ln, u2);
  __syncthreads();
  MatC Tb = zero<1>();
  mm<kCol, kBCol, C>(Tb, Ln, M, F32<kPc>{u2}, sb);  // M^T R; T' = -M^T R
  {
    // beta'_a += sum_b T'[a][b] N[a][b]: this wave's 16 columns, then across waves
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = sum16(-Tb.t[0][i] * N.t[0][i]);
    if (Ln.lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&gB[Ln.row(i)], s[i]);
    }
  }
  each(Tb, Ln, [&](int r, int c, float& x) { x = c > r ? -sb[r] * x : 0.f; });  // G' = strict_upper(diag(beta) T')

  __syncthreads();
  stage<kPc>(Tb, Ln, u3);
  __syncthreads();
  mm<kRow, kBCol, C>(Wb, Ln, F32<kPc>{u3}, W, sb);  // + G' W
  mm<kCol, kBCol, C>(Wb, Ln, F32<kPc>{u3}, W, sb);  // + G'^T W

  // ---- outputs (rows through LDS; W is dead, so dW takes units 4 and 5)
  __syncthreads();
  stage<kPd>(Qb, Ln, u0);
  stage<kPd>(Kb, Ln, u2);
  stage<kPd>(Wb, Ln, u4);
  __syncthreads();
  store_rows(dq + rb, u0, valid);
  store_rows(dk + rb, u2, valid);
  store_rows(dw + rb, u4, valid);
  if (tid < valid) {
    dbeta[hb + t0 + tid] = gB[tid];
    if (FOX) dc[hb + t0 + tid] = rsum[hb + t0 + tid] + rs[tid] - csum[hb + t0 + tid] - cs[tid];
  }
}

template <bool FOX>
static hipError_t launch_ut128_t(const BwdBlockArgs& a, hipStream_t stream) {
  const int Nb = static_cast<int>((a.L + kBlk - 1) / kBlk);
  hipLaunchKernelGGL((bwd_block_ut128_kernel<FOX>), dim3(static_cast<unsigned>(a.BH * Nb)), dim3(kNT), 0, stream,
                     a.L, Nb, a.BH, a.scale, static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                     static_cast<const bf16_t*>(a.v), static_cast<const bf16_t*>(a.w), a.beta,
                     static_cast<const bf16_t*>(a.dO), a.cum, a.lse, a.Dv, a.minv, a.dqh, a.dkh, a.dP, a.dV, a.rsum,
                     a.csum, static_cast<bf16_t*>(a.dq), static_cast<bf16_t*>(a.dk), static_cast<bf16_t*>(a.dv),
                     static_cast<bf16_t*>(a.dw), a.dbeta, a.dc);
  return hipGetLastError();
}

hipError_t launch_bwd_block_ut128(const BwdBlockArgs& a, hipStream_t stream) {
  return a.cum != nullptr ? launch_ut128_t<true>(a, stream) : launch_ut128_t<false>(a, stream);
}

}  // namespace path
