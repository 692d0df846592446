// Cross-block part of the PaTH backward for bf16 storage at head dimension 64,
// on the 16-bit matrix cores.
//
// The mathematics is that of bwd_pair_kernel (bwd.hip).  The forward [PaTH
// Attention summary (gist.science 2505.16381), §3 "Algoritmo Estilo
// FlashAttention"] gives, for query i of block m and key j of block n < m,
//     s_ij = scale khat_j . Qt_i^(n) + c_i - c_j,
//     Qt^(m-1) = Qhat_m,   Qt^(n-1) = P_n Qt^(n),
// and one workgroup per query block m runs
//   pass 1, right to left: Qt^(n) for n = m-1 .. 0, into a scratch buffer;
//   pass 2, left to right: p = exp(s - lse_i), dS = p (dO_i . v_j - D_i),
//       Lam^(n) = P_n^T Lam^(n-1) + scale Khat_n^T dS_n   (Lam^(-1) = 0),
//     with dV_n += p dO, dKhat_n += scale dS Qt^(n) and dP_n += Lam^(n-1) Qt^(n)^T
//     summed over query blocks by fp32 atomics; Lam^(m-1) is the gradient
//     reaching Qhat_m.
//
// Products are 16x16x32 bf16 MFMAs with fp32 accumulation.  An fp32 operand x
// is split into hi = bf16(x) and lo = bf16(x - hi), 16 significant bits in all;
// a product of two split operands takes lo*hi + hi*lo + hi*hi, one against a
// stored bf16 operand (v, dO) lo*x + hi*x, and V dO^T a single pass.  bf16 has
// fp32's exponent range, so no operand needs scaling.
//
// Wave w owns output rows 16w .. 16w+15 of every product: lane (g, l) of its
// accumulators holds rows 16w + 4g + r (r < 4) of column l of each 16-column
// tile.  A operands are the wave's own rows:
//   * Khat_n, Khat_n^T, P_n and P_n^T as split bf16 rows (written by the
//     backward's fp32 prepare, columns in perm32 order), fetched from global
//     memory one block ahead, right after their last use; the value rows
//     straight from v;
//   * p, scale dS and Lam, whose accumulators hold 4 consecutive rows of one
//     column per lane.  A 16x16x16 MFMA against the identity transposes each
//     16x16 tile in registers (exact: every product is by 1 or 0), leaving 4
//     consecutive columns of one row, the A layout of a 16-wide slice.
// B operands are whole 64x64 matrices in LDS as rows of 128 bytes, 16-byte
// chunk k of row r at slot k ^ (r & 7): Qt by query rows and by head-dim rows,
// dO both ways, scale dS and Lam by query rows.  80 KB: two workgroups per CU.
// Along a reduction index, a lane's 8 values of a 32-wide slice are rows
// 4g .. 4g+3 of two consecutive accumulator tiles, so every matrix read along
// a reduction index keeps index k at position perm32(k).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace path {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;         // tokens per block
constexpr int kD = 64;         // head dimension
constexpr int kNT = 256;       // four waves
constexpr int kMat = kC * kD;  // elements of a 64 x 64 matrix
constexpr int kRow = 128;      // bytes per LDS row (64 bf16)
constexpr float kLog2eF = 1.4426950408889634f;

// Position of reduction index k within its row (k = 32c + 16h + 4g + r sits at
// 32c + 8g + 4h + r), and its inverse.
__host__ __device__ constexpr int perm32(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}
__host__ __device__ constexpr int unperm32(int p) {
  return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}
static_assert(unperm32(perm32(45)) == 45 && perm32(unperm32(45)) == 45, "perm32 inverse");

__device__ __forceinline__ f4 mma32(const bf8& a, const bf8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A (16 x 16) times B (16 x 16), both bf16: lane (g, l) gives A[l][4g + r] and
// B[4g + r][l] and receives D[4g + r][l].
__device__ __forceinline__ f4 mma16(const bf4& a, const bf4& b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b),
                                                    f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

__device__ __forceinline__ bf4 to_bf4(const f4& x) {
  const bf2 a = __builtin_convertvector(f2{x[0], x[1]}, bf2);
  const bf2 b = __builtin_convertvector(f2{x[2], x[3]}, bf2);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3);
}
__device__ __forceinline__ f4 to_f4(const bf4& h) {
  return f4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]),
            static_cast<float>(h[3])};
}
struct Split4 {
  bf4 hi, lo;
};
__device__ __forceinline__ Split4 split4(const f4& x) {
  Split4 s;
  s.hi = to_bf4(x);
  s.lo = to_bf4(x - to_f4(s.hi));
  return s;
}
__device__ __forceinline__ bf8 cat8(const bf4& a, const bf4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The accumulator tile of lane (g, l) (rows 4g + r, column l) transposed: the
// lane receives row l, columns 4g + r of the tile, in bf16 (exact).
__device__ __forceinline__ bf4 transpose4(const bf4& x, const bf4& ident) { return to_bf4(mma16(x, ident)); }

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kRow + ((chunk ^ (row & 7)) << 4); }
__device__ __forceinline__ bf8 rd8(const uint8_t* m, int row, int chunk) {
  return *reinterpret_cast<const bf8*>(m + lds_off(row, chunk));
}
// 4 values at positions pos .. pos + 3 of a row (pos a multiple of 4)
__device__ __forceinline__ void wr4(uint8_t* m, int row, int pos, const bf4& x) {
  *reinterpret_cast<bf4*>(m + lds_off(row, pos >> 3) + ((pos & 4) << 1)) = x;
}

// A operand rows of a packed split matrix (hi matrix, then lo): row `row`,
// slices c = 0, 1, lane group g.
struct SplitRows {
  bf8 hi[2], lo[2];
};
__device__ __forceinline__ void load_rows(const __bf16* mat, int row, int g, SplitRows& f) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    f.hi[c] = *reinterpret_cast<const bf8*>(mat + row * kD + 32 * c + 8 * g);
    f.lo[c] = *reinterpret_cast<const bf8*>(mat + kMat + row * kD + 32 * c + 8 * g);
  }
}

// Sum over the 16 lanes of a row (DPP moves; the same bits in every lane).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x + dpp<0x140>(x);
}

// Packed matrices of a key block, each a hi matrix followed by its lo matrix:
// Khat rows j (columns e), Khat^T rows a (columns j), P_n rows a (columns b),
// P_n^T rows a (columns b), columns in perm32 order.
enum : int { kKh = 0, kKt = 2, kPa = 4, kPt = 6, kPacked = 8 };

}  // namespace

template <bool FOX>
__global__ __launch_bounds__(kNT, 2) void bwd_pair16_kernel(
    int64_t L, int Nb, int64_t BH, float scale, const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
    const float* __restrict__ qhat, const __bf16* __restrict__ packed, const float* __restrict__ cum,
    const float* __restrict__ lse, const float* __restrict__ Dv, float* __restrict__ qt_scratch,
    float* __restrict__ dqh, float* __restrict__ rsum, float* __restrict__ dPacc) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[9 * kC * kRow];
  uint8_t* const QAh = sm;                // Qt by query rows: row i, column a at perm32(a)
  uint8_t* const QAl = sm + 1 * kC * kRow;
  uint8_t* const QBh = sm + 2 * kC * kRow;  // Qt by head-dim rows: row a, column i at perm32(i)
  uint8_t* const QBl = sm + 3 * kC * kRow;
  uint8_t* const XBh = sm + 4 * kC * kRow;  // scale dS by query rows: row i, column j at perm32(j)
  uint8_t* const XBl = sm + 5 * kC * kRow;
  uint8_t* const LBh = sm + 6 * kC * kRow;  // Lam by query rows: row i, column a at perm32(a)
  uint8_t* const LBl = sm + 7 * kC * kRow;
  uint8_t* const DOq = sm + 8 * kC * kRow;  // dO by query rows, columns in order

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l = lane & 15;
  const int m = Nb - 1 - static_cast<int>(blockIdx.x / BH);  // longest query blocks first
  const int64_t bh = blockIdx.x % BH;
  const int64_t i0 = static_cast<int64_t>(m) * kC;
  const int valid = static_cast<int>(L - i0 < kC ? L - i0 : kC);
  const int64_t hb = bh * L;

  if (m == 0) {  // no earlier key blocks: nothing reaches this block's qhat
    for (int idx = tid; idx < valid * kD; idx += kNT) dqh[(hb + i0) * kD + idx] = 0.f;
    if (FOX && tid < valid) rsum[hb + i0 + tid] = 0.f;
    return;
  }

  const int own = 16 * w + l;                             // this lane's A-operand row
  const int apos = 32 * (w >> 1) + 8 * g + 4 * (w & 1);  // perm32 of accumulator rows 16w + 4g .. + 3
  bf4 ident;                                              // B of the transposing product
#pragma unroll
  for (int r = 0; r < 4; ++r) ident[r] = static_cast<__bf16>(4 * g + r == l ? 1.f : 0.f);

  // dO of the query block (rows past the sequence end are zero)
  for (int idx = tid; idx < kC * 8; idx += kNT) {
    const int i = idx >> 3, ch = idx & 7;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (i < valid) val = *reinterpret_cast<const uint4*>(dO + (hb + i0 + i) * kD + 8 * ch);
    *reinterpret_cast<uint4*>(DOq + lds_off(i, ch)) = val;
  }
  // per-query terms of this lane's columns i = 16t + l
  float lse_i[4], d_i[4], c_i[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = 16 * t + l;
    const bool ok = i < valid;
    lse_i[t] = ok ? lse[hb + i0 + i] : 0.f;
    d_i[t] = ok ? Dv[hb + i0 + i] : 0.f;
    c_i[t] = (FOX && ok) ? cum[hb + i0 + i] : 0.f;
  }

  const int64_t npairs = static_cast<int64_t>(Nb) * (Nb - 1) / 2;
  float* const scr = qt_scratch + (bh * npairs + static_cast<int64_t>(m) * (m - 1) / 2) * kMat;
  // Qt^(n) in the accumulator layout of the transport: each wave keeps its own rows
  const auto slot = [&](int n, int t) { return scr + static_cast<int64_t>(n) * kMat + ((w * 4 + t) * 64 + lane) * 4; };
  const __bf16* const pk = packed + bh * Nb * static_cast<int64_t>(kPacked * kMat);
  const auto mat = [&](int n, int which) { return pk + (static_cast<int64_t>(n) * kPacked + which) * kMat; };

  // ---- pass 1: Qt^(n), n = m-1 .. 0.  The state qs[t] holds Qt[i = 16t + l][a = 16w + 4g + r].
  f4 qs[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = 16 * t + l;
    qs[t] = i < valid ? *reinterpret_cast<const f4*>(qhat + (hb + i0 + i) * kD + 16 * w + 4 * g)
                      : f4{0.f, 0.f, 0.f, 0.f};
  }
  {
    SplitRows pa;
    if (m >= 2) load_rows(mat(m - 1, kPa), own, g, pa);
    for (int n = m - 1;; --n) {
#pragma unroll
      for (int t = 0; t < 4; ++t) *reinterpret_cast<f4*>(slot(n, t)) = qs[t];
      if (n == 0) break;
      // two staging buffers in turn: one barrier per step
      uint8_t* const sh = (n & 1) ? QAh : QBh;
      uint8_t* const sl = (n & 1) ? QAl : QBl;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const Split4 s = split4(qs[t]);
        wr4(sh, 16 * t + l, apos, s.hi);
        wr4(sl, 16 * t + l, apos, s.lo);
      }
      __syncthreads();
      f4 acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf8 bhv = rd8(sh, 16 * t + l, 4 * c + g), blv = rd8(sl, 16 * t + l, 4 * c + g);
          acc[t] = mma32(pa.lo[c], bhv, acc[t]);
          acc[t] = mma32(pa.hi[c], blv, acc[t]);
          acc[t] = mma32(pa.hi[c], bhv, acc[t]);
        }
      if (n >= 2) load_rows(mat(n - 1, kPa), own, g, pa);
#pragma unroll
      for (int t = 0; t < 4; ++t) qs[t] = acc[t];
    }
  }
  __syncthreads();  // the last transport's operand reads are done

  // ---- pass 2: key blocks left to right
  SplitRows kh, kt, pt;
  bf8 vf[2];
  float c_j[4] = {0.f, 0.f, 0.f, 0.f};  // gate prefix of keys j = 16w + 4g + r
  const auto load_key = [&](int n) {
    load_rows(mat(n, kKh), own, g, kh);
    const __bf16* vb = v + (hb + static_cast<int64_t>(n) * kC + own) * kD;
    vf[0] = *reinterpret_cast<const bf8*>(vb + 8 * g);
    vf[1] = *reinterpret_cast<const bf8*>(vb + 32 + 8 * g);
  };
  const auto load_adj = [&](int n) {
    load_rows(mat(n, kKt), own, g, kt);
    load_rows(mat(n, kPt), own, g, pt);
    if (FOX) {
      const float* cj = cum + hb + static_cast<int64_t>(n) * kC + 16 * w + 4 * g;  // rows of length L: no alignment
#pragma unroll
      for (int r = 0; r < 4; ++r) c_j[r] = cj[r];
    }
  };
  f4 qn[4], lam[4];
  float csm[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's share of sum_j dS[j][i], i = 16t + l
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    qn[t] = *reinterpret_cast<const f4*>(slot(0, t));
    lam[t] = f4{0.f, 0.f, 0.f, 0.f};
  }
  load_key(0);
  load_adj(0);

  for (int n = 0; n < m; ++n) {
    // Qt^(n) by query rows (QA) and, transposed in registers, by head-dim rows (QB)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const Split4 s = split4(qn[t]);
      wr4(QAh, 16 * t + l, apos, s.hi);
      wr4(QAl, 16 * t + l, apos, s.lo);
      const int ipos = 32 * (t >> 1) + 8 * g + 4 * (t & 1);  // perm32 of i = 16t + 4g .. + 3
      wr4(QBh, own, ipos, transpose4(s.hi, ident));
      wr4(QBl, own, ipos, transpose4(s.lo, ident));
    }
    if (n + 1 < m) {
#pragma unroll
      for (int t = 0; t < 4; ++t) qn[t] = *reinterpret_cast<const f4*>(slot(n + 1, t));
    }
    __syncthreads();  // Qt staged, Lam^(n-1) (written at the end of the last step) in LB

    // S = Khat_n Qt^T and dO . v, rows j of this wave's tile
    f4 s[4], pd[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = pd[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf8 bhv = rd8(QAh, 16 * t + l, 4 * c + g), blv = rd8(QAl, 16 * t + l, 4 * c + g);
        const bf8 bd = rd8(DOq, 16 * t + l, 4 * c + g);
        s[t] = mma32(kh.lo[c], bhv, s[t]);
        s[t] = mma32(kh.hi[c], blv, s[t]);
        s[t] = mma32(kh.hi[c], bhv, s[t]);
        pd[t] = mma32(vf[c], bd, pd[t]);
      }
    if (n + 1 < m) load_key(n + 1);

    // scale dS (row j = 16w + 4g + r, column i = 16t + l) by query rows, for the adjoint update
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool ok = 16 * t + l < valid;
      f4 dss;
      float colp = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = scale * s[t][r] + (FOX ? c_i[t] - c_j[r] : 0.f) - lse_i[t];
        const float p = ok ? __builtin_amdgcn_exp2f(x * kLog2eF) : 0.f;
        const float ds = p * (pd[t][r] - d_i[t]);
        dss[r] = scale * ds;
        colp += ds;
      }
      if (FOX) csm[t] += colp;
      const Split4 dsp = split4(dss);
      wr4(XBh, 16 * t + l, apos, dsp.hi);
      wr4(XBl, 16 * t + l, apos, dsp.lo);
    }

    // dP_n += Lam^(n-1) Qt^(n)^T (Lam^(n-1) transposed to rows a of this wave's tile)
    if (n >= 1) {
      bf4 tlh[4], tll[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const Split4 ls = split4(lam[t]);
        tlh[t] = transpose4(ls.hi, ident);
        tll[t] = transpose4(ls.lo, ident);
      }
      f4 dp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) dp[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf8 lh = cat8(tlh[2 * c], tlh[2 * c + 1]), ll = cat8(tll[2 * c], tll[2 * c + 1]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf8 bhv = rd8(QBh, 16 * u + l, 4 * c + g), blv = rd8(QBl, 16 * u + l, 4 * c + g);
          dp[u] = mma32(ll, bhv, dp[u]);
          dp[u] = mma32(lh, blv, dp[u]);
          dp[u] = mma32(lh, bhv, dp[u]);
        }
      }
      float* dstp = dPacc + ((bh * Nb + n) * kD + 16 * w + 4 * g) * kD + l;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) unsafeAtomicAdd(dstp + r * kD + 16 * u, dp[u][r]);
    }
    __syncthreads();  // every wave's scale dS rows are in XB

    // Lam^(n) = P_n^T Lam^(n-1) + Khat_n^T (scale dS), rows a of this wave's tile
    {
      f4 acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (n >= 1) {
            const bf8 lh = rd8(LBh, 16 * t + l, 4 * c + g), ll = rd8(LBl, 16 * t + l, 4 * c + g);
            acc[t] = mma32(pt.lo[c], lh, acc[t]);
            acc[t] = mma32(pt.hi[c], ll, acc[t]);
            acc[t] = mma32(pt.hi[c], lh, acc[t]);
          }
          const bf8 xh = rd8(XBh, 16 * t + l, 4 * c + g), xl = rd8(XBl, 16 * t + l, 4 * c + g);
          acc[t] = mma32(kt.lo[c], xh, acc[t]);
          acc[t] = mma32(kt.hi[c], xl, acc[t]);
          acc[t] = mma32(kt.hi[c], xh, acc[t]);
        }
#pragma unroll
      for (int t = 0; t < 4; ++t) lam[t] = acc[t];
    }
    if (n + 1 < m) load_adj(n + 1);
    __syncthreads();  // every wave is done with LB, XB and the Qt tiles
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const Split4 ls = split4(lam[t]);
      wr4(LBh, 16 * t + l, apos, ls.hi);
      wr4(LBl, 16 * t + l, apos, ls.lo);
    }
  }

  // lam[t] holds Lam^(m-1)[a = 16w + 4g + r][i = 16t + l]: the gradient reaching qhat
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = 16 * t + l;
    if (i < valid) *reinterpret_cast<f4*>(dqh + (hb + i0 + i) * kD + 16 * w + 4 * g) = lam[t];
  }
  if (FOX) {
    float* red = reinterpret_cast<float*>(XBh);  // no longer read
    if (tid < kC) red[tid] = 0.f;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) atomicAdd(&red[16 * t + l], csm[t]);
    __syncthreads();
    if (tid < valid) rsum[hb + i0 + tid] = red[tid];
  }
}

// Key-side sums: one workgroup per key block n (every block but a head's last),
// for the query blocks m = n+1 .. Nb-1 in turn:
//     dV_n = sum_m p^T dO_m,   dKhat_n = scale sum_m dS^T Qt^(n)_m,
//     and with gates the sums over queries of dS_ij for every key j,
// accumulated in registers and stored once, with no atomics.  Qt^(n)_m is
// read from the query-major kernel's scratch buffer (each wave reads the rows
// the same wave index wrote there); p and dS are formed from it exactly as in
// that kernel.
template <bool FOX>
__global__ __launch_bounds__(kNT, FOX ? 2 : 3) void bwd_key16_kernel(
    int64_t L, int Nb, int64_t BH, float scale, const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
    const __bf16* __restrict__ packed, const float* __restrict__ cum, const float* __restrict__ lse,
    const float* __restrict__ Dv, const float* __restrict__ qt_scratch, float* __restrict__ dkh,
    float* __restrict__ dVacc, float* __restrict__ csum) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[6 * kC * kRow];
  uint8_t* const QAh = sm;                  // Qt by query rows: row i, column a at perm32(a)
  uint8_t* const QAl = sm + 1 * kC * kRow;
  uint8_t* const QBh = sm + 2 * kC * kRow;  // Qt by head-dim rows: row a, column i at perm32(i)
  uint8_t* const QBl = sm + 3 * kC * kRow;
  uint8_t* const DOq = sm + 4 * kC * kRow;  // dO by query rows, columns in order
  uint8_t* const DOe = sm + 5 * kC * kRow;  // dO by head-dim rows: row e, column i at perm32(i)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l = lane & 15;
  const int n = static_cast<int>(blockIdx.x / BH);  // key block 0 meets the most query blocks: first
  const int64_t bh = blockIdx.x % BH;
  const int64_t hb = bh * L;
  const int64_t j0 = static_cast<int64_t>(n) * kC;
  const int own = 16 * w + l;
  const int apos = 32 * (w >> 1) + 8 * g + 4 * (w & 1);
  bf4 ident;
#pragma unroll
  for (int r = 0; r < 4; ++r) ident[r] = static_cast<__bf16>(4 * g + r == l ? 1.f : 0.f);

  SplitRows kh;
  load_rows(packed + ((bh * Nb + n) * kPacked + kKh) * static_cast<int64_t>(kMat), own, g, kh);
  bf8 vf[2];
  {
    const __bf16* vb = v + (hb + j0 + own) * kD;  // block n < Nb - 1 is whole
    vf[0] = *reinterpret_cast<const bf8*>(vb + 8 * g);
    vf[1] = *reinterpret_cast<const bf8*>(vb + 32 + 8 * g);
  }
  float c_j[4] = {0.f, 0.f, 0.f, 0.f};
  if (FOX) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c_j[r] = cum[hb + j0 + 16 * w + 4 * g + r];
  }

  const int64_t npairs = static_cast<int64_t>(Nb) * (Nb - 1) / 2;
  // Qt^(n) of query block m in the transport's accumulator layout (rows of wave w)
  const auto slot = [&](int m, int t) {
    return qt_scratch + (bh * npairs + static_cast<int64_t>(m) * (m - 1) / 2 + n) * kMat +
           ((w * 4 + t) * 64 + lane) * 4;
  };
  // dO_m in the same layout: rows i = 16t + l, columns 16w + 4g .. + 3 (zero past the end)
  const auto load_do = [&](int m, bf4 (&x)[4]) {
    const int64_t i0 = static_cast<int64_t>(m) * kC;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 16 * t + l;
      x[t] = i0 + i < L ? *reinterpret_cast<const bf4*>(dO + (hb + i0 + i) * kD + 16 * w + 4 * g)
                        : bf4{0, 0, 0, 0};
    }
  };

  f4 dv[4], dk[4], qn[4];
  bf4 dn[4];
  float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    dv[u] = dk[u] = f4{0.f, 0.f, 0.f, 0.f};
    qn[u] = *reinterpret_cast<const f4*>(slot(n + 1, u));
  }
  load_do(n + 1, dn);

  for (int m = n + 1; m < Nb; ++m) {
    const int64_t i0 = static_cast<int64_t>(m) * kC;
    const int valid = static_cast<int>(L - i0 < kC ? L - i0 : kC);
    // Qt^(n)_m and dO_m, each by query rows and (transposed in registers) by head-dim rows
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const Split4 sq = split4(qn[t]);
      wr4(QAh, 16 * t + l, apos, sq.hi);
      wr4(QAl, 16 * t + l, apos, sq.lo);
      const int ipos = 32 * (t >> 1) + 8 * g + 4 * (t & 1);
      wr4(QBh, own, ipos, transpose4(sq.hi, ident));
      wr4(QBl, own, ipos, transpose4(sq.lo, ident));
      wr4(DOq, 16 * t + l, 16 * w + 4 * g, dn[t]);
      wr4(DOe, own, ipos, transpose4(dn[t], ident));
    }
    float lse_i[4], d_i[4], c_i[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 16 * t + l;
      const bool ok = i < valid;
      lse_i[t] = ok ? lse[hb + i0 + i] : 0.f;
      d_i[t] = ok ? Dv[hb + i0 + i] : 0.f;
      c_i[t] = (FOX && ok) ? cum[hb + i0 + i] : 0.f;
    }
    if (m + 1 < Nb) {
#pragma unroll
      for (int t = 0; t < 4; ++t) qn[t] = *reinterpret_cast<const f4*>(slot(m + 1, t));
      load_do(m + 1, dn);
    }
    __syncthreads();  // Qt and dO staged

    f4 s[4], pd[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = pd[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf8 bhv = rd8(QAh, 16 * t + l, 4 * c + g), blv = rd8(QAl, 16 * t + l, 4 * c + g);
        const bf8 bd = rd8(DOq, 16 * t + l, 4 * c + g);
        s[t] = mma32(kh.lo[c], bhv, s[t]);
        s[t] = mma32(kh.hi[c], blv, s[t]);
        s[t] = mma32(kh.hi[c], bhv, s[t]);
        pd[t] = mma32(vf[c], bd, pd[t]);
      }
    // p and scale dS (row j = 16w + 4g + r, column i = 16t + l); p by rows j
    bf4 th[4], tl[4];
    Split4 dsp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool ok = 16 * t + l < valid;
      f4 pv, dss;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = scale * s[t][r] + (FOX ? c_i[t] - c_j[r] : 0.f) - lse_i[t];
        const float p = ok ? __builtin_amdgcn_exp2f(x * kLog2eF) : 0.f;
        const float ds = p * (pd[t][r] - d_i[t]);
        pv[r] = p;
        dss[r] = scale * ds;
        rowp[r] += ds;
      }
      const Split4 ps = split4(pv);
      th[t] = transpose4(ps.hi, ident);
      tl[t] = transpose4(ps.lo, ident);
      dsp[t] = split4(dss);
    }
    // dV_n += p dO_m
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf8 ph = cat8(th[2 * c], th[2 * c + 1]), pl = cat8(tl[2 * c], tl[2 * c + 1]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf8 bo = rd8(DOe, 16 * u + l, 4 * c + g);
        dv[u] = mma32(pl, bo, dv[u]);
        dv[u] = mma32(ph, bo, dv[u]);
      }
    }
    // scale dS by rows j; dKhat_n += scale dS Qt^(n)_m
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      th[t] = transpose4(dsp[t].hi, ident);
      tl[t] = transpose4(dsp[t].lo, ident);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf8 dh = cat8(th[2 * c], th[2 * c + 1]), dl = cat8(tl[2 * c], tl[2 * c + 1]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf8 bhv = rd8(QBh, 16 * u + l, 4 * c + g), blv = rd8(QBl, 16 * u + l, 4 * c + g);
        dk[u] = mma32(dl, bhv, dk[u]);
        dk[u] = mma32(dh, blv, dk[u]);
        dk[u] = mma32(dh, bhv, dk[u]);
      }
    }
    __syncthreads();  // every wave is done with this query block's tiles
  }

  // rows j = 16w + 4g + r, columns e = 16u + l
  float* dstv = dVacc + (hb + j0 + 16 * w + 4 * g) * kD + l;
  float* dstk = dkh + (hb + j0 + 16 * w + 4 * g) * kD + l;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dstv[r * kD + 16 * u] = dv[u][r];
      dstk[r * kD + 16 * u] = dk[u][r];
    }
  if (FOX) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rs = row16_sum(rowp[r]);
      if (l == 0) csum[hb + j0 + 16 * w + 4 * g + r] = rs;
    }
  }
}

hipError_t launch_bwd_pair16(const BwdArgs& a, hipStream_t stream) {
  const int64_t BH = a.BH, L = a.L;
  const int Nb = static_cast<int>((L + kC - 1) / kC);
  const __bf16* packed = static_cast<const __bf16*>(a.ws.packed);
  const dim3 grid(static_cast<unsigned>(BH * Nb));
  const __bf16* v = static_cast<const __bf16*>(a.v);
  const __bf16* dO = static_cast<const __bf16*>(a.dout);
  if (a.ws.cum) {
    hipLaunchKernelGGL(bwd_pair16_kernel<true>, grid, dim3(kNT), 0, stream, L, Nb, BH, a.scale, v, dO, a.ws.qhat,
                       packed, a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dqh, a.ws.rsum, a.ws.dP);
  } else {
    hipLaunchKernelGGL(bwd_pair16_kernel<false>, grid, dim3(kNT), 0, stream, L, Nb, BH, a.scale, v, dO, a.ws.qhat,
                       packed, a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dqh, a.ws.rsum, a.ws.dP);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || Nb < 2) return e;
  const dim3 kgrid(static_cast<unsigned>(BH * (Nb - 1)));
  if (a.ws.cum) {
    hipLaunchKernelGGL(bwd_key16_kernel<true>, kgrid, dim3(kNT), 0, stream, L, Nb, BH, a.scale, v, dO, packed,
                       a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dkh, a.ws.dV, a.ws.csum);
  } else {
    hipLaunchKernelGGL(bwd_key16_kernel<false>, kgrid, dim3(kNT), 0, stream, L, Nb, BH, a.scale, v, dO, packed,
                       a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dkh, a.ws.dV, a.ws.csum);
  }
  return hipGetLastError();
}

}  // namespace path
