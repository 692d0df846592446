// Cross-block part of the PaTH backward for bf16 storage, on the 16-bit matrix
// cores (head dimension D = 64 or 128).
//
// The mathematics is that of bwd_pair_kernel (bwd.hip).  The forward [PaTH
// Attention summary (gist.science 2505.16381), §3 "Algoritmo Estilo
// FlashAttention"] gives, for query i of block m and key j of block n < m,
//     s_ij = scale khat_j . Qt_i^(n) + c_i - c_j,
//     Qt^(m-1) = Qhat_m,   Qt^(n-1) = P_n Qt^(n),
// and the gradients need, with p = exp(s - lse_i) and dS = p (dO_i . v_j - D_i),
//     Lam^(n) = P_n^T Lam^(n-1) + scale Khat_n^T dS_n   (Lam^(-1) = 0),
//     dP_n += Lam^(n-1) Qt^(n)^T,  dV_n += p dO,  dKhat_n += scale dS Qt^(n),
// the last three summed over query blocks; Lam^(m-1) is the gradient reaching
// Qhat_m.  Three kernels:
//   bwd_transport16_kernel, one workgroup per group of kQG query blocks of a
//     head: right to left, Qt^(n) for n = m-1 .. 0 of every block m of the
//     group, into a scratch buffer; the group's blocks share each P_n fetch;
//   bwd_pair16_kernel, one workgroup per query block m: left to right, p, dS,
//     the adjoint Lam and dP_n (fp32 atomics);
//   bwd_key16_kernel, one workgroup per key block n: for m = n+1 .. Nb-1,
//     p and dS again from Qt^(n)_m in the scratch buffer, with dV_n, dKhat_n
//     and the gates' key sums in registers, stored once.
//
// Products are 16x16x32 bf16 MFMAs with fp32 accumulation.  An fp32 operand x
// is split into hi = bf16(x) and lo = bf16(x - hi), 16 significant bits in all;
// a product of two split operands takes lo*hi + hi*lo + hi*hi, one against a
// stored bf16 operand (v, dO) lo*x + hi*x, and V dO^T a single pass.  bf16 has
// fp32's exponent range, so no operand needs scaling.
//
// Each of the four waves owns output rows of every product: the 16 key rows
// 16w .. 16w+15 of the 64-row products, and the RT = D/64 head-dim row tiles
// RT w .. RT w + RT - 1 of the D-row ones.  Lane (g, l) of an accumulator tile
// holds rows 4g + r (r < 4) of column l.  A operands are the wave's own rows:
//   * Khat_n, Khat_n^T, P_n and P_n^T as split bf16 rows (written by the
//     backward's matrix-core prepare, columns in perm32 order), fetched from
//     global memory one block ahead, right after their last use; the value
//     rows straight from v;
//   * Lam, p and scale dS, whose accumulators hold 4 consecutive rows of one
//     column per lane.  A 16x16x16 MFMA against the identity transposes each
//     16x16 tile in registers (exact: every product is by 1 or 0), leaving 4
//     consecutive columns of one row, the A layout of a 16-wide slice.
// B operands are whole matrices in LDS as rows of W bf16 (W = 64 or D), the
// 16-byte chunk k of row r at slot k ^ (r & (W/8 - 1)): Qt by query rows and by
// head-dim rows, dO, scale dS and Lam by query rows.  72 KB at D = 64 (two
// workgroups per CU), 128 KB at D = 128 (one).  Along a reduction index, a
// lane's 8 values of a 32-wide slice are rows 4g .. 4g+3 of two consecutive
// accumulator tiles, so every matrix read along a reduction index keeps index
// k at position perm32(k).
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

constexpr int kC = 64;    // tokens per block
constexpr int kNT = 256;  // four waves
constexpr float kLog2eF = 1.4426950408889634f;

// Sizes at head dimension D.
template <int D>
struct Geo {
  static constexpr int RT = D / 64;   // head-dim row tiles per wave
  static constexpr int DK = D / 32;   // 32-wide reduction slices along the head dim
  static constexpr int DT = D / 16;   // 16-wide column tiles along the head dim
  static constexpr int QD = kC * D;   // elements of a 64 x D matrix
  // a key block's packed operands, each a hi matrix followed by its lo matrix:
  // Khat rows j (columns e), Khat^T rows a (columns j), P_n rows a (columns b),
  // P_n^T rows a (columns b), columns in perm32 order
  static constexpr int64_t kKh = 0, kKt = 2 * kC * D, kPa = 4 * kC * D, kPt = 4 * kC * D + 2 * D * D;
  static constexpr int64_t kBlock = 4 * kC * D + 4 * D * D;
};

// Position of reduction index k within its row (k = 32c + 16h + 4g + r sits at
// 32c + 8g + 4h + r), and its inverse.
__host__ __device__ constexpr int perm32(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}
__host__ __device__ constexpr int unperm32(int p) {
  return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}
static_assert(unperm32(perm32(45)) == 45 && perm32(unperm32(45)) == 45, "perm32 inverse");
// perm32 of rows 16T + 4g .. 16T + 4g + 3 of accumulator tile T
__device__ __forceinline__ int tile_pos(int T, int g) { return 32 * (T >> 1) + 8 * g + 4 * (T & 1); }

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

// LDS matrices with rows of W bf16.
template <int W>
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * (2 * W) + ((chunk ^ (row & (W / 8 - 1))) << 4);
}
template <int W>
__device__ __forceinline__ bf8 rd8(const uint8_t* m, int row, int chunk) {
  return *reinterpret_cast<const bf8*>(m + lds_off<W>(row, chunk));
}
// 4 values at positions pos .. pos + 3 of a row (pos a multiple of 4)
template <int W>
__device__ __forceinline__ void wr4(uint8_t* m, int row, int pos, const bf4& x) {
  *reinterpret_cast<bf4*>(m + lds_off<W>(row, pos >> 3) + ((pos & 4) << 1)) = x;
}

// A operand rows of a packed split matrix with rows of W elements (hi matrix,
// then lo): row `row`, slices c < W/32, lane group g.
template <int W>
struct SplitRows {
  bf8 hi[W / 32], lo[W / 32];
};
template <int W, int R>
__device__ __forceinline__ void load_rows(const __bf16* mat, int row, int g, SplitRows<W>& f) {
#pragma unroll
  for (int c = 0; c < W / 32; ++c) {
    f.hi[c] = *reinterpret_cast<const bf8*>(mat + row * W + 32 * c + 8 * g);
    f.lo[c] = *reinterpret_cast<const bf8*>(mat + R * W + row * W + 32 * c + 8 * g);
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

}  // namespace

// Scratch slot of Qt^(n)_m for the pair (m, n), n < m: the 64 x D fp32 matrix
// in the accumulator layout of wave w's tile h, query tile t (the query- and
// key-major kernels read back what the same wave index wrote).  The scratch
// is written and read with non-temporal accesses: each slot is read once per
// kernel, long after it was written, and kept out of the caches it leaves more
// room there for the key blocks' operands and the dP_n accumulators.
__device__ __forceinline__ int64_t pair_index(int64_t bh, int Nb, int m, int n) {
  return bh * (static_cast<int64_t>(Nb) * (Nb - 1) / 2) + static_cast<int64_t>(m) * (m - 1) / 2 + n;
}

constexpr int kQG = 4;  // query blocks per transport workgroup

template <int D>
__global__ __launch_bounds__(kNT, D == 64 ? 2 : 1) void bwd_transport16_kernel(
    int64_t L, int Nb, int64_t BH, const float* __restrict__ qhat, const __bf16* __restrict__ packed,
    float* __restrict__ qt_scratch) {
  using G = Geo<D>;
  constexpr int RT = G::RT, DK = G::DK, QD = G::QD;
  // per query block of the group: Qt by query rows, hi then lo (row i, column a at perm32(a)) [W = D]
  __shared__ __attribute__((aligned(16))) uint8_t sm[kQG * 4 * QD];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l = lane & 15;
  const int ngroups = (Nb - 1 + kQG - 1) / kQG;                      // groups of query blocks 1 .. Nb-1
  const int grp = ngroups - 1 - static_cast<int>(blockIdx.x / BH);   // longest first
  const int64_t bh = blockIdx.x % BH;
  const int mlo = 1 + kQG * grp;
  const int mhi = mlo + kQG - 1 < Nb - 1 ? mlo + kQG - 1 : Nb - 1;  // blocks mlo .. mhi
  const int64_t hb = bh * L;
  const __bf16* const pk = packed + bh * Nb * G::kBlock + G::kPa;
  const int64_t lane_off = ((w * RT) * 4 * 64 + lane) * 4;  // this lane's place in a slot (tile h, query tile t added below)

  // qs[q][h][t] holds Qt[i = 16t + l][a = 16(RT w + h) + 4g + r] of block mlo + q
  f4 qs[kQG][RT][4];
  SplitRows<D> pa[RT];
#pragma unroll
  for (int h = 0; h < RT; ++h) load_rows<D, D>(pk + static_cast<int64_t>(mhi - 1) * G::kBlock, 16 * (RT * w + h) + l, g, pa[h]);
  for (int n = mhi - 1;; --n) {
#pragma unroll
    for (int q = 0; q < kQG; ++q) {
      const int m = mlo + q;
      if (m > mhi || n > m - 1) continue;  // block not (yet) on the path
      if (n == m - 1) {  // Qt^(m-1) = Qhat_m (rows past the sequence end are zero)
        const int64_t i0 = static_cast<int64_t>(m) * kC;
        const int valid = static_cast<int>(L - i0 < kC ? L - i0 : kC);
#pragma unroll
        for (int h = 0; h < RT; ++h)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int i = 16 * t + l;
            qs[q][h][t] = i < valid ? *reinterpret_cast<const f4*>(qhat + (hb + i0 + i) * D + 16 * (RT * w + h) + 4 * g)
                                    : f4{0.f, 0.f, 0.f, 0.f};
          }
      }
      float* const slot = qt_scratch + pair_index(bh, Nb, m, n) * QD + lane_off;
#pragma unroll
      for (int h = 0; h < RT; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) __builtin_nontemporal_store(qs[q][h][t], reinterpret_cast<f4*>(slot + (h * 4 + t) * 256));
    }
    if (n == 0) break;
    // Qt^(n-1) = P_n Qt^(n) for every block on the path: stage, then multiply
#pragma unroll
    for (int q = 0; q < kQG; ++q) {
      if (mlo + q > mhi || n > mlo + q - 1) continue;
      uint8_t* const sh = sm + q * 4 * QD;
      uint8_t* const sl = sh + 2 * QD;
#pragma unroll
      for (int h = 0; h < RT; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const Split4 sp = split4(qs[q][h][t]);
          wr4<D>(sh, 16 * t + l, tile_pos(RT * w + h, g), sp.hi);
          wr4<D>(sl, 16 * t + l, tile_pos(RT * w + h, g), sp.lo);
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kQG; ++q) {
      if (mlo + q > mhi || n > mlo + q - 1) continue;
      const uint8_t* const sh = sm + q * 4 * QD;
      const uint8_t* const sl = sh + 2 * QD;
#pragma unroll
      for (int h = 0; h < RT; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) qs[q][h][t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DK; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf8 bhv = rd8<D>(sh, 16 * t + l, 4 * c + g), blv = rd8<D>(sl, 16 * t + l, 4 * c + g);
#pragma unroll
          for (int h = 0; h < RT; ++h) {
            qs[q][h][t] = mma32(pa[h].lo[c], bhv, qs[q][h][t]);
            qs[q][h][t] = mma32(pa[h].hi[c], blv, qs[q][h][t]);
            qs[q][h][t] = mma32(pa[h].hi[c], bhv, qs[q][h][t]);
          }
        }
    }
    if (n >= 2) {
#pragma unroll
      for (int h = 0; h < RT; ++h)
        load_rows<D, D>(pk + static_cast<int64_t>(n - 1) * G::kBlock, 16 * (RT * w + h) + l, g, pa[h]);
    }
    __syncthreads();  // the staged tiles are read before the next step overwrites them
  }
}

template <int D, bool FOX>
__global__ __launch_bounds__(kNT, D == 64 ? 2 : 1) void bwd_pair16_kernel(
    int64_t L, int Nb, int64_t BH, float scale, const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
    const __bf16* __restrict__ packed, const float* __restrict__ cum, const float* __restrict__ lse,
    const float* __restrict__ Dv, const float* __restrict__ qt_scratch, float* __restrict__ dqh,
    float* __restrict__ rsum, float* __restrict__ dPacc) {
  using G = Geo<D>;
  constexpr int RT = G::RT, DK = G::DK, DT = G::DT, QD = G::QD;
  // bytes: QA, QB, LB (hi and lo, 64 x D each), XB (hi and lo, 64 x 64), DOq (64 x D)
  __shared__ __attribute__((aligned(16))) uint8_t sm[14 * QD + 4 * kC * kC];
  uint8_t* const QAh = sm;                       // Qt by query rows: row i, column a at perm32(a) [W = D]
  uint8_t* const QAl = sm + 2 * QD;
  uint8_t* const QBh = sm + 4 * QD;              // Qt by head-dim rows: row a, column i at perm32(i) [W = 64]
  uint8_t* const QBl = sm + 6 * QD;
  uint8_t* const LBh = sm + 8 * QD;              // Lam by query rows: row i, column a at perm32(a) [W = D]
  uint8_t* const LBl = sm + 10 * QD;
  uint8_t* const XBh = sm + 12 * QD;             // scale dS by query rows: row i, column j at perm32(j) [W = 64]
  uint8_t* const XBl = XBh + 2 * kC * kC;
  uint8_t* const DOq = XBl + 2 * kC * kC;        // dO by query rows, columns in order [W = D]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l = lane & 15;
  const int m = Nb - 1 - static_cast<int>(blockIdx.x / BH);  // longest query blocks first
  const int64_t bh = blockIdx.x % BH;
  const int64_t i0 = static_cast<int64_t>(m) * kC;
  const int valid = static_cast<int>(L - i0 < kC ? L - i0 : kC);
  const int64_t hb = bh * L;

  if (m == 0) {  // no earlier key blocks: nothing reaches this block's qhat
    for (int idx = tid; idx < valid * D; idx += kNT) dqh[(hb + i0) * D + idx] = 0.f;
    if (FOX && tid < valid) rsum[hb + i0 + tid] = 0.f;
    return;
  }

  const int jown = 16 * w + l;  // this lane's A-operand row among the 64 keys
  bf4 ident;                     // B of the transposing product
#pragma unroll
  for (int r = 0; r < 4; ++r) ident[r] = static_cast<__bf16>(4 * g + r == l ? 1.f : 0.f);

  // dO of the query block (rows past the sequence end are zero)
  for (int idx = tid; idx < kC * (D / 8); idx += kNT) {
    const int i = idx / (D / 8), ch = idx % (D / 8);
    uint4 val = make_uint4(0, 0, 0, 0);
    if (i < valid) val = *reinterpret_cast<const uint4*>(dO + (hb + i0 + i) * D + 8 * ch);
    *reinterpret_cast<uint4*>(DOq + lds_off<D>(i, ch)) = val;
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

  // Qt^(n) as the transport kernel left it, in its accumulator layout: each wave reads its own rows
  const float* const scr = qt_scratch + pair_index(bh, Nb, m, 0) * QD;
  const auto slot = [&](int n, int h, int t) {
    return scr + static_cast<int64_t>(n) * QD + (((w * RT + h) * 4 + t) * 64 + lane) * 4;
  };
  const __bf16* const pk = packed + bh * Nb * G::kBlock;
  const auto mat = [&](int n, int64_t which) { return pk + static_cast<int64_t>(n) * G::kBlock + which; };

  // ---- key blocks left to right
  SplitRows<D> kh, pt[RT];
  SplitRows<kC> kt[RT];
  bf8 vf[DK];
  float c_j[4] = {0.f, 0.f, 0.f, 0.f};  // gate prefix of keys j = 16w + 4g + r
  const auto load_key = [&](int n) {
    load_rows<D, kC>(mat(n, G::kKh), jown, g, kh);
    const __bf16* vb = v + (hb + static_cast<int64_t>(n) * kC + jown) * D;
#pragma unroll
    for (int c = 0; c < DK; ++c) vf[c] = *reinterpret_cast<const bf8*>(vb + 32 * c + 8 * g);
  };
  const auto load_adj = [&](int n) {
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      load_rows<kC, D>(mat(n, G::kKt), 16 * (RT * w + h) + l, g, kt[h]);
      load_rows<D, D>(mat(n, G::kPt), 16 * (RT * w + h) + l, g, pt[h]);
    }
    if (FOX) {
      const float* cj = cum + hb + static_cast<int64_t>(n) * kC + 16 * w + 4 * g;  // rows of length L: no alignment
#pragma unroll
      for (int r = 0; r < 4; ++r) c_j[r] = cj[r];
    }
  };
  f4 qn[RT][4], lam[RT][4];
  float csm[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's share of sum_j dS[j][i], i = 16t + l
#pragma unroll
  for (int h = 0; h < RT; ++h)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qn[h][t] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(slot(0, h, t)));
      lam[h][t] = f4{0.f, 0.f, 0.f, 0.f};
    }
  load_key(0);
  load_adj(0);

  for (int n = 0; n < m; ++n) {
    // Qt^(n) by query rows (QA) and, transposed in registers, by head-dim rows (QB)
#pragma unroll
    for (int h = 0; h < RT; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const Split4 s = split4(qn[h][t]);
        wr4<D>(QAh, 16 * t + l, tile_pos(RT * w + h, g), s.hi);
        wr4<D>(QAl, 16 * t + l, tile_pos(RT * w + h, g), s.lo);
        const int arow = 16 * (RT * w + h) + l;
        wr4<kC>(QBh, arow, tile_pos(t, g), transpose4(s.hi, ident));
        wr4<kC>(QBl, arow, tile_pos(t, g), transpose4(s.lo, ident));
      }
    if (n + 1 < m) {
#pragma unroll
      for (int h = 0; h < RT; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) qn[h][t] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(slot(n + 1, h, t)));
    }
    __syncthreads();  // Qt staged, Lam^(n-1) (written at the end of the last step) in LB

    // S = Khat_n Qt^T and dO . v, rows j of this wave's tile
    f4 s[4], pd[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = pd[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DK; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf8 bhv = rd8<D>(QAh, 16 * t + l, 4 * c + g), blv = rd8<D>(QAl, 16 * t + l, 4 * c + g);
        const bf8 bd = rd8<D>(DOq, 16 * t + l, 4 * c + g);
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
      wr4<kC>(XBh, 16 * t + l, tile_pos(w, g), dsp.hi);
      wr4<kC>(XBl, 16 * t + l, tile_pos(w, g), dsp.lo);
    }

    // dP_n += Lam^(n-1) Qt^(n)^T (Lam^(n-1) transposed to rows a of this wave's tiles)
    if (n >= 1) {
#pragma unroll
      for (int h = 0; h < RT; ++h) {
        bf4 tlh[4], tll[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const Split4 ls = split4(lam[h][t]);
          tlh[t] = transpose4(ls.hi, ident);
          tll[t] = transpose4(ls.lo, ident);
        }
        f4 dp[DT];
#pragma unroll
        for (int u = 0; u < DT; ++u) dp[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf8 lh = cat8(tlh[2 * c], tlh[2 * c + 1]), ll = cat8(tll[2 * c], tll[2 * c + 1]);
#pragma unroll
          for (int u = 0; u < DT; ++u) {
            const bf8 bhv = rd8<kC>(QBh, 16 * u + l, 4 * c + g), blv = rd8<kC>(QBl, 16 * u + l, 4 * c + g);
            dp[u] = mma32(ll, bhv, dp[u]);
            dp[u] = mma32(lh, blv, dp[u]);
            dp[u] = mma32(lh, bhv, dp[u]);
          }
        }
        float* dstp = dPacc + ((bh * Nb + n) * D + 16 * (RT * w + h) + 4 * g) * D + l;
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) unsafeAtomicAdd(dstp + r * D + 16 * u, dp[u][r]);
      }
    }
    __syncthreads();  // every wave's scale dS rows are in XB

    // Lam^(n) = P_n^T Lam^(n-1) + Khat_n^T (scale dS), rows a of this wave's tiles
    {
      f4 acc[RT][4];
#pragma unroll
      for (int h = 0; h < RT; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[h][t] = f4{0.f, 0.f, 0.f, 0.f};
      if (n >= 1) {
#pragma unroll
        for (int c = 0; c < DK; ++c)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const bf8 lh = rd8<D>(LBh, 16 * t + l, 4 * c + g), ll = rd8<D>(LBl, 16 * t + l, 4 * c + g);
#pragma unroll
            for (int h = 0; h < RT; ++h) {
              acc[h][t] = mma32(pt[h].lo[c], lh, acc[h][t]);
              acc[h][t] = mma32(pt[h].hi[c], ll, acc[h][t]);
              acc[h][t] = mma32(pt[h].hi[c], lh, acc[h][t]);
            }
          }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf8 xh = rd8<kC>(XBh, 16 * t + l, 4 * c + g), xl = rd8<kC>(XBl, 16 * t + l, 4 * c + g);
#pragma unroll
          for (int h = 0; h < RT; ++h) {
            acc[h][t] = mma32(kt[h].lo[c], xh, acc[h][t]);
            acc[h][t] = mma32(kt[h].hi[c], xl, acc[h][t]);
            acc[h][t] = mma32(kt[h].hi[c], xh, acc[h][t]);
          }
        }
#pragma unroll
      for (int h = 0; h < RT; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) lam[h][t] = acc[h][t];
    }
    if (n + 1 < m) load_adj(n + 1);
    __syncthreads();  // every wave is done with LB, XB and the Qt tiles
#pragma unroll
    for (int h = 0; h < RT; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const Split4 ls = split4(lam[h][t]);
        wr4<D>(LBh, 16 * t + l, tile_pos(RT * w + h, g), ls.hi);
        wr4<D>(LBl, 16 * t + l, tile_pos(RT * w + h, g), ls.lo);
      }
  }

  // lam[h][t] holds Lam^(m-1)[a = 16(RT w + h) + 4g + r][i = 16t + l]: the gradient reaching qhat
#pragma unroll
  for (int h = 0; h < RT; ++h)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 16 * t + l;
      if (i < valid) *reinterpret_cast<f4*>(dqh + (hb + i0 + i) * D + 16 * (RT * w + h) + 4 * g) = lam[h][t];
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
template <int D, bool FOX>
__global__ __launch_bounds__(kNT, D == 64 ? (FOX ? 2 : 3) : 1) void bwd_key16_kernel(
    int64_t L, int Nb, int64_t BH, float scale, const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
    const __bf16* __restrict__ packed, const float* __restrict__ cum, const float* __restrict__ lse,
    const float* __restrict__ Dv, const float* __restrict__ qt_scratch, float* __restrict__ dkh,
    float* __restrict__ dVacc, float* __restrict__ csum) {
  using G = Geo<D>;
  constexpr int RT = G::RT, DK = G::DK, DT = G::DT, QD = G::QD;
  // bytes: QA, QB (hi and lo, 64 x D each), DOq and DOe (64 x D each)
  __shared__ __attribute__((aligned(16))) uint8_t sm[12 * QD];
  uint8_t* const QAh = sm;              // Qt by query rows: row i, column a at perm32(a) [W = D]
  uint8_t* const QAl = sm + 2 * QD;
  uint8_t* const QBh = sm + 4 * QD;     // Qt by head-dim rows: row a, column i at perm32(i) [W = 64]
  uint8_t* const QBl = sm + 6 * QD;
  uint8_t* const DOq = sm + 8 * QD;     // dO by query rows, columns in order [W = D]
  uint8_t* const DOe = sm + 10 * QD;    // dO by head-dim rows: row e, column i at perm32(i) [W = 64]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l = lane & 15;
  const int n = static_cast<int>(blockIdx.x / BH);  // key block 0 meets the most query blocks: first
  const int64_t bh = blockIdx.x % BH;
  const int64_t hb = bh * L;
  const int64_t j0 = static_cast<int64_t>(n) * kC;
  const int jown = 16 * w + l;
  bf4 ident;
#pragma unroll
  for (int r = 0; r < 4; ++r) ident[r] = static_cast<__bf16>(4 * g + r == l ? 1.f : 0.f);

  SplitRows<D> kh;
  load_rows<D, kC>(packed + (bh * Nb + n) * G::kBlock + G::kKh, jown, g, kh);
  bf8 vf[DK];
  {
    const __bf16* vb = v + (hb + j0 + jown) * D;  // block n < Nb - 1 is whole
#pragma unroll
    for (int c = 0; c < DK; ++c) vf[c] = *reinterpret_cast<const bf8*>(vb + 32 * c + 8 * g);
  }
  float c_j[4] = {0.f, 0.f, 0.f, 0.f};
  if (FOX) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c_j[r] = cum[hb + j0 + 16 * w + 4 * g + r];
  }

  const int64_t npairs = static_cast<int64_t>(Nb) * (Nb - 1) / 2;
  // Qt^(n) of query block m in the transport's accumulator layout (rows of wave w)
  const auto slot = [&](int m, int h, int t) {
    return qt_scratch + (bh * npairs + static_cast<int64_t>(m) * (m - 1) / 2 + n) * QD +
           (((w * RT + h) * 4 + t) * 64 + lane) * 4;
  };
  // dO_m in the same layout: rows i = 16t + l, columns 16(RT w + h) + 4g .. + 3 (zero past the end)
  const auto load_do = [&](int m, bf4 (&x)[RT][4]) {
    const int64_t i0 = static_cast<int64_t>(m) * kC;
#pragma unroll
    for (int h = 0; h < RT; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = 16 * t + l;
        x[h][t] = i0 + i < L ? *reinterpret_cast<const bf4*>(dO + (hb + i0 + i) * D + 16 * (RT * w + h) + 4 * g)
                             : bf4{0, 0, 0, 0};
      }
  };

  f4 dv[DT], dk[DT], qn[RT][4];
  bf4 dn[RT][4];
  float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < DT; ++u) dv[u] = dk[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < RT; ++h)
#pragma unroll
    for (int t = 0; t < 4; ++t) qn[h][t] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(slot(n + 1, h, t)));
  load_do(n + 1, dn);

  for (int m = n + 1; m < Nb; ++m) {
    const int64_t i0 = static_cast<int64_t>(m) * kC;
    const int valid = static_cast<int>(L - i0 < kC ? L - i0 : kC);
    // Qt^(n)_m and dO_m, each by query rows and (transposed in registers) by head-dim rows
#pragma unroll
    for (int h = 0; h < RT; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const Split4 sq = split4(qn[h][t]);
        const int arow = 16 * (RT * w + h) + l;
        wr4<D>(QAh, 16 * t + l, tile_pos(RT * w + h, g), sq.hi);
        wr4<D>(QAl, 16 * t + l, tile_pos(RT * w + h, g), sq.lo);
        wr4<kC>(QBh, arow, tile_pos(t, g), transpose4(sq.hi, ident));
        wr4<kC>(QBl, arow, tile_pos(t, g), transpose4(sq.lo, ident));
        wr4<D>(DOq, 16 * t + l, 16 * (RT * w + h) + 4 * g, dn[h][t]);
        wr4<kC>(DOe, arow, tile_pos(t, g), transpose4(dn[h][t], ident));
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
      for (int h = 0; h < RT; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) qn[h][t] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(slot(m + 1, h, t)));
      load_do(m + 1, dn);
    }
    __syncthreads();  // Qt and dO staged

    f4 s[4], pd[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = pd[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DK; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf8 bhv = rd8<D>(QAh, 16 * t + l, 4 * c + g), blv = rd8<D>(QAl, 16 * t + l, 4 * c + g);
        const bf8 bd = rd8<D>(DOq, 16 * t + l, 4 * c + g);
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
      for (int u = 0; u < DT; ++u) {
        const bf8 bo = rd8<kC>(DOe, 16 * u + l, 4 * c + g);
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
      for (int u = 0; u < DT; ++u) {
        const bf8 bhv = rd8<kC>(QBh, 16 * u + l, 4 * c + g), blv = rd8<kC>(QBl, 16 * u + l, 4 * c + g);
        dk[u] = mma32(dl, bhv, dk[u]);
        dk[u] = mma32(dh, blv, dk[u]);
        dk[u] = mma32(dh, bhv, dk[u]);
      }
    }
    __syncthreads();  // every wave is done with this query block's tiles
  }

  // rows j = 16w + 4g + r, columns e = 16u + l
  float* dstv = dVacc + (hb + j0 + 16 * w + 4 * g) * D + l;
  float* dstk = dkh + (hb + j0 + 16 * w + 4 * g) * D + l;
#pragma unroll
  for (int u = 0; u < DT; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dstv[r * D + 16 * u] = dv[u][r];
      dstk[r * D + 16 * u] = dk[u][r];
    }
  if (FOX) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rs = row16_sum(rowp[r]);
      if (l == 0) csum[hb + j0 + 16 * w + 4 * g + r] = rs;
    }
  }
}

template <int D>
static hipError_t launch_pair16_t(const BwdArgs& a, hipStream_t stream) {
  const int64_t BH = a.BH, L = a.L;
  const int Nb = static_cast<int>((L + kC - 1) / kC);
  const __bf16* packed = static_cast<const __bf16*>(a.ws.packed);
  const dim3 grid(static_cast<unsigned>(BH * Nb));
  const __bf16* v = static_cast<const __bf16*>(a.v);
  const __bf16* dO = static_cast<const __bf16*>(a.dout);
  hipError_t e;
  if (Nb >= 2) {
    const dim3 tgrid(static_cast<unsigned>(BH * ((Nb - 1 + kQG - 1) / kQG)));
    hipLaunchKernelGGL((bwd_transport16_kernel<D>), tgrid, dim3(kNT), 0, stream, L, Nb, BH, a.ws.qhat, packed,
                       a.ws.scratch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.ws.cum) {
    hipLaunchKernelGGL((bwd_pair16_kernel<D, true>), grid, dim3(kNT), 0, stream, L, Nb, BH, a.scale, v, dO, packed,
                       a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dqh, a.ws.rsum, a.ws.dP);
  } else {
    hipLaunchKernelGGL((bwd_pair16_kernel<D, false>), grid, dim3(kNT), 0, stream, L, Nb, BH, a.scale, v, dO, packed,
                       a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dqh, a.ws.rsum, a.ws.dP);
  }
  e = hipGetLastError();
  if (e != hipSuccess || Nb < 2) return e;
  const dim3 kgrid(static_cast<unsigned>(BH * (Nb - 1)));
  if (a.ws.cum) {
    hipLaunchKernelGGL((bwd_key16_kernel<D, true>), kgrid, dim3(kNT), 0, stream, L, Nb, BH, a.scale, v, dO, packed,
                       a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dkh, a.ws.dV, a.ws.csum);
  } else {
    hipLaunchKernelGGL((bwd_key16_kernel<D, false>), kgrid, dim3(kNT), 0, stream, L, Nb, BH, a.scale, v, dO, packed,
                       a.ws.cum, a.lse, a.ws.Dv, a.ws.scratch, a.ws.dkh, a.ws.dV, a.ws.csum);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_pair16(int64_t d, const BwdArgs& a, hipStream_t stream) {
  return d == 64 ? launch_pair16_t<64>(a, stream) : launch_pair16_t<128>(a, stream);
}

}  // namespace path
