// Matrix-core prepare stage of the bf16 PaTH forward (gfx950), and the same
// block work for the bf16 backward at d = 64 (prepare_mfma_bwd_kernel).
//
// One workgroup (4 waves) per 64-token block n of one head.  It computes the
// UT factor of the block [PaTH Attention summary (gist.science 2505.16381),
// §3 "Representação de Transformação UT"]:
//     G = W W^T,  X = T^{-1} = (I + diag(beta) strict_upper(G))^{-1} diag(beta)
// and from it [§3 "Algoritmo Estilo FlashAttention"]:
//     Z^T  = mask_{a>c}(W K^T)          Y^T = X^T Z^T       (so Y = Z X)
//     Khat = K - Y W                    (adjusted keys: H_{c+1}..H_63 folded into k_c)
//     F    = X^T W                      P = I - W^T X W = I - W^T F... stored as P rows
//     U    = W Q^T,  Ut = mask_{b<=r}(U)
//     Qhat = Q - F^T Ut                 (adjusted queries: H_0..H_r applied to q_r)
//     Sdiag^T = K Q^T - Y Ut            (in-block logits k_c^T H_{c+1}..H_r q_r, c <= r)
// Outputs (per block): Khat and P as fp16 hi/lo rows with the reduction
// index in mfma_perm order, c2*Qhat and c2*Sdiag in fp32 (Sdiag as a padded
// lower triangle, keys c <= r of query r), max |khat_c|, and
// V^T in fp16 with the keys in mfma_perm order (zero past the sequence end),
// the layout in which the scan feeds values to the matrix cores.
//
// The products are 16x16x32 MFMAs.  Wave w owns output column tile w (16
// columns), so the accumulator tile of one product is, after conversion to
// 16-bit, the B operand of the next one in the same wave.  Products of two
// stored inputs (bf16) are exact in one pass; a computed fp32 operand is split
// into fp16 hi + lo and costs two or three passes (hi*hi + hi*lo + lo*hi).
// Products that share an operand (Y and F, Khat and P) run side by side.
// T^{-1} is formed by 16-row blocks: each wave inverts one diagonal block by
// back substitution (4 lanes per column), and the off-diagonal blocks follow
// from fp32 16x16x4 MFMA products of those inverses with blocks of G.
// The transposes W^T and V^T are products too: the rows times a 32x16 slice of
// the identity leave 4 consecutive rows of one column in each lane.
// All global loads of a block are issued before the first is used.
//
// The backward's run of the stage (same block body, BWD = true) splits the
// computed operands into bf16 hi + lo instead (fp32's exponent range), and
// writes M = T^{-1} (fp32), Qhat unscaled in rows of length L, and Khat and P
// as bf16 hi/lo rows in both orientations (the second by a 16x16x16 product
// with the identity in registers).  It forms no in-block logits, V^T or
// bounds.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace path {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f4 mmb(const b8& a, const b8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

union H8u {
  h8 v;
  h2 p[4];
  uint4 u;
};

__device__ __forceinline__ h8 to_h8(const f4& x, const f4& y) {
  H8u r;
  r.p[0] = __builtin_convertvector(f2{x[0], x[1]}, h2);
  r.p[1] = __builtin_convertvector(f2{x[2], x[3]}, h2);
  r.p[2] = __builtin_convertvector(f2{y[0], y[1]}, h2);
  r.p[3] = __builtin_convertvector(f2{y[2], y[3]}, h2);
  return r.v;
}
__device__ __forceinline__ int perm32(int d) {  // mfma_perm of the prepare stage
  return (d & ~31) | (((d >> 2) & 3) << 3) | (((d >> 4) & 1) << 2) | (d & 3);
}

// Broadcast lane k of each quad of lanes to the whole quad (k folds to a constant).
__device__ __forceinline__ float quad_bcast(float x, int k) {
  const int v = __float_as_int(x);
  switch (k) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false));
  }
}

template <int D>
struct PGeo {
  static constexpr int C = 64;
  static constexpr int RP = D + 8;   // pitch (halfs) of input rows (bf16), natural column order
  static constexpr int TP = 64 + 8;  // pitch of rows with 64 reduction columns (perm order)
  static constexpr int DT = D / 16;  // head-dim tiles
  static constexpr int DC = D / 32;  // head-dim K chunks
  static constexpr int ET = DT / 4;  // head-dim tiles per wave
};

// Element type of the split (hi + lo) operands: fp16 for the forward (11
// significant bits per part), bf16 for the backward's run of this stage (16
// bits in all, with fp32's exponent range, so the backward keeps no range
// limit).
template <bool BWD>
struct Split16 {
  typedef _Float16 e;
  typedef _Float16 e8 __attribute__((ext_vector_type(8)));
  typedef _Float16 e2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f4 mma(const e8& a, const e8& b, const f4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Split16<true> {
  typedef __bf16 e;
  typedef __bf16 e8 __attribute__((ext_vector_type(8)));
  typedef __bf16 e2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f4 mma(const e8& a, const e8& b, const f4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <bool BWD>
__device__ __forceinline__ typename Split16<BWD>::e8 to_e8(const f4& x, const f4& y) {
  typedef typename Split16<BWD>::e2 e2;
  union {
    typename Split16<BWD>::e8 v;
    e2 p[4];
  } r;
  r.p[0] = __builtin_convertvector(f2{x[0], x[1]}, e2);
  r.p[1] = __builtin_convertvector(f2{x[2], x[3]}, e2);
  r.p[2] = __builtin_convertvector(f2{y[0], y[1]}, e2);
  r.p[3] = __builtin_convertvector(f2{y[2], y[3]}, e2);
  return r.v;
}
template <bool BWD>
struct SplitHL {
  typename Split16<BWD>::e8 hi, lo;
};
template <bool BWD>
__device__ __forceinline__ SplitHL<BWD> split8t(const f4& x, const f4& y) {
  SplitHL<BWD> r;
  r.hi = to_e8<BWD>(x, y);
  f4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = x[i] - static_cast<float>(r.hi[i]);
    b[i] = y[i] - static_cast<float>(r.hi[4 + i]);
  }
  r.lo = to_e8<BWD>(a, b);
  return r;
}
// The first four elements of an 8-element 16-bit vector (8 bytes).
template <typename V>
__device__ __forceinline__ uint2 low4(const V& v) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  return make_uint2(u.x, u.y);
}
// An accumulator tile of 4 bf16 per lane (rows 4lg + i, column ln) transposed
// by a 16x16x16 product with the identity (exact): the lane receives row ln,
// columns 4lg .. 4lg + 3, as 8 bytes.
__device__ __forceinline__ uint2 transpose_bits(const uint2& x, const uint2& ident) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const f4 y = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, x), __builtin_bit_cast(s4, ident),
                                                         f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 a = __builtin_convertvector(f2{y[0], y[1]}, bf2), b = __builtin_convertvector(f2{y[2], y[3]}, bf2);
  return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

}  // namespace

// One 64-token block.  BWD is the backward's run of the stage:
// bf16 splits, unscaled Qhat rows, M = T^{-1} diag(beta)^{-1}, and Khat and
// P_n in both orientations (kt_out, pt_out) for its 16-bit kernels; no
// in-block logits, V^T or bounds.
template <int D, bool BWD>
__device__ __forceinline__ void prepare_block(
    int64_t L, int Nb, float c2, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ v, const float* __restrict__ beta,
    typename Split16<BWD>::e* __restrict__ khat, typename Split16<BWD>::e* __restrict__ pmat,
    float* __restrict__ qhat, float* __restrict__ sdiag, float* __restrict__ kmax, float* __restrict__ pnorm,
    _Float16* __restrict__ vt, int* __restrict__ vexp, typename Split16<BWD>::e* __restrict__ kt_out,
    typename Split16<BWD>::e* __restrict__ pt_out, float* __restrict__ minv_out) {
  using SP = Split16<BWD>;
  using E = typename SP::e;
  using e8 = typename SP::e8;
  using G = PGeo<D>;
  constexpr int C = G::C, RP = G::RP, TP = G::TP, DT = G::DT, DC = G::DC, ET = G::ET;
  constexpr int GP = 68;  // row pitch (floats) of G in GY; 64 rows of it fit the C x TP floats
  // elements per block of the khat and pmat outputs (the backward's run packs
  // Khat, Khat^T, P_n and P_n^T, each hi and lo, per block)
  constexpr int64_t kst = BWD ? 4 * C * D + 4 * D * D : 2 * C * D;
  constexpr int64_t pst = BWD ? 4 * C * D + 4 * D * D : 2 * D * D;

  // LDS (halfs unless noted).  WK holds W rows then K rows; it is reused for
  // the blocks of T^{-1}, then for -F^T rows.  GY holds G (quarter layout),
  // then X^T rows hi/lo, then -Y rows hi/lo.  The query rows never enter LDS:
  // each wave reads its own 16 as B operands.
  __shared__ __attribute__((aligned(16))) uint16_t WK[2 * C * RP];
  __shared__ __attribute__((aligned(16))) E Wt[D * TP];             // W^T rows, perm(b)
  __shared__ __attribute__((aligned(16))) float GY[C * TP];
  __shared__ float bs[C];
  __shared__ float hn[C];
  __shared__ float kred[4];
  __shared__ float vred[4];

  uint16_t* Wb = WK;
  uint16_t* Kb = WK + C * RP;
  E* NY = reinterpret_cast<E*>(GY);   // [2][C*TP]
  E* XT = NY;                         // [2][C*TP], perm(a)
  E* NFT = reinterpret_cast<E*>(WK);  // [2][D*64] (pitch 64, no pad, swizzled chunks)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  // B operand of the backward's transposing products: lane (lg, ln) gives rows
  // 4lg .. 4lg + 3 of column ln of the 16 x 16 identity, as bf16 bits
  uint2 ident4 = make_uint2(0u, 0u);
  if constexpr (BWD) {
    uint32_t e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) e[r] = 4 * lg + r == ln ? 0x3F80u : 0u;
    ident4 = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
  }
  const int n = blockIdx.x % Nb;
  // Heads run from the last to the first.  The scan starts from the first
  // heads, and the blocks written last are the ones most likely to still sit
  // in the 256 MB last-level cache when it reads them.
  const int64_t bh = static_cast<int64_t>(gridDim.x / Nb) - 1 - blockIdx.x / Nb;
  const int64_t t0 = static_cast<int64_t>(n) * C;
  const int valid = static_cast<int>(L - t0 < C ? L - t0 : C);
  const int64_t base = (bh * L + t0) * D;

  // ---- load W, K, Q rows (bf16) ----------------------------------------------
  // Lanes idx .. idx + D/8 - 1 (consecutive, same wave) hold one row, so the
  // row norms |w_s|^2 come from a shuffle reduction over them.  The value rows
  // are fetched last (they are needed only at the end; loads complete in order).
  constexpr int VCH = C * (D / 8) / 256;
  // Every load is issued before any is used, from a row clamped into the
  // sequence (rows past its end are zeroed when stored), so they are all in
  // flight together.
  uint4 wv[VCH], kv[VCH];
  float br[VCH];
#pragma unroll
  for (int j = 0; j < VCH; ++j) {
    const int idx = tid + 256 * j;
    const int r = idx / (D / 8), c8 = idx % (D / 8);
    const int rr = r < valid ? r : valid - 1;
    wv[j] = *reinterpret_cast<const uint4*>(w + base + rr * D + 8 * c8);
    kv[j] = *reinterpret_cast<const uint4*>(k + base + rr * D + 8 * c8);
    br[j] = beta[bh * L + t0 + rr];
  }
  // this lane's key entries for the adjusted keys: row 16w + ln, columns 16et + 4lg .. + 3,
  // and its query entries as the B operand of products over the head dim:
  // row 16w + ln, columns 32c + 8lg .. + 7 (zero past the sequence end)
  uint2 kr[DT];
  b8 bq[DC];
  {
    const int r = 16 * wave + ln;
    const int rr = r < valid ? r : valid - 1;
#pragma unroll
    for (int et = 0; et < DT; ++et) {
      kr[et] = *reinterpret_cast<const uint2*>(k + base + rr * D + 16 * et + 4 * lg);  // masked at use
    }
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      union {
        uint4 u;
        b8 v;
      } t;
      t.u = *reinterpret_cast<const uint4*>(q + base + rr * D + 32 * c + 8 * lg);
      bq[c] = t.v;
    }
  }
  // value rows, already in the A-operand layout of the transposing product:
  // lane (ln, lg) of wave w holds row 16w + ln, columns 32h + 8lg .. 32h + 8lg + 7
  uint4 vraw[D / 32];
  if constexpr (!BWD) {
    const int r = 16 * wave + ln;
    const int rr = r < valid ? r : valid - 1;
#pragma unroll
    for (int h = 0; h < D / 32; ++h)
      vraw[h] = *reinterpret_cast<const uint4*>(v + base + rr * D + 32 * h + 8 * lg);
  }
#pragma unroll
  for (int j = 0; j < VCH; ++j) {
    const int idx = tid + 256 * j;
    const int r = idx / (D / 8), c8 = idx % (D / 8);
    const uint4 zero = make_uint4(0, 0, 0, 0);
    if (r >= valid) {
      wv[j] = kv[j] = zero;
      br[j] = 0.f;
    }
    *reinterpret_cast<uint4*>(Wb + r * RP + 8 * c8) = wv[j];
    *reinterpret_cast<uint4*>(Kb + r * RP + 8 * c8) = kv[j];
    const uint32_t ww[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(ww[e] << 16), hi = __uint_as_float(ww[e] & 0xffff0000u);
      sq += lo * lo + hi * hi;
    }
#pragma unroll
    for (int off = 1; off < D / 8; off <<= 1) sq += __shfl_xor(sq, off, 64);
    if (c8 == 0) {
      bs[r] = br[j];
      // |H_s|_2 = max(1, |1 - beta_s |w_s|^2|): its product bounds the growth
      // of a transported query across the block
      if constexpr (!BWD) hn[r] = fmaxf(1.f, fabsf(1.f - br[j] * sq));
    }
  }
  if (16 * wave + ln >= valid) {
#pragma unroll
    for (int c = 0; c < DC; ++c) bq[c] = b8{};
  }
  __syncthreads();

  // ---- products of stored inputs (exact, one bf16 pass); wave w = column tile w
  // W^T (fp16, rows e, columns perm(b)) comes from the same pass: this wave's
  // W rows b = 16w .. 16w + 15, the B operand below, times a 32x16 slice of the
  // identity give W[b][32c + 16s + ln] for b = 16w + 4lg .. 16w + 4lg + 3 in
  // lane (lg, ln), 8 contiguous bytes of W^T row 32c + 16s + ln.
  f4 gt[4], zt[4], ut[4], skq[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) gt[mt] = zt[mt] = ut[mt] = skq[mt] = f4{0.f, 0.f, 0.f, 0.f};
  b8 ident[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) ident[s][t] = static_cast<__bf16>((lg == ln / 8 + 2 * s && t == ln % 8) ? 1.f : 0.f);
  E* wtb = Wt + 32 * (wave >> 1) + 8 * lg + 4 * (wave & 1);
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const int col = 32 * c + 8 * lg;
    const b8 bw = *reinterpret_cast<const b8*>(Wb + (16 * wave + ln) * RP + col);
    const b8 bk = *reinterpret_cast<const b8*>(Kb + (16 * wave + ln) * RP + col);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const b8 aw = *reinterpret_cast<const b8*>(Wb + (16 * mt + ln) * RP + col);
      const b8 ak = *reinterpret_cast<const b8*>(Kb + (16 * mt + ln) * RP + col);
      gt[mt] = mmb(aw, bw, gt[mt]);    // G[s][t]      = w_s . w_t
      zt[mt] = mmb(aw, bk, zt[mt]);    // Z^T[a][c]    = w_a . k_c
      ut[mt] = mmb(aw, bq[c], ut[mt]);    // U[b][r]      = w_b . q_r
      if constexpr (!BWD) skq[mt] = mmb(ak, bq[c], skq[mt]);  // (K Q^T)[c][r] = k_c . q_r
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f4 y = mmb(bw, ident[s], f4{0.f, 0.f, 0.f, 0.f});
      *reinterpret_cast<uint2*>(wtb + (32 * c + 16 * s + ln) * TP) = low4(to_e8<BWD>(y, y));
    }
  }
  // Diagonal 16x16 blocks of G by columns in the quarter layout
  // GY[t*GP + q*16 + u] = G[4u+q][t] (rows above t only); wave w holds block (w, w).
  // The row pitch GP = 68 (not 64) spreads the 64 lanes of a store over distinct banks.
  {
    const int t = 16 * wave + ln;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      if (mt == wave) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * mt + 4 * lg + i;
          GY[t * GP + (s & 3) * 16 + (s >> 2)] = (s < t) ? gt[mt][i] : 0.f;
        }
      }
  }
  __syncthreads();

  // ---- X = T^{-1} diag(beta), T = I + diag(beta) strict_upper(G), by 16-row blocks -------
  // Row r of T^{-1} (last row first) is  Tinv[r][c] = delta_rc - beta_r sum_{t>r} G[r][t] Tinv[t][c].
  // With 16-row blocks I, J (T is block upper triangular):
  //   D_I = T_II^{-1}                          (wave I: a 16-step back substitution)
  //   E_IK = -D_I T_IK  (I < K)                (wave K: its G block column is in registers)
  //   Tinv_IJ = sum_{K=I+1..J} E_IK Tinv_KJ    (wave J, nearest block first; Tinv_JJ = D_J)
  // The block products are fp32 16x16x4 MFMAs.  Their operand B is the accumulator
  // layout of a 16x16 tile (lane (g, j) holds rows 4g..4g+3 of column j); the
  // reduction index of MFMA kc is then 4g + kc, which operand A (from LDS) follows.
  // A 16x16 block in LDS: element (r, c) at r * BP + (c ^ (r & 3)).  Pitch 20
  // and the swizzle keep both operand orientations of the 16x16x4 products
  // (16 rows x 4 columns a step apart, and its transpose) on 64 distinct banks.
  constexpr int BP = 20;       // pitch (floats) of a 16x16 block in LDS
  constexpr int BS = 16 * BP;  // floats per block
  auto bx = [](int r, int c) { return r * BP + (c ^ (r & 3)); };
  // The W and K rows are dead once the products are formed (the adjusted keys
  // read K again from global memory), so the blocks live in their space.
  float* SD = reinterpret_cast<float*>(WK);  // D_0..D_3
  float* SE = SD + 4 * BS;                   // E_IK, I < K, at index I(7-I)/2 + K-I-1
  {
    const int c = lane >> 2, qq = lane & 3;  // column c of block `wave`, rows 4u + qq
    const int I = wave;
    float bq[4], acc[4], d[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bq[u] = bs[16 * I + 4 * u + qq];
      acc[u] = d[u] = 0.f;
    }
    const float* gcol = GY + 16 * I * GP + qq * 16 + 4 * I;  // + r*GP: G[16I+4u+qq][16I+r], u = 0..3
    f4 gc = *reinterpret_cast<const f4*>(gcol + 15 * GP), gn = *reinterpret_cast<const f4*>(gcol + 14 * GP);
#pragma unroll
    for (int r = 15; r >= 0; --r) {
      f4 gnn = gn;
      if (r > 1) gnn = *reinterpret_cast<const f4*>(gcol + (r - 2) * GP);
      const int ur = r >> 2;
      float x = (r == c ? 1.f : 0.f) - bq[ur] * acc[ur];  // right on lanes qq == r % 4
      x = quad_bcast(x, r & 3);
      if (qq == (r & 3)) d[ur] = x;
#pragma unroll
      for (int u = 0; u < (r + 3) / 4; ++u) acc[u] += gc[u] * x;
      gc = gn;
      gn = gnn;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) SD[I * BS + bx(4 * u + qq, c)] = d[u];
  }
  __syncthreads();
  const int K = wave;
  {
    // E_IK = -D_I (diag(beta_I) G_IK); lane (lg, ln) holds G[16I+4lg+i][16K+ln] in gt[I][i]
#pragma unroll
    for (int I = 0; I < 3; ++I) {
      if (I < K) {
        f4 e = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const float b = bs[16 * I + 4 * lg + kc] * gt[I][kc];
          const float av = SD[I * BS + bx(ln, 4 * lg + kc)];
          e = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b, e, 0, 0, 0);
        }
        float* dst = SE + (I * (7 - I) / 2 + K - I - 1) * BS;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[bx(4 * lg + i, ln)] = -e[i];
      }
    }
  }
  __syncthreads();
  // column block J = wave of T^{-1}: tc[I] holds Tinv_IJ in the accumulator layout
  f4 tc[4];
  {
    const int J = wave;
#pragma unroll
    for (int I = 0; I < 4; ++I) tc[I] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int I = 0; I < 4; ++I)
      if (I == J) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tc[I][i] = SD[J * BS + bx(4 * lg + i, ln)];
      }
#pragma unroll
    for (int I = 2; I >= 0; --I) {
      if (I < J) {
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int Kb2 = I + 1; Kb2 < 4; ++Kb2) {
          if (Kb2 <= J) {
            const float* ea = SE + (I * (7 - I) / 2 + Kb2 - I - 1) * BS;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[bx(ln, 4 * lg + kc)], tc[Kb2][kc], acc, 0, 0, 0);
          }
        }
        tc[I] = acc;
      }
    }
  }
  {
    // X^T rows: XT[c][perm(a)] = X[a][c] = Tinv[a][c] beta_c, c = 16J + ln, a = 16I + 4lg + i
    const int cc = 16 * wave + ln;
    const float bc = bs[cc];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      if constexpr (BWD) {
        // M = T^{-1}, fp32 rows a = 16I + 4lg + i, column cc
        float* mo = minv_out + (bh * Nb + n) * (C * C) + (16 * I + 4 * lg) * C + cc;
#pragma unroll
        for (int i = 0; i < 4; ++i) mo[i * C] = tc[I][i];
      }
      f4 x = tc[I] * bc;
      const e8 hv = to_e8<BWD>(x, x);
      f4 lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) lo[i] = x[i] - static_cast<float>(hv[i]);
      const e8 lv = to_e8<BWD>(lo, lo);
      const int off = cc * TP + 32 * (I >> 1) + 8 * lg + 4 * (I & 1);
      *reinterpret_cast<uint2*>(&XT[off]) = low4(hv);
      *reinterpret_cast<uint2*>(&XT[C * TP + off]) = low4(lv);
    }
  }
  __syncthreads();  // XT ready (in G's place: G was last read by the substitution)

  // ---- Y^T = X^T Z^T (wave w: columns c in tile w) and F = X^T W (rows b,
  // columns e in head-dim tiles et = ET*w .. ET*w + ET - 1): one pass over the
  // X^T operands serves both
  f4 yt[4], ft[ET][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    yt[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < ET; ++j) ft[j][mt] = f4{0.f, 0.f, 0.f, 0.f};
  }
  {
    // mask Z^T to a > c (a = row, c = column)
    const int cc = 16 * wave + ln;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * mt + 4 * lg + i <= cc) zt[mt][i] = 0.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const SplitHL<BWD> b = split8t<BWD>(zt[2 * kc], zt[2 * kc + 1]);
      e8 bwt[ET];
#pragma unroll
      for (int j = 0; j < ET; ++j)
        bwt[j] = *reinterpret_cast<const e8*>(&Wt[(16 * (ET * wave + j) + ln) * TP + 32 * kc + 8 * lg]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int off = (16 * mt + ln) * TP + 32 * kc + 8 * lg;
        const e8 ah = *reinterpret_cast<const e8*>(&XT[off]);
        const e8 al = *reinterpret_cast<const e8*>(&XT[C * TP + off]);
        yt[mt] = SP::mma(al, b.hi, yt[mt]);
#pragma unroll
        for (int j = 0; j < ET; ++j) ft[j][mt] = SP::mma(al, bwt[j], ft[j][mt]);
        yt[mt] = SP::mma(ah, b.lo, yt[mt]);
#pragma unroll
        for (int j = 0; j < ET; ++j) ft[j][mt] = SP::mma(ah, bwt[j], ft[j][mt]);
        yt[mt] = SP::mma(ah, b.hi, yt[mt]);
      }
    }
  }
  __syncthreads();  // every wave's X^T reads are done: -Y rows take its place
  // -Y rows into NY: lane holds Y^T[b = 16mt+4lg+i][c] = Y[c][b]
  SplitHL<BWD> yb[2];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    yb[kc] = split8t<BWD>(yt[2 * kc], yt[2 * kc + 1]);
    const int off = (16 * wave + ln) * TP + 32 * kc + 8 * lg;
    *reinterpret_cast<e8*>(&NY[off]) = -yb[kc].hi;
    *reinterpret_cast<e8*>(&NY[C * TP + off]) = -yb[kc].lo;
  }
  // lane holds F[b = 16mt+4lg+i][e = 16et+ln] = F^T[e][b] -> -F^T rows (pitch 64, perm b;
  // unpadded, so the 16-byte chunks of a row are swizzled to keep 16-row reads off one bank)
  SplitHL<BWD> fb[ET][2];
#pragma unroll
  for (int j = 0; j < ET; ++j)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      fb[j][kc] = split8t<BWD>(ft[j][2 * kc], ft[j][2 * kc + 1]);
      const int row = 16 * (ET * wave + j) + ln;
      const int off = row * 64 + (((4 * kc + lg) ^ (row & 7)) << 3);  // 16-byte chunk j at slot j ^ (row & 7)
      *reinterpret_cast<e8*>(&NFT[off]) = -fb[j][kc].hi;
      *reinterpret_cast<e8*>(&NFT[D * 64 + off]) = -fb[j][kc].lo;
    }

  // ---- Khat^T = K^T - W^T Y^T (rows e, columns c in tile w) and
  // P^T = I - W^T F (stored as P rows e, perm(f)): one pass over the W^T operands
  {
    const int cc = 16 * wave + ln;
    float s2 = 0.f;
#pragma unroll
    for (int et = 0; et < DT; ++et) {
      f4 acc, pacc[ET];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wd = i < 2 ? kr[et].x : kr[et].y;
        acc[i] = cc < valid ? -__uint_as_float((i & 1) ? (wd & 0xffff0000u) : (wd << 16)) : 0.f;
#pragma unroll
        for (int j = 0; j < ET; ++j) pacc[j][i] = (16 * et + 4 * lg + i == 16 * (ET * wave + j) + ln) ? -1.f : 0.f;
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const e8 a = *reinterpret_cast<const e8*>(&Wt[(16 * et + ln) * TP + 32 * kc + 8 * lg]);
        acc = SP::mma(a, yb[kc].lo, acc);
#pragma unroll
        for (int j = 0; j < ET; ++j) pacc[j] = SP::mma(a, fb[j][kc].lo, pacc[j]);
        acc = SP::mma(a, yb[kc].hi, acc);
#pragma unroll
        for (int j = 0; j < ET; ++j) pacc[j] = SP::mma(a, fb[j][kc].hi, pacc[j]);
      }
      acc = -acc;  // Khat[c][e], e = 16et + 4lg + i
#pragma unroll
      for (int i = 0; i < 4; ++i) s2 += acc[i] * acc[i];
      // rows with perm columns: e = 32(et/2) + 16(et%2) + 4lg + i -> 32(et/2) + 8lg + 4(et%2) + i
      const int pcol = 32 * (et / 2) + 8 * lg + 4 * (et % 2);
      {
        E* dst = khat + (bh * Nb + n) * kst + cc * D + pcol;
        const e8 hv = to_e8<BWD>(acc, acc);
        f4 lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = acc[i] - static_cast<float>(hv[i]);
        const e8 lv = to_e8<BWD>(lo, lo);
        *reinterpret_cast<uint2*>(dst) = low4(hv);
        *reinterpret_cast<uint2*>(dst + C * D) = low4(lv);
        if constexpr (BWD) {
          // Khat^T: row e = 16et + ln, columns perm(c) for c = 16w + 4lg .. + 3
          E* dt = kt_out + (bh * Nb + n) * kst + (16 * et + ln) * C + 32 * (wave >> 1) + 8 * lg + 4 * (wave & 1);
          *reinterpret_cast<uint2*>(dt) = transpose_bits(low4(hv), ident4);
          *reinterpret_cast<uint2*>(dt + C * D) = transpose_bits(low4(lv), ident4);
        }
      }
#pragma unroll
      for (int j = 0; j < ET; ++j) {
        const f4 pv = -pacc[j];  // P[e][f], e = 16(ET w + j) + ln, f = 16et + 4lg + i
        E* dst = pmat + (bh * Nb + n) * pst + (16 * (ET * wave + j) + ln) * D + pcol;
        const e8 hv = to_e8<BWD>(pv, pv);
        f4 lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = pv[i] - static_cast<float>(hv[i]);
        const e8 lv = to_e8<BWD>(lo, lo);
        *reinterpret_cast<uint2*>(dst) = low4(hv);
        *reinterpret_cast<uint2*>(dst + D * D) = low4(lv);
        if constexpr (BWD) {
          // P^T: row a = f = 16et + ln, columns perm(b) for b = e = 16E + 4lg .. + 3
          const int E0 = ET * wave + j;
          E* dt = pt_out + (bh * Nb + n) * pst + (16 * et + ln) * D + 32 * (E0 >> 1) + 8 * lg + 4 * (E0 & 1);
          *reinterpret_cast<uint2*>(dt) = transpose_bits(low4(hv), ident4);
          *reinterpret_cast<uint2*>(dt + D * D) = transpose_bits(low4(lv), ident4);
        }
      }
    }
    if constexpr (!BWD) {
      s2 += __shfl_xor(s2, 16, 64);
      s2 += __shfl_xor(s2, 32, 64);
      s2 = wave_max(s2);
      if (lane == 0) kred[wave] = s2;
    }
  }
  if constexpr (!BWD) {
    // largest |v| of the block (this wave's rows; a clamped row repeats a valid one)
    uint32_t m = 0;
#pragma unroll
    for (int h = 0; h < D / 32; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wd = (&vraw[h].x)[i];
        m = max(m, max(wd & 0x7fffu, (wd >> 16) & 0x7fffu));
      }
    const float vm = wave_max(__uint_as_float(m << 16));
    if (lane == 0) vred[wave] = vm;
  }
  __syncthreads();  // -Y and -F^T rows complete

  // V^T[e][perm(c)] in fp16, transposed on the matrix cores: with the value
  // rows as operand A and a 32x16 slice of the identity as operand B, the
  // product is V[:, slice] in the accumulator layout, where lane (lg, ln) holds
  // the 4 consecutive keys 16w + 4lg .. 16w + 4lg + 3 of column 32h + 16s + ln:
  // 8 contiguous bytes of a V^T row.  Exact: every product is by 1 or 0.
  // The block is stored times 2^-e, e = max(0, exponent of max|v| - 14), so that
  // every stored value is below 2^15 (fp16 holds 65504): e = 0 unless some
  // |v| >= 2^15.  The scaling is exact (a power of two); e goes to vexp.
  if constexpr (!BWD) {
    int ve;
    float vsc;
    {
      const float vm = fmaxf(fmaxf(vred[0], vred[1]), fmaxf(vred[2], vred[3]));
      const int ex = static_cast<int>((__float_as_uint(vm) >> 23) & 0xff) - 127;  // finite inputs
      ve = ex > 14 ? ex - 14 : 0;
      vsc = __uint_as_float(static_cast<uint32_t>(127 - ve) << 23);
    }
    {
      const int r = 16 * wave + ln;
      _Float16* vtb = vt + (bh * Nb + n) * (D * C) + 32 * (wave >> 1) + 8 * lg + 4 * (wave & 1);
  #pragma unroll
      for (int s = 0; s < 2; ++s) {
  #pragma unroll
        for (int h = 0; h < D / 32; ++h) {
          union {
            uint4 u;
            b8 v;
          } av;
          av.u = r < valid ? vraw[h] : make_uint4(0, 0, 0, 0);
          const f4 y = mmb(av.v, ident[s], f4{0.f, 0.f, 0.f, 0.f}) * vsc;
          const H8u hv = {to_h8(y, y)};
          *reinterpret_cast<uint2*>(vtb + (32 * h + 16 * s + ln) * C) = make_uint2(hv.u.x, hv.u.y);
        }
      }
    }

    if (wave == 0) {
      // product of the 64 factors |H_s|_2 by a butterfly over the wave
      float g = hn[lane];
  #pragma unroll
      for (int off = 1; off < 64; off <<= 1) g *= __shfl_xor(g, off, 64);
      if (lane == 0) {
        const float mx = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
        kmax[bh * Nb + n] = sqrtf(mx);
        pnorm[bh * Nb + n] = g;
        vexp[bh * Nb + n] = ve;
      }
    }
  }

  // ---- in-block logits and adjusted queries (wave w: queries r in tile w) -------
  {
    const int r = 16 * wave + ln;
    // Ut = mask_{b <= r}(U)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * mt + 4 * lg + i > r) ut[mt][i] = 0.f;
    SplitHL<BWD> ub[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) ub[kc] = split8t<BWD>(ut[2 * kc], ut[2 * kc + 1]);

    // Sdiag^T[c][r] = (K Q^T)[c][r] - sum_b Y[c][b] Ut[b][r]   (tiles mt < 4)
    // Qhat^T[e][r] = Q^T[e][r] - sum_b F^T[e][b] Ut[b][r]     (tiles et < DT)
    // formed side by side: independent products on the same B operands
    // (the backward's run forms no in-block logits and keeps Qhat in rows of length L)
    constexpr bool SD = !BWD;
    float* sd = SD ? sdiag + (bh * Nb + n) * kDiagTri + diag_row(r) : nullptr;
    float* qd = BWD ? qhat + (bh * L + t0 + r) * D : qhat + ((bh * Nb + n) * C + r) * D;
    constexpr int NX = DT > 4 || !SD ? DT : 4;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      f4 sacc = SD && x < 4 ? skq[x < 4 ? x : 0] : f4{0.f, 0.f, 0.f, 0.f}, qacc;
      // Q^T tile x: 16 identity rows (offset 16(x&1)) times the query operand
      // of chunk x/2, exact; the lane gets q_r[16x + 4lg .. + 3]
      if (x < DT) qacc = mmb(ident[x & 1], bq[x < DT ? x >> 1 : 0], f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        e8 sh, sl, qh, ql;
        if (SD && x < 4) {
          const int off = (16 * x + ln) * TP + 32 * kc + 8 * lg;
          sh = *reinterpret_cast<const e8*>(&NY[off]);
          sl = *reinterpret_cast<const e8*>(&NY[C * TP + off]);
        }
        if (x < DT) {
          const int row = 16 * x + ln;
          const int off = row * 64 + (((4 * kc + lg) ^ (row & 7)) << 3);
          qh = *reinterpret_cast<const e8*>(&NFT[off]);
          ql = *reinterpret_cast<const e8*>(&NFT[D * 64 + off]);
        }
        if (SD && x < 4) sacc = SP::mma(sl, ub[kc].hi, sacc);
        if (x < DT) qacc = SP::mma(ql, ub[kc].hi, qacc);
        if (SD && x < 4) sacc = SP::mma(sh, ub[kc].lo, sacc);
        if (x < DT) qacc = SP::mma(qh, ub[kc].lo, qacc);
        if (SD && x < 4) sacc = SP::mma(sh, ub[kc].hi, sacc);
        if (x < DT) qacc = SP::mma(qh, ub[kc].hi, qacc);
      }
      if (SD && x < 4 && 16 * x + 4 * lg <= r) {  // chunks of the padded triangle
        f4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * x + 4 * lg + i;
          out[i] = (c <= r && r < valid) ? c2 * sacc[i] : 0.f;
        }
        *reinterpret_cast<f4*>(sd + 16 * x + 4 * lg) = out;
      }
      if (x < DT && (!BWD || r < valid))
        *reinterpret_cast<f4*>(qd + 16 * x + 4 * lg) = (r < valid) ? qacc * c2 : f4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void prepare_mfma_kernel(
    int64_t L, int Nb, float c2, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ v, const float* __restrict__ beta,
    _Float16* __restrict__ khat, _Float16* __restrict__ pmat, float* __restrict__ qhat,
    float* __restrict__ sdiag, float* __restrict__ kmax, float* __restrict__ pnorm,
    _Float16* __restrict__ vt, int* __restrict__ vexp) {
  prepare_block<D, false>(L, Nb, c2, q, k, w, v, beta, khat, pmat, qhat, sdiag, kmax, pnorm, vt, vexp, nullptr,
                          nullptr, nullptr);
}

// The backward's prepare for bf16 storage: per block, into `packed`
// (4*64*D + 4*D*D bf16, each matrix a hi matrix then its lo matrix): Khat
// rows j (columns e), Khat^T rows a (columns j), P_n rows a (columns b), P_n^T
// rows a (columns b), columns in mfma_perm order; Qhat unscaled in rows of
// length L; M = (I + diag(beta) strict_upper(W W^T))^{-1} in fp32.
template <int D>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void prepare_mfma_bwd_kernel(
    int64_t L, int Nb, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ w, const float* __restrict__ beta, __bf16* __restrict__ packed,
    float* __restrict__ qhat, float* __restrict__ minv) {
  constexpr int CD = 64 * D, DD = D * D;
  prepare_block<D, true>(L, Nb, 1.f, q, k, w, nullptr, beta, packed, packed + 4 * CD, qhat, nullptr, nullptr,
                         nullptr, nullptr, nullptr, packed + 2 * CD, packed + 4 * CD + 2 * DD, minv);
}

template <int D>
static hipError_t launch_prepare_mfma_t(int64_t BH, int64_t L, float c2, const void* q, const void* k,
                                        const void* w, const void* v, const float* beta, _Float16* khat,
                                        _Float16* pmat, float* qhat, float* sdiag, float* kmax,
                                        float* pnorm, _Float16* vt, int* vexp, hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  hipLaunchKernelGGL((prepare_mfma_kernel<D>), dim3(static_cast<unsigned>(BH * Nb)), dim3(256), 0, stream,
                     L, Nb, c2, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(w), static_cast<const uint16_t*>(v), beta, khat, pmat,
                     qhat, sdiag, kmax, pnorm, vt, vexp);
  return hipGetLastError();
}

hipError_t launch_prepare_mfma_bwd(int64_t BH, int64_t L, int64_t d, const void* q, const void* k,
                                   const void* w, const float* beta, void* packed, float* qhat, float* minv,
                                   hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  const dim3 grid(static_cast<unsigned>(BH * Nb));
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* ww = static_cast<const uint16_t*>(w);
  auto* pk = static_cast<__bf16*>(packed);
  if (d == 64) {
    hipLaunchKernelGGL(prepare_mfma_bwd_kernel<64>, grid, dim3(256), 0, stream, L, Nb, qq, kk, ww, beta, pk, qhat,
                       minv);
  } else {
    hipLaunchKernelGGL(prepare_mfma_bwd_kernel<128>, grid, dim3(256), 0, stream, L, Nb, qq, kk, ww, beta, pk, qhat,
                       minv);
  }
  return hipGetLastError();
}

hipError_t launch_prepare_mfma(int64_t B, int64_t H, int64_t L, int64_t d, float c2, const void* q,
                               const void* k, const void* w, const void* v, const float* beta,
                               _Float16* khat, _Float16* pmat, float* qhat, float* sdiag, float* kmax,
                               float* pnorm, _Float16* vt, int* vexp, hipStream_t stream) {
  return d == 64 ? launch_prepare_mfma_t<64>(B * H, L, c2, q, k, w, v, beta, khat, pmat, qhat, sdiag, kmax,
                                             pnorm, vt, vexp, stream)
                 : launch_prepare_mfma_t<128>(B * H, L, c2, q, k, w, v, beta, khat, pmat, qhat, sdiag, kmax,
                                              pnorm, vt, vexp, stream);
}

}  // namespace path
