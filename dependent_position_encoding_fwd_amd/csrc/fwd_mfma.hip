// Matrix-core (MFMA) right-to-left scan forward of PaTH attention, gfx950.
//
// [PaTH Attention summary (gist.science 2505.16381), §2 "Mecanismo Central"]
//     s_ij = scale * k_j^T (H_{j+1} ... H_i) q_i   (+ FoX bias), softmax over j <= i
// [§3 "Algoritmo Estilo FlashAttention"]  One workgroup owns one 64-query UT
// block m.  It starts from the in-block logits and the boundary-adjusted
// queries produced by the prepare stage, then scans key blocks n = m-1 .. 0
// right to left.  Per key block, with Qt = (transported queries)^T in fp32:
//     S^T  = Khat_n Qt                 (keys x queries, 16x16x32 f16 MFMA)
//     online softmax over keys         (running max / sum in registers, exp2)
//     O^T += V_n^T P^T                 (16x16x32 bf16 MFMA)
//     Qt   = P_n Qt                    (block transition P_n = H_0...H_63, f16 MFMA)
// [§2 "Extensões: PaTH-FoX"] adds cum_i - cum_j (log2 units) to each logit.
//
// Everything stays transposed (keys or head dims on MFMA rows, queries on
// columns) so that each 16x16 accumulator tile, converted to 16-bit, is
// directly the B operand of the next product: rows 4g..4g+3 of tiles 2c and
// 2c+1 form lane group g's 8 reduction slots of K-chunk c.  The A operands
// (Khat, P, V^T) are staged in LDS with their reduction index permuted the
// same way (mfma_perm in the prepare stage; the V transpose below), so every
// operand fetch is one 16-byte LDS read.
//
// Precision (PaTH summary §6 "Limitações" warns that bf16 makes the
// cumulative product unstable): Qt is carried in fp32 and both Qt and the
// stored Khat / P are split into fp16 hi + lo parts.  ACCURATE uses
// hi*hi + hi*lo + lo*hi for the logits and the transition on every block;
// AUTO drops the lo terms on a block when the bound
//     |Qt|_max * |khat|_max * 2^-10  (log2-logit units)
// is at most `tau`.  Probabilities and values meet in bf16 (fp32 accumulate).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace path {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f4 mma16(const h8& a, const h8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mmb16(const b8& a, const b8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

union H8 {
  h8 v;
  h2 p[4];
};
union B8 {
  b8 v;
  b2 p[4];
};

// 8 fp32 (two accumulator quads) -> packed fp16, round to nearest even.
__device__ __forceinline__ h8 pack_h8(const f4& x, const f4& y) {
  H8 r;
  r.p[0] = __builtin_convertvector(f2{x[0], x[1]}, h2);
  r.p[1] = __builtin_convertvector(f2{x[2], x[3]}, h2);
  r.p[2] = __builtin_convertvector(f2{y[0], y[1]}, h2);
  r.p[3] = __builtin_convertvector(f2{y[2], y[3]}, h2);
  return r.v;
}
// lo part: x - float(hi)
__device__ __forceinline__ h8 pack_lo(const f4& x, const f4& y, const h8& hi) {
  f4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = x[i] - static_cast<float>(hi[i]);
    b[i] = y[i] - static_cast<float>(hi[4 + i]);
  }
  return pack_h8(a, b);
}
__device__ __forceinline__ b8 pack_b8(const f4& x, const f4& y) {
  B8 r;
  r.p[0] = __builtin_convertvector(f2{x[0], x[1]}, b2);
  r.p[1] = __builtin_convertvector(f2{x[2], x[3]}, b2);
  r.p[2] = __builtin_convertvector(f2{y[0], y[1]}, b2);
  r.p[3] = __builtin_convertvector(f2{y[2], y[3]}, b2);
  return r.v;
}

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -INFINITY;

// Kernel geometry: D=64 -> 2 waves x 32 queries; D=128 -> 4 waves x 16 queries.
template <int D>
struct Geo {
  static constexpr int NW = D == 64 ? 2 : 4;     // waves per workgroup
  static constexpr int NCT = D == 64 ? 2 : 1;    // 16-query column tiles per wave
  static constexpr int KP = D + 8;               // LDS pitch (halfs) of Khat / P rows
  static constexpr int VP = kBlk + 8;            // LDS pitch of V^T rows
  static constexpr int DT = D / 16;              // 16-row tiles over the head dim
  static constexpr int DC = D / 32;              // 32-wide K chunks over the head dim
};

template <int D, bool FOX>
__global__ __launch_bounds__(Geo<D>::NW * 64) void fwd_mfma_kernel(
    int64_t L, int Nb, int BH, int accurate_all, float tau, const uint16_t* __restrict__ v,
    const _Float16* __restrict__ khat, const _Float16* __restrict__ pmat,
    const float* __restrict__ qhat, const float* __restrict__ sdiag,
    const float* __restrict__ kmax_head, const float* __restrict__ cum, uint16_t* __restrict__ o,
    float* __restrict__ lse) {
  using G = Geo<D>;
  constexpr int NW = G::NW, NCT = G::NCT, KP = G::KP, VP = G::VP, DT = G::DT, DC = G::DC;
  constexpr int C = kBlk;
  constexpr int NT = NW * 64;

  __shared__ __attribute__((aligned(16))) _Float16 Ks[2][C * KP];
  __shared__ __attribute__((aligned(16))) _Float16 Ps[2][D * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
  __shared__ float red[2][NW];

  // longest query blocks first, all heads of one block index together
  const int m = Nb - 1 - static_cast<int>(blockIdx.x / BH);
  const int64_t bh = blockIdx.x % BH;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 15;  // column (query) within a 16-query tile; row within A fetch
  const int lg = lane >> 4;  // lane group
  const int valid = static_cast<int>(L - static_cast<int64_t>(m) * C < C ? L - static_cast<int64_t>(m) * C : C);

  // query rows of this lane (local to block m): r = wave*16*NCT + 16*ct + ln
  const float khmax = kmax_head[bh];

  float cq[NCT];
  if constexpr (FOX) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) cq[ct] = cum[bh * Nb * C + m * C + wave * 16 * NCT + 16 * ct + ln];
  }

  f4 oacc[NCT][DT];
  f4 qf[NCT][DT];
  h8 qhi[NCT][DC], qlo[NCT][DC];
  float mrun[NCT], lrun[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    mrun[ct] = kNegInf;
    lrun[ct] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[ct][t] = f4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging helpers -------------------------------------------------------
  // V_n (64 keys x D, bf16) -> Vt[d][perm(key)]: each thread moves 4 keys x 8 dims.
  auto stage_v = [&](int n) {
    const uint16_t* src = v + (bh * L + static_cast<int64_t>(n) * C) * D;
    for (int item = tid; item < 16 * (D / 8); item += NT) {
      const int kg = item % 16;  // keys 4kg..4kg+3
      const int dg = item / 16;  // dims 8dg..8dg+7
      uint4 rw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 4 * kg + j;
        rw[j] = (static_cast<int64_t>(n) * C + key < L)
                    ? *reinterpret_cast<const uint4*>(src + key * D + 8 * dg)
                    : make_uint4(0, 0, 0, 0);
      }
      const int key0 = 4 * kg;
      const int pos = (key0 & ~31) | (((key0 >> 2) & 3) << 3) | (((key0 >> 4) & 1) << 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a0 = (&rw[0].x)[e], a1 = (&rw[1].x)[e], a2 = (&rw[2].x)[e], a3 = (&rw[3].x)[e];
        uint2 lo2, hi2;  // dims 8dg+2e (low halves) and 8dg+2e+1 (high halves)
        lo2.x = (a0 & 0xffffu) | (a1 << 16);
        lo2.y = (a2 & 0xffffu) | (a3 << 16);
        hi2.x = (a0 >> 16) | (a1 & 0xffff0000u);
        hi2.y = (a2 >> 16) | (a3 & 0xffff0000u);
        *reinterpret_cast<uint2*>(&Vt[(8 * dg + 2 * e) * VP + pos]) = lo2;
        *reinterpret_cast<uint2*>(&Vt[(8 * dg + 2 * e + 1) * VP + pos]) = hi2;
      }
    }
  };
  // rows x D halfs, contiguous in global -> LDS rows of pitch KP
  auto stage_rows = [&](_Float16* dst, const _Float16* src, int rows) {
    for (int idx = tid; idx < rows * (D / 8); idx += NT) {
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      *reinterpret_cast<uint4*>(dst + r * KP + 8 * c8) = *reinterpret_cast<const uint4*>(src + idx * 8);
    }
  };

  // ---- softmax over one 64-key tile held as S^T accumulators --------------------
  // s[ct][kt][i] = logit (log2 units) of key 16kt+4lg+i for query column ct.
  auto softmax_pv = [&](f4 (&s)[NCT][4]) {
    float mx[NCT];
    bool need = false;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float a = s[ct][0][0];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) a = fmaxf(a, s[ct][kt][i]);
      a = fmaxf(a, __shfl_xor(a, 16, 64));
      a = fmaxf(a, __shfl_xor(a, 32, 64));
      mx[ct] = a;
      need |= a > mrun[ct];
    }
    if (__any(need)) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float mn = fmaxf(mrun[ct], mx[ct]);
        const float alpha = (mrun[ct] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mrun[ct] - mn);
        lrun[ct] *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[ct][t] *= alpha;
        mrun[ct] = mn;
      }
    }
    b8 pb[NCT][2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f4 p[4];
      float acc = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kt][i] = __builtin_amdgcn_exp2f(s[ct][kt][i] - mrun[ct]);
          acc += p[kt][i];
        }
      }
      lrun[ct] += acc;
      pb[ct][0] = pack_b8(p[0], p[1]);
      pb[ct][1] = pack_b8(p[2], p[3]);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const b8 a = *reinterpret_cast<const b8*>(&Vt[(16 * t + ln) * VP + 32 * c + 8 * lg]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) oacc[ct][t] = mmb16(a, pb[ct][c], oacc[ct][t]);
      }
    }
  };

  // |Qt| max over this wave's queries -> red[slot][wave]
  auto publish_norm = [&](int slot) {
    float mx = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float s2 = 0.f;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s2 += qf[ct][t][i] * qf[ct][t][i];
      s2 += __shfl_xor(s2, 16, 64);
      s2 += __shfl_xor(s2, 32, 64);
      mx = fmaxf(mx, s2);
    }
    mx = wave_max(mx);
    if (lane == 0) red[slot][wave] = mx;
  };

  // ---- diagonal block: in-block logits from the prepare stage -------------------
  stage_v(m);
  {
    f4 s[NCT][4];
    const float* sd = sdiag + (bh * Nb + m) * (C * C);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int r = wave * 16 * NCT + 16 * ct + ln;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int c0 = 16 * kt + 4 * lg;
        f4 x = *reinterpret_cast<const f4*>(sd + r * C + c0);
        f4 ck;
        if constexpr (FOX) ck = *reinterpret_cast<const f4*>(cum + bh * Nb * C + m * C + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float val = x[i];
          if constexpr (FOX) val += cq[ct] - ck[i];
          s[ct][kt][i] = (c0 + i <= r) ? val : kNegInf;
        }
      }
    }
    __syncthreads();
    softmax_pv(s);
  }
  // boundary-adjusted queries (already multiplied by scale*log2e)
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int r = wave * 16 * NCT + 16 * ct + ln;
    const float* src = qhat + (bh * Nb * C + m * C + r) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[ct][t] = *reinterpret_cast<const f4*>(src + 16 * t + 4 * lg);
  }
  publish_norm(0);

  // ---- right-to-left scan over key blocks --------------------------------------
  for (int n = m - 1; n >= 0; --n) {
    const int slot = (m - 1 - n) & 1;
    __syncthreads();  // previous step's LDS reads are done; norms published
    float qn2 = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) qn2 = fmaxf(qn2, red[slot][w2]);
    const bool acc = accurate_all || (sqrtf(qn2) * khmax * 0.0009765625f > tau);

    const int64_t blk = bh * Nb + n;
    stage_rows(Ks[0], khat + blk * (2 * C * D), C);
    if (acc) stage_rows(Ks[1], khat + blk * (2 * C * D) + C * D, C);
    if (n > 0) {
      stage_rows(Ps[0], pmat + blk * (2 * D * D), D);
      if (acc) stage_rows(Ps[1], pmat + blk * (2 * D * D) + D * D, D);
    }
    stage_v(n);
    f4 ckv[4];
    if constexpr (FOX) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) ckv[kt] = *reinterpret_cast<const f4*>(cum + bh * Nb * C + n * C + 16 * kt + 4 * lg);
    }
    // Qt -> fp16 B operands
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        qhi[ct][c] = pack_h8(qf[ct][2 * c], qf[ct][2 * c + 1]);
        if (acc) qlo[ct][c] = pack_lo(qf[ct][2 * c], qf[ct][2 * c + 1], qhi[ct][c]);
      }
    __syncthreads();

    // S^T = Khat Qt
    f4 s[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[ct][kt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const h8 ah = *reinterpret_cast<const h8*>(&Ks[0][(16 * kt + ln) * KP + 32 * c + 8 * lg]);
        if (acc) {
          const h8 al = *reinterpret_cast<const h8*>(&Ks[1][(16 * kt + ln) * KP + 32 * c + 8 * lg]);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            s[ct][kt] = mma16(al, qhi[ct][c], s[ct][kt]);
            s[ct][kt] = mma16(ah, qlo[ct][c], s[ct][kt]);
          }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) s[ct][kt] = mma16(ah, qhi[ct][c], s[ct][kt]);
      }
    }
    if constexpr (FOX) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[ct][kt][i] += cq[ct] - ckv[kt][i];
    }
    softmax_pv(s);

    if (n > 0) {
      // Qt <- P_n Qt
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int t = 0; t < DT; ++t) qf[ct][t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const h8 ah = *reinterpret_cast<const h8*>(&Ps[0][(16 * t + ln) * KP + 32 * c + 8 * lg]);
          if (acc) {
            const h8 al = *reinterpret_cast<const h8*>(&Ps[1][(16 * t + ln) * KP + 32 * c + 8 * lg]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              qf[ct][t] = mma16(al, qhi[ct][c], qf[ct][t]);
              qf[ct][t] = mma16(ah, qlo[ct][c], qf[ct][t]);
            }
          }
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) qf[ct][t] = mma16(ah, qhi[ct][c], qf[ct][t]);
        }
      }
      publish_norm(slot ^ 1);
    }
  }

  // ---- epilogue -----------------------------------------------------------------
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float l = lrun[ct];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int r = wave * 16 * NCT + 16 * ct + ln;
    if (r < valid) {
      const float inv = 1.f / l;
      uint16_t* dst = o + (bh * L + static_cast<int64_t>(m) * C + r) * D;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const f4 x = oacc[ct][t] * inv;
        B8 pk;
        pk.p[0] = __builtin_convertvector(f2{x[0], x[1]}, b2);
        pk.p[1] = __builtin_convertvector(f2{x[2], x[3]}, b2);
        *reinterpret_cast<uint2*>(dst + 16 * t + 4 * lg) = make_uint2(
            *reinterpret_cast<const uint32_t*>(&pk.p[0]), *reinterpret_cast<const uint32_t*>(&pk.p[1]));
      }
      if (lg == 0) lse[bh * L + static_cast<int64_t>(m) * C + r] = (mrun[ct] + __log2f(l)) * kLn2;
    }
  }
}

template <int D>
static hipError_t launch_fwd_mfma_t(int64_t BH, int64_t L, int accurate, float tau, const void* v,
                                    const _Float16* khat, const _Float16* pmat, const float* qhat,
                                    const float* sdiag, const float* kmax_head, const float* cum,
                                    void* o, float* lse, hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  dim3 grid(static_cast<unsigned>(BH * Nb));
  dim3 block(Geo<D>::NW * 64);
  if (cum) {
    hipLaunchKernelGGL((fwd_mfma_kernel<D, true>), grid, block, 0, stream, L, Nb, static_cast<int>(BH),
                       accurate, tau, static_cast<const uint16_t*>(v), khat, pmat, qhat, sdiag,
                       kmax_head, cum, static_cast<uint16_t*>(o), lse);
  } else {
    hipLaunchKernelGGL((fwd_mfma_kernel<D, false>), grid, block, 0, stream, L, Nb, static_cast<int>(BH),
                       accurate, tau, static_cast<const uint16_t*>(v), khat, pmat, qhat, sdiag,
                       kmax_head, cum, static_cast<uint16_t*>(o), lse);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(int64_t B, int64_t H, int64_t L, int64_t d, int accurate, float tau,
                           const void* v, const _Float16* khat, const _Float16* pmat,
                           const float* qhat, const float* sdiag, const float* kmax_head,
                           const float* cum, void* o, float* lse, hipStream_t stream) {
  return d == 64 ? launch_fwd_mfma_t<64>(B * H, L, accurate, tau, v, khat, pmat, qhat, sdiag, kmax_head,
                                         cum, o, lse, stream)
                 : launch_fwd_mfma_t<128>(B * H, L, accurate, tau, v, khat, pmat, qhat, sdiag, kmax_head,
                                          cum, o, lse, stream);
}

}  // namespace path
