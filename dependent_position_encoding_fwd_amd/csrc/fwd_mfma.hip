// Matrix-core (MFMA) right-to-left scan forward of PaTH attention, gfx950.
//
// [PaTH Attention summary (gist.science 2505.16381), §2 "Mecanismo Central"]
//     s_ij = scale * k_j^T (H_{j+1} ... H_i) q_i   (+ FoX bias), softmax over j <= i
// [§3 "Algoritmo Estilo FlashAttention"]  A workgroup owns two consecutive
// 64-query UT blocks 2p (first half of its waves) and 2p+1 (second half).
// Each half starts from its in-block logits and its boundary-adjusted queries
// (prepare stage), then all waves scan key blocks n = 2p, 2p-1, ..., 0 right to
// left (the first half skips n = 2p, its own block).  Per key block, with
// Qt = (transported queries)^T in fp32 and logits in log2 units:
//     S^T  = Khat_n Qt - m           (keys x queries, 16x16x32 f16 MFMA; the
//                                     running max m enters as the accumulator seed)
//     online softmax over keys       (exp2; the max is only raised when a logit
//                                     exceeds it by more than kTheta)
//     O^T += V_n^T P^T               (16x16x32 f16 MFMA; an all-ones A operand
//                                     sums the same fp16 P for the denominator)
//     Qt   = P_n Qt                  (block transition P_n = H_0...H_63, f16 MFMA)
// [§2 "Extensões: PaTH-FoX"] adds cum_i - cum_j (log2 units) to each logit.
//
// Layout: everything is transposed (keys or head dims on MFMA rows, queries on
// columns) so that each 16x16 accumulator tile, converted to 16-bit, is
// directly the B operand of the next product: rows 4g..4g+3 of tiles 2c and
// 2c+1 form lane group g's 8 reduction slots of K-chunk c.  The A operands
// (Khat, P, V^T) are staged in LDS with their reduction index permuted the
// same way, so every operand fetch is one 16-byte LDS read.  The global loads
// of key block n-1 are issued into registers before the products of block n.
//
// Precision (PaTH summary §6 "Limitações" warns that bf16 makes the
// cumulative product unstable): Qt is carried in fp32 and both Qt and the
// stored Khat / P are split into fp16 hi + lo parts.  ACCURATE uses
// hi*hi + hi*lo + lo*hi for the logits and the transition on every block;
// AUTO drops the lo terms on a block when the bound
//     max|Qt| * max|khat| * 2^-10     (log2-logit units)
// is at most `tau`, where max|Qt| is measured while the split is in use and
// afterwards carried forward with the per-block bound |P_n|_2 <= pnorm_n.
// Probabilities and values meet in fp16 (fp32 accumulate).  Probabilities
// are formed as 2^(s - m + kOff): the offset keeps them clear of fp16's
// subnormal range while the lazy maximum keeps them below 2^(kTheta + kOff);
// numerator and denominator carry the same factor.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "mfma_util.h"

namespace path {
namespace {

using namespace mfma;

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -INFINITY;
constexpr float kTheta = 8.f;  // logits may exceed the running max by kTheta before it is raised
constexpr float kOff = 7.f;    // probabilities are scaled by 2^kOff (<= 2^15 < fp16 max)

// Kernel geometry: 128 queries (two UT blocks) per workgroup.
template <int D>
struct Geo {
  static constexpr int NW = D == 64 ? 4 : 8;   // waves
  static constexpr int NCT = D == 64 ? 2 : 1;  // 16-query column tiles per wave
  static constexpr int QPW = 16 * NCT;         // queries per wave
  static constexpr int WPB = 64 / QPW;         // waves per UT block
  static constexpr int NT = NW * 64;
  static constexpr int KP = D + 8;             // LDS pitch (halfs) of Khat / P rows
  static constexpr int VP = kBlk + 8;          // LDS pitch of V^T rows
  static constexpr int DT = D / 16;            // 16-row tiles over the head dim
  static constexpr int DC = D / 32;            // 32-wide K chunks over the head dim
  static constexpr int KCH = kBlk * (D / 8) / NT;  // 16-byte Khat chunks per thread
  static constexpr int PCH = D * (D / 8) / NT;     // 16-byte P chunks per thread
  static constexpr int VCH = D * (kBlk / 8) / NT;  // 16-byte V^T chunks per thread
};

}  // namespace

template <int D, bool FOX>
__global__ __launch_bounds__(Geo<D>::NT, 2) void fwd_mfma_kernel(
    int64_t L, int Nb, int BH, int accurate_all, float tau, const _Float16* __restrict__ vt,
    const _Float16* __restrict__ khat, const _Float16* __restrict__ pmat,
    const float* __restrict__ qhat, const float* __restrict__ sdiag,
    const float* __restrict__ kmax_head, const float* __restrict__ pnorm,
    const float* __restrict__ cum, uint16_t* __restrict__ o, float* __restrict__ lse) {
  using G = Geo<D>;
  constexpr int NW = G::NW, NCT = G::NCT, QPW = G::QPW, WPB = G::WPB, NT = G::NT;
  constexpr int KP = G::KP, VP = G::VP, DT = G::DT, DC = G::DC;
  constexpr int KCH = G::KCH, PCH = G::PCH, VCH = G::VCH;
  constexpr int C = kBlk;

  __shared__ __attribute__((aligned(16))) _Float16 Ks[2][C * KP];
  __shared__ __attribute__((aligned(16))) _Float16 Ps[2][D * KP];
  __shared__ __attribute__((aligned(16))) _Float16 Vt[D * VP];
  __shared__ float red[2][NW];

  const int NP = (Nb + 1) / 2;
  int p;
  int64_t bh;
  if (BH % 8 == 0) {
    // workgroups go to the 8 XCDs round robin; give XCD x the heads x, x+8, ...
    // so that the key blocks a head's tiles share stay in one L2, longest tiles first
    const int xcd = blockIdx.x % 8;
    const int j = blockIdx.x / 8;
    p = NP - 1 - (j % NP);
    bh = xcd + 8 * static_cast<int64_t>(j / NP);
  } else {
    p = NP - 1 - static_cast<int>(blockIdx.x / BH);  // longest tiles first
    bh = blockIdx.x % BH;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int half = wave / WPB;
  const int mb = 2 * p + half;                    // this wave's query block
  const bool live = mb < Nb;
  const int r0 = (wave % WPB) * QPW;              // first query row (local to block mb)
  const int64_t L64 = L;
  const float khmax = kmax_head[bh];
  const float* cumh = FOX ? cum + bh * Nb * C : nullptr;
  // this head's prepared blocks; per-block offsets stay 32-bit
  const u4* kh_h = reinterpret_cast<const u4*>(khat + bh * Nb * (2 * C * D));
  const u4* pm_h = reinterpret_cast<const u4*>(pmat + bh * Nb * (2 * D * D));
  const u4* vt_h = reinterpret_cast<const u4*>(vt + bh * Nb * (D * C));
  constexpr int KBLK = 2 * C * D / 8, PBLK = 2 * D * D / 8, VBLK = D * C / 8;  // u4 per block

  // ---- per-wave state ------------------------------------------------------------
  f4 oacc[NCT][DT], qf[NCT][DT];
  f4 lacc[NCT];  // softmax denominators (every element holds the column sum)
  h8 qhi[NCT][DC], qlo[NCT][DC];  // Qt as fp16 B operands (lo only when the split is used)
  auto to_b_operands = [&](bool with_lo) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        qhi[ct][c] = pack_h8(qf[ct][2 * c], qf[ct][2 * c + 1]);
        if (with_lo) qlo[ct][c] = pack_lo(qf[ct][2 * c], qf[ct][2 * c + 1], qhi[ct][c]);
      }
  };
  float mrun[NCT], cq[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    lacc[ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[ct][t] = f4{0.f, 0.f, 0.f, 0.f};
    cq[ct] = (FOX && live) ? cumh[mb * C + r0 + 16 * ct + ln] : 0.f;
  }

  // ---- staging helpers ----------------------------------------------------------
  // registers of the next key block (global -> VGPR prefetch)
  struct Pre {
    u4 kh[KCH], ph[PCH], vh[VCH];
    f4 ck[4];
  } pre;
  auto load_tile = [&](int n) __attribute__((always_inline)) {
    const u4* ksrc = kh_h + n * KBLK + tid;
    const u4* psrc = pm_h + n * PBLK + tid;
    const u4* vsrc = vt_h + n * VBLK + tid;
#pragma unroll
    for (int j = 0; j < KCH; ++j) pre.kh[j] = ksrc[j * NT];
    if (n > 0) {
#pragma unroll
      for (int j = 0; j < PCH; ++j) pre.ph[j] = psrc[j * NT];
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) pre.vh[j] = vsrc[j * NT];
    if constexpr (FOX) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) pre.ck[kt] = *reinterpret_cast<const f4*>(cumh + n * C + 16 * kt + 4 * lg);
    }
  };
  // 16-byte chunk idx of a row-major tile with 8 chunks (D chunks) per row -> LDS
  auto put_v = [&](_Float16* dst, int idx, const u4& x) __attribute__((always_inline)) {
    *reinterpret_cast<u4*>(&dst[(idx >> 3) * VP + 8 * (idx & 7)]) = x;
  };
  auto put_kp = [&](_Float16* dst, int idx, const u4& x) __attribute__((always_inline)) {
    *reinterpret_cast<u4*>(&dst[(idx / (D / 8)) * KP + 8 * (idx % (D / 8))]) = x;
  };
  auto store_tile = [&](int n, bool acc) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) put_kp(Ks[0], tid + j * NT, pre.kh[j]);
    if (n > 0) {
#pragma unroll
      for (int j = 0; j < PCH; ++j) put_kp(Ps[0], tid + j * NT, pre.ph[j]);
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) put_v(Vt, tid + j * NT, pre.vh[j]);
    if (acc) {
      // lo parts (split-precision blocks only) are fetched here, not prefetched
      const u4* ksrc = kh_h + n * KBLK + KBLK / 2 + tid;
#pragma unroll
      for (int j = 0; j < KCH; ++j) put_kp(Ks[1], tid + j * NT, ksrc[j * NT]);
      if (n > 0) {
        const u4* psrc = pm_h + n * PBLK + PBLK / 2 + tid;
#pragma unroll
        for (int j = 0; j < PCH; ++j) put_kp(Ps[1], tid + j * NT, psrc[j * NT]);
      }
    }
  };
  const h8 ones = h8{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};

  // ---- softmax step on logits relative to the running max -------------------------
  // x[ct][kt][i] = logit - mrun + kOff (log2 units) of key 16kt+4lg+i, query column ct.
  auto softmax_pv = [&](f4 (&x)[NCT][4], const _Float16* vts) {
    float mx[NCT];
    bool need = false;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float a = fmaxf(fmaxf(x[ct][0][0], x[ct][0][1]), fmaxf(x[ct][0][2], x[ct][0][3]));
#pragma unroll
      for (int kt = 1; kt < 4; ++kt)
        a = fmaxf(a, fmaxf(fmaxf(x[ct][kt][0], x[ct][kt][1]), fmaxf(x[ct][kt][2], x[ct][kt][3])));
      mx[ct] = grp_max(a);
      need |= mx[ct] > kTheta + kOff;
    }
    if (__any(need)) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float sh = fmaxf(mx[ct] - kOff, 0.f);
        const float alpha = __builtin_amdgcn_exp2f(-sh);
        mrun[ct] += sh;
        lacc[ct] *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[ct][t] *= alpha;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) x[ct][kt] -= sh;
      }
    }
    h8 pb[NCT][2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f4 pe[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pe[kt][i] = __builtin_amdgcn_exp2f(x[ct][kt][i]);
      pb[ct][0] = pack_h8(pe[0], pe[1]);
      pb[ct][1] = pack_h8(pe[2], pe[3]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const h8 a = *reinterpret_cast<const h8*>(&vts[(16 * t + ln) * VP + 32 * c + 8 * lg]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) oacc[ct][t] = mma16(a, pb[ct][c], oacc[ct][t]);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) lacc[ct] = mma16(ones, pb[ct][c], lacc[ct]);
    }
  };

  auto wave_qnorm = [&]() __attribute__((always_inline)) {
    float mx = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float s2 = 0.f;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s2 += qf[ct][t][i] * qf[ct][t][i];
      mx = fmaxf(mx, grp_sum(s2));
    }
    return sqrtf(wave_max(mx));
  };

  // ---- diagonal blocks: V^T of block 2p in Vt, of block 2p+1 in the Ps area -------
  _Float16* vt2 = &Ps[0][0];
  {
    const u4* va = vt_h + (2 * p) * VBLK + tid;
    const u4* vb = vt_h + (2 * p + 1) * VBLK + tid;
    const bool two = 2 * p + 1 < Nb;
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      put_v(Vt, tid + j * NT, va[j * NT]);
      if (two) put_v(vt2, tid + j * NT, vb[j * NT]);
    }
  }
  __syncthreads();
  if (live) {
    f4 x[NCT][4];
    const float* sd = sdiag + (bh * Nb + mb) * (C * C);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int r = r0 + 16 * ct + ln;
      float a = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int c0 = 16 * kt + 4 * lg;
        const f4 s = *reinterpret_cast<const f4*>(sd + r * C + c0);
        f4 ck;
        if constexpr (FOX) ck = *reinterpret_cast<const f4*>(cumh + mb * C + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float val = s[i];
          if constexpr (FOX) val += cq[ct] - ck[i];
          x[ct][kt][i] = (c0 + i <= r) ? val : kNegInf;
          a = fmaxf(a, x[ct][kt][i]);
        }
      }
      mrun[ct] = grp_max(a);  // finite: key r is always present
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) x[ct][kt] -= mrun[ct] - kOff;
    }
    softmax_pv(x, half == 0 ? Vt : vt2);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float* src = qhat + (bh * Nb * C + mb * C + r0 + 16 * ct + ln) * D;
#pragma unroll
      for (int t = 0; t < DT; ++t) qf[ct][t] = *reinterpret_cast<const f4*>(src + 16 * t + 4 * lg);
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      mrun[ct] = 0.f;
#pragma unroll
      for (int t = 0; t < DT; ++t) qf[ct][t] = f4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const float qn0 = wave_qnorm();
  if (lane == 0) red[0][wave] = qn0;
  __syncthreads();  // diagonal reads of Vt / Ps done; norms visible

  // precision of key block 2p from the norms of the adjusted queries
  float qbound = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) qbound = fmaxf(qbound, red[0][w2]);
  bool acc_cur = accurate_all || (qbound * khmax * 0.0009765625f > tau);
  load_tile(2 * p);
  to_b_operands(acc_cur);

  // ---- right-to-left scan ----------------------------------------------------------
  for (int n = 2 * p; n >= 0; --n) {
    store_tile(n, acc_cur);
    f4 ck[4];
    if constexpr (FOX) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) ck[kt] = pre.ck[kt];
    }
    __syncthreads();
    // precision of block n-1: bound on |Qt| after this block's transition
    const float qb_next = qbound * pnorm[bh * Nb + n];
    const bool acc_next = accurate_all || (qb_next * khmax * 0.0009765625f > tau);
    if (n > 0) load_tile(n - 1);
    const bool acc = acc_cur;
    const bool work = live && !(half == 0 && n == 2 * p);

    if (work) {
      // S^T - m = Khat Qt - m: the first chunk's products start from the seed
      // quad (-m, or cum_i - m with forget gates); the lo passes come last
      f4 x[NCT][4];
      f4 seed[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float sv = (FOX ? cq[ct] : 0.f) - mrun[ct] + kOff;
        seed[ct] = f4{sv, sv, sv, sv};
      }
#pragma unroll
      for (int c = 0; c < DC; ++c) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const h8 ah = *reinterpret_cast<const h8*>(&Ks[0][(16 * kt + ln) * KP + 32 * c + 8 * lg]);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) x[ct][kt] = mma16(ah, qhi[ct][c], c == 0 ? seed[ct] : x[ct][kt]);
        }
      }
      if (acc) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            const h8 al = *reinterpret_cast<const h8*>(&Ks[1][(16 * kt + ln) * KP + 32 * c + 8 * lg]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) x[ct][kt] = mma16(al, qhi[ct][c], x[ct][kt]);
          }
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            const h8 ah = *reinterpret_cast<const h8*>(&Ks[0][(16 * kt + ln) * KP + 32 * c + 8 * lg]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) x[ct][kt] = mma16(ah, qlo[ct][c], x[ct][kt]);
          }
        }
      }
      // the transition of Qt needs neither the softmax nor PV: issue it first so
      // that its products overlap the softmax arithmetic
      if (n > 0) {
        // Qt <- P_n Qt (first chunk from zero; lo passes last)
        const f4 zero = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DC; ++c) {
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            const h8 ah = *reinterpret_cast<const h8*>(&Ps[0][(16 * t + ln) * KP + 32 * c + 8 * lg]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) qf[ct][t] = mma16(ah, qhi[ct][c], c == 0 ? zero : qf[ct][t]);
          }
        }
        if (acc) {
#pragma unroll
          for (int c = 0; c < DC; ++c) {
#pragma unroll
            for (int t = 0; t < DT; ++t) {
              const h8 al = *reinterpret_cast<const h8*>(&Ps[1][(16 * t + ln) * KP + 32 * c + 8 * lg]);
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct) qf[ct][t] = mma16(al, qhi[ct][c], qf[ct][t]);
            }
#pragma unroll
            for (int t = 0; t < DT; ++t) {
              const h8 ah = *reinterpret_cast<const h8*>(&Ps[0][(16 * t + ln) * KP + 32 * c + 8 * lg]);
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct) qf[ct][t] = mma16(ah, qlo[ct][c], qf[ct][t]);
            }
          }
        }
      }
      if constexpr (FOX) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) x[ct][kt] -= ck[kt];
      }
      softmax_pv(x, Vt);
    }
    // measured norms while the split is in use; the carried bound otherwise
    const int slot = n & 1;
    if (acc_next && n > 0) {
      const float qn = (work || !live) ? wave_qnorm() : 0.f;
      if (lane == 0) red[slot][wave] = qn;
    }
    if (work && n > 0) to_b_operands(acc_next);
    __syncthreads();  // LDS reads of this block are done; norms visible
    if (acc_next && n > 0) {
      float qm = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) qm = fmaxf(qm, red[slot][w2]);
      // waves that skipped this block still hold their previous (untransported) queries
      qbound = fmaxf(qm, (n == 2 * p) ? qbound : 0.f);
    } else {
      qbound = qb_next;
    }
    // the measured norm never exceeds the carried bound, so block n-1 never
    // needs lo parts that were not fetched
    acc_cur = acc_next && (accurate_all || (qbound * khmax * 0.0009765625f > tau));
  }

  // ---- epilogue -------------------------------------------------------------------
  if (live) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float l = lacc[ct][0];
      const int r = r0 + 16 * ct + ln;
      const int64_t row = static_cast<int64_t>(mb) * C + r;
      if (row < L64) {
        const float inv = 1.f / l;
        uint16_t* dst = o + (bh * L64 + row) * D;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const f4 y = oacc[ct][t] * inv;
          B8 pk;
          pk.p[0] = __builtin_convertvector(f2{y[0], y[1]}, b2);
          pk.p[1] = __builtin_convertvector(f2{y[2], y[3]}, b2);
          *reinterpret_cast<uint2*>(dst + 16 * t + 4 * lg) = make_uint2(pk.u.x, pk.u.y);
        }
        if (lg == 0) lse[bh * L64 + row] = (mrun[ct] - kOff + __log2f(l)) * kLn2;
      }
    }
  }
}

template <int D>
static hipError_t launch_fwd_mfma_t(int64_t BH, int64_t L, int accurate, float tau, const _Float16* vt,
                                    const _Float16* khat, const _Float16* pmat, const float* qhat,
                                    const float* sdiag, const float* kmax_head, const float* pnorm,
                                    const float* cum, void* o, float* lse, hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  const int NP = (Nb + 1) / 2;
  dim3 grid(static_cast<unsigned>(BH * NP));
  dim3 block(Geo<D>::NT);
  if (cum) {
    hipLaunchKernelGGL((fwd_mfma_kernel<D, true>), grid, block, 0, stream, L, Nb, static_cast<int>(BH),
                       accurate, tau, vt, khat, pmat, qhat, sdiag,
                       kmax_head, pnorm, cum, static_cast<uint16_t*>(o), lse);
  } else {
    hipLaunchKernelGGL((fwd_mfma_kernel<D, false>), grid, block, 0, stream, L, Nb, static_cast<int>(BH),
                       accurate, tau, vt, khat, pmat, qhat, sdiag,
                       kmax_head, pnorm, cum, static_cast<uint16_t*>(o), lse);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(int64_t B, int64_t H, int64_t L, int64_t d, int accurate, float tau,
                           const _Float16* vt, const _Float16* khat, const _Float16* pmat,
                           const float* qhat, const float* sdiag, const float* kmax_head,
                           const float* kmax_blk, const float* pnorm, const float* cum, void* o, float* lse,
                           hipStream_t stream) {
  if (d == 64)
    return launch_scan64(B * H, L, accurate, tau, vt, khat, pmat, qhat, sdiag, kmax_head, kmax_blk, pnorm, cum, o,
                         lse, stream);
  return launch_scan128(B * H, L, accurate, tau, vt, khat, pmat, qhat, sdiag, kmax_head, kmax_blk, pnorm, cum, o,
                        lse, stream);
}

}  // namespace path
