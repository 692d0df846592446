// Right-to-left scan forward of PaTH attention for head dimension 128 (gfx950),
// with the key-side operands streamed into LDS by direct-to-LDS loads.
//
// [PaTH Attention summary (gist.science 2505.16381), §2 "Mecanismo Central"]
//     s_ij = scale * k_j^T (H_{j+1} ... H_i) q_i   (+ FoX bias), softmax over j <= i
// [§3 "Algoritmo Estilo FlashAttention"]  A workgroup of 8 waves owns the
// 64-query blocks 2p and 2p+1 (4 waves of 16 queries each), starts each from
// its in-block logits and boundary-adjusted queries, and walks key blocks
// n = 2p .. 0 with
//     S^T = Khat_n Qt - m,  online softmax (exp2),  O^T += V_n^T P^T,  Qt = P_n Qt.
// [§2 "Extensões: PaTH-FoX"] adds cum_i - cum_j (log2 units) to each logit.
//
// The arithmetic and data layouts are those of the head-dimension-64 scan; the
// tiles are larger (Khat_n 64x128, P_n 128x128, V_n^T 128x64 in fp16: 16, 32
// and 16 KB), which sets the LDS plan (144 KB, one workgroup per CU):
//   * Khat_n and V_n^T have two stages: block n-1 is fetched while block n is
//     computed; one barrier at the end of a block publishes it.
//   * P_n has one stage.  Once every wave has finished the transition of the
//     queries (the only reader of P_n), a barrier frees it and P_{n-1} is
//     fetched; it lands during the PV products and is published by the same
//     end-of-block barrier.
//   * The fp16 lo parts of Khat_n and P_n (split-precision blocks only) have
//     one stage.  They are fetched with P_{n-1}, once this block's
//     split-precision products are done.
//   * With forget gates, the gate prefix of the 64 keys (256 bytes) travels
//     with Khat and V^T.
//   * Rows of 16 chunks (Khat, P) keep chunk j of row r at j ^ (r & 15), rows
//     of 8 chunks (V^T) at j ^ (r & 7), so that the MFMA operand reads (16
//     rows, one chunk column) run at the full LDS read rate.
// Each tile is its own LDS object and every access names it at compile time.
// The direct loads are issued from asm (lds_dma16), so the compiler's waits on
// LDS reads stay counted; the barriers that publish a stage wait for them.
// Value range: prepare stores block n's V^T times 2^-e_n (e_n > 0 only when
// the block holds |v| >= 2^15); a tile takes E = max e_n over the blocks its
// queries weigh.  O accumulates in units of 2^E: on a block with e_n < E
// (never where all are 0, as on an ordinary head) a scalar branch multiplies
// the V^T operands by 2^(e_n - E).  The epilogue multiplies by 2^E.
#include <math.h>

#include <type_traits>

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

constexpr int kD = 128;            // head dimension
constexpr int kNW = 8;             // waves
constexpr int kNT = 64 * kNW;      // threads
constexpr int kWPB = 4;            // waves per 64-query block
constexpr int kKT = 64 * kD;       // halfs of a Khat tile (64 x 128)
constexpr int kPT = kD * kD;       // halfs of a P tile (128 x 128)
constexpr int kVT = kD * 64;       // halfs of a V^T tile (128 x 64)

// Barrier that also publishes every direct-to-LDS load this wave issued (see
// the head-dimension-64 scan for why the wait is a builtin and the barrier an
// asm statement with a memory clobber).
__device__ __forceinline__ void sync_dma() {
  __builtin_amdgcn_s_waitcnt(0x0070);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}
// Barrier after this wave's LDS reads are done (no wait on global loads).
__device__ __forceinline__ void sync_lds() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("s_barrier" ::: "memory");
}

}  // namespace

template <bool FOX>
__global__ __launch_bounds__(kNT, 1) void scan128_kernel(
    int64_t L, int Nb, int BH, int accurate_all, float tau, const _Float16* __restrict__ vt,
    const _Float16* __restrict__ khat, const _Float16* __restrict__ pmat,
    const float* __restrict__ qhat, const float* __restrict__ sdiag,
    const float* __restrict__ kmax_blk, const float* __restrict__ pnorm,
    const int* __restrict__ vexp, const float* __restrict__ cum, uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int D = kD, C = kBlk, DT = D / 16, DC = D / 32;

  __shared__ __attribute__((aligned(1024))) _Float16 sK0[kKT], sV0[kVT];
  __shared__ __attribute__((aligned(1024))) _Float16 sK1[kKT], sV1[kVT];
  __shared__ __attribute__((aligned(1024))) _Float16 sP[kPT];
  __shared__ __attribute__((aligned(1024))) _Float16 sKl[kKT], sPl[kPT];
  __shared__ __attribute__((aligned(16))) float sC0[64], sC1[64];  // gate prefix of the keys
  __shared__ float red[2][kNW];

  const int NP = (Nb + 1) / 2;
  int p;
  int64_t bh;
  if (BH % 8 == 0) {
    // XCD x takes the heads x, x+8, ... (their key blocks stay in one L2),
    // in pairs, the tiles of a pair longest first
    const int xcd = blockIdx.x % 8;
    const int j = blockIdx.x / 8;
    const int HX = BH / 8;
    const int g = j / (2 * NP), r = j % (2 * NP);
    int hh;
    if (2 * g + 1 < HX) {
      p = NP - 1 - r / 2;
      hh = 2 * g + (r & 1);
    } else {
      p = NP - 1 - r;
      hh = 2 * g;
    }
    bh = xcd + 8 * static_cast<int64_t>(hh);
  } else {
    p = NP - 1 - static_cast<int>(blockIdx.x / BH);  // longest tiles first
    bh = blockIdx.x % BH;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int half = wave / kWPB;
  const int mb = 2 * p + half;        // this wave's query block
  const bool live = mb < Nb;
  const int r0 = (wave % kWPB) * 16;  // first query row (local to block mb)
  // The largest key norm over the key blocks this tile scans (0 .. 2p: the
  // only logits that a transported query's rounding reaches) and the largest
  // value exponent over the blocks whose values it weighs (0 .. 2p+1), from
  // the per-block figures of the prepare stage.
  float khmax;
  int vE;  // 0 unless some value of those blocks reaches 2^15
  {
    const int nlast = 2 * p + 1 < Nb ? 2 * p + 1 : Nb - 1;
    float km = 0.f, vm = 0.f;
    for (int b0 = 0; b0 <= nlast; b0 += 64) {
      const int nb = b0 + lane;
      if (nb <= 2 * p) km = fmaxf(km, kmax_blk[bh * Nb + nb]);
      if (nb <= nlast) vm = fmaxf(vm, static_cast<float>(vexp[bh * Nb + nb]));
    }
    khmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max_dpp(km))));
    vE = __builtin_amdgcn_readfirstlane(static_cast<int>(wave_max_dpp(vm)));
  }
  // 2^(e_n - E) in fp16 for block n's V^T operands (0 below fp16's subnormals)
  auto vscale = [&](int n) __attribute__((always_inline)) {
    const int g = vE - vexp[bh * Nb + n];
    const _Float16 f = static_cast<_Float16>(g > 24 ? 0.f : __uint_as_float(static_cast<uint32_t>(127 - g) << 23));
    return h8{f, f, f, f, f, f, f, f};
  };
  const float* cumh = FOX ? cum + bh * Nb * C : nullptr;

  // this head's prepared blocks (hi tile, then lo tile, per block)
  const char* kh_h = reinterpret_cast<const char*>(khat + bh * Nb * (2 * kKT));
  const char* pm_h = reinterpret_cast<const char*>(pmat + bh * Nb * (2 * kPT));
  const char* vt_h = reinterpret_cast<const char*>(vt + bh * Nb * kVT);
  constexpr int TBK = kKT * 2, TBP = kPT * 2, TBV = kVT * 2;  // bytes per tile

  // ---- direct-to-LDS staging ------------------------------------------------------
  // Slot i of this wave covers LDS chunks (NS*wave + i)*64 + lane of a tile; the
  // lane fetches the logical chunk that belongs there.
  uint32_t goffK[2], goffP[4], goffV[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pos = (2 * wave + i) * 64 + lane;
    const int r = pos >> 4;
    goffK[i] = static_cast<uint32_t>(r * 256 + ((pos & 15) ^ (r & 15)) * 16);
    const int rv = pos >> 3;
    goffV[i] = static_cast<uint32_t>(rv * 128 + ((pos & 7) ^ (rv & 7)) * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pos = (4 * wave + i) * 64 + lane;
    const int r = pos >> 4;
    goffP[i] = static_cast<uint32_t>(r * 256 + ((pos & 15) ^ (r & 15)) * 16);
  }
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto tileK = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return sK0; else return sK1;
  };
  auto tileV = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return sV0; else return sV1;
  };
  auto dmaK = [&](int n, _Float16* ltile) __attribute__((always_inline)) {
    const char* g = kh_h + static_cast<int64_t>(n) * (2 * TBK);
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(g + goffK[i], ltile + (2 * wave + i) * 512);
  };
  auto dmaV = [&](int n, _Float16* ltile) __attribute__((always_inline)) {
    const char* g = vt_h + static_cast<int64_t>(n) * TBV;
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(g + goffV[i], ltile + (2 * wave + i) * 512);
  };
  auto dmaP = [&](int n) __attribute__((always_inline)) {
    const char* g = pm_h + static_cast<int64_t>(n) * (2 * TBP);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(g + goffP[i], sP + (4 * wave + i) * 512);
  };
  // lo parts: the same slots in the lo tiles
  auto dmaLo = [&](int n) __attribute__((always_inline)) {
    const char* gk = kh_h + static_cast<int64_t>(n) * (2 * TBK) + TBK;
    const char* gp = pm_h + static_cast<int64_t>(n) * (2 * TBP) + TBP;
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(gk + goffK[i], sKl + (2 * wave + i) * 512);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(gp + goffP[i], sPl + (4 * wave + i) * 512);
  };
  // gate prefix of block n's keys: 16 lanes of wave 0 move its 256 bytes
  auto tileC = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return sC0; else return sC1;
  };
  auto dmaC = [&](int n, float* ltile) __attribute__((always_inline)) {
    if (wave == 0 && lane < 16)
      lds_dma16(cumh + n * C + 4 * lane, ltile);
  };
  // MFMA A operands.  Khat / P (16 chunks per row): rows 16t + ln, logical chunk
  // 4c + lg.  V^T (8 chunks per row): rows 16t + ln, logical chunk 4c + lg, c < 2.
  int aoff16[DC], aoffV[2];
#pragma unroll
  for (int c = 0; c < DC; ++c) aoff16[c] = ln * 128 + ((4 * c + lg) ^ ln) * 8;
#pragma unroll
  for (int c = 0; c < 2; ++c) aoffV[c] = ln * 64 + ((4 * c + lg) ^ (ln & 7)) * 8;
  auto rdA16 = [&](const _Float16* tile, int t, int c) __attribute__((always_inline)) {
    return *reinterpret_cast<const h8*>(tile + t * 2048 + aoff16[c]);
  };
  auto rdV = [&](const _Float16* tile, int t, int c) __attribute__((always_inline)) {
    return *reinterpret_cast<const h8*>(tile + t * 1024 + aoffV[c]);
  };

  // ---- per-wave state (16 queries: column ln of the accumulator tiles) ------------
  f4 oacc[DT], qf[DT];
  f4 lacc;  // softmax denominator (every element holds the column sum)
  h8 qhi[DC], qlo[DC];
  auto to_b_operands = [&](bool with_lo) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      qhi[c] = pack_h8(qf[2 * c], qf[2 * c + 1]);
      if (with_lo) qlo[c] = pack_lo(qf[2 * c], qf[2 * c + 1], qhi[c]);
    }
  };
  float mrun, cq;
  f4 seed;         // cq - mrun + kOff: the accumulator start of S^T
  float mrun_min;  // min of mrun over the wave's queries
  auto set_seeds = [&]() __attribute__((always_inline)) {
    const float sv = (FOX ? cq : 0.f) - mrun + kOff;
    seed = f4{sv, sv, sv, sv};
    mrun_min = -wave_max_dpp(-mrun);
  };
  lacc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f4{0.f, 0.f, 0.f, 0.f};
  cq = (FOX && live) ? cumh[mb * C + r0 + ln] : 0.f;
  const h8 ones = h8{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};

  // exponentials of x (logit - mrun + kOff) as the two fp16 B operands of PV
  auto exps = [&](const f4 (&x)[4], h8 (&pb)[2]) __attribute__((always_inline)) {
    f4 pe[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pe[kt][i] = __builtin_amdgcn_exp2f(x[kt][i]);
    pb[0] = pack_h8(pe[0], pe[1]);
    pb[1] = pack_h8(pe[2], pe[3]);
  };
  auto rowmax = [&](const f4 (&x)[4]) __attribute__((always_inline)) {
    float a = fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3]));
#pragma unroll
    for (int kt = 1; kt < 4; ++kt) a = fmaxf(a, fmaxf(fmaxf(x[kt][0], x[kt][1]), fmaxf(x[kt][2], x[kt][3])));
    return grp_max(a);
  };
  auto rescale = [&](float mx, f4 (&x)[4]) __attribute__((always_inline)) {
    const float sh = fmaxf(mx - kOff, 0.f);
    const float alpha = __builtin_amdgcn_exp2f(-sh);
    mrun += sh;
    lacc *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) x[kt] -= sh;
  };
  auto pv = [&](const _Float16* vtile, const h8 (&pb)[2], bool vsc, h8 vs8) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] = mma16(vsc ? rdV(vtile, t, c) * vs8 : rdV(vtile, t, c), pb[c], oacc[t]);
      lacc = mma16(ones, pb[c], lacc);
    }
  };

  auto wave_qnorm = [&]() __attribute__((always_inline)) {
    float s2 = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) s2 += qf[t][i] * qf[t][i];
    return sqrtf(wave_max_dpp(grp_sum(s2)));
  };

  // ---- diagonal blocks, and the operands of key block 2p ------------------------------
  // V^T of block 2p lands in stage 0 (it is also the first scanned block); that
  // of block 2p+1 uses stage 1's V^T tile, free until the first prefetch.
  dmaK(2 * p, sK0);
  dmaV(2 * p, sV0);
  dmaP(2 * p);
  if (2 * p + 1 < Nb) dmaV(2 * p + 1, sV1);
  dmaLo(2 * p);  // used only if block 2p runs the split products
  if constexpr (FOX) dmaC(2 * p, sC0);
  f4 sdv[4], ckd[4];
  if (live) {
    const float* sd = sdiag + (bh * Nb + mb) * kDiagTri + diag_row(r0 + ln);
    const int r = r0 + ln;
    // the stored chunks of row r (padded triangle); the others are masked below
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      sdv[kt] = 16 * kt + 4 * lg <= r ? *reinterpret_cast<const f4*>(sd + 16 * kt + 4 * lg) : f4{0.f, 0.f, 0.f, 0.f};
    const float* src = qhat + (bh * Nb * C + mb * C + r) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = *reinterpret_cast<const f4*>(src + 16 * t + 4 * lg);
    if constexpr (FOX) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) ckd[kt] = *reinterpret_cast<const f4*>(cumh + mb * C + 16 * kt + 4 * lg);
    }
  }
  sync_dma();
  if (live) {
    f4 x[4];
    const int r = r0 + ln;
    float a = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int c0 = 16 * kt + 4 * lg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float val = sdv[kt][i];
        if constexpr (FOX) val += cq - ckd[kt][i];
        x[kt][i] = (c0 + i <= r) ? val : kNegInf;
        a = fmaxf(a, x[kt][i]);
      }
    }
    mrun = grp_max(a);  // finite: key r is always present
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) x[kt] -= mrun - kOff;
    h8 pb[2];
    exps(x, pb);
    const bool dsc = vE != 0 && vexp[bh * Nb + mb] != vE;
    pv(half == 0 ? sV0 : sV1, pb, dsc, dsc ? vscale(mb) : h8{});
  } else {
    mrun = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = f4{0.f, 0.f, 0.f, 0.f};
  }
  set_seeds();
  const float qn0 = wave_qnorm();
  if (lane == 0) red[0][wave] = qn0;
  sync_dma();  // stage 1 is free for the first prefetch; norms visible

  float qbound = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < kNW; ++w2) qbound = fmaxf(qbound, red[0][w2]);
  bool acc_cur = accurate_all || (qbound * khmax * 0.0009765625f > tau);
  to_b_operands(acc_cur);

  // ---- right-to-left scan ----------------------------------------------------------
  // Per-block transition norms and key maxima, 64 blocks per register window
  // (lane j holds block wb - j).  Vector loads: the waits on LDS reads in the
  // loop then never include a scalar-memory fetch.
  int wb = 2 * p;
  float pnw, knw;
  auto load_window = [&]() __attribute__((always_inline)) {
    const int64_t m = bh * Nb + (wb >= lane ? wb - lane : 0);
    pnw = pnorm[m];
    knw = kmax_blk[m];
  };
  load_window();
  auto step = [&](int n, auto st) __attribute__((always_inline)) {
    using SN = std::integral_constant<int, 1 - decltype(st)::value>;
    const _Float16* tK = tileK(st);
    const _Float16* tV = tileV(st);
    const float pn_cur = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pnw), wb - n));
    const float kn_cur = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(knw), wb - n));
    if (n > 0 && wb - n == 63) {  // block n-1 opens the next window
      wb = n - 1;
      load_window();
    }
    if (n > 0) {
      dmaK(n - 1, tileK(SN{}));
      dmaV(n - 1, tileV(SN{}));
      if constexpr (FOX) dmaC(n - 1, tileC(SN{}));
    }
    const float qb_next = qbound * pn_cur;
    const bool acc_next = accurate_all || (qb_next * khmax * 0.0009765625f > tau);
    const bool work = live && !(half == 0 && n == 2 * p);
    // no logit of this block can pass the running max by kTheta when
    // |Qt| * max|khat| (Cauchy-Schwarz; 1.01 covers the fp16 operands) stays below it
    const bool skip_max = !FOX && (qbound * kn_cur * 1.01f <= mrun_min + kTheta);

    // The block's operands stream from LDS in chunks of 8 reads (one 16-row
    // tile column each): Khat c=0,1 | Khat c=2,3 | P c=0 | P c=1 | P c=2 | P c=3 |
    // V^T c=0 | V^T c=1.  Each group issues the reads of the next chunk, then the
    // products of the current one, so one chunk's reads run under the previous
    // chunk's products; two chunks are live at a time.  The vector work (row
    // maximum, exponentials, conversion of the transported queries) sits beside
    // the products it does not feed.
    f4 x[4];
    h8 pb[2];
    h8 ch0[8], ch1[8];
    auto rdK = [&](h8 (&b)[8], int c0) __attribute__((always_inline)) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) b[4 * cc + kt] = rdA16(tK, kt, c0 + cc);
    };
    auto rdP = [&](h8 (&b)[8], int c) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < DT; ++t) b[t] = rdA16(sP, t, c);
    };
    auto rdVc = [&](h8 (&b)[8], int c) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < DT; ++t) b[t] = rdV(tV, t, c);
    };
    auto mmP = [&](const h8 (&b)[8], int c) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < DT; ++t) qf[t] = mma16(b[t], qhi[c], c == 0 ? f4{0.f, 0.f, 0.f, 0.f} : qf[t]);
    };
    auto mmV = [&](const h8 (&b)[8], int c) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] = mma16(b[t], pb[c], oacc[t]);
      lacc = mma16(ones, pb[c], lacc);
    };
    if (work) {
      // ---- S^T = Khat Qt - m + kOff
      rdK(ch0, 0);
      __builtin_amdgcn_sched_barrier(0);
      rdK(ch1, 2);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) x[kt] = mma16(ch0[4 * cc + kt], qhi[cc], cc == 0 ? seed : x[kt]);
      __builtin_amdgcn_sched_barrier(0);
      rdP(ch0, 0);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) x[kt] = mma16(ch1[4 * cc + kt], qhi[2 + cc], x[kt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (acc_cur) {
      // the lo tiles were published by the previous block's barrier.  The
      // logits' own correction needs only this block's max |khat|; the
      // transport's (below) reaches every earlier block and keeps the maximum
      // over all the key blocks the tile scans.
      if (work && (accurate_all || qbound * kn_cur * 0.0009765625f > tau)) {
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            x[kt] = mma16(rdA16(sKl, kt, c), qhi[c], x[kt]);
            x[kt] = mma16(rdA16(tK, kt, c), qlo[c], x[kt]);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (work) {
      // ---- Qt <- P_n Qt, chunk 0, beside the row maximum
      rdP(ch1, 1);
      mmP(ch0, 0);
      float mx = 0.f;
      if (!skip_max) {
        if constexpr (FOX) {
          const float* cs = tileC(st);
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) x[kt] -= *reinterpret_cast<const f4*>(cs + 16 * kt + 4 * lg);
        }
        mx = rowmax(x);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (!skip_max && __any(mx > kTheta + kOff)) {  // rare: raise the running max
        rescale(mx, x);
        set_seeds();
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- chunk 1 beside the exponentials
      rdP(ch0, 2);
      mmP(ch1, 1);
      exps(x, pb);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);  // exp
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // other vector ALU
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- chunks 2 and 3
      rdP(ch1, 3);
      mmP(ch0, 2);
      __builtin_amdgcn_sched_barrier(0);
      rdVc(ch0, 0);
      mmP(ch1, 3);
      __builtin_amdgcn_sched_barrier(0);
      if (acc_cur) {
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            qf[t] = mma16(rdA16(sPl, t, c), qhi[c], qf[t]);
            qf[t] = mma16(rdA16(sP, t, c), qlo[c], qf[t]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // P_n and the lo tiles are read by no one any more: fetch block n-1's
    if (n > 0) {
      sync_lds();
      dmaP(n - 1);
      if (acc_next) dmaLo(n - 1);
    }
    if (work) {
      // ---- PV beside the conversion of the transported queries
      const bool vsn = vE != 0 && vexp[bh * Nb + n] != vE;  // rare: values in the tile's units
      if (vsn) {
        const h8 f8 = vscale(n);
#pragma unroll
        for (int t = 0; t < DT; ++t) ch0[t] *= f8;
      }
      rdVc(ch1, 1);
      mmV(ch0, 0);
#pragma unroll
      for (int c = 0; c < DC; ++c) qhi[c] = pack_h8(qf[2 * c], qf[2 * c + 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (vsn) {
        const h8 f8 = vscale(n);
#pragma unroll
        for (int t = 0; t < DT; ++t) ch1[t] *= f8;
      }
      mmV(ch1, 1);
      if (acc_next) {
        asm volatile("");  // a real branch: the lo parts are rarely needed
#pragma unroll
        for (int c = 0; c < DC; ++c) qlo[c] = pack_lo(qf[2 * c], qf[2 * c + 1], qhi[c]);
      }
    }
    // measured norms while the split is in use; the carried bound otherwise
    const int slot = n & 1;
    if (acc_next && n > 0) {
      const float qn = (work || !live) ? wave_qnorm() : 0.f;
      if (lane == 0) red[slot][wave] = qn;
    }
    sync_dma();  // next stages landed; this stage's reads done; norms visible
    if (acc_next && n > 0) {
      float qm = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kNW; ++w2) qm = fmaxf(qm, red[slot][w2]);
      // waves that skipped this block still hold their previous (untransported) queries
      qbound = fmaxf(qm, (n == 2 * p) ? qbound : 0.f);
    } else {
      qbound = qb_next;
    }
    acc_cur = acc_next && (accurate_all || (qbound * khmax * 0.0009765625f > tau));
  };

  for (int n = 2 * p; n >= 0; n -= 2) {
    step(n, S0{});
    if (n > 0) step(n - 1, S1{});
  }

  // ---- epilogue -------------------------------------------------------------------
  if (live) {
    const float l = lacc[0];
    const int r = r0 + ln;
    const int64_t row = static_cast<int64_t>(mb) * C + r;
    if (row < L) {
      const float inv = __builtin_ldexpf(1.f / l, vE);
      uint16_t* dst = o + (bh * L + row) * D;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const f4 y = oacc[t] * inv;
        B8 pk;
        pk.p[0] = __builtin_convertvector(f2{y[0], y[1]}, b2);
        pk.p[1] = __builtin_convertvector(f2{y[2], y[3]}, b2);
        *reinterpret_cast<uint2*>(dst + 16 * t + 4 * lg) = make_uint2(pk.u.x, pk.u.y);
      }
      if (lg == 0) lse[bh * L + row] = (mrun - kOff + __log2f(l)) * kLn2;
    }
  }
}

hipError_t launch_scan128(int64_t BH, int64_t L, int accurate, float tau, const _Float16* vt,
                          const _Float16* khat, const _Float16* pmat, const float* qhat, const float* sdiag,
                          const float* kmax_blk, const float* pnorm, const int* vexp,
                          const float* cum, void* o, float* lse, hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  const int NP = (Nb + 1) / 2;
  dim3 grid(static_cast<unsigned>(BH * NP));
  dim3 block(kNT);
  if (cum) {
    hipLaunchKernelGGL((scan128_kernel<true>), grid, block, 0, stream, L, Nb, static_cast<int>(BH), accurate, tau,
                       vt, khat, pmat, qhat, sdiag, kmax_blk, pnorm, vexp, cum,
                       static_cast<uint16_t*>(o), lse);
  } else {
    hipLaunchKernelGGL((scan128_kernel<false>), grid, block, 0, stream, L, Nb, static_cast<int>(BH), accurate, tau,
                       vt, khat, pmat, qhat, sdiag, kmax_blk, pnorm, vexp, cum,
                       static_cast<uint16_t*>(o), lse);
  }
  return hipGetLastError();
}

}  // namespace path
