// Right-to-left scan forward of PaTH attention for head dimension 64 (gfx950),
// with the key-side operands streamed into LDS by direct-to-LDS loads.
//
// [PaTH Attention summary (gist.science 2505.16381), §2 "Mecanismo Central"]
//     s_ij = scale * k_j^T (H_{j+1} ... H_i) q_i   (+ FoX bias), softmax over j <= i
// [§3 "Algoritmo Estilo FlashAttention"]  A workgroup of 4 waves owns the
// 64-query blocks 2p and 2p+1, starts each from its in-block logits and
// boundary-adjusted queries, and walks key blocks n = 2p .. 0 with
//     S^T = Khat_n Qt - m,  online softmax (exp2),  O^T += V_n^T P^T,  Qt = P_n Qt.
// Products take fp16 operands and fp32 accumulators; a computed fp32 operand
// (Qt) is split into fp16 hi + lo on the blocks where a run-time estimate of
// the rounding error says the lo part matters (split precision), and
// probabilities are 2^(s - m + 7) in fp16.
//
// The data movement is built for CDNA4:
//   * Khat_n, P_n and V_n^T (fp16, 8 KB each) travel global -> LDS with
//     global_load_lds_dwordx4: each lane names its source, the data land at
//     consecutive 16-byte slots, no VGPRs or LDS store instructions involved.
//   * Two LDS stages: block n-1 is fetched while block n is computed, and one
//     barrier per key block both publishes the next stage and retires this one.
//   * Tiles are stored without padding; 16-byte chunk j of row r sits at slot
//     j ^ (r & 7), which keeps the MFMA operand reads (16 rows, one chunk
//     column) at the LDS's full 128-bit read rate.
//   * The fp16 lo parts of Khat_n and P_n, needed only on blocks that run the
//     split-precision products, are fetched one block ahead into registers
//     (4 x 16 bytes per thread), stored into a single LDS stage at the start
//     of the block and published by a second barrier once the hi products are
//     issued.
// [§2 "Extensões: PaTH-FoX"] adds cum_i - cum_j (log2 units) to each logit.
//
// Value range: prepare stores block n's V^T times 2^-e_n (e_n > 0 only when
// the block holds |v| >= 2^15); a tile takes E = max e_n over the blocks its
// queries weigh.  O accumulates in units of 2^E: on a block with e_n < E
// (never where all are 0, as on an ordinary head) a scalar branch multiplies
// the V^T operands by 2^(e_n - E) (exact, or below fp16's range only where
// the contribution is far below the largest values the tile weighs).  The
// epilogue multiplies by 2^E.
//
// LDS: 8 tiles x 8 KB = 64 KB per workgroup, so two workgroups share a CU.
// Each tile is its own LDS object and every access names its object at
// compile time (the scan is unrolled by the two stages).  The direct loads are
// issued from asm (lds_dma16), so the compiler's waits on LDS reads stay
// counted; the barrier that publishes a stage waits for them.
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

constexpr int kD = 64;                 // head dimension
constexpr int kNW = 4;                 // waves
constexpr int kNT = 64 * kNW;          // threads
constexpr int kTile = 64 * 64;         // halfs per 64 x 64 fp16 tile (8 KB)
constexpr int kRowT = 16 * 64;         // halfs per 16-row slab of a tile

__device__ __forceinline__ int swz(int r) { return r & 7; }

// Barrier that also publishes every direct-to-LDS load this wave issued.  The
// wait (vmcnt(0) lgkmcnt(0)) is a builtin so that the compiler knows every
// earlier load has landed; the asm statement repeats the vmcnt wait, since the
// compiler does not see the direct-to-LDS loads (they are issued from asm),
// and holds the barrier, with a memory clobber so that no LDS access moves
// across it.
__device__ __forceinline__ void sync_dma() {
  __builtin_amdgcn_s_waitcnt(0x0070);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace

template <bool FOX>
__global__ __launch_bounds__(kNT, 2) void scan64_kernel(
    int64_t L, int Nb, int BH, int accurate_all, float tau, const _Float16* __restrict__ vt,
    const _Float16* __restrict__ khat, const _Float16* __restrict__ pmat,
    const float* __restrict__ qhat, const float* __restrict__ sdiag,
    const float* __restrict__ kmax_blk, const float* __restrict__ pnorm,
    const int* __restrict__ vexp, const float* __restrict__ cum,
    uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int D = kD, C = kBlk, NCT = 2, DT = 4, DC = 2;

  // stage s: Khat hi, P hi, V^T; one stage of lo parts
  __shared__ __attribute__((aligned(1024))) _Float16 sK0[kTile], sP0[kTile], sV0[kTile];
  __shared__ __attribute__((aligned(1024))) _Float16 sK1[kTile], sP1[kTile], sV1[kTile];
  __shared__ __attribute__((aligned(1024))) _Float16 sKl[kTile], sPl[kTile];
  __shared__ float red[2][kNW];

  const int NP = (Nb + 1) / 2;
  int p;
  int64_t bh;
  if (BH % 8 == 0) {
    // Workgroups go to the 8 XCDs round robin; XCD x gets the heads x, x+8, ...
    // so that the key blocks a head's tiles share stay in one L2.  An XCD has
    // about two heads' tiles in flight, so its heads are taken in pairs and the
    // tiles of a pair longest first (a tile of query block pair p scans 2p+1 key
    // blocks): the short tiles of both heads fill in at the end.
    const int xcd = blockIdx.x % 8;
    const int j = blockIdx.x / 8;
    const int HX = BH / 8;
    const int g = j / (2 * NP), r = j % (2 * NP);
    int hh;
    if (2 * g + 1 < HX) {
      p = NP - 1 - r / 2;
      hh = 2 * g + (r & 1);
    } else {
      p = NP - 1 - r;  // a last, unpaired head
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
  const int half = wave / 2;
  const int mb = 2 * p + half;        // this wave's query block
  const bool live = mb < Nb;
  const int r0 = (wave % 2) * 32;     // first query row (local to block mb)
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
  const char* kh_h = reinterpret_cast<const char*>(khat + bh * Nb * (2 * C * D));
  const char* pm_h = reinterpret_cast<const char*>(pmat + bh * Nb * (2 * D * D));
  const char* vt_h = reinterpret_cast<const char*>(vt + bh * Nb * (D * C));
  constexpr int TB = kTile * 2;  // bytes per tile

  // ---- direct-to-LDS staging ------------------------------------------------------
  // Slot i of this wave covers LDS chunks (2*wave+i)*64 + lane of a tile; the
  // lane fetches the logical chunk that belongs there.
  uint32_t goff[2];  // unsigned: the loads take a uniform base plus a 32-bit lane offset
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pos = (2 * wave + i) * 64 + lane;
    const int r = pos >> 3;
    goff[i] = static_cast<uint32_t>(r * 128 + ((pos & 7) ^ swz(r)) * 16);
  }
  auto dma = [&](const char* gtile, _Float16* ltile) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      lds_dma16(gtile + goff[i], ltile + (2 * wave + i) * 512);
  };
  // stage tiles, selected at compile time
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto tileK = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return sK0; else return sK1;
  };
  auto tileP = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return sP0; else return sP1;
  };
  auto tileV = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return sV0; else return sV1;
  };
  auto dma_hi = [&](int n, auto st) __attribute__((always_inline)) {
    dma(kh_h + static_cast<int64_t>(n) * (2 * TB), tileK(st));
    dma(pm_h + static_cast<int64_t>(n) * (2 * TB), tileP(st));
    dma(vt_h + static_cast<int64_t>(n) * TB, tileV(st));
  };
  // lo parts: thread t owns LDS chunks t and t + 256 of each lo tile
  uint32_t loff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int pos = tid + 256 * j;
    const int r = pos >> 3;
    loff[j] = static_cast<uint32_t>(r * 128 + ((pos & 7) ^ swz(r)) * 16);
  }
  u4 lopre[4];  // lo parts of the next split-precision block (K lo, K lo, P lo, P lo)
  auto fetch_lo = [&](int n) __attribute__((always_inline)) {
    const char* kb = kh_h + static_cast<int64_t>(n) * (2 * TB) + TB;
    const char* pb = pm_h + static_cast<int64_t>(n) * (2 * TB) + TB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lopre[j] = *reinterpret_cast<const u4*>(kb + loff[j]);
      lopre[2 + j] = *reinterpret_cast<const u4*>(pb + loff[j]);
    }
  };
  auto put_lo = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<u4*>(sKl + 8 * (tid + 256 * j)) = lopre[j];
      *reinterpret_cast<u4*>(sPl + 8 * (tid + 256 * j)) = lopre[2 + j];
    }
  };
  // MFMA A operand: rows 16t + ln, logical chunk 4c + lg of a swizzled tile
  const int sw = swz(ln);
  const int aoff0 = (ln * 8 + (lg ^ sw)) * 8;
  const int aoff1 = (ln * 8 + ((4 + lg) ^ sw)) * 8;
  auto rdA = [&](const _Float16* tile, int t, int c) __attribute__((always_inline)) {
    return *reinterpret_cast<const h8*>(tile + t * kRowT + (c ? aoff1 : aoff0));
  };

  // ---- per-wave state ------------------------------------------------------------
  f4 oacc[NCT][DT], qf[NCT][DT];
  f4 lacc[NCT];  // softmax denominators (every element holds the column sum)
  h8 qhi[NCT][DC], qlo[NCT][DC];
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
  f4 seed[NCT];       // cq - mrun + kOff: the accumulator start of S^T (changes with mrun only)
  float mrun_min;     // min of mrun over the wave's queries
  auto set_seeds = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float sv = (FOX ? cq[ct] : 0.f) - mrun[ct] + kOff;
      seed[ct] = f4{sv, sv, sv, sv};
    }
    mrun_min = -wave_max_dpp(-fminf(mrun[0], mrun[1]));
  };
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    lacc[ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[ct][t] = f4{0.f, 0.f, 0.f, 0.f};
    cq[ct] = (FOX && live) ? cumh[mb * C + r0 + 16 * ct + ln] : 0.f;
  }
  const h8 ones = h8{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};

  // ---- softmax step on logits relative to the running max -------------------------
  // x[ct][kt][i] = logit - mrun + kOff (log2 units) of key 16kt+4lg+i, query column ct.
  auto softmax_pv = [&](f4 (&x)[NCT][4], const _Float16* vtile, bool vsc, h8 vs8) __attribute__((always_inline)) {
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
        h8 a = rdA(vtile, t, c);
        if (vsc) a *= vs8;
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
    return sqrtf(wave_max_dpp(mx));
  };

  // ---- diagonal blocks, and the operands of key block 2p ------------------------------
  // V^T of block 2p lands in stage 0 (it is also the first scanned block); that
  // of block 2p+1 uses stage 1's V^T tile, free until the first prefetch.
  dma_hi(2 * p, S0{});
  if (2 * p + 1 < Nb) dma(vt_h + static_cast<int64_t>(2 * p + 1) * TB, sV1);
  fetch_lo(2 * p);  // used only if block 2p runs the split products
  f4 ckn[4];  // FoX prefix of the key block being scanned
  if constexpr (FOX) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) ckn[kt] = *reinterpret_cast<const f4*>(cumh + (2 * p) * C + 16 * kt + 4 * lg);
  }
  // the in-block logits, forget-gate prefix and adjusted queries travel with
  // the first stage (one latency, not three)
  f4 sdv[NCT][4], ckd[4];
  if (live) {
    const float* sd = sdiag + (bh * Nb + mb) * kDiagTri;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int r = r0 + 16 * ct + ln;
      // the stored chunks of row r (padded triangle); the others are masked below
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        sdv[ct][kt] = 16 * kt + 4 * lg <= r ? *reinterpret_cast<const f4*>(sd + diag_row(r) + 16 * kt + 4 * lg)
                                            : f4{0.f, 0.f, 0.f, 0.f};
      const float* src = qhat + (bh * Nb * C + mb * C + r) * D;
#pragma unroll
      for (int t = 0; t < DT; ++t) qf[ct][t] = *reinterpret_cast<const f4*>(src + 16 * t + 4 * lg);
    }
    if constexpr (FOX) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) ckd[kt] = *reinterpret_cast<const f4*>(cumh + mb * C + 16 * kt + 4 * lg);
    }
  }
  sync_dma();
  if (live) {
    f4 x[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int r = r0 + 16 * ct + ln;
      float a = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int c0 = 16 * kt + 4 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float val = sdv[ct][kt][i];
          if constexpr (FOX) val += cq[ct] - ckd[kt][i];
          x[ct][kt][i] = (c0 + i <= r) ? val : kNegInf;
          a = fmaxf(a, x[ct][kt][i]);
        }
      }
      mrun[ct] = grp_max(a);  // finite: key r is always present
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) x[ct][kt] -= mrun[ct] - kOff;
    }
    const bool dsc = vE != 0 && vexp[bh * Nb + mb] != vE;
    softmax_pv(x, half == 0 ? sV0 : sV1, dsc, dsc ? vscale(mb) : h8{});
  } else {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      mrun[ct] = 0.f;
#pragma unroll
      for (int t = 0; t < DT; ++t) qf[ct][t] = f4{0.f, 0.f, 0.f, 0.f};
    }
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
  // one key block; its stage (n & 1, block 2p in stage 0) is a compile-time constant
  auto step = [&](int n, auto st) __attribute__((always_inline)) {
    using SN = std::integral_constant<int, 1 - decltype(st)::value>;
    const _Float16* tK = tileK(st);
    const _Float16* tP = tileP(st);
    const _Float16* tV = tileV(st);
    f4 ck[4];
    if constexpr (FOX) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        ck[kt] = ckn[kt];
        if (n > 0) ckn[kt] = *reinterpret_cast<const f4*>(cumh + (n - 1) * C + 16 * kt + 4 * lg);
      }
    }
    const float pn_cur = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pnw), wb - n));
    const float kn_cur = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(knw), wb - n));
    if (n > 0 && wb - n == 63) {  // block n-1 opens the next window
      wb = n - 1;
      load_window();
    }
    // this block's lo parts (fetched a block ahead) into their LDS stage; the
    // next block's hi parts, and its lo parts when it will need them
    if (acc_cur) put_lo();
    if (n > 0) dma_hi(n - 1, SN{});
    // precision of block n-1: bound on |Qt| after this block's transition
    const float qb_next = qbound * pn_cur;
    const bool acc_next = accurate_all || (qb_next * khmax * 0.0009765625f > tau);
    if (acc_next && n > 0) fetch_lo(n - 1);
    const bool work = live && !(half == 0 && n == 2 * p);

    // The block runs as five regions; in each, matrix-core products that do
    // not depend on the vector work are interleaved with it (1 MFMA : k VALU),
    // so one wave keeps both units busy:
    //   R1 S^T for both query tiles          R2 first half of P_n Qt | row maxima
    //   R3 second half of P_n Qt | exp tile 0  R4 PV tile 0 | exp tile 1
    //   R5 PV tile 1 | Qt -> fp16 operands
    // (P_n Qt is formed on block 0 too, where it is not used: it keeps the
    // regions free of branches.)
    // No logit of this block can pass the running max by kTheta when
    // |Qt| * max|khat| (Cauchy-Schwarz; 1.01 covers the fp16 operands) stays
    // below it: then the maxima and the rescale are skipped.  The forget-gate
    // bias is left out of the bound, so gated attention always takes the maxima.
    const bool skip_max = !FOX && (qbound * kn_cur * 1.01f <= mrun_min + kTheta);
    f4 x[NCT][4];
    h8 ap[DC][DT];
    if (work) {
      h8 ak[DC][4];
#pragma unroll
      for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) ak[c][kt] = rdA(tK, kt, c);
      // the transition's operands are read now, in registers by R2 (the
      // gated variant, short of registers, reads them at R2)
      if constexpr (!FOX) {
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
          for (int t = 0; t < DT; ++t) ap[c][t] = rdA(tP, t, c);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) x[ct][kt] = mma16(ak[c][kt], qhi[ct][c], c == 0 ? seed[ct] : x[ct][kt]);
    }
    if (acc_cur) {
      // every thread's share of the lo tiles is in LDS (no wait on the prefetch)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // The logits' own correction needs only this block's max |khat|; the
      // transport's (below) reaches every earlier block and keeps the maximum
      // over all the key blocks the tile scans.
      if (work && (accurate_all || qbound * kn_cur * 0.0009765625f > tau)) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            const h8 al = rdA(sKl, kt, c);
            const h8 ah = rdA(tK, kt, c);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              x[ct][kt] = mma16(al, qhi[ct][c], x[ct][kt]);
              x[ct][kt] = mma16(ah, qlo[ct][c], x[ct][kt]);
            }
          }
        }
      }
    }
    if (work) {
      const f4 zero = f4{0.f, 0.f, 0.f, 0.f};
      // ---- R2: first half of Qt <- P_n Qt beside the row maxima
      if constexpr (FOX) {
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
          for (int t = 0; t < DT; ++t) ap[c][t] = rdA(tP, t, c);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (skip_max) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) qf[ct][t] = mma16(ap[0][t], qhi[ct][0], zero);
      } else {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) qf[ct][t] = mma16(ap[0][t], qhi[ct][0], zero);
        if constexpr (FOX) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) x[ct][kt] -= ck[kt];
        }
        float mx[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float a = fmaxf(fmaxf(x[ct][0][0], x[ct][0][1]), fmaxf(x[ct][0][2], x[ct][0][3]));
#pragma unroll
          for (int kt = 1; kt < 4; ++kt)
            a = fmaxf(a, fmaxf(fmaxf(x[ct][kt][0], x[ct][kt][1]), fmaxf(x[ct][kt][2], x[ct][kt][3])));
          mx[ct] = grp_max(a);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // rare: raise the running max
        if (__any(mx[0] > kTheta + kOff || mx[1] > kTheta + kOff)) {
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
          set_seeds();
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- R3: second half of the transition beside the exponentials of tile 0
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) qf[ct][t] = mma16(ap[1][t], qhi[ct][1], qf[ct][t]);
      h8 pb[NCT][2];
      auto exps = [&](int ct) __attribute__((always_inline)) {
        f4 pe[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) pe[kt][i] = __builtin_amdgcn_exp2f(x[ct][kt][i]);
        pb[ct][0] = pack_h8(pe[0], pe[1]);
        pb[ct][1] = pack_h8(pe[2], pe[3]);
      };
      exps(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);  // exp
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // other vector ALU
      }
      // keep tile 0's exponentials in this region (not sunk to their use)
      asm volatile("" ::"v"(pb[0][0]), "v"(pb[0][1]));
      __builtin_amdgcn_sched_barrier(0);
      if (acc_cur) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            const h8 al = rdA(sPl, t, c);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              qf[ct][t] = mma16(al, qhi[ct][c], qf[ct][t]);
              qf[ct][t] = mma16(ap[c][t], qlo[ct][c], qf[ct][t]);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- R4: PV of tile 0 beside the exponentials of tile 1
      h8 av[2][DT];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < DT; ++t) av[c][t] = rdA(tV, t, c);
      if (vE != 0 && vexp[bh * Nb + n] != vE) {  // rare: this block's values in the tile's units
        const h8 f8 = vscale(n);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int t = 0; t < DT; ++t) av[c][t] *= f8;
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[0][t] = mma16(av[c][t], pb[0][c], oacc[0][t]);
        lacc[0] = mma16(ones, pb[0][c], lacc[0]);
      }
      exps(1);
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      }
      asm volatile("" ::"v"(pb[1][0]), "v"(pb[1][1]));
      __builtin_amdgcn_sched_barrier(0);
      // ---- R5: PV of tile 1 beside the conversion of the transported queries
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[1][t] = mma16(av[c][t], pb[1][c], oacc[1][t]);
        lacc[1] = mma16(ones, pb[1][c], lacc[1]);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int c = 0; c < DC; ++c) qhi[ct][c] = pack_h8(qf[ct][2 * c], qf[ct][2 * c + 1]);
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (acc_next) {
        asm volatile("");  // a real branch: the lo parts are rarely needed
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int c = 0; c < DC; ++c) qlo[ct][c] = pack_lo(qf[ct][2 * c], qf[ct][2 * c + 1], qhi[ct][c]);
      }
    }
    // measured norms while the split is in use; the carried bound otherwise
    const int slot = n & 1;
    if (acc_next && n > 0) {
      const float qn = (work || !live) ? wave_qnorm() : 0.f;
      if (lane == 0) red[slot][wave] = qn;
    }
    sync_dma();  // next stage landed; this stage's reads done; norms visible
    if (acc_next && n > 0) {
      float qm = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kNW; ++w2) qm = fmaxf(qm, red[slot][w2]);
      // waves that skipped this block still hold their previous (untransported) queries
      qbound = fmaxf(qm, (n == 2 * p) ? qbound : 0.f);
    } else {
      qbound = qb_next;
    }
    // the measured norm never exceeds the carried bound, so block n-1 never
    // needs lo parts that were not planned
    acc_cur = acc_next && (accurate_all || (qbound * khmax * 0.0009765625f > tau));
  };

  for (int n = 2 * p; n >= 0; n -= 2) {
    step(n, S0{});
    if (n > 0) step(n - 1, S1{});
  }

  // ---- epilogue -------------------------------------------------------------------
  if (live) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float l = lacc[ct][0];
      const int r = r0 + 16 * ct + ln;
      const int64_t row = static_cast<int64_t>(mb) * C + r;
      if (row < L) {
        const float inv = __builtin_ldexpf(1.f / l, vE);
        uint16_t* dst = o + (bh * L + row) * D;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const f4 y = oacc[ct][t] * inv;
          B8 pk;
          pk.p[0] = __builtin_convertvector(f2{y[0], y[1]}, b2);
          pk.p[1] = __builtin_convertvector(f2{y[2], y[3]}, b2);
          *reinterpret_cast<uint2*>(dst + 16 * t + 4 * lg) = make_uint2(pk.u.x, pk.u.y);
        }
        if (lg == 0) lse[bh * L + row] = (mrun[ct] - kOff + __log2f(l)) * kLn2;
      }
    }
  }
}

hipError_t launch_scan64(int64_t BH, int64_t L, int accurate, float tau, const _Float16* vt,
                         const _Float16* khat, const _Float16* pmat, const float* qhat, const float* sdiag,
                         const float* kmax_blk, const float* pnorm, const int* vexp,
                         const float* cum, void* o, float* lse, hipStream_t stream) {
  const int Nb = static_cast<int>((L + kBlk - 1) / kBlk);
  const int NP = (Nb + 1) / 2;
  dim3 grid(static_cast<unsigned>(BH * NP));
  dim3 block(kNT);
  if (cum) {
    hipLaunchKernelGGL((scan64_kernel<true>), grid, block, 0, stream, L, Nb, static_cast<int>(BH), accurate, tau,
                       vt, khat, pmat, qhat, sdiag, kmax_blk, pnorm, vexp, cum,
                       static_cast<uint16_t*>(o), lse);
  } else {
    hipLaunchKernelGGL((scan64_kernel<false>), grid, block, 0, stream, L, Nb, static_cast<int>(BH), accurate, tau,
                       vt, khat, pmat, qhat, sdiag, kmax_blk, pnorm, vexp, cum,
                       static_cast<uint16_t*>(o), lse);
  }
  return hipGetLastError();
}

}  // namespace path
