// Projection prologue of PaTH attention on the bf16 matrix cores.
//
// [PaTH Attention summary (gist.science 2505.16381), §2 "Mecanismo Central"]:
// the transition vector w_s and the factor beta_s are functions of the input
// token x_s, with beta_s = 2 sigmoid(u^T x_s + b).  The pages give no formula
// for w_s; here it is a per-head linear map scaled to unit length,
//     w_s = W_h x_s / max(|W_h x_s|, 1e-12),
// and [§6 "Limitações"]'s clipping of beta is an optional upper bound.
//
// One GEMM over all heads: tokens x [T, Dm] (T = B L, bf16) against the rows
// of Ww [H d, Dm] (head h owns rows h d .. h d + d - 1) and of u [H, Dm].  A
// workgroup takes 256 tokens and one group of 128 columns: either the rows of
// 128 / d whole heads (so each head's vector w_s is in the tile and is
// normalised in the epilogue) or the u rows of 128 consecutive heads (their
// beta logits).  Eight waves, each 32 tokens x 128 columns.
// Products are 16x16x32 bf16 MFMAs with fp32 accumulation.  Dm is reduced in
// chunks of 64 that travel global -> LDS with direct-to-LDS loads (issued from
// asm, lds_dma16) through a ring of three stages: chunk c + 2 is in flight
// while chunk c is multiplied,
// and one barrier per chunk both publishes the next stage and frees the oldest.
// Every load is unconditional: rows past the tokens or the weight rows read a
// clamped row, whose products land only in outputs that are not written.
// Tiles are unpadded 128-byte rows; 16-byte chunk j of row r sits at slot
// j ^ (r & 7), so the operand reads (16 rows, one chunk column) hit distinct
// banks.
// Workgroup ids are dealt to the 8 XCDs round robin; all column groups of a
// token tile are given ids on one XCD, so its L2 fetches the tile once.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"
#include "mfma_util.h"

namespace path {

namespace {

constexpr int kPW = 8;             // waves
constexpr int kRT = 256 / 16 / kPW;  // 16-token row tiles per wave
constexpr int kNS = 3;             // LDS stages of the ring (2 or 3)
constexpr int kPT = 64 * kPW;      // threads
constexpr int kPM = 16 * kRT * kPW;  // tokens per workgroup
constexpr int kPK = 64;            // reduction chunk (bf16 elements: one 128-byte row)
constexpr int kPN = 128;           // columns per workgroup
constexpr int kALd = kPM * kPK / 8 / kPT;  // direct-to-LDS loads per thread per chunk, tokens
constexpr int kBLd = kPN * kPK / 8 / kPT;  // the same, weight rows
constexpr int kOP = 72;            // output staging row pitch (bf16): 144 bytes, 16-byte aligned rows
// LDS bytes of a workgroup (ring stages, output staging) and the workgroups
// per CU they leave room for in 160 KB: one, for the configuration above.
constexpr int kLdsBytes = kNS * (kPM + kPN) * kPK * 2 + kPW * 8 * kOP * 2;
constexpr int kOcc = 163840 / kLdsBytes;
static_assert(kNS == 2 || kNS == 3, "ring depth");
static_assert(kOcc >= 1, "the LDS of one workgroup must fit a CU");
static_assert(kALd * kPT * 8 == kPM * kPK && kBLd * kPT * 8 == kPN * kPK, "whole 16-byte chunks per thread");

using mfma::b8;
using mfma::f4;

template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over a row of 16 lanes, the same bits in every lane of the row.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_row<0xB1>(x);
  x += dpp_row<0x4E>(x);
  x += dpp_row<0x141>(x);
  x += dpp_row<0x140>(x);
  return x;
}

// s_waitcnt with expcnt and lgkmcnt left open and vmcnt = N (N < 16).  The
// direct-to-LDS loads are issued from asm (lds_dma16: the compiler then keeps
// its waits on LDS reads counted), so the compiler does not count them: the
// wait is repeated in asm, where it cannot be dropped.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Calls f(integral_constant<int, I>) for each I of the sequence, in order.
template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

}  // namespace

// NCH > 0: Dm = 64 NCH, the chunk loop fully unrolled, so every wait is a
// constant and the compiler keeps track of which stage each load in flight
// writes (a loop merges that knowledge away and drains all loads before the
// operand reads).  NCH = 0: any Dm, a loop over chunks.
template <int D, int NCH>
__global__ __launch_bounds__(kPT, kOcc) void project_kernel(
    int64_t T, int64_t L, int64_t H, int64_t Dm, int ntiles, int ncol, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ Ww, const uint16_t* __restrict__ u, const float* __restrict__ bias,
    float beta_max, uint16_t* __restrict__ w_out, float* __restrict__ beta_out) {
  constexpr int NC = kPN / 16;         // column tiles
  constexpr int HT = D / 16;           // column tiles per head
  constexpr int NLD = kALd + kBLd;     // loads per thread per chunk
  // Three stages of the ring, each its own LDS object so that the compiler can
  // tell reads of one stage from loads still landing in another.
  // Stage s holds the token tile (kPM rows) followed by the weight tile (kPN rows).
  __shared__ __attribute__((aligned(1024))) uint16_t sT0[(kPM + kPN) * kPK], sT1[(kPM + kPN) * kPK],
      sT2[kNS > 2 ? (kPM + kPN) * kPK : 8];
  auto stageA = [&](auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return sT0; else if constexpr (S == 1) return sT1; else return sT2;
  };
  auto stageB = [&](auto st) __attribute__((always_inline)) { return stageA(st) + kPM * kPK; };
  __shared__ __attribute__((aligned(16))) uint16_t sOut[kPW * 8 * kOP];  // output staging, 8 rows per wave

  // XCD-aware map: ids i, i + 8, i + 16, ... run on one XCD; consecutive ids of
  // that stream walk the column groups of one token tile.
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int col = j % ncol;
  const int tile = (j / ncol) * 8 + xcd;
  if (tile >= ntiles) return;  // whole workgroup: no barrier reached
  const int64_t t0 = static_cast<int64_t>(tile) * kPM;
  const int64_t nwg = (H * D + kPN - 1) / kPN;  // column groups of w
  const bool beta_group = col >= nwg;
  const int64_t r0 = (beta_group ? col - nwg : col) * static_cast<int64_t>(kPN);
  const int64_t nrows = beta_group ? H : H * D;  // rows of the matrix this group reads
  const uint16_t* Wm = beta_group ? u : Ww;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;

  // Direct-to-LDS sources.  Load i of this wave fills the 64 consecutive
  // 16-byte LDS slots (i * kPW + wv) * 64 + lane of a tile; the lane fetches
  // the logical chunk that belongs in its slot, from a clamped row.
  const char* asrc[kALd];
  const char* bsrc[kBLd];
#pragma unroll
  for (int i = 0; i < kALd; ++i) {
    const int pos = (i * kPW + wv) * 64 + lane;
    const int r = pos >> 3, jc = (pos & 7) ^ (r & 7);
    const int64_t t = t0 + r < T ? t0 + r : T - 1;
    asrc[i] = reinterpret_cast<const char*>(x + t * Dm) + 16 * jc;
  }
#pragma unroll
  for (int i = 0; i < kBLd; ++i) {
    const int pos = (i * kPW + wv) * 64 + lane;
    const int r = pos >> 3, jc = (pos & 7) ^ (r & 7);
    const int64_t rr = r0 + r < nrows ? r0 + r : nrows - 1;
    bsrc[i] = reinterpret_cast<const char*>(Wm + rr * Dm) + 16 * jc;
  }
  auto dma_to = [&](int c, uint16_t* adst, uint16_t* bdst) __attribute__((always_inline)) {
    const int64_t off = static_cast<int64_t>(c) * (kPK * 2);
#pragma unroll
    for (int i = 0; i < kALd; ++i)
      mfma::lds_dma16(asrc[i] + off, adst + (i * kPW + wv) * 512);
#pragma unroll
    for (int i = 0; i < kBLd; ++i)
      mfma::lds_dma16(bsrc[i] + off, bdst + (i * kPW + wv) * 512);
  };
  auto dma = [&](int c, auto st) __attribute__((always_inline)) { dma_to(c, stageA(st), stageB(st)); };

  f4 acc[kRT][NC];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) acc[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};

  // LDS element offsets of this lane's operand chunks: row 16 tile + lr, logical
  // chunk 4 ks + lg at its swizzled slot (row & 7 == lr & 7 for every tile).
  int aoff[kRT][2], boff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int slot = ((4 * ks + lg) ^ (lr & 7)) * 8;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) aoff[rt][ks] = (16 * kRT * wv + 16 * rt + lr) * kPK + slot;
    boff[ks] = lr * kPK + slot;
  }

  const int nchunks = NCH > 0 ? NCH : static_cast<int>(Dm / kPK);
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // One chunk: wait for its loads, publish it (and free the stage the chunk
  // c + 2 loads go to), start those loads, multiply.
  auto step = [&](int c, auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    if (kNS == 3 && c + 1 < nchunks)
      wait_vm<NLD>();  // chunk c + 1's loads may still be in flight
    else
      wait_vm<0>();
    asm volatile("s_barrier" ::: "memory");
    if (c + kNS - 1 < nchunks) dma(c + kNS - 1, std::integral_constant<int, (S + kNS - 1) % kNS>{});
    const uint16_t* As = stageA(st);
    const uint16_t* Bs = stageB(st);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      b8 af[kRT], bf[NC];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) af[rt] = *reinterpret_cast<const b8*>(As + aoff[rt][ks]);
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) bf[ct] = *reinterpret_cast<const b8*>(Bs + boff[ks] + 16 * ct * kPK);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) acc[rt][ct] = mfma::mmb16(af[rt], bf[ct], acc[rt][ct]);
    }
  };

  dma(0, S0{});
  if (kNS == 3 && nchunks > 1) dma(1, S1{});
  if constexpr (NCH > 0) {
    static_for(std::make_integer_sequence<int, NCH>{}, [&](auto ic) __attribute__((always_inline)) {
      constexpr int c = decltype(ic)::value;
      step(c, std::integral_constant<int, c % kNS>{});
    });
  } else {
    int c0 = 0;
    for (; c0 + kNS <= nchunks; c0 += kNS)
      static_for(std::make_integer_sequence<int, kNS>{}, [&](auto ic) __attribute__((always_inline)) {
        step(c0 + decltype(ic)::value, ic);
      });
    static_for(std::make_integer_sequence<int, kNS - 1>{}, [&](auto ic) __attribute__((always_inline)) {
      if (c0 + decltype(ic)::value < nchunks) step(c0 + decltype(ic)::value, ic);
    });
  }

  // Epilogue.  acc[rt][ct][i] is token 16 (kRT wv + rt) + 4 lg + i, column 16 ct + lr.
  if (!beta_group) {
    // w: each head's row is scaled to unit length, rounded to bf16 and passed
    // through this wave's slice of sOut (8 tokens x 64 columns at a time), so
    // that every lane stores 16 contiguous bytes of one token's row.  The
    // slice is private to the wave, whose LDS operations run in order.
    uint16_t* so = sOut + wv * (8 * kOP);
    const int rr = lane >> 3, seg = lane & 7;  // read-back: staged row, 16-byte segment
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      float inv[kPN / D][4];
#pragma unroll
      for (int hh = 0; hh < kPN / D; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float n2 = 0.f;
#pragma unroll
          for (int ct = HT * hh; ct < HT * (hh + 1); ++ct) n2 = fmaf(acc[rt][ct][i], acc[rt][ct][i], n2);
          inv[hh][i] = 1.f / fmaxf(sqrtf(sum16(n2)), 1e-12f);
        }
#pragma unroll
      for (int half = 0; half < 2; ++half) {  // columns 64 half .. 64 half + 63 of the group
        constexpr int QT = 4;                   // column tiles per half
        const int hh = (64 * half) / D;         // head of the group these columns belong to
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {        // tokens 4 lg + 2 ip + {0, 1} of each lane group
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int q = 0; q < QT; ++q) {
              const int i = 2 * ip + i2;
              so[(2 * lg + i2) * kOP + 16 * q + lr] = f32_to_bf16(acc[rt][QT * half + q][i] * inv[hh][i]);
            }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const uint4 v = *reinterpret_cast<const uint4*>(so + rr * kOP + 8 * seg);
          const int64_t t = t0 + 16 * (kRT * wv + rt) + 4 * (rr >> 1) + 2 * ip + (rr & 1);
          const int64_t h = r0 / D + hh;
          if (t < T && h < H) {
            const int64_t bi = t / L, li = t - bi * L;
            *reinterpret_cast<uint4*>(w_out + ((bi * H + h) * L + li) * D + (64 * half) % D + 8 * seg) = v;
          }
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 16 * (kRT * wv + rt) + 4 * lg + i;
        if (t < T) {
          const int64_t bi = t / L, li = t - bi * L;
#pragma unroll
          for (int ct = 0; ct < NC; ++ct) {
            const int64_t h = r0 + 16 * ct + lr;
            if (h < H) {
              const float z = acc[rt][ct][i] + bias[h];
              float beta = 2.f / (1.f + expf(-z));
              if (beta_max > 0.f) beta = fminf(beta, beta_max);
              beta_out[(bi * H + h) * L + li] = beta;
            }
          }
        }
      }
    }
  }
}

hipError_t launch_project(int64_t B, int64_t L, int64_t Dm, int64_t H, int64_t d, const void* x, const void* Ww,
                          const void* u, const float* bias, float beta_max, void* w_out, float* beta_out,
                          hipStream_t stream) {
  const int64_t T = B * L;
  const int ntiles = static_cast<int>((T + kPM - 1) / kPM);
  const int ncol = static_cast<int>((H * d + kPN - 1) / kPN + (H + kPN - 1) / kPN);
  const int64_t per_xcd = (ntiles + 7) / 8;
  const dim3 grid(static_cast<unsigned>(8 * per_xcd * ncol));
  const auto* xs = static_cast<const uint16_t*>(x);
  const auto* ws = static_cast<const uint16_t*>(Ww);
  const auto* us = static_cast<const uint16_t*>(u);
  auto* wo = static_cast<uint16_t*>(w_out);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kPT), 0, stream, T, L, H, Dm, ntiles, ncol, xs, ws, us, bias, beta_max,
                       wo, beta_out);
  };
  auto pick = [&](auto dc) {
    constexpr int DD = decltype(dc)::value;
    switch (Dm) {
      case 512: go(project_kernel<DD, 8>); break;
      case 1024: go(project_kernel<DD, 16>); break;
      case 2048: go(project_kernel<DD, 32>); break;
      case 4096: go(project_kernel<DD, 64>); break;
      default: go(project_kernel<DD, 0>); break;
    }
  };
  if (d == 64)
    pick(std::integral_constant<int, 64>{});
  else
    pick(std::integral_constant<int, 128>{});
  return hipGetLastError();
}

}  // namespace path
