// Decode step of PaTH attention with an in-place key cache.
//
// [PaTH Attention summary (gist.science 2505.16381), §3 "Inferência"]: at step
// t every cached key absorbs the new transition, k_j <- H_t k_j with
// H_t = I - beta_t w_t w_t^T, so the cache always holds
// (H_{j+1}...H_t)^T k_j and no transition vectors are kept; the new key k_t
// enters untransformed (its path product is empty).  The attention itself is
// single-query softmax attention, split over key chunks and merged by
// log-sum-exp (the FlashDecoding pattern the same bullet names).
//
// Memory plan (HBM-bound): each cached key row is read once and written once,
// each value row read once, all with 16-byte coalesced accesses; consecutive
// lanes cover one row, so a wave touches 1 KiB of contiguous cache per pass.
// The chunk loop is software-pipelined: the loads of the next group of 8 rows
// per lane are issued before the current group is updated and attended to.
//
// Paged variant (FlashDecoding/paged-KV layout, which the same bullet says the
// method stays compatible with): the same kernels with another row map, pages
// [num_pages, H, page, d] addressed through a per-sequence page table, and one
// cache length per sequence read on the device.
//
// Gated variant (FOX) [same summary, §2 "Extensões: PaTH-FoX"]: the logit of
// cached key j gains the forget-gate sum over j < s <= t, kept as a difference
// of running prefixes c_t - c_j.  The prefix of every cached key sits in an
// fp32 cache beside the key cache (4 bytes per key against 2 d-element rows)
// with the key cache's row map (contiguous [B*H, capacity] or paged
// [num_pages, H, page]), is fetched in the same pipelined group as the key and
// value rows, and the step appends c_t = c_{t-1} + log f_t for the new key,
// whose own bias is 0.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace path {

constexpr int kDecThreads = 256;
constexpr int kDecChunk = 1024;  // keys per workgroup
// The decode workspace starts with a 512-byte slot that takes the stores of key
// slots past the end of a chunk (contiguous caches), so that every load and
// store of the key loop is unconditional; the chunk partials follow it.
constexpr int kDecTrashFloats = 128;

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec16;  // 16 bytes of storage, moved as one native 128-bit vector
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  using raw = u4;
  __device__ static void unpack(const raw& x, float* f) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f[2 * t] = __uint_as_float(x[t] << 16);
      f[2 * t + 1] = __uint_as_float(x[t] & 0xffff0000u);
    }
  }
  __device__ static raw pack(const float* f) {
    raw u;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      u[t] = static_cast<uint32_t>(f32_to_bf16(f[2 * t])) |
             (static_cast<uint32_t>(f32_to_bf16(f[2 * t + 1])) << 16);
    return u;
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  using raw = u4;
  __device__ static void unpack(const raw& x, float* f) {
#pragma unroll
    for (int t = 0; t < 4; ++t) f[t] = __uint_as_float(x[t]);
  }
  __device__ static raw pack(const float* f) {
    return raw{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64).
// Groups of up to 16 lanes use DPP lane moves (quad swaps, then mirrors within
// 8- and 16-lane rows); wider groups fall back to cross-lane permutes.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  const auto mv = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  if constexpr (G >= 2) x += mv(x, std::integral_constant<int, 0xB1>{});   // lanes i ^ 1
  if constexpr (G >= 4) x += mv(x, std::integral_constant<int, 0x4E>{});   // lanes i ^ 2
  if constexpr (G >= 8) x += mv(x, std::integral_constant<int, 0x141>{});  // mirror within 8
  if constexpr (G >= 16) x += mv(x, std::integral_constant<int, 0x140>{}); // mirror within 16
  if constexpr (G >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (G >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Where cached key j of head bh lives, in rows of d elements.  row() maps one
// key (the appended one); chunk_map() gives the map of one workgroup's chunk
// of keys [j0, j1), which every thread of the workgroup builds together.
// ContigRows: caches [B*H, capacity, d], one length for every head.
struct ContigRows {
  static constexpr int kMapSlots = 1;
  int64_t capacity, len;
  __device__ int64_t length(int64_t) const { return len; }
  __device__ int64_t row(int64_t bh, int64_t j) const { return bh * capacity + j; }
  __device__ static constexpr bool ok(int64_t) { return true; }
  struct Map {
    int64_t base;
    __device__ int64_t row(int64_t j) const { return base + j; }
  };
  __device__ Map chunk_map(int64_t bh, int64_t, int64_t, int32_t*) const { return Map{bh * capacity}; }
};
// PagedRows: pages [num_pages, H, page, d]; sequence b's logical page lp is
// table[b * max_pages + lp] and its length lens[b].  A slot whose page is not
// mapped (outside the table or the pool) is reported as row -1 and skipped.
// Keys are below 2^31 (the host checks max_pages * page), so logical pages come
// from a shift when page is a power of two (shift >= 0), else a 32-bit division.
struct PagedRows {
  static constexpr int kMapSlots = kDecChunk;
  const int32_t* table;
  const int32_t* lens;
  int64_t H, max_pages, num_pages, page;
  int shift;
  __device__ int64_t lpage(int64_t j) const {
    return shift >= 0 ? (j >> shift)
                      : static_cast<int64_t>(static_cast<uint32_t>(j) / static_cast<uint32_t>(page));
  }
  __device__ int64_t length(int64_t bh) const { return lens[bh / H]; }
  __device__ int64_t row(int64_t bh, int64_t j) const {
    if (j < 0) return -1;
    const int64_t lp = lpage(j);
    if (lp >= max_pages) return -1;
    const int64_t pg = table[(bh / H) * max_pages + lp];
    if (pg < 0 || pg >= num_pages) return -1;
    return (pg * H + bh % H) * page + (j - lp * page);
  }
  __device__ static bool ok(int64_t r) { return r >= 0; }
  struct Map {
    const int32_t* spg;  // validated page ids of the chunk's logical pages, from lp0
    int64_t lp0, h, H, page;
    int shift;
    __device__ int64_t row(int64_t j) const {
      const int64_t lp = shift >= 0 ? (j >> shift)
                                    : static_cast<int64_t>(static_cast<uint32_t>(j) / static_cast<uint32_t>(page));
      const int32_t pg = spg[lp - lp0];
      return pg < 0 ? -1 : (pg * H + h) * page + (j - lp * page);
    }
  };
  __device__ Map chunk_map(int64_t bh, int64_t j0, int64_t j1, int32_t* spg) const {
    const int64_t b = bh / H;
    const int64_t lp0 = j1 > j0 ? lpage(j0) : 0;
    const int64_t cnt = j1 > j0 ? lpage(j1 - 1) - lp0 + 1 : 0;  // <= j1 - j0 <= kDecChunk
    for (int64_t i = threadIdx.x; i < cnt; i += blockDim.x) {
      const int64_t lp = lp0 + i;
      int32_t pg = -1;
      if (lp < max_pages) {
        const int32_t t = table[b * max_pages + lp];
        if (t >= 0 && t < num_pages) pg = t;
      }
      spg[i] = pg;
    }
    __syncthreads();
    return Map{spg, lp0, bh % H, H, page, shift};
  }
};

// partial layout per (bh, chunk): [m, l, acc[D]]
template <typename T, int D, bool FOX, class Rows>
__global__ __launch_bounds__(kDecThreads) void decode_chunk_kernel(
    Rows rows, int nchunks, float scale, const T* __restrict__ q_t,
    const T* __restrict__ w_t, const float* __restrict__ beta_t, const float* __restrict__ log_f_t,
    T* __restrict__ k_cache, const T* __restrict__ v_cache, const float* __restrict__ cum_cache,
    float* __restrict__ trash, float* __restrict__ partials) {
  using V = Vec16<T>;
  constexpr int EPV = V::N;          // elements per 16-byte access
  constexpr int LPK = D / EPV;       // lanes per key row
  constexpr int KPW = 64 / LPK;      // key rows per wave pass
  constexpr int NW = kDecThreads / 64;
  constexpr int UNR = 8;             // key rows in flight per lane

  const int chunk = static_cast<int>(blockIdx.x % nchunks);
  const int64_t bh = blockIdx.x / nchunks;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPK;
  const int slot = lane / LPK;

  float qv[EPV], wv[EPV];
  {
    const typename V::raw* qp = reinterpret_cast<const typename V::raw*>(q_t + bh * D) + sub;
    const typename V::raw* wp = reinterpret_cast<const typename V::raw*>(w_t + bh * D) + sub;
    V::unpack(*qp, qv);
    V::unpack(*wp, wv);
  }
  float wq = 0.f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) wq += wv[e] * qv[e];
  wq = group_sum<LPK>(wq);
  const float bt = beta_t[bh];
  constexpr float kLog2e = 1.4426950408889634f;
  const float scale2 = scale * kLog2e;  // logits in log2 units
  const int64_t len = rows.length(bh);
  float ct = 0.f;
  if constexpr (FOX) {
    // c_t of the new query.  The prefix cache has the key cache's row map (one
    // float per key row); a sequence with no keys has no chunk work to bias.
    const int64_t prow = len > 0 ? rows.row(bh, len - 1) : -1;
    ct = (len > 0 && rows.ok(prow) ? cum_cache[prow] : 0.f) + log_f_t[bh];
  }

  const int64_t j0 = static_cast<int64_t>(chunk) * kDecChunk;
  const int64_t j1 = j0 + kDecChunk < len ? j0 + kDecChunk : len;
  __shared__ int32_t spg[Rows::kMapSlots];
  const auto map = rows.chunk_map(bh, j0, j1, spg);
  typename V::raw* kraw = reinterpret_cast<typename V::raw*>(k_cache);
  const typename V::raw* vraw = reinterpret_cast<const typename V::raw*>(v_cache);

  float mrun = -INFINITY, lrun = 0.f;
  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.f;

  constexpr int STRIDE = NW * KPW;  // key rows per workgroup pass
  typename V::raw kr[UNR], vr[UNR];
  float cr[UNR];
  // The loop's loads and stores carry no conditions, so the compiler can keep
  // the next group's loads and this group's stores in flight together.  A slot
  // past j1 (or, paged, on an unmapped page) stores into the trash slot and is
  // kept out of the softmax; it loads row j1 - 1 of a contiguous cache (finite
  // data) or, paged, the trash slot, whose value row is then zeroed.
  constexpr bool kDense = std::is_same_v<Rows, ContigRows>;
  typename V::raw* trash_slot = reinterpret_cast<typename V::raw*>(trash) + sub;
  auto fetch = [&](int64_t jb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t j = jb + static_cast<int64_t>(u) * STRIDE;
      if constexpr (kDense) {
        const int64_t jc = j < j1 ? j : j1 - 1;
        const int64_t rw = map.row(jc);
        kr[u] = __builtin_nontemporal_load(&kraw[rw * LPK + sub]);
        vr[u] = __builtin_nontemporal_load(&vraw[rw * LPK + sub]);
        if constexpr (FOX) cr[u] = cum_cache[rw];
      } else {
        const int64_t rw = j < j1 ? map.row(j) : -1;
        const bool ok = rows.ok(rw);
        kr[u] = __builtin_nontemporal_load(ok ? &kraw[rw * LPK + sub] : trash_slot);
        vr[u] = __builtin_nontemporal_load(ok ? &vraw[rw * LPK + sub] : trash_slot);
        // a slot that is not a key reads the trash slot's first word; its logit is discarded
        if constexpr (FOX) cr[u] = *(ok ? &cum_cache[rw] : trash);
        else cr[u] = 0.f;
      }
    }
  };
  // The wave walks rows jw + slot + u STRIDE from its base row jw, the same trip
  // count in every lane; a group entirely past j1 is only fetched, never used.
  const int64_t jw0 = j0 + wave * KPW;
  if (jw0 < j1) fetch(jw0 + slot);
  for (int64_t jw = jw0; jw < j1; jw += STRIDE * UNR) {
    const int64_t jb = jw + slot;
    typename V::raw kc[UNR], vc[UNR];
    float cc[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      kc[u] = kr[u];
      vc[u] = vr[u];
      cc[u] = cr[u];
    }
    fetch(jb + STRIDE * UNR);
    float sv[UNR];
    bool lv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t j = jb + static_cast<int64_t>(u) * STRIDE;
      const int64_t rw = kDense ? map.row(j < j1 ? j : j1 - 1) : (j < j1 ? map.row(j) : -1);
      const bool live = j < j1 && rows.ok(rw);
      lv[u] = live;
      float kf[EPV];
      V::unpack(kc[u], kf);
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        a += wv[e] * kf[e];
        b += qv[e] * kf[e];
      }
      a = group_sum<LPK>(a);
      b = group_sum<LPK>(b);
      const float ba = bt * a;
#pragma unroll
      for (int e = 0; e < EPV; ++e) kf[e] -= ba * wv[e];
      __builtin_nontemporal_store(V::pack(kf), live ? &kraw[rw * LPK + sub] : trash_slot);
      float su = scale2 * (b - ba * wq);
      if constexpr (FOX) su += kLog2e * (ct - cc[u]);
      sv[u] = live ? su : -INFINITY;
    }
    float mb = sv[0];
#pragma unroll
    for (int u = 1; u < UNR; ++u) mb = fmaxf(mb, sv[u]);
    const float mnew = fmaxf(mrun, mb);
    if (mnew != -INFINITY) {
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] *= alpha;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float p = __builtin_amdgcn_exp2f(sv[u] - mnew);
        float vf[EPV];
        V::unpack(vc[u], vf);
        if constexpr (!kDense) {
          if (!lv[u]) {  // a slot that is not a key: its value row may hold anything
#pragma unroll
            for (int e = 0; e < EPV; ++e) vf[e] = 0.f;
          }
        }
        lrun += p;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] += p * vf[e];
      }
      mrun = mnew;
    }
  }

  // Merge the key slots of the wave (lanes with equal `sub`).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(mrun, off, 64);
    const float l2 = __shfl_xor(lrun, off, 64);
    const float mnew = fmaxf(mrun, m2);
    const float a1 = (mrun == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun - mnew);
    const float a2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mnew);
    lrun = lrun * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float o2 = __shfl_xor(acc[e], off, 64);
      acc[e] = acc[e] * a1 + o2 * a2;
    }
    mrun = mnew;
  }

  // Merge the waves through LDS.
  __shared__ float sm[NW], sl[NW];
  __shared__ float sacc[NW][D];
  if (slot == 0) {
    if (sub == 0) {
      sm[wave] = mrun;
      sl[wave] = lrun;
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) sacc[wave][sub * EPV + e] = acc[e];
  }
  __syncthreads();
  float* out = partials + (bh * nchunks + chunk) * (D + 2);
  if (threadIdx.x < D) {
    float mm = -INFINITY;
#pragma unroll
    for (int t = 0; t < NW; ++t) mm = fmaxf(mm, sm[t]);
    float ll = 0.f, oo = 0.f;
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const float a = (sm[t] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm[t] - mm);
      ll += sl[t] * a;
      oo += sacc[t][threadIdx.x] * a;
    }
    out[2 + threadIdx.x] = oo;
    if (threadIdx.x == 0) {
      out[0] = mm;
      out[1] = ll;
    }
  }
}

// One wave per (b,h): merge chunk partials with the new key, write o and lse,
// then append k_t, v_t (and, gated, c_t) at slot cache_len.
template <typename T, int D, bool FOX, class Rows>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    Rows rows, int nchunks, float scale, const T* __restrict__ q_t,
    const T* __restrict__ k_t, const T* __restrict__ v_t, const float* __restrict__ log_f_t,
    T* __restrict__ k_cache, T* __restrict__ v_cache, float* __restrict__ cum_cache,
    const float* __restrict__ partials, T* __restrict__ o, float* __restrict__ lse) {
  constexpr int PER = D / 64;
  constexpr int kPre = 8;  // chunks whose partials are fetched with the new token
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  const float* pb = partials + bh * nchunks * (D + 2);
  // Every load is issued before any is used (one memory round trip): the new
  // token, and the partials of the first kPre chunks (a chunk past the last
  // re-reads the last; there is none to read when the cache is empty).
  float qf[PER], kf[PER], vf[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = lane + 64 * t;
    qf[t] = load_f32(q_t + bh * D + e);
    kf[t] = load_f32(k_t + bh * D + e);
    vf[t] = load_f32(v_t + bh * D + e);
  }
  const int npre = nchunks < kPre ? nchunks : kPre;
  float pm[kPre], pl[kPre], pa[kPre][PER];
  if (nchunks > 0) {
#pragma unroll
    for (int c = 0; c < kPre; ++c) {
      const float* p = pb + (c < nchunks ? c : nchunks - 1) * (D + 2);
      pm[c] = p[0];
      pl[c] = p[1];
#pragma unroll
      for (int t = 0; t < PER; ++t) pa[c][t] = p[2 + lane + 64 * t];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < PER; ++t) s += qf[t] * kf[t];
  s = scale * 1.4426950408889634f * wave_sum(s);  // log2 units, like the partials

  float mm = s;
#pragma unroll
  for (int c = 0; c < kPre; ++c)
    if (c < npre) mm = fmaxf(mm, pm[c]);
  for (int c = kPre; c < nchunks; ++c) mm = fmaxf(mm, pb[c * (D + 2)]);
  const float es = __builtin_amdgcn_exp2f(s - mm);
  float ll = es;
  float oo[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) oo[t] = es * vf[t];
#pragma unroll
  for (int c = 0; c < kPre; ++c) {
    if (c < npre) {
      const float a = __builtin_amdgcn_exp2f(pm[c] - mm);
      ll += a * pl[c];
#pragma unroll
      for (int t = 0; t < PER; ++t) oo[t] += a * pa[c][t];
    }
  }
  for (int c = kPre; c < nchunks; ++c) {
    const float* p = pb + c * (D + 2);
    const float a = __builtin_amdgcn_exp2f(p[0] - mm);
    ll += a * p[1];
#pragma unroll
    for (int t = 0; t < PER; ++t) oo[t] += a * p[2 + lane + 64 * t];
  }
  const float inv = 1.f / ll;
  const int64_t len = rows.length(bh);
  const int64_t slot = rows.row(bh, len);  // the new key's row (skipped when not mapped)
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = lane + 64 * t;
    store_f32(o + bh * D + e, oo[t] * inv);
    if (rows.ok(slot)) {
      k_cache[slot * D + e] = k_t[bh * D + e];
      v_cache[slot * D + e] = v_t[bh * D + e];
    }
  }
  if (lane == 0) {
    lse[bh] = (mm + __log2f(ll)) * 0.69314718055994531f;
    if constexpr (FOX) {
      // c_t at the new key's row of the prefix cache (same row map as the keys)
      // (ContigRows reports every row as mapped: len > 0 keeps row -1 unread)
      const int64_t prow = len > 0 ? rows.row(bh, len - 1) : -1;
      if (rows.ok(slot)) cum_cache[slot] = (len > 0 && rows.ok(prow) ? cum_cache[prow] : 0.f) + log_f_t[bh];
    }
  }
}

int64_t decode_num_chunks(int64_t cache_len) { return (cache_len + kDecChunk - 1) / kDecChunk; }

template <typename T, int D, bool FOX>
static hipError_t launch_dec_t(int64_t BH, float scale, const void* q_t, const void* k_t,
                               const void* v_t, const void* w_t, const float* beta_t,
                               const float* log_f_t, void* k_cache, void* v_cache, float* cum_cache,
                               int64_t cache_len, int64_t capacity, void* o, float* lse,
                               float* partials, hipStream_t stream) {
  const int nchunks = static_cast<int>(decode_num_chunks(cache_len));
  const ContigRows rows{capacity, cache_len};
  float* trash = partials;
  partials += kDecTrashFloats;
  if (nchunks > 0) {
    hipLaunchKernelGGL((decode_chunk_kernel<T, D, FOX, ContigRows>), dim3(static_cast<unsigned>(BH * nchunks)),
                       dim3(kDecThreads), 0, stream, rows, nchunks, scale,
                       static_cast<const T*>(q_t), static_cast<const T*>(w_t), beta_t, log_f_t,
                       static_cast<T*>(k_cache), static_cast<const T*>(v_cache), cum_cache, trash, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_merge_kernel<T, D, FOX, ContigRows>), dim3(static_cast<unsigned>(BH)), dim3(64), 0,
                     stream, rows, nchunks, scale, static_cast<const T*>(q_t),
                     static_cast<const T*>(k_t), static_cast<const T*>(v_t), log_f_t,
                     static_cast<T*>(k_cache), static_cast<T*>(v_cache), cum_cache, partials,
                     static_cast<T*>(o), lse);
  return hipGetLastError();
}

template <bool FOX>
static hipError_t launch_dec_fox(int dtype, int64_t BH, int64_t d, float scale, const void* q_t,
                                 const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                                 const float* log_f_t, void* k_cache, void* v_cache, float* cum_cache,
                                 int64_t cache_len, int64_t capacity, void* o, float* lse,
                                 float* partials, hipStream_t stream) {
  auto go = [&](auto launch) {
    return launch(BH, scale, q_t, k_t, v_t, w_t, beta_t, log_f_t, k_cache, v_cache, cum_cache, cache_len,
                  capacity, o, lse, partials, stream);
  };
  if (dtype == 0) return d == 64 ? go(launch_dec_t<float, 64, FOX>) : go(launch_dec_t<float, 128, FOX>);
  return d == 64 ? go(launch_dec_t<bf16_t, 64, FOX>) : go(launch_dec_t<bf16_t, 128, FOX>);
}

hipError_t launch_decode(int dtype, int64_t BH, int64_t d, float scale, const void* q_t,
                         const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                         const float* log_f_t, void* k_cache, void* v_cache, float* cum_cache,
                         int64_t cache_len, int64_t capacity, void* o, float* lse, float* partials,
                         hipStream_t stream) {
  if (log_f_t)
    return launch_dec_fox<true>(dtype, BH, d, scale, q_t, k_t, v_t, w_t, beta_t, log_f_t, k_cache,
                                v_cache, cum_cache, cache_len, capacity, o, lse, partials, stream);
  return launch_dec_fox<false>(dtype, BH, d, scale, q_t, k_t, v_t, w_t, beta_t, nullptr, k_cache, v_cache,
                               nullptr, cache_len, capacity, o, lse, partials, stream);
}

template <typename T, int D, bool FOX>
static hipError_t launch_dec_paged_t(int64_t BH, float scale, const void* q_t, const void* k_t, const void* v_t,
                                     const void* w_t, const float* beta_t, const float* log_f_t, void* k_pages,
                                     void* v_pages, float* cum_pages, const PagedRows& rows, int64_t max_len,
                                     void* o, float* lse, float* partials, hipStream_t stream) {
  const int nchunks = static_cast<int>(decode_num_chunks(max_len));
  float* trash = partials;
  partials += kDecTrashFloats;
  if (nchunks > 0) {
    hipLaunchKernelGGL((decode_chunk_kernel<T, D, FOX, PagedRows>), dim3(static_cast<unsigned>(BH * nchunks)),
                       dim3(kDecThreads), 0, stream, rows, nchunks, scale, static_cast<const T*>(q_t),
                       static_cast<const T*>(w_t), beta_t, log_f_t, static_cast<T*>(k_pages),
                       static_cast<const T*>(v_pages), cum_pages, trash, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_merge_kernel<T, D, FOX, PagedRows>), dim3(static_cast<unsigned>(BH)), dim3(64), 0,
                     stream, rows, nchunks, scale, static_cast<const T*>(q_t), static_cast<const T*>(k_t),
                     static_cast<const T*>(v_t), log_f_t, static_cast<T*>(k_pages), static_cast<T*>(v_pages),
                     cum_pages, partials, static_cast<T*>(o), lse);
  return hipGetLastError();
}

hipError_t launch_decode_paged(int dtype, int64_t B, int64_t H, int64_t d, float scale, const void* q_t,
                               const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                               const float* log_f_t, void* k_pages, void* v_pages, float* cum_pages,
                               int64_t num_pages, int64_t page_size, const int32_t* page_table, int64_t max_pages,
                               const int32_t* cache_lens, int64_t max_len, void* o, float* lse, float* partials,
                               hipStream_t stream) {
  int shift = -1;
  if ((page_size & (page_size - 1)) == 0)
    for (shift = 0; (int64_t(1) << shift) < page_size; ++shift) {
    }
  const PagedRows rows{page_table, cache_lens, H, max_pages, num_pages, page_size, shift};
  const int64_t BH = B * H;
  auto go = [&](auto launch) {
    return launch(BH, scale, q_t, k_t, v_t, w_t, beta_t, log_f_t, k_pages, v_pages, cum_pages, rows, max_len, o,
                  lse, partials, stream);
  };
  if (log_f_t) {
    if (dtype == 0)
      return d == 64 ? go(launch_dec_paged_t<float, 64, true>) : go(launch_dec_paged_t<float, 128, true>);
    return d == 64 ? go(launch_dec_paged_t<bf16_t, 64, true>) : go(launch_dec_paged_t<bf16_t, 128, true>);
  }
  if (dtype == 0) return d == 64 ? go(launch_dec_paged_t<float, 64, false>) : go(launch_dec_paged_t<float, 128, false>);
  return d == 64 ? go(launch_dec_paged_t<bf16_t, 64, false>) : go(launch_dec_paged_t<bf16_t, 128, false>);
}

}  // namespace path
