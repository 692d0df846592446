// C ABI of the PaTH attention library: argument checks on the host, workspace
// carve-up, and kernel launches on the caller's stream.  Nothing here touches
// the GPU before every argument has been validated.
#include "../../include/path_attn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "launch.h"

namespace {

constexpr int64_t kBlk = 64;
constexpr size_t kAlign = 256;
// Largest element count accepted for one tensor (keeps byte sizes and 64-bit
// index arithmetic far from overflow).
constexpr int64_t kMaxElems = int64_t(1) << 40;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// bf16 rows move in 16-byte pieces, so bf16 tensors must start on 16 bytes.
bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxElems / a) return false;
  *out = a * b;
  return *out <= kMaxElems;
}

int check_dtype(int dtype) {
  return (dtype == PATH_F32 || dtype == PATH_BF16) ? PATH_OK : PATH_ERR_UNSUPPORTED;
}

int check_d(int64_t d) { return (d == 64 || d == 128) ? PATH_OK : PATH_ERR_UNSUPPORTED; }

// Validates B, H, L, d and returns B*H and the padded block count.
int check_shape(int64_t B, int64_t H, int64_t L, int64_t d, int64_t* BH, int64_t* Nb) {
  if (B < 1 || H < 1 || L < 1) return PATH_ERR_SHAPE;
  int st = check_d(d);
  if (st) return st;
  int64_t bh, bhl, n;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, L, &bhl) || !mul_ok(bhl, d, &n)) return PATH_ERR_SHAPE;
  const int64_t nb = (L + kBlk - 1) / kBlk;
  int64_t pt;
  if (!mul_ok(bh * nb, d * d, &pt) || !mul_ok(bh * nb, kBlk * kBlk, &pt)) return PATH_ERR_SHAPE;
  // one workgroup per (b, h, block) must fit a 32-bit grid
  if (bh * nb > (int64_t(1) << 31) - 1) return PATH_ERR_SHAPE;
  *BH = bh;
  *Nb = nb;
  return PATH_OK;
}

constexpr float kLog2e = 1.4426950408889634f;

// Precision switch of the bf16 forward (AUTO).  With plain fp16 operands a
// logit k.q takes d rounding errors of at most 2^-11 relative on each operand.
// Modelled as independent and uniform, their sum has the rms
//     2^-11 sqrt(2/3) |q| |k| / sqrt(d),
// sqrt(d) below the worst case (all errors aligned).  AUTO drops a key block's
// lo terms while this estimate, taken with the largest transported query norm
// of the tile and the largest key norm of the block (its own logits) or of all
// the key blocks the tile scans (the query transport, whose error reaches
// every earlier block), is at most half the lse tolerance (kAutoRmsNats).  The scan kernels test
//     |Qt|_max |khat|_max 2^-10 > tau
// so tau = kAutoRmsNats log2(e) sqrt(6) sqrt(d).  This is an estimate, not a
// bound: ACCURATE runs the split everywhere.
constexpr float kAutoRmsNats = 0.5e-3f;
float auto_tau(int64_t d) { return kAutoRmsNats * kLog2e * 2.449489743f * sqrtf(static_cast<float>(d)); }

// Workspace of the forward.  fp32 inputs: khat, pT (fp32) and cum.  bf16
// inputs: the matrix-core layout written by the prepare stage.
struct FwdWs {
  size_t khat, pT, cum;                       // fp32 path
  size_t khl, pmat, qhat, sdiag, kmax, pnorm, vt, vexp;  // bf16 path (cum shared)
  size_t total;
};

FwdWs fwd_layout(int dtype, int64_t BH, int64_t L, int64_t d, int64_t Nb, bool with_forget) {
  FwdWs w{};
  size_t off = 0;
  const size_t bh = size_t(BH), nb = size_t(Nb), dd = size_t(d), lp = nb * size_t(kBlk);
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  if (dtype == PATH_F32) {
    w.khat = take(sizeof(float) * bh * size_t(L) * dd);
    w.pT = take(sizeof(float) * bh * nb * dd * dd);
    if (with_forget) w.cum = take(sizeof(float) * bh * size_t(L));
  } else {
    w.khl = take(2 * bh * nb * 2 * size_t(kBlk) * dd);
    w.pmat = take(2 * bh * nb * 2 * dd * dd);
    w.qhat = take(sizeof(float) * bh * lp * dd);
    w.sdiag = take(sizeof(float) * bh * nb * size_t(path::kDiagTri));
    w.kmax = take(sizeof(float) * bh * nb);
    w.pnorm = take(sizeof(float) * bh * nb);
    w.vt = take(2 * bh * nb * dd * size_t(kBlk));
    w.vexp = take(sizeof(int) * bh * nb);
    if (with_forget) w.cum = take(sizeof(float) * bh * lp);
  }
  w.total = off;
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PATH_OK : PATH_ERR_HIP; }

}  // namespace

extern "C" {

const char* path_status_string(int status) {
  switch (status) {
    case PATH_OK: return "ok";
    case PATH_ERR_NULL: return "a required pointer is NULL";
    case PATH_ERR_SHAPE: return "sizes out of range or overflowing";
    case PATH_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or precision";
    case PATH_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PATH_ERR_CAPACITY: return "decode cache is full (cache_len >= capacity)";
    case PATH_ERR_HIP: return "HIP kernel launch failed";
    case PATH_ERR_SCRATCH: return "needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int path_abi_version(void) { return 1; }

int path_prepare(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, const void* q,
                 const void* k, const void* w, const float* beta, const float* log_forget,
                 float* tinv, float* qhat, float* khat, float* pT, float* cum,
                 hipStream_t stream) {
  int64_t BH, Nb;
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_shape(B, H, L, d, &BH, &Nb))) return st;
  if (!w || !beta) return PATH_ERR_NULL;
  if (qhat && !q) return PATH_ERR_NULL;
  if (khat && !k) return PATH_ERR_NULL;
  if (cum && !log_forget) return PATH_ERR_NULL;
  if (tinv || qhat || khat || pT) {
    st = hip_status(path::launch_prepare_f32(dtype, B, H, L, d, q, k, w, beta, tinv, nullptr, qhat, khat, pT,
                                             nullptr, stream));
    if (st) return st;
  }
  if (cum) st = hip_status(path::launch_prefix_sum(BH, L, log_forget, cum, stream));
  return st;
}

size_t path_fwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d, int dtype,
                                int with_forget) {
  int64_t BH, Nb;
  if (check_dtype(dtype) || check_shape(B, H, L, d, &BH, &Nb)) return 0;
  return fwd_layout(dtype, BH, L, d, Nb, with_forget != 0).total;
}

}  // extern "C"

namespace {

struct FwdArgs {
  int64_t BH, Nb;
  FwdWs lay;
};

int fwd_check(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, int precision, const void* q,
              const void* k, const void* v, const void* w, const float* beta,
              const float* log_forget, void* workspace, size_t workspace_bytes, FwdArgs* a) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (precision != PATH_PREC_ACCURATE && precision != PATH_PREC_AUTO) return PATH_ERR_UNSUPPORTED;
  if ((st = check_shape(B, H, L, d, &a->BH, &a->Nb))) return st;
  if (!q || !k || !v || !w || !beta) return PATH_ERR_NULL;
  if (dtype == PATH_BF16 && (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(w)))
    return PATH_ERR_UNSUPPORTED;
  a->lay = fwd_layout(dtype, a->BH, L, d, a->Nb, log_forget != nullptr);
  if (!workspace || workspace_bytes < a->lay.total ||
      (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return PATH_ERR_WORKSPACE;
  return PATH_OK;
}

int fwd_prepare(const FwdArgs& a, int64_t B, int64_t H, int64_t L, int64_t d, int dtype,
                float scale, const void* q, const void* k, const void* v, const void* w,
                const float* beta, const float* log_forget, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  int st;
  if (dtype == PATH_F32) {
    float* khat = reinterpret_cast<float*>(ws + a.lay.khat);
    float* pT = reinterpret_cast<float*>(ws + a.lay.pT);
    st = hip_status(path::launch_prepare_f32(dtype, B, H, L, d, nullptr, k, w, beta, nullptr, nullptr,
                                             nullptr, khat, pT, nullptr, stream));
    if (st) return st;
    if (log_forget) {
      float* cum = reinterpret_cast<float*>(ws + a.lay.cum);
      st = hip_status(path::launch_prefix_sum(a.BH, L, log_forget, cum, stream));
    }
    return st;
  }
  float* kmax = reinterpret_cast<float*>(ws + a.lay.kmax);
  st = hip_status(path::launch_prepare_mfma(
      B, H, L, d, scale * kLog2e, q, k, w, v, beta, reinterpret_cast<_Float16*>(ws + a.lay.khl),
      reinterpret_cast<_Float16*>(ws + a.lay.pmat), reinterpret_cast<float*>(ws + a.lay.qhat),
      reinterpret_cast<float*>(ws + a.lay.sdiag), kmax, reinterpret_cast<float*>(ws + a.lay.pnorm),
      reinterpret_cast<_Float16*>(ws + a.lay.vt), reinterpret_cast<int*>(ws + a.lay.vexp), stream));
  if (st || !log_forget) return st;
  return hip_status(
      path::launch_cum_padded(a.BH, L, log_forget, kLog2e, reinterpret_cast<float*>(ws + a.lay.cum), stream));
}

int fwd_scan(const FwdArgs& a, int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale,
             int precision, const void* q, const void* k, const void* v, const void* w,
             const float* beta, const float* log_forget, void* o, float* lse, void* workspace,
             hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  const float* cum = log_forget ? reinterpret_cast<const float*>(ws + a.lay.cum) : nullptr;
  if (dtype == PATH_F32) {
    const float* khat = reinterpret_cast<const float*>(ws + a.lay.khat);
    const float* pT = reinterpret_cast<const float*>(ws + a.lay.pT);
    return hip_status(path::launch_fwd_scan_f32(dtype, B, H, L, d, scale, q, k, v, w, beta, cum,
                                                khat, pT, o, lse, stream));
  }
  // one matrix-core scan per head dimension (64 or 128; check_d rejects others)
  auto scan = d == 64 ? path::launch_scan64 : path::launch_scan128;
  return hip_status(scan(
      B * H, L, precision == PATH_PREC_ACCURATE ? 1 : 0, auto_tau(d),
      reinterpret_cast<const _Float16*>(ws + a.lay.vt), reinterpret_cast<const _Float16*>(ws + a.lay.khl),
      reinterpret_cast<const _Float16*>(ws + a.lay.pmat),
      reinterpret_cast<const float*>(ws + a.lay.qhat),
      reinterpret_cast<const float*>(ws + a.lay.sdiag),
      reinterpret_cast<const float*>(ws + a.lay.kmax), reinterpret_cast<const float*>(ws + a.lay.pnorm),
      reinterpret_cast<const int*>(ws + a.lay.vexp), cum, o, lse, stream));
}

}  // namespace

extern "C" {

int path_fwd_stage_prepare(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale,
                           int precision, const void* q, const void* k, const void* v,
                           const void* w, const float* beta, const float* log_forget,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  FwdArgs a;
  int st = fwd_check(B, H, L, d, dtype, precision, q, k, v, w, beta, log_forget, workspace,
                     workspace_bytes, &a);
  if (st) return st;
  return fwd_prepare(a, B, H, L, d, dtype, scale, q, k, v, w, beta, log_forget, workspace, stream);
}

int path_fwd_stage_scan(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale,
                        int precision, const void* q, const void* k, const void* v, const void* w,
                        const float* beta, const float* log_forget, void* o, float* lse,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  FwdArgs a;
  int st = fwd_check(B, H, L, d, dtype, precision, q, k, v, w, beta, log_forget, workspace,
                     workspace_bytes, &a);
  if (st) return st;
  if (!o || !lse) return PATH_ERR_NULL;
  if (dtype == PATH_BF16 && misaligned16(o)) return PATH_ERR_UNSUPPORTED;
  return fwd_scan(a, B, H, L, d, dtype, scale, precision, q, k, v, w, beta, log_forget, o, lse,
                  workspace, stream);
}

int path_attn_fwd(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale,
                  int precision, const void* q, const void* k, const void* v, const void* w,
                  const float* beta, const float* log_forget, void* o, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  FwdArgs a;
  int st = fwd_check(B, H, L, d, dtype, precision, q, k, v, w, beta, log_forget, workspace,
                     workspace_bytes, &a);
  if (st) return st;
  if (!o || !lse) return PATH_ERR_NULL;
  if (dtype == PATH_BF16 && misaligned16(o)) return PATH_ERR_UNSUPPORTED;
  if ((st = fwd_prepare(a, B, H, L, d, dtype, scale, q, k, v, w, beta, log_forget, workspace, stream)))
    return st;
  return fwd_scan(a, B, H, L, d, dtype, scale, precision, q, k, v, w, beta, log_forget, o, lse,
                  workspace, stream);
}

size_t path_decode_workspace_bytes(int64_t B, int64_t H, int64_t d, int64_t cache_len) {
  if (B < 1 || H < 1 || cache_len < 0 || check_d(d)) return 0;
  int64_t BH, n;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, path::decode_num_chunks(cache_len), &n) ||
      !mul_ok(n, d + 2, &n))
    return 0;
  // a 512-byte slot for the key loop's stores past a chunk's end, then the partials
  return 512 + align_up(sizeof(float) * size_t(n > 0 ? n : 1));
}

}  // extern "C"

namespace {

int decode_common(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t, const void* k_t,
                  const void* v_t, const void* w_t, const float* beta_t, const float* log_f_t, void* k_cache,
                  void* v_cache, float* cum_cache, int64_t cache_len, int64_t capacity, void* o, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_d(d))) return st;
  if (B < 1 || H < 1 || capacity < 1 || cache_len < 0) return PATH_ERR_SHAPE;
  int64_t BH, n;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, capacity, &n) || !mul_ok(n, d, &n)) return PATH_ERR_SHAPE;
  if (cache_len >= capacity) return PATH_ERR_CAPACITY;
  if (BH * path::decode_num_chunks(cache_len) > (int64_t(1) << 31) - 1) return PATH_ERR_SHAPE;
  if (!q_t || !k_t || !v_t || !w_t || !beta_t || !k_cache || !v_cache || !o || !lse)
    return PATH_ERR_NULL;
  const size_t need = path_decode_workspace_bytes(B, H, d, cache_len);
  if (!workspace || need == 0 || workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return PATH_ERR_WORKSPACE;
  return hip_status(path::launch_decode(dtype, BH, d, scale, q_t, k_t, v_t, w_t, beta_t, log_f_t, k_cache,
                                        v_cache, cum_cache, cache_len, capacity, o, lse,
                                        static_cast<float*>(workspace), stream));
}

}  // namespace

extern "C" {

int path_decode_step(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                     const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                     void* k_cache, void* v_cache, int64_t cache_len, int64_t capacity, void* o,
                     float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(B, H, d, dtype, scale, q_t, k_t, v_t, w_t, beta_t, nullptr, k_cache, v_cache, nullptr,
                       cache_len, capacity, o, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// ---- allocation-free decode --------------------------------------------------------
// path_decode_step_noalloc keeps the decode step's scratch (the store slot and the
// per-chunk partials) in this file-scope device array instead of a caller
// workspace.  Each GPU that runs the library holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel: its device address
// is resolved once per device with hipGetSymbolAddress and kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), resolved on the first call there.
int scratch_address(hipStream_t stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return PATH_ERR_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return PATH_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PATH_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return PATH_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return PATH_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PATH_OK;
}

}  // namespace

extern "C" {

size_t path_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int path_decode_step_noalloc(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                             const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                             void* k_cache, void* v_cache, int64_t cache_len, int64_t capacity, void* o,
                             float* lse, hipStream_t stream) {
  // the same checks as path_decode_step, in the same order, before the scratch size
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_d(d))) return st;
  if (B < 1 || H < 1 || capacity < 1 || cache_len < 0) return PATH_ERR_SHAPE;
  const size_t need = path_decode_workspace_bytes(B, H, d, cache_len);
  if (need == 0) return PATH_ERR_SHAPE;
  if (need > kScratchBytes) return PATH_ERR_SCRATCH;
  void* ws = nullptr;
  if (cache_len < capacity && q_t && k_t && v_t && w_t && beta_t && k_cache && v_cache && o && lse) {
    if ((st = scratch_address(stream, &ws))) return st;
  }
  return decode_common(B, H, d, dtype, scale, q_t, k_t, v_t, w_t, beta_t, nullptr, k_cache, v_cache, nullptr,
                       cache_len, capacity, o, lse, ws, kScratchBytes, stream);
}

int path_decode_step_fox(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                         const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                         const float* log_f_t, void* k_cache, void* v_cache, float* cum_cache,
                         int64_t cache_len, int64_t capacity, void* o, float* lse, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!log_f_t || !cum_cache) return PATH_ERR_NULL;
  return decode_common(B, H, d, dtype, scale, q_t, k_t, v_t, w_t, beta_t, log_f_t, k_cache, v_cache,
                       cum_cache, cache_len, capacity, o, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

struct BwdLayout {
  size_t qhat, khat, pT, minv, cum, Dv, dqh, rsum, dkh, dP, dV, csum, dc, scratch, packed, total;
  int64_t zero_count;
};

// Returns false when the sizes overflow.  `pack16` (bf16 storage) adds the
// split bf16 key-side operands of the 16-bit pair kernels: Khat, Khat^T, P_n
// and P_n^T, each hi and lo, 4*64*d + 4*d*d bf16 per block.
bool bwd_layout(int64_t BH, int64_t L, int64_t d, int64_t Nb, bool with_forget, bool pack16, BwdLayout* w) {
  int64_t pairs, scr;
  if (!mul_ok(BH, Nb * (Nb - 1) / 2, &pairs) || !mul_ok(pairs, d * kBlk, &scr)) return false;
  size_t off = 0;
  const size_t bh = size_t(BH), nb = size_t(Nb), dd = size_t(d), l = size_t(L);
  auto take = [&](size_t floats) {
    size_t at = off;
    off += align_up(sizeof(float) * floats);
    return at;
  };
  *w = BwdLayout{};
  w->qhat = take(bh * l * dd);
  w->khat = pack16 ? 0 : take(bh * l * dd);
  w->pT = pack16 ? 0 : take(bh * nb * dd * dd);
  w->minv = take(bh * nb * size_t(kBlk) * kBlk);
  if (with_forget) w->cum = take(bh * l);
  w->Dv = take(bh * l);
  w->dqh = take(bh * l * dd);
  w->rsum = take(bh * l);
  w->dc = take(bh * l);
  // cleared together, in this order and without gaps
  w->dkh = take(bh * l * dd);
  w->dP = take(bh * nb * dd * dd);
  w->dV = take(bh * l * dd);
  w->csum = take(bh * l);
  w->zero_count = int64_t((off - w->dkh) / sizeof(float));
  w->scratch = take(size_t(scr));
  w->packed = pack16 ? take(bh * nb * (4 * size_t(kBlk) * dd + 4 * dd * dd) / 2) : 0;
  w->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t path_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, int with_forget) {
  int64_t BH, Nb;
  if (check_dtype(dtype) || check_shape(B, H, L, d, &BH, &Nb)) return 0;
  BwdLayout lay;
  if (!bwd_layout(BH, L, d, Nb, with_forget != 0, dtype == PATH_BF16, &lay)) return 0;
  return lay.total;
}

int path_attn_bwd(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale, const void* q,
                  const void* k, const void* v, const void* w, const float* beta, const float* log_forget,
                  const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dw,
                  float* dbeta, float* dlog_forget, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  int64_t BH, Nb;
  if ((st = check_shape(B, H, L, d, &BH, &Nb))) return st;
  if (!q || !k || !v || !w || !beta || !o || !lse || !dout || !dq || !dk || !dv || !dw || !dbeta)
    return PATH_ERR_NULL;
  if (log_forget && !dlog_forget) return PATH_ERR_NULL;
  if (dtype == PATH_BF16) {
    for (const void* p : {q, k, v, w, o, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv), static_cast<const void*>(dw)})
      if (misaligned16(p)) return PATH_ERR_UNSUPPORTED;
  }
  BwdLayout lay;
  const bool pack16 = dtype == PATH_BF16;
  if (!bwd_layout(BH, L, d, Nb, log_forget != nullptr, pack16, &lay)) return PATH_ERR_SHAPE;
  if (!workspace || workspace_bytes < lay.total || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return PATH_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  path::BwdArgs a{};
  a.BH = BH;
  a.L = L;
  a.scale = scale;
  a.q = q;
  a.k = k;
  a.v = v;
  a.w = w;
  a.beta = beta;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dw = dw;
  a.dbeta = dbeta;
  a.dlog_forget = log_forget ? dlog_forget : nullptr;
  a.ws = path::BwdWs{at(lay.qhat), pack16 ? nullptr : at(lay.khat), pack16 ? nullptr : at(lay.pT), at(lay.minv), log_forget ? at(lay.cum) : nullptr,
                     at(lay.Dv),
                     at(lay.dqh), at(lay.rsum), at(lay.dkh), at(lay.dP), at(lay.dV), at(lay.csum), at(lay.dc),
                     at(lay.scratch), pack16 ? static_cast<void*>(ws + lay.packed) : nullptr,
                     at(lay.dkh), lay.zero_count};
  // bf16: the matrix-core prepare writes Khat and P_n straight into the split
  // bf16 operands of the 16-bit kernels; fp32: the fp32 prepare
  st = pack16 ? hip_status(path::launch_prepare_mfma_bwd(BH, L, d, q, k, w, beta, a.ws.packed, a.ws.qhat,
                                                         a.ws.minv, stream))
              : hip_status(path::launch_prepare_f32(dtype, B, H, L, d, q, k, w, beta, nullptr, a.ws.minv, a.ws.qhat,
                                                    a.ws.khat, a.ws.pT, nullptr, stream));
  if (st) return st;
  if (log_forget && (st = hip_status(path::launch_prefix_sum(BH, L, log_forget, a.ws.cum, stream)))) return st;
  return hip_status(path::launch_bwd(dtype, d, a, stream));
}

}  // extern "C"

extern "C" int path_project(int64_t B, int64_t L, int64_t Dm, int64_t H, int64_t d, const void* x,
                            const void* Ww, const void* u, const float* bias, float beta_max, void* w,
                            float* beta, hipStream_t stream) {
  if (B < 1 || L < 1 || H < 1 || Dm < 1 || Dm % 64 != 0) return PATH_ERR_SHAPE;
  int st = check_d(d);
  if (st) return st;
  int64_t T, xe, we, oe, tiles_cols;
  if (!mul_ok(B, L, &T) || !mul_ok(T, Dm, &xe) || !mul_ok(H * d, Dm, &we) || !mul_ok(T * H, d, &oe))
    return PATH_ERR_SHAPE;
  // token tiles (256 tokens; 128 bounds them) times 128-column groups (w of whole heads, then beta
  // logits) must fit a 32-bit grid
  const int64_t ncol = (H * d + 127) / 128 + (H + 127) / 128;
  if (!mul_ok(((T + 127) / 128 + 7) / 8 * 8, ncol, &tiles_cols) || tiles_cols > (int64_t(1) << 31) - 1)
    return PATH_ERR_SHAPE;
  if (!x || !Ww || !u || !bias || !w || !beta) return PATH_ERR_NULL;
  if (misaligned16(x) || misaligned16(Ww) || misaligned16(u) || misaligned16(w)) return PATH_ERR_UNSUPPORTED;
  return hip_status(path::launch_project(B, L, Dm, H, d, x, Ww, u, bias, beta_max, w, beta, stream));
}

namespace {

int paged_common(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t, const void* k_t,
                 const void* v_t, const void* w_t, const float* beta_t, const float* log_f_t, void* k_pages,
                 void* v_pages, float* cum_pages, int64_t num_pages, int64_t page_size, const int32_t* page_table,
                 int64_t max_pages, const int32_t* cache_lens, int64_t max_cache_len, void* o, float* lse,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_d(d))) return st;
  if (B < 1 || H < 1 || page_size < 1 || num_pages < 1 || max_pages < 1 || max_cache_len < 0)
    return PATH_ERR_SHAPE;
  int64_t BH, n, tbl, slots;
  if (!mul_ok(B, H, &BH) || !mul_ok(num_pages, H, &n) || !mul_ok(n, page_size, &n) || !mul_ok(n, d, &n) ||
      !mul_ok(B, max_pages, &tbl) || !mul_ok(max_pages, page_size, &slots))
    return PATH_ERR_SHAPE;
  // page ids are int32, rows are (page * H + h) * page_size + slot, and key
  // indices stay below 2^31 (the kernels map them with 32-bit arithmetic)
  if (num_pages > (int64_t(1) << 31) - 1 || slots > (int64_t(1) << 31) - 1) return PATH_ERR_SHAPE;
  if (max_cache_len >= slots) return PATH_ERR_CAPACITY;
  if (BH * path::decode_num_chunks(max_cache_len) > (int64_t(1) << 31) - 1) return PATH_ERR_SHAPE;
  if (!q_t || !k_t || !v_t || !w_t || !beta_t || !k_pages || !v_pages || !page_table || !cache_lens || !o || !lse)
    return PATH_ERR_NULL;
  const size_t need = path_decode_workspace_bytes(B, H, d, max_cache_len);
  if (!workspace || need == 0 || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return PATH_ERR_WORKSPACE;
  return hip_status(path::launch_decode_paged(dtype, B, H, d, scale, q_t, k_t, v_t, w_t, beta_t, log_f_t, k_pages,
                                              v_pages, cum_pages, num_pages, page_size, page_table, max_pages,
                                              cache_lens, max_cache_len, o, lse, static_cast<float*>(workspace),
                                              stream));
}

}  // namespace

extern "C" int path_decode_step_paged(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                                      const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                                      void* k_pages, void* v_pages, int64_t num_pages, int64_t page_size,
                                      const int32_t* page_table, int64_t max_pages, const int32_t* cache_lens,
                                      int64_t max_cache_len, void* o, float* lse, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return paged_common(B, H, d, dtype, scale, q_t, k_t, v_t, w_t, beta_t, nullptr, k_pages, v_pages, nullptr,
                      num_pages, page_size, page_table, max_pages, cache_lens, max_cache_len, o, lse, workspace,
                      workspace_bytes, stream);
}

extern "C" int path_decode_step_paged_fox(int64_t B, int64_t H, int64_t d, int dtype, float scale,
                                          const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                                          const float* beta_t, const float* log_f_t, void* k_pages, void* v_pages,
                                          float* cum_pages, int64_t num_pages, int64_t page_size,
                                          const int32_t* page_table, int64_t max_pages, const int32_t* cache_lens,
                                          int64_t max_cache_len, void* o, float* lse, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  if (!log_f_t || !cum_pages) return PATH_ERR_NULL;
  return paged_common(B, H, d, dtype, scale, q_t, k_t, v_t, w_t, beta_t, log_f_t, k_pages, v_pages, cum_pages,
                      num_pages, page_size, page_table, max_pages, cache_lens, max_cache_len, o, lse, workspace,
                      workspace_bytes, stream);
}
