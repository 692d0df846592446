// Host-side launchers of the gfx950 PaTH kernels (internal to the library).
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace path {

// In-block logits of one block, stored as a padded lower triangle: query row r
// keeps keys c = 0 .. 4 floor(r/4) + 3 (the keys past r are zeros), so rows
// 4a .. 4a+3 hold 4 (a + 1) floats each and every row starts on a 16-byte
// boundary: 2176 floats per block instead of 64 x 64.
constexpr int kDiagTri = 2176;

// Per-block UT transform in fp32 (one workgroup per 64-token block).  Any of
// the outputs may be null.  Layouts as documented for path_prepare.  `packed`
// (d = 64 only) replaces khat and pT by the split bf16 operands of the 16-bit
// backward (eight 64 x 64 bf16 matrices per block, see prepare.hip).
hipError_t launch_prepare_f32(int dtype, int64_t B, int64_t H, int64_t L, int64_t d,
                              const void* q, const void* k, const void* w, const float* beta,
                              float* tinv, float* minv, float* qhat, float* khat, float* pT, void* packed,
                              hipStream_t stream);

// Per-block UT data in the layout of the matrix-core forward (bf16 inputs),
// computed on the matrix cores: khat and P (fp16 hi/lo rows, reduction index in
// mfma_perm order), c2 * adjusted queries and c2 * in-block logits (fp32, c2 =
// scale * log2(e)), kmax[bh][n] = max_c |khat_c|, pnorm[bh][n] >= |P_n|_2
// (product of the transitions' spectral norms) and V^T (fp16, keys permuted),
// each block times 2^-vexp[bh][n] (vexp = 0 unless the block holds |v| >= 2^15).
hipError_t launch_prepare_mfma(int64_t B, int64_t H, int64_t L, int64_t d, float c2, const void* q,
                               const void* k, const void* w, const void* v, const float* beta,
                               _Float16* khat, _Float16* pmat, float* qhat, float* sdiag, float* kmax,
                               float* pnorm, _Float16* vt, int* vexp, hipStream_t stream);

// The backward's block prepare with bf16 storage, on the matrix cores: Khat
// and P_n (both orientations) as split bf16 operands into `packed`
// (4*64*d + 4*d*d bf16 per block), Qhat [BH, L, d] fp32 and M [BH, Nb, 64, 64]
// fp32 (prepare_mfma.hip).
hipError_t launch_prepare_mfma_bwd(int64_t BH, int64_t L, int64_t d, const void* q, const void* k,
                                   const void* w, const float* beta, void* packed, float* qhat, float* minv,
                                   hipStream_t stream);

// Per head: cum = mult * prefix sum of log_forget (fp64 accumulation), padded
// to whole 64-token blocks by repeating the last value.
hipError_t launch_cum_padded(int64_t BH, int64_t L, const float* log_forget, float mult, float* cum,
                             hipStream_t stream);

// Matrix-core right-to-left scan forward (bf16 storage), head dimension 64
// and 128, from the prepared blocks; operands reach LDS by direct-to-LDS loads.
hipError_t launch_scan64(int64_t BH, int64_t L, int accurate, float tau, const _Float16* vt,
                         const _Float16* khat, const _Float16* pmat, const float* qhat, const float* sdiag,
                         const float* kmax_blk, const float* pnorm, const int* vexp, const float* cum,
                         void* o, float* lse, hipStream_t stream);
hipError_t launch_scan128(int64_t BH, int64_t L, int accurate, float tau, const _Float16* vt,
                          const _Float16* khat, const _Float16* pmat, const float* qhat, const float* sdiag,
                          const float* kmax_blk, const float* pnorm, const int* vexp, const float* cum,
                          void* o, float* lse, hipStream_t stream);

// c[bh, i] = sum_{s<=i} x[bh, s], accumulated in fp64.
hipError_t launch_prefix_sum(int64_t BH, int64_t L, const float* x, float* c, hipStream_t stream);

// Right-to-left block scan forward, fp32 arithmetic on the vector ALUs.
hipError_t launch_fwd_scan_f32(int dtype, int64_t B, int64_t H, int64_t L, int64_t d, float scale,
                               const void* q, const void* k, const void* v, const void* w,
                               const float* beta, const float* cum, const float* khat,
                               const float* pT, void* o, float* lse, hipStream_t stream);

// Decode: number of key chunks and partial-result floats per (b,h).  `partials`
// is the whole decode workspace: 128 floats of store slot, then the partials.  With
// log_f_t != null the step is gated: cum_cache [BH, capacity] holds the gate
// prefixes of the cached keys and receives c_t at slot cache_len.
int64_t decode_num_chunks(int64_t cache_len);
hipError_t launch_decode(int dtype, int64_t BH, int64_t d, float scale, const void* q_t,
                         const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                         const float* log_f_t, void* k_cache, void* v_cache, float* cum_cache,
                         int64_t cache_len, int64_t capacity, void* o, float* lse, float* partials,
                         hipStream_t stream);

// Decode over a paged cache: pages [num_pages, H, page_size, d]; sequence b's
// logical page lp is page_table[b * max_pages + lp] and its length
// cache_lens[b] (both int32, device); the grid covers max_len keys.
// With log_f_t != null the step is gated: cum_pages [num_pages, H, page_size]
// fp32 holds the gate prefixes of the cached keys in the key pages' layout and
// receives c_t at the new key's slot.
hipError_t launch_decode_paged(int dtype, int64_t B, int64_t H, int64_t d, float scale, const void* q_t,
                               const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                               const float* log_f_t, void* k_pages, void* v_pages, float* cum_pages,
                               int64_t num_pages, int64_t page_size, const int32_t* page_table, int64_t max_pages,
                               const int32_t* cache_lens, int64_t max_len, void* o, float* lse, float* partials,
                               hipStream_t stream);

// Projection prologue (bf16 matrix cores): w [B,H,L,d] bf16 and beta [B,H,L]
// fp32 from tokens x [B,L,Dm], Ww [H,d,Dm], u [H,Dm] (bf16) and bias [H].
hipError_t launch_project(int64_t B, int64_t L, int64_t Dm, int64_t H, int64_t d, const void* x, const void* Ww,
                          const void* u, const float* bias, float beta_max, void* w_out, float* beta_out,
                          hipStream_t stream);

// Backward pass (fp32 arithmetic).  Workspace regions, all fp32; the run from
// zero_begin over zero_count floats (dkh, dP, dV, csum) is cleared first.
struct BwdWs {
  float *qhat, *khat, *pT, *minv, *cum, *Dv, *dqh, *rsum, *dkh, *dP, *dV, *csum, *dc, *scratch;
  void* packed;  // split bf16 key-side operands (bf16 storage), else null
  float* zero_begin;
  int64_t zero_count;
};
struct BwdArgs {
  int64_t BH, L;
  float scale;
  const void *q, *k, *v, *w;
  const float* beta;
  const void* o;
  const float* lse;
  const void* dout;
  void *dq, *dk, *dv, *dw;
  float* dbeta;
  float* dlog_forget;
  BwdWs ws;  // ws.cum != null selects the gated form
};
// Launches everything after the fp32 prepare and the gate prefix sums.
hipError_t launch_bwd(int dtype, int64_t d, const BwdArgs& a, hipStream_t stream);
// The cross-block part for bf16 storage (d = 64 or 128) on the 16-bit matrix
// cores (bwd_pair16.hip), from the split operands the matrix-core prepare wrote
// to ws.packed: the query-major pair kernel, then the key-major one.
hipError_t launch_bwd_pair16(int64_t d, const BwdArgs& a, hipStream_t stream);
// The in-block part of the backward in matrix form: d = 64 (bwd_block_ut.hip).
struct BwdBlockArgs {
  int64_t BH, L;
  float scale;
  const void *q, *k, *v, *w, *dO;
  const float *beta, *cum, *lse, *Dv, *minv, *dqh, *dkh, *dP, *dV, *rsum, *csum;
  void *dq, *dk, *dv, *dw;
  float *dbeta, *dc;
};
hipError_t launch_bwd_block_ut(int dtype, const BwdBlockArgs& a, hipStream_t stream);
// The same at d = 128 for bf16 storage (bwd_block_ut128.hip).
hipError_t launch_bwd_block_ut128(const BwdBlockArgs& a, hipStream_t stream);

}  // namespace path
