/*
 * path_attn.h - C ABI of the MI355X (gfx950) PaTH attention library.
 *
 * PaTH attention [PaTH Attention technical summary, gist.science 2505.16381,
 * §2 "Mecanismo Central"]: causal softmax attention whose logit for query i
 * and key j <= i is
 *     s_ij = scale * k_j^T (H_{j+1} H_{j+2} ... H_i) q_i  (+ FoX bias),
 * with data-dependent Householder-like transitions H_s = I - beta_s w_s w_s^T.
 * The product for j = i is the identity; H_i is the first factor to act on q_i.
 *
 * Conventions shared by every call
 *  - Layouts are dense row-major.  q, k, v, w, o: [B, H, L, d] in `dtype`;
 *    beta, log_forget, lse: [B, H, L] fp32.
 *  - dtype: PATH_F32 (fp32 storage) or PATH_BF16 (bfloat16 storage).  All
 *    arithmetic accumulates in fp32 on the GPU.
 *  - d (head dimension) must be 64 or 128.  Any L >= 1 is accepted: a partial
 *    last 64-token block is padded internally with identity transitions.
 *  - Every device pointer is owned by the caller; the library allocates no
 *    memory and keeps no state between calls.  Work is enqueued on `stream`
 *    (may be NULL for the null stream) and runs asynchronously: outputs are
 *    ready once the stream reaches that point.
 *  - Arguments are checked on the host before anything is enqueued.  A
 *    non-zero return leaves all buffers untouched, except PATH_ERR_HIP, which
 *    means a launch failed after earlier work may already have been enqueued
 *    (for path_decode_step the key cache is then undefined).
 *  - No exceptions cross the ABI; calls are thread-compatible (calls on
 *    distinct buffers may run concurrently on different streams).
 */
#ifndef PATH_ATTN_H_
#define PATH_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PATH_OK = 0,
  PATH_ERR_NULL = 1,        /* a required pointer is NULL */
  PATH_ERR_SHAPE = 2,       /* a size is out of range or the sizes overflow */
  PATH_ERR_UNSUPPORTED = 3, /* d not 64/128, unknown dtype / precision, or a
                               bf16 tensor not 16-byte aligned */
  PATH_ERR_WORKSPACE = 4,   /* workspace NULL, too small or not 256-byte aligned */
  PATH_ERR_CAPACITY = 5,    /* decode: cache_len >= capacity */
  PATH_ERR_HIP = 6,         /* a kernel launch failed (see hipGetLastError) */
  PATH_ERR_SCRATCH = 7      /* path_decode_step_noalloc: the step needs more than the static scratch */
} path_status;

typedef enum { PATH_F32 = 0, PATH_BF16 = 1 } path_dtype;

/*
 * Precision policy of the bf16 forward.  ACCURATE feeds every matrix-core
 * product that involves a transported query or key with a two-term (hi + lo)
 * split of its fp32 value, on every key block.  AUTO uses the split only on
 * the key blocks where a run-time estimate of the logit rounding error of
 * plain half-precision operands (the rms of d independent roundings, with the
 * tile's largest transported query norm) exceeds half the lse tolerance of
 * 1e-3: for the block's own logits with the block's largest key norm, for
 * the query transport (whose error reaches every earlier key block) with the
 * head's largest key norm.  Transported queries shrink block by block, so
 * these are the blocks nearest the query.  AUTO's switch is an
 * estimate, not a bound; ACCURATE is the mode with no such assumption.
 * fp32 inputs always take the fp32 path and ignore this flag.
 */
typedef enum { PATH_PREC_ACCURATE = 0, PATH_PREC_AUTO = 1 } path_precision;

/* Human-readable name of a status code (static storage, never NULL). */
const char* path_status_string(int status);

/* ABI version of this header (bumped on any incompatible change). */
int path_abi_version(void);

/*
 * path_prepare - per-block UT transform and boundary-adjusted queries/keys.
 * [PaTH summary §3 "Representação de Transformação UT" and "Algoritmo Estilo
 * FlashAttention"]: the sequence is cut into Nb = ceil(L/64) blocks of 64
 * tokens; for block n with rows w_s (local index s = 0..63) and beta_s,
 *   tinv = T^{-1} = (I + diag(beta) strict_upper(W W^T))^{-1} diag(beta)
 *          (upper triangular; T = diag(1/beta) + strict_upper(W W^T)),
 *   qhat_r = H_0 H_1 ... H_r q_r                 = q_r - W^T T^{-1} ((W q_r) masked to s <= r),
 *   khat_c = (H_{c+1} ... H_63)^T k_c            = k_c - W^T T^{-T} ((W k_c) masked to s > c),
 *   pT     = (H_0 H_1 ... H_63)^T                = I - W^T T^{-T} W,
 *   cum_i  = sum_{s <= i} log_forget_s           (accumulated in fp64, stored fp32).
 * Inputs: q, k, w [B,H,L,d] (dtype); beta [B,H,L]; log_forget [B,H,L] or NULL.
 * Outputs (fp32, caller-allocated, each may be NULL to skip it):
 *   tinv [B,H,Nb,64,64], qhat [B,H,L,d], khat [B,H,L,d], pT [B,H,Nb,d,d],
 *   cum [B,H,L] (requires log_forget).
 */
int path_prepare(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, const void* q,
                 const void* k, const void* w, const float* beta, const float* log_forget,
                 float* tinv, float* qhat, float* khat, float* pT, float* cum,
                 hipStream_t stream);

/* Workspace bytes path_attn_fwd needs for these sizes (0 on invalid sizes). */
size_t path_fwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d, int dtype,
                                int with_forget);

/*
 * path_attn_fwd - PaTH causal attention forward [PaTH summary §2 "Mecanismo
 * Central"; PaTH-FoX bias from §2 "Extensões: PaTH-FoX"]:
 *   s_ij = scale * k_j^T (H_{j+1}...H_i) q_i + (log_forget ? sum_{s=j+1..i} log_forget_s : 0)
 *   o_i  = sum_{j<=i} softmax_j(s_ij) v_j,   lse_i = log sum_{j<=i} exp(s_ij)  (natural log)
 * Runs the block prepare into `workspace`, then a right-to-left scan over key
 * blocks per query tile [§3 "Algoritmo Estilo FlashAttention"].
 * Inputs: q, k, v, w [B,H,L,d] (dtype); beta [B,H,L]; log_forget [B,H,L] or
 *   NULL; scale multiplies the PaTH term only.  Every input must be finite.
 * Outputs: o [B,H,L,d] (dtype, bf16 rounded to nearest even), lse [B,H,L] fp32.
 * Alignment: with PATH_BF16, q, k, v, w and o must be 16-byte aligned (rows
 *   move in 16-byte pieces); PATH_ERR_UNSUPPORTED otherwise, before any launch.
 * workspace: device buffer of at least path_fwd_workspace_bytes(...) bytes,
 *   256-byte aligned; its contents on entry are irrelevant.
 * Range and accuracy.  PATH_F32 accepts any finite inputs with beta >= 0 and
 *   computes in fp32 throughout.  PATH_BF16 feeds the matrix cores half
 *   precision (fp16) operands, so it states its range:
 *   - v: any finite bf16 value.  Each 64-token block of V is scaled by a power
 *     of two before its fp16 conversion (exact) and o is scaled back, so o is
 *     accurate to 2e-2 + 2^-8 * max_j |v_j| (the head's largest value) absolute.
 *   - k, q: |k_j|_2 <= 2^15 and |scale| * |q_i|_2 <= 2^14 for every token, so
 *     every fp16 operand (adjusted keys and queries, transported queries) is
 *     finite.  lse is then accurate to 1e-3 + 2^-18 * max_j |s_ij| and o to
 *     the bound above.
 *   - w, beta: |w_s|_2 <= 1 + 2^-7 (unit vectors stored in bf16) and
 *     0 <= beta_s <= 2 (the range 2 sigmoid(.) gives), so that no transition
 *     expands a vector by more than rounding.
 *   Outside these ranges the results are undefined (an fp16 operand may
 *   overflow and turn o or lse into inf or NaN).  path_attn_bwd keeps fp32
 *   range throughout (bf16 operands have it) and has no such limit.
 */
int path_attn_fwd(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale,
                  int precision, const void* q, const void* k, const void* v, const void* w,
                  const float* beta, const float* log_forget, void* o, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two stages of path_attn_fwd, for callers that time or overlap them:
 * path_fwd_stage_prepare writes the per-block UT data into `workspace`;
 * path_fwd_stage_scan runs the right-to-left scan from it.  Called in that
 * order on one stream with identical arguments they produce exactly what
 * path_attn_fwd produces.  The workspace layout is internal.
 */
int path_fwd_stage_prepare(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale,
                           int precision, const void* q, const void* k, const void* v,
                           const void* w, const float* beta, const float* log_forget,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);
int path_fwd_stage_scan(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale,
                        int precision, const void* q, const void* k, const void* v, const void* w,
                        const float* beta, const float* log_forget, void* o, float* lse,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes path_attn_bwd needs for these sizes (0 on invalid sizes). */
size_t path_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d, int dtype,
                                int with_forget);

/*
 * path_attn_bwd - gradients of the PaTH forward [PaTH summary §2 "Mecanismo
 * Central", §2 "Extensões: PaTH-FoX", in the blockwise form of §3
 * "Representação de Transformação UT" and "Algoritmo Estilo FlashAttention";
 * the pages describe no backward pass, so this is the exact derivative of
 * path_attn_fwd's definition]: with dO the gradient reaching o (lse receives
 * none), writes the gradients of sum(dO * o) with respect to every input.
 * Inputs: q, k, v, w, beta, log_forget (or NULL), scale as given to
 *   path_attn_fwd; o [B,H,L,d] (dtype) and lse [B,H,L] fp32 as it returned
 *   them (used to rebuild the softmax: p = exp(s - lse), D_i = dO_i . o_i);
 *   dout = dO [B,H,L,d] (dtype).
 * Outputs (caller-allocated): dq, dk, dv, dw [B,H,L,d] in dtype (bf16 rounded
 *   to nearest even); dbeta [B,H,L] fp32; dlog_forget [B,H,L] fp32, required
 *   when log_forget is given and ignored otherwise.
 * Alignment: with PATH_BF16, q, k, v, w, o, dout, dq, dk, dv and dw must be
 *   16-byte aligned; PATH_ERR_UNSUPPORTED otherwise, before any launch.
 * Arithmetic: an fp32 re-run of the prepare stage, then the cross-block and
 *   in-block gradient kernels, all accumulating in fp32.  With PATH_F32 every
 *   product is fp32.  With PATH_BF16 the block prepare and the cross-block
 *   products take each fp32 operand as bf16 hi + lo (16 significant bits,
 *   fp32's exponent range), well below the bf16 rounding of the outputs.
 *   Some cross-block sums use fp32 atomics, so results may differ in the
 *   last bits between runs.
 * workspace: >= path_bwd_workspace_bytes(...) bytes, 256-byte aligned.  It
 *   holds, among fp32 intermediates, the transported queries of every
 *   (query block, earlier key block) pair: B*H*Nb*(Nb-1)/2 * d * 64 floats
 *   (plus 8*64*d + 8*d*d bytes per block of split bf16 key-side operands
 *   with PATH_BF16: 64 KB at d = 64, 192 KB at d = 128).
 */
int path_attn_bwd(int64_t B, int64_t H, int64_t L, int64_t d, int dtype, float scale, const void* q,
                  const void* k, const void* v, const void* w, const float* beta, const float* log_forget,
                  const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dw,
                  float* dbeta, float* dlog_forget, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* Workspace bytes path_decode_step needs (0 on invalid sizes). */
size_t path_decode_workspace_bytes(int64_t B, int64_t H, int64_t d, int64_t cache_len);

/*
 * path_decode_step - one generation step with an in-place key cache
 * [PaTH summary §3 "Inferência"]: with H_t = I - beta_t w_t w_t^T,
 *   k_cache[b,h,j] <- H_t k_cache[b,h,j]   for every j < cache_len (in place;
 *                                          stored in dtype, bf16 rounded to nearest even),
 *   s_j = scale * q_t . k_j (j < cache_len, from the fp32 updated key before rounding),
 *   s_t = scale * q_t . k_t (the new key enters untransformed),
 *   o   = softmax over the cache_len + 1 keys applied to [v_cache[:cache_len], v_t],
 *   lse = log of the softmax denominator,
 *   then k_t, v_t are written to slot cache_len of the caches.
 * Inputs: q_t, k_t, v_t, w_t [B,H,d] (dtype); beta_t [B,H] fp32.
 * Caches: k_cache, v_cache [B,H,capacity,d] (dtype); slots >= cache_len + 1
 *   are not touched.  Requires 0 <= cache_len < capacity (else PATH_ERR_CAPACITY).
 * Outputs: o [B,H,d] (dtype), lse [B,H] fp32.
 * workspace: >= path_decode_workspace_bytes(...) bytes, 256-byte aligned.
 * After PATH_ERR_HIP the key cache contents are undefined (no undo exists for
 * an in-place update).
 */
int path_decode_step(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                     const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                     void* k_cache, void* v_cache, int64_t cache_len, int64_t capacity, void* o,
                     float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * path_decode_step_noalloc - path_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same step, bit for bit, with its scratch (a
 * 512-byte store slot and the per-chunk partials, path_decode_workspace_bytes
 * of them) in a static device array of path_decode_noalloc_max_bytes() = 8 MiB
 * that the library holds on each GPU it runs on until the process ends.
 * Arguments, layouts, outputs and errors are those of path_decode_step without
 * the workspace; PATH_ERR_SCRATCH (nothing enqueued) when
 * path_decode_workspace_bytes(B, H, d, cache_len) exceeds 8 MiB, i.e. when
 * B*H*ceil(cache_len/1024)*(d+2)*4 + 512 bytes, rounded up to 256, is larger.
 * The first call on a GPU resolves the array's device address there (once,
 * under a lock); no call allocates.  All calls on one GPU share the array: calls
 * that overlap in time on one GPU (different streams or threads) race and
 * must not be issued.  Nothing in the array needs to start at zero.
 */
int path_decode_step_noalloc(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                             const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                             void* k_cache, void* v_cache, int64_t cache_len, int64_t capacity, void* o,
                             float* lse, hipStream_t stream);

/* Bytes of the static scratch path_decode_step_noalloc uses on each GPU. */
size_t path_decode_noalloc_max_bytes(void);

/*
 * path_decode_step_fox - one PaTH-FoX generation step [PaTH summary §2
 * "Extensões: PaTH-FoX" with §3 "Inferência"]: path_decode_step with the
 * forget-gate bias.  The gate prefix of key j is c_j = sum_{s<=j} log f_s
 * (natural log); the logit of cached key j gains c_t - c_j, the new key's
 * logit gains nothing, where
 *   c_t = cum_cache[b,h,cache_len-1] + log_f_t[b,h]   (c_t = log_f_t[b,h] when cache_len == 0),
 * formed in fp32.  Everything else is exactly path_decode_step.
 * Inputs: as path_decode_step, plus log_f_t [B,H] fp32 (log of the gate, <= 0
 *   for a forget gate; any finite value is accepted).
 * cum_cache [B,H,capacity] fp32, caller-owned: slots j < cache_len hold c_j on
 *   entry (for a prefilled prompt: path_prepare's cum); the step writes c_t at
 *   slot cache_len and touches no other slot.
 * Workspace: path_decode_workspace_bytes(...), as for path_decode_step.
 * Errors: as path_decode_step; PATH_ERR_NULL also when log_f_t or cum_cache is
 *   NULL.  After PATH_ERR_HIP the key cache and cum_cache[cache_len] are undefined.
 */
int path_decode_step_fox(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                         const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                         const float* log_f_t, void* k_cache, void* v_cache, float* cum_cache,
                         int64_t cache_len, int64_t capacity, void* o, float* lse, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * path_decode_step_paged - path_decode_step over a paged key/value cache
 * with one length per sequence [PaTH summary §3 "Inferência": the in-place
 * update k_j <- H_t k_j keeps the method compatible with FlashDecoding-style
 * caches].  For every sequence b and head h, with len = cache_lens[b]:
 *   keys j < len are updated in place, k_j <- H_t k_j (stored in dtype),
 *   o, lse = single-query softmax attention over those len keys and k_t
 *            (exactly path_decode_step with cache_len = len),
 *   then k_t, v_t are written at logical slot len.
 * Cache layout: k_pages, v_pages [num_pages, H, page_size, d] (dtype); slot j
 *   of sequence b is row j % page_size of page page_table[b * max_pages +
 *   j / page_size], head h.  page_table [B, max_pages] and cache_lens [B] are
 *   int32 in device memory, owned by the caller; pages no sequence maps are
 *   not touched.
 * max_cache_len (host): an upper bound on every cache_lens[b]; it sizes the
 *   launch (keys beyond it are not visited) and must be < max_pages * page_size.
 * The device-side values are not checked on the host: a slot whose page id
 *   is outside [0, num_pages) or whose logical page is >= max_pages is skipped
 *   (never read or written), so a bad table gives wrong results, not an
 *   out-of-bounds access.
 * Each physical page may appear at most once in the whole page table.  The
 *   update k_j <- H_t k_j is per sequence (H_t is that sequence's transition),
 *   so a page shared by two sequences (a shared prompt prefix) would receive
 *   both transitions, and a page mapped twice would be updated twice
 *   concurrently; PaTH's in-place cache cannot share pages.
 * Workspace: path_decode_workspace_bytes(B, H, d, max_cache_len).
 * Errors: as path_decode_step (PATH_ERR_CAPACITY when max_cache_len >=
 *   max_pages * page_size); PATH_ERR_SHAPE for page_size < 1, num_pages < 1,
 *   max_pages < 1 or max_pages * page_size >= 2^31.  Any page_size >= 1 works;
 *   a power of two saves a division per key.
 */
int path_decode_step_paged(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                           const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                           void* k_pages, void* v_pages, int64_t num_pages, int64_t page_size,
                           const int32_t* page_table, int64_t max_pages, const int32_t* cache_lens,
                           int64_t max_cache_len, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * path_decode_step_paged_fox - the gated (PaTH-FoX) step over a paged cache
 * [PaTH summary §2 "Extensões: PaTH-FoX" with §3 "Inferência"]: for every
 * sequence b and head h, exactly path_decode_step_fox on the first
 * cache_lens[b] keys of that sequence, with the pages of
 * path_decode_step_paged.  The gate prefix of key j, c_j, sits in cum_pages
 * [num_pages, H, page_size] fp32 at the key's own slot (same page table, same
 * row within the page); the step reads c_{len-1} (0 when len = 0), adds
 * log_f_t[b,h] in fp32 and writes c_t at logical slot len, next to k_t, v_t.
 * Inputs: as path_decode_step_paged, plus log_f_t [B,H] fp32 and cum_pages.
 * Slots no sequence maps are not touched in any of the three page pools.
 * Each physical page may appear at most once in the whole page table: the
 * in-place update applies one sequence's transition to its keys, so pages
 * cannot be shared between sequences (this holds for path_decode_step_paged
 * too).
 * Errors: as path_decode_step_paged; PATH_ERR_NULL also when log_f_t or
 * cum_pages is NULL.
 */
int path_decode_step_paged_fox(int64_t B, int64_t H, int64_t d, int dtype, float scale, const void* q_t,
                               const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                               const float* log_f_t, void* k_pages, void* v_pages, float* cum_pages,
                               int64_t num_pages, int64_t page_size, const int32_t* page_table, int64_t max_pages,
                               const int32_t* cache_lens, int64_t max_cache_len, void* o, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * path_project - projection prologue [PaTH summary §2 "Mecanismo Central":
 * w_s and beta_s are functions of the input token x_s, beta_s =
 * 2 sigmoid(u^T x_s + b); §6 "Limitações" mentions clipping beta]: for every
 * token s = (b, l) and head h,
 *   w[b,h,l,:] = W_h x_s / max(|W_h x_s|_2, 1e-12)       (bf16, rounded to nearest even)
 *   beta[b,h,l] = min(2 sigmoid(u_h . x_s + bias_h), beta_max)   (fp32; no bound
 *                 when beta_max <= 0 or NaN)
 * computed on the bf16 matrix cores with fp32 accumulation.  The pages give no
 * formula for w_s; a per-head linear map scaled to unit length is the reading
 * taken (the attention workloads use unit-norm w).
 * Inputs (bf16): x [B,L,Dm] tokens; Ww [H,d,Dm] (row e of head h maps x to
 *   component e); u [H,Dm]; bias [H] fp32.  Dm must be a positive multiple of
 *   64 and d is 64 or 128.  x, Ww, u and w must be 16-byte aligned.
 * Outputs (caller-allocated): w [B,H,L,d] bf16, beta [B,H,L] fp32, in the
 *   layouts path_attn_fwd takes.
 * Errors: PATH_ERR_NULL for a null pointer, PATH_ERR_SHAPE for non-positive
 *   or overflowing sizes or Dm not a multiple of 64, PATH_ERR_UNSUPPORTED for
 * *   another d or a misaligned pointer; nothing is launched then.  PATH_ERR_HIP if
 *   the launch fails.  Asynchronous on `stream`; allocates nothing.
 */
int path_project(int64_t B, int64_t L, int64_t Dm, int64_t H, int64_t d, const void* x, const void* Ww,
                 const void* u, const float* bias, float beta_max, void* w, float* beta, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PATH_ATTN_H_ */
