/*
 * spacache.h -- C ABI of libspacache, the SPA-Cache per-layer decoding step on MI355X (gfx950).
 *
 * Method: "SPA-Cache: Singular Proxies for Adaptive Caching in Diffusion Language Models"
 * (arXiv 2602.02544). Citations name the page and section:
 *   [PN]  papernotes.org notes (ICML 2026): "方法详解 / 整体框架" (Algorithm 1, phases 1-3),
 *         "关键设计 2" (singular proxy W_r = Lambda_r V_r^T), "关键设计 3" (rho(l) equation).
 *   [GS]  gist.science technical summary, "Methodology: SPA-Cache", parts 1-3.
 *
 * Conventions shared by every entry point
 *   - Memory. Every pointer except those of spa_budget and spa_workspace_bytes is a DEVICE pointer
 *     owned by the caller; the library never allocates, frees or keeps a pointer after returning.
 *     Every device pointer must be 16-byte aligned (SPA_ERR_ALIGN otherwise).
 *   - Layouts. Row-major everywhere. Weight matrices are [out][in], so y = x W^T.
 *       X (h_in)      B x N x d            dtype
 *       K^c, V^c      B x H_kv x N x hd    dtype (head-major: one head's keys are contiguous)
 *       H^c           B x N x d            dtype (the layer output)
 *       P^c           B x N x r            float32 (the proxy cache)
 *       scores        B x N                float32
 *       idx           B x k                int32, ascending within each sequence
 *   - dtype. SPA_BF16 (bfloat16 storage, fp32 accumulation) or SPA_F32 (fp32 throughout).
 *   - Streams. Calls only enqueue work on `stream` (0 = the null stream): no host synchronisation,
 *     no allocation, so a sequence of calls can be captured in a HIP graph. k is a host integer.
 *   - Errors. Every call validates its arguments before any launch and returns a spa_status;
 *     nothing aborts or throws. SPA_ERR_HIP reports a launch failure; faults inside kernels surface
 *     at the caller's next synchronisation.
 *   - Aliasing. The buffers a call writes (the caches, idx_out, scores_out, p_out, o_out and the
 *     workspace) must not overlap one another nor any buffer the call only reads (h_in, the packed
 *     weights and biases, idx, the p_cache of spa_identify, the scores of spa_topk, q and K^c/V^c of
 *     spa_attend): SPA_ERR_ALIAS otherwise. Read-only buffers may overlap each other.
 *   - Threads. Concurrent calls on different streams with disjoint buffers are safe, except
 *     spa_layer_step_noalloc: its calls share one device scratch per GPU (see there).
 *   - Supported shapes: 1 <= N <= 16384; d % 64 == 0, d <= 8192 (bf16) or 4096 (fp32);
 *     d_ffn % 16 == 0; head_dim in {64, 128};
 *     n_q_heads % n_kv_heads == 0; r % 16 == 0, 16 <= r <= min(d, d_kv) (r = d_kv with W_r = W_v diag(g)
 *     is the full-dimension Value identifier).
 */
#ifndef SPACACHE_H
#define SPACACHE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPA_OK = 0,
  SPA_ERR_INVALID_ARG = -1,  /* null pointer, negative or inconsistent size, k out of range      */
  SPA_ERR_UNSUPPORTED = -2,  /* a shape or dtype outside the supported set above                  */
  SPA_ERR_ALIAS = -3,        /* an output overlaps an input it must not overlap                    */
  SPA_ERR_ALIGN = -4,        /* a device pointer is not 16-byte aligned                            */
  SPA_ERR_WORKSPACE = -5,    /* workspace pointer null or smaller than spa_workspace_bytes()       */
  SPA_ERR_HIP = -6           /* a HIP launch returned an error                                     */
} spa_status;

typedef enum { SPA_F32 = 0, SPA_BF16 = 1 } spa_dtype;

/* Which rows the proxy cache P^c takes after a cached step ([PN] 整体框架 Phase 1 compares with
 * "the proxy cached at the previous step"): ALL = every token's new proxy (default), SELECTED =
 * only the recomputed rows, so P^c always matches the inputs of the cached K/V/H rows. */
typedef enum { SPA_PROXY_WRITE_ALL = 0, SPA_PROXY_WRITE_SELECTED = 1 } spa_proxy_policy;

typedef struct {
  int32_t batch;       /* B: independent sequences                                   */
  int32_t n_tokens;    /* N                                                          */
  int32_t d_model;     /* d                                                          */
  int32_t n_q_heads;   /* H_q                                                        */
  int32_t n_kv_heads;  /* H_kv (grouped-query attention when < H_q)                  */
  int32_t head_dim;    /* hd                                                         */
  int32_t d_ffn;       /* F: SwiGLU hidden size                                      */
  int32_t rank;        /* r: rows of the singular proxy W_r                          */
  int32_t dtype;       /* spa_dtype                                                  */
  float norm_eps;      /* RMSNorm epsilon                                            */
  float rope_theta;    /* > 1: rotary embedding of q and k at each token's index in its sequence,
                          dims (2j, 2j + 1) of a head rotated by pos * rope_theta^(-2j / hd), applied
                          before K is cached (LLaDA / Dream attention); 0: none. Not from the pages:
                          an option for fidelity to the real layers.                   */
} spa_shape;

/* Fragment-packed weight layout. The GEMM weights below are passed packed, once per model, by
 * spa_pack_weight: a row-major [rows][cols] matrix (y = x W^T) is cut into 1 KB blocks, one per
 * (32-row block rb, K block kb) with 16 bf16 or 8 fp32 elements of K per block, stored at byte offset
 * (rb * cols_pad / kbe + kb) * 1024 (kbe = 16 for bf16, 8 for fp32). Inside a block, the 16 bytes at
 * l * 16 (l = 0..63) hold row 32 rb + l % 32 and K elements 16 kb + 8 (l / 32) + j, j = 0..7 (bf16)
 * or 8 kb + 2 j + l / 32, j = 0..3 (fp32): the lane order of a 32x32 MFMA B operand, so a GEMM wave
 * loads its weight fragments with one coalesced 16-byte load per lane and streams every panel
 * sequentially. Rows are zero-padded to a multiple of 32, columns to a multiple of 64.
 * SPA_PACK_GATE_UP takes the [W_gate; W_up] matrix (2F rows) and emits 2 F_pad rows
 * (F_pad = ceil(F / 64) * 64) where 32-row block rb holds the gate rows of hidden units
 * 16 rb .. 16 rb + 15 followed by the up rows of the same units. */
typedef enum { SPA_PACK_PLAIN = 0, SPA_PACK_GATE_UP = 1 } spa_pack_kind;

/* Bytes of a packed [rows][cols] matrix of `dtype`. Host only. cols % 16 == 0 (and F % 16 == 0 for
 * SPA_PACK_GATE_UP, where rows = 2F). */
int spa_packed_weight_bytes(int32_t dtype, int32_t rows, int32_t cols, int32_t kind, size_t *bytes_out);

/* Pack a row-major device matrix src (rows x cols of dtype) into the fragment-packed layout (device,
 * spa_packed_weight_bytes bytes, must not overlap src). col_scale (nullable; device, cols entries of
 * dtype) packs W diag(col_scale) instead, the product taken in fp32 and rounded once to dtype: this is
 * how an RMSNorm gain is folded into the weight that consumes the normalised rows. Stream-ordered;
 * offline, once per model. */
int spa_pack_weight(int32_t dtype, int32_t rows, int32_t cols, int32_t kind, const void *src,
                    const void *col_scale, void *dst, hipStream_t stream);

/* Layer weights (device, read-only). The block is pre-norm: RMSNorm(g_attn) -> QKV -> attention ->
 * W_o -> residual -> RMSNorm(g_ffn) -> SwiGLU -> W_down -> residual. Matrices are fragment-packed.
 * The two RMSNorm gains are folded into the matrices that follow them (spa_pack_weight's col_scale):
 * since RMSNorm(x) W^T = (x W'^T) / rms(x) with W' = W diag(g), the library applies only the 1 / rms
 * row scale, computed on the fly inside those GEMMs. */
typedef struct {
  const void *w_r;        /* packed r x d: Lambda_r V_r^T of W_v diag(g_attn) ([PN] 关键设计 2)   */
  const void *w_qkv;      /* packed (d_q + 2 d_kv) x d: rows [W_q; W_k; W_v], col_scale g_attn     */
  const void *w_o;        /* packed d x d_q                                                       */
  const void *w_gate_up;  /* packed SPA_PACK_GATE_UP of [W_gate; W_up] (2F x d), col_scale g_ffn  */
  const void *w_down;     /* packed d x F                                                         */
  const void *b_qkv;      /* NULL, or d_q + 2 d_kv biases [b_q; b_k; b_v] (plain, storage dtype),
                             added to q, k, v after the normalisation, before the rotary embedding
                             (Dream's attention has them)                                          */
} spa_layer_weights;

/* Per-layer caches (device, read-write), owned by the caller across steps. */
typedef struct {
  void *k_cache;   /* B x H_kv x N x hd */
  void *v_cache;   /* B x H_kv x N x hd */
  void *h_cache;   /* B x N x d: the layer output; rows outside the update set keep their values */
  float *p_cache;  /* B x N x r */
} spa_layer_cache;

/* Per-layer row budget ([PN] 关键设计 3, the piecewise-Gaussian rho(l)). Host only.
 * rho(l) = rho_p exp(ln(rho_1/rho_p) ((l - l_p)/(l_p - 1))^2) for l <= l_p, and the mirrored branch
 * rho_p exp(ln(rho_L/rho_p) ((l - l_p)/(L - l_p))^2) for l > l_p; layers are 1-based and the peak
 * and endpoints are exact. k_l = clamp(floor(N rho(l) + 1e-9), 1, N).
 * rho_out (double[n_layers]) and k_out (int32[n_layers]) are host arrays; either may be NULL.
 * SPA_ERR_INVALID_ARG unless n_layers >= 1, 1 <= l_peak <= n_layers, n_tokens >= 1 and every
 * budget lies in (0, 1]. */
int spa_budget(int32_t n_layers, int32_t l_peak, double rho_peak, double rho_first,
               double rho_last, int32_t n_tokens, double *rho_out, int32_t *k_out);

/* Device workspace needed by calls on `shape` that update at most k_max rows per sequence
 * (spa_layer_full needs k_max >= N). Host only; writes *bytes_out. */
int spa_workspace_bytes(const spa_shape *shape, int32_t k_max, size_t *bytes_out);

/* Warm-up step t = 0 and the vanilla full recompute ([PN] 整体框架 with every token updated):
 * fills K^c, V^c, H^c from the full block over all N tokens and sets P^c = X W_r^T.
 * h_in must not overlap h_cache (SPA_ERR_ALIAS). */
int spa_layer_full(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                   const void *h_in, void *ws, size_t ws_bytes, hipStream_t stream);

/* One cached SPA-Cache layer step t >= 1 ([PN] 整体框架 phases 1-3; [GS] parts 1 and 3):
 *  1. P = X W_r^T; s_i = <p_i, p^c_i> / (max(|p_i|,1e-8) max(|p^c_i|,1e-8)); I = the k least similar
 *     tokens of each sequence (ties to the lower index, NaN first), ascending; P^c updated by policy.
 *  2. Q/K/V for rows in I; K, V scattered into K^c, V^c; the k queries attend to all N cached keys.
 *  3. W_o + residual, RMSNorm, SwiGLU FFN + residual on those rows, scattered into H^c[I].
 * k in [0, N]. idx_out (B x k int32) receives I; scores_out (B x N float32) may be NULL.
 * h_in must not overlap h_cache. */
int spa_layer_step(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                   const void *h_in, int32_t k, int32_t policy, int32_t *idx_out, float *scores_out,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/* Timing probe for profiling tools (not needed for results). The caller creates `capacity` HIP
 * events; spa_layer_step_timed records marks[0] on the stream before its first kernel and
 * marks[i + 1] right after its i-th kernel, stopping when capacity is reached, and sets `count` to
 * the number recorded. names (optional, capacity - 1 entries) receives a static name per kernel:
 * proxy_gemm, cosine_topk (the cosine of every token and, in the workgroup that completes a
 * sequence, its Top-k; up to 8192 rows B N, beyond that proxy_cosine then topk; proxy_cosine alone
 * when k = 0), [proxy_copy_selected], qkv_gemm_scatter,
 * attention, wo_gemm_residual, gate_up_gemm_swiglu, down_gemm_scatter (a GEMM that splits K adds a
 * second kernel, its reduce, under the same name; so does a gate/up product split into whole rounds of
 * 256 x 256 tiles and a remainder of columns). */
typedef struct {
  hipEvent_t *marks;
  int32_t capacity;
  int32_t count;
  const char **names;
} spa_timing;

/* spa_layer_step plus the timing probe above; timing may be NULL. Results are identical. */
int spa_layer_step_timed(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                         const void *h_in, int32_t k, int32_t policy, int32_t *idx_out, float *scores_out,
                         void *ws, size_t ws_bytes, hipStream_t stream, spa_timing *timing);

/* spa_layer_step without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The library's own
 * scratch serves as the workspace: a static device array of 64 MiB on each GPU, held until the
 * process ends, laid out exactly for the call; the call allocates and frees nothing. Arguments,
 * results and errors are those of spa_layer_step; SPA_ERR_WORKSPACE when the call would need more than
 * 64 MiB of scratch (the llada-shaped layer of N = 1024, d = 4096, F = 12288 needs about 33 MiB at
 * k = 256). The stream must belong to the current device. Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents: calls that overlap in time on one GPU (other streams,
 * other host threads) race and must be serialised by the caller. */
int spa_layer_step_noalloc(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                           const void *h_in, int32_t k, int32_t policy, int32_t *idx_out, float *scores_out,
                           hipStream_t stream);

/* Phase 1 scores only ([PN] 整体框架 Phase 1; [GS] part 1), with w_r fragment-packed (spa_pack_weight of
 * the r x d matrix): p_out = X W_r^T (B x N x r float32) and,
 * when p_cache is not NULL, scores_out = cosine(p, p^c) (B x N). Never writes p_cache.
 * p_out may be NULL when only scores are wanted; scores_out may be NULL when p_cache is. */
int spa_identify(const spa_shape *shape, const void *h_in, const void *w_r, const float *p_cache,
                 float *p_out, float *scores_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* Top-k least similar ([PN] 整体框架 Phase 1): for each of `batch` rows of `scores` (n floats),
 * the k indices of the smallest scores under the order (value, index), NaN lowest, -0 = +0,
 * written ascending to idx_out (batch x k). 1 <= n <= 16384, 0 <= k <= n. No workspace. */
int spa_topk(int32_t batch, int32_t n, const float *scores, int32_t k, int32_t *idx_out,
             hipStream_t stream);

/* Phases 2-3 for a given update set idx (B x k int32, entries in [0, N); ascending order is not
 * required; a repeated index writes identical rows twice). Rows outside idx keep their cached
 * K/V/H values; P^c is not touched. Entries outside [0, N) are skipped by every write. */
int spa_sparse_update(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                      const void *h_in, const int32_t *idx, int32_t k, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/* Phase 2b alone ([PN] 整体框架 Phase 2): q (M x H_q x hd, dtype, M = B * m_per_seq rows, the first
 * m_per_seq belonging to sequence 0, ...) attends to every key of its sequence's K^c/V^c with
 * scale 1/sqrt(hd), no mask; o_out (M x H_q x hd, dtype). */
int spa_attend(const spa_shape *shape, const void *q, int32_t m_per_seq, const void *k_cache,
               const void *v_cache, void *o_out, hipStream_t stream);

/* Human-readable name of a spa_status value. */
const char *spa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPACACHE_H */
