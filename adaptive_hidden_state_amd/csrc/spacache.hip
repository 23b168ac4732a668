// C ABI of libspacache: argument validation, workspace layout and the launch sequence of the
// SPA-Cache layer step ([PN] 整体框架, Algorithm 1's three phases). Every check runs on the host
// before the first launch, so invalid calls fail without touching the GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "spacache.h"
#include "step_plan.hpp"

using namespace spa;

namespace {

struct Dims {
  int B, N, d, hq, hkv, hd, F, Fp, r, dq, dkv, e, dtype;
  float eps;
  float rope_log2;  // log2(rope_theta), or 0 without rotary embedding
};

int check_shape(const spa_shape *s, Dims *o) {
  if (s == nullptr) return SPA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->n_tokens < 1 || s->d_model < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 ||
      s->head_dim < 1 || s->d_ffn < 1 || s->rank < 1)
    return SPA_ERR_INVALID_ARG;
  if (!(s->norm_eps >= 0.0f) || !isfinite(s->norm_eps)) return SPA_ERR_INVALID_ARG;
  if (!(s->rope_theta >= 0.0f) || !isfinite(s->rope_theta)) return SPA_ERR_INVALID_ARG;
  if (s->rope_theta > 0.0f && !(s->rope_theta > 1.0f)) return SPA_ERR_INVALID_ARG;
  if (s->dtype != SPA_F32 && s->dtype != SPA_BF16) return SPA_ERR_UNSUPPORTED;
  if (s->n_tokens > 16384) return SPA_ERR_UNSUPPORTED;
  if (s->d_model % 64 != 0 || s->d_ffn % 16 != 0) return SPA_ERR_UNSUPPORTED;
  if (s->d_model > (s->dtype == SPA_BF16 ? 8192 : 4096)) return SPA_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return SPA_ERR_UNSUPPORTED;
  if (s->n_q_heads % s->n_kv_heads != 0) return SPA_ERR_UNSUPPORTED;
  const long long dkv = (long long)s->n_kv_heads * s->head_dim;
  const long long dq = (long long)s->n_q_heads * s->head_dim;
  if (s->rank % 16 != 0 || s->rank > s->d_model || s->rank > dkv) return SPA_ERR_UNSUPPORTED;
  // every index computed in 32 bits stays below 2^31
  const long long rows = (long long)s->batch * s->n_tokens;
  long long widest = 2LL * s->d_ffn;
  if (dq + 2 * dkv > widest) widest = dq + 2 * dkv;
  if (s->d_model > widest) widest = s->d_model;
  if (rows * widest >= (1LL << 31) || dq > (1 << 20) || dkv > (1 << 20)) return SPA_ERR_UNSUPPORTED;
  o->B = s->batch;
  o->N = s->n_tokens;
  o->d = s->d_model;
  o->hq = s->n_q_heads;
  o->hkv = s->n_kv_heads;
  o->hd = s->head_dim;
  o->F = s->d_ffn;
  o->Fp = pad_to(s->d_ffn, 64);
  o->r = s->rank;
  o->dq = (int)dq;
  o->dkv = (int)dkv;
  o->dtype = s->dtype;
  o->e = s->dtype == SPA_BF16 ? 2 : 4;
  o->eps = s->norm_eps;
  o->rope_log2 = s->rope_theta > 0.0f ? log2f(s->rope_theta) : 0.0f;
  return SPA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

StepShape step_shape(const Dims &D) { return StepShape{D.dtype, D.B, D.N, D.d, D.hq, D.hkv, D.hd, D.F, D.r}; }

// Workspace regions. Offsets are multiples of 256 bytes.
struct Layout {
  GemmPlan proxy;
  size_t ppart, pbuf, scores, ssp, rinv, counters, q, o, y, z, ss32, gpart, total;
};

// exact = true: the split-K partials are sized for the plans of exactly k_max rows per sequence (the
// layout of one call); otherwise for any k <= k_max (a workspace shared by calls of different k).
Layout make_layout(const Dims &D, int k_max, bool exact = false) {
  Layout L{};
  const size_t rows = (size_t)D.B * D.N;
  const size_t m = (size_t)D.B * (size_t)k_max;
  L.proxy = plan_step(step_shape(D), 0, false).proxy;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up256(bytes);
    return at;
  };
  L.ppart = take(gemm_partial_bytes(L.proxy, (int)rows, D.r));
  L.pbuf = take(rows * D.r * 4);
  L.scores = take(rows * 4);
  L.ssp = take((size_t)L.proxy.splits * rows * 4);  // per-split sums of squares of the hidden rows
  L.rinv = take(rows * 4);                          // their 1 / rms (attention RMSNorm)
  L.counters = take((size_t)D.B * 4);               // per-sequence counters of the fused Top-k
  L.q = take(m * D.dq * D.e);
  L.o = take(m * D.dq * D.e);
  L.y = take(m * D.d * D.e);
  L.z = take(m * D.Fp * D.e);
  L.ss32 = take(m * (D.d / 32) * 4);  // sums of squares of y per 32 columns (FFN RMSNorm)
  // Split-K partials of the four k-row GEMMs: gemm_partial_bound(M, N) covers every plan with
  // M <= B * k_max rows.
  size_t gp = 0;
  if (m > 0 && exact) {
    const StepPlan P = plan_step(step_shape(D), k_max, false);
    const GemmPlan *plans[4] = {&P.qkv, &P.wo, &P.gu, &P.dn};
    const int widths[4] = {D.dq + 2 * D.dkv, D.d, 2 * D.Fp, D.d};
    for (int i = 0; i < 4; ++i) {
      const size_t b = plans[i]->splits > 1 ? gemm_partial_bytes(*plans[i], (int)m, widths[i]) : 0;
      if (b > gp) gp = b;
    }
  } else if (m > 0) {
    const int widths[4] = {D.dq + 2 * D.dkv, D.d, 2 * D.Fp, D.d};
    for (int n : widths) {
      const size_t b = gemm_partial_bound((int)m, n);
      if (b > gp) gp = b;
    }
  }
  L.gpart = take(gp);
  L.total = off;
  return L;
}

char *at(void *ws, size_t off) { return (char *)ws + off; }

// Optional timing probe: an event recorded on the stream after each kernel (see spa_timing).
struct Marks {
  spa_timing *t;
  hipStream_t s;
  hipError_t mark(const char *name, int n_kernels = 1) {
    if (t == nullptr) return hipSuccess;
    for (int i = 0; i < n_kernels; ++i) {
      if (t->count >= t->capacity) return hipSuccess;
      hipError_t e = hipEventRecord(t->marks[t->count], s);
      if (e != hipSuccess) return e;
      if (t->names != nullptr && t->count > 0) t->names[t->count - 1] = name;
      ++t->count;
    }
    return hipSuccess;
  }
};

int hip_status(hipError_t e) { return e == hipSuccess ? SPA_OK : SPA_ERR_HIP; }

#define SPA_TRY(expr)                              \
  do {                                             \
    const hipError_t _e = (expr);                  \
    if (_e != hipSuccess) return SPA_ERR_HIP;      \
  } while (0)

int check_weights(const spa_layer_weights *w) {
  if (w == nullptr) return SPA_ERR_INVALID_ARG;
  const void *p[5] = {w->w_r, w->w_qkv, w->w_o, w->w_gate_up, w->w_down};
  for (const void *x : p) {
    if (x == nullptr) return SPA_ERR_INVALID_ARG;
    if (!aligned16(x)) return SPA_ERR_ALIGN;
  }
  if (w->b_qkv != nullptr && !aligned16(w->b_qkv)) return SPA_ERR_ALIGN;  // optional
  return SPA_OK;
}

int check_cache(const spa_layer_cache *c, const Dims &D, const void *h_in) {
  if (c == nullptr || c->k_cache == nullptr || c->v_cache == nullptr || c->h_cache == nullptr ||
      c->p_cache == nullptr || h_in == nullptr)
    return SPA_ERR_INVALID_ARG;
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache) || !aligned16(c->h_cache) || !aligned16(c->p_cache) ||
      !aligned16(h_in))
    return SPA_ERR_ALIGN;
  const size_t xb = (size_t)D.B * D.N * D.d * D.e;
  const size_t kvb = (size_t)D.B * D.hkv * D.N * D.hd * D.e;
  const size_t pb = (size_t)D.B * D.N * D.r * 4;
  if (overlap(h_in, xb, c->h_cache, xb) || overlap(h_in, xb, c->k_cache, kvb) ||
      overlap(h_in, xb, c->v_cache, kvb) || overlap(h_in, xb, c->p_cache, pb))
    return SPA_ERR_ALIAS;
  if (overlap(c->k_cache, kvb, c->v_cache, kvb) || overlap(c->h_cache, xb, c->k_cache, kvb) ||
      overlap(c->h_cache, xb, c->v_cache, kvb) || overlap(c->p_cache, pb, c->h_cache, xb) ||
      overlap(c->p_cache, pb, c->k_cache, kvb) || overlap(c->p_cache, pb, c->v_cache, kvb))
    return SPA_ERR_ALIAS;
  return SPA_OK;
}

// A device buffer as (pointer, bytes) for the overlap checks; null pointers and empty spans overlap
// nothing.
struct Span {
  const void *p;
  size_t n;
};

bool spans_overlap(const Span &a, const Span &b) {
  return a.p != nullptr && b.p != nullptr && a.n > 0 && b.n > 0 && overlap(a.p, a.n, b.p, b.n);
}

// SPA_ERR_ALIAS unless the buffers a call writes are pairwise disjoint and disjoint from every buffer
// it only reads.
int check_disjoint(const Span *written, int nw, const Span *read, int nr) {
  for (int i = 0; i < nw; ++i) {
    for (int j = i + 1; j < nw; ++j)
      if (spans_overlap(written[i], written[j])) return SPA_ERR_ALIAS;
    for (int j = 0; j < nr; ++j)
      if (spans_overlap(written[i], read[j])) return SPA_ERR_ALIAS;
  }
  return SPA_OK;
}

size_t packed_bytes(const Dims &D, int rows, int cols, int kind) {
  int rp, cp;
  packed_dims(kind, rows, cols, &rp, &cp);
  return (size_t)rp * cp * D.e;
}

// The read-only inputs of a layer call: h_in and the packed weights (and the optional q/k/v biases).
int read_spans(const Dims &D, const spa_layer_weights *w, const void *h_in, Span *out) {
  const int nqkv = D.dq + 2 * D.dkv;
  out[0] = Span{h_in, (size_t)D.B * D.N * D.d * D.e};
  out[1] = Span{w->w_r, packed_bytes(D, D.r, D.d, kPackPlain)};
  out[2] = Span{w->w_qkv, packed_bytes(D, nqkv, D.d, kPackPlain)};
  out[3] = Span{w->w_o, packed_bytes(D, D.d, D.dq, kPackPlain)};
  out[4] = Span{w->w_gate_up, packed_bytes(D, 2 * D.F, D.d, kPackGateUp)};
  out[5] = Span{w->w_down, packed_bytes(D, D.d, D.F, kPackPlain)};
  out[6] = Span{w->b_qkv, (size_t)nqkv * D.e};
  return 7;
}

// The caches a layer call writes: K^c, V^c, H^c and P^c.
int cache_spans(const Dims &D, const spa_layer_cache *c, Span *out) {
  const size_t kvb = (size_t)D.B * D.hkv * D.N * D.hd * D.e;
  out[0] = Span{c->k_cache, kvb};
  out[1] = Span{c->v_cache, kvb};
  out[2] = Span{c->h_cache, (size_t)D.B * D.N * D.d * D.e};
  out[3] = Span{c->p_cache, (size_t)D.B * D.N * D.r * 4};
  return 4;
}

int check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need > ws_bytes) return SPA_ERR_WORKSPACE;
  if (need > 0 && ws == nullptr) return SPA_ERR_WORKSPACE;
  if (ws != nullptr && !aligned16(ws)) return SPA_ERR_ALIGN;
  return SPA_OK;
}

// Phase 1 on device: proxy GEMM (fp32 split-K partials) then reduce + cosine + writes. With plan
// kIdFusedTopk / kIdSeparateTopk (k > 0, pc_read and scores set) the Top-k of every sequence is taken
// too (idx_out, B x k): up to kFusedTopkRows hidden rows inside the cosine kernel, beyond that (where
// the waiting of every wave for its stores before the counter update, repeated over many rounds of
// waves, costs more than the separate launch saves; measured at 32768 rows) by the Top-k kernel after
// it. kIdScores: only the scores.
int run_identify(const Dims &D, const Layout &L, const StepPlan &P, const void *h_in, const void *w_r,
                 const float *pc_read, float *pc_write, float *p_out, float *scores, void *ws, hipStream_t s,
                 Marks &mk, int k = 0, int32_t *idx_out = nullptr) {
  const int rows = D.B * D.N;
  float *part = (float *)at(ws, L.ppart);
  float *ssp = (float *)at(ws, L.ssp), *rinv = (float *)at(ws, L.rinv);
  uint32_t *counters = (uint32_t *)at(ws, L.counters);
  const bool topk = P.identify == kIdFusedTopk;
  EpiArgs ea{};
  ea.ss_out = ssp;  // the projection streams every hidden row: it also sums their squares
  if (topk) {       // and clears the Top-k counters of the cosine kernel that follows
    ea.clear = counters;
    ea.clear_n = D.B;
  }
  SPA_TRY(launch_gemm(D.dtype, kEpiPartial, L.proxy, h_in, D.d, w_r, packed_wkb(D.dtype, D.d), rows, D.r, D.d, part,
                      ea, s));
  SPA_TRY(mk.mark("proxy_gemm"));
  if (topk) {
    SPA_TRY(launch_cosine_topk(part, L.proxy.splits, D.B, D.N, D.r, pc_read, pc_write, p_out, scores, ssp, D.d, D.eps,
                               rinv, k, idx_out, counters, s));
    SPA_TRY(mk.mark("cosine_topk"));
  } else {
    SPA_TRY(launch_proxy_cosine(part, L.proxy.splits, rows, D.r, pc_read, pc_write, p_out, scores, ssp, D.d, D.eps,
                                rinv, s));
    SPA_TRY(mk.mark("proxy_cosine"));
    if (P.identify == kIdSeparateTopk) {
      SPA_TRY(launch_topk(scores, D.B, D.N, k, idx_out, s));
      SPA_TRY(mk.mark("topk"));
    }
  }
  return SPA_OK;
}

// number of kernels launch_gemm enqueues for a plan (the GEMM, plus the split-K reduce)
int gemm_kernels(const GemmPlan &p) { return p.splits > 1 || p.n_main > 0 ? 2 : 1; }

// Phases 2 and 3 for update sets idx (B x k_per_seq; nullptr = every token, k_per_seq = N). The 1 / rms
// of every row of h_in must already be in the workspace (run_identify or launch_row_rinv).
int run_sparse(const Dims &D, const Layout &L, const StepPlan &P, const spa_layer_weights *w,
               const spa_layer_cache *c, const void *h_in, const int32_t *idx, int k_per_seq, void *ws, hipStream_t s,
               Marks &mk) {
  const int M = P.M;
  if (M == 0) return SPA_OK;
  void *q = at(ws, L.q), *o = at(ws, L.o), *y = at(ws, L.y), *z = at(ws, L.z);
  float *gpart = (float *)at(ws, L.gpart), *ss32 = (float *)at(ws, L.ss32);

  // RMSNorm(g_attn) is fused into the QKV GEMM: it reads the raw rows of h_in gathered through idx
  EpiArgs qkv{};
  qkv.out = q;
  qkv.out2 = c->k_cache;
  qkv.out3 = c->v_cache;
  qkv.idx = idx;
  qkv.k_per_seq = k_per_seq;
  qkv.n_tok = D.N;
  qkv.dq = D.dq;
  qkv.dkv = D.dkv;
  qkv.hkv = D.hkv;
  qkv.hd = D.hd;
  qkv.norm_d = D.d;
  qkv.norm_eps = D.eps;
  qkv.bias = w->b_qkv;
  qkv.rope_log2_theta = D.rope_log2;
  qkv.row_rinv = (const float *)at(ws, L.rinv);
  const int nqkv = D.dq + 2 * D.dkv;
  const GemmPlan &p_qkv = P.qkv;
  SPA_TRY(launch_gemm(D.dtype, kEpiQKV, p_qkv, h_in, D.d, w->w_qkv, packed_wkb(D.dtype, D.d), M, nqkv, D.d, gpart,
                      qkv, s));
  SPA_TRY(mk.mark("qkv_gemm_scatter", gemm_kernels(p_qkv)));

  SPA_TRY(launch_attention(D.dtype, P.attn, q, c->k_cache, c->v_cache, o, D.B, k_per_seq, D.N, D.hq, D.hkv, D.hd,
                           s));
  SPA_TRY(mk.mark("attention"));

  EpiArgs wo{};
  wo.out = y;
  wo.src = h_in;
  wo.idx = idx;
  wo.k_per_seq = k_per_seq;
  wo.n_tok = D.N;
  wo.ld_src = D.d;
  wo.ldo = D.d;
  wo.ss_out = ss32;  // statistics of y for the FFN RMSNorm
  const GemmPlan &p_wo = P.wo;
  SPA_TRY(launch_gemm(D.dtype, kEpiResid, p_wo, o, D.dq, w->w_o, packed_wkb(D.dtype, D.dq), M, D.d, D.dq, gpart, wo,
                      s));
  SPA_TRY(mk.mark("wo_gemm_residual", gemm_kernels(p_wo)));

  // RMSNorm(g_ffn) is fused into the gate/up GEMM, which reads y directly
  EpiArgs gu{};
  gu.out = z;
  gu.f = D.Fp;  // Z is M x F_pad; the zero-padded gate/up rows write zeros into the pad columns
  gu.norm_d = D.d;
  gu.norm_eps = D.eps;
  gu.ss_in = ss32;
  gu.ss_n = D.d / 32;
  const GemmPlan &p_gu = P.gu;
  SPA_TRY(launch_gemm(D.dtype, kEpiSwiGLU, p_gu, y, D.d, w->w_gate_up, packed_wkb(D.dtype, D.d), M, 2 * D.Fp, D.d,
                      gpart, gu, s));
  SPA_TRY(mk.mark("gate_up_gemm_swiglu", gemm_kernels(p_gu)));

  EpiArgs dn{};
  dn.out = c->h_cache;
  dn.src = y;
  dn.idx = idx;
  dn.k_per_seq = k_per_seq;
  dn.n_tok = D.N;
  dn.ld_src = D.d;
  dn.ldo = D.d;
  const GemmPlan &p_dn = P.dn;
  SPA_TRY(launch_gemm(D.dtype, kEpiResidScatter, p_dn, z, D.Fp, w->w_down, packed_wkb(D.dtype, D.F), M, D.d, D.Fp,
                      gpart, dn, s));
  SPA_TRY(mk.mark("down_gemm_scatter", gemm_kernels(p_dn)));
  return SPA_OK;
}

// Device scratch of spa_layer_step_noalloc, for callers that cannot allocate: one static array per
// device, held until the process ends. Host code never uses the array's name as an address: each
// device's address is looked up once (hipGetSymbolAddress with that device current) and kept.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the scratch array on the current device.
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SPA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SPA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SPA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPA_OK;
}

}  // namespace

extern "C" {

const char *spa_status_string(int status) {
  switch (status) {
    case SPA_OK: return "SPA_OK";
    case SPA_ERR_INVALID_ARG: return "SPA_ERR_INVALID_ARG: null pointer or size out of range";
    case SPA_ERR_UNSUPPORTED: return "SPA_ERR_UNSUPPORTED: shape or dtype outside the supported set";
    case SPA_ERR_ALIAS: return "SPA_ERR_ALIAS: an output overlaps an input";
    case SPA_ERR_ALIGN: return "SPA_ERR_ALIGN: device pointer not 16-byte aligned";
    case SPA_ERR_WORKSPACE: return "SPA_ERR_WORKSPACE: workspace missing or too small";
    case SPA_ERR_HIP: return "SPA_ERR_HIP: a HIP launch failed";
    default: return "unknown spa_status";
  }
}

int spa_budget(int32_t n_layers, int32_t l_peak, double rho_peak, double rho_first, double rho_last,
               int32_t n_tokens, double *rho_out, int32_t *k_out) {
  if (n_layers < 1 || l_peak < 1 || l_peak > n_layers || n_tokens < 1) return SPA_ERR_INVALID_ARG;
  const double rs[3] = {rho_peak, rho_first, rho_last};
  for (double v : rs)
    if (!(v > 0.0 && v <= 1.0)) return SPA_ERR_INVALID_ARG;
  for (int l = 1; l <= n_layers; ++l) {
    double rho;
    if (l == l_peak) {
      rho = rho_peak;
    } else if (l < l_peak) {
      const double t = (double)(l - l_peak) / (double)(l_peak - 1);
      rho = (l == 1) ? rho_first : rho_peak * exp(log(rho_first / rho_peak) * t * t);
    } else {
      const double t = (double)(l - l_peak) / (double)(n_layers - l_peak);
      rho = (l == n_layers) ? rho_last : rho_peak * exp(log(rho_last / rho_peak) * t * t);
    }
    double kk = floor((double)n_tokens * rho + 1e-9);
    if (kk < 1.0) kk = 1.0;
    if (kk > (double)n_tokens) kk = (double)n_tokens;
    if (rho_out != nullptr) rho_out[l - 1] = rho;
    if (k_out != nullptr) k_out[l - 1] = (int32_t)kk;
  }
  return SPA_OK;
}

int spa_packed_weight_bytes(int32_t dtype, int32_t rows, int32_t cols, int32_t kind, size_t *bytes_out) {
  if (dtype != SPA_F32 && dtype != SPA_BF16) return SPA_ERR_UNSUPPORTED;
  if (kind != SPA_PACK_PLAIN && kind != SPA_PACK_GATE_UP) return SPA_ERR_INVALID_ARG;
  if (rows < 1 || cols < 1 || bytes_out == nullptr) return SPA_ERR_INVALID_ARG;
  if (kind == SPA_PACK_GATE_UP && rows % 2 != 0) return SPA_ERR_INVALID_ARG;
  if (cols % 16 != 0 || (kind == SPA_PACK_GATE_UP && (rows / 2) % 16 != 0)) return SPA_ERR_UNSUPPORTED;
  int rp, cp;
  packed_dims(kind, rows, cols, &rp, &cp);
  *bytes_out = (size_t)rp * cp * (dtype == SPA_BF16 ? 2 : 4);
  return SPA_OK;
}

int spa_pack_weight(int32_t dtype, int32_t rows, int32_t cols, int32_t kind, const void *src,
                    const void *col_scale, void *dst, hipStream_t stream) {
  size_t bytes = 0;
  const int st = spa_packed_weight_bytes(dtype, rows, cols, kind, &bytes);
  if (st != SPA_OK) return st;
  if (src == nullptr || dst == nullptr) return SPA_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(dst) || (col_scale != nullptr && !aligned16(col_scale))) return SPA_ERR_ALIGN;
  const size_t e = dtype == SPA_BF16 ? 2 : 4;
  if (overlap(src, (size_t)rows * cols * e, dst, bytes)) return SPA_ERR_ALIAS;
  if (col_scale != nullptr && overlap(col_scale, (size_t)cols * e, dst, bytes)) return SPA_ERR_ALIAS;
  return hip_status(launch_pack_weight(dtype, kind, rows, cols, src, col_scale, dst, stream));
}

int spa_workspace_bytes(const spa_shape *shape, int32_t k_max, size_t *bytes_out) {
  Dims D;
  const int st = check_shape(shape, &D);
  if (st != SPA_OK) return st;
  if (bytes_out == nullptr || k_max < 0 || k_max > D.N) return SPA_ERR_INVALID_ARG;
  *bytes_out = make_layout(D, k_max).total;
  return SPA_OK;
}

int spa_layer_full(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                   const void *h_in, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int st = check_shape(shape, &D);
  if (st != SPA_OK) return st;
  if ((st = check_weights(w)) != SPA_OK) return st;
  if ((st = check_cache(cache, D, h_in)) != SPA_OK) return st;
  const Layout L = make_layout(D, D.N);
  if ((st = check_ws(ws, ws_bytes, L.total)) != SPA_OK) return st;
  {
    Span wr[5], rd[7];
    const int nw = cache_spans(D, cache, wr);
    wr[nw] = Span{ws, L.total};
    if ((st = check_disjoint(wr, nw + 1, rd, read_spans(D, w, h_in, rd))) != SPA_OK) return st;
  }
  const StepPlan P = plan_step(step_shape(D), D.N, false);
  Marks mk{nullptr, stream};
  if ((st = run_identify(D, L, P, h_in, w->w_r, nullptr, cache->p_cache, nullptr, nullptr, ws, stream, mk)) != SPA_OK)
    return st;
  return run_sparse(D, L, P, w, cache, h_in, nullptr, D.N, ws, stream, mk);
}

}  // extern "C"

namespace {

// The cached step. noalloc: ws is ignored and the static scratch serves as the workspace, laid out
// exactly for this call (SPA_ERR_WORKSPACE past kStaticScratchBytes).
int layer_step(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache, const void *h_in,
               int32_t k, int32_t policy, int32_t *idx_out, float *scores_out, void *ws, size_t ws_bytes,
               hipStream_t stream, spa_timing *timing, bool noalloc) {
  if (timing != nullptr) {
    if (timing->capacity < 0 || (timing->capacity > 0 && timing->marks == nullptr)) return SPA_ERR_INVALID_ARG;
    timing->count = 0;
  }
  Dims D;
  int st = check_shape(shape, &D);
  if (st != SPA_OK) return st;
  if ((st = check_weights(w)) != SPA_OK) return st;
  if ((st = check_cache(cache, D, h_in)) != SPA_OK) return st;
  if (k < 0 || k > D.N) return SPA_ERR_INVALID_ARG;
  if (policy != SPA_PROXY_WRITE_ALL && policy != SPA_PROXY_WRITE_SELECTED) return SPA_ERR_INVALID_ARG;
  if (k > 0 && idx_out == nullptr) return SPA_ERR_INVALID_ARG;
  if ((idx_out && !aligned16(idx_out)) || (scores_out && !aligned16(scores_out))) return SPA_ERR_ALIGN;
  const Layout L = make_layout(D, k, noalloc);
  if (noalloc) {
    if (L.total > kStaticScratchBytes) return SPA_ERR_WORKSPACE;
    if ((st = scratch_address(&ws)) != SPA_OK) return st;
    ws_bytes = kStaticScratchBytes;
  }
  if ((st = check_ws(ws, ws_bytes, L.total)) != SPA_OK) return st;
  {
    Span wr[7], rd[7];
    int nw = cache_spans(D, cache, wr);
    wr[nw++] = Span{idx_out, (size_t)D.B * k * 4};
    wr[nw++] = Span{scores_out, (size_t)D.B * D.N * 4};
    wr[nw++] = Span{ws, L.total};
    if ((st = check_disjoint(wr, nw, rd, read_spans(D, w, h_in, rd))) != SPA_OK) return st;
  }
  float *scores = scores_out ? scores_out : (float *)at(ws, L.scores);
  const bool sel = policy == SPA_PROXY_WRITE_SELECTED;
  float *pbuf = (float *)at(ws, L.pbuf);
  const StepPlan P = plan_step(step_shape(D), k, true);
  Marks mk{timing, stream};
  SPA_TRY(mk.mark("start"));
  if ((st = run_identify(D, L, P, h_in, w->w_r, cache->p_cache, sel ? nullptr : cache->p_cache,
                         sel ? pbuf : nullptr, scores, ws, stream, mk, k, idx_out)) != SPA_OK)
    return st;
  if (k == 0) return SPA_OK;
  if (sel) {
    SPA_TRY(launch_copy_selected(pbuf, cache->p_cache, idx_out, D.B, D.N, k, D.r, stream));
    SPA_TRY(mk.mark("proxy_copy_selected"));
  }
  return run_sparse(D, L, P, w, cache, h_in, idx_out, k, ws, stream, mk);
}

}  // namespace

extern "C" {

int spa_layer_step_timed(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                         const void *h_in, int32_t k, int32_t policy, int32_t *idx_out, float *scores_out, void *ws,
                         size_t ws_bytes, hipStream_t stream, spa_timing *timing) {
  return layer_step(shape, w, cache, h_in, k, policy, idx_out, scores_out, ws, ws_bytes, stream, timing, false);
}

int spa_layer_step_noalloc(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                           const void *h_in, int32_t k, int32_t policy, int32_t *idx_out, float *scores_out,
                           hipStream_t stream) {
  return layer_step(shape, w, cache, h_in, k, policy, idx_out, scores_out, nullptr, 0, stream, nullptr, true);
}

int spa_layer_step(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                   const void *h_in, int32_t k, int32_t policy, int32_t *idx_out, float *scores_out, void *ws,
                   size_t ws_bytes, hipStream_t stream) {
  return spa_layer_step_timed(shape, w, cache, h_in, k, policy, idx_out, scores_out, ws, ws_bytes, stream, nullptr);
}

int spa_identify(const spa_shape *shape, const void *h_in, const void *w_r, const float *p_cache, float *p_out,
                 float *scores_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int st = check_shape(shape, &D);
  if (st != SPA_OK) return st;
  if (h_in == nullptr || w_r == nullptr) return SPA_ERR_INVALID_ARG;
  if (p_out == nullptr && (p_cache == nullptr || scores_out == nullptr)) return SPA_ERR_INVALID_ARG;
  if (scores_out != nullptr && p_cache == nullptr) return SPA_ERR_INVALID_ARG;
  if (!aligned16(h_in) || !aligned16(w_r) || (p_cache && !aligned16(p_cache)) || (p_out && !aligned16(p_out)) ||
      (scores_out && !aligned16(scores_out)))
    return SPA_ERR_ALIGN;
  const size_t pb = (size_t)D.B * D.N * D.r * 4;
  const Layout L = make_layout(D, 0);
  if ((st = check_ws(ws, ws_bytes, L.total)) != SPA_OK) return st;
  {
    const Span wr[3] = {{p_out, pb}, {scores_out, (size_t)D.B * D.N * 4}, {ws, L.total}};
    const Span rd[3] = {{h_in, (size_t)D.B * D.N * D.d * D.e}, {w_r, packed_bytes(D, D.r, D.d, kPackPlain)},
                        {p_cache, pb}};
    if ((st = check_disjoint(wr, 3, rd, 3)) != SPA_OK) return st;
  }
  const StepPlan P = plan_step(step_shape(D), 0, false);
  Marks mk{nullptr, stream};
  return run_identify(D, L, P, h_in, w_r, p_cache, nullptr, p_out, scores_out, ws, stream, mk);
}

int spa_topk(int32_t batch, int32_t n, const float *scores, int32_t k, int32_t *idx_out, hipStream_t stream) {
  if (batch < 1 || n < 1 || k < 0 || k > n) return SPA_ERR_INVALID_ARG;
  if (n > 16384) return SPA_ERR_UNSUPPORTED;
  if (scores == nullptr || (k > 0 && idx_out == nullptr)) return SPA_ERR_INVALID_ARG;
  if (!aligned16(scores) || (idx_out && !aligned16(idx_out))) return SPA_ERR_ALIGN;
  const Span wr[1] = {{idx_out, (size_t)batch * k * 4}}, rd[1] = {{scores, (size_t)batch * n * 4}};
  if (check_disjoint(wr, 1, rd, 1) != SPA_OK) return SPA_ERR_ALIAS;
  return hip_status(launch_topk(scores, batch, n, k, idx_out, stream));
}

int spa_sparse_update(const spa_shape *shape, const spa_layer_weights *w, const spa_layer_cache *cache,
                      const void *h_in, const int32_t *idx, int32_t k, void *ws, size_t ws_bytes,
                      hipStream_t stream) {
  Dims D;
  int st = check_shape(shape, &D);
  if (st != SPA_OK) return st;
  if ((st = check_weights(w)) != SPA_OK) return st;
  if ((st = check_cache(cache, D, h_in)) != SPA_OK) return st;
  if (k < 0 || k > D.N || (k > 0 && idx == nullptr)) return SPA_ERR_INVALID_ARG;
  if (idx && !aligned16(idx)) return SPA_ERR_ALIGN;
  const Layout L = make_layout(D, k);
  if ((st = check_ws(ws, ws_bytes, L.total)) != SPA_OK) return st;
  {
    Span wr[5], rd[8];
    const int nw = cache_spans(D, cache, wr) - 1;  // P^c is not touched
    wr[nw] = Span{ws, L.total};
    int nr = read_spans(D, w, h_in, rd);
    rd[nr++] = Span{idx, (size_t)D.B * k * 4};
    if ((st = check_disjoint(wr, nw + 1, rd, nr)) != SPA_OK) return st;
  }
  const StepPlan P = plan_step(step_shape(D), k, false);
  Marks mk{nullptr, stream};
  if (k > 0) SPA_TRY(launch_row_rinv(D.dtype, h_in, D.B * D.N, D.d, D.eps, (float *)at(ws, L.rinv), stream));
  return run_sparse(D, L, P, w, cache, h_in, idx, k, ws, stream, mk);
}

int spa_attend(const spa_shape *shape, const void *q, int32_t m_per_seq, const void *k_cache, const void *v_cache,
               void *o_out, hipStream_t stream) {
  Dims D;
  int st = check_shape(shape, &D);
  if (st != SPA_OK) return st;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || o_out == nullptr || m_per_seq < 0)
    return SPA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o_out)) return SPA_ERR_ALIGN;
  const size_t ob = (size_t)D.B * m_per_seq * D.dq * D.e;
  const size_t kvb = (size_t)D.B * D.hkv * D.N * D.hd * D.e;
  const Span wr[1] = {{o_out, ob}};
  const Span rd[3] = {{q, ob}, {k_cache, kvb}, {v_cache, kvb}};
  if ((st = check_disjoint(wr, 1, rd, 3)) != SPA_OK) return st;
  const AttnPlan ap = plan_attention(D.dtype, D.B, m_per_seq, D.N, D.hq, D.hkv, D.hd);
  return hip_status(
      launch_attention(D.dtype, ap, q, k_cache, v_cache, o_out, D.B, m_per_seq, D.N, D.hq, D.hkv, D.hd, stream));
}

}  // extern "C"
