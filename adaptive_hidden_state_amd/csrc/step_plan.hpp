// Kernel choices of one SPA-Cache layer step, made on the host before any launch. The launcher runs
// exactly these plans; host-side checks enumerate them to tell which kernel instances a shape reaches.
#pragma once

#include "launch.hpp"

namespace spa {

struct StepShape {
  int dtype;
  int B, N, d, hq, hkv, hd, F, r;
};

// How phase 1 ends: scores only (spa_identify, the full recompute), the Top-k inside the cosine kernel,
// or the cosine kernel followed by the Top-k kernel (more than kFusedTopkRows hidden rows).
enum IdentifyKind { kIdScores = 0, kIdFusedTopk = 1, kIdSeparateTopk = 2 };

struct StepPlan {
  GemmPlan proxy;  // P = X W_r^T over the B N hidden rows (fp32 split-K partials)
  int identify;    // IdentifyKind
  int M;           // rows of the k-row products: B k (0: phase 1 only)
  GemmPlan qkv, wo, gu, dn;
  AttnPlan attn;
};

inline int step_fpad(const StepShape &s) { return pad_to(s.F, 64); }

// k_per_seq rows per sequence are updated (N for the full recompute, 0 for phase 1 alone); topk:
// phase 1 selects them (the cached step).
inline StepPlan plan_step(const StepShape &s, int k_per_seq, bool topk) {
  StepPlan p{};
  const int rows = s.B * s.N;
  const int dq = s.hq * s.hd, dkv = s.hkv * s.hd, fp = step_fpad(s);
  p.proxy = plan_gemm(s.dtype, rows, s.r, s.d, kEpiPartial);
  p.identify = !topk || k_per_seq <= 0 ? kIdScores : (rows <= kFusedTopkRows ? kIdFusedTopk : kIdSeparateTopk);
  p.M = s.B * k_per_seq;
  if (p.M > 0) {
    p.qkv = plan_gemm(s.dtype, p.M, dq + 2 * dkv, s.d, kEpiQKV);
    p.attn = plan_attention(s.dtype, s.B, k_per_seq, s.N, s.hq, s.hkv, s.hd);
    p.wo = plan_gemm(s.dtype, p.M, s.d, dq, kEpiResid);
    p.gu = plan_gemm(s.dtype, p.M, 2 * fp, s.d, kEpiSwiGLU);
    p.dn = plan_gemm(s.dtype, p.M, s.d, fp, kEpiResidScatter);
  }
  return p;
}

}  // namespace spa
