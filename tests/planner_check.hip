// Host-side checks of the kernel planners (built by the host tests with hipcc and run on the CPU; no
// HIP call is made).
//
// With no argument: over a sweep of shapes, every GEMM plan must cover the output with its tiles and K
// with its splits, keep split-K within the partial workspace bound, and pick only kernels valid for
// the shape (the LDS-DMA and large-M kernels: bf16, no partial-only output; split-K never for the
// SwiGLU or QKV epilogues, whose RMSNorm needs all of K; a column split only for SwiGLU on whole
// rounds of large-M tiles, 256 x 256 or 192 x 256).
//
// With "instances": reads lines "tag dtype B N d hq hkv hd F r k mode" from stdin (mode step: the
// cached step with Top-k of k rows; full: the full recompute; identify: spa_identify; sparse:
// spa_sparse_update of k rows; attend: spa_attend of k queries per sequence) and prints
// "tag key key ...": one key per kernel instance the call runs (kernel and tile, split-K or not, one
// or several column tiles, a ragged last row tile or not, and the variants of the identification and
// attention kernels).
#include <stdio.h>
#include <string.h>

#include <string>

#include "../adaptive_hidden_state_amd/csrc/attention.hip"
#include "../adaptive_hidden_state_amd/csrc/gemm.hip"
#include "../adaptive_hidden_state_amd/csrc/identify.hip"
#include "../adaptive_hidden_state_amd/csrc/step_plan.hpp"

using namespace spa;

static int failures = 0;
static void fail(const char *what, int dtype, int M, int N, int K, int kind, const GemmPlan &p) {
  if (++failures <= 20)
    printf("FAIL %s: dtype %d M %d N %d K %d kind %d -> cfg %d bm %d bn %d tiles %dx%d splits %d k_split %d\n", what,
           dtype, M, N, K, kind, p.cfg, p.bm, p.bn, p.tiles_m, p.tiles_n, p.splits, p.k_split);
}

static int sweep() {
  static const int Ms[] = {1,   2,   3,   7,   16,  31,  32,  33,  51,  63,   64,   65,   87,   100,  127,
                           128, 129, 133, 191, 192, 193, 200, 255, 256, 257,  311,  383,  384,  428,  512,
                           513, 700, 1000, 1024, 1030, 2048, 2624, 4096, 5248, 8192, 32768};
  static const int Ns[] = {16, 32, 64, 96, 128, 192, 256, 512, 1376, 2048, 3584, 4096, 4608, 12288, 24576, 37888};
  static const int Ks[] = {64, 128, 256, 512, 704, 1024, 3584, 4096, 12288, 18944};
  long long plans = 0, splits_n = 0;
  for (int dtype : {kBF16, kF32})
    for (int kind = 0; kind < 5; ++kind)
      for (int M : Ms)
        for (int N : Ns)
          for (int K : Ks) {
            const int slab = dtype == kF32 ? 32 : 64;
            if (K % slab != 0) continue;
            const GemmPlan p = plan_gemm(dtype, M, N, K, kind);
            ++plans;
            if (p.n_main != 0) ++splits_n;
            const bool big = p.cfg == kBigTileCfg || p.cfg == kBig192Cfg;
            const bool dma = p.cfg >= kDmaCfg0 && p.cfg < kDmaCfg0 + kDmaTileCount;
            const bool proxy = p.cfg == kProxyCfg;
            int bm = 0, bn = 0;
            if (proxy) {
              bm = 32;
              bn = 128;
              if (dtype != kBF16 || kind != kEpiPartial || N != 128)
                fail("proxy kernel outside the bf16 rank-128 projection", dtype, M, N, K, kind, p);
            } else if (big) {
              bm = p.cfg == kBigTileCfg ? 256 : 192;
              bn = 256;
            } else if (dma) {
              bm = kDmaTiles[p.cfg - kDmaCfg0][0];
              bn = kDmaTiles[p.cfg - kDmaCfg0][1];
            } else if (p.cfg >= 0 && p.cfg < 6) {
              bm = kTiles[p.cfg].bm;
              bn = kTiles[p.cfg].bn;
            } else {
              fail("unknown configuration", dtype, M, N, K, kind, p);
              continue;
            }
            if (p.bm != bm || p.bn != bn) fail("tile size does not match the configuration", dtype, M, N, K, kind, p);
            if (p.n_main != 0) {  // SwiGLU: whole rounds of large-M tiles over n_main columns, then the rest
              if (kind != kEpiSwiGLU || dtype != kBF16 || !big || p.n_main % 256 != 0 || p.n_main <= 0 ||
                  p.n_main >= N || p.tiles_n != p.n_main / 256 ||
                  (long long)p.tiles_m * p.tiles_n > (long long)p.tiles_m * ((N + 255) / 256) / 256 * 256)
                fail("bad column split", dtype, M, N, K, kind, p);
            } else if (p.tiles_m != (M + bm - 1) / bm || p.tiles_n != (N + bn - 1) / bn) {
              fail("tiles do not cover the output", dtype, M, N, K, kind, p);
            }
            if (p.splits < 1 || p.k_split <= 0 || p.k_split % slab != 0)
              fail("bad K split", dtype, M, N, K, kind, p);
            else if ((long long)p.splits * p.k_split < K || (long long)(p.splits - 1) * p.k_split >= K)
              fail("splits do not cover K exactly once", dtype, M, N, K, kind, p);
            if (dtype == kF32 && p.cfg != 5) fail("fp32 takes the 64 x 64 register tile only", dtype, M, N, K, kind, p);
            if ((big || dma) && (dtype != kBF16 || kind == kEpiPartial))
              fail("LDS-DMA / large-M kernel outside bf16 products", dtype, M, N, K, kind, p);
            if (big && p.splits != 1) fail("the large-M kernel never splits K", dtype, M, N, K, kind, p);
            if (p.splits > 1) {
              if (kind == kEpiSwiGLU || kind == kEpiQKV) fail("split-K of a normalised epilogue", dtype, M, N, K, kind, p);
              if ((long long)p.tiles_m * p.tiles_n * p.splits > kMaxSplitWGs)
                fail("split-K past the workgroup bound", dtype, M, N, K, kind, p);
            }
            if ((p.splits > 1 || kind == kEpiPartial) && kind != kEpiPartial &&
                gemm_partial_bytes(p, M, N) > gemm_partial_bound(M, N))
              fail("partials exceed the workspace bound", dtype, M, N, K, kind, p);
          }
  printf("%lld plans checked (%lld with a column split), %d failures\n", plans, splits_n, failures);
  return failures == 0 ? 0 : 1;
}

// ---------------------------------------------------------------------------------------------
// instance keys
// ---------------------------------------------------------------------------------------------
static std::string tile_name(int dtype, const GemmPlan &p) {
  char b[64];
  if (p.cfg == kProxyCfg)
    snprintf(b, sizeof b, "proxy%dx%d", p.bm, p.bn);
  else if (p.cfg == kBigTileCfg || p.cfg == kBig192Cfg)
    snprintf(b, sizeof b, "big%dx256", p.bm);
  else if (p.cfg >= kDmaCfg0 && p.cfg < kDmaCfg0 + kDmaTileCount)
    snprintf(b, sizeof b, "dma%dx%d", p.bm, p.bn);
  else
    snprintf(b, sizeof b, "reg%dx%d%s", p.bm, p.bn, dtype == kF32 ? "f32" : "");
  return b;
}

static std::string plan_key(int dtype, const GemmPlan &p, int M) {
  std::string k = tile_name(dtype, p);
  k += p.splits > 1 ? "/splitk" : "/nosplit";
  k += p.tiles_n > 1 ? "/ncols" : "/1col";
  k += M % p.bm != 0 ? "/ragged" : "/whole";
  return k;
}

static std::string gemm_key(const char *op, int dtype, int M, int N, int K, int kind, const GemmPlan &p) {
  std::string k = std::string(op) + ":" + plan_key(dtype, p, M);
  if (p.n_main > 0) k += "+tail:" + plan_key(dtype, gemm_tail_plan(dtype, M, N, K, kind, p), M);
  return k;
}

static std::string attn_key(const StepShape &s, int m, const AttnPlan &a) {
  static const char *names[] = {"qg1", "qg2", "packed"};
  static const int rows[] = {32, 64, 256};  // rows of a workgroup's block (packed: rows of grp heads)
  const long long r = a.kind == kAttnPacked ? (long long)(s.hq / s.hkv) * m : m;
  char b[128];
  snprintf(b, sizeof b, "attn:%s:%s:hd%d:%s:%s:%s", names[a.kind], s.dtype == kF32 ? "f32" : "bf16", s.hd,
           s.hq != s.hkv ? "gqa" : "mha", r % rows[a.kind] ? "raggedrows" : "wholerows",
           s.N % 32 ? "raggedkeys" : "wholekeys");
  return b;
}

static void print_sparse(const StepShape &s, const StepPlan &P, int k) {
  const int dq = s.hq * s.hd, dkv = s.hkv * s.hd, fp = step_fpad(s);
  printf(" %s", gemm_key("qkv", s.dtype, P.M, dq + 2 * dkv, s.d, kEpiQKV, P.qkv).c_str());
  printf(" %s", attn_key(s, k, P.attn).c_str());
  printf(" %s", gemm_key("wo", s.dtype, P.M, s.d, dq, kEpiResid, P.wo).c_str());
  printf(" %s", gemm_key("gu", s.dtype, P.M, 2 * fp, s.d, kEpiSwiGLU, P.gu).c_str());
  printf(" %s", gemm_key("dn", s.dtype, P.M, s.d, fp, kEpiResidScatter, P.dn).c_str());
}

static int instances() {
  char line[512];
  while (fgets(line, sizeof line, stdin)) {
    char tag[256], dt[16], mode[32];
    StepShape s{};
    int k = 0;
    if (sscanf(line, "%255s %15s %d %d %d %d %d %d %d %d %d %31s", tag, dt, &s.B, &s.N, &s.d, &s.hq, &s.hkv, &s.hd,
               &s.F, &s.r, &k, mode) != 12) {
      if (line[0] != '\n') printf("BAD %s", line);
      continue;
    }
    s.dtype = strcmp(dt, "f32") == 0 ? kF32 : kBF16;
    const bool step = strcmp(mode, "step") == 0, full = strcmp(mode, "full") == 0;
    const bool identify = strcmp(mode, "identify") == 0, sparse = strcmp(mode, "sparse") == 0;
    if (strcmp(mode, "attend") == 0) {
      const AttnPlan a = plan_attention(s.dtype, s.B, k, s.N, s.hq, s.hkv, s.hd);
      printf("%s %s\n", tag, k > 0 ? attn_key(s, k, a).c_str() : "");
      continue;
    }
    if (!step && !full && !identify && !sparse) {
      printf("BAD %s", line);
      continue;
    }
    const int kk = full ? s.N : (identify ? 0 : k);
    const StepPlan P = plan_step(s, kk, step);
    printf("%s", tag);
    if (!sparse) {
      const int rows = s.B * s.N;
      printf(" %s", gemm_key("proxy", s.dtype, rows, s.r, s.d, kEpiPartial, P.proxy).c_str());
      const char *wide = s.r > 256 ? ":wide" : "";
      const int lpr = cosine_lanes_per_row(s.r);
      if (P.identify == kIdFusedTopk)
        printf(" cos+topk:per%d:lpr%d%s", topk_keys_per_thread(s.N, true), lpr, wide);
      else
        printf(" cos:lpr%d%s", lpr, wide);
      if (P.identify == kIdSeparateTopk) printf(" topk:per%d", topk_keys_per_thread(s.N, false));
    } else {
      printf(" rinv");
    }
    if (P.M > 0) print_sparse(s, P, kk);
    printf("\n");
  }
  return 0;
}

int main(int argc, char **argv) {
  if (argc > 1 && strcmp(argv[1], "instances") == 0) return instances();
  return sweep();
}
