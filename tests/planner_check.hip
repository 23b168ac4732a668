// Host-side check of the GEMM planner (built by tests/test_planner.py and run on the CPU; it makes no
// HIP call): over a sweep of shapes, every plan must cover the output with its tiles and K with its
// splits, keep split-K within the partial workspace bound, and pick only kernels valid for the
// shape (the LDS-DMA and 256 x 256 kernels: bf16, no partial-only output; split-K never for the
// SwiGLU or QKV epilogues, whose RMSNorm needs all of K; a column split only for SwiGLU on whole
// rounds of 256 x 256 tiles).
#include <stdio.h>

#include "../adaptive_hidden_state_amd/csrc/gemm.hip"

using namespace spa;

static int failures = 0;
static void fail(const char *what, int dtype, int M, int N, int K, int kind, const GemmPlan &p) {
  if (++failures <= 20)
    printf("FAIL %s: dtype %d M %d N %d K %d kind %d -> cfg %d bm %d bn %d tiles %dx%d splits %d k_split %d\n", what,
           dtype, M, N, K, kind, p.cfg, p.bm, p.bn, p.tiles_m, p.tiles_n, p.splits, p.k_split);
}

int main() {
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
            const bool big = p.cfg == kBigTileCfg, dma = p.cfg >= kDmaCfg0 && p.cfg < kDmaCfg0 + kDmaTileCount;
            int bm = 0, bn = 0;
            if (big) {
              bm = bn = 256;
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
            if (p.n_main != 0) {  // SwiGLU: whole rounds of 256 x 256 tiles over n_main columns, then the rest
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
              fail("LDS-DMA / 256-tile kernel outside bf16 products", dtype, M, N, K, kind, p);
            if (big && p.splits != 1) fail("the 256 x 256 kernel never splits K", dtype, M, N, K, kind, p);
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
