// Internal launchers of the SPA-Cache kernels. Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spa {

enum DTypeId { kF32 = 0, kBF16 = 1 };

// Epilogue of a GEMM C = A W^T (A: M x K, W: rows x K, both K-contiguous).
enum EpiKind {
  kEpiPartial = 0,       // fp32 partial sums [split][M][N] (split-K, and the proxy projection)
  kEpiQKV = 1,           // columns [0,dq) -> Q (M x dq); [dq,dq+dkv) -> K^c[row]; rest -> V^c[row]
  kEpiResid = 2,         // out[m][n] = src[row(m)][n] + acc     (W_o with the residual of x)
  kEpiSwiGLU = 3,        // W = [gate; up] (2F rows): z[m][j] = silu(gate) * up
  kEpiResidScatter = 4,  // out[row(m)][n] = src[m][n] + acc     (W_down + residual into H^c)
};

// Row m of a GEMM over update sets: sequence b = m / k_per_seq, token i = idx ? idx[m] : m % k_per_seq,
// and the token's row in a B x N x ... tensor is b * n_tok + i. Out-of-range i is skipped on writes.
struct EpiArgs {
  void *out;
  void *out2;
  void *out3;
  const void *src;
  const int32_t *idx;
  int k_per_seq;
  int n_tok;
  int dq, dkv, hkv, hd;
  int ld_src;
  int ldo;
  int f;
  int ldz;  // kEpiSwiGLU: row stride of Z in elements (0: f)
  // kEpiQKV only: `bias` (d_q + 2 d_kv values of T, nullptr for none) is added after the RMSNorm row
  // scale; then, when rope_log2_theta > 0, q and k get the rotary embedding at the row's token index
  // (dims 2j, 2j + 1 of a head rotate by pos * theta^(-2j / hd); rope_log2_theta = log2 theta).
  const void *bias;
  float rope_log2_theta;
  // RMSNorm fused into the A operand (kinds kEpiQKV and kEpiSwiGLU): A rows are the raw hidden rows
  // (gathered through idx when it is set), the RMSNorm gain is folded into the packed weight, and
  // each output row is scaled by 1 / sqrt(mean(a^2) + norm_eps) over the norm_d columns of A. The
  // statistics come from the producers of A: row_rinv[source row] holds the scale itself (QKV: from
  // the proxy GEMM over the same rows), or ss_in[m * ss_n + j], j < ss_n, holds partial sums of
  // squares of row m (gate/up: from the W_o epilogue, one per 32 output columns).
  int norm_d;
  float norm_eps;
  const float *row_rinv;
  const float *ss_in;
  int ss_n;
  // Producer side: kEpiPartial with ss_out set also writes, for each A row, the sum of squares of its
  // elements in the split's K range to ss_out[split * M + m]; kEpiResid with ss_out set writes the sum
  // of squares of each row's stored outputs per 32 columns to ss_out[m * (N / 32) + n / 32].
  float *ss_out;
  // Register-path kernel only: workgroup 0 sets clear[0 .. clear_n) to 0 (counters that the next
  // kernel on the stream expects at 0).
  uint32_t *clear;
  int clear_n;
};

struct GemmPlan {
  int cfg;       // tile configuration id
  int bm, bn;
  int tiles_m, tiles_n;
  int splits;    // > 1: fp32 partials + a reduce kernel that applies the epilogue
  int k_split;   // K elements per split (multiple of the K slab)
  // kEpiSwiGLU on the 256 x 256 kernel: columns [0, n_main) run as whole rounds of its tiles, the
  // remaining columns as a second launch on the best smaller tile (0: one launch over all columns)
  int n_main;
};

// Tile configurations of the large-M kernel: bf16 only, 256 x 256 (or 192 x 256) tiles, never split,
// no kEpiPartial.
constexpr int kBigTileCfg = 6;
constexpr int kBig192Cfg = 17;
// Tile configurations of the LDS-DMA small-M kernel (bf16, no kEpiPartial): kDmaCfg0 + i for tiles
// kDmaTiles[i] (BM x BN).
constexpr int kDmaCfg0 = 7;
// The proxy projection's own kernel (bf16, kEpiPartial, N = 128): 32-row x 128-column tiles, split-K.
constexpr int kProxyCfg = 16;
constexpr int kDmaTileCount = 4;
constexpr int kDmaTiles[kDmaTileCount][2] = {{128, 192}, {128, 128}, {128, 64}, {128, 96}};

GemmPlan plan_gemm(int dtype, int M, int N, int K, int kind);
// Plan of the columns [p.n_main, N) of a column-split SwiGLU plan (p.n_main > 0), launched after the
// whole rounds of 256 x 256 tiles.
GemmPlan gemm_tail_plan(int dtype, int M, int N, int K, int kind, const GemmPlan &p);
size_t gemm_partial_bytes(const GemmPlan &p, int M, int N);

// A: M x K row-major (lda elements per row). W: fragment-packed (see below), wkb = packed blocks per
// 32-row block. K must be a multiple of the slab width (64 bf16 / 32 fp32 elements).
// part: workspace for fp32 partials (gemm_partial_bytes), required when plan.splits > 1 or kind is
// kEpiPartial (then the partials are the result).
hipError_t launch_gemm(int dtype, int kind, const GemmPlan &plan, const void *A, int lda, const void *W,
                       int wkb, int M, int N, int K, float *part, const EpiArgs &ea, hipStream_t s);

// Split-K plans keep splits * tiles <= kMaxSplitWGs, so their partials never exceed
// kMaxSplitWGs * 128 * 192 fp32 values, nor 16 * M * N.
constexpr int kMaxSplitWGs = 512;
inline size_t gemm_partial_bound(int M, int N) {
  const size_t a = (size_t)16 * M * N * 4, b = (size_t)kMaxSplitWGs * 128 * 192 * 4;
  return a < b ? a : b;
}

// Fragment-packed weight layout: a row-major R x C matrix becomes 1 KB blocks, one per (32-row block
// rb, K block kb) with 16 bf16 or 8 fp32 K elements per block, at byte offset (rb * wkb + kb) * 1024,
// wkb = C_pad / (16 or 8). Inside a block, lane l = 0..63 of a wave owns the 16 bytes at l * 16: the
// B operand of a 32x32 MFMA for output column l % 32 -- bf16: k = 16 kb + 8 (l / 32) + j, j = 0..7;
// fp32: k = 8 kb + 2 j + l / 32, j = 0..3 (four 32x32x2 k-steps). Rows are padded to a multiple of
// 32 and columns to a multiple of 64 with zeros. kind kPackGateUp reads a [gate; up] source of 2F
// rows and packs 2 F_pad rows (F_pad = ceil(F / 64) * 64) where 32-row block rb holds the gate rows
// of units 16 rb .. 16 rb + 15 followed by the up rows of the same units.
enum PackKind { kPackPlain = 0, kPackGateUp = 1 };
inline int pad_to(int v, int m) { return (v + m - 1) / m * m; }
inline void packed_dims(int kind, int rows, int cols, int *rows_pad, int *cols_pad) {
  *rows_pad = kind == kPackGateUp ? 2 * pad_to(rows / 2, 64) : pad_to(rows, 32);
  *cols_pad = pad_to(cols, 64);
}
inline int packed_wkb(int dtype, int cols) { return pad_to(cols, 64) / (dtype == kBF16 ? 16 : 8); }
// col_scale (nullable, cols entries of the matrix dtype): pack W diag(col_scale), rounded once.
hipError_t launch_pack_weight(int dtype, int kind, int rows, int cols, const void *src, const void *col_scale,
                              void *dst, hipStream_t s);

// Phase 1 pieces.
// Up to this many hidden rows (B N) the Top-k runs inside the cosine kernel (launch_cosine_topk);
// beyond it the cosine kernel and the Top-k kernel run one after the other.
constexpr int kFusedTopkRows = 8192;
// Keys held per thread by the Top-k of an n-token sequence (fused: inside the cosine kernel).
int topk_keys_per_thread(int n, bool fused);
// Lanes that serve one hidden row in the cosine pass at proxy rank r (16, 32 or 64).
int cosine_lanes_per_row(int r);
// ss_part (splits x rows, nullable): the proxy GEMM's per-split sums of squares of each hidden row;
// with rinv set, rinv[row] = 1 / sqrt(sum / d + eps) is written as well.
hipError_t launch_proxy_cosine(const float *part, int splits, int rows, int r, const float *pc_read,
                               float *pc_write, float *p_out, float *scores, const float *ss_part, int d,
                               float eps, float *rinv, hipStream_t s);
// The same cosine pass fused with the Top-k of each of the batch sequences (n <= 16384 tokens each,
// 1 <= k): idx_out (batch x k) as launch_topk; counters (batch entries) must be 0 at launch and are
// left 0.
hipError_t launch_cosine_topk(const float *part, int splits, int batch, int n, int r, const float *pc_read,
                              float *pc_write, float *p_out, float *scores, const float *ss_part, int d, float eps,
                              float *rinv, int k, int32_t *idx_out, uint32_t *counters, hipStream_t s);
// rinv[row] = 1 / sqrt(mean(x_row^2) + eps) for rows x d.
hipError_t launch_row_rinv(int dtype, const void *x, int rows, int d, float eps, float *rinv, hipStream_t s);
hipError_t launch_topk(const float *scores, int batch, int n, int k, int32_t *idx_out, hipStream_t s);
hipError_t launch_copy_selected(const float *p_src, float *pc, const int32_t *idx, int batch, int n,
                                int k, int r, hipStream_t s);

// Sparse-query attention: q (B*m_per_seq x hq*hd) against K^c/V^c (B x hkv x n_tok x hd).
// The kernel that serves a launch is chosen on the host: kAttnQG1 / kAttnQG2 = workgroups of 32 / 64
// queries of one head with the keys split over their waves; kAttnPacked (bf16) = blocks of 256 rows
// that pack the query heads of a KV group, for launches with many rows per KV head.
enum AttnKind { kAttnQG1 = 0, kAttnQG2 = 1, kAttnPacked = 2 };
struct AttnPlan {
  int kind;
};
AttnPlan plan_attention(int dtype, int batch, int m_per_seq, int n_tok, int hq, int hkv, int hd);
hipError_t launch_attention(int dtype, const AttnPlan &plan, const void *q, const void *kc, const void *vc, void *o,
                            int batch, int m_per_seq, int n_tok, int hq, int hkv, int hd, hipStream_t s);

}  // namespace spa
