// Update identification ([PN] 整体框架 Phase 1; [GS] part 1): cosine similarity of every token's
// singular proxy against the cached proxy, the proxy-cache update, and the Top-k least similar
// tokens per sequence. The proxy projection itself (P = X W_r^T) runs on the MFMA GEMM with fp32
// split-K partials; the kernel below sums those partials in a fixed order, so scores are
// deterministic run to run.
#include "common.hpp"
#include "launch.hpp"

namespace spa {

// ---------------------------------------------------------------------------------------------
// partial-sum reduce + cosine + proxy-cache write; 16, 32 or 64 lanes per token row
// ---------------------------------------------------------------------------------------------
// Reduce the proxy GEMM's split-K partials (in split order: deterministic), take the cosine against
// the cached proxy, write the new proxy. LPR lanes serve one row (64 / LPR rows per wave), streaming it
// in chunks of LPR lanes x 4 columns (16-byte accesses; r % 16 == 0), so any rank works, up to the full
// Value width; ranks up to 128 take 32 lanes per row and up to 64 take 16, so no lane idles on a short
// row. Each lane reads its columns of the cached proxy before it writes the same columns, so the cache
// may be updated in place (pc_write == pc_read). The same lanes also write the row's 1 / rms from the
// per-split sums of squares. Every lane of the wave calls this (the sums cross lanes); `ok` is false for
// a row past the end, whose loads are clamped to the last row and whose stores are skipped.
template <bool COHERENT = false, int LPR = 64>
__device__ __forceinline__ void cosine_row(const float *__restrict__ part, int splits, int rows, int r, int row, bool ok,
                                           const float *pc_read, float *pc_write, float *__restrict__ p_out,
                                           float *scores, const float *__restrict__ ss_part, int d, float eps,
                                           float *__restrict__ rinv) {
  static_assert(LPR == 16 || LPR == 32 || LPR == 64, "lanes per row");
  const int sl = threadIdx.x & (LPR - 1);  // lane within the row's group
  const size_t plane = (size_t)rows * r;
  if (!ok) row = rows - 1;
  const size_t base = (size_t)row * r;
  float dot = 0.f, n1 = 0.f, n2 = 0.f;
  for (int col = sl * 4; col < r; col += 4 * LPR) {
    floatx4 v = *reinterpret_cast<const floatx4 *>(part + base + col);
    // the other splits eight at a time: the loads of a group are all in flight before the first add
    // (one memory round trip per group instead of one per split; measured 1 us off the fused kernel
    // at 8 splits), and the adds keep split order
    for (int sp = 1; sp < splits; sp += 8) {
      floatx4 t[8];
      const int nb = min(8, splits - sp);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < nb) t[j] = *reinterpret_cast<const floatx4 *>(part + (size_t)(sp + j) * plane + base + col);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < nb) v += t[j];
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) n1 += v[x] * v[x];
    if (pc_read != nullptr) {
      const floatx4 w = *reinterpret_cast<const floatx4 *>(pc_read + base + col);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        dot += v[x] * w[x];
        n2 += w[x] * w[x];
      }
    }
    if (ok && p_out != nullptr) *reinterpret_cast<floatx4 *>(p_out + base + col) = v;
    if (ok && pc_write != nullptr) *reinterpret_cast<floatx4 *>(pc_write + base + col) = v;
  }
  // the row's 1 / rms for the RMSNorm fused into the QKV GEMM: lane sl adds splits sl, sl + LPR, ... in
  // that order, then a fixed reduction tree over the row's lanes
  if (rinv != nullptr) {
    float ss = 0.f;
    for (int sp = sl; sp < splits; sp += LPR) ss += ss_part[(size_t)sp * rows + row];
    ss = group_sum<LPR>(ss);
    if (ok && sl == 0) rinv[row] = 1.0f / sqrtf(ss / (float)d + eps);
  }
  if (pc_read != nullptr && scores != nullptr) {
    dot = group_sum<LPR>(dot);
    n1 = group_sum<LPR>(n1);
    n2 = group_sum<LPR>(n2);
    const float c = dot / (fmaxf(sqrtf(n1), 1e-8f) * fmaxf(sqrtf(n2), 1e-8f));
    if (ok && sl == 0) {
      if constexpr (COHERENT)
        __hip_atomic_store(scores + row, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        scores[row] = c;
    }
  }
}

// Lanes per row of the cosine pass for proxy rank r (each lane takes 4 columns per chunk).
int cosine_lanes_per_row(int r) { return r <= 64 ? 16 : (r <= 128 ? 32 : 64); }

template <int LPR>
__global__ __launch_bounds__(256) void proxy_cosine_kernel(const float *__restrict__ part, int splits, int rows,
                                                           int r, const float *pc_read, float *pc_write,
                                                           float *__restrict__ p_out, float *__restrict__ scores,
                                                           const float *__restrict__ ss_part, int d, float eps,
                                                           float *__restrict__ rinv) {
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + (threadIdx.x & 63) / LPR;
  if ((blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW >= rows) return;  // whole waves past the end
  cosine_row<false, LPR>(part, splits, rows, r, row, row < rows, pc_read, pc_write, p_out, scores, ss_part, d, eps,
                         rinv);
}

hipError_t launch_proxy_cosine(const float *part, int splits, int rows, int r, const float *pc_read, float *pc_write,
                               float *p_out, float *scores, const float *ss_part, int d, float eps, float *rinv,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int lpr = cosine_lanes_per_row(r), per_wg = 4 * (64 / lpr);
  const dim3 grid((rows + per_wg - 1) / per_wg), block(256);
  if (lpr == 16)
    hipLaunchKernelGGL(proxy_cosine_kernel<16>, grid, block, 0, s, part, splits, rows, r, pc_read, pc_write, p_out,
                       scores, ss_part, d, eps, rinv);
  else if (lpr == 32)
    hipLaunchKernelGGL(proxy_cosine_kernel<32>, grid, block, 0, s, part, splits, rows, r, pc_read, pc_write, p_out,
                       scores, ss_part, d, eps, rinv);
  else
    hipLaunchKernelGGL(proxy_cosine_kernel<64>, grid, block, 0, s, part, splits, rows, r, pc_read, pc_write, p_out,
                       scores, ss_part, d, eps, rinv);
  return hipGetLastError();
}


// rinv[row] = 1 / sqrt(mean(x_row^2) + eps) over d columns; one wave per row (for the sparse update
// called without the identification pass that otherwise produces these scales).
template <typename T>
__global__ __launch_bounds__(64) void row_rinv_kernel(const T *__restrict__ x, int d, float eps,
                                                      float *__restrict__ rinv) {
  constexpr int VEC = 16 / (int)sizeof(T);
  const T *row = x + (size_t)blockIdx.x * d;
  float ss = 0.f;
  for (int v = threadIdx.x; v < d / VEC; v += 64) {
    float f[VEC];
    unpack16(ld16(row + v * VEC), f, row);
#pragma unroll
    for (int e = 0; e < VEC; ++e) ss = fmaf(f[e], f[e], ss);
  }
  ss = wave_sum(ss);
  if (threadIdx.x == 0) rinv[blockIdx.x] = 1.0f / sqrtf(ss / (float)d + eps);
}

hipError_t launch_row_rinv(int dtype, const void *x, int rows, int d, float eps, float *rinv, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == kBF16)
    hipLaunchKernelGGL(row_rinv_kernel<bf16_t>, dim3(rows), dim3(64), 0, s, (const bf16_t *)x, d, eps, rinv);
  else
    hipLaunchKernelGGL(row_rinv_kernel<float>, dim3(rows), dim3(64), 0, s, (const float *)x, d, eps, rinv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Top-k least similar: one 512-thread workgroup per sequence, keys held in registers (up to 32 per
// thread: n <= 16384). 512 threads measured faster than 256 or 1024 at every n from 1024 to 8192
// (fewer keys per thread than 256, fewer waves to synchronise than 1024).
// ---------------------------------------------------------------------------------------------
constexpr int kTopkThreads = 512;

// Unsigned key with the float order of s: NaN lowest, -0 equal to +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over a wave with DPP: shifts of 1, 2, 4, 8 inside each 16-lane row, then the
// row totals are carried into rows 1 and 3 (row_bcast:15) and into rows 2 and 3 (row_bcast:31).
// Lanes without a source read 0 (bound_ctrl) or are masked off, which adds nothing.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return (uint32_t)x;
}

// Exclusive prefix sum over the workgroup (kTopkThreads = 512 threads, 8 waves; wsum has room for up
// to 16 waves). The _open form leaves out the closing barrier: the caller must pass another barrier
// before anything writes wsum again.
__device__ __forceinline__ uint32_t block_exclusive_scan_open(uint32_t v, uint32_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  return base + x - v;
}
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wsum) {
  const uint32_t e = block_exclusive_scan_open(v, wsum);
  __syncthreads();
  return e;
}

// AND / OR over a wave: rotations inside each 16-lane row (DPP row_ror), then the four row results.
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  int x = (int)v;
  x &= __builtin_amdgcn_update_dpp(x, x, 0x121, 0xf, 0xf, false);  // row_ror:1
  x &= __builtin_amdgcn_update_dpp(x, x, 0x122, 0xf, 0xf, false);  // row_ror:2
  x &= __builtin_amdgcn_update_dpp(x, x, 0x124, 0xf, 0xf, false);  // row_ror:4
  x &= __builtin_amdgcn_update_dpp(x, x, 0x128, 0xf, 0xf, false);  // row_ror:8
  return (uint32_t)(__builtin_amdgcn_readlane(x, 0) & __builtin_amdgcn_readlane(x, 16) &
                    __builtin_amdgcn_readlane(x, 32) & __builtin_amdgcn_readlane(x, 48));
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  int x = (int)v;
  x |= __builtin_amdgcn_update_dpp(x, x, 0x121, 0xf, 0xf, false);
  x |= __builtin_amdgcn_update_dpp(x, x, 0x122, 0xf, 0xf, false);
  x |= __builtin_amdgcn_update_dpp(x, x, 0x124, 0xf, 0xf, false);
  x |= __builtin_amdgcn_update_dpp(x, x, 0x128, 0xf, 0xf, false);
  return (uint32_t)(__builtin_amdgcn_readlane(x, 0) | __builtin_amdgcn_readlane(x, 16) |
                    __builtin_amdgcn_readlane(x, 32) | __builtin_amdgcn_readlane(x, 48));
}

// Radix select of the k smallest keys, emitted in ascending index order. The bits every key shares
// are skipped first (scores of one step often share sign, exponent and leading mantissa bits, which
// would otherwise pile every key into one histogram bin); the rest is resolved with digits of up to
// 11 bits, stopping as soon as the selected bin fits exactly. Equal keys at the boundary are taken in
// index order.
struct TopkShared {
  static constexpr int kBins = 2048;
  uint32_t hist[2][kBins];
  uint32_t wsum[16], wand[16], wor[16];
  uint32_t sel_prefix, sel_krem, sel_full;
};

// The k smallest of the n scores s[0 .. n) by a workgroup of TH threads (TH PER >= n), indices written
// ascending to out[0 .. k). Every thread of the workgroup calls it (it has barriers).
// COHERENT: the scores were written by other workgroups in the same launch with agent-scope atomic
// stores; they are read with agent-scope atomic loads (no stale cached copy).
template <int TH, int PER, bool COHERENT = false>
__device__ void topk_block(const float *s, int n, int k, int32_t *out, TopkShared &sh) {
  static_assert(TH % 64 == 0 && TH <= 1024 && TopkShared::kBins % TH == 0 && PER <= 64, "top-k block shape");
  constexpr int kBins = TopkShared::kBins;
  uint32_t(&hist)[2][kBins] = sh.hist;
  uint32_t *wsum = sh.wsum, *wand = sh.wand, *wor = sh.wor;
  uint32_t &sel_prefix = sh.sel_prefix, &sel_krem = sh.sel_krem, &sel_full = sh.sel_full;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = (n + TH - 1) / TH;
  const int start = tid * chunk;
  if (k >= n) {  // every token
    for (int i = tid; i < n; i += TH) out[i] = i;
    return;
  }

  uint32_t key[PER];
  uint64_t valid = 0;
  uint32_t kand = 0xffffffffu, kor = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = start + j;
    const bool ok = j < chunk && i < n;
    float v = 0.f;
    if (ok) v = COHERENT ? __hip_atomic_load(s + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : s[i];
    key[j] = ok ? order_key(v) : 0u;
    valid |= (ok ? 1ull : 0ull) << j;
    if (ok) {
      kand &= key[j];
      kor |= key[j];
    }
  }
  for (int i = tid; i < 2 * kBins; i += TH) (&hist[0][0])[i] = 0u;
  kand = wave_and(kand);
  kor = wave_or(kor);
  if (lane == 0) {
    wand[wave] = kand;
    wor[wave] = kor;
  }
  __syncthreads();
  kand = 0xffffffffu;
  kor = 0u;
#pragma unroll
  for (int w = 0; w < TH / 64; ++w) {
    kand &= wand[w];
    kor |= wor[w];
  }
  // bits above `hi` are common to every key
  int hi = 31 - __clz(kand ^ kor);  // -1 when all keys are equal
  uint32_t prefix = hi >= 31 ? 0u : (kand & (0xffffffffu << (hi + 1)));
  uint32_t krem = (uint32_t)k;
  bool full = false;
  int pass = 0;
  while (hi >= 0) {
    const int lo = hi >= 10 ? hi - 10 : 0;
    const uint32_t above = hi >= 31 ? 0u : (0xffffffffu << (hi + 1));
    const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
    uint32_t *h = hist[pass & 1];
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (((valid >> j) & 1ull) && (key[j] & above) == prefix) atomicAdd(&h[(key[j] >> lo) & dmask], 1u);
    __syncthreads();
    // BPT consecutive bins per thread; inclusive counts by a block scan
    constexpr int BPT = kBins / TH;
    uint32_t v[BPT], tot = 0;
    uint32_t *hn = hist[(pass + 1) & 1];  // next pass's bins (last read one pass ago)
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      v[q] = h[BPT * tid + q];
      hn[BPT * tid + q] = 0u;
      tot += v[q];
    }
    // three barriers per pass: the wsum reads of this scan and the sel_* reads below end before the
    // next pass's histogram barrier, the first point where wsum and sel_* are written again
    uint32_t e = block_exclusive_scan_open(tot, wsum);
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const uint32_t i1 = e + v[q];
      if (e < krem && krem <= i1) {
        sel_prefix = prefix | ((uint32_t)(BPT * tid + q) << lo);
        sel_krem = krem - e;
        sel_full = (i1 == krem) ? 1u : 0u;
      }
      e = i1;
    }
    __syncthreads();
    prefix = sel_prefix;
    krem = sel_krem;
    full = sel_full != 0u;
    hi = lo - 1;
    ++pass;
    if (full) break;
  }

  // Emit in index order: keys whose resolved bits are below the prefix, plus those equal to it --
  // all of them when the last bin fitted exactly, else the first `krem` in index order. Thread t holds
  // the contiguous index range [start, start + chunk), so a key's output position is the number of
  // keys below the prefix at lower indices plus the number of boundary keys taken at lower indices,
  // min(equal keys before it, krem). One exclusive scan yields both counts: below-prefix keys in the
  // low 16 bits, equal keys in the high 16 (n <= 16384, so neither field carries into the other).
  const uint32_t mask = hi >= 31 ? 0u : (0xffffffffu << (hi + 1));
  const uint32_t eq_cap = full ? 0xffffffffu : krem;
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (!((valid >> j) & 1ull)) continue;
    const uint32_t km = key[j] & mask;
    cnt += km < prefix ? 1u : (km == prefix ? 0x10000u : 0u);
  }
  // no closing barrier: callers pass a barrier before the shared state is written again
  const uint32_t before = block_exclusive_scan_open(cnt, wsum);
  uint32_t eq = before >> 16;
  uint32_t pos = (before & 0xffffu) + min(eq, eq_cap);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (!((valid >> j) & 1ull)) continue;
    const uint32_t km = key[j] & mask;
    bool take = km < prefix;
    if (km == prefix) take = eq++ < eq_cap;
    if (take && pos < (uint32_t)k) out[pos++] = start + j;
  }
}

template <int PER>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float *__restrict__ scores, int n, int k,
                                                            int32_t *__restrict__ idx_out) {
  __shared__ TopkShared sh;
  const int b = blockIdx.x;
  topk_block<kTopkThreads, PER>(scores + (size_t)b * n, n, k, idx_out + (size_t)b * k, sh);
}

// The cosine pass fused with the Top-k of each sequence (n tokens per sequence, k of them selected):
// every workgroup scores 8 (64 / LPR) tokens as proxy_cosine_kernel, then adds the number of its tokens
// in each sequence to that sequence's counter; the workgroup whose addition completes a sequence runs
// the Top-k of that sequence (topk_block with all kTopkThreads = 512 threads) and resets its counter to
// 0. The scores cross workgroups through agent-scope atomic stores and loads, which are coherent
// across the XCDs' L2 caches without cache-wide write-backs or invalidations (release / acquire fences
// would flush the whole L2, including this kernel's P^c writes); each wave waits until its score stores
// have completed before the workgroup's counter addition, which is itself an agent-scope atomic, and the
// Top-k's loads are issued only after that addition returned the completing count. Two rows per wave
// (LPR = 32) give half the workgroups of one row per wave, and so half the additions to each counter.
// The counters must be 0 at launch (the proxy projection that precedes this kernel clears them).
template <int PER, int LPR>
__global__ __launch_bounds__(kTopkThreads) void cosine_topk_kernel(const float *__restrict__ part, int splits,
                                                                   int rows, int r, const float *pc_read,
                                                                   float *pc_write, float *__restrict__ p_out,
                                                                   float *scores, const float *__restrict__ ss_part,
                                                                   int d, float eps, float *__restrict__ rinv, int n,
                                                                   int k, int32_t *__restrict__ idx_out,
                                                                   uint32_t *counters) {
  constexpr int RPW = 64 / LPR;                      // rows per wave
  constexpr int RW = kTopkThreads / 64 * RPW;        // rows of a workgroup
  __shared__ TopkShared sh;
  __shared__ uint32_t last[RW];
  const int tid = threadIdx.x, row0 = blockIdx.x * RW;
  const int wrow0 = row0 + (tid >> 6) * RPW;         // first row of this wave
  const int row = wrow0 + (tid & 63) / LPR;
  if (wrow0 < rows)  // uniform over the wave
    cosine_row<true, LPR>(part, splits, rows, r, row, row < rows, pc_read, pc_write, p_out, scores, ss_part, d, eps,
                          rinv);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's memory operations (its score stores included) completed
  __syncthreads();
  if (tid == 0) {  // the (at most RW) sequences of this workgroup's rows, in order
    int nl = 0;
    for (int rr = row0; rr < min(row0 + RW, rows);) {
      const int b = rr / n;
      const int end = min(min(row0 + RW, rows), (b + 1) * n);
      const uint32_t cnt = (uint32_t)(end - rr);
      const uint32_t before = __hip_atomic_fetch_add(&counters[b], cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (before + cnt == (uint32_t)n) last[nl++] = (uint32_t)b;
      rr = end;
    }
    for (int j = nl; j < RW; ++j) last[j] = 0xffffffffu;
  }
  __syncthreads();
#pragma unroll 1
  for (int j = 0; j < RW; ++j) {
    const uint32_t b = last[j];  // uniform
    if (b == 0xffffffffu) break;
    topk_block<kTopkThreads, PER, true>(scores + (size_t)b * n, n, k, idx_out + (size_t)b * k, sh);
    if (tid == 0) __hip_atomic_store(&counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();  // the shared state is reused by the next sequence
  }
}

template <int LPR>
hipError_t launch_cosine_topk_lpr(const float *part, int splits, int rows, int n, int r, const float *pc_read,
                                  float *pc_write, float *p_out, float *scores, const float *ss_part, int d,
                                  float eps, float *rinv, int k, int32_t *idx_out, uint32_t *counters,
                                  hipStream_t s) {
  constexpr int RW = kTopkThreads / 64 * (64 / LPR);
  const dim3 grid((rows + RW - 1) / RW), block(kTopkThreads);
#define SPA_COSINE_TOPK(PER)                                                                                       \
  hipLaunchKernelGGL((cosine_topk_kernel<PER, LPR>), grid, block, 0, s, part, splits, rows, r, pc_read, pc_write, \
                     p_out, scores, ss_part, d, eps, rinv, n, k, idx_out, counters)
  if (n <= 2 * kTopkThreads)
    SPA_COSINE_TOPK(2);
  else if (n <= 4 * kTopkThreads)
    SPA_COSINE_TOPK(4);
  else if (n <= 8 * kTopkThreads)
    SPA_COSINE_TOPK(8);
  else if (n <= 16 * kTopkThreads)
    SPA_COSINE_TOPK(16);
  else
    SPA_COSINE_TOPK(32);
#undef SPA_COSINE_TOPK
  return hipGetLastError();
}

hipError_t launch_cosine_topk(const float *part, int splits, int batch, int n, int r, const float *pc_read,
                              float *pc_write, float *p_out, float *scores, const float *ss_part, int d, float eps,
                              float *rinv, int k, int32_t *idx_out, uint32_t *counters, hipStream_t s) {
  const int rows = batch * n;
  if (rows <= 0) return hipSuccess;
  if (n > 32 * kTopkThreads || k <= 0 || pc_read == nullptr || scores == nullptr) return hipErrorInvalidValue;
  const int lpr = cosine_lanes_per_row(r);
  if (lpr == 16)
    return launch_cosine_topk_lpr<16>(part, splits, rows, n, r, pc_read, pc_write, p_out, scores, ss_part, d, eps,
                                      rinv, k, idx_out, counters, s);
  if (lpr == 32)
    return launch_cosine_topk_lpr<32>(part, splits, rows, n, r, pc_read, pc_write, p_out, scores, ss_part, d, eps,
                                      rinv, k, idx_out, counters, s);
  return launch_cosine_topk_lpr<64>(part, splits, rows, n, r, pc_read, pc_write, p_out, scores, ss_part, d, eps, rinv,
                                    k, idx_out, counters, s);
}

int topk_keys_per_thread(int n, bool fused) {
  for (int per = fused ? 2 : 4; per < 32; per *= 2)
    if (n <= per * kTopkThreads) return per;
  return 32;
}

hipError_t launch_topk(const float *scores, int batch, int n, int k, int32_t *idx_out, hipStream_t s) {
  if (batch <= 0 || k <= 0) return hipSuccess;
  if (n > 32 * kTopkThreads) return hipErrorInvalidValue;
  const dim3 grid(batch), block(kTopkThreads);
  if (n <= 4 * kTopkThreads)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, scores, n, k, idx_out);
  else if (n <= 8 * kTopkThreads)
    hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, scores, n, k, idx_out);
  else if (n <= 16 * kTopkThreads)
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, scores, n, k, idx_out);
  else
    hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, s, scores, n, k, idx_out);
  return hipGetLastError();
}

// P^c[I] <- P[I] (proxy-cache policy SELECTED); one wave per selected row.
__global__ __launch_bounds__(256) void copy_selected_kernel(const float *__restrict__ p_src, float *__restrict__ pc,
                                                            const int32_t *__restrict__ idx, int batch, int n, int k,
                                                            int r) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= batch * k) return;
  const int b = w / k;
  const int i = idx[w];
  if ((unsigned)i >= (unsigned)n) return;
  const size_t base = ((size_t)b * n + i) * r;
  for (int c = lane; c < r; c += 64) pc[base + c] = p_src[base + c];
}

hipError_t launch_copy_selected(const float *p_src, float *pc, const int32_t *idx, int batch, int n, int k, int r,
                                hipStream_t s) {
  if (batch <= 0 || k <= 0) return hipSuccess;
  const int waves = batch * k;
  hipLaunchKernelGGL(copy_selected_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, p_src, pc, idx, batch, n, k, r);
  return hipGetLastError();
}

}  // namespace spa
