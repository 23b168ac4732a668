// Update identification ([PN] 整体框架 Phase 1; [GS] part 1): cosine similarity of every token's
// singular proxy against the cached proxy, the proxy-cache update, and the Top-k least similar
// tokens per sequence. The proxy projection itself (P = X W_r^T) runs on the MFMA GEMM with fp32
// split-K partials; the kernel below sums those partials in a fixed order, so scores are
// deterministic run to run.
#include "common.hpp"
#include "launch.hpp"

namespace spa {

// ---------------------------------------------------------------------------------------------
// partial-sum reduce + cosine + proxy-cache write; one wave per token row
// ---------------------------------------------------------------------------------------------
constexpr int kMaxRankPerLane = 16;  // r <= 1024
constexpr int kMaxSplits = 16;       // the proxy GEMM never splits K more than this

__global__ __launch_bounds__(256) void proxy_cosine_kernel(const float *__restrict__ part, int splits, int rows,
                                                           int r, const float *pc_read, float *pc_write,
                                                           float *__restrict__ p_out, float *__restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const size_t plane = (size_t)rows * r;
  const size_t base = (size_t)row * r;
  float p[kMaxRankPerLane];
  float dot = 0.f, n1 = 0.f, n2 = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxRankPerLane; ++c) {
    const int col = lane + 64 * c;
    float v = 0.f;
    if (col < r) {
      float ps[kMaxSplits];
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s) ps[s] = s < splits ? part[s * plane + base + col] : 0.f;
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s) v += ps[s];
      n1 += v * v;
      if (pc_read != nullptr) {
        const float w = pc_read[base + col];
        dot += v * w;
        n2 += w * w;
      }
    }
    p[c] = v;
  }
  if (pc_read != nullptr && scores != nullptr) {
    dot = wave_sum(dot);
    n1 = wave_sum(n1);
    n2 = wave_sum(n2);
    if (lane == 0) scores[row] = dot / (fmaxf(sqrtf(n1), 1e-8f) * fmaxf(sqrtf(n2), 1e-8f));
  }
#pragma unroll
  for (int c = 0; c < kMaxRankPerLane; ++c) {
    const int col = lane + 64 * c;
    if (col < r) {
      if (p_out != nullptr) p_out[base + col] = p[c];
      if (pc_write != nullptr) pc_write[base + col] = p[c];
    }
  }
}

hipError_t launch_proxy_cosine(const float *part, int splits, int rows, int r, const float *pc_read, float *pc_write,
                               float *p_out, float *scores, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(proxy_cosine_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, part, splits, rows, r, pc_read,
                     pc_write, p_out, scores);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Top-k least similar: one 1024-thread workgroup per sequence, keys held in registers
// ---------------------------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kTopkPerThread = 16;  // n <= 16384

// Unsigned key with the float order of s: NaN lowest, -0 equal to +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (1024 threads = 16 waves); wsum holds 16 entries.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  __syncthreads();
  return base + x - v;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float *__restrict__ scores, int n, int k,
                                                            int32_t *__restrict__ idx_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t sel_prefix, sel_krem;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *s = scores + (size_t)b * n;
  const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
  const int start = tid * chunk;

  uint32_t key[kTopkPerThread];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kTopkPerThread; ++j) {
    const int i = start + j;
    const bool ok = j < chunk && i < n;
    key[j] = ok ? order_key(s[i]) : 0u;
    valid |= (ok ? 1u : 0u) << j;
  }

  // Radix select (8 bits per pass, most significant first) of the k-th smallest key.
  uint32_t prefix = 0, krem = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTopkPerThread; ++j)
      if (((valid >> j) & 1u) && (key[j] & hmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    uint32_t v = 0, incl = 0;
    if (tid < 256) {
      v = hist[tid];
      incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, off, kWave);
        if (lane >= off) incl += y;
      }
      if (lane == 63) wsum[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) incl += wsum[w];
      const uint32_t excl = incl - v;
      if (excl < krem && krem <= incl) {
        sel_prefix = prefix | ((uint32_t)tid << shift);
        sel_krem = krem - excl;
      }
    }
    __syncthreads();
    prefix = sel_prefix;
    krem = sel_krem;
    __syncthreads();
  }

  // Emit in index order: every key below the threshold, and the first `krem` keys equal to it.
  const uint32_t thr = prefix;
  uint32_t ceq = 0;
#pragma unroll
  for (int j = 0; j < kTopkPerThread; ++j) ceq += (((valid >> j) & 1u) && key[j] == thr) ? 1u : 0u;
  uint32_t r = block_exclusive_scan(ceq, wsum);
  uint32_t sel = 0, csel = 0;
#pragma unroll
  for (int j = 0; j < kTopkPerThread; ++j) {
    if (!((valid >> j) & 1u)) continue;
    bool take = key[j] < thr;
    if (key[j] == thr) {
      take = r < krem;
      ++r;
    }
    if (take) {
      sel |= 1u << j;
      ++csel;
    }
  }
  uint32_t pos = block_exclusive_scan(csel, wsum);
  int32_t *out = idx_out + (size_t)b * k;
#pragma unroll
  for (int j = 0; j < kTopkPerThread; ++j)
    if (((sel >> j) & 1u) && pos < (uint32_t)k) out[pos++] = start + j;
}

hipError_t launch_topk(const float *scores, int batch, int n, int k, int32_t *idx_out, hipStream_t s) {
  if (batch <= 0 || k <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(batch), dim3(kTopkThreads), 0, s, scores, n, k, idx_out);
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

// ---------------------------------------------------------------------------------------------
// RMSNorm of (gathered) rows: dst[m] = x / sqrt(mean(x^2) + eps) * g; one wave per row.
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T *__restrict__ src, const int32_t *__restrict__ idx,
                                                      int k_per_seq, int n_tok, int rows, int d,
                                                      const T *__restrict__ g, float eps, T *__restrict__ dst) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int MAXV = 16;  // 16-byte vectors per lane held in registers: d <= 1024 * VEC
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= rows) return;
  size_t srow = (size_t)m;
  if (idx != nullptr) {
    const int b = m / k_per_seq;
    const int i = min(max(idx[m], 0), n_tok - 1);
    srow = (size_t)b * n_tok + i;
  }
  const T *x = src + srow * d;
  T *y = dst + (size_t)m * d;
  const int nvec = d / VEC;
  u32x4 xv[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int v = lane + 64 * j;
    xv[j] = v < nvec ? ld16(x + v * VEC) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    float f[VEC];
    unpack16(xv[j], f, (const T *)nullptr);
#pragma unroll
    for (int e = 0; e < VEC; ++e) ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int v = lane + 64 * j;
    if (v < nvec) {
      float f[VEC], w[VEC];
      unpack16(xv[j], f, (const T *)nullptr);
      unpack16(ld16(g + v * VEC), w, (const T *)nullptr);
#pragma unroll
      for (int e = 0; e < VEC; ++e) f[e] = f[e] * rinv * w[e];
      st16(y + v * VEC, pack16(f, (const T *)nullptr));
    }
  }
}

hipError_t launch_rmsnorm(int dtype, const void *src, const int32_t *idx, int k_per_seq, int n_tok, int rows, int d,
                          const void *g, float eps, void *dst, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4);
  if (dtype == kBF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t *)src, idx, k_per_seq, n_tok,
                       rows, d, (const bf16_t *)g, eps, (bf16_t *)dst);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, grid, dim3(256), 0, s, (const float *)src, idx, k_per_seq, n_tok,
                       rows, d, (const float *)g, eps, (float *)dst);
  return hipGetLastError();
}

}  // namespace spa
