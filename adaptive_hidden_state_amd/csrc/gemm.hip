// MFMA GEMM C = A W^T with the fused epilogues of the SPA-Cache sparse update
// ([PN] 整体框架 phases 2 and 3: Q/K/V of the update set with the K/V cache scatter, W_o with the
// residual, the SwiGLU gate/up product, and W_down with the residual scattered into H^c).
//
// A (M x K) and W (rows x K) are both K-contiguous, which is the operand order the 16x16 MFMA wants:
// every lane reads 16 contiguous bytes of a row for each k-step. Tiles are staged through LDS in
// 128-byte K slabs (64 bf16 / 32 fp32), double-buffered, with a 16-byte row pad so that the 16 rows a
// quarter-wave reads land on distinct LDS banks. Workgroups of one XCD get a contiguous range of
// tiles, M fastest, so tiles that share a weight panel run together behind the same L2.
#include "common.hpp"
#include "launch.hpp"

namespace spa {

// The gate/up weight is packed with its rows interleaved in groups of 64 (32 gate rows j..j+31, then
// the 32 up rows with the same j), so one lane of a pair of 32x32 MFMA blocks holds gate and up of
// the same unit: output column n holds hidden unit (n / 64) * 32 + n % 32, gate when n % 64 < 32.

__device__ __forceinline__ int map_token(const EpiArgs &ea, int m, int &b) {
  b = m / ea.k_per_seq;
  return ea.idx ? ea.idx[m] : (m - b * ea.k_per_seq);
}

template <typename T, int KIND>
__device__ __forceinline__ void epi_store(const EpiArgs &ea, int m, int n, float v) {
  if constexpr (KIND == kEpiQKV) {
    if (n < ea.dq) {
      ((T *)ea.out)[(size_t)m * ea.dq + n] = from_f32<T>(v);
      return;
    }
    int b;
    const int i = map_token(ea, m, b);
    if ((unsigned)i >= (unsigned)ea.n_tok) return;
    int nn = n - ea.dq;
    T *dst = (T *)ea.out2;
    if (nn >= ea.dkv) {
      nn -= ea.dkv;
      dst = (T *)ea.out3;
    }
    const int g = nn / ea.hd, e = nn - g * ea.hd;
    dst[(((size_t)b * ea.hkv + g) * ea.n_tok + i) * ea.hd + e] = from_f32<T>(v);
  } else if constexpr (KIND == kEpiResid) {
    int b;
    int i = map_token(ea, m, b);
    i = min(max(i, 0), ea.n_tok - 1);
    const float r = to_f32<T>(((const T *)ea.src)[((size_t)b * ea.n_tok + i) * ea.ld_src + n]);
    ((T *)ea.out)[(size_t)m * ea.ldo + n] = from_f32<T>(r + v);
  } else if constexpr (KIND == kEpiResidScatter) {
    int b;
    const int i = map_token(ea, m, b);
    if ((unsigned)i >= (unsigned)ea.n_tok) return;
    const float r = to_f32<T>(((const T *)ea.src)[(size_t)m * ea.ld_src + n]);
    ((T *)ea.out)[((size_t)b * ea.n_tok + i) * ea.ldo + n] = from_f32<T>(r + v);
  } else if constexpr (KIND == kEpiPartial) {
    ((float *)ea.out)[(size_t)m * ea.ldo + n] = v;
  }
}

template <typename T>
__device__ __forceinline__ void epi_swiglu(const EpiArgs &ea, int m, int j, float g, float u) {
  const float s = g / (1.0f + __expf(-g));
  ((T *)ea.out)[(size_t)m * ea.f + j] = from_f32<T>(s * u);
}

template <bool BF16> struct Frag;
template <> struct Frag<true> { typedef u32x4 type; };
template <> struct Frag<false> { typedef float type; };

// C[m][n] = sum_k A[m][k] W[n][k] on 32x32 MFMA blocks. A is row-major (lda elements per row). W is
// tile-packed: blocks of 64 rows x 128 bytes, block (i, j) at byte offset (i * wkb + j) * 8192, so
// the K slab of one 64-row panel is a contiguous 8 KB run and a workgroup streams its weight panel
// sequentially. K (and every split) is a multiple of the slab width; rows past N are zero.
template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, int KIND, int PF>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(
    const T *__restrict__ A, int lda, const T *__restrict__ W, int wkb, int M, int N, int K, int tiles_m,
    int tiles_n, int k_split, float *__restrict__ part, EpiArgs ea) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int BK = 128 / sizeof(T);
  constexpr int ROWB = 144;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_PER = BM * 8 / NT, B_PER = BN * 8 / NT;
  constexpr bool IS_BF16 = sizeof(T) == 2;
  constexpr int KSTEP_B = IS_BF16 ? 32 : 8;   // bytes of one row per MFMA k-step
  constexpr int LANE_B = IS_BF16 ? 16 : 4;    // bytes per lane per k-step
  constexpr int KSTEPS = 128 / KSTEP_B;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile loads must divide evenly");
  static_assert(BN % 64 == 0, "weight panels are 64 rows");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles are made of 32x32 blocks");
  static_assert(KIND != kEpiSwiGLU || (WTN % 64 == 0), "gate/up pairs must stay inside a wave");
  static_assert(PF == 2 || PF == 4, "prefetch depth must be even");
  typedef typename Frag<IS_BF16>::type FragT;

  __shared__ __attribute__((aligned(16))) char lds[2][(BM + BN) * ROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int tm = bid % tiles_m;
  const int rest = bid / tiles_m;
  const int tn = rest % tiles_n;
  const int split = rest / tiles_n;
  const int k0 = split * k_split;
  const int k1 = min(K, k0 + k_split);
  const int nk = k1 > k0 ? (k1 - k0) / BK : 0;

  const char *a_src[A_PER];
  const char *b_src[B_PER];
  int a_dst[A_PER], b_dst[B_PER];
#pragma unroll
  for (int j = 0; j < A_PER; ++j) {
    const int c = tid + j * NT, row = c >> 3, col = c & 7;
    const int gr = min(tm * BM + row, M - 1);
    a_src[j] = reinterpret_cast<const char *>(A + (size_t)gr * lda + k0) + col * 16;
    a_dst[j] = row * ROWB + col * 16;
  }
#pragma unroll
  for (int j = 0; j < B_PER; ++j) {
    const int c = tid + j * NT, row = c >> 3, col = c & 7;
    const int panel = tn * (BN / 64) + (row >> 6);
    b_src[j] = reinterpret_cast<const char *>(W) + (((size_t)panel * wkb + k0 / BK) * 64 + (row & 63)) * 128 + col * 16;
    b_dst[j] = BM * ROWB + row * ROWB + col * 16;
  }

  // Register ring of PF K slabs in flight: slab kt lives in slot kt % PF from its load until it is
  // written to LDS one iteration before it is used. Loads are unconditional (the slab index is
  // clamped), so the compiler waits for exactly the oldest slab; the slab count is padded to a
  // multiple of PF and padding slabs enter LDS with A zeroed, contributing nothing.
  u32x4 ra[PF][A_PER], rb[PF][B_PER];
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int kt, u32x4 *xa, u32x4 *xb) {
    const int kc = min(kt, nk - 1);
#pragma unroll
    for (int j = 0; j < A_PER; ++j) xa[j] = ld16(a_src[j] + (size_t)kc * 128);
#pragma unroll
    for (int j = 0; j < B_PER; ++j) xb[j] = ld16(b_src[j] + (size_t)kc * 8192);
  };
  auto lstore = [&](int buf, int kt, const u32x4 *xa, const u32x4 *xb) {
    if (kt < nk) {
#pragma unroll
      for (int j = 0; j < A_PER; ++j) st16(&lds[buf][a_dst[j]], xa[j]);
    } else {
#pragma unroll
      for (int j = 0; j < A_PER; ++j) st16(&lds[buf][a_dst[j]], zero);
    }
#pragma unroll
    for (int j = 0; j < B_PER; ++j) st16(&lds[buf][b_dst[j]], xb[j]);
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int nk_pad = (nk + PF - 1) / PF * PF;
  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < PF; ++u) gload(u, ra[u], rb[u]);
    lstore(0, 0, ra[0], rb[0]);
    gload(PF, ra[0], rb[0]);
  }
  __syncthreads();

  const int frag_off = (lane & 31) * ROWB + (lane >> 5) * LANE_B;
  for (int kt0 = 0; kt0 < nk_pad; kt0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kt = kt0 + u;
      const int cur = u & 1;  // PF is even, so slab kt0 + u sits in LDS buffer u & 1
      const char *As = &lds[cur][(wm * WTM) * ROWB + frag_off];
      const char *Bs = &lds[cur][BM * ROWB + (wn * WTN) * ROWB + frag_off];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        FragT af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const FragT *>(As + i * 32 * ROWB + ks * KSTEP_B);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const FragT *>(Bs + j * 32 * ROWB + ks * KSTEP_B);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
      }
      const int nslot = (u + 1) % PF;
      lstore(cur ^ 1, kt + 1, ra[nslot], rb[nslot]);
      gload(kt + 1 + PF, ra[nslot], rb[nslot]);
      __syncthreads();
    }
  }

  // lane holds column lane % 32 and rows 8 * (q / 4) + 4 * (lane / 32) + q % 4 of each 32x32 block
  const int row0 = tm * BM + wm * WTM + (lane >> 5) * 4;
  const int col0 = tn * BN + wn * WTN + (lane & 31);
  if (part != nullptr) {
    float *P = part + (size_t)split * M * N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = row0 + i * 32 + (q >> 2) * 8 + (q & 3), n = col0 + j * 32;
          if (m < M && n < N) P[(size_t)m * N + n] = acc[i][j][q];
        }
    return;
  }
  if constexpr (KIND == kEpiSwiGLU) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; j += 2)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = row0 + i * 32 + (q >> 2) * 8 + (q & 3), n = col0 + j * 32;
          if (m < M && n < N) epi_swiglu<T>(ea, m, (n >> 6) * 32 + (n & 63), acc[i][j][q], acc[i][j + 1][q]);
        }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = row0 + i * 32 + (q >> 2) * 8 + (q & 3), n = col0 + j * 32;
          if (m < M && n < N) epi_store<T, KIND>(ea, m, n, acc[i][j][q]);
        }
  }
}

// Sum of the split-K partials in split order (deterministic), then the epilogue.
template <typename T, int KIND>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int splits, int M,
                                                            int N, EpiArgs ea) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t plane = (size_t)M * N;
  if constexpr (KIND == kEpiSwiGLU) {
    const int f = ea.f;
    if (t >= (size_t)M * f) return;
    const int m = (int)(t / f), j = (int)(t - (size_t)m * f);
    const int ng = (j >> 5) * 64 + (j & 31);
    float g = 0.f, u = 0.f;
    for (int s = 0; s < splits; ++s) {
      g += part[s * plane + (size_t)m * N + ng];
      u += part[s * plane + (size_t)m * N + ng + 32];
    }
    epi_swiglu<T>(ea, m, j, g, u);
  } else {
    if (t >= plane) return;
    const int m = (int)(t / N), n = (int)(t - (size_t)m * N);
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += part[s * plane + t];
    epi_store<T, KIND>(ea, m, n, v);
  }
}

// ---------------------------------------------------------------------------------------------
// host side: tile plans and dispatch
// ---------------------------------------------------------------------------------------------
namespace {
constexpr int kTargetWGs = 256;  // one workgroup per CU of an MI355X

struct TileCfg {
  int bm, bn;
};
// 0: fp32 128x64 (4x1 waves of 32x64); 1: bf16 128x128 (2x2 waves of 64x64); 2: bf16 64x128 (2x2 waves
// of 32x64); 3: bf16 128x64 (2x2 waves of 64x32, not for the gate/up pairs)
constexpr TileCfg kTiles[4] = {{128, 64}, {128, 128}, {64, 128}, {128, 64}};

int ceil_div(int a, int b) { return (a + b - 1) / b; }
}  // namespace

GemmPlan plan_gemm(int dtype, int M, int N, int K, int kind) {
  // Measured on MI355X for the k-row GEMMs (M = 256): 128x128 tiles without split-K whenever they
  // give at least half a workgroup per CU; otherwise split K so the grid reaches one workgroup per CU,
  // on 128x128 tiles when each split keeps >= 2048 of K, else on 128x64 tiles.
  GemmPlan p{};
  const int bk = dtype == kF32 ? 32 : 64;
  int splits = 1;
  if (dtype == kF32) {
    p.cfg = 0;
  } else if (M <= 64) {
    p.cfg = 2;
    const int t2 = ceil_div(N, 128);
    if (kind != kEpiPartial && t2 < kTargetWGs / 2) splits = ceil_div(kTargetWGs, t2);
  } else {
    p.cfg = 1;
    const int t1 = ceil_div(M, 128) * ceil_div(N, 128);
    if (kind != kEpiPartial && t1 < kTargetWGs / 2) {
      splits = ceil_div(kTargetWGs, t1);
      if (K / splits < 2048 && kind != kEpiSwiGLU) {
        p.cfg = 3;
        splits = ceil_div(kTargetWGs, ceil_div(M, 128) * ceil_div(N, 64));
      }
    }
  }
  p.bm = kTiles[p.cfg].bm;
  p.bn = kTiles[p.cfg].bn;
  p.tiles_m = ceil_div(M, p.bm);
  p.tiles_n = ceil_div(N, p.bn);
  const int tiles = p.tiles_m * p.tiles_n;
  if (kind == kEpiPartial) splits = ceil_div(kTargetWGs, tiles);
  int max_splits = K / (bk * 4) > 1 ? K / (bk * 4) : 1;
  if (max_splits > 16) max_splits = 16;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int ks = ceil_div(K, splits);
  ks = ceil_div(ks, bk) * bk;
  p.k_split = ks;
  p.splits = ceil_div(K, ks);
  return p;
}

size_t gemm_partial_bytes(const GemmPlan &p, int M, int N) {
  return (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

template <typename T, int BM, int BN, int WMv, int WNv, int KIND>
static hipError_t run_gemm(const GemmPlan &p, const void *A, int lda, const void *W, int wkb, int M, int N,
                           int K, float *part, const EpiArgs &ea, hipStream_t s) {
  constexpr int PF = 4;
  const bool use_part = (KIND == kEpiPartial) || p.splits > 1;
  const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n * p.splits);
  EpiArgs e = ea;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WMv, WNv, KIND, PF>), dim3(grid), dim3(64 * WMv * WNv), 0, s,
                     (const T *)A, lda, (const T *)W, wkb, M, N, K, p.tiles_m, p.tiles_n, p.k_split,
                     use_part ? part : nullptr, e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || KIND == kEpiPartial || p.splits == 1) return err;
  const size_t work = KIND == kEpiSwiGLU ? (size_t)M * ea.f : (size_t)M * N;
  const unsigned rgrid = (unsigned)((work + 255) / 256);
  hipLaunchKernelGGL((splitk_reduce_kernel<T, KIND>), dim3(rgrid), dim3(256), 0, s, part, p.splits, M, N, e);
  return hipGetLastError();
}

template <typename T, int KIND>
static hipError_t run_cfg(const GemmPlan &p, const void *A, int lda, const void *W, int wkb, int M, int N, int K,
                          float *part, const EpiArgs &ea, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    return run_gemm<T, 128, 64, 4, 1, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
  } else {
    switch (p.cfg) {
      case 1: return run_gemm<T, 128, 128, 2, 2, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case 3:
        if constexpr (KIND != kEpiSwiGLU) return run_gemm<T, 128, 64, 2, 2, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
        return hipErrorInvalidValue;
      default: return run_gemm<T, 64, 128, 2, 2, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
    }
  }
}

template <typename T>
static hipError_t run_kind(int kind, const GemmPlan &p, const void *A, int lda, const void *W, int wkb, int M,
                           int N, int K, float *part, const EpiArgs &ea, hipStream_t s) {
  switch (kind) {
    case kEpiPartial: return run_cfg<T, kEpiPartial>(p, A, lda, W, wkb, M, N, K, part, ea, s);
    case kEpiQKV: return run_cfg<T, kEpiQKV>(p, A, lda, W, wkb, M, N, K, part, ea, s);
    case kEpiResid: return run_cfg<T, kEpiResid>(p, A, lda, W, wkb, M, N, K, part, ea, s);
    case kEpiSwiGLU: return run_cfg<T, kEpiSwiGLU>(p, A, lda, W, wkb, M, N, K, part, ea, s);
    case kEpiResidScatter: return run_cfg<T, kEpiResidScatter>(p, A, lda, W, wkb, M, N, K, part, ea, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int dtype, int kind, const GemmPlan &plan, const void *A, int lda, const void *W, int wkb,
                       int M, int N, int K, float *part, const EpiArgs &ea, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dtype == kF32) return run_kind<float>(kind, plan, A, lda, W, wkb, M, N, K, part, ea, s);
  return run_kind<bf16_t>(kind, plan, A, lda, W, wkb, M, N, K, part, ea, s);
}

}  // namespace spa
