// MFMA GEMM C = A W^T with the fused epilogues of the SPA-Cache sparse update
// ([PN] 整体框架 phases 2 and 3: Q/K/V of the update set with the K/V cache scatter, W_o with the
// residual, the SwiGLU gate/up product, and W_down with the residual scattered into H^c).
//
// Weights are fragment-packed (pack.hip): every (32-row block, 16-k step) of W is one contiguous
// kilobyte laid out in the lane order of the 32x32 MFMA B operand, so a wave loads its B fragments
// straight from memory into registers with one fully coalesced 16-byte load per lane; weights never
// pass through LDS. Only the activation tile A (BM rows x 128-byte K slabs) is staged through LDS,
// double-buffered, rows padded to 144 bytes so the 32 rows a fragment read touches sit on distinct
// banks.
//
// A workgroup has four waves: two column halves (wn) x two K halves (wk). Wave (wn, wk) owns all BM
// rows and BN/2 columns and runs the MFMA k-steps of its K half of every slab, so no weight fragment
// is loaded twice in a workgroup and each A fragment read from LDS feeds BN/64 MFMAs. The two K
// halves are added through LDS at the end; each wave then finishes half of the rows.
// Workgroups of one XCD get a contiguous range of tiles, M fastest, so the M tiles that share a
// weight panel run together behind the same L2.
#include "common.hpp"
#include "launch.hpp"

namespace spa {

// The gate/up weight is packed so that each 32-row block holds the gate rows of 16 hidden units
// followed by the up rows of the same 16 units: output column n is unit (n / 32) * 16 + n % 16, gate
// when n % 32 < 16, and lanes l and l ^ 16 of a 32x32 MFMA block hold gate and up of one unit.

__device__ __forceinline__ int map_token(const EpiArgs &ea, int m, int &b) {
  b = m / ea.k_per_seq;
  return ea.idx ? ea.idx[m] : (m - b * ea.k_per_seq);
}

// Eight consecutive elements of T <-> floats (one 16-byte access for bf16, two for fp32).
__device__ __forceinline__ void load8(const bf16_t *p, float *v) { unpack16(ld16(p), v, p); }
__device__ __forceinline__ void load8(const float *p, float *v) {
  unpack16(ld16(p), v, p);
  unpack16(ld16(p + 4), v + 4, p);
}
__device__ __forceinline__ void store8(bf16_t *p, const float *v) { st16(p, pack16(v, p)); }
__device__ __forceinline__ void store8(float *p, const float *v) {
  st16(p, pack16(v, p));
  st16(p + 4, pack16(v + 4, p));
}

// Epilogue of output row m, columns n0 .. n0 + 7 (n0 % 8 == 0; every width here is a multiple of 8,
// and so is every head or hidden-unit boundary, so the eight never straddle one).
template <typename T> __device__ __forceinline__ float stored_sq8(const float *r);
template <> __device__ __forceinline__ float stored_sq8<float>(const float *r) {
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) s = fmaf(r[x], r[x], s);
  return s;
}
template <> __device__ __forceinline__ float stored_sq8<bf16_t>(const float *r) {  // of the bf16-rounded values
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < 8; x += 2) {
    const uint32_t h = pack_bf16x2(r[x], r[x + 1]);
    const float lo = __uint_as_float(h << 16), hi = __uint_as_float(h & 0xffff0000u);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

// Sum of squares of a row's 32-column block, kept by the first of the 4 consecutive lanes (or
// threads) that handle its four 8-column chunks: every lane calls this (shuffles), valid or not.
__device__ __forceinline__ void write_ss32(const EpiArgs &ea, int m, int n0, int N, float ss, bool valid,
                                           bool first) {
  ss += xor_lane<1>(ss);
  ss += xor_lane<2>(ss);
  if (valid && first) ea.ss_out[(size_t)m * (N / 32) + n0 / 32] = ss;
}

// Rotary embedding of head dims e .. e + 7 (e even) at position pos: the pair (2j, 2j + 1) rotates by
// pos * theta^(-2j / hd). The angle is taken in revolutions and reduced to [0, 1) before the hardware
// sine and cosine (which take revolutions); the fp32 product pos * frequency bounds the accuracy
// (about 1e-3 rad at position 16383), below one bf16 step of the rotated values.
__device__ __forceinline__ void rope8(float *v, int pos, int e, int hd, float log2_theta) {
  constexpr float kInvTwoPi = 0.15915494309189535f;
#pragma unroll
  for (int x = 0; x < 8; x += 2) {
    float rev = (float)pos * (exp2f(-(float)(e + x) / (float)hd * log2_theta) * kInvTwoPi);
    rev -= floorf(rev);
    const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
    const float a = v[x], c = v[x + 1];
    v[x] = a * cs - c * sn;
    v[x + 1] = a * sn + c * cs;
  }
}

// The two residual epilogues in two steps, so that the split-K reduce can issue its loads before any
// of them lands. resid_load8: the raw token index of row m and the raw residual row (kEpiResid: source
// row b n_tok + i, i clamped, which needs the index first; kEpiResidScatter: row m, loaded whether or
// not the row is written). Without an update set the index load reads a harmless word at `any` and is
// ignored, so no load sits under a branch. resid_store8: r = residual + v and the store (kEpiResid: row
// m of out, with the sum of squares of the stored values; kEpiResidScatter: H^c row b n_tok + i,
// skipped out of range).
template <typename T> struct Raw8 {
  u32x4 w[sizeof(T) / 2];
  int32_t idx;
};
template <typename T, int KIND>
__device__ __forceinline__ void resid_load8(const EpiArgs &ea, int m, int n0, const void *any, Raw8<T> &raw) {
  raw.idx = *(ea.idx != nullptr ? ea.idx + m : reinterpret_cast<const int32_t *>(any));
  const T *src = (const T *)ea.src + n0;
  if constexpr (KIND == kEpiResid) {
    const int b = m / ea.k_per_seq;
    const int i = ea.idx != nullptr ? raw.idx : m - b * ea.k_per_seq;
    src += ((size_t)b * ea.n_tok + min(max(i, 0), ea.n_tok - 1)) * ea.ld_src;
  } else {
    src += (size_t)m * ea.ld_src;
  }
#pragma unroll
  for (int h = 0; h < (int)(sizeof(T) / 2); ++h) raw.w[h] = ld16(src + h * (8 / (sizeof(T) / 2)));
}
template <typename T, int KIND>
__device__ __forceinline__ void resid_store8(const EpiArgs &ea, int m, int n0, const Raw8<T> &raw, const float *v,
                                             float *ssq) {
  const int b = m / ea.k_per_seq;
  const int i = ea.idx != nullptr ? raw.idx : m - b * ea.k_per_seq;
  if constexpr (KIND == kEpiResidScatter)
    if ((unsigned)i >= (unsigned)ea.n_tok) return;
  float r[8];
#pragma unroll
  for (int h = 0; h < (int)(sizeof(T) / 2); ++h) unpack16(raw.w[h], r + h * (8 / (sizeof(T) / 2)), (const T *)nullptr);
#pragma unroll
  for (int x = 0; x < 8; ++x) r[x] += v[x];
  if constexpr (KIND == kEpiResid) {
    store8((T *)ea.out + (size_t)m * ea.ldo + n0, r);
    if (ssq != nullptr) *ssq = stored_sq8<T>(r);
  } else {
    store8((T *)ea.out + ((size_t)b * ea.n_tok + i) * ea.ldo + n0, r);
  }
}

template <typename T, int KIND>
__device__ __forceinline__ void epi8(const EpiArgs &ea, int m, int n0, const float *v, float *ssq = nullptr) {
  if constexpr (KIND == kEpiQKV) {
    float w8[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) w8[x] = v[x];
    if (ea.bias != nullptr) {
      float bb[8];
      load8((const T *)ea.bias + n0, bb);
#pragma unroll
      for (int x = 0; x < 8; ++x) w8[x] += bb[x];
    }
    int b;
    const bool rope = ea.rope_log2_theta > 0.f;
    if (n0 < ea.dq) {
      if (rope) rope8(w8, map_token(ea, m, b), n0 % ea.hd, ea.hd, ea.rope_log2_theta);  // at the token's index
      store8((T *)ea.out + (size_t)m * ea.dq + n0, w8);
      return;
    }
    const int i = map_token(ea, m, b);  // the row's token index: its position
    if ((unsigned)i >= (unsigned)ea.n_tok) return;
    int nn = n0 - ea.dq;
    T *dst = (T *)ea.out2;
    const bool is_k = nn < ea.dkv;
    if (!is_k) {
      nn -= ea.dkv;
      dst = (T *)ea.out3;
    }
    const int g = nn / ea.hd, e = nn - g * ea.hd;
    if (is_k && rope) rope8(w8, i, e, ea.hd, ea.rope_log2_theta);
    store8(dst + (((size_t)b * ea.hkv + g) * ea.n_tok + i) * ea.hd + e, w8);
  } else if constexpr (KIND == kEpiResid || KIND == kEpiResidScatter) {
    Raw8<T> raw;
    resid_load8<T, KIND>(ea, m, n0, v, raw);
    resid_store8<T, KIND>(ea, m, n0, raw, v, ssq);
  } else if constexpr (KIND == kEpiPartial) {
    store8((float *)ea.out + (size_t)m * ea.ldo + n0, v);
  }
}

// z[m][j0 .. j0 + 7] = silu(gate) * up
template <typename T>
__device__ __forceinline__ void epi8_swiglu(const EpiArgs &ea, int m, int j0, const float *g, const float *u) {
  float z[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) z[x] = g[x] / (1.0f + __expf(-g[x])) * u[x];
  store8((T *)ea.out + (size_t)m * (ea.ldz ? ea.ldz : ea.f) + j0, z);
}

template <int BM, int BN> struct GemmLds {
  static constexpr int kA = 2 * BM * 144;                        // double-buffered A slabs
  static constexpr int kRed = 2 * (BM / 32) * (BN / 64) * 4096;  // one K half's blocks, both column halves
  static constexpr int kStride = BN / 2 + 4;                     // staged output row (floats)
  static constexpr int kEpi = 4 * (BM / 2) * kStride * 4;        // each wave's BM/2 x BN/2 fp32 rows
  static constexpr int kBytes = kA > kRed ? (kA > kEpi ? kA : kEpi) : (kRed > kEpi ? kRed : kEpi);
};

// C[m][n] = sum_k A[m][k] W[n][k]. A is row-major (lda elements per row). W is fragment-packed with
// wkb blocks per 32-row block. K (and every split) is a multiple of the 128-byte slab; columns past
// N are computed from clamped blocks and never stored.
template <typename T, int BM, int BN, int KIND, int PF>
__global__ __launch_bounds__(256) void gemm_kernel(const T *__restrict__ A, int lda, const char *__restrict__ W,
                                                   int wkb, int M, int N, int K, int tiles_m, int tiles_n,
                                                   int k_split, float *__restrict__ part, EpiArgs ea) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int BK = 128 / (int)sizeof(T);   // K elements per slab
  constexpr int BKF = BF ? 16 : 8;           // K elements per packed block
  constexpr int ROWB = 144;
  constexpr int FM = BM / 32, FN = BN / 64;  // 32x32 blocks of a wave tile (BM x BN/2)
  constexpr int A_PER = BM * 8 / 256;        // 16-byte A chunks per thread per slab
  constexpr int KSTEP_B = BF ? 32 : 8;       // bytes of an A row per MFMA k-step
  constexpr int LANE_B = BF ? 16 : 4;        // bytes per lane per k-step
  constexpr int KPB = BF ? 1 : 4;            // MFMA k-steps per packed block
  static_assert(FM % 2 == 0 && FN >= 1 && BM * 8 % 256 == 0, "tile shape");
  static_assert(PF == 2 || PF == 4, "prefetch depth must be even");
  typedef GemmLds<BM, BN> L;
  constexpr bool NORM = KIND == kEpiQKV || KIND == kEpiSwiGLU;  // A is RMSNorm's input (never split)

  __shared__ __attribute__((aligned(16))) char lds[L::kBytes];
  __shared__ float row_scale[NORM ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wk = wave >> 1;
  if (ea.clear != nullptr && blockIdx.x == 0)
    for (int i = tid; i < ea.clear_n; i += 256) ea.clear[i] = 0u;

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
  int a_dst[A_PER];
#pragma unroll
  for (int j = 0; j < A_PER; ++j) {
    const int c = tid + j * 256, row = c >> 3, col = c & 7;
    const int m = min(tm * BM + row, M - 1);
    size_t gr = (size_t)m;
    if (NORM && ea.idx != nullptr) {  // A rows gathered through the update set
      int b;
      const int i = map_token(ea, m, b);
      gr = (size_t)b * ea.n_tok + min(max(i, 0), ea.n_tok - 1);
    }
    a_src[j] = reinterpret_cast<const char *>(A + gr * lda + k0) + col * 16;
    a_dst[j] = row * ROWB + col * 16;
  }
  // Proxy projection over the hidden rows: this thread's share (16 bytes per slab) of the sum of
  // squares of its A rows, for the RMSNorm fused into the QKV GEMM (one column tile writes it).
  const bool acc_ss = KIND == kEpiPartial && ea.ss_out != nullptr && tn == 0;
  float ssq[A_PER];
#pragma unroll
  for (int j = 0; j < A_PER; ++j) ssq[j] = 0.f;
  // RMSNorm row scales of this tile, from the producers' statistics (computed after the first slabs'
  // loads are issued, visible after the first barrier)
  auto norm_scales = [&]() {
    if (ea.row_rinv != nullptr) {
      for (int r = tid; r < BM; r += 256) {
        const int m = min(tm * BM + r, M - 1);
        size_t src = (size_t)m;
        if (ea.idx != nullptr) {
          int b;
          const int i = map_token(ea, m, b);
          src = (size_t)b * ea.n_tok + min(max(i, 0), ea.n_tok - 1);
        }
        row_scale[r] = ea.row_rinv[src];
      }
    } else {  // 256 / BM consecutive threads per row sum its partials (4 at a time) in a fixed order
      constexpr int TPR = 256 / BM;
      const int r = tid / TPR, part_i = tid % TPR;
      const int m = min(tm * BM + r, M - 1);
      const floatx4 *ps = reinterpret_cast<const floatx4 *>(ea.ss_in + (size_t)m * ea.ss_n);
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int j = part_i; j < ea.ss_n / 4; j += TPR) v += ps[j];
      float t = (v[0] + v[1]) + (v[2] + v[3]);
      if constexpr (TPR >= 2) t += xor_lane<1>(t);
      if constexpr (TPR >= 4) t += xor_lane<2>(t);
      if (part_i == 0) row_scale[r] = 1.0f / sqrtf(t / (float)ea.norm_d + ea.norm_eps);
    }
  };
  // B: this wave's column blocks, blocks 2 wk and 2 wk + 1 of every slab (four blocks per slab)
  const int cb0 = (tn * BN + wn * (BN / 2)) / 32;
  const int cb_last = (N + 31) / 32 - 1;
  const char *b_src[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int cb = min(cb0 + j, cb_last);
    b_src[j] = W + ((size_t)cb * wkb + k0 / BKF + 2 * wk) * 1024 + lane * 16;
  }

  // Register ring of PF K slabs in flight: slab kt lives in slot kt % PF from its load until its A part
  // is written to LDS (at the start of the iteration before its use) and its B fragments are consumed. Loads are
  // unconditional (the slab index is clamped), so the compiler waits for exactly the oldest slab; the
  // slab count is padded to a multiple of PF and padding slabs enter LDS with A zeroed.
  u32x4 ra[PF][A_PER], rb[PF][2 * FN];
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int kt, u32x4 *xa, u32x4 *xb) {
    const int kc = min(kt, nk - 1);
#pragma unroll
    for (int j = 0; j < A_PER; ++j) xa[j] = ld16(a_src[j] + (size_t)kc * 128);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      xb[2 * j] = ld16(b_src[j] + (size_t)kc * 4096);
      xb[2 * j + 1] = ld16(b_src[j] + (size_t)kc * 4096 + 1024);
    }
  };
  auto lstore = [&](int buf, int kt, const u32x4 *xa) {
    char *dst = lds + buf * BM * ROWB;
    if (kt < nk) {
#pragma unroll
      for (int j = 0; j < A_PER; ++j) {
        st16(dst + a_dst[j], xa[j]);
        if (acc_ss) {
          if constexpr (BF) {  // exact fp32 squares (bf16 -> fp32 is a shift), fp32 accumulation
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const float lo = __uint_as_float(xa[j][x] << 16), hi = __uint_as_float(xa[j][x] & 0xffff0000u);
              ssq[j] = fmaf(lo, lo, ssq[j]);
              ssq[j] = fmaf(hi, hi, ssq[j]);
            }
          } else {
#pragma unroll
            for (int x = 0; x < 4; ++x) ssq[j] = fmaf(__uint_as_float(xa[j][x]), __uint_as_float(xa[j][x]), ssq[j]);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < A_PER; ++j) st16(dst + a_dst[j], zero);
    }
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
  }
  if constexpr (NORM) norm_scales();
  if (nk > 0) lstore(0, 0, ra[0]);
  __syncthreads();

  const int frag_off = (lane & 31) * ROWB + (lane >> 5) * LANE_B;
  for (int kt0 = 0; kt0 < nk_pad; kt0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kt = kt0 + u;
      // stage slab kt + 1 into the other buffer first (its VALU work then precedes the MFMA burst)
      lstore((u + 1) & 1, kt + 1, ra[(u + 1) % PF]);
      const char *As = lds + (u & 1) * BM * ROWB + frag_off;  // PF is even: slab kt0 + u is in buffer u & 1
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < KPB; ++s) {
          const int ks = (2 * wk + t) * KPB + s;  // k-step within the slab
          if constexpr (BF) {
            u32x4 af[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = ld16(As + i * 32 * ROWB + ks * KSTEP_B);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[i], rb[u][2 * j + t], acc[i][j]);
          } else {
            float af[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const float *>(As + i * 32 * ROWB + ks * KSTEP_B);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[i], __uint_as_float(rb[u][2 * j + t][s]), acc[i][j]);
          }
        }
      gload(kt + PF, ra[u], rb[u]);
      __syncthreads();
    }
  }

  if (acc_ss) {  // 8 consecutive lanes share a row; lane 0 of the 8 writes the split's sum of squares
#pragma unroll
    for (int j = 0; j < A_PER; ++j) {
      float v = ssq[j];
      v += xor_lane<1>(v);
      v += xor_lane<2>(v);
      v += xor_lane<4>(v);
      const int m = tm * BM + ((tid + j * 256) >> 3);
      if ((tid & 7) == 0 && m < M) ea.ss_out[(size_t)split * M + m] = v;
    }
  }

  // Add the two K halves: wave (wn, wk) keeps row blocks [wk FM/2, (wk+1) FM/2) and hands the others
  // to its partner (wn, 1 - wk) through LDS (16-byte chunks, lane-contiguous: conflict-free).
  constexpr int HM = FM / 2;
  auto red_at = [&](int i, int j, int c) { return lds + (((wn * FM + i) * FN + j) * 4 + c) * 1024 + lane * 16; };
  floatx16 own[HM][FN];
#pragma unroll
  for (int hi = 0; hi < HM; ++hi)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const floatx16 give = wk ? acc[hi][j] : acc[HM + hi][j];
      own[hi][j] = wk ? acc[HM + hi][j] : acc[hi][j];
      const int gi = wk ? hi : HM + hi;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        st16(red_at(gi, j, c), u32x4{__float_as_uint(give[4 * c]), __float_as_uint(give[4 * c + 1]),
                                     __float_as_uint(give[4 * c + 2]), __float_as_uint(give[4 * c + 3])});
    }
  __syncthreads();
#pragma unroll
  for (int hi = 0; hi < HM; ++hi)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int oi = wk ? HM + hi : hi;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 v = ld16(red_at(oi, j, c));
#pragma unroll
        for (int x = 0; x < 4; ++x) own[hi][j][4 * c + x] += __uint_as_float(v[x]);
      }
    }
  __syncthreads();

  // Stage this wave's BM/2 x BN/2 result row-major in its own LDS region, then let every lane finish
  // eight consecutive columns of a row at a time (one 16-byte store for bf16; per-row indexing once).
  // A lane holds column lane % 32 and rows 8 (q / 4) + 4 (lane / 32) + q % 4 of each 32x32 block.
  constexpr int ER = HM * 32, EC = FN * 32, ES = L::kStride;
  float *ep = reinterpret_cast<float *>(lds) + wave * ER * ES;
#pragma unroll
  for (int hi = 0; hi < HM; ++hi)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        ep[(hi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3)) * ES + j * 32 + (lane & 31)] = own[hi][j][q];
  // the wave reads back only what it wrote (in-order LDS within a wave)
  const int mbase = tm * BM + wk * ER;
  const int nbase = tn * BN + wn * EC;
  if (part != nullptr) {
    EpiArgs pe{};
    pe.out = part + (size_t)split * M * N;
    pe.ldo = N;
    for (int idx = lane; idx < ER * EC / 8; idx += 64) {
      const int lr = idx / (EC / 8), c8 = idx - lr * (EC / 8);
      const int m = mbase + lr, n0 = nbase + c8 * 8;
      if (m < M && n0 < N) epi8<T, kEpiPartial>(pe, m, n0, ep + lr * ES + c8 * 8);
    }
    return;
  }
  if constexpr (KIND == kEpiSwiGLU) {
    // columns 32 c + 0..15 are the gate rows of units 16 c + 0..15, columns 32 c + 16..31 their up rows
    for (int idx = lane; idx < ER * EC / 16; idx += 64) {
      const int lr = idx / (EC / 16), g8 = idx - lr * (EC / 16);
      const int c = g8 >> 1, h = g8 & 1;
      const int m = mbase + lr, j0 = (nbase / 32 + c) * 16 + h * 8;
      const float *row = ep + lr * ES + c * 32 + h * 8;
      if (m < M && j0 < ea.f) {
        float g[8], u[8];
        const float sc = NORM ? row_scale[wk * ER + lr] : 1.0f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          g[x] = row[x] * sc;
          u[x] = row[16 + x] * sc;
        }
        epi8_swiglu<T>(ea, m, j0, g, u);
      }
    }
  } else {
    for (int idx = lane; idx < ER * EC / 8; idx += 64) {  // uniform trip count (ER EC / 8 % 64 == 0)
      const int lr = idx / (EC / 8), c8 = idx - lr * (EC / 8);
      const int m = mbase + lr, n0 = nbase + c8 * 8;
      if (m < M && n0 < N) {
        if constexpr (NORM) {
          float v[8];
          const float sc = row_scale[wk * ER + lr];
#pragma unroll
          for (int x = 0; x < 8; ++x) v[x] = ep[lr * ES + c8 * 8 + x] * sc;
          epi8<T, KIND>(ea, m, n0, v);
        } else if constexpr (KIND != kEpiResid) {
          epi8<T, KIND>(ea, m, n0, ep + lr * ES + c8 * 8);
        }
      }
      if constexpr (KIND == kEpiResid) {  // EC / 8 is a multiple of 4: chunks c8 & ~3 .. | 3 share a block
        float ss = 0.f;
        const bool valid = m < M && n0 < N;
        if (valid) epi8<T, KIND>(ea, m, n0, ep + lr * ES + c8 * 8, &ss);
        if (ea.ss_out != nullptr) write_ss32(ea, m, n0, N, ss, valid, (c8 & 3) == 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Large-M GEMM (bf16, M in the hundreds to thousands): 256 x 256 output tiles. At this M the weight
// panel is reused by many row tiles, so the kernel is bound by MFMA issue and by the L2 -> CU
// traffic per flop, which a 256 x 256 tile halves against 128 x 192. Both operands are copied from
// global memory straight into LDS (global_load_lds, 16 bytes per lane, no registers and no LDS
// store instructions on the way) through a ring of four 32-k slab stages, three in flight while one
// is consumed. A sits in LDS row-major, 64 bytes per row, its 16-byte chunks XOR-swizzled by bits
// 1..2 of the row so that both the copy (four lanes per row) and the MFMA fragment reads (32 rows
// of one chunk) are free of bank conflicts; the packed weight blocks are copied as they are. Each
// of the four waves owns a 128 x 128 quarter of the tile (16 accumulator blocks, 256 registers).
// A 192-row variant (96 x 128 per wave) serves row counts just above a multiple of 256, where whole
// 256-row tiles would compute up to a third of their rows for nothing.
// ---------------------------------------------------------------------------------------------
template <int BM> struct BigLds {
  static_assert(BM == 256 || BM == 192, "big tile rows");
  static constexpr int kA = BM * 64;                      // A bytes of one 32-k slab
  static constexpr int kStage = kA + 16 * 1024;           // + B 16 KB
  static constexpr int kStages = 4;
  static constexpr int kStride = 132;                     // staged output row (floats)
  static constexpr int kEpi = 4 * 64 * kStride * 4;       // each wave's 64 x 128 output rows at a time
  static constexpr int kBytes = kEpi > kStages * kStage ? kEpi : kStages * kStage;
  static constexpr int CA = BM / 64;                      // A copy instructions per wave per slab
  static constexpr int FM = BM / 64;                      // 32-row accumulator blocks per wave
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_void_t;

// 16 bytes per lane from global memory into LDS at l + 16 lane (l uniform across the wave).
__device__ __forceinline__ void copy_to_lds(const void *g, char *l) {
  __builtin_amdgcn_global_load_lds((global_void_t *)g, (lds_void_t *)l, 16, 0, 0);
}
// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N> __device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// The same copy issued from inline asm: the compiler does not see it as an LDS write, so it puts no
// wait for copies in flight before later LDS reads, which it can then schedule among the MFMAs; the
// caller orders those reads after the copies they depend on (explicit vmcnt wait and barrier). M0
// takes the wave-uniform LDS base for the copy (one wait state between the M0 write and the copy
// that reads it) and gets its previous value back afterwards, so no value the compiler keeps in M0
// is lost. The copy writes no register, so its address registers may be reused once it has issued.
__device__ __forceinline__ void copy_to_lds_asm(const void *g, const char *l) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)l);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(g)
      : "memory");
}

// Per-thread copy plan of one slab: BM / 64 A instructions (16 rows x 64 bytes each) and 4 weight-block
// instructions (1 KB each) per wave.
template <int BM> struct BigCopy {
  const char *a_src[BM / 64];  // this lane's source 16 bytes of each A instruction, at slab 0
  const char *b_src[2];  // this lane's 16 bytes of the wave's two weight column blocks, at slab 0
  int wave;
  int nk;
};

// The main loop, with the four stage buffers as distinct restrict pointers: the compiler can then
// tell the fragment reads of one stage from the copies in flight into the others and needs no wait
// for them; the copies a stage's reads depend on are waited for explicitly (each wave its own,
// then a barrier).
template <int BM>
__device__ __forceinline__ void big_main_loop(char *__restrict__ s0, char *__restrict__ s1, char *__restrict__ s2,
                                              char *__restrict__ s3, const BigCopy<BM> &cp, int wm, int wn, int lane,
                                              floatx16 (&acc)[BM / 64][4]) {
  constexpr int CA = BigLds<BM>::CA, FM = BigLds<BM>::FM, KA = BigLds<BM>::kA;
  const int nk = cp.nk;
  // fragment offsets: A row wm BM / 2 + 32 i + lane % 32, logical chunk 2 s + lane / 32 (swizzled);
  // weight block (wn 4 + j, k-step s)
  const int arow = wm * (BM / 2) + (lane & 31), sw = ((lane & 31) >> 1) & 3;
  const int a_off0 = arow * 64 + ((0 + (lane >> 5)) ^ sw) * 16;
  const int a_off1 = arow * 64 + ((2 + (lane >> 5)) ^ sw) * 16;
  const int b_off = KA + (wn * 8) * 1024 + lane * 16;
  const int dst_a = cp.wave * CA * 1024, dst_b = KA + cp.wave * 4 * 1024;

// Slab KT (clamped) into stage DST.
#define SPA_BIG_ISSUE(KT, DST)                                                                         \
  do {                                                                                                 \
    const int kc_ = min((KT), nk - 1);                                                                 \
    _Pragma("unroll") for (int j = 0; j < CA; ++j)                                                     \
        copy_to_lds_asm(cp.a_src[j] + (size_t)kc_ * 64, (DST) + dst_a + j * 1024);                    \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                      \
        copy_to_lds_asm(cp.b_src[j >> 1] + ((size_t)kc_ * 2 + (j & 1)) * 1024, (DST) + dst_b + j * 1024); \
  } while (0)
// Slab KT from stage CUR after this wave's copies of it landed (slabs KT + 1, KT + 2 may stay in
// flight) and every wave passed the barrier; slab KT + 3 into stage NXT, which every wave finished
// reading before the barrier.
#define SPA_BIG_STEP(KT, CUR, NXT)                                                                     \
  do {                                                                                                 \
    wait_vmem<2 * (CA + 4)>();                                                                         \
    __builtin_amdgcn_s_barrier();                                                                      \
    SPA_BIG_ISSUE((KT) + 3, NXT);                                                                      \
    _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_) {                                                 \
      u32x4 af[FM], bf[4];                                                                             \
      const char *ar_ = (CUR) + (h_ ? a_off1 : a_off0), *br_ = (CUR) + b_off + h_ * 1024;              \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) af[i] = ld16(ar_ + i * 2048);                     \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) bf[j] = ld16(br_ + j * 2048);                      \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                                   \
          _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);   \
    }                                                                                                  \
  } while (0)

  SPA_BIG_ISSUE(0, s0);
  SPA_BIG_ISSUE(1, s1);
  SPA_BIG_ISSUE(2, s2);
  for (int kt = 0; kt < nk; kt += 4) {
    SPA_BIG_STEP(kt, s0, s3);
    if (kt + 1 < nk) SPA_BIG_STEP(kt + 1, s1, s0);
    if (kt + 2 < nk) SPA_BIG_STEP(kt + 2, s2, s1);
    if (kt + 3 < nk) SPA_BIG_STEP(kt + 3, s3, s2);
  }
#undef SPA_BIG_STEP
#undef SPA_BIG_ISSUE
  wait_vmem<0>();  // no copy may land in LDS after this point
}

template <int KIND, int BM>
__global__ __launch_bounds__(256) void gemm_big_kernel(const bf16_t *__restrict__ A, int lda,
                                                       const char *__restrict__ W, int wkb, int M, int N, int K,
                                                       int tiles_m, int tiles_n, EpiArgs ea) {
  typedef bf16_t T;
  typedef BigLds<BM> L;
  constexpr int BN = 256;
  constexpr int STAGE = L::kStage, ES = L::kStride, CA = L::CA, FM = L::FM;
  constexpr bool NORM = KIND == kEpiQKV || KIND == kEpiSwiGLU;
  __shared__ __attribute__((aligned(1024))) char lds[L::kBytes];
  __shared__ float row_scale[NORM ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // XCD-contiguous ranges of the launch order (as the small-M kernel), and within the order groups
  // of 8 row tiles: a group's A panels and the weight panel they share are read close together.
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int group = bid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_g = bid - group * GM * tiles_n;
  const int tm = first_m + in_g % gsize;
  const int tn = in_g / gsize;

  // copy plan: A instruction j of a wave covers rows r0 .. r0 + 15 (r0 = 16 (CA wave + j)); lane l
  // lands at LDS byte 16 l of it, i.e. row r0 + l / 4, physical chunk l % 4, and so fetches logical
  // chunk (l % 4) ^ ((row >> 1) & 3) of that row. Weight instruction j copies block 4 wave + j of the
  // slab (column block 2 wave + j / 2, k-step j % 2).
  BigCopy<BM> cp;
  cp.wave = wave;
  cp.nk = K / 32;
#pragma unroll
  for (int j = 0; j < CA; ++j) {
    const int row = (wave * CA + j) * 16 + (lane >> 2);
    const int m = min(tm * BM + row, M - 1);
    size_t gr = (size_t)m;
    if (NORM && ea.idx != nullptr) {  // A rows gathered through the update set
      int b;
      const int i = map_token(ea, m, b);
      gr = (size_t)b * ea.n_tok + min(max(i, 0), ea.n_tok - 1);
    }
    const int chunk = (lane & 3) ^ ((row >> 1) & 3);
    cp.a_src[j] = reinterpret_cast<const char *>(A + gr * lda) + chunk * 16;
  }
  const int cb_last = (N + 31) / 32 - 1;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cb = min(tn * 8 + 2 * wave + h, cb_last);
    cp.b_src[h] = W + (size_t)cb * wkb * 1024 + lane * 16;
  }

  auto norm_scales = [&]() {
    if constexpr (BM < 256) {
      if (tid >= BM) return;  // one thread per row
    }
    if (ea.row_rinv != nullptr) {
      const int m = min(tm * BM + tid, M - 1);
      size_t src = (size_t)m;
      if (ea.idx != nullptr) {
        int b;
        const int i = map_token(ea, m, b);
        src = (size_t)b * ea.n_tok + min(max(i, 0), ea.n_tok - 1);
      }
      row_scale[tid] = ea.row_rinv[src];
    } else {  // one thread per row sums its partials (4 at a time) in a fixed order
      const int m = min(tm * BM + tid, M - 1);
      const floatx4 *ps = reinterpret_cast<const floatx4 *>(ea.ss_in + (size_t)m * ea.ss_n);
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int j = 0; j < ea.ss_n / 4; ++j) v += ps[j];
      const float t = (v[0] + v[1]) + (v[2] + v[3]);
      row_scale[tid] = 1.0f / sqrtf(t / (float)ea.norm_d + ea.norm_eps);
    }
  };

  floatx16 acc[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  if constexpr (NORM) norm_scales();  // visible after the loop's barriers (and the one below)
  if (cp.nk > 0) big_main_loop<BM>(lds, lds + STAGE, lds + 2 * STAGE, lds + 3 * STAGE, cp, wm, wn, lane, acc);
  __syncthreads();

  // Epilogue in passes of up to 64 rows per wave (two; the 192-row tile's second pass has 32): stage
  // row-major in the wave's own LDS region (the wave reads back only what it wrote), then every lane
  // finishes eight consecutive columns of a row.
  constexpr int EC = 128;
  float *ep = reinterpret_cast<float *>(lds) + wave * 64 * ES;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ER = h == 0 ? 64 : BM / 2 - 64;  // rows of this pass
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      if (2 * h + ii >= FM) break;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          ep[(ii * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3)) * ES + j * 32 + (lane & 31)] = acc[2 * h + ii][j][q];
    }
    const int rbase = wm * (BM / 2) + h * 64;  // row of the tile
    const int mbase = tm * BM + rbase, nbase = tn * BN + wn * EC;
    if constexpr (KIND == kEpiSwiGLU) {
      for (int idx = lane; idx < ER * EC / 16; idx += 64) {
        const int lr = idx / (EC / 16), g8 = idx - lr * (EC / 16);
        const int c = g8 >> 1, hh = g8 & 1;
        const int m = mbase + lr, j0 = (nbase / 32 + c) * 16 + hh * 8;
        const float *row = ep + lr * ES + c * 32 + hh * 8;
        if (m < M && j0 < ea.f) {
          float g[8], u[8];
          const float sc = row_scale[rbase + lr];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            g[x] = row[x] * sc;
            u[x] = row[16 + x] * sc;
          }
          epi8_swiglu<T>(ea, m, j0, g, u);
        }
      }
    } else {
      for (int idx = lane; idx < ER * EC / 8; idx += 64) {  // uniform trip count
        const int lr = idx / (EC / 8), c8 = idx - lr * (EC / 8);
        const int m = mbase + lr, n0 = nbase + c8 * 8;
        if constexpr (KIND == kEpiResid) {  // chunks c8 & ~3 .. c8 | 3 share a 32-column block
          float ss = 0.f;
          const bool valid = m < M && n0 < N;
          if (valid) epi8<T, KIND>(ea, m, n0, ep + lr * ES + c8 * 8, &ss);
          if (ea.ss_out != nullptr) write_ss32(ea, m, n0, N, ss, valid, (c8 & 3) == 0);
        } else if (m < M && n0 < N) {
          if constexpr (NORM) {
            float v[8];
            const float sc = row_scale[rbase + lr];
#pragma unroll
            for (int x = 0; x < 8; ++x) v[x] = ep[lr * ES + c8 * 8 + x] * sc;
            epi8<T, KIND>(ea, m, n0, v);
          } else {
            epi8<T, KIND>(ea, m, n0, ep + lr * ES + c8 * 8);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Small-M GEMM fed by LDS DMA (bf16; the k-row products of the cached step, M in the hundreds), for
// the tiles where it beats the register-path kernel (measured on MI355X at M = 256: gate/up 128 x 192
// ~10% faster, W_down 128 x 128 split 4 ~6%; equal or slower on the narrower tiles). Both operands are
// copied from global memory into LDS with global_load_lds through a ring of NS 64-k stages. The
// workgroup has eight waves: waves 4..7 only issue the copies (each its quarter of every stage) and
// wait for them; waves 0..3 only compute, each a (BM/2) x (BN/2) quarter of the tile from fragments
// read out of LDS. A copy issue that stalls on a full memory pipeline thus never holds up the MFMA
// waves, and since the MFMA waves have no copies of their own in flight, the wait for outstanding
// copies that the compiler places before their LDS reads is immediate, so it schedules those reads
// freely under the MFMAs. One barrier per stage: the copiers arrive once their share of slab kt has
// landed, the MFMA waves once they finished slab kt - 1, whose stage then takes slab kt + NS - 1.
// LDS layout of a stage: A row-major, 128 bytes per row, 16-byte chunks XOR-swizzled by bits 1..3 of
// the row (conflict-free copies and fragment reads), then the packed weight blocks of the tile's
// column blocks as stored (four 16-k blocks per column block). A split-K launch writes fp32 partials
// that splitk_reduce_kernel sums and finishes.
// ---------------------------------------------------------------------------------------------
template <int BM, int BN> struct DmaCfg {
  // MFMA waves as 2 x 2 quarters of the tile, or as 4 x 1 row quarters when half of BN is not a
  // whole number of 32-column blocks (BN = 96)
  static constexpr int WM = (BN / 2) % 32 == 0 ? 2 : 4, WN = 4 / WM;
  static constexpr int TM = BM / WM, TN = BN / WN;      // MFMA-wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;      // its 32x32 blocks
  static constexpr int A_B = BM * 128, B_B = BN * 128;  // bytes of A and of W in one 64-k stage
  static constexpr int STAGE = A_B + B_B;
  static constexpr int NS = 147456 / STAGE < 8 ? 147456 / STAGE : 8;
  static constexpr int CA = BM / 32, CB = BN / 32;      // copy instructions per copy wave per stage
  static constexpr int ER = TM < 64 ? TM : 64;          // epilogue rows per pass
  static constexpr int ES = TN + 4;                     // staged output row (floats)
  static constexpr int EPI = 4 * ER * ES * 4;
  static constexpr int BYTES = NS * STAGE > EPI ? NS * STAGE : EPI;
  static_assert(TM % 32 == 0 && TN % 32 == 0 && BM <= 256 && BN <= 256, "tile shape");
  static_assert(NS >= 3 && (NS - 1) * (CA + CB) < 64, "ring depth");
};

// C[m][n] = sum_k A[m][k] W[n][k] over the workgroup's K range (bf16; K and k_split multiples of 64);
// part != nullptr: fp32 partials of split `split` at part + split M N, else the epilogue KIND.
template <int BM, int BN, int KIND>
__global__ __launch_bounds__(512) void gemm_dma_kernel(const bf16_t *__restrict__ A, int lda,
                                                       const char *__restrict__ W, int wkb, int M, int N, int K,
                                                       int tiles_m, int tiles_n, int k_split,
                                                       float *__restrict__ part, EpiArgs ea) {
  typedef bf16_t T;
  typedef DmaCfg<BM, BN> C;
  constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN, NS = C::NS, STAGE = C::STAGE;
  constexpr int CA = C::CA, CB = C::CB, ES = C::ES, ER = C::ER;
  constexpr bool NORM = KIND == kEpiQKV || KIND == kEpiSwiGLU;
  static_assert(KIND != kEpiPartial, "the proxy projection stays on the register-path kernel");
  __shared__ __attribute__((aligned(1024))) char lds[C::BYTES];
  __shared__ float row_scale[NORM ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool copier = wave >= 4;
  const int qw = wave & 3;  // quarter of the tile (MFMA waves) or of each stage's copies (copy waves)
  const int wm = qw % C::WM, wn = qw / C::WM;

  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int tm = bid % tiles_m;
  const int rest = bid / tiles_m;
  const int tn = rest % tiles_n;
  const int split = rest / tiles_n;
  const int k0 = split * k_split;
  const int k1 = min(K, k0 + k_split);
  const int nk = k1 > k0 ? (k1 - k0) / 64 : 0;

  // Copy plan. A instruction j of a copy wave covers tile rows r0 .. r0 + 7, r0 = 8 (CA qw + j): lane l
  // lands at byte 16 l of it (row r0 + l / 8, physical chunk l % 8) and so fetches logical chunk
  // (l % 8) ^ ((row >> 1) & 7) of the row's 128-byte stage slice. Weight instruction j copies stage
  // block q = CB qw + j: column block q / 4 of the tile, 16-k step q % 4 (the four steps of a column
  // block are adjacent in memory).
  const char *a_src[CA];
#pragma unroll
  for (int j = 0; j < CA; ++j) {
    const int row = (qw * CA + j) * 8 + (lane >> 3);
    const int m = min(tm * BM + row, M - 1);
    size_t gr = (size_t)m;
    if (NORM && ea.idx != nullptr) {  // A rows gathered through the update set
      int b;
      const int i = map_token(ea, m, b);
      gr = (size_t)b * ea.n_tok + min(max(i, 0), ea.n_tok - 1);
    }
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    a_src[j] = reinterpret_cast<const char *>(A + gr * lda + k0) + chunk * 16;
  }
  const int cb_last = (N + 31) / 32 - 1;
  const char *b_src[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int q = qw * CB + j;
    const int cb = min(tn * (BN / 32) + (q >> 2), cb_last);
    b_src[j] = W + ((size_t)cb * wkb + k0 / 16 + (q & 3)) * 1024 + lane * 16;
  }
  auto issue = [&](int kt, char *dst) {
    const int kc = min(kt, nk - 1);
#pragma unroll
    for (int j = 0; j < CA; ++j) copy_to_lds(a_src[j] + (size_t)kc * 128, dst + (qw * CA + j) * 1024);
#pragma unroll
    for (int j = 0; j < CB; ++j) copy_to_lds(b_src[j] + (size_t)kc * 4096, dst + C::A_B + (qw * CB + j) * 1024);
  };

  if (NORM && !copier) {  // RMSNorm row scales from the producers' statistics (as gemm_kernel)
    if (ea.row_rinv != nullptr) {
      for (int r = tid; r < BM; r += 256) {
        const int m = min(tm * BM + r, M - 1);
        size_t src = (size_t)m;
        if (ea.idx != nullptr) {
          int b;
          const int i = map_token(ea, m, b);
          src = (size_t)b * ea.n_tok + min(max(i, 0), ea.n_tok - 1);
        }
        row_scale[r] = ea.row_rinv[src];
      }
    } else {
      constexpr int TPR = 256 / BM;
      const int r = tid / TPR, part_i = tid % TPR;
      const int m = min(tm * BM + r, M - 1);
      const floatx4 *ps = reinterpret_cast<const floatx4 *>(ea.ss_in + (size_t)m * ea.ss_n);
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int j = part_i; j < ea.ss_n / 4; j += TPR) v += ps[j];
      float t = (v[0] + v[1]) + (v[2] + v[3]);
      if constexpr (TPR >= 2) t += xor_lane<1>(t);
      if constexpr (TPR >= 4) t += xor_lane<2>(t);
      if (part_i == 0) row_scale[r] = 1.0f / sqrtf(t / (float)ea.norm_d + ea.norm_eps);
    }
  }

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  if (nk > 0) {
    // fragment offsets inside a stage: A row wm TM + 32 i + lane % 32, logical chunk 2 s + lane / 32
    // (swizzled); weight block (column block wn FN + j, k-step s)
    const int sw = ((lane & 31) >> 1) & 7;
    const int arow = (wm * TM + (lane & 31)) * 128;
    int a_off[4], b_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a_off[s] = arow + ((2 * s + (lane >> 5)) ^ sw) * 16;
      b_off[s] = C::A_B + (wn * FN * 4 + s) * 1024 + lane * 16;
    }
    if (copier) {
#pragma unroll
      for (int u = 0; u < NS - 1; ++u) issue(u, lds + u * STAGE);
    }
    int cur = 0;  // stage of slab kt
    for (int kt = 0; kt < nk; ++kt) {
      if (copier) wait_vmem<(NS - 2) * (CA + CB)>();  // this wave's copies of slab kt landed
      __builtin_amdgcn_s_barrier();  // everyone's did, and everyone finished reading slab kt - 1
      if (copier) {
        issue(kt + NS - 1, lds + (cur == 0 ? NS - 1 : cur - 1) * STAGE);
      } else {
        const char *st = lds + cur * STAGE;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u32x4 af[FM], bf[FN];
#pragma unroll
          for (int i = 0; i < FM; ++i) af[i] = ld16(st + a_off[s] + i * 4096);
#pragma unroll
          for (int j = 0; j < FN; ++j) bf[j] = ld16(st + b_off[s] + j * 4096);
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
        }
      }
      cur = cur == NS - 1 ? 0 : cur + 1;
    }
    if (copier) wait_vmem<0>();  // no copy may land in LDS after this point
  }
  __syncthreads();
  if (copier) return;

  // Epilogue in passes of ER rows per MFMA wave: stage row-major in the wave's own LDS region (the
  // wave reads back only what it wrote), then every lane finishes eight consecutive columns of a row.
  float *ep = reinterpret_cast<float *>(lds) + qw * ER * ES;
#pragma unroll
  for (int h = 0; h < TM / ER; ++h) {
#pragma unroll
    for (int ii = 0; ii < ER / 32; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          ep[(ii * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3)) * ES + j * 32 + (lane & 31)] =
              acc[h * (ER / 32) + ii][j][q];
    const int rbase = wm * TM + h * ER;  // row of the tile
    const int mbase = tm * BM + rbase, nbase = tn * BN + wn * TN;
    if (part != nullptr) {
      EpiArgs pe{};
      pe.out = part + (size_t)split * M * N;
      pe.ldo = N;
      for (int idx = lane; idx < ER * TN / 8; idx += 64) {
        const int lr = idx / (TN / 8), c8 = idx - lr * (TN / 8);
        const int m = mbase + lr, n0 = nbase + c8 * 8;
        if (m < M && n0 < N) epi8<T, kEpiPartial>(pe, m, n0, ep + lr * ES + c8 * 8);
      }
    } else if constexpr (KIND == kEpiSwiGLU) {
      // columns 32 c + 0..15 are the gate rows of units 16 c + 0..15, columns 32 c + 16..31 their up rows
      for (int idx = lane; idx < ER * TN / 16; idx += 64) {
        const int lr = idx / (TN / 16), g8 = idx - lr * (TN / 16);
        const int c = g8 >> 1, hh = g8 & 1;
        const int m = mbase + lr, j0 = (nbase / 32 + c) * 16 + hh * 8;
        const float *row = ep + lr * ES + c * 32 + hh * 8;
        if (m < M && j0 < ea.f) {
          float g[8], u[8];
          const float sc = row_scale[rbase + lr];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            g[x] = row[x] * sc;
            u[x] = row[16 + x] * sc;
          }
          epi8_swiglu<T>(ea, m, j0, g, u);
        }
      }
    } else {
      for (int idx = lane; idx < ER * TN / 8; idx += 64) {  // uniform trip count (ER TN / 8 % 64 == 0)
        const int lr = idx / (TN / 8), c8 = idx - lr * (TN / 8);
        const int m = mbase + lr, n0 = nbase + c8 * 8;
        if constexpr (KIND == kEpiResid) {  // chunks c8 & ~3 .. c8 | 3 share a 32-column block
          float ss = 0.f;
          const bool valid = m < M && n0 < N;
          if (valid) epi8<T, KIND>(ea, m, n0, ep + lr * ES + c8 * 8, &ss);
          if (ea.ss_out != nullptr) write_ss32(ea, m, n0, N, ss, valid, (c8 & 3) == 0);
        } else if (m < M && n0 < N) {
          if constexpr (NORM) {
            float v[8];
            const float sc = row_scale[rbase + lr];
#pragma unroll
            for (int x = 0; x < 8; ++x) v[x] = ep[lr * ES + c8 * 8 + x] * sc;
            epi8<T, KIND>(ea, m, n0, v);
          } else {
            epi8<T, KIND>(ea, m, n0, ep + lr * ES + c8 * 8);
          }
        }
      }
    }
  }
}

// v[0..7] (+)= the sum over S consecutive splits of p[s plane + 0..7], added in split order; all S
// loads are issued before the first addition.
template <int S>
__device__ __forceinline__ void add_partials8(const float *p, size_t plane, float *v) {
  floatx4 a[S][2];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    a[j][0] = *reinterpret_cast<const floatx4 *>(p + (size_t)j * plane);
    a[j][1] = *reinterpret_cast<const floatx4 *>(p + (size_t)j * plane + 4);
  }
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      v[x] += a[j][0][x];
      v[4 + x] += a[j][1][x];
    }
}
// v[0..7] = the sum over the splits s of p[s plane + 0..7], added in split order from zero
// (deterministic), up to eight splits' loads in flight together.
__device__ __forceinline__ void sum_partials8(const float *p, size_t plane, int splits, float *v) {
#pragma unroll
  for (int x = 0; x < 8; ++x) v[x] = 0.f;
  int s = 0;
  for (; s + 8 <= splits; s += 8) add_partials8<8>(p + (size_t)s * plane, plane, v);
  switch (splits - s) {
    case 1: add_partials8<1>(p + (size_t)s * plane, plane, v); break;
    case 2: add_partials8<2>(p + (size_t)s * plane, plane, v); break;
    case 3: add_partials8<3>(p + (size_t)s * plane, plane, v); break;
    case 4: add_partials8<4>(p + (size_t)s * plane, plane, v); break;
    case 5: add_partials8<5>(p + (size_t)s * plane, plane, v); break;
    case 6: add_partials8<6>(p + (size_t)s * plane, plane, v); break;
    case 7: add_partials8<7>(p + (size_t)s * plane, plane, v); break;
    default: break;
  }
}

// Sum of the split-K partials in split order (deterministic), then the epilogue, eight columns (or
// eight hidden units) per thread. The residual epilogues issue their token-index and residual loads
// before the partial loads, so each thread waits about one memory round trip.
template <typename T, int KIND>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int splits, int M,
                                                            int N, EpiArgs ea) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t plane = (size_t)M * N;
  if constexpr (KIND == kEpiSwiGLU) {
    const int f8 = ea.f / 8;
    if (t >= (size_t)M * f8) return;
    const int m = (int)(t / f8), j0 = (int)(t - (size_t)m * f8) * 8;
    const int ng = (j0 >> 4) * 32 + (j0 & 15);
    float g[8], u[8];
    sum_partials8(part + (size_t)m * N + ng, plane, splits, g);
    sum_partials8(part + (size_t)m * N + ng + 16, plane, splits, u);
    epi8_swiglu<T>(ea, m, j0, g, u);
  } else {
    const int n8 = N / 8;
    const bool valid = t < (size_t)M * n8;
    const size_t tc = valid ? t : (size_t)M * n8 - 1;
    const int m = (int)(tc / n8), n0 = (int)(tc - (size_t)m * n8) * 8;
    float ss = 0.f;
    if (valid) {
      float v[8];
      if constexpr (KIND == kEpiResid || KIND == kEpiResidScatter) {
        Raw8<T> raw;
        resid_load8<T, KIND>(ea, m, n0, part, raw);
        sum_partials8(part + (size_t)m * N + n0, plane, splits, v);
        resid_store8<T, KIND>(ea, m, n0, raw, v, &ss);
      } else {
        sum_partials8(part + (size_t)m * N + n0, plane, splits, v);
        epi8<T, KIND>(ea, m, n0, v, &ss);
      }
    }
    // N % 32 == 0, so threads t & ~3 .. t | 3 hold the four chunks of one 32-column block
    if constexpr (KIND == kEpiResid)
      if (ea.ss_out != nullptr) write_ss32(ea, m, n0, N, ss, valid, (t & 3) == 0);
  }
}

// ---------------------------------------------------------------------------------------------
// Proxy projection P = X W_r^T at rank 128 (bf16): fp32 split-K partials of 32-row x 128-column tiles
// ---------------------------------------------------------------------------------------------
// With the whole rank in one tile, a 1024-row projection split 8 ways over K is 256 workgroups that
// each pull 32 rows x 512 k of X and 128 x 512 of W_r (160 KB), against 128 KB for the 64 x 64 tiles of
// the register-path kernel but with no second column tile re-reading the rows: measured 5.7 against
// 7.0 us at 1024 rows, 8.7 against 10.2 at 2048 (split 4). Four waves, one 32-column block of W_r
// each; the 32 x 64 A slab goes through LDS (double-buffered, 144-byte rows), each wave streams its
// packed W_r blocks into registers, a ring of PF slabs in flight as in gemm_kernel. Output: the
// partials of split s at part + s M 128 and, when ss_out is set, each row's sum of squares over the
// split's K range at ss_out[s M + m] (the statistics of the RMSNorm fused into the QKV GEMM).
constexpr int kProxyRows = 32, kProxyCols = 128;

template <int PF>
__global__ __launch_bounds__(256) void proxy_gemm_kernel(const bf16_t *__restrict__ A, int lda,
                                                         const char *__restrict__ W, int wkb, int M, int K,
                                                         int tiles_m, int k_split, float *__restrict__ part,
                                                         float *__restrict__ ss_out, uint32_t *clear, int clear_n) {
  constexpr int ROWB = 144;
  __shared__ __attribute__((aligned(16))) char lds[2 * kProxyRows * ROWB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (clear != nullptr && blockIdx.x == 0)
    for (int i = tid; i < clear_n; i += 256) clear[i] = 0u;

  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);  // XCD i runs a contiguous range
  const int tm = bid % tiles_m, split = bid / tiles_m;
  const int k0 = split * k_split;
  const int k1 = min(K, k0 + k_split);
  const int nk = k1 > k0 ? (k1 - k0) / 64 : 0;

  // A: thread t copies 16 bytes (chunk t % 8) of row t / 8 of each slab
  const int arow = tid >> 3, achunk = tid & 7;
  const int m_a = min(tm * kProxyRows + arow, M - 1);
  const char *a_src = reinterpret_cast<const char *>(A + (size_t)m_a * lda + k0) + achunk * 16;
  const int a_dst = arow * ROWB + achunk * 16;
  // B: this wave's column block (columns 32 wave .. 32 wave + 31), the four 16-k blocks of each slab
  const char *b_src = W + ((size_t)wave * wkb + k0 / 16) * 1024 + lane * 16;

  u32x4 ra[PF], rb[PF][4];
  auto gload = [&](int kt, u32x4 &xa, u32x4 *xb) {  // clamped slab index: unconditional loads
    const int kc = min(kt, max(nk - 1, 0));
    xa = ld16(a_src + (size_t)kc * 128);
#pragma unroll
    for (int s = 0; s < 4; ++s) xb[s] = ld16(b_src + ((size_t)kc * 4 + s) * 1024);
  };
  float ssq = 0.f;
  auto lstore = [&](int buf, int kt, const u32x4 &xa) {
    if (kt >= nk) return;
    st16(lds + buf * kProxyRows * ROWB + a_dst, xa);
#pragma unroll
    for (int x = 0; x < 4; ++x) {  // exact fp32 squares of the bf16 pair, fp32 accumulation
      const float lo = __uint_as_float(xa[x] << 16), hi = __uint_as_float(xa[x] & 0xffff0000u);
      ssq = fmaf(lo, lo, ssq);
      ssq = fmaf(hi, hi, ssq);
    }
  };

  floatx16 acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < PF; ++u) gload(u, ra[u], rb[u]);
    lstore(0, 0, ra[0]);
  }
  __syncthreads();
  const int nk_pad = (nk + PF - 1) / PF * PF;
  const int frag_off = (lane & 31) * ROWB + (lane >> 5) * 16;
  // One group of PF slabs; LOAD: refill each slot with the slab PF ahead. The last group issues no
  // loads (every slab it would fetch lies past the end), so no clamped re-read of the last slab is
  // requested (at 8 slabs per workgroup, PF = 4, that was a third of the loads), and its waits stay
  // exact in straight-line code.
  auto group = [&](int kt0, auto load_tag) {
    constexpr bool LOAD = decltype(load_tag)::value;
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kt = kt0 + u;
      lstore((u + 1) & 1, kt + 1, ra[(u + 1) % PF]);  // PF is even: slab kt0 + u is in buffer u & 1
      if (kt < nk) {
        const char *As = lds + (u & 1) * kProxyRows * ROWB + frag_off;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma32(ld16(As + s * 32), rb[u][s], acc);
      }
      if constexpr (LOAD) gload(kt + PF, ra[u], rb[u]);
      __syncthreads();
    }
  };
  for (int kt0 = 0; kt0 + PF < nk_pad; kt0 += PF) group(kt0, BoolTag<true>{});
  if (nk_pad > 0) group(nk_pad - PF, BoolTag<false>{});

  // lane holds column 32 wave + lane % 32 and rows 8 (q / 4) + 4 (lane / 32) + q % 4 of the tile
  float *pp = part + (size_t)split * M * kProxyCols + wave * 32 + (lane & 31);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int m = tm * kProxyRows + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
    if (m < M) pp[(size_t)m * kProxyCols] = acc[q];
  }
  if (ss_out != nullptr) {  // the 8 threads of a row add their squares in a fixed order
    ssq += xor_lane<1>(ssq);
    ssq += xor_lane<2>(ssq);
    ssq += xor_lane<4>(ssq);
    const int m = tm * kProxyRows + arow;
    if (achunk == 0 && m < M) ss_out[(size_t)split * M + m] = ssq;
  }
}

// ---------------------------------------------------------------------------------------------
// host side: tile plans and dispatch
// ---------------------------------------------------------------------------------------------
namespace {
constexpr int kCUs = 256;

struct TileCfg {
  int bm, bn;
};
// bf16 tiles 0..5; fp32 uses tile 5 only
constexpr TileCfg kTiles[6] = {{128, 192}, {64, 192}, {128, 128}, {128, 64}, {64, 128}, {64, 64}};

int ceil_div(int a, int b) { return (a + b - 1) / b; }
long long ceil_div_ll(long long a, long long b) { return (a + b - 1) / b; }

// Workgroups of the bf16 register-path kernel resident per CU, by tile configuration and epilogue kind
// (register-limited: each 256-thread workgroup puts one wave on each SIMD).
constexpr int kRegTileWgsPerCU[6][5] = {{1, 1, 1, 1, 1}, {2, 1, 2, 1, 2}, {1, 1, 1, 1, 1},
                                        {2, 2, 2, 2, 2}, {2, 2, 2, 2, 2}, {4, 3, 4, 3, 4}};

// Cost model of one launch in CU clocks, fitted to MI355X measurements of these kernels over M = 51 ..
// 2048 on the llada and Dream shapes (over 85 shapes its picks sum to within 2% of the fastest
// measured tile and split per shape): a
// workgroup costs its K range times its load time (weight panel from HBM, A tile mostly from L2) plus
// its MFMA time, which overlap little; w workgroups resident on a CU share its read path and together
// run 1.2 (w = 2), 1.3 (3) or 1.4 (4) times as fast as one; split-K adds the fp32 partial round trip
// (~2.6 TB/s) and a second launch. dma: cost factor of the LDS-DMA kernel that runs the tile (1 = none).
double plan_cost(int bm, int bn, int M, int N, int K, int splits, int kc, int wpc, double dma) {
  static const double kShared[5] = {1.0, 1.0, 1.2, 1.3, 1.4};
  const long long tiles = (long long)ceil_div(M, bm) * ceil_div(N, bn);
  const long long wgs = tiles * splits;
  const int w = (int)std::max(1LL, std::min((long long)wpc, ceil_div_ll(wgs, kCUs)));
  const double rounds = (double)ceil_div_ll(wgs, (long long)kCUs * w);
  const double load = (bn + 0.6 * bm) / 14.0;
  const double mfma = (double)bm * bn / 1660.0;
  double t = rounds * kc * (load + mfma) * w / kShared[w] * dma;
  if (splits > 1) t += (double)M * N * splits * 0.00646 + 4200.0;
  return t;
}
}  // namespace

namespace {
// Best register-path or LDS-DMA plan (no 256 x 256 tiles) and its modelled cost.
GemmPlan plan_small(int dtype, int M, int N, int K, int kind, double *cost_out) {
  GemmPlan best{};
  const int bk = dtype == kF32 ? 32 : 64;
  double best_cost = 0.0;
  const int ncfg = dtype == kF32 ? 1 : 6;
  for (int ci = 0; ci < ncfg; ++ci) {
    const int cfg = dtype == kF32 ? 5 : ci;
    const TileCfg tc = kTiles[cfg];
    for (int s = 1; s <= 16; ++s) {
      int kc = ceil_div(ceil_div(K, s), bk) * bk;
      const int splits = ceil_div(K, kc);
      if (splits != s) continue;                  // duplicate of a smaller split count
      if (splits > 1 && (kind == kEpiQKV || kind == kEpiSwiGLU)) break;  // fused RMSNorm needs all of K
      if (splits > 1 && kc < 4 * bk) break;       // keep at least four slabs per split
      if (splits > 1 && (long long)ceil_div(M, tc.bm) * ceil_div(N, tc.bn) * splits > kMaxSplitWGs) break;
      const bool bf = dtype == kBF16;
      const int wpc = bf && kind >= 0 && kind < 5 ? kRegTileWgsPerCU[cfg][kind] : 1;
      // the 128-row tiles run on the LDS-DMA kernel (remapped below); relative to the register-path
      // model of the same tile its cost is fitted as 0.9 for 128 x 192 and 128 x 128 (level for 128 x 64)
      const bool dma = bf && kind != kEpiPartial && K % 64 == 0 && kc % 64 == 0 && tc.bm == 128;
      const double dma_f = dma && tc.bn != 64 ? 0.9 : 1.0;
      double cost = plan_cost(tc.bm, tc.bn, M, N, K, splits, kc, wpc, dma_f);
      if (kind == kEpiPartial && splits > 1) cost -= 4200.0;  // partials are the output anyway
      if (best.bm == 0 || cost < best_cost) {
        best_cost = cost;
        best.cfg = cfg;
        best.bm = tc.bm;
        best.bn = tc.bn;
        best.splits = splits;
        best.k_split = kc;
      }
    }
  }
  // The 128-row tiles run on the LDS-DMA kernel (same tile and split); on the 64-row tiles it measured
  // level or slower.
  if (dtype == kBF16 && kind != kEpiPartial && K % 64 == 0 && best.k_split % 64 == 0) {
    for (int i = 0; i < kDmaTileCount; ++i)
      if (kDmaTiles[i][0] == best.bm && kDmaTiles[i][1] == best.bn) {
        best.cfg = kDmaCfg0 + i;
        break;
      }
  }
  // 128 x 96, a tile of the LDS-DMA kernel only (its MFMA waves take row quarters): with two row
  // tiles it fills the chip with 2 N / 96 workgroups where 128 x 128 leaves a quarter of it idle.
  // Fitted as the register-path model at factor 1.0 (measured on the llada QKV shape, M = 256:
  // 41.8 us against 46.1 for 128 x 128 and 43.6 for 64 x 192).
  if (dtype == kBF16 && kind != kEpiPartial && K % 64 == 0) {
    for (int s = 1; s <= 16; ++s) {
      const int kc = ceil_div(ceil_div(K, s), bk) * bk;
      const int splits = ceil_div(K, kc);
      if (splits != s) continue;
      if (splits > 1 && (kind == kEpiQKV || kind == kEpiSwiGLU)) break;
      if (splits > 1 && kc < 4 * bk) break;
      if (splits > 1 && (long long)ceil_div(M, 128) * ceil_div(N, 96) * splits > kMaxSplitWGs) break;
      double cost = plan_cost(128, 96, M, N, K, splits, kc, 1, 1.0);
      if (cost < best_cost) {
        best_cost = cost;
        best.cfg = kDmaCfg0 + 3;
        best.bm = 128;
        best.bn = 96;
        best.splits = splits;
        best.k_split = kc;
      }
    }
  }
  best.tiles_m = ceil_div(M, best.bm);
  best.tiles_n = ceil_div(N, best.bn);
  *cost_out = best_cost;
  return best;
}

// The large-M kernel (bf16, no split), 256 x 256 tiles: one 32-k slab per ~70 clocks when its tiles
// fit in one round, ~75 under full load (measured over M = 256 .. 8192, N = 3584 .. 37888); 192 x 256
// tiles take 0.82 of that per round (measured on the Dream gate/up, N = 37888, K = 3584: ~100 us for
// a round of 256 tiles against ~120).
double big_cost(int bm, int M, int N, int K) {
  const long long tiles = (long long)ceil_div(M, bm) * ceil_div(N, 256);
  return (double)ceil_div_ll(tiles, kCUs) * K * (tiles <= kCUs ? 70.0 : 75.0) * (bm == 256 ? 1.0 : 0.82);
}
}  // namespace

GemmPlan plan_gemm(int dtype, int M, int N, int K, int kind) {
  if (dtype == kBF16 && kind == kEpiPartial && N == kProxyCols && M <= 4096 && K % 64 == 0) {
    // the proxy kernel: about 256 workgroups, K split in whole 64-k slabs (measured: 1024 rows split
    // 8, 2048 rows split 4 fastest)
    GemmPlan p{};
    p.cfg = kProxyCfg;
    p.bm = kProxyRows;
    p.bn = kProxyCols;
    p.tiles_m = ceil_div(M, kProxyRows);
    p.tiles_n = 1;
    const int want = std::max(1, std::min(16, kCUs / p.tiles_m));
    p.k_split = ceil_div(ceil_div(K, want), 64) * 64;
    p.splits = ceil_div(K, p.k_split);
    return p;
  }
  double cost;
  GemmPlan best = plan_small(dtype, M, N, K, kind, &cost);
  if (dtype != kBF16 || kind == kEpiPartial) return best;
  for (const int bm : {256, 192}) {
    GemmPlan big{};
    big.cfg = bm == 256 ? kBigTileCfg : kBig192Cfg;
    big.bm = bm;
    big.bn = 256;
    big.splits = 1;
    big.k_split = K;
    big.tiles_m = ceil_div(M, bm);
    big.tiles_n = ceil_div(N, 256);
    // the large-M kernel wins once its tiles fill the chip
    const double c_big = big_cost(bm, M, N, K);
    if (c_big < cost) {
      best = big;
      cost = c_big;
    }
    // SwiGLU at up to two row tiles with a last round of tiles less than half full: the columns of the
    // whole rounds on the large-M kernel, the rest on the best smaller tile (measured on the Dream
    // gate/up at M = 512: 142 + 31 us against 210 for the best single launch, at M = 428 132 + 31
    // against 189; at M = 334 .. 384 192 x 256 rounds and the tail took 122-125 us against 151-155
    // for 256 x 256 rounds and the tail; at M = 2616 on the llada gate/up it measured level to 1.5%
    // slower, so larger M keep one launch)
    const long long tiles = (long long)big.tiles_m * big.tiles_n;
    if (kind == kEpiSwiGLU && big.tiles_m <= 2 && tiles > kCUs && tiles % kCUs < kCUs / 2) {
      const int tn0 = (int)((tiles / kCUs) * kCUs / big.tiles_m);  // tile columns of the whole rounds
      if (tn0 > 0 && tn0 < big.tiles_n) {
        const int n0 = tn0 * 256;
        double c_tail;
        plan_small(dtype, M, N - n0, K, kind, &c_tail);
        const double c_split = big_cost(bm, M, n0, K) + c_tail;
        if (c_split < cost) {
          best = big;
          best.tiles_n = tn0;
          best.n_main = n0;
          cost = c_split;
        }
      }
    }
  }
  return best;
}

GemmPlan gemm_tail_plan(int dtype, int M, int N, int K, int kind, const GemmPlan &p) {
  double c;
  return plan_small(dtype, M, N - p.n_main, K, kind, &c);
}

size_t gemm_partial_bytes(const GemmPlan &p, int M, int N) {
  return (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

template <typename T, int BM, int BN, int KIND>
static hipError_t run_gemm(const GemmPlan &p, const void *A, int lda, const void *W, int wkb, int M, int N,
                           int K, float *part, const EpiArgs &ea, hipStream_t s) {
  constexpr int PF = 4;
  const bool use_part = (KIND == kEpiPartial) || p.splits > 1;
  const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n * p.splits);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, KIND, PF>), dim3(grid), dim3(256), 0, s, (const T *)A, lda,
                     (const char *)W, wkb, M, N, K, p.tiles_m, p.tiles_n, p.k_split, use_part ? part : nullptr, ea);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || KIND == kEpiPartial || p.splits == 1) return err;
  const size_t work = (KIND == kEpiSwiGLU ? (size_t)M * ea.f : (size_t)M * N) / 8;
  const unsigned rgrid = (unsigned)((work + 255) / 256);
  hipLaunchKernelGGL((splitk_reduce_kernel<T, KIND>), dim3(rgrid), dim3(256), 0, s, part, p.splits, M, N, ea);
  return hipGetLastError();
}

template <int BM, int BN, int KIND>
static hipError_t run_dma(const GemmPlan &p, const void *A, int lda, const void *W, int wkb, int M, int N, int K,
                          float *part, const EpiArgs &ea, hipStream_t s) {
  if constexpr (KIND == kEpiPartial) {
    return hipErrorInvalidValue;
  } else {
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n * p.splits);
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, KIND>), dim3(grid), dim3(512), 0, s, (const bf16_t *)A, lda,
                       (const char *)W, wkb, M, N, K, p.tiles_m, p.tiles_n, p.k_split, p.splits > 1 ? part : nullptr,
                       ea);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || p.splits == 1) return err;
    const size_t work = (KIND == kEpiSwiGLU ? (size_t)M * ea.f : (size_t)M * N) / 8;
    const unsigned rgrid = (unsigned)((work + 255) / 256);
    hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, KIND>), dim3(rgrid), dim3(256), 0, s, part, p.splits, M, N, ea);
    return hipGetLastError();
  }
}

template <typename T, int KIND>
static hipError_t run_cfg(const GemmPlan &p, const void *A, int lda, const void *W, int wkb, int M, int N, int K,
                          float *part, const EpiArgs &ea, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    return run_gemm<T, 64, 64, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
  } else {
    switch (p.cfg) {
      case 0: return run_gemm<T, 128, 192, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case 1: return run_gemm<T, 64, 192, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case 2: return run_gemm<T, 128, 128, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case 3: return run_gemm<T, 128, 64, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case 4: return run_gemm<T, 64, 128, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case kBigTileCfg:
      case kBig192Cfg:
        if constexpr (KIND != kEpiPartial) {
          if (p.cfg == kBigTileCfg)
            hipLaunchKernelGGL((gemm_big_kernel<KIND, 256>), dim3((unsigned)(p.tiles_m * p.tiles_n)), dim3(256), 0, s,
                               (const bf16_t *)A, lda, (const char *)W, wkb, M, N, K, p.tiles_m, p.tiles_n, ea);
          else
            hipLaunchKernelGGL((gemm_big_kernel<KIND, 192>), dim3((unsigned)(p.tiles_m * p.tiles_n)), dim3(256), 0, s,
                               (const bf16_t *)A, lda, (const char *)W, wkb, M, N, K, p.tiles_m, p.tiles_n, ea);
          return hipGetLastError();
        }
        return hipErrorInvalidValue;
      case kDmaCfg0 + 0: return run_dma<128, 192, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case kDmaCfg0 + 1: return run_dma<128, 128, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case kDmaCfg0 + 2: return run_dma<128, 64, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      case kDmaCfg0 + 3: return run_dma<128, 96, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
      default: return run_gemm<T, 64, 64, KIND>(p, A, lda, W, wkb, M, N, K, part, ea, s);
    }
  }
}

template <typename T>
static hipError_t run_kind(int kind, const GemmPlan &p, const void *A, int lda, const void *W, int wkb, int M,
                           int N, int K, float *part, const EpiArgs &ea, hipStream_t s) {
  if (p.cfg == kProxyCfg) {
    if constexpr (sizeof(T) == 2) {
      if (kind != kEpiPartial || N != kProxyCols || p.tiles_m != ceil_div(M, kProxyRows) || p.k_split % 64 != 0 ||
          K % 64 != 0 || part == nullptr)
        return hipErrorInvalidValue;
      const unsigned grid = (unsigned)(p.tiles_m * p.splits);
      hipLaunchKernelGGL(proxy_gemm_kernel<4>, dim3(grid), dim3(256), 0, s, (const bf16_t *)A, lda, (const char *)W, wkb,
                         M, K, p.tiles_m, p.k_split, part, ea.ss_out, ea.clear, ea.clear_n);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
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
  if (plan.n_main > 0) {  // SwiGLU: whole rounds of large-M tiles, then the remaining columns
    const int n0 = plan.n_main;
    if (dtype != kBF16 || kind != kEpiSwiGLU || (plan.cfg != kBigTileCfg && plan.cfg != kBig192Cfg) || n0 % 256 != 0 || n0 >= N ||
        plan.tiles_n != n0 / 256)
      return hipErrorInvalidValue;
    GemmPlan pm = plan;
    pm.n_main = 0;
    hipError_t err = run_kind<bf16_t>(kind, pm, A, lda, W, wkb, M, n0, K, part, ea, s);
    if (err != hipSuccess) return err;
    const GemmPlan pt = gemm_tail_plan(dtype, M, N, K, kind, plan);
    EpiArgs et = ea;  // units n0 / 2 .. of Z: same rows, Z offset by n0 / 2 columns
    et.ldz = ea.ldz ? ea.ldz : ea.f;
    et.out = (bf16_t *)ea.out + n0 / 2;
    et.f = ea.f - n0 / 2;
    const char *wt = (const char *)W + (size_t)(n0 / 32) * wkb * 1024;  // weight column blocks n0 / 32 ..
    return run_kind<bf16_t>(kind, pt, A, lda, wt, wkb, M, N - n0, K, part, et, s);
  }
  if (dtype == kF32) return run_kind<float>(kind, plan, A, lda, W, wkb, M, N, K, part, ea, s);
  return run_kind<bf16_t>(kind, plan, A, lda, W, wkb, M, N, K, part, ea, s);
}

}  // namespace spa
