// Partial cached attention ([PN] 整体框架 Phase 2): the k queries of the update set attend,
// bidirectionally and without a mask, to all N keys of the (already scattered) K^c/V^c cache.
//
// One workgroup = one (sequence, query head, block of 32 QG queries). Its waves form QG query groups
// (32 queries each) x KR key ranges: the keys are split into KR contiguous ranges, each streamed in
// tiles of 32 keys through a double-buffered LDS stage that the QG waves of the range load together
// and all read, so every K/V byte fetched from L2 serves 32 QG queries. QG = 2 halves the L2 traffic
// of QG = 1 but halves the number of workgroups; the launcher takes QG = 2 unless that would leave CUs
// idle while QG = 1 fills them in one round. Each wave runs an online softmax over its range; the KR
// partial results (running max, running sum, unnormalised output) of a query group are merged through
// LDS at the end. K is staged as [key][hd] and V
// transposed to [hd][key], so that both products read contiguous LDS. A wave computes S^T = K Q^T
// (keys x queries) on 32x32 MFMA blocks; in that layout a lane holds the scores of one query, so the
// softmax (fp32, base-2 exponent) needs one cross-lane step, and the probabilities feed O^T = V^T P^T
// straight from registers. V is transposed on the way into LDS: a lane loads an 8-key x 8-dim block
// (eight 16-byte row pieces), transposes it in registers and writes eight 16-byte rows of V^T.
//
// Workgroup ids are remapped so that each XCD (which receives every eighth workgroup) runs a
// contiguous range of (sequence, KV head, query head, query block): the blocks that read the same K/V
// head share that XCD's L2, and HBM sees each head's K/V about once.
// Query head h reads KV head h / (H_q / H_kv) (grouped-query attention).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace spa {

template <bool BF16> struct AFrag;
template <> struct AFrag<true> { typedef u32x4 type; };
template <> struct AFrag<false> { typedef float type; };

// 8x8 transpose of 16-bit values held as 8 rows of 8 (u32x4 each): out[e] holds column e. Each output
// word takes one half-word from each of two rows: one v_perm_b32.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 *in, u32x4 *out) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of {row 2p, row 2p+1}
#pragma unroll
    for (int p = 0; p < 4; ++p) out[e][p] = __builtin_amdgcn_perm(in[2 * p + 1][w], in[2 * p][w], sel);
  }
}

template <typename T, int HD, int QG> struct AttnCfg {
  static constexpr int Q = 32 * QG;                                // queries per workgroup
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int KT = 32;                                    // keys per tile
  static constexpr int KROWB = HD * (int)sizeof(T) + 16;           // K tile row stride (bytes)
  static constexpr int VROWB = KT * (int)sizeof(T) + 16;           // V^T tile row stride (bytes)
  static constexpr int STAGE = KT * KROWB + HD * VROWB;            // one K + V^T tile
  // Shared stages (QG > 1) are double-buffered with a barrier per tile; a key range owned by a single
  // wave (QG = 1) has one private stage and needs no barrier (a wave's LDS accesses are in order).
  static constexpr int NBUF = QG > 1 ? 2 : 1;
  // key ranges: as many of 8, 4, 2 as fit in LDS, at most 8 waves per workgroup
  static constexpr int KR0 = 8 / QG;
  static constexpr int KR = NBUF * KR0 * STAGE <= 160 * 1024 ? KR0 : (NBUF * (KR0 / 2) * STAGE <= 160 * 1024 ? KR0 / 2 : KR0 / 4);
  static constexpr int W = QG * KR;                                // waves per workgroup
  static constexpr int PROWB = (HD + 4) * 4;                       // merge buffer row (fp32 O of a query)
  static constexpr int MERGE = 32 * PROWB + 32 * 8;                // one wave's partial state
  static constexpr int LDS = NBUF * KR * STAGE;
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int TPQ = (64 * W / Q) < (HD / VEC) ? (64 * W / Q) : (HD / VEC);  // merge threads per query
  static constexpr int SEG = HD / TPQ;                             // dims per merge thread
  static_assert(W * MERGE <= LDS && LDS <= 160 * 1024, "LDS budget");
  static_assert(SEG % VEC == 0, "whole 16-byte stores in the merge");
};

template <typename T, int HD, int QG>
__global__ __launch_bounds__((64 * AttnCfg<T, HD, QG>::W)) void attention_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc, T *__restrict__ o,
    int m_per_seq, int n_tok, int hq, int hkv, int qblocks, int nwg, float scale_log2) {
  typedef AttnCfg<T, HD, QG> C;
  constexpr int kAttnQG = QG, kAttnQueries = C::Q;
  constexpr bool BF = C::BF;
  constexpr int KT = C::KT, KR = C::KR;
  constexpr int KROWB = C::KROWB, VROWB = C::VROWB;
  constexpr int VEC = C::VEC;
  constexpr int KCH = KT * HD / VEC / (64 * kAttnQG);     // K 16-byte chunks per lane per tile
  // V: bf16 uses 8x8 blocks (8 key rows x one 16-byte chunk); fp32 uses 4x4 blocks
  constexpr int VB = BF ? 8 : 4;
  constexpr int VTASKS = (KT / VB) * (HD / VB);           // blocks per tile
  constexpr int VW = (VTASKS + kAttnQG - 1) / kAttnQG;    // blocks per wave of a key range
  constexpr int VPER = (VW + 63) / 64;
  constexpr int QSTEPS = BF ? HD / 16 : HD / 2;           // MFMA k-steps over the head dim
  constexpr int KSTEP_B = BF ? 32 : 8;
  constexpr int LANE_B = BF ? 16 : 4;
  constexpr int HB = HD / 32;                             // 32-row blocks of the head dim
  static_assert(KT * HD % (VEC * 64 * kAttnQG) == 0, "K tile load split");
  typedef typename AFrag<BF>::type FragT;

  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  // XCD-aware order: hardware hands workgroup i to XCD i % 8
  const int nb = gridDim.x;
  const int lid = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (lid >= nwg) return;  // grid padding (whole workgroup, before any barrier)
  const int grp = hq / hkv;
  const int qb = lid % qblocks;
  int rest = lid / qblocks;
  const int h_in = rest % grp;
  rest /= grp;
  const int g = rest % hkv;
  const int b = rest / hkv;
  const int h = g * grp + h_in;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qg = wave % kAttnQG, kr = wave / kAttnQG;
  const int m0 = qb * kAttnQueries + qg * 32;
  const int ldq = hq * HD;
  auto stage = [&](int buf) { return smem + ((C::NBUF > 1 ? buf : 0) * KR + kr) * C::STAGE; };

  // Q fragments: B operand of S^T = K Q^T (column = query lane%32, k = head dim).
  FragT qf[QSTEPS];
  {
    const int qrow = min(m0 + (lane & 31), m_per_seq - 1);
    const T *qp = q + ((size_t)b * m_per_seq + qrow) * ldq + (size_t)h * HD;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) {
      if constexpr (BF)
        qf[st] = ld16(qp + st * 16 + (lane >> 5) * 8);
      else
        qf[st] = qp[st * 2 + (lane >> 5)];
    }
  }

  const size_t head_off = ((size_t)b * hkv + g) * (size_t)n_tok * HD;
  const T *kbase = kc + head_off;
  const T *vbase = vc + head_off;

  floatx16 oacc[HB];
#pragma unroll
  for (int i = 0; i < HB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  // Key range kr covers tiles [kr * tper, (kr + 1) * tper); every wave runs tper tiles (a barrier per
  // tile), tiles past the end are clamped loads whose keys are all masked.
  const int ntiles = (n_tok + KT - 1) / KT;
  const int tper = (ntiles + KR - 1) / KR;
  const int t_begin = kr * tper;

  // The QG waves of a key range split the tile loads: K chunks lane + 64 (j * QG + qg); V blocks
  // qg * VW + lane + 64 p, block v -> key block kb = v % (KT / VB), dim chunk cc = v / (KT / VB), so
  // the lanes that write one V^T row segment hold consecutive key blocks (conflict-free LDS).
  u32x4 rk[KCH], rv[VPER][VB];
  // This lane's element offsets inside a tile (constant over the tiles): K chunk j covers key row
  // c / (HD / VEC), chunk c % (HD / VEC); V block p covers keys kb VB .. kb VB + VB - 1 of dim chunk cc.
  // (row = offset / HD, column = offset % HD: HD is a power of two)
  int koff[KCH], voff[VPER];
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int c = lane + 64 * (j * kAttnQG + qg);
    koff[j] = (c / (HD / VEC)) * HD + (c % (HD / VEC)) * VEC;
  }
#pragma unroll
  for (int p = 0; p < VPER; ++p) {
    const int v = min(qg * VW + min(lane + 64 * p, VW - 1), VTASKS - 1);
    const int kb = v % (KT / VB), cc = v / (KT / VB);
    voff[p] = kb * VB * HD + cc * VB;
  }
  auto gload = [&](int t) {
    const int key0 = t * KT;
    // tile base (uniform across the wave) + the lane's offset: no per-load address arithmetic
    const T *kt = kbase + (size_t)key0 * HD;
    const T *vt = vbase + (size_t)key0 * HD;
    if (key0 + KT <= n_tok) {  // uniform: the whole tile lies inside the keys
#pragma unroll
      for (int j = 0; j < KCH; ++j) rk[j] = ld16(kt + koff[j]);
#pragma unroll
      for (int p = 0; p < VPER; ++p)
#pragma unroll
        for (int j = 0; j < VB; ++j) rv[p][j] = ld16(vt + voff[p] + j * HD);
    } else {  // a tile reaching past the last key (or wholly past it, in a short key range): rows past
              // the end read the last key and are masked later
#pragma unroll
      for (int j = 0; j < KCH; ++j) {
        const int key = min(key0 + koff[j] / HD, n_tok - 1);
        rk[j] = ld16(kbase + (size_t)key * HD + koff[j] % HD);
      }
#pragma unroll
      for (int p = 0; p < VPER; ++p)
#pragma unroll
        for (int j = 0; j < VB; ++j) {
          const int key = min(key0 + voff[p] / HD + j, n_tok - 1);
          rv[p][j] = ld16(vbase + (size_t)key * HD + voff[p] % HD);
        }
    }
  };
  auto lstore = [&](int buf) {
    char *ks = stage(buf), *vts = ks + KT * KROWB;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = lane + 64 * (j * kAttnQG + qg);
      const int row = c / (HD / VEC), col = c % (HD / VEC);
      st16(ks + row * KROWB + col * 16, rk[j]);
    }
#pragma unroll
    for (int p = 0; p < VPER; ++p) {
      const int vi = lane + 64 * p, v = qg * VW + vi;
      if (vi >= VW || v >= VTASKS) continue;
      const int kb = v % (KT / VB), cc = v / (KT / VB);
      if constexpr (BF) {
        u32x4 tr[8];
        transpose8x8_b16(rv[p], tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) st16(vts + (cc * 8 + e) * VROWB + kb * 16, tr[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u32x4 col = {rv[p][0][e], rv[p][1][e], rv[p][2][e], rv[p][3][e]};
          st16(vts + (cc * 4 + e) * VROWB + kb * 16, col);
        }
      }
    }
  };

  // MASKED: the tile reaches past the last key (only the last tile of a range can)
  auto compute = [&](int t, int buf, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const char *ks = stage(buf), *vts = ks + KT * KROWB;
    // S^T block of 32 keys: lane holds query lane%32 and keys 8*(r/4) + 4*(lane/32) + r%4, r = 0..15;
    // two independent MFMA chains over the even and odd head-dim steps
    floatx16 s, s2;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = s2[r] = 0.f;
    const char *krow = ks + (lane & 31) * KROWB + (lane >> 5) * LANE_B;
#pragma unroll
    for (int st = 0; st < QSTEPS; st += 2) {
      s = mfma32(*reinterpret_cast<const FragT *>(krow + st * KSTEP_B), qf[st], s);
      s2 = mfma32(*reinterpret_cast<const FragT *>(krow + (st + 1) * KSTEP_B), qf[st + 1], s2);
    }
    s += s2;
    // raw scores; the softmax scale (and log2 e) is applied inside one FMA per score
    if constexpr (MASKED) {  // keys past the end score -inf
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t * KT + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (key >= n_tok) s[r] = -INFINITY;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)) * scale_log2;
    // The exponentials are taken against a reference maximum mref that moves only when a query's
    // maximum exceeds it by more than 8 (so every p <= 2^8, safe in fp32 and in the bf16 P): the
    // running sums are rescaled rarely instead of on most tiles, and the result is the same softmax.
    const float mnew = fmaxf(mrun, tmax);
    const bool grow = mnew > mrun + 8.f;  // false while no key was seen (-inf)
    if (__any(grow)) {
      const float mto = grow ? mnew : mrun;
      // 1 for queries that keep their reference, 0 from -inf (sums still empty)
      const float alpha = mto == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mto);
      lrun *= alpha;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) oacc[hb] *= alpha;
      mrun = mto;
    }
    const float msub = mrun == -INFINITY ? 0.f : mrun;  // no key seen yet: every p is 0
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // hardware 2^x: results below 2^-126 (of a row whose largest p is >= 1) flush to 0
      const float p = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -msub));
      s[r] = p;
      psum += p;
    }
    lrun += psum;

    // O^T += V^T P^T. In k-step `half` lane group G = lane/32 supplies its scores r = half*8..
    // half*8+7, i.e. keys half*16 + {4G..4G+3, 8+4G..8+4G+3}; A = V^T rows at those keys.
    const int G = lane >> 5;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if constexpr (BF) {
        u32x4 pf;
        pf[0] = pack_bf16x2(s[half * 8 + 0], s[half * 8 + 1]);
        pf[1] = pack_bf16x2(s[half * 8 + 2], s[half * 8 + 3]);
        pf[2] = pack_bf16x2(s[half * 8 + 4], s[half * 8 + 5]);
        pf[3] = pack_bf16x2(s[half * 8 + 6], s[half * 8 + 7]);
        const int c0 = (half * 16 + 4 * G) * 2, c1 = c0 + 16;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const char *vrow = vts + (hb * 32 + (lane & 31)) * VROWB;
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + c0);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + c1);
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
          oacc[hb] = mfma32(vf, pf, oacc[hb]);
        }
      } else {
        // fp32 MFMA takes one key per lane group: MFMA r covers keys of score r for G = 0 and 1
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = half * 8 + i;
          const int key = (r >> 2) * 8 + G * 4 + (r & 3);
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            const float vf = *reinterpret_cast<const float *>(vts + (hb * 32 + (lane & 31)) * VROWB + key * 4);
            oacc[hb] = mfma32(vf, s[r], oacc[hb]);
          }
        }
      }
    }
  };

  // Tile i + 1 is loaded into registers during tile i and written to the (other) stage after it; with
  // shared stages one barrier per tile (every wave runs the same tper tiles).
  gload(t_begin);
  lstore(0);
  gload(t_begin + 1);
  if constexpr (QG > 1) __syncthreads();
  for (int i = 0; i < tper; ++i) {
    const int t = t_begin + i;
    if (t * KT + KT > n_tok)
      compute(t, i & 1, std::true_type());
    else
      compute(t, i & 1, std::false_type());
    if (i + 1 < tper) {
      lstore((i + 1) & 1);
      gload(t_begin + i + 2);
    }
    if constexpr (QG > 1) __syncthreads();
  }
  if constexpr (QG == 1) __syncthreads();  // the merge below overwrites other waves' stages

  // Merge the key ranges of each query group. Every wave parks its partial state in LDS (the stages
  // are free after the last barrier), then all threads combine.
  lrun += __shfl_xor(lrun, 32, kWave);
  {
    char *part = smem + wave * C::MERGE;
    const int G = lane >> 5;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<floatx4 *>(part + (lane & 31) * C::PROWB + (hb * 32 + r4 * 8 + G * 4) * 4) =
            floatx4{oacc[hb][r4 * 4 + 0], oacc[hb][r4 * 4 + 1], oacc[hb][r4 * 4 + 2], oacc[hb][r4 * 4 + 3]};
    if (lane < 32) {
      float *ml = reinterpret_cast<float *>(part + 32 * C::PROWB);
      ml[2 * lane] = mrun;
      ml[2 * lane + 1] = lrun;
    }
  }
  __syncthreads();
  {
    constexpr int SEG = C::SEG, TPQ = C::TPQ;
    const int qi = tid / TPQ, d0 = (tid % TPQ) * SEG;  // query qi of the block: group qi / 32
    if (qi >= kAttnQueries) return;                    // after the last barrier
    const int gq = qi >> 5, ql = qi & 31;
    float mw[KR], lw[KR];
    float mmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const float *ml = reinterpret_cast<const float *>(smem + (r * kAttnQG + gq) * C::MERGE + 32 * C::PROWB);
      mw[r] = ml[2 * ql];
      lw[r] = ml[2 * ql + 1];
      mmax = fmaxf(mmax, mw[r]);
    }
    float aw[KR], lsum = 0.f;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      aw[r] = mw[r] == -INFINITY ? 0.f : exp2f(mw[r] - mmax);  // a range without keys adds nothing
      lsum = fmaf(aw[r], lw[r], lsum);
    }
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int r = 0; r < KR; ++r) aw[r] *= inv;
    float acc[SEG];
#pragma unroll
    for (int e = 0; e < SEG; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const char *row = smem + (r * kAttnQG + gq) * C::MERGE + ql * C::PROWB + d0 * 4;
#pragma unroll
      for (int e = 0; e < SEG; e += 4) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(row + e * 4);
        acc[e] = fmaf(aw[r], v[0], acc[e]);
        acc[e + 1] = fmaf(aw[r], v[1], acc[e + 1]);
        acc[e + 2] = fmaf(aw[r], v[2], acc[e + 2]);
        acc[e + 3] = fmaf(aw[r], v[3], acc[e + 3]);
      }
    }
    const int qo = qb * kAttnQueries + qi;
    if (qo < m_per_seq) {
      T *dst = o + ((size_t)b * m_per_seq + qo) * ldq + (size_t)h * HD + d0;
#pragma unroll
      for (int e = 0; e < SEG; e += VEC) {
        if constexpr (BF)
          st16(dst + e, pack16(acc + e, (const bf16_t *)nullptr));
        else
          st16(dst + e, pack16(acc + e, (const float *)nullptr));
      }
    }
  }
}

// Many sparse queries per head (bf16): one workgroup = (sequence, query head, block of 256 queries),
// four waves of 64 queries each (two 32-query MFMA column blocks). All four waves stream every key of
// the head through a double-buffered stage that they load together (one barrier per 32-key tile), so
// each K/V byte fetched from L2 serves 256 queries, and each K or V^T fragment read from LDS feeds
// two MFMAs (one per query block): half the LDS bytes per MFMA of the 32-query waves. No key split,
// hence no merge: the softmax state stays in the wave and the output is normalised in place.
template <int HD> struct WideAttnCfg {
  static constexpr int QPW = 64, W = 4, Q = QPW * W;               // queries per wave / per workgroup
  static constexpr int KT = 32;                                    // keys per tile
  static constexpr int KROWB = HD * 2 + 16, VROWB = KT * 2 + 16;   // K row / V^T row strides (bytes)
  static constexpr int STAGE = KT * KROWB + HD * VROWB;
  static constexpr int OROWB = (HD + 4) * 4;                       // staged fp32 output row
  static constexpr int OUT = W * QPW * OROWB;
  static constexpr int LDS = 2 * STAGE > OUT ? 2 * STAGE : OUT;
  static constexpr int KCH = KT * HD / 8 / (64 * W);               // K 16-byte chunks per lane per tile
  static constexpr int VTASKS = (KT / 8) * (HD / 8);               // 8x8 V blocks per tile
  static constexpr int VW = VTASKS / W;                            // per wave (one per lane < VW)
  static_assert(KCH >= 1 && KT * HD / 8 % (64 * W) == 0 && VTASKS % W == 0 && VW <= 64, "tile split");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int HD>
__global__ __launch_bounds__(256) void attention_wide_kernel(const bf16_t *__restrict__ q,
                                                             const bf16_t *__restrict__ kc,
                                                             const bf16_t *__restrict__ vc, bf16_t *__restrict__ o,
                                                             int m_per_seq, int n_tok, int hq, int hkv, int qblocks,
                                                             int nwg, float scale_log2) {
  typedef bf16_t T;
  typedef WideAttnCfg<HD> C;
  constexpr int KT = C::KT, KROWB = C::KROWB, VROWB = C::VROWB, KCH = C::KCH, VW = C::VW;
  constexpr int QSTEPS = HD / 16, HB = HD / 32;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int nb = gridDim.x;
  const int lid = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (lid >= nwg) return;  // grid padding (whole workgroup, before any barrier)
  const int grp = hq / hkv;
  const int qb = lid % qblocks;
  int rest = lid / qblocks;
  const int h_in = rest % grp;
  rest /= grp;
  const int g = rest % hkv;
  const int b = rest / hkv;
  const int h = g * grp + h_in;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = qb * C::Q + wave * C::QPW;  // this wave's queries m0 .. m0 + 63
  const int ldq = hq * HD;
  auto stage = [&](int buf) { return smem + buf * C::STAGE; };

  // Q fragments of both query blocks: B operand of S^T = K Q^T (column = query lane % 32)
  u32x4 qf[2][QSTEPS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qrow = min(m0 + 32 * j + (lane & 31), m_per_seq - 1);
    const T *qp = q + ((size_t)b * m_per_seq + qrow) * ldq + (size_t)h * HD;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) qf[j][st] = ld16(qp + st * 16 + (lane >> 5) * 8);
  }

  const size_t head_off = ((size_t)b * hkv + g) * (size_t)n_tok * HD;
  const T *kbase = kc + head_off;
  const T *vbase = vc + head_off;

  floatx16 oacc[2][HB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < HB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[j][i][r] = 0.f;
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};

  // tile loads split over the four waves: K chunks c = lane + 64 (4 jj + wave); V block v = VW wave + lane
  u32x4 rk[KCH], rv[8];
  int koff[KCH];
#pragma unroll
  for (int jj = 0; jj < KCH; ++jj) {
    const int c = lane + 64 * (jj * C::W + wave);
    koff[jj] = (c / (HD / 8)) * HD + (c % (HD / 8)) * 8;
  }
  const bool vlane = lane < VW;
  const int vtask = wave * VW + (vlane ? lane : 0);
  const int vkb = vtask % (KT / 8), vcc = vtask / (KT / 8);
  const int voff = vkb * 8 * HD + vcc * 8;
  auto gload = [&](int t) {
    const int key0 = t * KT;
    if (key0 + KT <= n_tok) {
      const T *kt = kbase + (size_t)key0 * HD;
      const T *vt = vbase + (size_t)key0 * HD;
#pragma unroll
      for (int jj = 0; jj < KCH; ++jj) rk[jj] = ld16(kt + koff[jj]);
      if (vlane) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rv[e] = ld16(vt + voff + e * HD);
      }
    } else {  // rows past the last key read the last key (masked later)
#pragma unroll
      for (int jj = 0; jj < KCH; ++jj) {
        const int key = min(key0 + koff[jj] / HD, n_tok - 1);
        rk[jj] = ld16(kbase + (size_t)key * HD + koff[jj] % HD);
      }
      if (vlane) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = min(key0 + voff / HD + e, n_tok - 1);
          rv[e] = ld16(vbase + (size_t)key * HD + voff % HD);
        }
      }
    }
  };
  auto lstore = [&](int buf) {
    char *ks = stage(buf), *vts = ks + KT * KROWB;
#pragma unroll
    for (int jj = 0; jj < KCH; ++jj) {
      const int c = lane + 64 * (jj * C::W + wave);
      st16(ks + (c / (HD / 8)) * KROWB + (c % (HD / 8)) * 16, rk[jj]);
    }
    if (vlane) {
      u32x4 tr[8];
      transpose8x8_b16(rv, tr);
#pragma unroll
      for (int e = 0; e < 8; ++e) st16(vts + (vcc * 8 + e) * VROWB + vkb * 16, tr[e]);
    }
  };

  // S^T = K Q^T of the tile in stage buf, both query blocks (each K fragment feeds two MFMAs)
  auto qk = [&](int buf, floatx16 (&s)[2]) {
    const char *krow = stage(buf) + (lane & 31) * KROWB + (lane >> 5) * 16;
#pragma unroll
    for (int jq = 0; jq < 2; ++jq)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[jq][r] = 0.f;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) {
      const u32x4 kf = *reinterpret_cast<const u32x4 *>(krow + st * 32);
      s[0] = mfma32(kf, qf[0][st], s[0]);
      s[1] = mfma32(kf, qf[1][st], s[1]);
    }
  };
  // Online softmax of tile t in place (scores -> probabilities). masked: the tile reaches past the
  // last key (a runtime branch: two inlined variants would not fit the register file).
  auto softmax = [&](int t, floatx16 (&s)[2], bool masked) {
#pragma unroll
    for (int jq = 0; jq < 2; ++jq) {
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * KT + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          if (key >= n_tok) s[jq][r] = -INFINITY;
        }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[jq][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)) * scale_log2;
      // reference maximum that moves only when a query's maximum exceeds it by more than 8 (p <= 2^8)
      const float mnew = fmaxf(mrun[jq], tmax);
      const bool grow = mnew > mrun[jq] + 8.f;
      if (__any(grow)) {
        const float mto = grow ? mnew : mrun[jq];
        const float alpha = mto == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun[jq] - mto);
        lrun[jq] *= alpha;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) oacc[jq][hb] *= alpha;
        mrun[jq] = mto;
      }
      const float msub = mrun[jq] == -INFINITY ? 0.f : mrun[jq];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[jq][r], scale_log2, -msub));
        s[jq][r] = p;
        psum += p;
      }
      lrun[jq] += psum;
    }
  };
  // O^T += V^T P^T from the tile in stage buf, each V^T fragment shared by the two query blocks
  auto pv = [&](int buf, const floatx16 (&s)[2]) {
    const char *vts = stage(buf) + KT * KROWB;
    const int G = lane >> 5;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 pf[2];
#pragma unroll
      for (int jq = 0; jq < 2; ++jq) {
        pf[jq][0] = pack_bf16x2(s[jq][half * 8 + 0], s[jq][half * 8 + 1]);
        pf[jq][1] = pack_bf16x2(s[jq][half * 8 + 2], s[jq][half * 8 + 3]);
        pf[jq][2] = pack_bf16x2(s[jq][half * 8 + 4], s[jq][half * 8 + 5]);
        pf[jq][3] = pack_bf16x2(s[jq][half * 8 + 6], s[jq][half * 8 + 7]);
      }
      const int c0 = (half * 16 + 4 * G) * 2, c1 = c0 + 16;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const char *vrow = vts + (hb * 32 + (lane & 31)) * VROWB;
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + c0);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + c1);
        const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
        oacc[0][hb] = mfma32(vf, pf[0], oacc[0][hb]);
        oacc[1][hb] = mfma32(vf, pf[1], oacc[1][hb]);
      }
    }
  };

  const int ntiles = (n_tok + KT - 1) / KT;
  gload(0);
  lstore(0);
  gload(1);
  __syncthreads();
  for (int i = 0; i < ntiles; ++i) {
    floatx16 s[2];
    qk(i & 1, s);
    softmax(i, s, i * KT + KT > n_tok);
    pv(i & 1, s);
    if (i + 1 < ntiles) {
      lstore((i + 1) & 1);
      gload(i + 2);
    }
    __syncthreads();  // tile i + 1 stored; tile i read by every wave (its buffer is refilled next)
  }

  // Normalise and stage this wave's 64 x HD outputs row-major in its own LDS region (the stages are
  // free after the last barrier), then write whole 16-byte rows pieces.
  char *ob = smem + wave * C::QPW * C::OROWB;
  const int G = lane >> 5;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float l = lrun[j] + __shfl_xor(lrun[j], 32, kWave);
    const float inv = 1.0f / l;
    char *orow = ob + (32 * j + (lane & 31)) * C::OROWB;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<floatx4 *>(orow + (hb * 32 + r4 * 8 + G * 4) * 4) =
            floatx4{oacc[j][hb][r4 * 4 + 0] * inv, oacc[j][hb][r4 * 4 + 1] * inv, oacc[j][hb][r4 * 4 + 2] * inv,
                    oacc[j][hb][r4 * 4 + 3] * inv};
  }
  // the wave reads back only what it wrote (in-order LDS within a wave)
#pragma unroll
  for (int it = 0; it < C::QPW * HD / 8 / 64; ++it) {
    const int c = lane + 64 * it;
    const int ql = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
    const int qo = m0 + ql;
    if (qo < m_per_seq) {
      const float *src = reinterpret_cast<const float *>(ob + ql * C::OROWB) + d0;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = src[e];
      st16(o + ((size_t)b * m_per_seq + qo) * ldq + (size_t)h * HD + d0, pack16(v, (const bf16_t *)nullptr));
    }
  }
}

template <int HD>
static hipError_t launch_wide(const void *q, const void *kc, const void *vc, void *o, int batch, int m_per_seq,
                              int n_tok, int hq, int hkv, hipStream_t s) {
  typedef WideAttnCfg<HD> C;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  const int qblocks = (m_per_seq + C::Q - 1) / C::Q;
  const long long nwg = (long long)qblocks * hq * batch;
  if (nwg > (1LL << 30)) return hipErrorInvalidValue;
  const int grid = (int)((nwg + 7) / 8 * 8);
  hipLaunchKernelGGL((attention_wide_kernel<HD>), dim3(grid), dim3(256), 0, s, (const bf16_t *)q,
                     (const bf16_t *)kc, (const bf16_t *)vc, (bf16_t *)o, m_per_seq, n_tok, hq, hkv, qblocks,
                     (int)nwg, scale_log2);
  return hipGetLastError();
}

template <typename T, int HD, int QG>
static hipError_t launch_qg(const void *q, const void *kc, const void *vc, void *o, int batch, int m_per_seq,
                            int n_tok, int hq, int hkv, hipStream_t s) {
  typedef AttnCfg<T, HD, QG> C;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  const int qblocks = (m_per_seq + C::Q - 1) / C::Q;
  const long long nwg = (long long)qblocks * hq * batch;
  if (nwg > (1LL << 30)) return hipErrorInvalidValue;
  const int grid = (int)((nwg + 7) / 8 * 8);
  hipLaunchKernelGGL((attention_kernel<T, HD, QG>), dim3(grid), dim3(64 * C::W), 0, s, (const T *)q,
                     (const T *)kc, (const T *)vc, (T *)o, m_per_seq, n_tok, hq, hkv, qblocks, (int)nwg,
                     scale_log2);
  return hipGetLastError();
}

template <typename T, int HD>
static hipError_t run_attention(const void *q, const void *kc, const void *vc, void *o, int batch, int m_per_seq,
                                int n_tok, int hq, int hkv, hipStream_t s) {
  constexpr int kCUs = 256;
  const long long heads = (long long)hq * batch;
  if constexpr (sizeof(T) == 2) {
    // The 256-query kernel once it fills the chip and its query blocks are at least 3/4 full: measured
    // at B = 8, N = 4096, 32 heads, 1024 and 656 queries per sequence 0.84 and 0.91 of the time of the
    // kernel below, at 328 queries (blocks 64% full) 1.08.
    const long long qb256 = (m_per_seq + 255) / 256;
    if (heads * qb256 >= kCUs && 4LL * m_per_seq >= 3LL * 256 * qb256)
      return launch_wide<HD>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  }
  const long long wg64 = heads * ((m_per_seq + 63) / 64), wg32 = heads * ((m_per_seq + 31) / 32);
  if (wg64 < kCUs && wg32 <= kCUs) return launch_qg<T, HD, 1>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  return launch_qg<T, HD, 2>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
}

hipError_t launch_attention(int dtype, const void *q, const void *kc, const void *vc, void *o, int batch,
                            int m_per_seq, int n_tok, int hq, int hkv, int hd, hipStream_t s) {
  if (m_per_seq <= 0 || batch <= 0) return hipSuccess;
  if (dtype == kBF16) {
    if (hd == 128) return run_attention<bf16_t, 128>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
    return run_attention<bf16_t, 64>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  }
  if (hd == 128) return run_attention<float, 128>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  return run_attention<float, 64>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
}

}  // namespace spa
