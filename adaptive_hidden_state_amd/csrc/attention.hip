// Partial cached attention ([PN] 整体框架 Phase 2): the k queries of the update set attend,
// bidirectionally and without a mask, to all N keys of the (already scattered) K^c/V^c cache.
//
// One workgroup = one (sequence, query head, block of 32 QG queries). Its waves form QG query groups
// (32 queries each) x KR key ranges: the keys are split into KR contiguous ranges, each streamed in
// tiles of 32 keys through LDS (QG = 1: one stage private to the range's wave; QG = 2: a
// double-buffered stage that the two waves of the range load together and both read), so every K/V
// byte fetched from L2 serves 32 QG queries. QG = 2 halves the L2 traffic
// of QG = 1 but halves the number of workgroups; the launcher takes QG = 2 unless that would leave CUs
// idle while QG = 1 fills them in one round. Each wave runs an online softmax over its range; the KR
// partial results (running max, running sum, unnormalised output) of a query group are merged through
// LDS at the end. K and (bf16) V are staged as [key][hd] rows, copied as loaded. A wave computes
// S^T = K Q^T (keys x queries) on 32x32 MFMA blocks; in that layout a lane holds the scores of one
// query, so the softmax (fp32, base-2 exponent) needs one cross-lane step, and the probabilities feed
// O^T = V^T P^T straight from registers. The V^T operand of that product (eight keys of one head dim
// per lane) comes out of the [key][hd] rows through the LDS transpose read (ds_read_b64_tr_b16: in
// each group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces that lanes i / 4,
// i / 4 + 4, i / 4 + 8 and i / 4 + 12 address), two reads per fragment. fp32 V is transposed on the
// way into LDS instead: a lane loads a 4-key x 4-dim block and writes four 16-byte rows of V^T.
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

// ds_read_b64_tr_b16 at byte address p of LDS (see the kernel comment for its lane layout).
__device__ __forceinline__ u32x2 lds_read_tr16(const char *p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s *)(__attribute__((address_space(3))) const char *)p);
  return __builtin_bit_cast(u32x2, r);
}

template <typename T, int HD, int QG> struct AttnCfg {
  static constexpr int Q = 32 * QG;                                // queries per workgroup
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int KT = 32;                                    // keys per tile
  static constexpr int KROWB = HD * (int)sizeof(T) + 16;           // K tile row stride (bytes)
  // bf16: V stays [key][hd] (rows padded by 64 bytes, so the four keys of a transposed fragment read
  // sit on disjoint banks); fp32: V^T [hd][key]
  static constexpr int VROWB = BF ? HD * 2 + 64 : KT * (int)sizeof(T) + 16;
  static constexpr int STAGE = KT * KROWB + (BF ? KT : HD) * VROWB;  // one K + V tile
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
  // fp32 V goes in as 4-key x 4-dim blocks (transposed on the way into LDS); bf16 V rows take the K
  // chunk mapping, and the block constants below are unused for it
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
  const int ldq = hq * HD;
  auto stage = [&](int buf) { return smem + ((C::NBUF > 1 ? buf : 0) * KR + kr) * C::STAGE; };

  FragT qf[QSTEPS];  // Q fragments (filled below, once the first tile's loads are out)
  const size_t head_off = ((size_t)b * hkv + g) * (size_t)n_tok * HD;
  const T *kbase = kc + head_off;
  const T *vbase = vc + head_off;

  floatx16 oacc[HB];
#pragma unroll
  for (int i = 0; i < HB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  // Key range kr covers tiles [kr * tper, (kr + 1) * tper); every wave runs tper tiles (with a barrier
  // per tile when the stage is shared), tiles past the end are clamped loads whose keys are all masked.
  const int ntiles = (n_tok + KT - 1) / KT;
  const int tper = (ntiles + KR - 1) / KR;
  const int t_begin = kr * tper;

  // The QG waves of a key range split the tile loads: K (and bf16 V) chunks c = lane + 64 (j QG + qg),
  // i.e. key row krow0 + KRS j, 16-byte chunk kcol0 of the row (64 QG chunks are KRS whole rows, so
  // the offsets of a lane's chunks differ by constants); fp32 V blocks qg * VW + lane + 64 p, block
  // v -> key block kb = v % (KT / VB), dim chunk cc = v / (KT / VB), so the lanes that write one V^T
  // row segment hold consecutive key blocks (conflict-free LDS).
  u32x4 rk[KCH], rvr[BF ? KCH : 1], rv[BF ? 1 : VPER][VB];  // K rows; V rows (bf16) or V blocks (fp32)
  constexpr int KRS = 64 * kAttnQG / (HD / VEC);
  static_assert(64 * kAttnQG % (HD / VEC) == 0, "whole rows per load pass");
  const int krow0 = (lane + 64 * qg) / (HD / VEC), kcol0 = (lane + 64 * qg) % (HD / VEC);
  const int koff0 = krow0 * HD + kcol0 * VEC;  // element offset of chunk j = 0 in a tile
  // fp32 V block p covers keys kb VB .. kb VB + VB - 1 of dim chunk cc (element offset voff[p])
  int voff[VPER];
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
      for (int j = 0; j < KCH; ++j) rk[j] = ld16(kt + koff0 + j * KRS * HD);
      if constexpr (BF) {
#pragma unroll
        for (int j = 0; j < KCH; ++j) rvr[j] = ld16(vt + koff0 + j * KRS * HD);
      } else {
#pragma unroll
        for (int p = 0; p < VPER; ++p)
#pragma unroll
          for (int j = 0; j < VB; ++j) rv[p][j] = ld16(vt + voff[p] + j * HD);
      }
    } else {  // a tile reaching past the last key (or wholly past it, in a short key range): rows past
              // the end read the last key and are masked later
#pragma unroll
      for (int j = 0; j < KCH; ++j) {
        const int key = min(key0 + krow0 + j * KRS, n_tok - 1);
        rk[j] = ld16(kbase + (size_t)key * HD + kcol0 * VEC);
        if constexpr (BF) rvr[j] = ld16(vbase + (size_t)key * HD + kcol0 * VEC);
      }
      if constexpr (!BF) {
#pragma unroll
        for (int p = 0; p < VPER; ++p)
#pragma unroll
          for (int j = 0; j < VB; ++j) {
            const int key = min(key0 + voff[p] / HD + j, n_tok - 1);
            rv[p][j] = ld16(vbase + (size_t)key * HD + voff[p] % HD);
          }
      }
    }
  };
  auto lstore = [&](int buf) {
    char *ks = stage(buf), *vts = ks + KT * KROWB;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      st16(ks + (krow0 + j * KRS) * KROWB + kcol0 * 16, rk[j]);
      if constexpr (BF) st16(vts + (krow0 + j * KRS) * VROWB + kcol0 * 16, rvr[j]);
    }
    if constexpr (!BF) {
#pragma unroll
      for (int p = 0; p < VPER; ++p) {
        const int vi = lane + 64 * p, v = qg * VW + vi;
        if (vi >= VW || v >= VTASKS) continue;
        const int kb = v % (KT / VB), cc = v / (KT / VB);
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
    tmax = fmaxf(tmax, xor_lane<32>(tmax)) * scale_log2;
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
        // A = V^T: lane l needs head dim hb 32 + l % 32 at keys half 16 + {4G..4G+3} (elements 0..3)
        // and half 16 + 8 + {4G..4G+3} (4..7). In the transpose read, lane j of 16-lane group g
        // addresses key half 16 + 4 (g / 2) + j / 4 (+ 8 for the second read), dims 16 (g % 2) +
        // 4 (j % 4) .. + 3, so lane i of the group receives dim 16 (g % 2) + i at the four keys.
        const int tg = lane >> 4, tj = lane & 15;
        const char *vrd = vts + (half * 16 + 4 * (tg >> 1) + (tj >> 2)) * VROWB + (16 * (tg & 1) + 4 * (tj & 3)) * 2;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const u32x2 lo = lds_read_tr16(vrd + hb * 64);
          const u32x2 hi = lds_read_tr16(vrd + hb * 64 + 8 * VROWB);
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

  // Q fragments: B operand of S^T = K Q^T (column = query lane%32, k = head dim). The KR waves of a
  // query group need the same fragments: the workgroup loads its Q block from memory once, each thread
  // a share of its 16-byte chunks, into LDS (rows of QROWB bytes at the start of the stage area, free
  // until the first tile store), and every wave reads its fragments from there. The first tile's loads
  // go out before the Q block lands.
  constexpr int QROWB = HD * (int)sizeof(T) + 16;
  constexpr int QCH = HD * (int)sizeof(T) / 16;            // 16-byte chunks per query row
  static_assert(C::Q * QROWB <= C::LDS, "Q block in the stage area");
  {
    u32x4 qc[(C::Q * QCH + 64 * C::W - 1) / (64 * C::W)];
#pragma unroll
    for (int j = 0; j < (int)(sizeof(qc) / sizeof(qc[0])); ++j) {
      const int c = tid + j * 64 * C::W;
      if (c < C::Q * QCH) {
        const int qrow = min(qb * kAttnQueries + c / QCH, m_per_seq - 1);
        qc[j] = ld16(q + ((size_t)b * m_per_seq + qrow) * ldq + (size_t)h * HD + (c % QCH) * VEC);
      }
    }
    gload(t_begin);
#pragma unroll
    for (int j = 0; j < (int)(sizeof(qc) / sizeof(qc[0])); ++j) {
      const int c = tid + j * 64 * C::W;
      if (c < C::Q * QCH) st16(smem + (c / QCH) * QROWB + (c % QCH) * 16, qc[j]);
    }
    __syncthreads();
    const char *qrow = smem + (qg * 32 + (lane & 31)) * QROWB;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) {
      if constexpr (BF)
        qf[st] = *reinterpret_cast<const u32x4 *>(qrow + (st * 16 + (lane >> 5) * 8) * 2);
      else
        qf[st] = *reinterpret_cast<const float *>(qrow + (st * 2 + (lane >> 5)) * 4);
    }
    __syncthreads();  // every wave holds its fragments before the first tile store overwrites the block
  }

  // Tile i + 1 is loaded into registers during tile i and written to the (other) stage after it; with
  // shared stages one barrier per tile (every wave runs the same tper tiles).
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
  lrun += xor_lane<32>(lrun);
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

// Many query rows per KV head (bf16): the query heads of a KV group packed into the MFMA rows. One
// workgroup = (sequence b, KV head g, block of 256 packed rows). The packed rows of (b, g) are its m
// queries times its grp query heads, query-major: row t is query t / grp of query head g grp + t % grp,
// so with grouped-query attention every K/V byte fetched from L2 serves all the heads that read it
// (Dream: 7 per KV head). Eight waves of 32 rows (two per SIMD, so one wave's MFMAs overlap another's
// softmax and LDS traffic) stream every 32-key tile of the head through a double-buffered LDS stage that
// they load together (one barrier per tile). S^T = K Q^T and O^T = V^T P^T on 32x32 MFMA blocks, online
// softmax in fp32 base 2 with a lazily moved reference maximum, as in attention_kernel; no key split,
// so the output is normalised in place. (Measured on MI355X: 807 us against 935 for four waves of 64
// rows at B = 8, N = 4096, 32 heads, 1024 queries; a key split over workgroups with a merge of the
// partial states lost to attention_kernel at every row count too small to fill the chip without it.)
template <int HD, int QB, int NW> struct PackAttnCfg {
  static constexpr int W = NW, QPW = 32 * QB, R = QPW * W;         // waves, rows per wave / per workgroup
  static constexpr int KT = 32;                                    // keys per tile
  // K and V rows [key][hd] as loaded; V rows padded by 64 bytes for the transposed fragment reads
  static constexpr int KROWB = HD * 2 + 16, VROWB = HD * 2 + 64;
  static constexpr int STAGE = KT * KROWB + KT * VROWB;
  static constexpr int OROWB = (HD + 4) * 4;                       // staged fp32 output row
  static constexpr int OUT = W * 32 * OROWB;                       // one 32-row block per wave at a time
  static constexpr int LDS = 2 * STAGE > OUT ? 2 * STAGE : OUT;
  static constexpr int KCHUNKS = KT * HD / 8;                      // K 16-byte chunks per tile
  static constexpr int KCH = (KCHUNKS + 64 * W - 1) / (64 * W);    // per lane (the last pass partial)
  static_assert(QB == 1 || QB == 2, "one or two column blocks per wave");
  static_assert(KCHUNKS % (64 * W) == 0 || KCH == 1, "tile split");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int HD, int QB, int NW>
__global__ __launch_bounds__(64 * NW) void attention_packed_kernel(const bf16_t *__restrict__ q,
                                                                   const bf16_t *__restrict__ kc,
                                                                   const bf16_t *__restrict__ vc,
                                                                   bf16_t *__restrict__ o, int m_per_seq, int n_tok,
                                                                   int hq, int hkv, int rblocks, int nwg,
                                                                   float scale_log2) {
  typedef bf16_t T;
  typedef PackAttnCfg<HD, QB, NW> C;
  constexpr int KT = C::KT, KROWB = C::KROWB, VROWB = C::VROWB, KCH = C::KCH;
  constexpr int QSTEPS = HD / 16, HB = HD / 32;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  // XCD-aware order (hardware hands workgroup i to XCD i % 8): each XCD runs a contiguous range of
  // (sequence, KV head, row block), so the row blocks that read one head's K/V share an L2
  const int nb = gridDim.x;
  const int lid = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (lid >= nwg) return;  // grid padding (whole workgroup, before any barrier)
  const int grp = hq / hkv;
  const int rb = lid % rblocks;
  const int g = (lid / rblocks) % hkv;
  const int b = lid / rblocks / hkv;
  const int rows = grp * m_per_seq;            // packed rows of (b, g)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = rb * C::R + wave * C::QPW;  // this wave's first packed row
  auto stage = [&](int buf) { return smem + buf * C::STAGE; };
  // output row (in the B x m x hq layout of q and o) of packed row t of (b, g)
  auto out_row = [&](int t) { return ((long long)b * m_per_seq + t / grp) * hq + g * grp + t % grp; };

  // Q fragments of the wave's column blocks: B operand of S^T = K Q^T (column = packed row lane % 32)
  u32x4 qf[QB][QSTEPS];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int t = min(row0 + 32 * j + (lane & 31), rows - 1);
    const T *qp = q + out_row(t) * HD;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) qf[j][st] = ld16(qp + st * 16 + (lane >> 5) * 8);
  }

  const size_t head_off = ((size_t)b * hkv + g) * (size_t)n_tok * HD;
  const T *kbase = kc + head_off;
  const T *vbase = vc + head_off;

  floatx16 oacc[QB][HB];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int i = 0; i < HB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[j][i][r] = 0.f;
  float mrun[QB], lrun[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    mrun[j] = -INFINITY;
    lrun[j] = 0.f;
  }

  // tile loads split over the waves: K and V 16-byte chunks c = lane + 64 (W jj + wave) of the tile
  u32x4 rk[KCH], rv[KCH];
  int koff[KCH];
#pragma unroll
  for (int jj = 0; jj < KCH; ++jj) {
    const int c = lane + 64 * (jj * C::W + wave);
    koff[jj] = (c / (HD / 8)) * HD + (c % (HD / 8)) * 8;
  }
  // lanes past the tile's K chunks (hd 64 with eight waves) load and store none
  auto kchunk = [&](int jj) { return C::KCHUNKS % (64 * C::W) == 0 || lane + 64 * (jj * C::W + wave) < C::KCHUNKS; };
  auto gload = [&](int t) {
    const int key0 = t * KT;
    if (key0 + KT <= n_tok) {
      const T *kt = kbase + (size_t)key0 * HD;
      const T *vt = vbase + (size_t)key0 * HD;
#pragma unroll
      for (int jj = 0; jj < KCH; ++jj)
        if (kchunk(jj)) {
          rk[jj] = ld16(kt + koff[jj]);
          rv[jj] = ld16(vt + koff[jj]);
        }
    } else {  // rows past the last key read the last key (masked later)
#pragma unroll
      for (int jj = 0; jj < KCH; ++jj) {
        const size_t off = (size_t)min(key0 + koff[jj] / HD, n_tok - 1) * HD + koff[jj] % HD;
        if (kchunk(jj)) {
          rk[jj] = ld16(kbase + off);
          rv[jj] = ld16(vbase + off);
        }
      }
    }
  };
  auto lstore = [&](int buf) {
    char *ks = stage(buf), *vs = ks + KT * KROWB;
#pragma unroll
    for (int jj = 0; jj < KCH; ++jj) {
      const int c = lane + 64 * (jj * C::W + wave);
      if (kchunk(jj)) {
        st16(ks + (c / (HD / 8)) * KROWB + (c % (HD / 8)) * 16, rk[jj]);
        st16(vs + (c / (HD / 8)) * VROWB + (c % (HD / 8)) * 16, rv[jj]);
      }
    }
  };

  // S^T = K Q^T of the tile in stage buf, every column block (each K fragment feeds QB MFMAs)
  auto qk = [&](int buf, floatx16 (&sc)[QB]) {
    const char *krow = stage(buf) + (lane & 31) * KROWB + (lane >> 5) * 16;
#pragma unroll
    for (int jq = 0; jq < QB; ++jq)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[jq][r] = 0.f;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) {
      const u32x4 kf = *reinterpret_cast<const u32x4 *>(krow + st * 32);
#pragma unroll
      for (int jq = 0; jq < QB; ++jq) sc[jq] = mfma32(kf, qf[jq][st], sc[jq]);
    }
  };
  // Online softmax of tile t in place (scores -> probabilities). masked: the tile reaches past the
  // last key (a runtime branch: two inlined variants would not fit the register file).
  auto softmax = [&](int t, floatx16 (&sc)[QB], bool masked) {
#pragma unroll
    for (int jq = 0; jq < QB; ++jq) {
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * KT + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          if (key >= n_tok) sc[jq][r] = -INFINITY;
        }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sc[jq][r]);
      tmax = fmaxf(tmax, xor_lane<32>(tmax)) * scale_log2;
      // reference maximum that moves only when a row's maximum exceeds it by more than 8 (p <= 2^8)
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
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[jq][r], scale_log2, -msub));
        sc[jq][r] = p;
        psum += p;
      }
      lrun[jq] += psum;
    }
  };
  // O^T += V^T P^T from the tile in stage buf, each V^T fragment (two transposed reads of the V rows,
  // as in attention_kernel) shared by the column blocks
  auto pv = [&](int buf, const floatx16 (&sc)[QB]) {
    const char *vs = stage(buf) + KT * KROWB;
    const int tg = lane >> 4, tj = lane & 15;
    const char *vrd0 = vs + (4 * (tg >> 1) + (tj >> 2)) * VROWB + (16 * (tg & 1) + 4 * (tj & 3)) * 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 pf[QB];
#pragma unroll
      for (int jq = 0; jq < QB; ++jq) {
        pf[jq][0] = pack_bf16x2(sc[jq][half * 8 + 0], sc[jq][half * 8 + 1]);
        pf[jq][1] = pack_bf16x2(sc[jq][half * 8 + 2], sc[jq][half * 8 + 3]);
        pf[jq][2] = pack_bf16x2(sc[jq][half * 8 + 4], sc[jq][half * 8 + 5]);
        pf[jq][3] = pack_bf16x2(sc[jq][half * 8 + 6], sc[jq][half * 8 + 7]);
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const char *vrd = vrd0 + half * 16 * VROWB + hb * 64;
        const u32x2 lo = lds_read_tr16(vrd);
        const u32x2 hi = lds_read_tr16(vrd + 8 * VROWB);
        const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int jq = 0; jq < QB; ++jq) oacc[jq][hb] = mfma32(vf, pf[jq], oacc[jq][hb]);
      }
    }
  };

  const int ntiles = (n_tok + KT - 1) / KT;
  gload(0);
  lstore(0);
  gload(1);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    floatx16 sc[QB];
    qk(t & 1, sc);
    softmax(t, sc, t * KT + KT > n_tok);
    pv(t & 1, sc);
    if (t + 1 < ntiles) {
      lstore((t + 1) & 1);
      gload(t + 2);
    }
    __syncthreads();  // tile t + 1 stored; tile t read by every wave (its buffer is refilled next)
  }

  // Epilogue, one 32-row column block at a time: stage the block's normalised rows row-major in the
  // wave's own LDS region (the stages are free after the last barrier; the wave reads back only what it
  // wrote), then write whole 16-byte bf16 row pieces of O.
  char *ob = smem + wave * 32 * C::OROWB;
  const int G = lane >> 5;
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float l = lrun[j] + xor_lane<32>(lrun[j]);
    const float sc = 1.0f / l;
    char *orow = ob + (lane & 31) * C::OROWB;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<floatx4 *>(orow + (hb * 32 + r4 * 8 + G * 4) * 4) =
            floatx4{oacc[j][hb][r4 * 4 + 0] * sc, oacc[j][hb][r4 * 4 + 1] * sc, oacc[j][hb][r4 * 4 + 2] * sc,
                    oacc[j][hb][r4 * 4 + 3] * sc};
    const int tb = row0 + 32 * j;  // first packed row of the block
#pragma unroll
    for (int it = 0; it < 32 * HD / 8 / 64; ++it) {
      const int c = lane + 64 * it;
      const int rl = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      if (tb + rl < rows) {
        const float *src = reinterpret_cast<const float *>(ob + rl * C::OROWB) + d0;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = src[e];
        st16(o + out_row(tb + rl) * HD + d0, pack16(v, (const bf16_t *)nullptr));
      }
    }
  }
}

template <int HD>
static hipError_t launch_packed(const void *q, const void *kc, const void *vc, void *o, int batch, int m_per_seq,
                                int n_tok, int hq, int hkv, hipStream_t s) {
  typedef PackAttnCfg<HD, 1, 8> C;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  const int rblocks = (int)(((long long)(hq / hkv) * m_per_seq + C::R - 1) / C::R);
  const long long nwg = (long long)batch * hkv * rblocks;
  if (nwg > (1LL << 30)) return hipErrorInvalidValue;
  const int grid = (int)((nwg + 7) / 8 * 8);
  hipLaunchKernelGGL((attention_packed_kernel<HD, 1, 8>), dim3(grid), dim3(64 * C::W), 0, s, (const bf16_t *)q,
                     (const bf16_t *)kc, (const bf16_t *)vc, (bf16_t *)o, m_per_seq, n_tok, hq, hkv, rblocks, (int)nwg,
                     scale_log2);
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

AttnPlan plan_attention(int dtype, int batch, int m_per_seq, int n_tok, int hq, int hkv, int hd) {
  (void)n_tok;
  (void)hd;
  constexpr int kCUs = 256;
  if (dtype == kBF16) {
    // The packed kernel once its 256-row blocks give at least 3/4 of a round of workgroups (measured:
    // B = 8, N = 4096, 32 heads at 327 / 655 / 1024 queries 411 / 605 / 807 us against 430 / 748 / 1084
    // for the 64-query kernel; the Dream full recompute, 224 workgroups, 102 against 139 us; the llada
    // full recompute, 128 workgroups, 53 against 42 us).
    const long long units = (long long)batch * hkv * (((long long)(hq / hkv) * m_per_seq + 255) / 256);
    if (4 * units >= 3 * kCUs) return AttnPlan{kAttnPacked};
  }
  // 64-query workgroups unless 32-query ones fill the chip in one round
  const long long heads = (long long)hq * batch;
  const long long wg64 = heads * ((m_per_seq + 63) / 64), wg32 = heads * ((m_per_seq + 31) / 32);
  return AttnPlan{wg64 < kCUs && wg32 <= kCUs ? kAttnQG1 : kAttnQG2};
}

template <typename T, int HD>
static hipError_t run_attention(const AttnPlan &p, const void *q, const void *kc, const void *vc, void *o, int batch,
                                int m_per_seq, int n_tok, int hq, int hkv, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (p.kind == kAttnPacked) return launch_packed<HD>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  }
  if (p.kind == kAttnQG1) return launch_qg<T, HD, 1>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  if (p.kind == kAttnQG2) return launch_qg<T, HD, 2>(q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int dtype, const AttnPlan &plan, const void *q, const void *kc, const void *vc, void *o,
                            int batch, int m_per_seq, int n_tok, int hq, int hkv, int hd, hipStream_t s) {
  if (m_per_seq <= 0 || batch <= 0) return hipSuccess;
  if (dtype == kBF16) {
    if (hd == 128) return run_attention<bf16_t, 128>(plan, q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
    return run_attention<bf16_t, 64>(plan, q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  }
  if (hd == 128) return run_attention<float, 128>(plan, q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
  return run_attention<float, 64>(plan, q, kc, vc, o, batch, m_per_seq, n_tok, hq, hkv, s);
}

}  // namespace spa
