// Partial cached attention ([PN] 整体框架 Phase 2): the k queries of the update set attend,
// bidirectionally and without a mask, to all N keys of the (already scattered) K^c/V^c cache.
//
// One workgroup = one (sequence, query head, block of 32 * QW queries); each wave owns 32 queries.
// Keys stream through LDS in tiles of 64: K as [key][hd] and V transposed to [hd][key], so that both
// products read contiguous LDS. A wave computes S^T = K Q^T (keys x queries) on 32x32 MFMA blocks;
// in that layout a lane holds 32 scores of one query, so the online softmax (fp32, base-2 exponent)
// needs one cross-lane step, and the probabilities feed O^T = V^T P^T straight from registers.
// V is transposed on the way into LDS: each thread loads an 8-key x 8-dim block (eight 16-byte row
// pieces), transposes it in registers and writes eight 16-byte rows of V^T.
// Query head h reads KV head h / (H_q / H_kv) (grouped-query attention).
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

template <typename T, int HD, int QW>
__global__ __launch_bounds__(64 * QW) void attention_kernel(const T *__restrict__ q, const T *__restrict__ kc,
                                                            const T *__restrict__ vc, T *__restrict__ o,
                                                            int m_per_seq, int n_tok, int hq, int hkv,
                                                            float scale_log2) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int NT = 64 * QW;
  constexpr int KT = 64;                                  // keys per tile
  constexpr int KROWB = HD * (int)sizeof(T) + 16;         // K tile row stride (bytes)
  constexpr int VROWB = KT * (int)sizeof(T) + 16;         // V^T tile row stride (bytes)
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int KCH = KT * HD / VEC / NT;                 // K 16-byte chunks per thread per tile
  // V: bf16 uses 8x8 blocks (8 key rows x one 16-byte chunk); fp32 uses 4x4 blocks
  constexpr int VB = BF ? 8 : 4;
  constexpr int VTASKS = (KT / VB) * (HD / VB);           // blocks per tile
  constexpr int VPER = (VTASKS + NT - 1) / NT;
  constexpr int QSTEPS = BF ? HD / 16 : HD / 2;           // MFMA k-steps over the head dim
  constexpr int KSTEP_B = BF ? 32 : 8;
  constexpr int LANE_B = BF ? 16 : 4;
  constexpr int HB = HD / 32;                             // 32-row blocks of the head dim
  constexpr int PF = 2;                                   // key tiles in flight in registers
  static_assert(KT * HD % (VEC * NT) == 0, "K tile load split");
  typedef typename AFrag<BF>::type FragT;

  __shared__ __attribute__((aligned(16))) char ks[2][KT * KROWB];
  __shared__ __attribute__((aligned(16))) char vts[2][HD * VROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z, h = blockIdx.y;
  const int g = h / (hq / hkv);
  const int m0 = blockIdx.x * (32 * QW) + wave * 32;
  const int ldq = hq * HD;

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

  // V block assignment: block id v -> key block kb = v % (KT / VB), dim chunk cc = v / (KT / VB), so
  // the lanes that write one V^T row segment hold consecutive key blocks (conflict-free LDS).
  u32x4 rk[PF][KCH], rv[PF][VPER][VB];
  auto gload = [&](int t, u32x4 *xk, u32x4 (*xv)[VB]) {
    const int key0 = t * KT;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + j * NT;
      const int row = c / (HD / VEC), col = c % (HD / VEC);
      const int key = min(key0 + row, n_tok - 1);
      xk[j] = ld16(reinterpret_cast<const char *>(kbase + (size_t)key * HD) + col * 16);
    }
#pragma unroll
    for (int p = 0; p < VPER; ++p) {
      const int v = min(tid + p * NT, VTASKS - 1);
      const int kb = v % (KT / VB), cc = v / (KT / VB);
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        const int key = min(key0 + kb * VB + j, n_tok - 1);
        xv[p][j] = ld16(vbase + (size_t)key * HD + cc * VB);
      }
    }
  };
  auto lstore = [&](int buf, const u32x4 *xk, u32x4 (*xv)[VB]) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + j * NT;
      const int row = c / (HD / VEC), col = c % (HD / VEC);
      st16(ks[buf] + row * KROWB + col * 16, xk[j]);
    }
#pragma unroll
    for (int p = 0; p < VPER; ++p) {
      const int v = tid + p * NT;
      if (v < VTASKS) {
        const int kb = v % (KT / VB), cc = v / (KT / VB);
        if constexpr (BF) {
          u32x4 tr[8];
          transpose8x8_b16(xv[p], tr);
#pragma unroll
          for (int e = 0; e < 8; ++e) st16(vts[buf] + (cc * 8 + e) * VROWB + kb * 16, tr[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32x4 col = {xv[p][0][e], xv[p][1][e], xv[p][2][e], xv[p][3][e]};
            st16(vts[buf] + (cc * 4 + e) * VROWB + kb * 16, col);
          }
        }
      }
    }
  };

  auto compute = [&](int t, int buf) {
    // S^T blocks (64 keys = 2 blocks of 32): lane holds query lane%32 and keys
    // kb*32 + 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15
    floatx16 s[2], s2[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = s2[kb][r] = 0.f;
      const char *krow = ks[buf] + (kb * 32 + (lane & 31)) * KROWB + (lane >> 5) * LANE_B;
#pragma unroll
      for (int st = 0; st < QSTEPS; st += 2) {
        s[kb] = mfma32(*reinterpret_cast<const FragT *>(krow + st * KSTEP_B), qf[st], s[kb]);
        s2[kb] = mfma32(*reinterpret_cast<const FragT *>(krow + (st + 1) * KSTEP_B), qf[st + 1], s2[kb]);
      }
      s[kb] += s2[kb];
    }
    // raw scores; the softmax scale (and log2 e) is applied inside one FMA per score
    if (t * KT + KT > n_tok) {  // partial last tile (uniform branch): mask keys past the end
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * KT + kb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          if (key >= n_tok) s[kb][r] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[kb][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)) * scale_log2;
    const float mnew = fmaxf(mrun, tmax);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(fmaf(s[kb][r], scale_log2, -mnew));
        s[kb][r] = p;
        psum += p;
      }
    // rescale the running sums only when some query of this wave raised its maximum
    if (__any(mnew > mrun)) {
      const float alpha = exp2f(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) oacc[hb] *= alpha;
    }
    lrun += psum;
    mrun = mnew;

    // O^T += V^T P^T. In k-step (kb, half) lane group G = lane/32 supplies its scores r = half*8..
    // half*8+7, i.e. keys kb*32 + half*16 + {4G..4G+3, 8+4G..8+4G+3}; A = V^T rows at those keys.
    const int G = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if constexpr (BF) {
          u32x4 pf;
          pf[0] = pack_bf16x2(s[kb][half * 8 + 0], s[kb][half * 8 + 1]);
          pf[1] = pack_bf16x2(s[kb][half * 8 + 2], s[kb][half * 8 + 3]);
          pf[2] = pack_bf16x2(s[kb][half * 8 + 4], s[kb][half * 8 + 5]);
          pf[3] = pack_bf16x2(s[kb][half * 8 + 6], s[kb][half * 8 + 7]);
          const int c0 = (kb * 32 + half * 16 + 4 * G) * 2, c1 = c0 + 16;
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            const char *vrow = vts[buf] + (hb * 32 + (lane & 31)) * VROWB;
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
            const int key = kb * 32 + (r >> 2) * 8 + G * 4 + (r & 3);
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
              const float vf = *reinterpret_cast<const float *>(vts[buf] + (hb * 32 + (lane & 31)) * VROWB + key * 4);
              oacc[hb] = mfma32(vf, s[kb][r], oacc[hb]);
            }
          }
        }
      }
  };

  // Tiles padded to a multiple of PF keep the loop free of branches around its loads; a padding
  // tile reads clamped rows and every one of its keys is masked out.
  const int ntiles = (n_tok + KT - 1) / KT;
  const int ntiles_pad = (ntiles + PF - 1) / PF * PF;
#pragma unroll
  for (int u = 0; u < PF; ++u) gload(u, rk[u], rv[u]);
  lstore(0, rk[0], rv[0]);
  gload(PF, rk[0], rv[0]);
  __syncthreads();
  for (int t0 = 0; t0 < ntiles_pad; t0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int t = t0 + u;
      compute(t, u & 1);
      const int nslot = (u + 1) % PF;
      lstore((u + 1) & 1, rk[nslot], rv[nslot]);
      gload(t + 1 + PF, rk[nslot], rv[nslot]);
      __syncthreads();
    }
  }

  lrun += __shfl_xor(lrun, 32, kWave);
  const float inv = 1.0f / lrun;
  const int qo = m0 + (lane & 31);
  if (qo < m_per_seq) {
    // lane holds O^T[hd = hb*32 + 8*(r/4) + 4*(lane/32) + r%4][query]: 4 consecutive dims per r/4
    T *op = o + ((size_t)b * m_per_seq + qo) * ldq + (size_t)h * HD + (lane >> 5) * 4;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float v0 = oacc[hb][r4 * 4 + 0] * inv, v1 = oacc[hb][r4 * 4 + 1] * inv;
        const float v2 = oacc[hb][r4 * 4 + 2] * inv, v3 = oacc[hb][r4 * 4 + 3] * inv;
        T *dst = op + hb * 32 + r4 * 8;
        if constexpr (BF) {
          u32x2 w;
          w[0] = pack_bf16x2(v0, v1);
          w[1] = pack_bf16x2(v2, v3);
          *reinterpret_cast<u32x2 *>(dst) = w;
        } else {
          *reinterpret_cast<floatx4 *>(dst) = floatx4{v0, v1, v2, v3};
        }
      }
  }
}

template <typename T, int HD>
static hipError_t run_attention(const void *q, const void *kc, const void *vc, void *o, int batch, int m_per_seq,
                                int n_tok, int hq, int hkv, hipStream_t s) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  dim3 grid((m_per_seq + 63) / 64, hq, batch);
  hipLaunchKernelGGL((attention_kernel<T, HD, 2>), grid, dim3(128), 0, s, (const T *)q, (const T *)kc,
                     (const T *)vc, (T *)o, m_per_seq, n_tok, hq, hkv, scale_log2);
  return hipGetLastError();
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
