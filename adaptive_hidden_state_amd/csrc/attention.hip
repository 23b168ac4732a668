// Partial cached attention ([PN] 整体框架 Phase 2): the k queries of the update set attend,
// bidirectionally and without a mask, to all N keys of the (already scattered) K^c/V^c cache.
//
// One workgroup = one (sequence, query head, block of 64 queries); each of its 4 waves owns 16
// queries. Keys stream through LDS in tiles of 64: K as [key][hd], V transposed to [hd][key] so
// that both products read contiguous LDS. The wave computes S^T = K Q^T (keys x queries) with
// 16x16 MFMAs; in that layout a lane holds one query's scores, so the online softmax (fp32, base-2
// exponent) needs only two cross-lane steps, and the probabilities feed O^T = V^T P^T straight
// from registers. Query head h reads KV head h / (H_q / H_kv) (grouped-query attention).
#include "common.hpp"
#include "launch.hpp"

namespace spa {

template <bool BF16> struct AFrag;
template <> struct AFrag<true> { typedef u32x4 type; };
template <> struct AFrag<false> { typedef float type; };

template <typename T, int HD, int QW>
__global__ __launch_bounds__(64 * QW) void attention_kernel(const T *__restrict__ q, const T *__restrict__ kc,
                                                            const T *__restrict__ vc, T *__restrict__ o,
                                                            int m_per_seq, int n_tok, int hq, int hkv,
                                                            float scale_log2) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int NT = 64 * QW;
  constexpr int KT = 64;                                      // keys per tile
  constexpr int KROWB = HD * (int)sizeof(T) + 16;             // K tile row stride (bytes)
  constexpr int VROWB = KT * (int)sizeof(T) + (BF ? 8 : 16);  // V^T tile row stride (bytes)
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int CPR = HD / VEC;                               // 16-byte chunks per key row
  constexpr int KCH = KT * CPR / NT;                          // chunks per thread per tile (each of K, V)
  constexpr int QSTEPS = BF ? HD / 32 : HD / 4;
  constexpr int KSTEP_B = BF ? 64 : 16;
  constexpr int LANE_B = BF ? 16 : 4;
  constexpr int HB = HD / 16;
  constexpr int PF = 2;                                       // key tiles in flight in registers
  static_assert(KT * CPR % NT == 0, "tile load split");
  typedef typename AFrag<BF>::type FragT;

  __shared__ __attribute__((aligned(16))) char ks[2][KT * KROWB];
  __shared__ __attribute__((aligned(16))) char vts[2][HD * VROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z, h = blockIdx.y;
  const int g = h / (hq / hkv);
  const int m0 = blockIdx.x * (16 * QW) + wave * 16;
  const int ldq = hq * HD;

  // Q fragments: B operand of S^T = K Q^T (column = query lane&15, k = head dim).
  FragT qf[QSTEPS];
  {
    const int qrow = min(m0 + (lane & 15), m_per_seq - 1);
    const T *qp = q + ((size_t)b * m_per_seq + qrow) * ldq + (size_t)h * HD;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) {
      if constexpr (BF)
        qf[st] = ld16(qp + st * 32 + (lane >> 4) * 8);
      else
        qf[st] = qp[st * 4 + (lane >> 4)];
    }
  }

  const size_t head_off = ((size_t)b * hkv + g) * (size_t)n_tok * HD;
  const T *kbase = kc + head_off;
  const T *vbase = vc + head_off;

  floatx4 oacc[HB];
#pragma unroll
  for (int i = 0; i < HB; ++i) oacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  u32x4 rk[PF][KCH], rv[PF][KCH];
  auto gload = [&](int t, u32x4 *xk, u32x4 *xv) {
    const int key0 = t * KT;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + j * NT;
      const int row = c / CPR, col = c % CPR;
      const int key = min(key0 + row, n_tok - 1);
      xk[j] = ld16(reinterpret_cast<const char *>(kbase + (size_t)key * HD) + col * 16);
    }
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + j * NT;
      const int row = c % KT, col = c / KT;
      const int key = min(key0 + row, n_tok - 1);
      xv[j] = ld16(reinterpret_cast<const char *>(vbase + (size_t)key * HD) + col * 16);
    }
  };
  auto lstore = [&](int buf, const u32x4 *xk, const u32x4 *xv) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + j * NT;
      const int row = c / CPR, col = c % CPR;
      st16(ks[buf] + row * KROWB + col * 16, xk[j]);
    }
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + j * NT;
      const int key = c % KT, e0 = (c / KT) * VEC;
      if constexpr (BF) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          *reinterpret_cast<uint16_t *>(vts[buf] + (e0 + u) * VROWB + key * 2) =
              (uint16_t)(xv[j][u >> 1] >> (16 * (u & 1)));
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) *reinterpret_cast<uint32_t *>(vts[buf] + (e0 + u) * VROWB + key * 4) = xv[j][u];
      }
    }
  };

  auto compute = [&](int t, int buf) {
    // S^T blocks: rows = keys kb*16 + 4*(lane>>4) + i, column = query lane & 15
    floatx4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      const char *krow = ks[buf] + (kb * 16 + (lane & 15)) * KROWB + (lane >> 4) * LANE_B;
#pragma unroll
      for (int st = 0; st < QSTEPS; ++st)
        s[kb] = mfma16(*reinterpret_cast<const FragT *>(krow + st * KSTEP_B), qf[st], s[kb]);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = t * KT + kb * 16 + (lane >> 4) * 4 + i;
        const float v = key < n_tok ? s[kb][i] * scale_log2 : -INFINITY;
        s[kb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float mnew = fmaxf(mrun, tmax);
    const float alpha = exp2f(mrun - mnew);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(s[kb][i] - mnew);
        s[kb][i] = p;
        psum += p;
      }
    lrun = lrun * alpha + psum;
    mrun = mnew;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) oacc[hb] *= alpha;

    // O^T += V^T P^T: A = V^T rows (head dim), B = P^T (lane's own probabilities)
    if constexpr (BF) {
#pragma unroll
      for (int kb = 0; kb < 4; kb += 2) {
        u32x4 pf;
        pf[0] = pack_bf16x2(s[kb][0], s[kb][1]);
        pf[1] = pack_bf16x2(s[kb][2], s[kb][3]);
        pf[2] = pack_bf16x2(s[kb + 1][0], s[kb + 1][1]);
        pf[3] = pack_bf16x2(s[kb + 1][2], s[kb + 1][3]);
        const int c0 = (kb * 16 + (lane >> 4) * 4) * 2;
        const int c1 = c0 + 32;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const char *vrow = vts[buf] + (hb * 16 + (lane & 15)) * VROWB;
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + c0);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + c1);
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
          oacc[hb] = mfma16(vf, pf, oacc[hb]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = (kb * 16 + (lane >> 4) * 4 + i) * 4;
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            const float vf = *reinterpret_cast<const float *>(vts[buf] + (hb * 16 + (lane & 15)) * VROWB + c);
            oacc[hb] = mfma16(vf, s[kb][i], oacc[hb]);
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
      compute(t, t & 1);
      const int nslot = (u + 1) % PF;
      lstore((t + 1) & 1, rk[nslot], rv[nslot]);
      gload(t + 1 + PF, rk[nslot], rv[nslot]);
      __syncthreads();
    }
  }

  lrun += __shfl_xor(lrun, 16, kWave);
  lrun += __shfl_xor(lrun, 32, kWave);
  const float inv = 1.0f / lrun;
  const int qo = m0 + (lane & 15);
  if (qo < m_per_seq) {
    T *op = o + ((size_t)b * m_per_seq + qo) * ldq + (size_t)h * HD + (lane >> 4) * 4;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      if constexpr (BF) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[hb][0] * inv, oacc[hb][1] * inv);
        w[1] = pack_bf16x2(oacc[hb][2] * inv, oacc[hb][3] * inv);
        *reinterpret_cast<u32x2 *>(op + hb * 16) = w;
      } else {
        floatx4 w = oacc[hb] * inv;
        *reinterpret_cast<floatx4 *>(op + hb * 16) = w;
      }
    }
  }
}

template <typename T, int HD>
static hipError_t run_attention(const void *q, const void *kc, const void *vc, void *o, int batch, int m_per_seq,
                                int n_tok, int hq, int hkv, hipStream_t s) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  // 64 queries per workgroup when that already fills the chip, else 32
  const long wg64 = (long)((m_per_seq + 63) / 64) * hq * batch;
  if (wg64 >= 256) {
    dim3 grid((m_per_seq + 63) / 64, hq, batch);
    hipLaunchKernelGGL((attention_kernel<T, HD, 4>), grid, dim3(256), 0, s, (const T *)q, (const T *)kc,
                       (const T *)vc, (T *)o, m_per_seq, n_tok, hq, hkv, scale_log2);
  } else {
    dim3 grid((m_per_seq + 31) / 32, hq, batch);
    hipLaunchKernelGGL((attention_kernel<T, HD, 2>), grid, dim3(128), 0, s, (const T *)q, (const T *)kc,
                       (const T *)vc, (T *)o, m_per_seq, n_tok, hq, hkv, scale_log2);
  }
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
