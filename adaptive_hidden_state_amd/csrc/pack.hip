// Fragment-packed weight layout (the layout is defined next to packed_dims in launch.hpp). A GEMM
// wave consumes its weights as 32x32 MFMA B fragments: for every (32-row block, 16-k step) each lane
// holds 16 bytes of one row. Storing each such fragment as one contiguous kilobyte in lane order
// lets the wave fetch it with a single fully coalesced 16-byte load per lane, straight into the
// registers the MFMA reads, and lets every weight panel stream from HBM as long sequential runs. The
// zero padding (rows to 32, columns to 64) removes the K-tail and N-tail cases from the GEMM. An
// optional column scale folds an RMSNorm gain into the weight that consumes the normalised rows.
#include "common.hpp"
#include "launch.hpp"

namespace spa {

template <typename T>
__global__ __launch_bounds__(256) void pack_weight_kernel(const T *__restrict__ src, int rows, int cols,
                                                          int rows_pad, int cols_pad, int gate_up_f,
                                                          const T *__restrict__ scale, T *__restrict__ dst) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int BKF = BF ? 16 : 8;  // K elements per block
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte chunk of dst
  const size_t nchunks = (size_t)rows_pad * cols_pad * sizeof(T) / 16;
  if (t >= nchunks) return;
  const int wkb = cols_pad / BKF;
  const size_t blk = t >> 6;
  const int l = (int)(t & 63);
  const int rb = (int)(blk / wkb), kb = (int)(blk % wkb);
  const int w = l & 31;
  const int r = rb * 32 + w;
  int sr = r;
  bool valid = r < rows;
  if (gate_up_f > 0) {  // block rb: gate rows of units 16 rb .. 16 rb + 15, then their up rows
    const int u = rb * 16 + (w & 15);
    valid = u < gate_up_f;
    sr = (w < 16) ? u : gate_up_f + u;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if constexpr (BF) {
    const int c0 = kb * BKF + (l >> 5) * 8;  // 8 consecutive K elements (cols is a multiple of 16)
    u32x4 v = (valid && c0 < cols) ? ld16(src + (size_t)sr * cols + c0) : zero;
    if (scale != nullptr && valid && c0 < cols) {  // W diag(scale): product in fp32, one rounding
      float x[8], g[8];
      unpack16(v, x, src);
      unpack16(ld16(scale + c0), g, src);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= g[e];
      v = pack16(x, src);
    }
    st16(dst + t * 8, v);
  } else {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = kb * BKF + 2 * j + (l >> 5);
      v[j] = (valid && c < cols) ? src[(size_t)sr * cols + c] * (scale != nullptr ? scale[c] : 1.0f) : 0.f;
    }
    st16(dst + t * 4, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                            __float_as_uint(v[3])});
  }
}

hipError_t launch_pack_weight(int dtype, int kind, int rows, int cols, const void *src, const void *col_scale,
                              void *dst, hipStream_t s) {
  int rp, cp;
  packed_dims(kind, rows, cols, &rp, &cp);
  const int f = kind == kPackGateUp ? rows / 2 : 0;
  const size_t chunks = (size_t)rp * cp * (dtype == kBF16 ? 2 : 4) / 16;
  const unsigned grid = (unsigned)((chunks + 255) / 256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(pack_weight_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, (const bf16_t *)src, rows, cols, rp,
                       cp, f, (const bf16_t *)col_scale, (bf16_t *)dst);
  else
    hipLaunchKernelGGL(pack_weight_kernel<float>, dim3(grid), dim3(256), 0, s, (const float *)src, rows, cols, rp, cp,
                       f, (const float *)col_scale, (float *)dst);
  return hipGetLastError();
}

}  // namespace spa
