// Tile-packed weight layout. A GEMM workgroup reads its weight panel one K slab (64 rows x 128 bytes)
// at a time; in a row-major matrix those 64 rows are 128-byte pieces scattered C * e bytes apart,
// which HBM serves at a small fraction of its bandwidth. Packing each 64 x 128-byte block into one
// contiguous 8 KB run turns every workgroup's panel into a sequential stream. The padding (rows to
// 128, columns to 64, zero-filled) also removes every K-tail and N-tail case from the GEMM.
#include "common.hpp"
#include "launch.hpp"

namespace spa {

template <typename T>
__global__ __launch_bounds__(256) void pack_weight_kernel(const T *__restrict__ src, int rows, int cols,
                                                          int rows_pad, int cols_pad, int gate_up_f,
                                                          T *__restrict__ dst) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int BKE = 128 / (int)sizeof(T);
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte chunk of dst
  const size_t nchunks = (size_t)rows_pad * cols_pad / VEC;
  if (t >= nchunks) return;
  const int kb = cols_pad / BKE;
  const size_t blk = t / 512;
  const int within = (int)(t % 512);
  const int bi = (int)(blk / kb), bj = (int)(blk % kb);
  const int r = bi * 64 + within / 8;
  const int c0 = bj * BKE + (within % 8) * VEC;
  int sr = r;
  bool valid = r < rows && c0 < cols;
  if (gate_up_f > 0) {  // logical row r = 64 q + w: gate (w < 32) or up row of unit 32 q + w % 32
    const int q = r >> 6, w = r & 63;
    const int j = q * 32 + (w & 31);
    valid = j < gate_up_f && c0 < cols;
    sr = (w < 32) ? j : gate_up_f + j;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  st16(dst + t * VEC, valid ? ld16(src + (size_t)sr * cols + c0) : zero);
}

hipError_t launch_pack_weight(int dtype, int kind, int rows, int cols, const void *src, void *dst, hipStream_t s) {
  int rp, cp;
  packed_dims(kind, rows, cols, &rp, &cp);
  const int f = kind == kPackGateUp ? rows / 2 : 0;
  const size_t chunks = (size_t)rp * cp * (dtype == kBF16 ? 2 : 4) / 16;
  const unsigned grid = (unsigned)((chunks + 255) / 256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(pack_weight_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, (const bf16_t *)src, rows, cols, rp,
                       cp, f, (bf16_t *)dst);
  else
    hipLaunchKernelGGL(pack_weight_kernel<float>, dim3(grid), dim3(256), 0, s, (const float *)src, rows, cols, rp, cp,
                       f, (float *)dst);
  return hipGetLastError();
}

}  // namespace spa
