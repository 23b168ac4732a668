// Shared device helpers for the SPA-Cache kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

typedef uint16_t bf16_t;  // raw bfloat16 storage (upper half of an IEEE binary32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// float -> bfloat16 with the hardware conversion (v_cvt_pk_bf16_f32: round to nearest, ties to
// even; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2v v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Elements per 16-byte vector.
template <typename T> struct Vec { static constexpr int kN = 16 / sizeof(T); };

// Unpack a 16-byte vector of T into floats.
__device__ __forceinline__ void unpack16(const u32x4 &v, float *out, const bf16_t *) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(v[j] << 16);
    out[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const u32x4 &v, float *out, const float *) {
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = __uint_as_float(v[j]);
}
__device__ __forceinline__ u32x4 pack16(const float *in, const bf16_t *) {
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(in[2 * j], in[2 * j + 1]);
  return v;
}
__device__ __forceinline__ u32x4 pack16(const float *in, const float *) {
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = __float_as_uint(in[j]);
  return v;
}

// 16x16 MFMA tiles. bf16: K = 32 per instruction, 8 values per lane (k = 8*(lane/16) + 0..7).
// fp32: K = 4 per instruction, 1 value per lane (k = lane/16). Output: lane holds column lane%16,
// rows 4*(lane/16) + 0..3. The k order inside an instruction only has to agree between A and B.
__device__ __forceinline__ floatx4 mfma16(const u32x4 &a, const u32x4 &b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 32x32 MFMA blocks. bf16: K = 16 per instruction, 8 values per lane (k = 8*(lane/32) + 0..7).
// fp32: K = 2 per instruction, 1 value per lane (k = lane/32). A: lane holds row lane%32; B: column
// lane%32. Output: lane holds column lane%32 and rows 8*(i/4) + 4*(lane/32) + i%4 for i = 0..15.
typedef float floatx16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ floatx16 mfma32(const u32x4 &a, const u32x4 &b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// The value that lane l ^ OFF of the wave holds (OFF = 1, 2, 4, 8, 16 or 32; every lane active), the
// same exchange as __shfl_xor without its LDS round trip: DPP permutes within quads (1, 2), a half-row
// mirror followed by a quad reversal (4), a rotation by 8 within each 16-lane row (8), and gfx950's
// v_permlane16_swap / v_permlane32_swap across rows (16) and wave halves (32), whose two results hold
// the pair's values in either order.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int OFF> __device__ __forceinline__ float xor_lane(float v) {
  static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "xor offset");
  if constexpr (OFF == 1) {
    return dpp_mov<0xB1>(v);                 // quad_perm [1, 0, 3, 2]
  } else if constexpr (OFF == 2) {
    return dpp_mov<0x4E>(v);                 // quad_perm [2, 3, 0, 1]
  } else if constexpr (OFF == 4) {
    return dpp_mov<0x1B>(dpp_mov<0x141>(v)); // row_half_mirror, then quad_perm [3, 2, 1, 0]
  } else if constexpr (OFF == 8) {
    return dpp_mov<0x128>(v);                // row_ror:8
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
  }
}

// Butterfly sum / max over the wave (xor 32, 16, ..., 1): every lane ends with the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane<32>(v);
  v += xor_lane<16>(v);
  v += xor_lane<8>(v);
  v += xor_lane<4>(v);
  v += xor_lane<2>(v);
  v += xor_lane<1>(v);
  return v;
}
// The same butterfly over each aligned group of G lanes (G = 16, 32 or 64; G = 64 is wave_sum).
template <int G> __device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 16 || G == 32 || G == 64, "group size");
  if constexpr (G == 64) v += xor_lane<32>(v);
  if constexpr (G >= 32) v += xor_lane<16>(v);
  v += xor_lane<8>(v);
  v += xor_lane<4>(v);
  v += xor_lane<2>(v);
  v += xor_lane<1>(v);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lane<32>(v));
  v = fmaxf(v, xor_lane<16>(v));
  v = fmaxf(v, xor_lane<8>(v));
  v = fmaxf(v, xor_lane<4>(v));
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<1>(v));
  return v;
}

// A compile-time flag passed to generic lambdas (bodies instantiated with and without a step).
template <bool B> struct BoolTag { static constexpr bool value = B; };

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

}  // namespace spa
