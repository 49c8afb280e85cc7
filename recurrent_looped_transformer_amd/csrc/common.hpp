// Device-side building blocks shared by the kernels: storage types (fp32, bf16,
// fp16), conversions, 16-byte vector loads, the gfx950 16-bit MFMA tiles,
// wave/block reductions. CDNA4: 64-lane wavefronts, 160 KB LDS per CU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlt {

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory
typedef _Float16 f16_t;   // IEEE binary16 in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));   // bf16 operand of the 16x16x16 MFMA
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
// round to nearest even (NaN kept quiet)
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Activation / cache element type: float for the fp32 configuration, bf16 bits otherwise.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static constexpr int VEC = 4;   // elements per 16-byte vector
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
  static __device__ __forceinline__ uint32_t bits(float v) { return f2bf(v); }
  static __device__ __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
  static constexpr int VEC = 8;
};
template <> struct Elem<f16_t> {
  static __device__ __forceinline__ float ld(const f16_t* p) { return (float)*p; }
  static __device__ __forceinline__ void st(f16_t* p, float v) { *p = (f16_t)v; }   // round to nearest even
  static __device__ __forceinline__ uint32_t bits(float v) { return __builtin_bit_cast(uint16_t, (f16_t)v); }
  static __device__ __forceinline__ float round(float v) { return (float)(f16_t)v; }
  static constexpr int VEC = 8;
};
// Store v as one 16-bit term at p, or, when lo_off > 0, as two: hi = round(v) at p and
// lo = round(v - hi) at p + lo_off (a two-term value carries about twice the significand).
template <typename T>
__device__ __forceinline__ void store_act(T* p, int64_t lo_off, float v) {
  const float hi = Elem<T>::round(v);
  Elem<T>::st(p, hi);
  if (lo_off) Elem<T>::st(p + lo_off, v - hi);
}
template <>
__device__ __forceinline__ void store_act<float>(float* p, int64_t, float v) { *p = v; }
// two values rounded to the 16-bit type T, packed low | high << 16
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return Elem<T>::bits(lo) | (Elem<T>::bits(hi) << 16);
}

// 16-byte load of VEC elements converted to float.
__device__ __forceinline__ void load16(const float* p, float* o) {
  float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load16(const bf16_t* p, float* o) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
// the VEC elements of a 16-byte register value as float
template <typename T> __device__ __forceinline__ void unpack16(const uint4& v, float* o);
template <> __device__ __forceinline__ void unpack16<float>(const uint4& v, float* o) {
  o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y); o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}
template <> __device__ __forceinline__ void unpack16<bf16_t>(const uint4& v, float* o) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void unpack16<f16_t>(const uint4& v, float* o) {
  const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)h[i];
}
__device__ __forceinline__ void load16(const f16_t* p, float* o) {
  unpack16<f16_t>(*reinterpret_cast<const uint4*>(p), o);
}
__device__ __forceinline__ void store16(f16_t* p, const float* v) {
  uint4 o;
  o.x = pack2<f16_t>(v[0], v[1]);
  o.y = pack2<f16_t>(v[2], v[3]);
  o.z = pack2<f16_t>(v[4], v[5]);
  o.w = pack2<f16_t>(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = o;
}
__device__ __forceinline__ void store16(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store16(bf16_t* p, const float* v) {
  uint4 o;
  o.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  o.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  o.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
  o.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = o;
}

// 16-byte load with the nontemporal hint: for streams read once per launch and larger than the
// last-level cache (measured on MI355X: a 4 GB read streams at 7.1 TB/s this way against 6.25
// TB/s with plain loads)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if constexpr (NT) return ld16_nt(p);
  else return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------- MFMA
// D(16x16, fp32) += A(16x32) * B(32x16), 16-bit inputs of type T (gfx950
// v_mfma_f32_16x16x32_bf16 / _f16). Lane l supplies A row (l % 16), k = 8*(l / 16) .. +7
// and B column (l % 16), same k; it receives D rows 4*(l / 16) .. +3 of column (l % 16).
template <typename T = bf16_t>
__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, f32x4 c) {
  if constexpr (sizeof(T) == 2 && __is_same(T, f16_t)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
}
// D(16x16) += A(16x16) * B(16x16): lane l supplies row/column (l % 16), k = 4*(l / 16) .. +3.
template <typename T = bf16_t>
__device__ __forceinline__ f32x4 mfma16x16x16(const uint2& a, const uint2& b, f32x4 c) {
  if constexpr (__is_same(T, f16_t)) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                                 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
  }
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
// Wavefront sum through DPP lane moves (no LDS round trips): quad swaps, half-row and row
// mirrors give every lane its 16-lane row sum, two row broadcasts carry the rows into lane 63,
// which is read back as a wave-uniform value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf,
                                                               true));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_<0xb1, 0xf>(v);    // quad_perm [1,0,3,2]
  v += dpp_<0x4e, 0xf>(v);    // quad_perm [2,3,0,1]
  v += dpp_<0x141, 0xf>(v);   // row_half_mirror
  v += dpp_<0x140, 0xf>(v);   // row_mirror
  v += dpp_<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Sum over aligned groups of G lanes (G a power of two <= 64), result in every lane of the
// group: DPP moves within 16-lane rows, lane shuffles across rows.
template <int G>
__device__ __forceinline__ float group_sum_dpp(float v) {
  if constexpr (G >= 2) v += dpp_<0xb1, 0xf>(v);    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp_<0x4e, 0xf>(v);    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp_<0x141, 0xf>(v);   // row_half_mirror: lane i + lane 7 - i (quad sums)
  if constexpr (G >= 16) v += dpp_<0x140, 0xf>(v);  // row_mirror: lane i + lane 15 - i (half-row sums)
  if constexpr (G >= 32) v += __shfl_xor(v, 16, WAVE);
  if constexpr (G >= 64) v += __shfl_xor(v, 32, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
// Block-wide reductions for blockDim.x a multiple of 64 (<= 1024); red has >= 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  float s = -INFINITY;
  for (int i = 0; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

}  // namespace rlt
