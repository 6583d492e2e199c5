// Device helpers shared by the gfx950 kernels: vector types, storage-format
// decoders/encoders (OCP FP8 E4M3FN, BF16, MXFP4 E2M1/E8M0) and small reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hca {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ decoders
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}


// --------------------------------------------------------- encoders (from fp64)
// Each rounds |v| once to the nearest point of the format's grid (ties to even):
// the grid spacing inside binade 2^e is 2^(e - mantissa_bits), clamped at the
// smallest normal binade (subnormal spacing below it).
__device__ __forceinline__ double rne_grid(double a, int min_binade, int mant_bits) {
  int e = (a == 0.0) ? min_binade : ilogb(a);
  if (e < min_binade) e = min_binade;
  return ldexp(rint(ldexp(a, mant_bits - e)), e - mant_bits);
}

// OCP E4M3FN code of v (saturating at +-448); sign bit = sign of v.
__device__ __forceinline__ uint8_t encode_fp8(double v) {
  const uint8_t s = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a != a) return 0x7F;
  double r = rne_grid(a, -6, 3);
  if (r >= 448.0) return s | 0x7E;
  if (r < 0.015625) return s | (uint8_t)(int)ldexp(r, 9);     // subnormal: r = m * 2^-9
  int E = ilogb(r);
  int mant = (int)ldexp(r, 3 - E) - 8;
  return s | (uint8_t)(((E + 7) << 3) | mant);
}

// BF16 bits of v (no overflow handling: |v| stays far below 2^127 here).
__device__ __forceinline__ uint16_t encode_bf16(double v) {
  const uint16_t s = signbit(v) ? 0x8000 : 0;
  double r = rne_grid(fabs(v), -126, 7);
  return s | (uint16_t)(__float_as_uint((float)r) >> 16);
}

// E2M1 code of v (already divided by its block scale), saturating at +-6.
__device__ __forceinline__ uint8_t encode_e2m1(double v) {
  const uint8_t s = signbit(v) ? 8 : 0;
  double r = rne_grid(fabs(v), 0, 1);
  if (r > 6.0) r = 6.0;
  uint8_t c = r < 2.0 ? (uint8_t)(r * 2.0) : (r == 2.0 ? 4 : (r == 3.0 ? 5 : (r == 4.0 ? 6 : 7)));
  return s | c;
}

// Exponent e of the per-entry FP8 scale 2^e: the smallest e with amax <= 448 * 2^e.
__device__ __forceinline__ int fp8_entry_scale_exp(double amax) {
  if (!(amax > 0.0)) return 0;
  int e0 = ilogb(amax);
  double f = ldexp(amax, -e0);            // in [1, 2)
  return (f <= 1.75) ? e0 - 8 : e0 - 7;   // 448 = 1.75 * 2^8
}

// E8M0 exponent of an MXFP4 block: floor(log2 amax) - 2, clamped; -127 for amax = 0.
__device__ __forceinline__ int mx_scale_exp(double amax) {
  if (!(amax > 0.0)) return -127;
  int e = ilogb(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ---------------------------------------------------------------- reductions
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { T u = __shfl_xor(v, o, 64); v = u > v ? u : v; }
  return v;
}

// Orderable key of a float: larger float <=> larger key; -0 and +0 map together.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t double_key(double f) {
  uint64_t b = (uint64_t)__double_as_longlong(f);
  if (b == 0x8000000000000000ull) b = 0;
  return (b & 0x8000000000000000ull) ? ~b : (b | 0x8000000000000000ull);
}

}  // namespace hca
