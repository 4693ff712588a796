// Device-side helpers shared by the gfx950 kernels of the DCA sparse prefill library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) double f64x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

namespace dca {

constexpr int D = 128;          // head dimension
constexpr int HALF = 64;        // RoPE pairs (c, c + 64)

// RoPE frequencies theta_c = base^(-2c/d), c < 64, computed on the host in fp64
struct Freqs { double v[HALF]; };
constexpr int QB = 64;          // rows of a query block (sparse-cover granule)
constexpr int NXCD = 8;         // MI355X: 8 accelerator dies, workgroups dispatched round-robin

// 2*pi split for Cody-Waite reduction of fp64 angles.
constexpr double TWO_PI_HI = 6.283185307179586232;       // nearest double to 2*pi
constexpr double TWO_PI_LO = 2.4492935982947064e-16;     // 2*pi - TWO_PI_HI
constexpr double INV_TWO_PI = 0.15915494309189535;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  // round to nearest even (inputs here are finite)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ __bf16 bits_as_bf16(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

// IEEE half: round to nearest even, and back (exact)
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Angle pos * theta reduced to [-pi, pi] in fp64, returned as fp32.
__device__ __forceinline__ float reduce_angle(double pos, double theta) {
  double a = pos * theta;
  double n = rint(a * INV_TWO_PI);
  double r = fma(-n, TWO_PI_HI, a);
  r = fma(-n, TWO_PI_LO, r);
  return (float)r;
}

// Double-double accumulation (Knuth TwoSum): (hi, lo) += x, nearly exact for
// sums of non-negative terms, so the rounded result hardly depends on order.
__device__ __forceinline__ void dd_add(double& hi, double& lo, double x) {
  double s = hi + x;
  double bp = s - hi;
  double err = (hi - (s - bp)) + (x - bp);
  hi = s;
  lo += err;
}
__device__ __forceinline__ void dd_add_dd(double& hi, double& lo, double xh, double xl) {
  dd_add(hi, lo, xh);
  lo += xl;
}
__device__ __forceinline__ double dd_round(double hi, double lo) {
  double s = hi + lo;
  return s;
}

}  // namespace dca
