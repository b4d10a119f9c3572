// Device-side helpers shared by the libmoe kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest, ties to even (finite inputs; NaN maps to a quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// round a binary64 value directly to bf16 (nearest, ties to even), so that a
// value computed exactly in double is rounded once.  Values below the bf16
// normal range go through fp32 (they do not occur on the layer's data).
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(d));
  const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
  const int e = static_cast<int>((u >> 52) & 0x7ffu) - 1023;
  if (e < -126) return f32_to_bf16(static_cast<float>(d));
  if (e > 127) return static_cast<uint16_t>(sign | 0x7f80u);
  const uint64_t mant = u & 0xfffffffffffffull;
  const uint32_t keep = static_cast<uint32_t>(mant >> 45);
  const uint64_t rest = mant & ((1ull << 45) - 1);
  uint32_t bits = (static_cast<uint32_t>(e + 127) << 7) | keep;
  if (rest > (1ull << 44) || (rest == (1ull << 44) && (keep & 1u))) ++bits;  // carries into the exponent
  return static_cast<uint16_t>(sign | bits);
}

// bf16(relu(h)^2), rounded once (nearest, ties to even) from the exact
// square: h*h = hi + lo exactly, hi = fp32(h*h) and lo = fma(h, h, -hi).
// The nearest bf16 of hi + lo is that of hi unless hi lies exactly on a bf16
// midpoint (low 16 bits 0x8000): every other fp32 value is at least one fp32
// ulp from the midpoints, farther than |lo| <= ulp(hi) / 2.  On a midpoint
// the sign of lo breaks the tie; lo == 0 is a true tie (to even).
__device__ __forceinline__ uint16_t relu_sq_bf16(float h) {
  if (!(h > 0.f)) return 0;
  const float hi = h * h;
  const float lo = __builtin_fmaf(h, h, -hi);
  uint32_t u = __float_as_uint(hi);
  if ((u & 0xffffu) == 0x8000u && lo != 0.f) {
    if (lo > 0.f) u += 0x8000u;  // above the midpoint: up; below: truncate
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
  }
  return static_cast<uint16_t>(u >> 16);
}

// ----------------------------------------------------------------- E4M3 (OCP E4M3FN)
// 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, largest finite 448,
// subnormals m * 2^-9.  Encode: nearest-even, finite inputs saturate to 448,
// sign bit set iff v < 0.
//
// The encoders use the hardware converts (v_cvt_pk_fp8_f32 here,
// v_cvt_scalef32_pk_fp4_f32 for E2M1 below, unit scale).  Over all fp32 bit
// patterns with |v| <= 464 (E4M3) or |v| <= 1e30 (E2M1) they give the codes of
// a bit-level encoder of the definition, except that they keep the sign of
// -0.  Clamping to the largest finite value first makes saturation hold for
// every input, and adding +0 turns -0 into +0.
__device__ __forceinline__ float e4m3_prep(float v) {
  return __builtin_amdgcn_fmed3f(v, -448.f, 448.f) + 0.f;
}

// codes of a, b, c, d in bytes 0, 1, 2, 3
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(a), e4m3_prep(b), 0, false);
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(c), e4m3_prep(d), lo, true));
}

__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(v), 0.f, 0, false)) &
         0xffu;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 0u) {
    v = static_cast<float>(m) * 0.001953125f;  // m * 2^-9
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) 2^(e-7)
  }
  return (c & 0x80u) ? -v : v;
}

// ----------------------------------------------------------------- E2M1 (OCP FP4)
// 1 sign, 2 exponent bits (bias 1), 1 mantissa bit: {0, .5, 1, 1.5, 2, 3, 4, 6}.
// Encode: nearest-even, saturating to 6, sign bit set iff v < 0 (hardware
// convert, see the E4M3 encoders).
__device__ __forceinline__ float e2m1_prep(float v) {
  return __builtin_amdgcn_fmed3f(v, -6.f, 6.f) + 0.f;
}

__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, e2m1_prep(v), 0.f, 1.0f, 0) & 0xfu;
}

// codes of v[0..7]: element 2i in the low nibble of byte i
__device__ __forceinline__ uint32_t e2m1_encode8(const float* v) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_prep(v[0]), e2m1_prep(v[1]), 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_prep(v[2]), e2m1_prep(v[3]), 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_prep(v[4]), e2m1_prep(v[5]), 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_prep(v[6]), e2m1_prep(v[7]), 1.0f, 3);
  return w;
}

__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  // magnitudes by code: 0 .5 1 1.5 2 3 4 6
  const uint32_t m = c & 7u;
  const float mag = (m < 2u) ? 0.5f * static_cast<float>(m)
                             : __uint_as_float(((((m >> 1) - 1u) + 127u) << 23) | ((m & 1u) << 22));
  return (c & 8u) ? -mag : mag;
}

// ----------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// non-negative floats order like their bit patterns
__device__ __forceinline__ void atomic_max_nonneg(uint32_t* slot, float v) {
  atomicMax(slot, __float_as_uint(v));
}

// A tensor amax is accumulated into kAmaxSlots words (block b uses slot
// b % kAmaxSlots) so that thousands of blocks do not serialise on one
// address; readers take the max over the slots.
constexpr int kAmaxSlots = 64;

// max over the slots, computed by one wave (every lane gets the result)
__device__ __forceinline__ float read_amax_slots(const uint32_t* slots) {
  const int lane = threadIdx.x & 63;
  float v = lane < kAmaxSlots ? __uint_as_float(slots[lane]) : 0.f;
  return wave_max(v);
}

// block-wide max of a per-thread value, one atomic per block (blockDim.x <= 1024)
__device__ __forceinline__ void block_amax_to_slots(float v, uint32_t* slots) {
  __shared__ float part[16];
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.f;
    for (int w = 0; w < static_cast<int>((blockDim.x + 63) / 64); ++w) m = fmaxf(m, part[w]);
    atomic_max_nonneg(slots + (blockIdx.x % kAmaxSlots), m);
  }
}

}  // namespace moe
