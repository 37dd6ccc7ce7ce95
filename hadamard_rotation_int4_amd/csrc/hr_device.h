// Device helpers shared by the kernels of libhr.so (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hr {

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

template <typename T>
__device__ __forceinline__ float load_as_float(const T* p);

template <>
__device__ __forceinline__ float load_as_float<float>(const float* p) { return *p; }

template <>
__device__ __forceinline__ float load_as_float<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_float(*p);
}

// Store a group scale in the caller's scale dtype; returns the value the codes
// must be taken against (the stored one, widened to fp32).
__device__ __forceinline__ float store_scale(void* scales, int64_t idx, float s32, int scale_f16) {
  if (scale_f16) {
    _Float16 h = (_Float16)s32;  // v_cvt_f16_f32: round to nearest even
    reinterpret_cast<_Float16*>(scales)[idx] = h;
    return (float)h;
  }
  reinterpret_cast<float*>(scales)[idx] = s32;
  return s32;
}

// Reference-style code of one value: round half away from zero, clamp to +-7,
// zero for a zero scale.  Used by the straightforward kernels.
__device__ __forceinline__ int quant_code_exact(float y, float s, float qmax = 7.0f) {
  if (s == 0.0f) return 0;
  float t = y / s;                       // IEEE division
  float a = floorf(fabsf(t) + 0.5f);     // exact for |t| < 2^22
  a = fminf(a, qmax);
  int q = (int)a;
  return t < 0.0f ? -q : q;
}

// nibbles 0..3 of t moved to bits 0, 6, 12, 18
__device__ __forceinline__ uint32_t f6_spread4(uint32_t t) {
  const uint32_t u = (t & 0x00FFu) | ((t & 0xFF00u) << 4);   // nibbles at 0, 4, 12, 16
  return (u & 0x0F00Fu) | ((u & 0xF00F0u) << 2);              // nibbles at 0, 6, 12, 18
}

// 8 two's-complement nibbles (code e in bits 4 e .. 4 e + 3) -> 8 fp6 e2m3
// fields (q < 0) << 5 | |q| (field e in bits 6 e .. 6 e + 5 of 48)
__device__ __forceinline__ uint64_t f6_fields8(uint32_t x) {
  const uint32_t s = (x >> 3) & 0x11111111u;                 // sign of each nibble at its bit 0
  const uint32_t m = (x ^ (s * 15u)) + s;                     // |code| per nibble (0..8), no carries
  const uint32_t lo = f6_spread4(m & 0xFFFFu) | (f6_spread4(s & 0xFFFFu) << 5);
  const uint32_t hi = f6_spread4(m >> 16) | (f6_spread4(s >> 16) << 5);
  return (uint64_t)lo | ((uint64_t)hi << 24);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace hr
