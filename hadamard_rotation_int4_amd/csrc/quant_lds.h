// Per-group int4 or int8 quantization of one row held in LDS, done by a whole
// workgroup (blockDim.x a multiple of 64).  Used by the workgroup-per-row
// kernels (generic rotation, mixed radix, butterfly).
#pragma once

#include "hr_device.h"

namespace hr {

// vals: the row in LDS (n floats); each value is multiplied by `norm` first.
// One wave handles one group at a time: lanes reduce the group absmax, lane 0
// stores the scale (absmax / 7, or absmax / 127 for 8 bits), then lanes store
// pairs of codes packed into bytes (4 bits) or one int8 code per byte (8 bits).
__device__ __forceinline__ void quant_row_from_lds(const float* vals, float norm, int n, int G,
                                                   uint8_t* __restrict__ codes_row,
                                                   void* __restrict__ scales,
                                                   int64_t scale_base, int scale_f16,
                                                   int bits = 4) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int g = wave; g < n / G; g += nwaves) {
    const float* yg = vals + g * G;
    float mx = 0.0f;
    for (int e = lane; e < G; e += 64) mx = fmaxf(mx, fabsf(yg[e] * norm));
    mx = wave_max(mx);
    const float s32 = bits == 8 ? mx / 127.0f : mx / 7.0f;
    float s;
    if (scale_f16) s = (float)(_Float16)s32; else s = s32;
    if (lane == 0) store_scale(scales, scale_base + g, s32, scale_f16);
    if (bits == 8) {
      for (int e = lane; e < G; e += 64)
        codes_row[g * G + e] = (uint8_t)(int8_t)quant_code_exact(yg[e] * norm, s, 127.0f);
      continue;
    }
    for (int e = 2 * lane; e < G; e += 128) {
      const int q0 = quant_code_exact(yg[e] * norm, s);
      const int q1 = quant_code_exact(yg[e + 1] * norm, s);
      codes_row[(g * G + e) >> 1] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
    }
  }
}

}  // namespace hr
