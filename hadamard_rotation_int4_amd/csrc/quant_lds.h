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

// The same quantization for nr rows held in LDS at a pitch of `pitch` floats
// (values already normalised), spread over the whole workgroup: G / 4 lanes
// share a group, each owning 4 consecutive values (one 16-byte LDS read, no
// bank conflicts), so a wave covers 256 / G groups at a time.  The group
// absmax is reduced with shuffles inside the lane group; codes are taken
// against the stored scale with IEEE division and ties away from zero, and
// each lane stores its 4 codes as one 16-bit word.  pos maps an in-row index
// (a multiple of 4) to its LDS position (groups of 4 contiguous).
struct IdentityPos {
  __device__ int operator()(int i) const { return i; }
};
template <typename Pos = IdentityPos>
__device__ __forceinline__ void quant_rows_from_lds(const float* vals, int pitch, int nr, int n,
                                                    int G, uint8_t* __restrict__ codes,
                                                    int64_t row0, void* __restrict__ scales,
                                                    int scale_f16, Pos pos = Pos()) {
  const int lpg = G >> 2;                       // lanes per group: 8, 16, 32 or 64
  const int gpr = n / G;                        // groups per row
  const int total = nr * gpr * lpg;             // (row, group, lane) items
  for (int it = threadIdx.x; it - (int)(threadIdx.x & 63) < total; it += blockDim.x) {
    // every lane of a wave runs the shuffles; items past the end use value 0
    const bool live = it < total;
    const int item = live ? it : 0;
    const int l = item % lpg, rg = item / lpg;
    const int r = rg / gpr, g = rg - r * gpr;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) v = *reinterpret_cast<const float4*>(vals + r * pitch + pos(g * G + 4 * l));
    float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    for (int o = lpg >> 1; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (!live) continue;
    const float s32 = mx / 7.0f;
    const float sc = scale_f16 ? (float)(_Float16)s32 : s32;
    const int64_t row = row0 + r;
    if (l == 0) store_scale(scales, row * gpr + g, s32, scale_f16);
    const int q0 = quant_code_exact(v.x, sc), q1 = quant_code_exact(v.y, sc);
    const int q2 = quant_code_exact(v.z, sc), q3 = quant_code_exact(v.w, sc);
    const uint16_t w = (uint16_t)((q0 & 0xF) | ((q1 & 0xF) << 4) | ((q2 & 0xF) << 8) | ((q3 & 0xF) << 12));
    reinterpret_cast<uint16_t*>(codes + row * (n / 2) + g * (G / 2))[l] = w;
  }
}

}  // namespace hr
