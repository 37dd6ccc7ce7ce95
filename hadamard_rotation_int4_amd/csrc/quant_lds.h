// Per-group int4 or int8 quantization of one row held in LDS, done by a whole
// workgroup (blockDim.x a multiple of 64).  Used by the workgroup-per-row
// kernels (generic rotation, mixed radix, butterfly).
#pragma once

#include "hr_device.h"
#include "fwht2048.h"

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
// (values already normalised), spread over the whole workgroup: G / 8 lanes
// share a group, each owning 8 consecutive values (two 16-byte LDS reads), so
// a wave covers 512 / G groups at a time.  The group absmax is reduced by DPP
// and permlane steps inside the lane group; the scale is the correctly
// rounded absmax / 7, and the codes are the fused kernels': y times the
// reciprocal of the stored scale, rounded by the magic-number fma (the
// decision differs from y / s with ties away from zero only within a few ulps
// of a midpoint), clamped to +-7 where some group of the wave has a scale
// below the normal range; each lane stores its 8 codes as one 32-bit word.
// pos maps an in-row index (a multiple of 4) to its LDS position (groups of 4
// contiguous).
struct IdentityPos {
  __device__ int operator()(int i) const { return i; }
};
template <typename Pos = IdentityPos>
__device__ __forceinline__ void quant_rows_from_lds(const float* vals, int pitch, int nr, int n,
                                                    int G, uint8_t* __restrict__ codes,
                                                    int64_t row0, void* __restrict__ scales,
                                                    int scale_f16, Pos pos = Pos()) {
  const int lpg = G >> 3;                       // lanes per group: 4, 8, 16 or 32
  const int gpr = n / G;                        // groups per row
  const int total = nr * gpr * lpg;             // (row, group, lane) items
  for (int it = threadIdx.x; it - (int)(threadIdx.x & 63) < total; it += blockDim.x) {
    // every lane of a wave runs the shuffles; items past the end use value 0
    const bool live = it < total;
    const int item = live ? it : 0;
    const int l = item % lpg, rg = item / lpg;
    const int r = rg / gpr, g = rg - r * gpr;
    float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
    if (live) {
      const float* rowp = vals + r * pitch;
      v0 = *reinterpret_cast<const float4*>(rowp + pos(g * G + 8 * l));
      v1 = *reinterpret_cast<const float4*>(rowp + pos(g * G + 8 * l + 4));
    }
    // group absmax over the lpg lanes: DPP steps inside a 16-lane row, then
    // row pairs by a permlane swap (non-negative values compare as unsigned
    // bit patterns)
    const float m0 = fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fabsf(v0.z));
    const float m1 = fmaxf(fmaxf(fabsf(v0.w), fabsf(v1.x)), fabsf(v1.y));
    uint32_t mu = __float_as_uint(fmaxf(fmaxf(m0, m1), fmaxf(fabsf(v1.z), fabsf(v1.w))));
    mu = umax_dpp<kQuadXor1>(mu);
    mu = umax_dpp<kQuadXor2>(mu);
    if (lpg >= 8) mu = umax_dpp<kRowHalfMirror>(mu);
    if (lpg >= 16) mu = umax_dpp<kRowMirror>(mu);
    if (lpg >= 32) {
      const auto sw = __builtin_amdgcn_permlane16_swap(mu, mu, false, false);
      mu = sw[0] > sw[1] ? sw[0] : sw[1];
    }
    const float mx = __uint_as_float(mu);
    if (!live) continue;
    const float s32 = div_const<7>(mx);
    const float sc = scale_f16 ? (float)(_Float16)s32 : s32;
    const int64_t row = row0 + r;
    if (l == 0) store_scale(scales, row * gpr + g, s32, scale_f16);
    // an fp32 scale below 2^-100 would overflow its reciprocal: y and s are
    // then both taken x 2^64 (exact; same quotients)
    const float up = (!scale_f16 && sc < 0x1p-100f) ? 0x1p64f : 1.0f;
    const float k = sc > 0.0f ? __builtin_amdgcn_rcpf(sc * up) : 0.0f;
    // the x 2^64 and the clamp only where some group of the wave needs them
    // (wave-uniform branches); elsewhere |y k| rounds to at most 7
    const bool tiny = __builtin_amdgcn_ballot_w64(!scale_f16 && sc > 0.0f && sc < 0x1p-100f) != 0;
    const bool clamp =
        __builtin_amdgcn_ballot_w64(sc > 0.0f && sc < (scale_f16 ? 6.103515625e-05f : 1.17549435e-38f)) != 0;
    float y[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    if (tiny) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= up;
    }
    // q + 1.5 * 2^23 + 8 holds q + 8 in its low nibble (ties to even)
    constexpr float MQ = 12582920.0f;
    float rr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rr[e] = fmaf(y[e], k, MQ);
    if (clamp) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rr[e] = __builtin_amdgcn_fmed3f(rr[e], MQ - 7.0f, MQ + 7.0f);
    }
    reinterpret_cast<uint32_t*>(codes + row * (n / 2) + g * (G / 2))[l] = pack8(rr);
  }
}

}  // namespace hr
