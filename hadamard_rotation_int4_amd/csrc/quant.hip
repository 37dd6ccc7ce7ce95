// Per-group symmetric absmax quantization without a rotation: int4 (packed
// two per byte) or int8 codes with fp16 or fp32 group scales.
//
// What is computed ("Experiment -- Hadamard rotation for int4 (W4A4)
// accuracy", Method: per-group symmetric integer quantization at any bit
// width; its Results table quantizes the operands both plain and after the
// Hadamard rotation, and this kernel is the plain case): for every group of G
// consecutive values y of a row, s32 = max|y| / qmax (correctly rounded fp32),
// s = fp16(s32) or s32 (stored), q = y / s rounded to nearest, clamped to
// [-qmax, qmax], qmax = 7 (int4) or 127 (int8); q = 0 when s = 0.
//
// The [rows][n] input is one flat stream: G divides n, so flat group f holds
// elements f G .. f G + G - 1 and its scale is scales[f].  Lane l of a wave
// takes octet o0 + l (elements 8 o .. 8 o + 7: one 16-byte bf16 load or two
// fp32 loads), so a group is G / 8 consecutive lanes.  The group absmax is a
// max over the lane's 8 values and then over its G / 8 lanes (DPP quad
// exchanges, row half-mirror, row mirror, permlane16 swap).  Codes leave as
// one dword (int4) or two (int8) per lane, contiguous across the wave.
#include "hr_internal.h"
#include "fwht2048.h"

namespace hr {

constexpr int kQuantThreads = 256;

template <int G, int BITS, bool SCALE_F16, bool IN_BF16>
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const void* __restrict__ x,
                                                              int64_t octets,
                                                              uint8_t* __restrict__ codes,
                                                              void* __restrict__ scales, bool nt) {
  constexpr int L = G / 8;                       // lanes per group
  constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
  // y k + M leaves the rounded code in the low mantissa bits (ties to even);
  // + 8 biases int4 codes to the nibble range pack8 expects
  constexpr float M = BITS == 8 ? 12582912.0f : 12582920.0f;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  // every lane of a wave runs the same number of iterations (the exchanges
  // below need the whole wave); lanes past the end load zeros and store nothing
  const int64_t base0 = (int64_t)blockIdx.x * kQuantThreads + (threadIdx.x & ~63);
  for (int64_t wbase = base0; wbase < octets; wbase += stride) {
    const int64_t o = wbase + lane;
    const bool live = o < octets;
    float y[8];
    if (IN_BF16) {
      const u32x4* xp = reinterpret_cast<const u32x4*>(x) + o;
      const u32x4 r = live ? (nt ? __builtin_nontemporal_load(xp) : *xp) : (u32x4){0u, 0u, 0u, 0u};
      const uint32_t w[4] = {r[0], r[1], r[2], r[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] = __uint_as_float(w[i] << 16);
        y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4* xp = reinterpret_cast<const f32x4*>(x) + 2 * o;
      const f32x4 r0 = live ? (nt ? __builtin_nontemporal_load(xp) : xp[0]) : z;
      const f32x4 r1 = live ? (nt ? __builtin_nontemporal_load(xp + 1) : xp[1]) : z;
      y[0] = r0[0]; y[1] = r0[1]; y[2] = r0[2]; y[3] = r0[3];
      y[4] = r1[0]; y[5] = r1[1]; y[6] = r1[2]; y[7] = r1[3];
    }
    float m = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fabsf(y[2]));
    m = fmaxf(fmaxf(m, fabsf(y[3])), fabsf(y[4]));
    m = fmaxf(fmaxf(m, fabsf(y[5])), fmaxf(fabsf(y[6]), fabsf(y[7])));
    // absmax over the group's L lanes (non-negative floats compare as integers)
    uint32_t a = __float_as_uint(m);
    a = umax_dpp<kQuadXor1>(a);
    a = umax_dpp<kQuadXor2>(a);
    if (L >= 8) a = umax_dpp<kRowHalfMirror>(a);
    if (L >= 16) a = umax_dpp<kRowMirror>(a);
    if (L >= 32) {
      const auto sw = __builtin_amdgcn_permlane16_swap(a, a, false, false);
      a = sw[0] > sw[1] ? sw[0] : sw[1];
    }
    const float s32 = div_const<BITS == 8 ? 127 : 7>(__uint_as_float(a));
    const float s = SCALE_F16 ? (float)(_Float16)s32 : s32;
    // a scale below 2^-100 (fp32 scales of tiny groups) would overflow its
    // reciprocal: the group's values and scale are then both taken x 2^64,
    // which is exact and leaves every quotient unchanged
    const float up = s < 0x1p-100f ? 0x1p64f : 1.0f;
    const float k = s > 0.0f ? __builtin_amdgcn_rcpf(s * up) : 0.0f;
    float rr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      rr[e] = __builtin_amdgcn_fmed3f(fmaf(y[e] * up, k, M), M - QMAX, M + QMAX);
    if (live) {
      if (BITS == 4) {
        reinterpret_cast<uint32_t*>(codes)[o] = pack8(rr);
      } else {
        uint32_t u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = __float_as_uint(rr[e]);
        const uint32_t d0 = (__builtin_amdgcn_perm(u[3], u[2], 0x0c0c0400u) << 16) |
                            __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u);
        const uint32_t d1 = (__builtin_amdgcn_perm(u[7], u[6], 0x0c0c0400u) << 16) |
                            __builtin_amdgcn_perm(u[5], u[4], 0x0c0c0400u);
        reinterpret_cast<uint2*>(codes)[o] = make_uint2(d0, d1);
      }
      if ((lane & (L - 1)) == 0) {
        const int64_t f = o / L;
        if (SCALE_F16) reinterpret_cast<_Float16*>(scales)[f] = (_Float16)s32;
        else reinterpret_cast<float*>(scales)[f] = s32;
      }
    }
  }
}

template <int G, int BITS, bool F16>
static void launch_q3(const QuantArgs& a, int64_t octets, int64_t blocks, hipStream_t s) {
  if (a.x_bf16)
    hipLaunchKernelGGL((quant_kernel<G, BITS, F16, true>), dim3((unsigned)blocks), dim3(kQuantThreads),
                       0, s, a.x, octets, a.codes, a.scales,
                       octets * (a.x_bf16 ? 16 : 32) >= kStreamBytes);
  else
    hipLaunchKernelGGL((quant_kernel<G, BITS, F16, false>), dim3((unsigned)blocks), dim3(kQuantThreads),
                       0, s, a.x, octets, a.codes, a.scales,
                       octets * (a.x_bf16 ? 16 : 32) >= kStreamBytes);
}

template <int G>
static void launch_q2(const QuantArgs& a, int64_t octets, int64_t blocks, hipStream_t s) {
  if (a.bits == 8) {
    if (a.scale_f16) launch_q3<G, 8, true>(a, octets, blocks, s);
    else launch_q3<G, 8, false>(a, octets, blocks, s);
  } else {
    if (a.scale_f16) launch_q3<G, 4, true>(a, octets, blocks, s);
    else launch_q3<G, 4, false>(a, octets, blocks, s);
  }
}

hipError_t launch_quant(const QuantArgs& a, hipStream_t s) {
  const int64_t octets = a.rows * (int64_t)(a.n / 8);
  int64_t blocks = (octets + kQuantThreads - 1) / kQuantThreads;
  // one octet per lane: the hardware hands workgroups to the CUs that finish
  // first (bf16 65536 x 2048, G = 128, HBM-resident, same box, with the
  // nontemporal loads: 63.8 -> 57.4 us against a grid of 2048 workgroups
  // striding over the rows); grid-stride only beyond 2^20 workgroups
  if (blocks > (1 << 20)) blocks = 1 << 20;
  switch (a.group) {
    case 32: launch_q2<32>(a, octets, blocks, s); break;
    case 64: launch_q2<64>(a, octets, blocks, s); break;
    case 128: launch_q2<128>(a, octets, blocks, s); break;
    default: launch_q2<256>(a, octets, blocks, s); break;
  }
  return hipGetLastError();
}

}  // namespace hr
