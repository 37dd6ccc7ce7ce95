// Register-resident 2048-point randomized Walsh-Hadamard transform for one
// wave64, plus the fused int4 group quantizer and fp32 store of its result.
// Used by the n = 2048 row kernel and the mixed-radix (m x 2048) kernel.
//
// What is computed: v = H_2048 (d * x) for one 2048-element chunk (the
// normalisation 1/sqrt(2048) is applied by the caller's output step);
// "Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Hypothesis and
// Method; the 2048-point Hadamard of the "Llama-3.2-1B-Instruct-HadamardSpin-
// 4bits" card, How it Works.
//
// Data placement.  Lane l loads bf16 elements j*512 + 8L + e (j < 4, e < 8,
// L the lane's logical index, below) with four 16-byte loads, so element-index
// bits 0-2 (e) and 9-10 (j) live in registers and bits 3-8 in lane bits 0-5.
// The Walsh-Hadamard butterfly over a bit never moves data, so the stages run
// in any order:
//   bits 0,1     the 4-point transform of (d*x) from two packed bf16 pairs as
//                six v_dot2_f32_bf16 (widening, sign diagonal and two stages);
//   bits 2,9,10  register butterflies;
//   bit 8        v_permlane32_swap exchanges lane bit 5 with register bit j1
//                (already transformed), then a register butterfly;
//   bit 7        v_permlane16_swap exchanges lane bit 4 with register bit j0;
//   bits 3-6     lane bits 0-3, one v_fmac_f32_dpp each (partner through DPP,
//                per-lane +-1 multiplier).  DPP offers lane xor 1, 2 (quad_perm),
//                7 (row_half_mirror) and 8 (row_ror:8) but no xor 4, so within
//                each 16-lane row the lanes are relabelled by a GF(2)-linear map:
//                logical index a = (a0, a1, a2, a3) sits in physical lane
//                q = a0*1 ^ a1*2 ^ a2*7 ^ a3*8, making logical bit 2 physical
//                xor 7.  The loads stay coalesced (a permutation of 16 lanes).
//                Lane sign bookkeeping: the fmac computes own + beta * partner,
//                which is the butterfly up to a per-lane sign tau that depends
//                only on the transformed bits; tau = (-1)^popcount(a) at the end
//                and is folded into the output multiplier.
// Final placement: register (j, e) of lane l holds tau times element
//   e | a << 3 | j0 << 7 | j1 << 8 | (l >> 4) << 9.
// A quantization group of 128 is then 8 registers x one 16-lane row, 32 is 8
// registers x a quad, 64 is 8 registers x 8 lanes, 256 spans j0 too.
#pragma once

#include "hr_device.h"

namespace hr {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// DPP controls
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// w[i] += dpp(w[i]) * sigma for 16 registers.  All 16 are operands of one
// asm block that opens with s_nop 1, so every VALU write of them has retired
// at least two wait states before its DPP read.
#define HR_FMAC_DPP16(w, sigma, CTRL) \
  asm volatile("s_nop 1\n\t" \
"v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
"v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]), "+v"(w[6]), "+v"(w[7]), "+v"(w[8]), "+v"(w[9]), "+v"(w[10]), "+v"(w[11]), "+v"(w[12]), "+v"(w[13]), "+v"(w[14]), "+v"(w[15]) \
  : "v"(sigma))

__device__ __forceinline__ void bfly(float& a, float& b) {
  const float t = a;
  a = t + b;
  b = t - b;
}

// v_dot2_f32_bf16 in its VOP3P form (separate accumulator, sign modifiers on
// the halves of the second operand): d = x.lo * s.lo + x.hi * s.hi + c.
__device__ __forceinline__ float dot2_pp(uint32_t x, uint32_t s) {  // ( s.lo,  s.hi) + 0
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(x), "v"(s));
  return d;
}
__device__ __forceinline__ float dot2_pm(uint32_t x, uint32_t s) {  // ( s.lo, -s.hi) + 0
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(d) : "v"(x), "v"(s));
  return d;
}
__device__ __forceinline__ float dot2_pp_c(uint32_t x, uint32_t s, float c) {  // ( s.lo,  s.hi) + c
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(x), "v"(s), "v"(c));
  return d;
}
__device__ __forceinline__ float dot2_pm_c(uint32_t x, uint32_t s, float c) {  // ( s.lo, -s.hi) + c
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3 neg_hi:[0,1,0]" : "=v"(d) : "v"(x), "v"(s), "v"(c));
  return d;
}
__device__ __forceinline__ float dot2_mm_c(uint32_t x, uint32_t s, float c) {  // (-s.lo, -s.hi) + c
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3 neg_lo:[0,1,0] neg_hi:[0,1,0]" : "=v"(d) : "v"(x), "v"(s), "v"(c));
  return d;
}
__device__ __forceinline__ float dot2_mp_c(uint32_t x, uint32_t s, float c) {  // (-s.lo,  s.hi) + c
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3 neg_lo:[0,1,0]" : "=v"(d) : "v"(x), "v"(s), "v"(c));
  return d;
}

// Max over lanes of non-negative fp32 values, compared as unsigned bit
// patterns (same order for non-negative floats, and no NaN canonicalisation).
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t a) {
  const uint32_t b = (uint32_t)__builtin_amdgcn_mov_dpp((int)a, CTRL, 0xf, 0xf, true);
  return a > b ? a : b;
}

// Correctly rounded fp32 a / D for D = 7 and D = 127 (one residual
// correction of a * RN(1/D); checked against IEEE division over every
// mantissa at several exponents and over all subnormal inputs).
template <int D>
__device__ __forceinline__ float div_const(float a) {
  static_assert(D == 7 || D == 127, "checked divisors only");
  const float rd = 1.0f / (float)D;
  const float q0 = a * rd;
  const float r = fmaf(-q0, (float)D, a);
  return fmaf(r, rd, q0);
}
__device__ __forceinline__ float div7(float a) { return div_const<7>(a); }

// Pack 8 codes held as magic-rounded floats (bits = 0x4B400008 + q, so the
// low byte is q + 8 in [1, 15] with clean high nibble) into one dword of
// two's-complement nibbles, element 0 in the low nibble.
__device__ __forceinline__ uint32_t pack8(const float* r) {
  uint32_t u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) u[e] = __float_as_uint(r[e]);
  const uint32_t p01 = (u[1] << 4) | u[0];
  const uint32_t p23 = (u[3] << 4) | u[2];
  const uint32_t p45 = (u[5] << 4) | u[4];
  const uint32_t p67 = (u[7] << 4) | u[6];
  const uint32_t lo = (p23 << 8) | p01;      // bits 0-15 clean
  const uint32_t hi = (p67 << 8) | p45;
  const uint32_t w = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  return w ^ 0x88888888u;
}

// Per-lane constants of the 2048-point transform.
struct Lane2048 {
  int lane;          // physical lane 0..63
  int a4;            // logical index within the 16-lane row
  int lg;            // logical lane: element bits 3-8 at load time
  float beta0, beta1, beta2, beta3;
  float tau;         // sign of the lane's results after the DPP stages
  uint32_t sp[4][4]; // bf16 sign pairs (d_{2k}, d_{2k+1}) of the lane's elements
};

// signs: the chunk's 2048 +-1 entries, or null for all +1.
__device__ __forceinline__ void lane2048_init(Lane2048& L, const int8_t* __restrict__ signs) {
  L.lane = threadIdx.x & 63;
  const int q = L.lane & 15;
  L.a4 = (q & 12) | ((q ^ (q >> 2)) & 1) | ((((q >> 1) ^ (q >> 2)) & 1) << 1);
  L.lg = (L.lane & 48) | L.a4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (signs) {
      const uint2 s8 = *reinterpret_cast<const uint2*>(signs + j * 512 + 8 * L.lg);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = k < 2 ? s8.x : s8.y;
        const int b0 = (int8_t)((w >> (16 * (k & 1))) & 0xFF);
        const int b1 = (int8_t)((w >> (16 * (k & 1) + 8)) & 0xFF);
        L.sp[j][k] = (b0 < 0 ? 0xBF80u : 0x3F80u) | ((b1 < 0 ? 0xBF80u : 0x3F80u) << 16);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) L.sp[j][k] = 0x3F803F80u;
    }
  }
  L.beta0 = (L.a4 & 1) ? -1.0f : 1.0f;
  L.beta1 = (L.a4 & 2) ? -1.0f : 1.0f;
  L.beta2 = (L.a4 & 4) ? -1.0f : 1.0f;
  L.beta3 = (L.a4 & 8) ? -1.0f : 1.0f;
  L.tau = (__builtin_popcount(L.a4) & 1) ? -1.0f : 1.0f;
}

// The four 16-byte bf16 loads of a 2048-element chunk.
__device__ __forceinline__ void load2048_bf16(const Lane2048& L, const uint16_t* __restrict__ chunk,
                                              u32x4 (&raw)[4]) {
  const u32x4* xr = reinterpret_cast<const u32x4*>(chunk);
#pragma unroll
  for (int j = 0; j < 4; ++j) raw[j] = __builtin_nontemporal_load(xr + j * 64 + L.lg);
}

// Element bits 0 and 1 from packed bf16 pairs (dot products).
__device__ __forceinline__ void fwht2048_first_bf16(const Lane2048& L, const u32x4 (&raw)[4],
                                                    float (&v)[4][8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t p0 = w[2 * h], p1 = w[2 * h + 1];
      const uint32_t s0 = L.sp[j][2 * h], s1 = L.sp[j][2 * h + 1];
      const float A = dot2_pp(p0, s0);           // u0 + u1
      const float B = dot2_pm(p0, s0);           // u0 - u1
      v[j][4 * h + 0] = dot2_pp_c(p1, s1, A);    // u0 + u1 + u2 + u3
      v[j][4 * h + 1] = dot2_pm_c(p1, s1, B);    // u0 - u1 + u2 - u3
      v[j][4 * h + 2] = dot2_mm_c(p1, s1, A);    // u0 + u1 - u2 - u3
      v[j][4 * h + 3] = dot2_mp_c(p1, s1, B);    // u0 - u1 - u2 + u3
    }
  }
}

// Element bits 0 and 1 from fp32 input.
__device__ __forceinline__ void fwht2048_first_f32(const Lane2048& L, const float* __restrict__ chunk,
                                                   float (&v)[4][8]) {
  const f32x4* xr = reinterpret_cast<const f32x4*>(chunk);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 a = __builtin_nontemporal_load(xr + j * 128 + 2 * L.lg);
    const f32x4 b = __builtin_nontemporal_load(xr + j * 128 + 2 * L.lg + 1);
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float d0 = (L.sp[j][k] & 0x8000u) ? -1.0f : 1.0f;
      const float d1 = (L.sp[j][k] & 0x80000000u) ? -1.0f : 1.0f;
      const float u0 = f[2 * k] * d0;
      v[j][2 * k] = fmaf(f[2 * k + 1], d1, u0);
      v[j][2 * k + 1] = fmaf(f[2 * k + 1], -d1, u0);
    }
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      bfly(v[j][e], v[j][e + 2]);
      bfly(v[j][e + 1], v[j][e + 3]);
    }
  }
}

// Remaining stages: element bits 2, 9, 10 in registers, 8 and 7 through the
// permlane swaps, 3-6 through DPP.  Afterwards the placement is the final one.
__device__ __forceinline__ void fwht2048_rest(const Lane2048& L, float (&v)[4][8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) bfly(v[j][e], v[j][e + 4]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bfly(v[0][e], v[1][e]);
    bfly(v[2][e], v[3][e]);
    bfly(v[0][e], v[2][e]);
    bfly(v[1][e], v[3][e]);
  }
  // element bit 8: lane bit 5 <-> register bit j1, then butterfly
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j][e]),
                                                      __float_as_uint(v[j + 2][e]), false, false);
      v[j][e] = __uint_as_float(r[0]);
      v[j + 2][e] = __uint_as_float(r[1]);
      bfly(v[j][e], v[j + 2][e]);
    }
  // element bit 7: lane bit 4 <-> register bit j0, then butterfly
#pragma unroll
  for (int j = 0; j < 4; j += 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j][e]),
                                                      __float_as_uint(v[j + 1][e]), false, false);
      v[j][e] = __uint_as_float(r[0]);
      v[j + 1][e] = __uint_as_float(r[1]);
      bfly(v[j][e], v[j + 1][e]);
    }
  // element bits 3-6 (lane bits 0-3), logical bits 0, 1, 3, 2 via DPP
  float* lo = &v[0][0];   // registers of j = 0, 1
  float* hi = &v[2][0];   // registers of j = 2, 3
  HR_FMAC_DPP16(lo, L.beta0, "quad_perm:[1,0,3,2]");
  HR_FMAC_DPP16(hi, L.beta0, "quad_perm:[1,0,3,2]");
  HR_FMAC_DPP16(lo, L.beta1, "quad_perm:[2,3,0,1]");
  HR_FMAC_DPP16(hi, L.beta1, "quad_perm:[2,3,0,1]");
  HR_FMAC_DPP16(lo, L.beta3, "row_ror:8");
  HR_FMAC_DPP16(hi, L.beta3, "row_ror:8");
  HR_FMAC_DPP16(lo, L.beta2, "row_half_mirror");
  HR_FMAC_DPP16(hi, L.beta2, "row_half_mirror");
}

// Element offset (within the chunk) of register block j, element 0, in the
// final placement.
__device__ __forceinline__ int elem2048(const Lane2048& L, int j) {
  return L.a4 * 8 + (j & 1) * 128 + (j >> 1) * 256 + (L.lane >> 4) * 512;
}

// Store ymul * v as fp32 (ymul folds tau and the normalisation).
__device__ __forceinline__ void store2048_f32(const Lane2048& L, const float (&v)[4][8], float ymul,
                                              float* __restrict__ ychunk) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x4* dst = reinterpret_cast<f32x4*>(ychunk + elem2048(L, j));
    const f32x4 o0 = {v[j][0] * ymul, v[j][1] * ymul, v[j][2] * ymul, v[j][3] * ymul};
    const f32x4 o1 = {v[j][4] * ymul, v[j][5] * ymul, v[j][6] * ymul, v[j][7] * ymul};
    __builtin_nontemporal_store(o0, dst);
    __builtin_nontemporal_store(o1, dst + 1);
  }
}

// Quantize the chunk: y = v * norm * tau (tau = +-1 per lane), groups of G
// consecutive elements, scale = fp32 absmax / 7 (stored as fp16 or fp32),
// codes by a magic-number fma (round to nearest even) and nibble packing.
//   codes_dw  the chunk's packed codes as dwords (2048 codes = 256 dwords)
//   scales    scale array; the chunk's first group is at index sbase
template <int G, bool SCALE_F16>
__device__ __forceinline__ void quant2048(const Lane2048& L, const float (&v)[4][8], float norm,
                                          float tau, uint32_t* __restrict__ codes_dw,
                                          void* __restrict__ scales, int64_t sbase) {
  const int lane = L.lane;
  // group absmax of the unnormalised values
  float m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = fmaxf(fabsf(v[j][0]), fabsf(v[j][1]));
#pragma unroll
    for (int e = 2; e < 8; ++e) a = fmaxf(a, fabsf(v[j][e]));
    uint32_t ab = __float_as_uint(a);
    ab = umax_dpp<kQuadXor1>(ab);
    ab = umax_dpp<kQuadXor2>(ab);
    if (G >= 64) ab = umax_dpp<kRowHalfMirror>(ab);
    if (G >= 128) ab = umax_dpp<kRowMirror>(ab);
    m[j] = __uint_as_float(ab);
  }
  if (G == 256) {
    m[0] = m[1] = fmaxf(m[0], m[1]);
    m[2] = m[3] = fmaxf(m[2], m[3]);
  }
  // scale of one group per lane: the lane computes the group of register
  // block js (G <= 128: js = lane & 3; G = 256: js = 2 * (lane & 1))
  const int js = (G == 256) ? 2 * (lane & 1) : (lane & 3);
  const float mv = js == 0 ? m[0] : js == 1 ? m[1] : js == 2 ? m[2] : m[3];
  const float a = mv * norm;                 // absmax of y = v * norm (norm > 0)
  const float s32 = div7(a);
  float s;
  if (SCALE_F16) s = (float)(_Float16)s32; else s = s32;
  // an fp32 scale below 2^-100 would overflow its reciprocal: the group's
  // values and scale are then both taken x 2^64 (exact; same quotients)
  const float up = (!SCALE_F16 && s < 0x1p-100f) ? 0x1p64f : 1.0f;
  const float k = s > 0.0f ? norm * __builtin_amdgcn_rcpf(s * up) : 0.0f;
  const bool need_up = !SCALE_F16 && s > 0.0f && s < 0x1p-100f;
  // fp16-subnormal (or fp32-denormal) scales are imprecise: clamp needed
  const bool need_clamp = s > 0.0f && s < (SCALE_F16 ? 6.103515625e-05f : 1.17549435e-38f);
  // writer lanes store the scale of their group
  {
    int g = -1;
    if (G == 32) g = (L.a4 >> 2) + 4 * js + 16 * (lane >> 4);
    else if (G == 64) g = (lane & 4) ? -1 : (L.a4 >> 3) + 2 * js + 8 * (lane >> 4);
    else if (G == 128) g = (lane & 12) ? -1 : js + 4 * (lane >> 4);
    else g = (lane & 14) ? -1 : (js >> 1) + 2 * (lane >> 4);
    if (g >= 0) {
      if (SCALE_F16) reinterpret_cast<_Float16*>(scales)[sbase + g] = (_Float16)s32;
      else reinterpret_cast<float*>(scales)[sbase + g] = s32;
    }
  }
  // broadcast each group's multiplier to every lane of its quad; the lane
  // sign tau is this lane's own, so it is applied after the broadcast
  float kj[4];
  if (G == 256) {
    kj[0] = kj[1] = dpp<0x00>(k);          // quad_perm [0,0,0,0]
    kj[2] = kj[3] = dpp<0x55>(k);          // quad_perm [1,1,1,1]
  } else {
    kj[0] = dpp<0x00>(k);
    kj[1] = dpp<0x55>(k);
    kj[2] = dpp<0xAA>(k);
    kj[3] = dpp<0xFF>(k);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) kj[j] *= tau;
  const bool clamp = __builtin_amdgcn_ballot_w64(need_clamp) != 0;
  const bool tiny = !SCALE_F16 && __builtin_amdgcn_ballot_w64(need_up) != 0;
  float uj[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  if (tiny) {
    if (G == 256) {
      uj[0] = uj[1] = dpp<0x00>(up);
      uj[2] = uj[3] = dpp<0x55>(up);
    } else {
      uj[0] = dpp<0x00>(up);
      uj[1] = dpp<0x55>(up);
      uj[2] = dpp<0xAA>(up);
      uj[3] = dpp<0xFF>(up);
    }
  }
  const float M = 12582920.0f;              // 1.5 * 2^23 + 8
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r[8];
    if (tiny) {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = fmaf(v[j][e] * uj[j], kj[j], M);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = fmaf(v[j][e], kj[j], M);
    }
    if (clamp) {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = __builtin_amdgcn_fmed3f(r[e], M - 7.0f, M + 7.0f);
    }
    __builtin_nontemporal_store(pack8(r), codes_dw + (elem2048(L, j) >> 3));
  }
}

}  // namespace hr
