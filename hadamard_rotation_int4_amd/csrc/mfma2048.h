// The 2048-point Sylvester Hadamard transform of one wave's bf16 chunk on
// bf16 matrix cores ("Experiment -- Hadamard rotation for int4 (W4A4)
// accuracy", Hypothesis and Method; "Llama-3.2-1B-Instruct-HadamardSpin-
// 4bits", How it Works), shared by the n = 2048 kernel and the mixed-radix
// kernel.
//
// Factorisation.  Write an element index as 128 a + k (a < 16, k < 128).
// H_2048[128a + k][128a' + c] = H_16[a][a'] H_128[k][c], so
//   Z[a][c]  = sum_k H_128[c][k] u[a][k]      u = d * x (exact in bf16)
//   Y[a'][c] = sum_a H_16[a'][a] Z[a][c]
// The first is a 128 x 128 contraction with +-1 entries and bf16 data; it runs
// on v_mfma_f32_16x16x32_bf16 with fp32 accumulation (every product is
// exact).  The second is four butterfly stages across the 16 lanes of a DPP
// row (one v_fmac_f32_dpp per register and stage, after a GF(2) relabel A of
// the lanes so that every partner is a DPP pattern; each lane's result then
// carries the sign tau, folded into the caller's output multiplier).
//
// Placement, lane l = q + 16 g:
//   B operand (data): for K-step s < 4, lane l holds the 8 elements
//     k = 8 g + 32 s + e (e < 8) of chunk a = A(q) (16 bytes at element
//     128 A(q) + 8 g + 32 s).
//   Result (tile T < 8): lane l register v holds tau * Y[A(q)][c] for
//     c = v + 4 T0 + 8 g + 32 T1 + 64 T2 (T = T0 + 2 T1 + 4 T2).
//   A operand (H_128): lane l holds tile row i = q and K group g.  With k bits
//     (e0 e1 e2 g0 g1 s0 s1) and c bits (i0 i1 T0 i2 i3 T1 T2), the entry is
//     (-1)^(i0 e0 + i1 e1 + i2 g0 + i3 g1) (-1)^(T0 e2) (-1)^(T1 s0 + T2 s1):
//     four distinct fragments cover all 32 (T, s) pairs.
#pragma once

#include "hr_internal.h"
#include "fwht2048.h"

namespace hr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The H_16 stages on the eight accumulator tiles, pinned to v[96:127] so that
// the MFMA results are transformed in place.  One v_fmac_f32_dpp per register
// and stage: own + beta * partner (partner through DPP).  The block opens with
// 24 wait states, more than the longest MFMA-write to VALU-read distance (the
// compiler does not guard inline asm against that hazard); between stages a
// register is rewritten 32 instructions before its next DPP read, far beyond
// the two wait states DPP needs.
#define HR_F1(r, b, CTRL) "v_fmac_f32_dpp v" #r ", v" #r ", %" #b " " CTRL " row_mask:0xf bank_mask:0xf\n\t"
#define HR_F4(r0, r1, r2, r3, b, CTRL) \
  HR_F1(r0, b, CTRL) HR_F1(r1, b, CTRL) HR_F1(r2, b, CTRL) HR_F1(r3, b, CTRL)
#define HR_STAGE32(b, CTRL)         \
  HR_F4(96, 97, 98, 99, b, CTRL)     \
  HR_F4(100, 101, 102, 103, b, CTRL) \
  HR_F4(104, 105, 106, 107, b, CTRL) \
  HR_F4(108, 109, 110, 111, b, CTRL) \
  HR_F4(112, 113, 114, 115, b, CTRL) \
  HR_F4(116, 117, 118, 119, b, CTRL) \
  HR_F4(120, 121, 122, 123, b, CTRL) \
  HR_F4(124, 125, 126, 127, b, CTRL)

// Max over lanes l and l ^ 16 (permlane16_swap exchanges odd and even rows).
__device__ __forceinline__ uint32_t umax_row_pair(uint32_t a) {
  const auto s = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  const uint32_t x = s[0], y = s[1];
  return x > y ? x : y;
}

// Max over the four lanes q, q + 16, q + 32, q + 48 (same DPP-row position).
__device__ __forceinline__ float max_over_rows(float m) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Per-lane constants of the transform.
struct Mfma2048 {
  int q, g, a4;           // DPP-row position, lane group, relabelled chunk A(q)
  u32x4 F[2][2];          // H_128 fragments [T0][global sign]
  u32x4 sm[4];            // bf16 sign-bit masks of the lane's B operands
  float beta0, beta1, beta2, beta3;
  float tau;              // sign of the lane's results after the DPP stages
};

// The chunk A(q) whose B operands lane q of a DPP row holds (a GF(2) relabel
// of the 16 positions that makes every H_16 partner a DPP pattern).
__device__ __forceinline__ int mfma2048_a4(int q) {
  return (q & 12) | ((q ^ (q >> 2)) & 1) | ((((q >> 1) ^ (q >> 2)) & 1) << 1);
}

// The sign bytes of a lane's B operands (8 per K-step), loaded apart from
// the rest of the setup: a kernel can issue these loads ahead of its first
// row loads and compute the setup after them.
struct Mfma2048Signs {
  uint2 s8[4];
};

// All +1: read in place of a null sign vector, so that the loads are
// unconditional (a value merged from a load and a constant would make the
// compiler wait for the load at the merge).
static __device__ int8_t kMfmaNoSigns[2048] = {};

// signs: the chunk's 2048 signs (int8 +-1) or null (all +1).
__device__ __forceinline__ void mfma2048_load_signs(Mfma2048Signs& S, int lane, const int8_t* signs) {
  const int a4 = mfma2048_a4(lane & 15), g = lane >> 4;
  const int8_t* sp = signs ? signs : kMfmaNoSigns;
#pragma unroll
  for (int s = 0; s < 4; ++s) S.s8[s] = *reinterpret_cast<const uint2*>(sp + a4 * 128 + 32 * s + 8 * g);
}

__device__ __forceinline__ void mfma2048_init(Mfma2048& M, int lane, const Mfma2048Signs& S) {
  const int q = lane & 15, g = lane >> 4;
  const int a4 = mfma2048_a4(q);
  M.q = q;
  M.g = g;
  M.a4 = a4;
  const int i0 = q & 1, i1 = (q >> 1) & 1, i2 = (q >> 2) & 1, i3 = (q >> 3) & 1;
  const int pl = (i2 & g) ^ (i3 & (g >> 1));
#pragma unroll
  for (int t0 = 0; t0 < 2; ++t0)
#pragma unroll
    for (int gs = 0; gs < 2; ++gs) {
      uint32_t w[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int e = 2 * d + hb;
          const int par = ((i0 & e) ^ (i1 & (e >> 1)) ^ (t0 & (e >> 2)) ^ pl ^ gs) & 1;
          word |= (par ? 0xBF80u : 0x3F80u) << (16 * hb);
        }
        w[d] = word;
      }
      M.F[t0][gs] = (u32x4){w[0], w[1], w[2], w[3]};
    }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    // (no signs: zero bytes, zero masks)
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t src = d < 2 ? S.s8[s].x : S.s8[s].y;
      const uint32_t b0 = (src >> (16 * (d & 1))) & 0x80u;
      const uint32_t b1 = (src >> (16 * (d & 1) + 8)) & 0x80u;
      w[d] = (b0 << 8) | (b1 << 24);
    }
    M.sm[s] = (u32x4){w[0], w[1], w[2], w[3]};
  }
  M.beta0 = (a4 & 1) ? -1.0f : 1.0f;
  M.beta1 = (a4 & 2) ? -1.0f : 1.0f;
  M.beta2 = (a4 & 4) ? -1.0f : 1.0f;
  M.beta3 = (a4 & 8) ? -1.0f : 1.0f;
  M.tau = (__builtin_popcount(a4) & 1) ? -1.0f : 1.0f;
}

__device__ __forceinline__ void mfma2048_init(Mfma2048& M, int lane, const int8_t* signs) {
  Mfma2048Signs S;
  mfma2048_load_signs(S, lane, signs);
  mfma2048_init(M, lane, S);
}

// Transform one chunk: b[s] are the lane's raw bf16 B operands; on return
// acc[T][v] = tau * Y[A(q)][v + 4 T0 + 8 g + 32 T1 + 64 T2].
__device__ __forceinline__ void mfma2048_transform(const Mfma2048& M, const u32x4 (&b)[4],
                                                   f32x4 (&acc)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8 bb = __builtin_bit_cast(bf16x8, b[s] ^ M.sm[s]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int gs = (((t >> 1) & s) ^ ((t >> 2) & (s >> 1))) & 1;
      const bf16x8 aa = __builtin_bit_cast(bf16x8, M.F[t & 1][gs]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, bb, acc[t], 0, 0, 0);
    }
  }
  // H_16 across the lanes of each DPP row (logical chunk bits 0, 1, 3, 2)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
               HR_STAGE32(8, "quad_perm:[1,0,3,2]")
               HR_STAGE32(9, "quad_perm:[2,3,0,1]")
               HR_STAGE32(10, "row_ror:8")
               HR_STAGE32(11, "row_half_mirror")
               : "+{v[96:99]}"(acc[0]), "+{v[100:103]}"(acc[1]), "+{v[104:107]}"(acc[2]),
                 "+{v[108:111]}"(acc[3]), "+{v[112:115]}"(acc[4]), "+{v[116:119]}"(acc[5]),
                 "+{v[120:123]}"(acc[6]), "+{v[124:127]}"(acc[7])
               : "v"(M.beta0), "v"(M.beta1), "v"(M.beta3), "v"(M.beta2));
}

}  // namespace hr
