// Mixed-radix randomized Hadamard transform of bf16 rows, n = m * 2048 with
// 2 <= m <= 8, on bf16 matrix cores, fused with int4 quantization (or an
// fp32 store).
//
// What is computed: y = (O kron H_2048) D x / sqrt(2048) per row (HARP
// abstract: mixed-radix schedules for dimensions that are not powers of two;
// HARP technical summary (gist.science), section 2.1: a radix that is not a
// power of two uses a fixed orthogonal block O), then groups of G consecutive
// outputs quantized with scale absmax / 7 ("Experiment -- Hadamard rotation
// for int4 (W4A4) accuracy", Method).  With the Sylvester block O = H_m
// (p = m * 2048, m = 2, 4, 8) the product is H_p itself.
//
// One workgroup of 8 waves per row, persistent over rows, two per CU.
//   Phase 1: wave c < m transforms chunk c of the row with the matrix-core
//     routine of mfma2048.h (its next row's chunk already in registers) and
//     writes Z_c = H_2048 D_c x_c to LDS, 128-element block a in 32 16-byte
//     slots at 32 a + zslot(j, a) (conflict-free writes and reads).
//   Phase 2: wave w takes 512 positions and half of the output chunks; a
//     lane reads 8 of these positions (two 16-byte slots) of every Z_c and
//     mixes them, y_b = sum_c O[b][c] Z_c, on the matrix cores as fp32 4x4x1
//     products (the Sylvester block O = H_M by add/sub stages), then
//     quantizes: the G / 8 lanes of a group reduce its absmax by DPP (and a
//     permlane swap for G = 256), and each lane stores its 8 codes (32 bits)
//     per output chunk.
#include "mfma2048.h"

namespace hr {

constexpr int kMixWaves = 8;
constexpr int kMixBlocksPerCu = 2;

// Lane r's value of each quad, to the whole quad (DPP quad_perm [r, r, r, r];
// r a constant once the caller's loop is unrolled).
__device__ __forceinline__ float quad_bcast(float v, int r) {
  switch (r) {
    case 0: return dpp<0x00>(v);
    case 1: return dpp<0x55>(v);
    case 2: return dpp<0xAA>(v);
    default: return dpp<0xFF>(v);
  }
}

// LDS slot of 16-byte slot j (0..31) of 128-element block a (0..15).  A
// 16-byte access is served 8 lanes at a time, so every aligned group of 8
// lanes must reach 8 different 16-byte bank groups (mod 8), and 16 lanes 16
// (mod 16): phase-1 writes (one j, blocks a of a lane group) and phase-2 reads
// (one block; slots 2k, 2k + 1, k or k + 16 for k = 0..15) both do.
__device__ __forceinline__ int zslot(int j, int a) { return j ^ ((j >> 3) & 1) ^ ((j & 16) >> 1) ^ a; }

template <int M, int G, bool SF16, bool OUT_F32, bool SYLV>
__global__ __launch_bounds__(kMixWaves * 64, kMixBlocksPerCu) void mixed2048_mfma_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ signs,
    const float* __restrict__ block, int64_t rows, float* __restrict__ yout,
    uint8_t* __restrict__ codes, void* __restrict__ scales, float norm) {
  static_assert(M >= 2 && M <= kMixWaves, "one transform wave per chunk");
  static_assert(!SYLV || M == 2 || M == 4 || M == 8, "Sylvester blocks are powers of two");
  constexpr int P = 2048;
  constexpr int64_t NR = (int64_t)M * P;          // row length
  __shared__ __attribute__((aligned(16))) f32x4 zbuf[M][P / 4];
  // the H_128 operand fragments depend on the lane only: one copy in LDS,
  // reloaded for each transform, keeps 16 registers free for phase 2
  __shared__ __attribute__((aligned(16))) u32x4 flds[4][64];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const bool xw = w < M;                          // transform wave of chunk w
  Mfma2048 Mc;
  mfma2048_init(Mc, lane, (signs && xw) ? signs + (int64_t)w * P : nullptr);
  const int a4 = Mc.a4, g = Mc.g;
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) flds[i][lane] = Mc.F[i >> 1][i & 1];
  }
  // element offset of this lane's B-operand pieces within its chunk: + 32 s
  const int src = 128 * a4 + 8 * g;
  auto load_chunk = [&](int64_t row, u32x4 (&b)[4]) {
    const uint16_t* base = x + row * NR + (int64_t)w * P + src;
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = *reinterpret_cast<const u32x4*>(base + 32 * s);
  };

  // phase 2 placement: wave w forms the output chunks ob .. ob + nout - 1
  // (half w & 1 of the M outputs) at positions 512 (w >> 1) .. + 511; the 16
  // lanes of DPP row gam = 4 (w >> 1) + lane / 16 cover block gam.  Lane
  // k = lane & 15 takes two 16-byte slots of it: 2k and 2k + 1 (8 consecutive
  // positions, one 32-bit code word) for quantization, k and k + 16 for the
  // fp32 store (each store instruction then fills whole lines)
  constexpr int OA = (M + 1) / 2;
  const int ob = (w & 1) ? OA : 0;
  const int nout = (w & 1) ? M - OA : OA;
  const int k = lane & 15;
  const int gam = 4 * (w >> 1) + (lane >> 4);
  const int j0 = OUT_F32 ? k : 2 * k, j1 = OUT_F32 ? k + 16 : 2 * k + 1;
  const int rs0 = 32 * gam + zslot(j0, gam), rs1 = 32 * gam + zslot(j1, gam);
  const int pos = 128 * gam + 4 * j0;             // the second slot: pos + 4 (j1 - j0)
  // phase 1 leaves every value of block gam multiplied by the same sign
  // tau(gam); the mixing is linear, so it is folded into the output multiplier
  const float taug = (__builtin_popcount(gam) & 1) ? -1.0f : 1.0f;
  // A operand of the 4x4x1 products (dense O): every 4-lane block holds rows
  // ob .. ob + 3 of O (zero past the wave's outputs), the lane row ob + (lane & 3)
  float coef[M];
  if (!SYLV) {
    const int ri = lane & 3, rw = ob + ri;
#pragma unroll
    for (int c = 0; c < M; ++c) {
      const float o = block[ri < nout ? rw * M + c : 0];   // in bounds for every lane
      coef[c] = ri < nout ? o : 0.0f;
    }
  }

  u32x4 nxt[4];
  if (xw && (int64_t)blockIdx.x < rows) load_chunk(blockIdx.x, nxt);
  __syncthreads();

  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    if (xw) {
      u32x4 b[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) b[s] = nxt[s];
      // unconditional (past the end the row reloads itself, never used): a
      // merge of loaded and unloaded registers would wait for this load
      load_chunk(row + gridDim.x < rows ? row + gridDim.x : row, nxt);
      Mfma2048 Mt;
      Mt.sm[0] = Mc.sm[0];
      Mt.sm[1] = Mc.sm[1];
      Mt.sm[2] = Mc.sm[2];
      Mt.sm[3] = Mc.sm[3];
      Mt.beta0 = Mc.beta0;
      Mt.beta1 = Mc.beta1;
      Mt.beta2 = Mc.beta2;
      Mt.beta3 = Mc.beta3;
#pragma unroll
      for (int i = 0; i < 4; ++i) Mt.F[i >> 1][i & 1] = flds[i][lane];
      f32x4 acc[8];
      mfma2048_transform(Mt, b, acc);
      // acc[T][v] = tau(a4) * Z[128 a4 + v + 4 T0 + 8 g + 32 T1 + 64 T2]:
      // 16-byte slot j = T0 + 2 g + 8 T1 + 16 T2 of block a4
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int j = (t & 1) + 2 * g + 8 * ((t >> 1) & 1) + 16 * (t >> 2);
        zbuf[w][32 * a4 + zslot(j, a4)] = acc[t];
      }
    }
    __syncthreads();

    // this lane's 8 positions of every chunk (two 16-byte slots)
    f32x4 z[M][2];
#pragma unroll
    for (int c = 0; c < M; ++c) {
      z[c][0] = zbuf[c][rs0];
      z[c][1] = zbuf[c][rs1];
    }
    __syncthreads();                            // zbuf is rewritten by the next row
    // acc[e][r] = y_{ob + r} at the lane's position e
    f32x4 acc[8];
    if constexpr (SYLV) {
      // H_M = H_2 kron H_{M/2}: the wave's half (w & 1) of the outputs is
      // H_{M/2} applied to u_c = Z_c +- Z_{c + M/2}; in-place add/sub stages
      // leave output r in u[r]
      constexpr int H2 = M / 2;
      const float sg = (w & 1) ? -1.0f : 1.0f;
      f32x4 u[H2][2];
#pragma unroll
      for (int c = 0; c < H2; ++c)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int e = 0; e < 4; ++e) u[c][s2][e] = fmaf(sg, z[c + H2][s2][e], z[c][s2][e]);
#pragma unroll
      for (int hb = 1; hb < H2; hb <<= 1)
#pragma unroll
        for (int c = 0; c < H2; ++c)
          if (!(c & hb)) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const f32x4 a = u[c][s2], b = u[c | hb][s2];
              u[c][s2] = a + b;
              u[c | hb][s2] = a - b;
            }
          }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[e][r] = r < H2 ? u[r][e >> 2][e & 3] : 0.0f;
    } else {
      // y_{ob + r} = sum_c O[ob + r][c] Z_c at the lane's 8 positions: one
      // 4x4x1 fp32 matrix-core product per position and c (A: the lane's
      // coefficient, B: the lane's own Z value), rows r of acc[e] = outputs
#pragma unroll
      for (int c = 0; c < M; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_4x4x1f32(coef[c], z[c][e >> 2][e & 3],
                                                       c == 0 ? (f32x4){0.0f, 0.0f, 0.0f, 0.0f} : acc[e],
                                                       0, 0, 0);
    }
    if constexpr (OUT_F32) {
      const float ym = norm * taug;
#pragma unroll
      for (int r = 0; r < OA; ++r) {
        if (r >= nout) break;
        float* dst = yout + row * NR + (int64_t)(ob + r) * P + pos;
        __builtin_nontemporal_store((f32x4){acc[0][r] * ym, acc[1][r] * ym, acc[2][r] * ym, acc[3][r] * ym},
                                    reinterpret_cast<f32x4*>(dst));
        __builtin_nontemporal_store((f32x4){acc[4][r] * ym, acc[5][r] * ym, acc[6][r] * ym, acc[7][r] * ym},
                                    reinterpret_cast<f32x4*>(dst + 64));
      }
    } else {
      // this row's codes and scales through buffer resources (32-bit offsets)
      const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
          codes + row * (NR / 2), 0, (int)(NR / 2), 0x00020000);
      const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<char*>(scales) + row * (NR / G) * (SF16 ? 2 : 4), 0, (int)(NR / G) * (SF16 ? 2 : 4),
          0x00020000);
      // group absmax of the unnormalised outputs over the G / 8 lanes of a
      // group, all output rows interleaved (each DPP step reads a value
      // written several instructions earlier: no wait states)
      uint32_t am[OA];
#pragma unroll
      for (int r = 0; r < OA; ++r) {
        float m = fmaxf(fmaxf(fabsf(acc[0][r]), fabsf(acc[1][r])), fabsf(acc[2][r]));
        m = fmaxf(fmaxf(m, fabsf(acc[3][r])), fabsf(acc[4][r]));
        m = fmaxf(fmaxf(m, fabsf(acc[5][r])), fabsf(acc[6][r]));
        am[r] = __float_as_uint(fmaxf(m, fabsf(acc[7][r])));
      }
#pragma unroll
      for (int r = 0; r < OA; ++r) am[r] = umax_dpp<kQuadXor1>(am[r]);
#pragma unroll
      for (int r = 0; r < OA; ++r) am[r] = umax_dpp<kQuadXor2>(am[r]);
      if (G >= 64) {
#pragma unroll
        for (int r = 0; r < OA; ++r) am[r] = umax_dpp<kRowHalfMirror>(am[r]);   // 8 lanes: 64 positions
      }
      if (G >= 128) {
#pragma unroll
        for (int r = 0; r < OA; ++r) am[r] = umax_dpp<kRowMirror>(am[r]);
      }
      if (G >= 256) {
#pragma unroll
        for (int r = 0; r < OA; ++r) am[r] = umax_row_pair(am[r]);
      }
      // the scale arithmetic once per lane: lane r of each quad (a quad lies
      // inside one group, G / 8 >= 4 lanes) takes output r, and DPP quad
      // broadcasts hand every lane the multipliers of all outputs
      const int rl = lane & 3;
      uint32_t amsel = am[0];
#pragma unroll
      for (int r = 1; r < OA; ++r) amsel = rl == r ? am[r] : amsel;
      const bool rvalid = rl < nout;
      const float s32 = div_const<7>(__uint_as_float(amsel) * norm);
      const float sq = SF16 ? (float)(_Float16)s32 : s32;
      // an fp32 scale below 2^-100 would overflow its reciprocal: the group's
      // values and scale are then both taken x 2^64 (exact)
      const float up = (!SF16 && sq < 0x1p-100f) ? 0x1p64f : 1.0f;
      const float kq = sq > 0.0f ? norm * taug * __builtin_amdgcn_rcpf(sq * up) : 0.0f;
      // the clamp and the x 2^64 only where some group of the wave needs
      // them (a wave-uniform branch)
      const bool clamp = __builtin_amdgcn_ballot_w64(
                             rvalid && sq > 0.0f && sq < (SF16 ? 6.103515625e-05f : 1.17549435e-38f)) != 0;
      const bool tiny = !SF16 && __builtin_amdgcn_ballot_w64(rvalid && sq > 0.0f && sq < 0x1p-100f) != 0;
      // the group's first quad stores the scales: lane r that of output r
      if ((lane & (G / 8 - 1)) < 4 && rvalid) {
        const int so = ((ob + rl) * (P / G) + pos / G) * (SF16 ? 2 : 4);
        if (SF16)
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)s32), rsc, so, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s32), rsc, so, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < OA; ++r) {
        if (r >= nout) break;
        const int bo = ob + r;
        const float kr = quad_bcast(kq, r);
        const float ur = SF16 ? 1.0f : quad_bcast(up, r);
        // q + 1.5 * 2^23 + 8 rounds y k to an integer in the low mantissa
        // bits (ties to even); its low byte is q + 8 in [1, 15].  The clamp
        // to [-7, 7] only acts for fp16-subnormal (or fp32-denormal) scales,
        // whose reciprocal is imprecise; elsewhere |y k| rounds to at most 7.
        constexpr float MQ = 12582920.0f;
        float qf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[e] = fmaf(tiny ? acc[e][r] * ur : acc[e][r], kr, MQ);
        if (clamp) {
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[e] = __builtin_amdgcn_fmed3f(qf[e], MQ - 7.0f, MQ + 7.0f);
        }
        uint32_t q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = __float_as_uint(qf[e]);
        // nibble e of the word is code e; low bytes of the pairs first
        const uint32_t p01 = (q[1] << 4) | q[0], p23 = (q[3] << 4) | q[2];
        const uint32_t p45 = (q[5] << 4) | q[4], p67 = (q[7] << 4) | q[6];
        const uint32_t word =
            ((p01 & 0xFFu) | ((p23 & 0xFFu) << 8) | ((p45 & 0xFFu) << 16) | (p67 << 24)) ^ 0x88888888u;
        __builtin_amdgcn_raw_buffer_store_b32(word, rc, pos / 2, bo * (P / 2), 0);
      }
    }
  }
}

template <int M, int G, bool SF16, bool OUT_F32, bool SYLV>
static void launch_mix(const RhtArgs& a, float norm, hipStream_t s) {
  const int64_t cap = 256 * kMixBlocksPerCu;
  const int64_t blocks = a.rows < cap ? a.rows : cap;
  hipLaunchKernelGGL((mixed2048_mfma_kernel<M, G, SF16, OUT_F32, SYLV>), dim3((unsigned)blocks),
                     dim3(kMixWaves * 64), 0, s, static_cast<const uint16_t*>(a.x), a.signs, a.block,
                     a.rows, a.y, a.codes, a.scales, norm);
}

template <int M, bool SYLV>
static bool launch_m(const RhtArgs& a, float norm, hipStream_t s) {
  if (a.y && !a.codes) {
    launch_mix<M, 128, false, true, SYLV>(a, norm, s);
    return true;
  }
  if (!a.codes || a.y) return false;
#define HR_MIXQ(G)                                                          \
  case G:                                                                   \
    if (a.scale_f16) launch_mix<M, G, true, false, SYLV>(a, norm, s);       \
    else launch_mix<M, G, false, false, SYLV>(a, norm, s);                  \
    return true;
  switch (a.group) {
    HR_MIXQ(32)
    HR_MIXQ(64)
    HR_MIXQ(128)
    HR_MIXQ(256)
    default: return false;
  }
#undef HR_MIXQ
}

// bf16 rows of n = m * 2048 (2 <= m <= 8) with the caller's block O, and of
// n = p = 4096, 8192, 16384 (m = 1) as H_{p/2048} kron H_2048; fp32 output
// or fused int4 quantization.  Returns false when the case belongs to
// another kernel.
bool launch_mixed2048_mfma(const RhtArgs& a, hipStream_t s) {
  if (!a.x_bf16 || (a.codes && a.bits == 8)) return false;
  if (a.m == 1) {
    const float norm = (float)(1.0 / sqrt((double)a.p));
    switch (a.p) {
      case 4096: return launch_m<2, true>(a, norm, s);
      case 8192: return launch_m<4, true>(a, norm, s);
      case 16384: return launch_m<8, true>(a, norm, s);
      default: return false;
    }
  }
  if (a.p != 2048) return false;
  const float norm = (float)(1.0 / sqrt(2048.0));
  switch (a.m) {
    case 2: return launch_m<2, false>(a, norm, s);
    case 3: return launch_m<3, false>(a, norm, s);
    case 4: return launch_m<4, false>(a, norm, s);
    case 5: return launch_m<5, false>(a, norm, s);
    case 6: return launch_m<6, false>(a, norm, s);
    case 7: return launch_m<7, false>(a, norm, s);
    case 8: return launch_m<8, false>(a, norm, s);
    default: return false;
  }
}

}  // namespace hr
