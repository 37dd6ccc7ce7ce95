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
//     writes Z_c = H_2048 D_c x_c to LDS in natural element order: the
//     16-byte slot j of 128-element block a sits at 32 a + (j ^ a), so the 16
//     lanes of a write phase (16 different a) and of a read phase (16
//     consecutive j) hit 16 different bank groups.
//   Phase 2: every wave takes 256 positions of all m chunks (lane: 4
//     consecutive positions), reads each Z_c once, mixes y_b = sum_c O[b][c]
//     Z_c (m fmas per output; log2 m add/sub stages for O = H_m) and
//     quantizes: the G / 4 lanes of a group reduce its absmax by DPP and
//     permlane swaps, and each lane stores its 4 codes (16 bits) per chunk.
#include "mfma2048.h"

namespace hr {

constexpr int kMixWaves = 8;
constexpr int kMixBlocksPerCu = 2;

// Max over lanes l and l ^ 16 (permlane16_swap exchanges odd and even rows).
__device__ __forceinline__ uint32_t umax_row_pair(uint32_t a) {
  const auto s = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  const uint32_t x = s[0], y = s[1];
  return x > y ? x : y;
}
// Max over lanes l and l ^ 32.
__device__ __forceinline__ uint32_t umax_half_pair(uint32_t a) {
  const auto s = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const uint32_t x = s[0], y = s[1];
  return x > y ? x : y;
}

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

  // phase 2 placement: 128-position block gam, positions 128 gam + 4 k .. + 3
  const int k = lane & 31;
  const int gam = 2 * w + (lane >> 5);
  const int rslot = 32 * gam + (k ^ gam);
  const int pos = 128 * gam + 4 * k;
  // phase 1 leaves every value of block gam multiplied by the same sign
  // tau(gam); the mixing is linear, so it is folded into the output multiplier
  const float taug = (__builtin_popcount(gam) & 1) ? -1.0f : 1.0f;

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
        zbuf[w][32 * a4 + (j ^ a4)] = acc[t];
      }
    }
    __syncthreads();

    // this lane's 4 positions of every chunk; with O = H_M they become the
    // outputs in place (log2 M stages of (u + v, u - v) on chunk pairs)
    f32x4 z[M];
#pragma unroll
    for (int c = 0; c < M; ++c) z[c] = zbuf[c][rslot];
    __syncthreads();                              // zbuf is rewritten by the next row
    if (SYLV) {
#pragma unroll
      for (int hb = 1; hb < M; hb <<= 1)
#pragma unroll
        for (int c = 0; c < M; ++c)
          if (!(c & hb)) {
            const f32x4 u = z[c], v = z[c | hb];
            z[c] = u + v;
            z[c | hb] = u - v;
          }
    }
    // output chunk bo: y = sum_c O[bo][c] Z_c (or the butterfly result)
    auto out_chunk = [&](int bo) -> f32x4 {
      if (SYLV) return z[bo];
      f32x4 acc = z[0] * block[bo * M];
#pragma unroll
      for (int c = 1; c < M; ++c) {
        const float o = block[bo * M + c];
        acc = (f32x4){fmaf(o, z[c][0], acc[0]), fmaf(o, z[c][1], acc[1]), fmaf(o, z[c][2], acc[2]),
                      fmaf(o, z[c][3], acc[3])};
      }
      return acc;
    };

    if (OUT_F32) {
      const float ym = norm * taug;
#pragma unroll
      for (int bo = 0; bo < M; ++bo) {
        const f32x4 v = out_chunk(bo);
        __builtin_nontemporal_store((f32x4){v[0] * ym, v[1] * ym, v[2] * ym, v[3] * ym},
                                    reinterpret_cast<f32x4*>(yout + row * NR + (int64_t)bo * P + pos));
      }
      continue;
    }
    // this row's codes and scales through buffer resources (32-bit offsets)
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        codes + row * (NR / 2), 0, (int)(NR / 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(scales) + row * (NR / G) * (SF16 ? 2 : 4), 0, (int)(NR / G) * (SF16 ? 2 : 4),
        0x00020000);
    // group absmax of the unnormalised outputs over the G / 4 lanes of a
    // group; two chunks at a time, so that each DPP step reads a value
    // written two instructions earlier (no wait states)
    auto absmax4 = [](const f32x4& v) {
      return __float_as_uint(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    };
    auto reduce2 = [](uint32_t& a0, uint32_t& a1) {
      a0 = umax_dpp<kQuadXor1>(a0);
      a1 = umax_dpp<kQuadXor1>(a1);
      a0 = umax_dpp<kQuadXor2>(a0);
      a1 = umax_dpp<kQuadXor2>(a1);
      a0 = umax_dpp<kRowHalfMirror>(a0);          // 8 lanes: 32 positions
      a1 = umax_dpp<kRowHalfMirror>(a1);
      if (G >= 64) {
        a0 = umax_dpp<kRowMirror>(a0);
        a1 = umax_dpp<kRowMirror>(a1);
      }
      if (G >= 128) {
        a0 = umax_row_pair(a0);
        a1 = umax_row_pair(a1);
      }
      if (G >= 256) {
        a0 = umax_half_pair(a0);
        a1 = umax_half_pair(a1);
      }
    };
    // scale, codes and stores of chunk bo from its group absmax ab
    auto quant_chunk = [&](int bo, const f32x4& v, uint32_t ab) {
      const float s32 = div_const<7>(__uint_as_float(ab) * norm);
      const float sq = SF16 ? (float)(_Float16)s32 : s32;
      const float kq = sq > 0.0f ? norm * taug * __builtin_amdgcn_rcpf(sq) : 0.0f;
      // the first lane of each group stores its scale
      if ((lane & (G / 4 - 1)) == 0) {
        const int so = (bo * (P / G) + pos / G) * (SF16 ? 2 : 4);
        if (SF16)
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)s32), rsc, so, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s32), rsc, so, 0, 0);
      }
      // q + 1.5 * 2^23 + 8 rounds y k to an integer in the low mantissa bits
      // (ties to even); its low byte is q + 8 in [1, 15].  The clamp to
      // [-7, 7] only acts for fp16-subnormal (or fp32-denormal) scales, whose
      // reciprocal is imprecise; elsewhere |y k| rounds to at most 7.
      constexpr float MQ = 12582920.0f;
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r[e] = __builtin_amdgcn_fmed3f(fmaf(v[e], kq, MQ), MQ - 7.0f, MQ + 7.0f);
      const uint32_t p01 = (__float_as_uint(r[1]) << 4) | __float_as_uint(r[0]);
      const uint32_t p23 = (__float_as_uint(r[3]) << 4) | __float_as_uint(r[2]);
      const uint32_t c16 = (((p23 << 8) | (p01 & 0xFFu)) & 0xFFFFu) ^ 0x8888u;
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)c16, rc, pos / 2, bo * (P / 2), 0);
    };
#pragma unroll
    for (int bo = 0; bo < M; bo += 2) {
      const f32x4 v0 = out_chunk(bo);
      const f32x4 v1 = out_chunk(bo + 1 < M ? bo + 1 : bo);
      uint32_t a0 = absmax4(v0), a1 = absmax4(v1);
      reduce2(a0, a1);
      quant_chunk(bo, v0, a0);
      if (bo + 1 < M) quant_chunk(bo + 1, v1, a1);
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
