// Randomized Hadamard transform of bf16 rows of 2048 (or 4096) elements, fused
// with int4 or int8 quantization (or an fp32 store), with the 128-point factor
// of the transform on bf16 matrix cores.
//
// What is computed: y = H_n (d * x) / sqrt(n) per row, Sylvester order
// ("Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Hypothesis and
// Method; "Llama-3.2-1B-Instruct-HadamardSpin-4bits", How it Works), then
// groups of G consecutive outputs quantized with scale absmax / 7 (same
// pages, Method); or, for the int8 activations of W4A8, with scale absmax / 127
// (same page, the W4A8 rows of Results).
//
// The transform is the matrix-core routine of mfma2048.h (H_128 on
// v_mfma_f32_16x16x32_bf16, H_16 as DPP butterflies).  A row of n = 4096 is
// two 2048-point chunks in the same wave: H_4096 = H_2 kron H_2048, and the
// two chunk transforms leave each output position in the same lane, so the
// H_2 stage is a lane-local sum and difference.
//
//   Staging: each wave streams its rows through two 4 KB LDS stages filled by
//     nontemporal global_load_lds_dwordx4 (two rows in flight per wave
//     without holding registers).  Load j < 4 of a 2048-point chunk covers
//     its bytes 1024 j .. 1024 j + 1023, whole cache lines; lane i fetches
//     piece u of 128-element chunk 4 j + h (h = i >> 4, u = i - 4 j - h mod
//     16), so chunk a, piece p lands in LDS slot 16 a + (p + a mod 16) and
//     the 16 pieces a lane group reads for one MFMA (piece 4 s + g of the 16
//     chunks) fall in 16 different bank groups.
//   Codes: a lane owns four runs of 8 consecutive outputs; they are staged
//     through LDS (swizzled, conflict-free) and written as contiguous 1 KB
//     runs, one per store instruction (one per int4 row, two per int8 row).
//   fp6 output (BITS = 6): the int4 codes as fp6 e2m3 fields in the tiled
//     operand format of the fp6 GEMM (panels of 128 rows, 12288-byte tiles of
//     128 codes, two planes each holding slots h and h + 2 of a row at row *
//     48), and the scales transposed to [n / G][padded rows].  A row holds
//     only 48 contiguous bytes per plane of a tile, so a wave takes its rows
//     in groups of 4 consecutive ones (a workgroup 16) and stages a group's
//     codes in LDS in the tiles' byte order: per chunk, 32 regions (block,
//     plane) of 4 x 48 = 192 contiguous bytes, which go out as 16-byte
//     stores covering whole 64-byte sectors.  A run of 8 codes (slot m,
//     offset 8 g) is 6 bytes at byte 24 (m >> 1) + 6 g of its row in region
//     (block, m & 1).  The two regions of a block sit 400 bytes apart from
//     the next block's in LDS (384 would put the 16 blocks a staging store
//     touches in the same banks).  The fields come from the fp32 -> fp6
//     pack conversion of the exact integer codes with scale 8 (code / 8 is
//     an e2m3 value), 32 codes per instruction.  The scales are staged per
//     group too and leave transposed, one 8-byte (fp16) or 16-byte (fp32)
//     piece per group of quantization and 4 rows.
#include "mfma2048.h"

namespace hr {

// Workgroups (of four waves) per CU: three for the quantizing 2048-point
// instances (36 KB of LDS each; 61.9 us against 65.0 us with two, same box,
// bf16 65536 x 2048, G = 128), two for the fp32 output and the 4096-point
// rows, whose 68 KB would not fit three times, and one for the fp32 output of
// 4096-point rows (its registers leave room for one wave per SIMD).  The fp6
// output's group staging takes 59 KB (2048-point rows: two fit) or 117 KB
// (4096-point rows: one fits).
template <bool OUT_F32, int CH, int BITS>
constexpr int mfma_blocks_per_cu() {
  return BITS == 6 ? (CH == 2 ? 1 : 2) : (OUT_F32 && CH == 2) ? 1 : (OUT_F32 || CH == 2) ? 2 : 3;
}

// 16-byte global -> LDS copy, nontemporal when nt (the builtin sits in a
// device function: used directly in a kernel template it can cost the
// instance its host stub).  With HBM-resident input (bf16 65536 x 2048,
// three buffer sets, same box) the hint on whole-line loads took the kernel
// from 63.8 to 62.9 us; on the earlier 64-byte runs it had cost 0.7 us.
__device__ __forceinline__ void mfma_lds_load16(const void* gp, void* lp, bool nt) {
  if (nt) __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 2);
  else __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 0);
}

template <int G, bool SCALE_F16, bool OUT_F32, int BITS, int CH = 1>
__global__ __launch_bounds__(256, (mfma_blocks_per_cu<OUT_F32, CH, BITS>())) void rht2048_mfma_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ signs, int64_t rows,
    float* __restrict__ yout, uint8_t* __restrict__ codes, void* __restrict__ scales, float norm,
    bool nt) {
  static_assert(CH == 1 || CH == 2, "rows of one or two 2048-point chunks");
  constexpr int P = 2048;          // chunk
  constexpr int N = CH * P;        // row
  const int lane = threadIdx.x & 63;
  const int wib = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // (an XCD-aware order for the fp6 output, each XCD taking runs of
  // consecutive rows, measured 83.7 against 76.2 us with HBM-resident
  // buffers, bf16 65536 x 2048)
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + wib;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  // the k-th row of this wave: rows wave + k nwaves, or for fp6 output groups
  // of 4 consecutive rows (group wave + (k / 4) nwaves)
  auto row_at = [&](int k) -> int64_t {
    if (BITS == 6) return 4 * (wave + (int64_t)(k >> 2) * nwaves) + (k & 3);
    return wave + (int64_t)k * nwaves;
  };
  // (the sign loads go first; the rest of the setup is computed after the
  // first rows' loads are issued, so that it overlaps them: 62.9 -> 60.6 us,
  // same box, bf16 65536 x 2048)
  Mfma2048Signs SG[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) mfma2048_load_signs(SG[c], lane, signs ? signs + c * P : nullptr);
  Mfma2048 M[CH];
  const int g = lane >> 4, a4 = mfma2048_a4(lane & 15);
  const float tau = (__builtin_popcount(a4) & 1) ? -1.0f : 1.0f;

  // LDS of this wave: NST row stages (256 slots of 16 bytes per chunk; a
  // third stage measured slower for every output) and one chunk of codes
  // (fp6: the codes of a group of 4 rows, every chunk)
  constexpr int NST = 2;
  __shared__ __attribute__((aligned(16))) u32x4 stage_lds[4][NST][CH * 256];
  __shared__ __attribute__((aligned(16))) u32x4 code_lds[4][BITS == 8 ? 128 : BITS == 6 ? CH * 400 : 64];
  // fp6: the group's scales, [group][row of the group] (fp16 or fp32 bits)
  constexpr int SES = SCALE_F16 ? 2 : 4;
  __shared__ __attribute__((aligned(16))) uint8_t scale_lds[4][BITS == 6 ? 4 * (N / G) * SES : 16];
  // fp32 output: this wave's 8 KB output row, staged so it leaves as 1 KB stores
  __shared__ __attribute__((aligned(16))) f32x4 out_lds[OUT_F32 ? 4 : 1][OUT_F32 ? 512 : 1];
  // element offset within a chunk of this lane's piece for load j
  int lane_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = lane >> 4, u = ((lane & 15) - 4 * j - h) & 15;
    lane_src[j] = 512 * j + 128 * h + 8 * u;
  }
  auto issue = [&](int64_t row, int st) {
    // (one branch on nt per row, not one per load)
    if (nt) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          mfma_lds_load16(x + row * N + c * P + lane_src[j], &stage_lds[wib][st][256 * c + 64 * j], true);
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          mfma_lds_load16(x + row * N + c * P + lane_src[j], &stage_lds[wib][st][256 * c + 64 * j], false);
    }
  };
  // B operands of one row from stage st: lane (q, g) takes piece 4 s + g of
  // chunk A(q), slot 16 A(q) + (4 s + g + A(q) mod 16), for K-step s.  First a wait for the stage's loads:
  // vector-memory operations complete in issue order (loads and stores
  // alike), so it is a wait until at most `younger` operations are
  // outstanding, where younger counts what this wave issued after the
  // stage's loads -- the next row's loads and the stores of the rows
  // processed since (see the loop).  Then one asm block reads the stage and
  // waits for its own results.
  uint32_t rd_lane[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) rd_lane[k] = 16u * (uint32_t)(16 * a4 + ((a4 + 4 * k + g) & 15));
  auto read_stage = [&](int st, int younger, u32x4 (&b)[CH][4]) {
    // s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
    // left at their maxima (no wait)
    switch (younger) {
#define HR_VMW(V) \
      case V: __builtin_amdgcn_s_waitcnt(((V) & 15) | (((V) >> 4) << 14) | 0x0F70); break;
      HR_VMW(0) HR_VMW(1) HR_VMW(2) HR_VMW(3) HR_VMW(4) HR_VMW(5) HR_VMW(6) HR_VMW(7) HR_VMW(8)
      HR_VMW(9) HR_VMW(10) HR_VMW(11) HR_VMW(12) HR_VMW(13) HR_VMW(14) HR_VMW(15) HR_VMW(16)
      HR_VMW(20) HR_VMW(21) HR_VMW(24) HR_VMW(29) HR_VMW(32) HR_VMW(40)
#undef HR_VMW
      default: __builtin_amdgcn_s_waitcnt(0x0F70); break;   // vmcnt(0)
    }
    const uint32_t sb = (uint32_t)(uintptr_t)&stage_lds[wib][st][0];
    if (CH == 1)
      asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\t"
                   "ds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=v"(b[0][0]), "=v"(b[0][1]), "=v"(b[0][2]), "=v"(b[0][3])
                   : "v"(sb + rd_lane[0]), "v"(sb + rd_lane[1]), "v"(sb + rd_lane[2]), "v"(sb + rd_lane[3])
                   : "memory");
    else
      asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\t"
                   "ds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
                   "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %9 offset:4096\n\t"
                   "ds_read_b128 %6, %10 offset:4096\n\tds_read_b128 %7, %11 offset:4096\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=v"(b[0][0]), "=v"(b[0][1]), "=v"(b[0][2]), "=v"(b[0][3]),
                     "=v"(b[CH - 1][0]), "=v"(b[CH - 1][1]), "=v"(b[CH - 1][2]), "=v"(b[CH - 1][3])
                   : "v"(sb + rd_lane[0]), "v"(sb + rd_lane[1]), "v"(sb + rd_lane[2]), "v"(sb + rd_lane[3])
                   : "memory");
  };

  // outputs of chunk ch of a row: acc[T][v] = tau * Y[a4][c] of the chunk,
  // c = v + 4 T0 + 8 g + 32 T1 + 64 T2
  auto emit = [&](int64_t row, int ch, const f32x4 (&acc)[8]) {
    if (OUT_F32) {
      // 16-byte slot 32 a + s of the row (s = 8 m + 2 g + h) sits at 32 a +
      // (s ^ a): the lanes of a write phase, which differ in a, then hit
      // different bank groups, and a lane's read phase stays inside one a
      const float ym = norm * tau;
      f32x4* ol = &out_lds[wib][0];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 lo = acc[2 * m], hi = acc[2 * m + 1];
        ol[32 * a4 + ((8 * m + 2 * g) ^ a4)] = (f32x4){lo[0] * ym, lo[1] * ym, lo[2] * ym, lo[3] * ym};
        ol[32 * a4 + ((8 * m + 2 * g + 1) ^ a4)] = (f32x4){hi[0] * ym, hi[1] * ym, hi[2] * ym, hi[3] * ym};
      }
      __builtin_amdgcn_wave_barrier();
      f32x4* dst = reinterpret_cast<f32x4*>(yout + row * N + ch * P);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int sl = 64 * i + lane, a = sl >> 5;
        __builtin_nontemporal_store(ol[32 * a + ((sl & 31) ^ a)], dst + sl);
      }
      __builtin_amdgcn_wave_barrier();
      return;
    }
    // group absmax: run m (outputs 32 m + 8 g + 0..7) is tiles 2m, 2m+1
    float mr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // three-input maxima (v_max3_f32 with |.| modifiers): 4 ops for 8 values
      const f32x4 lo = acc[2 * m], hi = acc[2 * m + 1];
      const float m1 = fmaxf(fmaxf(fabsf(lo[0]), fabsf(lo[1])), fabsf(lo[2]));
      const float m2 = fmaxf(fmaxf(fabsf(lo[3]), fabsf(hi[0])), fabsf(hi[1]));
      const float m3 = fmaxf(fmaxf(m1, fabsf(hi[2])), fabsf(hi[3]));
      mr[m] = fmaxf(m2, m3);
    }
    constexpr int NG = G == 32 ? 4 : G == 64 ? 2 : 1;   // groups per lane (shared by its 4 rows)
    float kk[NG], upv[NG];
    float s_own = 0.0f;                  // scale of the group this lane stores
    bool need_clamp = false, need_up = false;
    if constexpr (G == 32 || G == 64) {
      // Reduce-scatter over the lanes q, q + 16, q + 32, q + 48 (rows of the
      // same DPP position): permlane16 swaps pair rows 0/1 and 2/3, permlane32
      // pairs the halves, and lane row g ends with the absmax of group g % NG
      // of its block -- the group whose scale it stores.  The scale arithmetic
      // runs once per lane, and swaps in the opposite order give every lane
      // the multipliers of all NG groups.
      float own;
      if (G == 32) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(mr[0]), __float_as_uint(mr[1]), false, false);
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(mr[2]), __float_as_uint(mr[3]), false, false);
        const float pm = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
        const float qm = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm), __float_as_uint(qm), false, false);
        own = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
      } else {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(fmaxf(mr[0], mr[1])),
                                                        __float_as_uint(fmaxf(mr[2], mr[3])), false, false);
        const float pm = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm), __float_as_uint(pm), false, false);
        own = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
      }
      const float s32 = div_const<BITS == 8 ? 127 : 7>(own * norm);
      const float s = SCALE_F16 ? (float)(_Float16)s32 : s32;
      // an fp32 scale below 2^-100 would overflow its reciprocal: the group's
      // values and scale are then both taken x 2^64 (exact; same quotients)
      const float up = (!SCALE_F16 && s < 0x1p-100f) ? 0x1p64f : 1.0f;
      need_up = !SCALE_F16 && s > 0.0f && s < 0x1p-100f;
      const float k = s > 0.0f ? norm * __builtin_amdgcn_rcpf(s * up) * tau : 0.0f;
      need_clamp = s > 0.0f && s < (SCALE_F16 ? 6.103515625e-05f : 1.17549435e-38f);
      s_own = s32;
      auto gather = [&](float v, float (&out)[NG]) {
        if constexpr (G == 32) {
          const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
          const auto a = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
          const auto b = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
          out[0] = __uint_as_float(a[0]);
          out[1] = __uint_as_float(a[1]);
          out[2] = __uint_as_float(b[0]);
          out[3] = __uint_as_float(b[1]);
        } else {
          const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
          out[0] = __uint_as_float(a[0]);
          out[NG - 1] = __uint_as_float(a[1]);
        }
      };
      gather(k, kk);
      if (!SCALE_F16) gather(up, upv);
      else {
#pragma unroll
        for (int i = 0; i < NG; ++i) upv[i] = 1.0f;
      }
    } else {
      float mg = fmaxf(fmaxf(mr[0], mr[1]), fmaxf(mr[2], mr[3]));
      mg = max_over_rows(mg);
      if (G == 256) mg = __uint_as_float(umax_dpp<kQuadXor1>(__float_as_uint(mg)));
      const float s32 = div_const<BITS == 8 ? 127 : 7>(mg * norm);
      const float s = SCALE_F16 ? (float)(_Float16)s32 : s32;
      // an fp32 scale below 2^-100 would overflow its reciprocal: the group's
      // values and scale are then both taken x 2^64 (exact; same quotients)
      upv[0] = (!SCALE_F16 && s < 0x1p-100f) ? 0x1p64f : 1.0f;
      need_up = !SCALE_F16 && s > 0.0f && s < 0x1p-100f;
      kk[0] = s > 0.0f ? norm * __builtin_amdgcn_rcpf(s * upv[0]) * tau : 0.0f;
      need_clamp = s > 0.0f && s < (SCALE_F16 ? 6.103515625e-05f : 1.17549435e-38f);
      s_own = s32;
    }
    {
      int64_t si = -1;
      const int64_t s0 = row * (N / G) + ch * (P / G);   // the chunk's first group
      if (G == 32) si = s0 + 4 * a4 + g;
      else if (G == 64) si = g < 2 ? s0 + 2 * a4 + g : -1;
      else if (G == 128) si = g == 0 ? s0 + a4 : -1;
      else si = (g == 0 && (a4 & 1) == 0) ? s0 + (a4 >> 1) : -1;
      if (BITS == 6) {
        // staged for flush6 (transposed there), in asm like the codes
        if (si >= 0) {
          const uint32_t a = (uint32_t)(uintptr_t)&scale_lds[wib][0] +
                             (uint32_t)(4 * (si - row * (N / G)) + (row & 3)) * SES;
          if (SCALE_F16)
            asm volatile("ds_write_b16 %0, %1" : : "v"(a), "v"((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s_own))
                         : "memory");
          else
            asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(__float_as_uint(s_own)) : "memory");
        }
      } else if (si >= 0) {
        if (SCALE_F16) reinterpret_cast<_Float16*>(scales)[si] = (_Float16)s_own;
        else reinterpret_cast<float*>(scales)[si] = s_own;
      }
    }
    const bool clamp = __builtin_amdgcn_ballot_w64(need_clamp) != 0;
    const bool tiny = !SCALE_F16 && __builtin_amdgcn_ballot_w64(need_up) != 0;
    // q + M rounds y k to an integer in the low mantissa bits (ties to even)
    constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
    const float M = BITS == 4 ? 12582920.0f : 12582912.0f;   // 1.5 * 2^23 (+ 8 for nibbles)
    u32x4* cl = &code_lds[wib][0];
    // fp6: the codes as floats, in the conversion's operand order (field 2 i
    // from qa[i], 2 i + 1 from qb[i]): run m, element e at field 8 m + e
    float qa[BITS == 6 ? 16 : 1], qb[BITS == 6 ? 16 : 1];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int gl = G == 32 ? m : G == 64 ? (m >> 1) : 0;
      const float k = kk[gl];
      f32x4 lo = acc[2 * m], hi = acc[2 * m + 1];
      if (tiny) {
        lo *= upv[gl];
        hi *= upv[gl];
      }
      float rr[8] = {fmaf(lo[0], k, M), fmaf(lo[1], k, M), fmaf(lo[2], k, M), fmaf(lo[3], k, M),
                     fmaf(hi[0], k, M), fmaf(hi[1], k, M), fmaf(hi[2], k, M), fmaf(hi[3], k, M)};
      if (clamp) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rr[e] = __builtin_amdgcn_fmed3f(rr[e], M - QMAX, M + QMAX);
      }
      if (BITS == 4) {
        // dword 16 a + 4 m + g of the row: 16-byte block (a, m) at 4 a + (m ^ (a >> 2 & 3))
        reinterpret_cast<uint32_t*>(cl)[4 * (4 * a4 + (m ^ ((a4 >> 2) & 3))) + g] = pack8(rr);
      } else if (BITS == 6) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qa[4 * m + i] = rr[2 * i] - M;        // exact
          qb[4 * m + i] = rr[2 * i + 1] - M;
        }
      } else {
        // the low byte of each float is its two's-complement code
        uint32_t u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = __float_as_uint(rr[e]);
        const uint32_t d0 = (__builtin_amdgcn_perm(u[3], u[2], 0x0c0c0400u) << 16) |
                            __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u);
        const uint32_t d1 = (__builtin_amdgcn_perm(u[7], u[6], 0x0c0c0400u) << 16) |
                            __builtin_amdgcn_perm(u[5], u[4], 0x0c0c0400u);
        // 8-byte slot 16 a + 4 m + g of the row, its low 4 bits XOR 2 (a >> 1):
        // the 32 lanes of a write phase hit 32 different bank pairs
        reinterpret_cast<uint2*>(cl)[16 * a4 + ((4 * m + g) ^ (2 * (a4 >> 1)))] = make_uint2(d0, d1);
      }
    }
    if (BITS == 6) {
      typedef float f32x16 __attribute__((ext_vector_type(16)));
      typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
      f32x16 va, vb;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        va[i] = qa[i];
        vb[i] = qb[i];
      }
      // 32 fields of 6 bits: run m at bits 48 m .. 48 m + 47
      const u32x6 d = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(va, vb, 8.0f);
      // run m goes to byte 192 (m & 1) + 24 (m >> 1) of the lane's base, as
      // three 16-bit pieces (in asm: compiler-visible stores here were given
      // a wait for the row stages' pending loads, a different array)
      const uint32_t la =
          (uint32_t)(uintptr_t)cl + 6400 * ch + 400 * a4 + 48 * (int)(row & 3) + 6 * g;
      asm volatile(
          "ds_write_b16 %0, %1\n\tds_write_b16_d16_hi %0, %1 offset:2\n\tds_write_b16 %0, %2 offset:4\n\t"
          "ds_write_b16_d16_hi %0, %2 offset:192\n\tds_write_b16 %0, %3 offset:194\n\t"
          "ds_write_b16_d16_hi %0, %3 offset:196\n\t"
          "ds_write_b16 %0, %4 offset:24\n\tds_write_b16_d16_hi %0, %4 offset:26\n\tds_write_b16 %0, %5 offset:28\n\t"
          "ds_write_b16_d16_hi %0, %5 offset:216\n\tds_write_b16 %0, %6 offset:218\n\t"
          "ds_write_b16_d16_hi %0, %6 offset:220"
          :
          : "v"(la), "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(d[4]), "v"(d[5])
          : "memory");
      // stored by flush6 once the group's rows are staged
    } else if (BITS == 4) {
      // lane i stores bytes 16 i .. 16 i + 15 of the row: block (i >> 2, i & 3)
      const int ra = lane >> 2, rm = lane & 3;
      const u32x4 out = cl[4 * ra + (rm ^ ((ra >> 2) & 3))];
      __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(codes + row * (N / 2) + ch * (P / 2)) + lane);
    } else if (BITS == 8) {
      // 16-byte block b = 8 a + k of the row sits at 8 a + (k ^ (a >> 1))
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = 64 * h + lane, ra = b >> 3;
        const u32x4 out = cl[8 * ra + ((b & 7) ^ (ra >> 1))];
        __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(codes + row * N + ch * P) + b);
      }
    }
  };

  auto process = [&](int64_t row, const u32x4 (&b)[CH][4]) {
    f32x4 acc[8];
    mfma2048_transform(M[0], b[0], acc);
    if (CH == 1) {
      emit(row, 0, acc);
      return;
    }
    f32x4 acc1[8], dif[8];
    mfma2048_transform(M[CH - 1], b[CH - 1], acc1);
    // H_2 across the chunks: the same lane holds the same position (and the
    // same sign tau) of both
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      dif[t] = acc[t] - acc1[t];
      acc[t] = acc[t] + acc1[t];
    }
    emit(row, 0, acc);
    emit(row, 1, dif);
  };

  // fp6: the staged group of rows r0 .. r0 + 3 (those below rows) to the
  // tiles; lane i of store t takes 16-byte piece 64 t + i of a chunk's image,
  // region p / 12, row (p % 12) / 3.  Then lane i < n / G stores group i's
  // scales of the 4 rows (contiguous in the transposed scale array).
  auto flush6 = [&](int64_t r0) {
    const int64_t valid = rows - r0;
    const int64_t prow = (rows + 127) / 128 * 128;
    if (lane < N / (G ? G : 1)) {   // (G = 0, the fp32 output, never flushes)
      const uint8_t* src = &scale_lds[wib][4 * SES * lane];
      uint8_t* dst = static_cast<uint8_t*>(scales) + (lane * prow + r0) * SES;
      if (valid >= 4) {
        if (SCALE_F16) *reinterpret_cast<uint64_t*>(dst) = *reinterpret_cast<const uint64_t*>(src);
        else *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
      } else {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          if (j >= valid) break;
          if (SCALE_F16) reinterpret_cast<uint16_t*>(dst)[j] = reinterpret_cast<const uint16_t*>(src)[j];
          else reinterpret_cast<uint32_t*>(dst)[j] = reinterpret_cast<const uint32_t*>(src)[j];
        }
      }
    }
    // LDS address and tile offset of each of the lane's 6 pieces per chunk
    const uint32_t lb = (uint32_t)(uintptr_t)&code_lds[wib][0];
    uint32_t la[6];
    int32_t go[6];
    bool ok[6];
#pragma unroll
    for (int t = 0; t < 6; ++t) {
      const int p = 64 * t + lane, region = p / 12, in = p % 12;
      la[t] = lb + 16 * (25 * (region >> 1) + 12 * (region & 1) + in);
      go[t] = (region >> 1) * 12288 + (region & 1) * 6144 + 16 * in;
      ok[t] = in / 3 < valid;
    }
    uint8_t* const gb = codes + (r0 >> 7) * (N / 128) * 12288 + (r0 & 127) * 48;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // (reads in asm: compiler-visible ones were given a wait for every
      // outstanding memory operation)
      u32x4 v[6];
      asm volatile(
          "ds_read_b128 %0, %6\n\tds_read_b128 %1, %7\n\tds_read_b128 %2, %8\n\t"
          "ds_read_b128 %3, %9\n\tds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\ts_waitcnt lgkmcnt(0)"
          : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]), "=v"(v[4]), "=v"(v[5])
          : "v"(la[0] + 6400 * c), "v"(la[1] + 6400 * c), "v"(la[2] + 6400 * c), "v"(la[3] + 6400 * c),
            "v"(la[4] + 6400 * c), "v"(la[5] + 6400 * c)
          : "memory");
#pragma unroll
      for (int t = 0; t < 6; ++t)
        if (ok[t]) __builtin_nontemporal_store(v[t], reinterpret_cast<u32x4*>(gb + c * (P / 128) * 12288 + go[t]));
    }
  };

  // Vector-memory operations issued while processing the k-th row (every
  // wave issues each of them: the scale-storing lanes are in every wave):
  // per chunk one scale store and one code store (two for int8), or eight
  // fp32 stores; for fp6 six per chunk and one scale store after the fourth
  // row of a group, none otherwise
  auto stores_at = [&](int k) -> int {
    if (OUT_F32) return 8 * CH;
    if (BITS == 6) return (k & 3) == 3 ? 6 * CH + 1 : 0;
    return CH * (BITS == 8 ? 3 : 2);
  };
  constexpr int LPR = 4 * CH;      // loads per row
  int64_t row = row_at(0);
#pragma unroll
  for (int i = 0; i < NST; ++i)
    if (row_at(i) < rows) issue(row_at(i), i);
#pragma unroll
  for (int c = 0; c < CH; ++c) mfma2048_init(M[c], lane, SG[c]);
  for (int st = 0, k = 0; row < rows; ++k, row = row_at(k), st = st + 1 == NST ? 0 : st + 1) {
    u32x4 b[CH][4];
    // issued after this row's loads: the loads of the next NST - 1 rows (those
    // that exist), and the stores of the rows processed since this row's
    // loads were issued (up to NST of them; a wave's last fp6 flush is never
    // followed by a wait).
    int younger = 0;
#pragma unroll
    for (int i = 1; i < NST; ++i)
      if (row_at(k + i) < rows) younger += LPR;
#pragma unroll
    for (int j = 1; j <= NST; ++j)
      if (k - j >= 0) younger += stores_at(k - j);
    read_stage(st, younger, b);
    if (row_at(k + NST) < rows) issue(row_at(k + NST), st);
    process(row, b);
    if (BITS == 6 && ((row & 3) == 3 || row + 1 == rows)) flush6(row & ~(int64_t)3);
  }
}

template <int G, bool SCALE_F16, bool OUT_F32, int BITS = 4>
static void launch_mfma(const RhtArgs& a, float norm, hipStream_t s) {
  // 4 waves per block.  Units of work: rows, or for fp6 groups of 4 rows.
  // Up to one grid of resident workgroups, a unit per wave.  Beyond that,
  // UPW units per wave in at least two rounds of resident workgroups, so
  // that the hardware hands the later ones to the CUs that finish first
  // (bf16 65536 x 2048, HBM-resident, same box: 8 rows per wave 58.2-58.7
  // us, 16 (one resident grid) 61.3 us, 4 58.6-59.0 us, 2 63.6 us); with
  // fewer, one resident grid (a partial second round idles most of the chip:
  // int8 20000 x 4096 took 56.7 us spread over 1.2 rounds, 51.1 us
  // resident).  The fp32 output of 2048-point rows stays on one resident
  // grid (145.1 against 149.7 us spread).
  constexpr int64_t UPW = BITS == 6 ? 2 : 8;
  const int64_t units = BITS == 6 ? (a.rows + 3) / 4 : a.rows;
  const int64_t resident =
      256 * (a.p == 4096 ? mfma_blocks_per_cu<OUT_F32, 2, BITS>() : mfma_blocks_per_cu<OUT_F32, 1, BITS>());
  int64_t blocks = (units + 3) / 4;
  if (blocks > resident) {
    const int64_t spread = (units + 4 * UPW - 1) / (4 * UPW);
    blocks = (spread < 2 * resident || (OUT_F32 && a.p == 2048)) ? resident : spread;
  }
  const bool nt = a.rows * a.n * 2 >= kStreamBytes;
  if (a.p == 4096)
    hipLaunchKernelGGL((rht2048_mfma_kernel<G, SCALE_F16, OUT_F32, BITS, 2>), dim3((unsigned)blocks),
                       dim3(256), 0, s, static_cast<const uint16_t*>(a.x), a.signs, a.rows, a.y, a.codes,
                       a.scales, norm, nt);
  else
    hipLaunchKernelGGL((rht2048_mfma_kernel<G, SCALE_F16, OUT_F32, BITS>), dim3((unsigned)blocks),
                       dim3(256), 0, s, static_cast<const uint16_t*>(a.x), a.signs, a.rows, a.y, a.codes,
                       a.scales, norm, nt);
}

// bf16 rows of n = 2048 or 4096: fused int4 quantization with the codes in
// the tiled fp6 format and the scales transposed (G = 128 or 256), any row
// count.  Returns false for other cases.
bool launch_rotate_quant_fp6(const RhtArgs& a, hipStream_t s) {
  if (!a.x_bf16 || (a.p != 2048 && a.p != 4096) || a.m != 1 || !a.codes || a.y) return false;
  const float norm = (float)(1.0 / sqrt((double)a.p));
  if (a.group == 128) {
    if (a.scale_f16) launch_mfma<128, true, false, 6>(a, norm, s);
    else launch_mfma<128, false, false, 6>(a, norm, s);
  } else if (a.group == 256) {
    if (a.scale_f16) launch_mfma<256, true, false, 6>(a, norm, s);
    else launch_mfma<256, false, false, 6>(a, norm, s);
  } else {
    return false;
  }
  return true;
}

// bf16 rows of n = 2048 or 4096 (m = 1): fp32 output or fused int4 / int8
// quantization.  Returns false when the case belongs to another kernel.
bool launch_rht2048_mfma(const RhtArgs& a, hipStream_t s) {
  if (!a.x_bf16 || (a.p != 2048 && a.p != 4096) || a.m != 1) return false;
  // n = 4096 with fewer rows than one resident wave per row: the mixed-radix
  // kernel, which spreads each row over eight waves, has the lower latency
  // (16 rows: 3.3 us against 5.0 us)
  if (a.p == 4096 && a.rows < 256 * mfma_blocks_per_cu<false, 2, 4>() * 4) return false;
  const float norm = (float)(1.0 / sqrt((double)a.p));
  if (a.y && !a.codes) {
    launch_mfma<0, false, true>(a, norm, s);
    return true;
  }
  if (!a.codes || a.y) return false;
#define HR_MQ(G)                                                             \
  case G:                                                                    \
    if (a.bits == 8) {                                                       \
      if (a.scale_f16) launch_mfma<G, true, false, 8>(a, norm, s);           \
      else launch_mfma<G, false, false, 8>(a, norm, s);                      \
    } else {                                                                 \
      if (a.scale_f16) launch_mfma<G, true, false>(a, norm, s);              \
      else launch_mfma<G, false, false>(a, norm, s);                         \
    }                                                                        \
    return true;
  switch (a.group) {
    HR_MQ(32)
    HR_MQ(64)
    HR_MQ(128)
    HR_MQ(256)
    default: return false;
  }
#undef HR_MQ
}

}  // namespace hr
