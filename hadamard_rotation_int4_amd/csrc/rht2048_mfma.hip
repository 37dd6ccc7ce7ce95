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
//     global_load_lds_dwordx4 (two rows in flight per wave without holding
//     registers).  Load j < 4, lane i fetches the 16-byte piece (chunk i & 15,
//     piece 4 j + (i >> 4) of the chunk), so global reads come in 64-byte
//     runs and the 16 pieces a lane group needs for one MFMA are consecutive
//     LDS slots (no bank conflicts).
//   Codes: a lane owns four runs of 8 consecutive outputs; they are staged
//     through LDS (swizzled, conflict-free) and written as contiguous 1 KB
//     runs, one per store instruction (one per int4 row, two per int8 row).
#include "mfma2048.h"

namespace hr {

constexpr int kMfmaBlocksPerCu = 2;

// 16-byte global -> LDS copy (the builtin sits in a device function: used
// directly in a kernel template it can cost the instance its host stub)
__device__ __forceinline__ void mfma_lds_load16(const void* gp, void* lp) {
  __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 0);
}

template <int G, bool SCALE_F16, bool OUT_F32, int BITS, int CH = 1>
__global__ __launch_bounds__(256, kMfmaBlocksPerCu) void rht2048_mfma_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ signs, int64_t rows,
    float* __restrict__ yout, uint8_t* __restrict__ codes, void* __restrict__ scales, float norm) {
  static_assert(CH == 1 || CH == 2, "rows of one or two 2048-point chunks");
  constexpr int P = 2048;          // chunk
  constexpr int N = CH * P;        // row
  const int lane = threadIdx.x & 63;
  const int wib = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + wib;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  Mfma2048 M[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) mfma2048_init(M[c], lane, signs ? signs + c * P : nullptr);
  const int g = M[0].g, a4 = M[0].a4;
  const float tau = M[0].tau;

  // LDS of this wave: two row stages (256 slots of 16 bytes per chunk) and
  // one chunk of codes
  __shared__ __attribute__((aligned(16))) u32x4 stage_lds[4][2][CH * 256];
  __shared__ __attribute__((aligned(16))) u32x4 code_lds[4][BITS == 8 ? 128 : 64];
  // fp32 output: this wave's 8 KB output row, staged so it leaves as 1 KB stores
  __shared__ __attribute__((aligned(16))) f32x4 out_lds[OUT_F32 ? 4 : 1][OUT_F32 ? 512 : 1];
  // element offset of this lane's piece within a row, per load j: + 32 j
  const int lane_src = 128 * (lane & 15) + 8 * (lane >> 4);
  auto issue = [&](int64_t row, int st) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint16_t* base = x + row * N + c * P + lane_src;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        mfma_lds_load16(base + 32 * j, &stage_lds[wib][st][256 * c + 64 * j]);
    }
  };
  // B operands of one row from stage st: lane (q, g) takes slot 64 s + 16 g +
  // A(q) of each chunk for K-step s.  One asm block waits for the stage (at
  // most 4 CH younger vector-memory ops, the other stage's loads, may still be
  // pending; loads complete in order) and for its own results.
  const uint32_t rd_lane = 16u * (uint32_t)(16 * g + a4);
  auto read_stage = [&](int st, bool next_pending, u32x4 (&b)[CH][4]) {
    const uint32_t addr = (uint32_t)(uintptr_t)&stage_lds[wib][st][0] + rd_lane;
#define HR_DSR4(WAIT)                                                                    \
    asm volatile(WAIT "\n\t"                                                             \
                 "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"             \
                 "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t" \
                 "s_waitcnt lgkmcnt(0)"                                                  \
                 : "=v"(b[0][0]), "=v"(b[0][1]), "=v"(b[0][2]), "=v"(b[0][3])             \
                 : "v"(addr)                                                             \
                 : "memory")
#define HR_DSR8(WAIT)                                                                    \
    asm volatile(WAIT "\n\t"                                                             \
                 "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"             \
                 "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t" \
                 "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t" \
                 "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t" \
                 "s_waitcnt lgkmcnt(0)"                                                  \
                 : "=v"(b[0][0]), "=v"(b[0][1]), "=v"(b[0][2]), "=v"(b[0][3]),            \
                   "=v"(b[CH - 1][0]), "=v"(b[CH - 1][1]), "=v"(b[CH - 1][2]), "=v"(b[CH - 1][3]) \
                 : "v"(addr)                                                             \
                 : "memory")
    if (CH == 1) {
      if (next_pending) HR_DSR4("s_waitcnt vmcnt(4)");
      else HR_DSR4("s_waitcnt vmcnt(0)");
    } else {
      if (next_pending) HR_DSR8("s_waitcnt vmcnt(8)");
      else HR_DSR8("s_waitcnt vmcnt(0)");
    }
#undef HR_DSR4
#undef HR_DSR8
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
    float mg[NG];
    if (G == 32) {
#pragma unroll
      for (int m = 0; m < 4; ++m) mg[m] = mr[m];
    } else if (G == 64) {
      mg[0] = fmaxf(mr[0], mr[1]);
      mg[NG - 1] = fmaxf(mr[2], mr[3]);
    } else {
      mg[0] = fmaxf(fmaxf(mr[0], mr[1]), fmaxf(mr[2], mr[3]));
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) mg[i] = max_over_rows(mg[i]);
    if (G == 256) mg[0] = __uint_as_float(umax_dpp<kQuadXor1>(__float_as_uint(mg[0])));
    float kk[NG];
    float s_own = 0.0f;                  // scale of the group this lane stores
    bool need_clamp = false;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const float s32 = div_const<BITS == 8 ? 127 : 7>(mg[i] * norm);
      const float s = SCALE_F16 ? (float)(_Float16)s32 : s32;
      kk[i] = s > 0.0f ? norm * __builtin_amdgcn_rcpf(s) * tau : 0.0f;
      need_clamp |= s > 0.0f && s < (SCALE_F16 ? 6.103515625e-05f : 1.17549435e-38f);
      if (NG == 1 || i == (g & (NG - 1))) s_own = s32;
    }
    {
      int64_t si = -1;
      const int64_t s0 = row * (N / G) + ch * (P / G);   // the chunk's first group
      if (G == 32) si = s0 + 4 * a4 + g;
      else if (G == 64) si = g < 2 ? s0 + 2 * a4 + g : -1;
      else if (G == 128) si = g == 0 ? s0 + a4 : -1;
      else si = (g == 0 && (a4 & 1) == 0) ? s0 + (a4 >> 1) : -1;
      if (si >= 0) {
        if (SCALE_F16) reinterpret_cast<_Float16*>(scales)[si] = (_Float16)s_own;
        else reinterpret_cast<float*>(scales)[si] = s_own;
      }
    }
    const bool clamp = __builtin_amdgcn_ballot_w64(need_clamp) != 0;
    // q + M rounds y k to an integer in the low mantissa bits (ties to even)
    constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
    const float M = BITS == 8 ? 12582912.0f : 12582920.0f;   // 1.5 * 2^23 (+ 8 for nibbles)
    u32x4* cl = &code_lds[wib][0];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float k = kk[G == 32 ? m : G == 64 ? (m >> 1) : 0];
      const f32x4 lo = acc[2 * m], hi = acc[2 * m + 1];
      float rr[8] = {fmaf(lo[0], k, M), fmaf(lo[1], k, M), fmaf(lo[2], k, M), fmaf(lo[3], k, M),
                     fmaf(hi[0], k, M), fmaf(hi[1], k, M), fmaf(hi[2], k, M), fmaf(hi[3], k, M)};
      if (clamp) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rr[e] = __builtin_amdgcn_fmed3f(rr[e], M - QMAX, M + QMAX);
      }
      if (BITS == 4) {
        // dword 16 a + 4 m + g of the row: 16-byte block (a, m) at 4 a + (m ^ (a >> 2 & 3))
        reinterpret_cast<uint32_t*>(cl)[4 * (4 * a4 + (m ^ ((a4 >> 2) & 3))) + g] = pack8(rr);
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
    if (BITS == 4) {
      // lane i stores bytes 16 i .. 16 i + 15 of the row: block (i >> 2, i & 3)
      const int ra = lane >> 2, rm = lane & 3;
      const u32x4 out = cl[4 * ra + (rm ^ ((ra >> 2) & 3))];
      __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(codes + row * (N / 2) + ch * (P / 2)) + lane);
    } else {
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

  int64_t row = wave;
  if (row < rows) issue(row, 0);
  if (row + nwaves < rows) issue(row + nwaves, 1);
  for (int st = 0; row < rows; row += nwaves, st ^= 1) {
    u32x4 b[CH][4];
    read_stage(st, row + nwaves < rows, b);
    if (row + 2 * nwaves < rows) issue(row + 2 * nwaves, st);
    process(row, b);
  }
}

template <int G, bool SCALE_F16, bool OUT_F32, int BITS = 4>
static void launch_mfma(const RhtArgs& a, float norm, hipStream_t s) {
  int64_t blocks = (a.rows + 3) / 4;              // 4 waves per block, one row per wave
  const int64_t cap = 256 * kMfmaBlocksPerCu;
  if (blocks > cap) blocks = cap;
  if (a.p == 4096)
    hipLaunchKernelGGL((rht2048_mfma_kernel<G, SCALE_F16, OUT_F32, BITS, 2>), dim3((unsigned)blocks),
                       dim3(256), 0, s, static_cast<const uint16_t*>(a.x), a.signs, a.rows, a.y, a.codes,
                       a.scales, norm);
  else
    hipLaunchKernelGGL((rht2048_mfma_kernel<G, SCALE_F16, OUT_F32, BITS>), dim3((unsigned)blocks),
                       dim3(256), 0, s, static_cast<const uint16_t*>(a.x), a.signs, a.rows, a.y, a.codes,
                       a.scales, norm);
}

// bf16 rows of n = 2048 or 4096 (m = 1): fp32 output or fused int4 / int8
// quantization.  Returns false when the case belongs to another kernel.
bool launch_rht2048_mfma(const RhtArgs& a, hipStream_t s) {
  if (!a.x_bf16 || (a.p != 2048 && a.p != 4096) || a.m != 1) return false;
  // n = 4096 with fewer rows than one resident wave per row: the mixed-radix
  // kernel, which spreads each row over eight waves, has the lower latency
  // (16 rows: 3.3 us against 5.0 us)
  if (a.p == 4096 && a.rows < 256 * kMfmaBlocksPerCu * 4) return false;
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
