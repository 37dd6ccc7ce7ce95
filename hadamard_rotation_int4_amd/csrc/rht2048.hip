// Randomized Hadamard transform of rows built from 2048-point chunks, fused
// with int4 quantization (or an fp32 store).  The chunk transform itself is
// the register-resident wave64 routine of fwht2048.h.
//
// rht2048_kernel: n = 2048 ("Experiment -- Hadamard rotation for int4 (W4A4)
//   accuracy", Hypothesis and Method; "Llama-3.2-1B-Instruct-HadamardSpin-
//   4bits", How it Works).  One wave per row, persistent over rows, the next
//   row's loads in flight while the current one is transformed.
//
// mixed2048_kernel: n = m * 2048, y = (O kron H_2048) D x / sqrt(2048) (HARP
//   abstract: mixed-radix schedules for dimensions that are not powers of two;
//   HARP technical summary (gist.science), section 2.1: a radix that is not a
//   power of two uses a fixed orthogonal block).  One workgroup of m waves per
//   row: wave w transforms chunk w in registers and writes it to LDS; after a
//   barrier wave w forms output chunk w = sum_c O[w][c] * chunk_c from LDS (m
//   fma per element, same register placement) and quantizes or stores it.
#include "hr_internal.h"
#include "fwht2048.h"

namespace hr {

template <bool IN_BF16, int G, bool SCALE_F16, bool OUT_F32>
__global__ __launch_bounds__(256) void rht2048_kernel(const void* __restrict__ xin,
                                                       const int8_t* __restrict__ signs,
                                                       int64_t rows, float* __restrict__ yout,
                                                       uint8_t* __restrict__ codes,
                                                       void* __restrict__ scales, float norm) {
  constexpr int N = 2048;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  Lane2048 L;
  lane2048_init(L, signs);

  u32x4 nxt[4];
  if (IN_BF16 && wave < rows) load2048_bf16(L, static_cast<const uint16_t*>(xin) + wave * N, nxt);

  for (int64_t row = wave; row < rows; row += nwaves) {
    float v[4][8];
    if (IN_BF16) {
      u32x4 raw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) raw[j] = nxt[j];
      if (row + nwaves < rows)
        load2048_bf16(L, static_cast<const uint16_t*>(xin) + (row + nwaves) * N, nxt);
      fwht2048_first_bf16(L, raw, v);
    } else {
      fwht2048_first_f32(L, static_cast<const float*>(xin) + row * N, v);
    }
    fwht2048_rest(L, v);
    if (OUT_F32) {
      store2048_f32(L, v, norm * L.tau, yout + row * N);
    } else {
      quant2048<G, SCALE_F16>(L, v, norm, L.tau,
                              reinterpret_cast<uint32_t*>(codes + row * (N / 2)), scales,
                              row * (N / (G > 0 ? G : 1)));
    }
  }
}

template <bool IN_BF16, int G, bool SCALE_F16, bool OUT_F32, bool SYLV = false>
__global__ __launch_bounds__(1024) void mixed2048_kernel(const void* __restrict__ xin,
                                                          const int8_t* __restrict__ signs,
                                                          const float* __restrict__ block, int m,
                                                          int64_t rows, float* __restrict__ yout,
                                                          uint8_t* __restrict__ codes,
                                                          void* __restrict__ scales, float norm) {
  constexpr int P = 2048;
  extern __shared__ f32x4 lds4[];               // m chunks x 2048 floats
  float* lds = reinterpret_cast<float*>(lds4);
  const int w = threadIdx.x >> 6;               // chunk of this wave
  const int64_t n = (int64_t)m * P;
  Lane2048 L;
  lane2048_init(L, signs ? signs + (int64_t)w * P : nullptr);
  // row w of the block: the given orthogonal O, or (SYLV) the +-1 Sylvester
  // matrix H_m, so that H_m kron H_2048 = H_{m 2048} exactly
  float o[16];
#pragma unroll
  for (int c = 0; c < 16; ++c)
    o[c] = c < m ? (SYLV ? ((__builtin_popcount(w & c) & 1) ? -1.0f : 1.0f) : block[w * m + c]) : 0.0f;

  u32x4 nxt[4];
  if (IN_BF16 && (int64_t)blockIdx.x < rows)
    load2048_bf16(L, static_cast<const uint16_t*>(xin) + (int64_t)blockIdx.x * n + (int64_t)w * P, nxt);

  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    float v[4][8];
    if (IN_BF16) {
      u32x4 raw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) raw[j] = nxt[j];
      if (row + gridDim.x < rows)
        load2048_bf16(L, static_cast<const uint16_t*>(xin) + (row + gridDim.x) * n + (int64_t)w * P, nxt);
      fwht2048_first_bf16(L, raw, v);
    } else {
      fwht2048_first_f32(L, static_cast<const float*>(xin) + row * n + (int64_t)w * P, v);
    }
    fwht2048_rest(L, v);
    // chunk w (true values) to LDS in natural element order
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4* dst = reinterpret_cast<f32x4*>(lds + w * P + elem2048(L, j));
      dst[0] = (f32x4){v[j][0] * L.tau, v[j][1] * L.tau, v[j][2] * L.tau, v[j][3] * L.tau};
      dst[1] = (f32x4){v[j][4] * L.tau, v[j][5] * L.tau, v[j][6] * L.tau, v[j][7] * L.tau};
    }
    __syncthreads();
    // output chunk w at the same positions: sum_c O[w][c] * chunk_c
    float acc[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
    for (int c = 0; c < m; ++c) {
      const float oc = o[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4* src = reinterpret_cast<const f32x4*>(lds + c * P + elem2048(L, j));
        const f32x4 p0 = src[0], p1 = src[1];
        acc[j][0] = fmaf(oc, p0.x, acc[j][0]);
        acc[j][1] = fmaf(oc, p0.y, acc[j][1]);
        acc[j][2] = fmaf(oc, p0.z, acc[j][2]);
        acc[j][3] = fmaf(oc, p0.w, acc[j][3]);
        acc[j][4] = fmaf(oc, p1.x, acc[j][4]);
        acc[j][5] = fmaf(oc, p1.y, acc[j][5]);
        acc[j][6] = fmaf(oc, p1.z, acc[j][6]);
        acc[j][7] = fmaf(oc, p1.w, acc[j][7]);
      }
    }
    if (OUT_F32) {
      store2048_f32(L, acc, norm, yout + row * n + (int64_t)w * P);
    } else {
      quant2048<G, SCALE_F16>(L, acc, norm, 1.0f,
                              reinterpret_cast<uint32_t*>(codes + row * (n / 2) + (int64_t)w * (P / 2)),
                              scales, row * (n / (G > 0 ? G : 1)) + (int64_t)w * (P / (G > 0 ? G : 1)));
    }
    __syncthreads();                            // LDS is rewritten by the next row
  }
}

template <bool IN_BF16, int G, bool SCALE_F16, bool OUT_F32>
static void launch_one(const RhtArgs& a, float norm, hipStream_t s) {
  if (a.p > 2048) {
    // p = m' * 2048 with m = 1: the mixed-radix kernel with the Sylvester block
    const int mm = a.p / 2048;
    const size_t lds = (size_t)mm * 2048 * sizeof(float);
    const int per_cu = lds <= 80 * 1024 ? 2 : 1;
    const int64_t blocks = a.rows < 256 * per_cu ? a.rows : 256 * per_cu;
    hipLaunchKernelGGL((mixed2048_kernel<IN_BF16, G, SCALE_F16, OUT_F32, true>), dim3((unsigned)blocks),
                       dim3(64 * mm), lds, s, a.x, a.signs, (const float*)nullptr, mm, a.rows, a.y,
                       a.codes, a.scales, norm);
    return;
  }
  if (a.m == 1) {
    // persistent grid: as many 4-wave blocks as are resident at once (a block
    // past that would only start when another has finished all its rows)
    static const int per_cu = [] {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &nb, reinterpret_cast<const void*>(&rht2048_kernel<IN_BF16, G, SCALE_F16, OUT_F32>), 256, 0) !=
              hipSuccess ||
          nb < 1)
        nb = 1;
      return nb;
    }();
    int64_t blocks = (a.rows + 3) / 4;   // one wave per row, 4 waves per block
    const int64_t cap = 256 * (int64_t)per_cu;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL((rht2048_kernel<IN_BF16, G, SCALE_F16, OUT_F32>), dim3((unsigned)blocks),
                       dim3(256), 0, s, a.x, a.signs, a.rows, a.y, a.codes, a.scales, norm);
  } else {
    // one row per workgroup of m waves; LDS holds the row (m * 8 KB)
    const size_t lds = (size_t)a.m * 2048 * sizeof(float);
    const int per_cu = lds <= 80 * 1024 ? 2 : 1;
    const int64_t blocks = a.rows < 256 * per_cu ? a.rows : 256 * per_cu;
    hipLaunchKernelGGL((mixed2048_kernel<IN_BF16, G, SCALE_F16, OUT_F32>), dim3((unsigned)blocks),
                       dim3(64 * a.m), lds, s, a.x, a.signs, a.block, a.m, a.rows, a.y, a.codes,
                       a.scales, norm);
  }
}

template <bool IN_BF16>
static bool dispatch_in(const RhtArgs& a, float norm, hipStream_t s) {
  if (a.y && !a.codes) {
    launch_one<IN_BF16, 0, false, true>(a, norm, s);
    return true;
  }
  if (!a.codes || a.y) return false;
#define HR_Q(G)                                                              \
  case G:                                                                    \
    if (a.scale_f16) launch_one<IN_BF16, G, true, false>(a, norm, s);        \
    else launch_one<IN_BF16, G, false, false>(a, norm, s);                   \
    return true;
  switch (a.group) {
    HR_Q(32)
    HR_Q(64)
    HR_Q(128)
    HR_Q(256)
    default: return false;
  }
#undef HR_Q
}

// Handles p == 2048 (n = m * 2048, 1 <= m <= 16), and the plain transform of
// p = 4096, 8192, 16384 (m = 1) as H_{p/2048} kron H_2048; fp32 output or
// fused int4 quantization.  Returns false when the case belongs to the
// general kernel.
bool launch_rht2048(const RhtArgs& a, hipStream_t s) {
  if (a.codes && a.bits == 8) return false;     // int8 codes: generic kernel
  if (a.m == 1 && (a.p == 4096 || a.p == 8192 || a.p == 16384)) {
    const float norm = (float)(1.0 / sqrt((double)a.p));
    return a.x_bf16 ? dispatch_in<true>(a, norm, s) : dispatch_in<false>(a, norm, s);
  }
  if (a.p != 2048 || a.m < 1 || a.m > 16) return false;
  if (a.m > 1 && (size_t)a.m * 2048 * sizeof(float) > 160 * 1024) return false;
  const float norm = (float)(1.0 / sqrt(2048.0));
  return a.x_bf16 ? dispatch_in<true>(a, norm, s) : dispatch_in<false>(a, norm, s);
}

}  // namespace hr
