// Randomized (mixed-radix) Hadamard rotation, optionally fused with int4
// quantization.
//
// What is computed: for each row, y = (O kron H_p) (d * x) / sqrt(p), n = m*p
// ("Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Hypothesis and
// Method; HARP abstract and technical summary section 2.1 for the mixed-radix
// case), then per-group absmax int4 codes (same page, Method).
//
// This file holds the general workgroup-per-row kernel: the row is staged in
// LDS, the Walsh-Hadamard butterflies run stage by stage over LDS, the m x m
// block mixes the chunks at each position, and the row is quantized from LDS.
#include "hr_internal.h"
#include "hr_device.h"
#include "quant_lds.h"

namespace hr {

constexpr int kGenericThreads = 256;

template <bool IN_BF16>
__global__ __launch_bounds__(kGenericThreads) void rht_generic_kernel(RhtArgs a, float norm) {
  extern __shared__ float sm[];
  const int tid = threadIdx.x;
  const int n = a.n, m = a.m, p = a.p;
  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    // load, widen, apply the sign diagonal
    if (IN_BF16) {
      const uint16_t* xr = static_cast<const uint16_t*>(a.x) + row * n;
      for (int i = tid; i < n; i += kGenericThreads) {
        float v = bf16_bits_to_float(xr[i]);
        if (a.signs && a.signs[i] < 0) v = -v;
        sm[i] = v;
      }
    } else {
      const float* xr = static_cast<const float*>(a.x) + row * n;
      for (int i = tid; i < n; i += kGenericThreads) {
        float v = xr[i];
        if (a.signs && a.signs[i] < 0) v = -v;
        sm[i] = v;
      }
    }
    __syncthreads();
    // Walsh-Hadamard butterflies within each chunk of p (pairs never cross a
    // chunk because every stride h < p and chunks are p-aligned)
    for (int h = 1; h < p; h <<= 1) {
      for (int t = tid; t < (n >> 1); t += kGenericThreads) {
        const int i = (t / h) * 2 * h + (t % h);
        const float u = sm[i], v = sm[i + h];
        sm[i] = u + v;
        sm[i + h] = u - v;
      }
      __syncthreads();
    }
    // mix the m chunks at every position with the orthogonal block
    if (m > 1) {
      for (int r = tid; r < p; r += kGenericThreads) {
        float v[16];
        for (int j = 0; j < m; ++j) v[j] = sm[j * p + r];
        for (int i = 0; i < m; ++i) {
          float acc = 0.0f;
          for (int j = 0; j < m; ++j) acc = fmaf(a.block[i * m + j], v[j], acc);
          sm[i * p + r] = acc;
        }
      }
      __syncthreads();
    }
    if (a.y) {
      float* yr = a.y + row * n;
      for (int i = tid; i < n; i += kGenericThreads) yr[i] = sm[i] * norm;
    }
    if (a.codes) {
      const int64_t row_bytes = a.bits == 8 ? n : (n >> 1);
      quant_row_from_lds(sm, norm, n, a.group, a.codes + row * row_bytes, a.scales,
                         row * (n / a.group), a.scale_f16, a.bits);
    }
    __syncthreads();
  }
}

hipError_t launch_rht(const RhtArgs& a, hipStream_t s) {
  if (launch_rht2048_mfma(a, s)) return hipGetLastError();
  if (launch_mixed2048_mfma(a, s)) return hipGetLastError();
  if (launch_rht2048(a, s)) return hipGetLastError();
  const float norm = (float)(1.0 / sqrt((double)a.p));
  const int64_t grid64 = a.rows < 4096 ? a.rows : 4096;
  const dim3 grid((unsigned)grid64), block(kGenericThreads);
  const size_t lds = sizeof(float) * (size_t)a.n;
  if (a.x_bf16)
    hipLaunchKernelGGL(rht_generic_kernel<true>, grid, block, lds, s, a, norm);
  else
    hipLaunchKernelGGL(rht_generic_kernel<false>, grid, block, lds, s, a, norm);
  return hipGetLastError();
}

}  // namespace hr
