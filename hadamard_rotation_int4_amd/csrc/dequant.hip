// int4 dequantization: x_hat = q * s, one fp32 product per element (exact
// relative to the stored codes and scales).
// Source: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Method
// (per-group quantize -> dequantize).
#include "hr_internal.h"
#include "hr_device.h"

namespace hr {

// One thread expands one dword of packed codes (8 codes) into two float4.
template <bool F16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                      const void* __restrict__ scales,
                                                      int64_t total_words, int words_per_row,
                                                      int words_per_group, int groups_per_row,
                                                      float4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total_words; w += stride) {
    const int64_t row = w / words_per_row;
    const int col = (int)(w - row * words_per_row);
    const int64_t sidx = row * groups_per_row + col / words_per_group;
    const float s = F16 ? (float)reinterpret_cast<const _Float16*>(scales)[sidx]
                        : reinterpret_cast<const float*>(scales)[sidx];
    const uint32_t q = codes[w];
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int nib = (int)((q >> (4 * e)) & 0xF);
      v[e] = (float)(nib >= 8 ? nib - 16 : nib) * s;
    }
    out[2 * w] = make_float4(v[0], v[1], v[2], v[3]);
    out[2 * w + 1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

hipError_t launch_dequant(const uint8_t* codes, const void* scales, int scale_f16, int64_t rows,
                          int n, int group, float* out, hipStream_t s) {
  const int words_per_row = n / 8;
  const int64_t total = rows * words_per_row;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  float4* o4 = reinterpret_cast<float4*>(out);
  if (scale_f16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, s, cw,
                       scales, total, words_per_row, group / 8, n / group, o4);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, s, cw,
                       scales, total, words_per_row, group / 8, n / group, o4);
  return hipGetLastError();
}

}  // namespace hr
