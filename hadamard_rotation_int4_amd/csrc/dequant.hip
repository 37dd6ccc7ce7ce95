// int4 dequantization: x_hat = q * s, one fp32 product per element (exact
// relative to the stored codes and scales).
// Source: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Method
// (per-group quantize -> dequantize).
//
// The [rows][n] output is treated as one flat array: since G divides n, the
// scale of flat element e is scales[e / G].  Lane l of a wave expands quad
// q0 + l (outputs 4 q .. 4 q + 3, the 16 bits of codes at byte 2 q), so a
// wave reads 128 contiguous bytes of codes and writes 1 KB of fp32 with one
// nontemporal store; each thread handles kUnroll quads a grid stride apart,
// loading all of them before it stores.
#include "hr_internal.h"
#include "hr_device.h"

namespace hr {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDeqThreads = 256;
constexpr int kUnroll = 4;

template <bool F16>
__global__ __launch_bounds__(kDeqThreads) void dequant_kernel(const uint16_t* __restrict__ codes,
                                                              const void* __restrict__ scales,
                                                              int64_t quads, int group,
                                                              f32x4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kDeqThreads;
  for (int64_t q0 = (int64_t)blockIdx.x * kDeqThreads + threadIdx.x; q0 < quads;
       q0 += kUnroll * stride) {
    uint32_t c[kUnroll];
    float s[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t q = q0 + u * stride < quads ? q0 + u * stride : q0;   // in bounds
      c[u] = codes[q];
      const int64_t si = 4 * q / group;
      s[u] = F16 ? (float)reinterpret_cast<const _Float16*>(scales)[si]
                 : reinterpret_cast<const float*>(scales)[si];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t q = q0 + u * stride;
      if (q < quads) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // two's-complement nibble e, sign-extended by an arithmetic shift
          const int nib = ((int)(c[u] << (28 - 4 * e))) >> 28;
          v[e] = (float)nib * s[u];
        }
        __builtin_nontemporal_store((f32x4){v[0], v[1], v[2], v[3]}, out + q);
      }
    }
  }
}

hipError_t launch_dequant(const uint8_t* codes, const void* scales, int scale_f16, int64_t rows,
                          int n, int group, float* out, hipStream_t s) {
  const int64_t quads = rows * (int64_t)(n / 4);
  int64_t blocks = (quads + (int64_t)kDeqThreads * kUnroll - 1) / ((int64_t)kDeqThreads * kUnroll);
  // two workgroups per CU, each thread with kUnroll stores in flight: the
  // best of a sweep over 256..4096 workgroups and 1, 2, 4, 8 quads per thread
  if (blocks > 512) blocks = 512;
  const uint16_t* c16 = reinterpret_cast<const uint16_t*>(codes);
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  if (scale_f16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)blocks), dim3(kDeqThreads), 0, s, c16,
                       scales, quads, group, o4);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)blocks), dim3(kDeqThreads), 0, s, c16,
                       scales, quads, group, o4);
  return hipGetLastError();
}

}  // namespace hr
